"""hipGraph capture of the entry points around the RG-LRU branch: the recurrent block, the
gated MLP and local MQA forwards, and the block's and local MQA's decode steps.  Each call
initialises whatever it needs with kernels (no memset nodes), so a captured call replayed
several times, with unrelated eager work and synchronisations between the replays, must
give the eager result bit for bit; a captured decode step replayed n times must give the
n eager steps, since it updates its state in place.
"""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import TORCH_IO, dev

pytestmark = pytest.mark.gpu


def _replay_equals_eager(run, outs, reps=3, reset=None):
    """Eager run, then capture `run` once and replay it `reps` times; every replay's `outs`
    must equal the eager ones.  `reset` (optional) restores in-place state before each."""
    if reset:
        reset()
    run()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    if reset:
        reset()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(reps):
        for o in outs:
            o.zero_()
        if reset:               # after the zeroing: in-place state among `outs` is restored
            reset()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (o, r) in enumerate(zip(outs, ref)):
            assert torch.equal(o, r), (rep, i)
        _ = torch.ones(1 << 20, device="cuda").sum().item()     # unrelated eager work


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_block_forward_graph(lib, io):
    w = workloads.TRAIN_FWD.with_shape(B=2, T=300, D=192, io=io, h0="normal", history="normal")
    p = workloads.make_block_inputs(w, d_model=320)
    t = TORCH_IO[io]
    xb, W_in, W_out = dev(p["x_block"], t), dev(p["W_in"], t), dev(p["W_out"], t)
    cw, cb, cs = dev(p["conv_w"], t), dev(p["conv_b"]), dev(p["conv_state"], t)
    Wa, Wx, ba, bx, lam, h0 = (dev(p["W_a"], t), dev(p["W_x"], t), dev(p["b_a"]), dev(p["b_x"]),
                               dev(p["lam"]), dev(p["h0"]))
    B, T, D, R = 2, 300, 320, 192
    out = torch.empty((B, T, D), dtype=t, device="cuda")
    hT = torch.empty((B, R), device="cuda")
    cso = torch.empty((B, 3, R), dtype=t, device="cuda")
    ws = lib.workspace(lib.block_fwd_workspace_bytes(B, T, D, R, t))
    _replay_equals_eager(lambda: lib.rglru_block_fwd(xb, W_in, cw, cb, cs, Wa, Wx, ba, bx, lam, h0,
                                                     W_out, out, hT, cso, ws, p["c"]),
                         [out, hT, cso])


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_mlp_forward_graph(lib, io):
    w = workloads.TRAIN_FWD.with_shape(B=2, T=257, D=192, io=io)
    p = workloads.make_mlp_inputs(w, expansion=3)
    t = TORCH_IO[io]
    x, W1, W2, W3 = dev(p["x"], t), dev(p["W_1"], t), dev(p["W_2"], t), dev(p["W_3"], t)
    out = torch.empty((2, 257, 192), dtype=t, device="cuda")
    ws = lib.workspace(lib.mlp_fwd_workspace_bytes(2, 257, 192, 3 * 192, t))
    _replay_equals_eager(lambda: lib.gated_mlp_fwd(x, W1, W2, W3, out, ws), [out])


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_mqa_forward_graph(lib, io):
    B, T, D, W = 2, 300, 256, 64
    w = workloads.TRAIN_FWD.with_shape(B=B, T=T, D=D, io=io)
    p = workloads.make_mqa_inputs(w, W)
    t = TORCH_IO[io]
    x = dev(p["x"], t)
    Wqkv = dev(np.concatenate([p["W_q"], p["W_k"], p["W_v"]]), t)
    Wo = dev(p["W_o"], t)
    out = torch.empty((B, T, D), dtype=t, device="cuda")
    k = torch.empty((B, T, 128), dtype=t, device="cuda")
    v = torch.empty_like(k)
    ws = lib.workspace(lib.mqa_fwd_workspace_bytes(B, T, D, t))
    _replay_equals_eager(lambda: lib.local_mqa_fwd(x, Wqkv, Wo, out, k, v, ws, W, 5), [out, k, v])


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_block_decode_step_graph(lib, io):
    """Three replays of one captured block decode step continue the state like three eager
    steps on the same token."""
    B, D, R = 3, 256, 192
    w = workloads.DECODE.with_shape(B=B, D=R, T=1, io=io, decode=False)
    p = workloads.make_block_inputs(w, d_model=D)
    t = TORCH_IO[io]
    x_t = dev(p["x_block"][:, 0], t)
    W_in, W_out = dev(p["W_in"], t), dev(p["W_out"], t)
    cw, cb = dev(p["conv_w"], t), dev(p["conv_b"])
    Wa, Wx, ba, bx, lam = dev(p["W_a"], t), dev(p["W_x"], t), dev(p["b_a"]), dev(p["b_x"]), dev(p["lam"])
    cs0, h0 = dev(p["conv_state"], t), dev(p["h0"])
    cs, h = cs0.clone(), h0.clone()
    out = torch.empty((B, D), dtype=t, device="cuda")
    ws = lib.workspace(lib.block_decode_workspace_bytes(B, D, R, t))
    step = lambda: lib.rglru_block_decode_step(x_t, W_in, cw, cb, cs, Wa, Wx, ba, bx, lam, h,
                                               W_out, out, ws, p["c"])
    eager = []
    for _ in range(3):
        step()
        eager.append((out.clone(), h.clone(), cs.clone()))
    torch.cuda.synchronize()
    cs.copy_(cs0)
    h.copy_(h0)
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            step()
    torch.cuda.current_stream().wait_stream(s)
    cs.copy_(cs0)
    h.copy_(h0)
    torch.cuda.synchronize()
    for i in range(3):
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager[i][0]) and torch.equal(h, eager[i][1]), i
        assert torch.equal(cs, eager[i][2]), i


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_mqa_decode_step_graph(lib, io):
    """Replays of one captured MQA decode step at a fixed position rewrite the same cache slot
    from the same token: every replay equals the eager step."""
    B, D, W = 2, 256, 16
    w = workloads.TRAIN_FWD.with_shape(B=B, T=1, D=D, io=io)
    p = workloads.make_mqa_inputs(w, W)
    t = TORCH_IO[io]
    x_t = dev(p["x"][:, 0], t)
    Wqkv = dev(np.concatenate([p["W_q"], p["W_k"], p["W_v"]]), t)
    Wo = dev(p["W_o"], t)
    pos = torch.tensor([5, 21], dtype=torch.int32, device="cuda")
    kc = torch.randn((B, W, 128), generator=torch.Generator().manual_seed(3)).to(t).cuda()
    vc = torch.randn((B, W, 128), generator=torch.Generator().manual_seed(4)).to(t).cuda()
    kc0, vc0 = kc.clone(), vc.clone()
    out = torch.empty((B, D), dtype=t, device="cuda")
    ws = lib.workspace(lib.mqa_decode_workspace_bytes(B, D, t))

    def reset():
        kc.copy_(kc0)
        vc.copy_(vc0)
    _replay_equals_eager(lambda: lib.local_mqa_decode_step(pos, x_t, Wqkv, Wo, kc, vc, out, ws),
                         [out, kc, vc], reset=reset)
