"""Parity of the local-MQA decode step with its bounded key/value cache
(local_mqa_decode_step) with the oracle (the Griffin model-architecture page, section "Local
sliding-window attention": the cache holds at most the window).

Decode from an empty cache over more steps than the window (slots are reused) against the
oracle forward at every position; distinct positions per sequence against the oracle's own
decode step; a prefill (local_mqa_fwd's rotated keys and values placed in their slots) handed
over to decode; and one step at the full decode shape (B=256, D=2560, window 1024) from
random caches on a seeded subset of sequences.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import TOL, TORCH_IO, dev, err, host

pytestmark = pytest.mark.gpu


def _weights(p, io):
    t = TORCH_IO[io]
    return dev(np.concatenate([p["W_q"], p["W_k"], p["W_v"]]), t), dev(p["W_o"], t)


def _decode_run(g, p, window, steps, start=None):
    """Run `steps` decode steps over x[:, :steps] from zero caches; sequence b starts at
    position start[b].  Returns the outputs [B, steps, D] and the final caches."""
    w = p["workload"]
    io = TORCH_IO[w.io]
    B, D = w.B, w.D
    Wqkv, Wo = _weights(p, w.io)
    kc = torch.zeros((B, window, 128), dtype=io, device="cuda")
    vc = torch.zeros_like(kc)
    start = np.zeros(B, dtype=np.int32) if start is None else np.asarray(start, dtype=np.int32)
    ws = g.workspace(g.mqa_decode_workspace_bytes(B, D, io))
    x = dev(p["x"], io)
    outs = []
    for t in range(steps):
        pos = torch.from_numpy(start + t).to("cuda")
        out = torch.empty((B, D), dtype=io, device="cuda")
        g.local_mqa_decode_step(pos, x[:, t].contiguous(), Wqkv, Wo, kc, vc, out, ws)
        outs.append(out)
    torch.cuda.synchronize()
    return host(torch.stack(outs, 1)), host(kc), host(vc)


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("window", [16, 64])
def test_decode_from_empty_cache_matches_forward(lib, io, window):
    T = 2 * window + 9
    w = workloads.TRAIN_FWD.with_shape(B=2, T=T, D=256, io=io)
    p = workloads.make_mqa_inputs(w, window)
    got, kc, vc = _decode_run(lib, p, window, T)
    f = oracle.local_mqa_forward(p["x"], p["W_q"], p["W_k"], p["W_v"], p["W_o"], window, io, keep=True)
    e = err(got, f["out"])
    slots = [s % window for s in range(T - window, T)]
    ek = err(kc[:, slots], f["k"][:, T - window:])
    print(f"decode io={io} W={window} T={T} err(out)={e:.3e} err(kcache)={ek:.3e}", flush=True)
    assert e <= TOL[io] and ek <= TOL[io]
    assert err(vc[:, slots], f["v"][:, T - window:]) <= TOL[io]


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_decode_distinct_positions_per_sequence(lib, io):
    """Sequences at different positions (and so different live slots and RoPE angles) in one
    batch, zero caches, against the oracle's decode step step by step."""
    window, steps = 32, 12
    w = workloads.TRAIN_FWD.with_shape(B=3, T=steps, D=384, io=io)
    p = workloads.make_mqa_inputs(w, window)
    start = np.array([0, 5, 40], dtype=np.int32)
    got, _, _ = _decode_run(lib, p, window, steps, start)
    kc = np.zeros((3, window, 128))
    vc = np.zeros((3, window, 128))
    want = []
    for t in range(steps):
        o, kc, vc = oracle.local_mqa_decode_step(p["x"][:, t], p["W_q"], p["W_k"], p["W_v"], p["W_o"],
                                                 kc, vc, start + t, window, io)
        want.append(o)
    e = err(got, np.stack(want, 1))
    print(f"distinct positions io={io} err(out)={e:.3e}", flush=True)
    assert e <= TOL[io]


def test_prefill_hands_over_to_decode(lib):
    """local_mqa_fwd over 150 tokens, its rotated keys and values of the last `window`
    positions placed in slot position % window, then 20 decode steps: equal to the oracle
    forward over the 170 tokens."""
    window, T0, steps = 64, 150, 20
    w = workloads.TRAIN_FWD.with_shape(B=2, T=T0 + steps, D=512)
    p = workloads.make_mqa_inputs(w, window)
    io = TORCH_IO[w.io]
    Wqkv, Wo = _weights(p, w.io)
    x = dev(p["x"], io)
    out0, k, v = lib.mqa_forward(x[:, :T0].contiguous(), Wqkv, Wo, window, 0, with_kv=True)
    kc = torch.zeros((2, window, 128), dtype=io, device="cuda")
    vc = torch.zeros_like(kc)
    last = torch.arange(T0 - window, T0, device="cuda")
    kc[:, last % window] = k[:, last]
    vc[:, last % window] = v[:, last]
    ws = lib.workspace(lib.mqa_decode_workspace_bytes(2, w.D, io))
    outs = []
    for t in range(T0, T0 + steps):
        pos = torch.full((2,), t, dtype=torch.int32, device="cuda")
        o = torch.empty((2, w.D), dtype=io, device="cuda")
        lib.local_mqa_decode_step(pos, x[:, t].contiguous(), Wqkv, Wo, kc, vc, o, ws)
        outs.append(o)
    torch.cuda.synchronize()
    f = oracle.local_mqa_forward(p["x"], p["W_q"], p["W_k"], p["W_v"], p["W_o"], window, "bf16")
    e0, e1 = err(host(out0), f[:, :T0]), err(host(torch.stack(outs, 1)), f[:, T0:])
    print(f"prefill->decode err(prefill)={e0:.3e} err(decode)={e1:.3e}", flush=True)
    assert e0 <= TOL["bf16"] and e1 <= TOL["bf16"]


@pytest.mark.timeout(600)
def test_decode_full_shape_sampled_sequences(lib):
    """B=256, D=2560 (20 heads), window 1024, seeded positions in [0, 3000) and random bf16
    caches: one step, 6 sequences against the oracle's decode step."""
    B, D, window = 256, 2560, 1024
    w = workloads.DECODE.with_shape(T=1, decode=False)
    p = workloads.make_mqa_inputs(w, window)
    rng = np.random.default_rng(31)
    pos = rng.integers(0, 3000, size=B).astype(np.int32)
    pos[:3] = [0, 1023, 1024]
    kc0 = workloads.bf16_round(rng.standard_normal((B, window, 128)).astype(np.float32))
    vc0 = workloads.bf16_round(rng.standard_normal((B, window, 128)).astype(np.float32))
    io = torch.bfloat16
    Wqkv, Wo = _weights(p, "bf16")
    kc, vc = dev(kc0, io), dev(vc0, io)
    out = torch.empty((B, D), dtype=io, device="cuda")
    ws = lib.workspace(lib.mqa_decode_workspace_bytes(B, D, io))
    lib.local_mqa_decode_step(torch.from_numpy(pos).to("cuda"), dev(p["x"][:, 0], io), Wqkv, Wo, kc, vc,
                              out, ws)
    torch.cuda.synchronize()
    sel = np.array([0, 1, 2, 77, 200, 255])
    o, kco, vco = oracle.local_mqa_decode_step(p["x"][sel, 0], p["W_q"], p["W_k"], p["W_v"], p["W_o"],
                                               kc0[sel], vc0[sel], pos[sel], window, "bf16")
    e = err(host(out)[sel], o)
    ek = err(host(kc)[sel], kco)
    print(f"full decode err(out)={e:.3e} err(kcache)={ek:.3e}", flush=True)
    assert e <= TOL["bf16"] and ek <= TOL["bf16"]
