"""Decode-step parity: the fixed-size state (conv history [B,3,D] and h [B,D]) carried
through consecutive single-token steps (the blog page "Griffin's Compromise", section
"Hawk": generation reads and writes only the current token and a fixed-size state)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import TOL, TORCH_IO, dev, err, host, sample_channels

pytestmark = pytest.mark.gpu


def _run(g, p, steps, channels=None, conv=True, rows=None):
    """Run `steps` decode steps on the GPU; compare every y_t (and the final state) with the
    oracle, restricted to `channels` when given.  `rows`: sequences that are also compared
    on every channel (sequences are independent, so the oracle runs on those rows alone)."""
    w = p["workload"]
    io = TORCH_IO[w.io]
    B, D = w.B, w.D
    S = np.arange(D) if channels is None else channels
    St = torch.from_numpy(S).cuda()
    R = np.arange(0) if rows is None else np.asarray(rows)
    Rt = torch.from_numpy(R).cuda()
    x = dev(p["x"][:steps], io)                        # [steps, B, D]
    cw = dev(p["conv_w"], io) if conv else None
    cb = dev(p["conv_b"]) if conv else None
    hist = dev(p["conv_state"], io)
    Wa, Wx, ba, bx, lam = (dev(p["W_a"], io), dev(p["W_x"], io), dev(p["b_a"]), dev(p["b_x"]),
                           dev(p["lam"]))
    h = dev(p["h0"])
    ws = g.workspace(g.decode_workspace_bytes(B, D, io))
    ys = torch.empty((steps, B, len(S)), dtype=torch.float32, device="cuda")
    yr = torch.empty((steps, len(R), D), dtype=torch.float32, device="cuda")
    y_t = torch.empty((B, D), dtype=io, device="cuda")
    for t in range(steps):
        g.rglru_decode_step(x[t], cw, cb, hist, Wa, Wx, ba, bx, lam, h, y_t, ws, p["c"])
        ys[t] = y_t.float().index_select(1, St)
        if len(R):
            yr[t] = y_t.float().index_select(0, Rt)
    torch.cuda.synchronize()
    # oracle, channel subset: the conv history is kept for every channel (the gates read all
    # of u), the state only matters on S
    hist_o = p["conv_state"].astype(np.float64)
    h_o = p["h0"].astype(np.float64).copy()
    worst = 0.0
    for t in range(steps):
        o = oracle.forward(p["x"][t][:, None, :], p["conv_w"] if conv else None,
                           p["conv_b"] if conv else None, hist_o if conv else None, p["W_a"],
                           p["W_x"], p["b_a"], p["b_x"], p["lam"], h_o, p["c"], w.io, channels=S)
        worst = max(worst, err(host(ys[t]), o["y"][:, 0, :]))
        h_o[:, S] = o["h_T"]
        if conv:
            hist_o = o["conv_state_out"]
    eh = err(host(h)[:, S], h_o[:, S])
    print(f"decode io={w.io} B={B} D={D} steps={steps} err(y)={worst:.3e} err(h)={eh:.3e}", flush=True)
    assert worst <= TOL[w.io] and eh <= TOL[w.io]
    if conv:
        np.testing.assert_array_equal(host(hist), hist_o)
    if len(R):
        hist_r = p["conv_state"][R].astype(np.float64)
        h_r = p["h0"][R].astype(np.float64).copy()
        worst_r = 0.0
        for t in range(steps):
            o = oracle.forward(p["x"][t][R][:, None, :], p["conv_w"] if conv else None,
                               p["conv_b"] if conv else None, hist_r if conv else None, p["W_a"],
                               p["W_x"], p["b_a"], p["b_x"], p["lam"], h_r, p["c"], w.io)
            worst_r = max(worst_r, err(host(yr[t]), o["y"][:, 0, :]))
            h_r = o["h_T"]
            if conv:
                hist_r = o["conv_state_out"]
        eh_r = err(host(h)[R], h_r)
        print(f"decode rows {R.tolist()}, all {D} channels: err(y)={worst_r:.3e} err(h)={eh_r:.3e}",
              flush=True)
        assert worst_r <= TOL[w.io] and eh_r <= TOL[w.io]


@pytest.mark.parametrize("io,B,D", [("f32", 3, 128), ("bf16", 16, 256), ("bf16", 5, 192),
                                    ("bf16", 300, 64)])
def test_decode_small_elementwise(lib, io, B, D):
    p = workloads.make_inputs(workloads.DECODE.with_shape(B=B, D=D, T=40, io=io))
    _run(lib, p, 40)


def test_decode_f32_many_steps(lib):
    """600 fp32 steps: the state carried in fp32 between steps, each step's gates formed in
    fp64 and rounded once, so no rounding bias of a_t compounds over the steps."""
    p = workloads.make_inputs(workloads.DECODE.with_shape(B=2, D=128, T=600, io="f32"))
    _run(lib, p, 600)


@pytest.mark.parametrize("B,D", [(1, 2560), (2, 192), (3, 320), (4, 256), (4, 4096)])
def test_decode_small_batch_single_launch(lib, B, D):
    """B <= 4 takes the one-launch matrix-vector form of the step (per-channel waves,
    u staged in LDS); every element of every step against the oracle."""
    p = workloads.make_inputs(workloads.DECODE.with_shape(B=B, D=D, T=12))
    _run(lib, p, 12)


def test_decode_small_batch_is_bitwise_reproducible(lib):
    p = workloads.make_inputs(workloads.DECODE.with_shape(B=3, D=640, T=4))
    io = TORCH_IO["bf16"]
    outs = []
    for _ in range(2):
        x = dev(p["x"], io)
        hist, h = dev(p["conv_state"], io), dev(p["h0"])
        y = torch.empty((3, 640), dtype=io, device="cuda")
        ws = lib.workspace(lib.decode_workspace_bytes(3, 640, io))
        for t in range(4):
            lib.rglru_decode_step(x[t], dev(p["conv_w"], io), dev(p["conv_b"]), hist,
                                  dev(p["W_a"], io), dev(p["W_x"], io), dev(p["b_a"]),
                                  dev(p["b_x"]), dev(p["lam"]), h, y, ws, p["c"])
        torch.cuda.synchronize()
        outs.append((y.clone(), h.clone(), hist.clone()))
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a, b)


def test_decode_without_conv(lib):
    p = workloads.make_inputs(workloads.DECODE.with_shape(B=4, D=128, T=10))
    _run(lib, p, 10, conv=False)


def test_decode_continues_forward(lib):
    """Prefill with rglru_fwd, then decode: equals one forward over the whole sequence
    (state consistency on streaming input)."""
    w = workloads.TRAIN_FWD.with_shape(B=2, T=150, D=128, h0="normal", history="normal")
    p = workloads.make_inputs(w)
    io = TORCH_IO[w.io]
    T1 = 140
    d = {k: dev(p[k], io) for k in ("x", "conv_w", "W_a", "W_x", "conv_state")}
    f = {k: dev(p[k]) for k in ("conv_b", "b_a", "b_x", "lam", "h0")}
    y1, hT, cso = lib.forward(d["x"][:, :T1].contiguous(), d["conv_w"], f["conv_b"], d["conv_state"],
                              d["W_a"], d["W_x"], f["b_a"], f["b_x"], f["lam"], f["h0"], p["c"])
    ws = lib.workspace(lib.decode_workspace_bytes(2, 128, io))
    ys = []
    y_t = torch.empty((2, 128), dtype=io, device="cuda")
    for t in range(T1, w.T):
        lib.rglru_decode_step(d["x"][:, t].contiguous(), d["conv_w"], f["conv_b"], cso, d["W_a"],
                              d["W_x"], f["b_a"], f["b_x"], f["lam"], hT, y_t, ws, p["c"])
        ys.append(host(y_t))
    torch.cuda.synchronize()
    o = oracle.forward(p["x"], p["conv_w"], p["conv_b"], p["conv_state"], p["W_a"], p["W_x"],
                       p["b_a"], p["b_x"], p["lam"], p["h0"], p["c"], w.io)
    assert err(host(y1), o["y"][:, :T1]) <= TOL[w.io]
    assert err(np.stack(ys, 1), o["y"][:, T1:]) <= TOL[w.io]
    assert err(host(hT), o["h_T"]) <= TOL[w.io]
    np.testing.assert_array_equal(host(cso), o["conv_state_out"])


@pytest.mark.timeout(900)
def test_decode_full_workload(lib):
    """All 1024 steps at B = 256, D = 2560: a channel subset of every sequence, and every
    channel of four sequences (first, last and two inside)."""
    p = workloads.make_inputs(workloads.DECODE)
    S = sample_channels(workloads.DECODE.D, 24, seed=5)
    _run(lib, p, workloads.DECODE.T, channels=S, rows=[0, 77, 128, workloads.DECODE.B - 1])


def test_decode_graph_replays_match_eager(lib):
    """A captured hipGraph of decode steps, replayed several times with eager work and
    synchronisations in between; every replay equals the eager run from the same state."""
    w = workloads.DECODE.with_shape(B=32, D=256, T=8)
    p = workloads.make_inputs(w)
    io = TORCH_IO[w.io]
    toks = dev(p["x"], io)
    cw, cb = dev(p["conv_w"], io), dev(p["conv_b"])
    Wa, Wx, ba, bx, lam = dev(p["W_a"], io), dev(p["W_x"], io), dev(p["b_a"]), dev(p["b_x"]), dev(p["lam"])
    hist0, h0 = dev(p["conv_state"], io), dev(p["h0"])
    hist, h = hist0.clone(), h0.clone()
    y = torch.empty((w.B, w.D), dtype=io, device="cuda")
    ws = lib.workspace(lib.decode_workspace_bytes(w.B, w.D, io))

    def run():
        for t in range(w.T):
            lib.rglru_decode_step(toks[t], cw, cb, hist, Wa, Wx, ba, bx, lam, h, y, ws, p["c"])

    run()                                           # eager reference from (hist0, h0)
    torch.cuda.synchronize()
    ref = (hist.clone(), h.clone(), y.clone())
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            run()
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(4):
        hist.copy_(hist0)
        h.copy_(h0)
        y.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(hist, ref[0]) and torch.equal(h, ref[1]) and torch.equal(y, ref[2]), rep
        _ = (toks.float() * 2).sum().item()         # unrelated eager work between replays
