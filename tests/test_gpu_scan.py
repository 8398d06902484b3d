"""The forward scan's look-back computed both ways: from the summaries other workgroups
publish, and from memory when a predecessor chunk's summary is missing (the path that keeps
the chained scan (the blog page "Griffin's Compromise", "Term explanation: Parallel scan")
independent of the order in which the GPU starts workgroups).  The test-only entry points
(rglru_testing.h) force the second path for every chunk; the results must be bitwise the
same as the normal ones (the carry is canonical), and both must match the oracle.
"""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import TOL, device_inputs, err, host, make, oracle_forward

pytestmark = pytest.mark.gpu


def _split_scan(g, p, d, conv=True, knobs=None):
    """conv -> rglru_gates -> rglru_scan (rglru_testing_scan with `knobs`); returns (y, h_T)
    on the host."""
    u = torch.empty_like(d["x"])
    a = torch.empty(d["x"].shape, dtype=torch.float32, device="cuda")
    beta = torch.empty_like(a)
    y = torch.empty_like(d["x"])
    B, T, D = d["x"].shape
    hT = torch.empty((B, D), dtype=torch.float32, device="cuda")
    ws = g.workspace(g.scan_workspace_bytes(B, T, D, d["x"].dtype))
    if conv:
        g.conv1d_causal4(d["x"], d["conv_w"], d["conv_b"], d["conv_state"], u, None)
    else:
        u = d["x"]
    g.rglru_gates(u, d["W_a"], d["W_x"], d["b_a"], d["b_x"], d["lam"], a, beta, p["c"])
    args = (d["x"], d["conv_w"] if conv else None, d["conv_b"] if conv else None,
            d["conv_state"] if conv else None, a, beta, d["h0"], y, hT, ws)
    if knobs is None:
        g.rglru_scan(*args)
    else:
        from gated_linear_rnn_amd import testing
        testing.rglru_scan(knobs, *args)
    torch.cuda.synchronize()
    return host(y), host(hT)


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("conv", [True, False])
def test_direct_summaries_give_the_same_bits(lib, io, conv):
    # T = 333: six 64-step chunks, the last one partial
    p = make(workloads.TRAIN_FWD, B=2, T=333, D=128, io=io, h0="normal", history="normal")
    d = device_inputs(p)
    from gated_linear_rnn_amd import testing
    y0, h0 = _split_scan(lib, p, d, conv)
    # every summary computed from memory; computed whenever not yet published
    y1, h1 = _split_scan(lib, p, d, conv, testing.knobs(scan_direct_polls=-1))
    y2, h2 = _split_scan(lib, p, d, conv, testing.knobs(scan_direct_polls=0))
    np.testing.assert_array_equal(y0, y1)
    np.testing.assert_array_equal(h0, h1)
    np.testing.assert_array_equal(y0, y2)
    np.testing.assert_array_equal(h0, h2)
    o = oracle_forward(p, conv=conv)
    ey, eh = err(y0, o["y"]), err(h0, o["h_T"])
    print(f"direct look-back io={io} conv={conv} err(y)={ey:.2e} err(h_T)={eh:.2e}", flush=True)
    assert ey <= TOL[io] and eh <= TOL[io]


def test_backward_with_direct_summaries_gives_the_same_bits(lib):
    """rglru_bwd recomputes every state with the forward scan (gates from r and i): its
    gradients must not depend on how the look-back found its summaries."""
    p = workloads.make_inputs(workloads.TRAIN_BWD.with_shape(B=2, T=200, D=128))
    d = device_inputs(p)
    args = (d["x"], d["conv_w"], d["conv_b"], None, d["W_a"], d["W_x"], d["b_a"], d["b_x"],
            d["lam"], None, d["dy"])
    names = ["dx", "dconv_w", "dconv_b", "dW_a", "dW_x", "db_a", "db_x", "dlambda", "dh0"]
    from gated_linear_rnn_amd import testing
    g0 = lib.backward(*args, c=p["c"])
    g1, _ = testing.backward(testing.knobs(scan_direct_polls=-1), *args, c=p["c"])
    torch.cuda.synchronize()
    for n in names:
        assert torch.equal(g0[n], g1[n]), n


def test_full_size_scan_sampled_channels(lib):
    """B=8, T=2048, D=2560 (the training workload) through conv -> gates -> scan: y and h_T
    on a seeded subset of channels against the oracle on those channels."""
    from gpu_util import sample_channels
    w = workloads.TRAIN_FWD
    p = workloads.make_inputs(w)
    d = device_inputs(p)
    y, hT = _split_scan(lib, p, d)
    ch = sample_channels(w.D, 24, seed=5)
    o = oracle_forward(p, channels=ch)
    ey, eh = err(y[:, :, ch], o["y"]), err(hT[:, ch], o["h_T"])
    print(f"full-size split scan err(y)={ey:.2e} err(h_T)={eh:.2e}", flush=True)
    assert ey <= TOL["bf16"] and eh <= TOL["bf16"]


EDGES = [
    # (io, B, T, D): one step, two steps, exactly one 64-step chunk, one chunk and one step,
    # two full chunks, the largest tile count along T among the small cases
    ("bf16", 1, 1, 64), ("bf16", 2, 2, 64), ("bf16", 1, 64, 128), ("bf16", 2, 65, 64),
    ("bf16", 1, 128, 192), ("f32", 1, 3, 64), ("f32", 2, 129, 64), ("bf16", 3, 1000, 64),
]


@pytest.mark.parametrize("io,B,T,D", EDGES, ids=[f"{io}-{B}x{T}x{D}" for io, B, T, D in EDGES])
def test_split_scan_edge_lengths(lib, io, B, T, D):
    p = make(workloads.TRAIN_FWD, B=B, T=T, D=D, io=io, h0="normal", history="normal")
    d = device_inputs(p)
    y, hT = _split_scan(lib, p, d)
    o = oracle_forward(p)
    ey, eh = err(y, o["y"]), err(hT, o["h_T"])
    print(f"split scan io={io} {B}x{T}x{D} err(y)={ey:.2e} err(h_T)={eh:.2e}", flush=True)
    assert ey <= TOL[io] and eh <= TOL[io]


def test_direct_summaries_over_a_long_chain(lib):
    """T = 2500: 40 chunks, so a look-back can collect more summaries than its 16-entry
    window (the rest are read again, or computed again, on the way forward)."""
    p = make(workloads.TRAIN_FWD, B=1, T=2500, D=64, h0="normal", history="normal")
    d = device_inputs(p)
    from gated_linear_rnn_amd import testing
    y0, h0 = _split_scan(lib, p, d)
    y1, h1 = _split_scan(lib, p, d, knobs=testing.knobs(scan_direct_polls=-1))
    np.testing.assert_array_equal(y0, y1)
    np.testing.assert_array_equal(h0, h1)
    o = oracle_forward(p)
    ey, eh = err(y0, o["y"]), err(h0, o["h_T"])
    print(f"long chain err(y)={ey:.2e} err(h_T)={eh:.2e}", flush=True)
    assert ey <= TOL["bf16"] and eh <= TOL["bf16"]
