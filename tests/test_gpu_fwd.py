"""Forward parity of the HIP path (conv -> gate GEMM -> chunked scan) with the oracle.

Element-by-element at sizes the oracle finishes in seconds (several GEMM tiles of 256 rows
and 128 channels, several scan tiles of 128 steps, ragged tails), and at the full workload
sizes on a seeded channel subset (channels are independent through the diagonal
recurrence, so the oracle evaluates only those channels exactly).
"""
import numpy as np
import pytest

import workloads
from gpu_util import TOL, device_inputs, err, gpu_forward, make, oracle_forward, sample_channels

pytestmark = pytest.mark.gpu


def _forced_fused(d, c, conv=True):
    """The forward with the bf16 RG-LRU layer in the fused kernel whatever the shape (the
    test-only entry point; the public call picks the form by shape)."""
    import torch
    from gated_linear_rnn_amd import testing
    from gpu_util import host
    y, hT, cso, _ = testing.forward(testing.knobs(lru_force_fused=1), d["x"],
                                    d["conv_w"] if conv else None, d["conv_b"] if conv else None,
                                    d["conv_state"] if conv else None, d["W_a"], d["W_x"],
                                    d["b_a"], d["b_x"], d["lam"], d["h0"], c)
    torch.cuda.synchronize()
    return host(y), host(hT), None if cso is None else host(cso)


def _check(g, p, conv=True, channels=None, what="", fused=False):
    io = p["workload"].io
    d = device_inputs(p)
    if fused:
        y, hT, cso = _forced_fused(d, p["c"], conv=conv)
        what = what + " (fused)"
    else:
        y, hT, cso = gpu_forward(g, d, p["c"], conv=conv)
    o = oracle_forward(p, channels=channels, conv=conv)
    S = slice(None) if channels is None else channels
    ey, eh = err(y[:, :, S], o["y"]), err(hT[:, S], o["h_T"])
    print(f"{what} io={io} shape={p['x'].shape} err(y)={ey:.3e} err(h_T)={eh:.3e}", flush=True)
    assert ey <= TOL[io] and eh <= TOL[io]
    if conv:
        np.testing.assert_array_equal(cso, o["conv_state_out"])   # a copy of inputs: exact


SMALL = [
    # (workload recipe, B, T, D)
    (workloads.TINY_F32, 1, 256, 256),
    (workloads.TINY_F32, 2, 300, 192),
    (workloads.TINY_F32, 1, 1, 64),
    (workloads.TINY_F32, 3, 5, 128),
    (workloads.TRAIN_FWD, 2, 700, 384),
    (workloads.TRAIN_FWD, 4, 130, 64),
    (workloads.TRAIN_FWD, 1, 2, 64),
    (workloads.LONG_FWD, 1, 3000, 256),
    (workloads.TRAIN_BWD, 1, 257, 320),
]


@pytest.mark.parametrize("w,B,T,D", SMALL, ids=[f"{w.io}-{B}x{T}x{D}" for w, B, T, D in SMALL])
def test_forward_small_elementwise(lib, w, B, T, D):
    p = make(w, B=B, T=T, D=D)
    _check(lib, p, what=w.name)
    if w.io == "bf16":   # small bf16 shapes take the unfused form: check the fused kernel too
        _check(lib, p, what=w.name, fused=True)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_forward_with_conv_state_and_h0(lib, io):
    w = workloads.TRAIN_FWD.with_shape(B=2, T=333, D=128, io=io, h0="normal", history="normal")
    p = workloads.make_inputs(w)
    p["conv_b"] = np.random.default_rng(0).standard_normal(128).astype(np.float32) * 0.1
    _check(lib, p, what="state")
    if io == "bf16":
        _check(lib, p, what="state", fused=True)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_forward_without_conv(lib, io):
    p = make(workloads.TRAIN_FWD, B=2, T=200, D=128, io=io)
    _check(lib, p, conv=False, what="noconv")
    if io == "bf16":
        _check(lib, p, conv=False, what="noconv", fused=True)


def test_f32_gates_formed_in_the_scan(lib):
    """fp32 forward whose scan fills the CUs (2 x 9 channel tiles x 16 chunks = 288
    workgroups): the projections go straight to the scan, which forms the gates itself;
    the same bits whether chunk carries come from published summaries or from memory."""
    import torch
    from gated_linear_rnn_amd import testing
    from gpu_util import host
    p = make(workloads.TRAIN_FWD, B=2, T=1000, D=576, io="f32", h0="normal", history="normal")
    _check(lib, p, what="gates-in-scan")
    d = device_inputs(p)
    args = (d["x"], d["conv_w"], d["conv_b"], d["conv_state"], d["W_a"], d["W_x"], d["b_a"],
            d["b_x"], d["lam"], d["h0"], p["c"])
    outs = []
    for polls in (2048, -1, 0):
        y, hT, _, _ = testing.forward(testing.knobs(scan_direct_polls=polls), *args)
        torch.cuda.synchronize()
        outs.append((host(y), host(hT)))
    for y, hT in outs[1:]:
        np.testing.assert_array_equal(y, outs[0][0])
        np.testing.assert_array_equal(hT, outs[0][1])


@pytest.mark.parametrize("B,T,D", [(2, 2049, 704), (1, 4000, 64)])
def test_f32_long_sequences(lib, B, T, D):
    """fp32 I/O over thousands of steps with slowly decaying gates (a^c in [0.999, 0.9999]),
    where a rounding bias in a_t would compound along the recurrence: 2 x 2049 x 704 forms
    the gates inside the scan, 1 x 4000 x 64 (63 scan workgroups) in the elementwise
    launch.  Every element against the oracle."""
    p = make(workloads.LONG_FWD, B=B, T=T, D=D, io="f32", h0="normal", history="normal")
    _check(lib, p, what="f32-long")


def test_tiny_f32_workload_full(lib):
    p = workloads.make_inputs(workloads.TINY_F32)
    _check(lib, p, what="tiny")


def _one_sequence(p, b):
    """The inputs of sequence b alone (sequences are independent: the recurrence is per
    (sequence, channel) and the gate projection per (sequence, step))."""
    q = dict(p)
    for k in ("x", "conv_state", "h0"):
        if q.get(k) is not None:
            q[k] = q[k][b:b + 1]
    return q


@pytest.mark.timeout(900)
@pytest.mark.parametrize("w", [workloads.TRAIN_FWD, workloads.LONG_FWD, workloads.TRAIN_BWD],
                         ids=lambda w: w.name)
def test_forward_full_size(lib, w):
    """The full workload in one call: a seeded channel subset of every sequence, and every
    channel of one whole sequence (all channel tiles and time tiles of the fused kernel)."""
    p = workloads.make_inputs(w)
    d = device_inputs(p)
    y, hT, _ = gpu_forward(lib, d, p["c"])
    S = sample_channels(w.D, 40, seed=w.seed)
    o = oracle_forward(p, channels=S)
    ey, eh = err(y[:, :, S], o["y"]), err(hT[:, S], o["h_T"])
    print(f"{w.name} channel subset ({len(S)} of {w.D}) err(y)={ey:.3e} err(h_T)={eh:.3e}", flush=True)
    assert ey <= TOL[w.io] and eh <= TOL[w.io]
    b = w.B - 1
    del o
    o = oracle_forward(_one_sequence(p, b))
    ey, eh = err(y[b:b + 1], o["y"]), err(hT[b:b + 1], o["h_T"])
    print(f"{w.name} sequence {b}, all {w.D} channels err(y)={ey:.3e} err(h_T)={eh:.3e}", flush=True)
    assert ey <= TOL[w.io] and eh <= TOL[w.io]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("B,T,D", [(2, 2048, 4608), (3, 1700, 2752), (1, 512, 2560),
                                   (8, 512, 2560)])
def test_forward_where_fused_rounds_fill_poorly(lib, B, T, D):
    """The forward's form by shape: shapes whose fused tiles (256 steps x 128 channels)
    leave the last of their rounds of 256 CUs at most 60% full run as the gate GEMM with its
    split-K tail, then the scan (2 x 8 x 36 = 576 tiles: a quarter-full third round; 1 x 2 x 20
    = 40 tiles; 8 x 2 x 20 = 320 tiles: a quarter-full second round); 3 x 7 x 22 = 462 tiles
    fill their second round to 80% and stay fused.  Every channel of every sequence against
    the oracle in both forms, and bitwise repeatable."""
    import torch
    p = make(workloads.TRAIN_BWD, B=B, T=T, D=D, h0="normal", history="normal")
    _check(lib, p, what=f"rounds {B}x{T}x{D}")
    _check(lib, p, what=f"rounds {B}x{T}x{D}", fused=True)
    d = device_inputs(p)
    y1, h1, _ = gpu_forward(lib, d, p["c"])
    y2, h2, _ = gpu_forward(lib, d, p["c"])
    assert np.array_equal(y1, y2) and np.array_equal(h1, h2)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_forward_as_conv_gates_scan(lib, io):
    """rglru_fwd split into its three entry points (the benchmark's timed step)."""
    import oracle
    import torch
    from gpu_util import host
    p = make(workloads.TRAIN_FWD, B=2, T=500, D=192, io=io, h0="normal", history="normal")
    d = device_inputs(p)
    u = torch.empty_like(d["x"])
    a = torch.empty(d["x"].shape, dtype=torch.float32, device="cuda")
    beta = torch.empty_like(a)
    y = torch.empty_like(d["x"])
    hT = torch.empty_like(d["h0"])
    ws = lib.workspace(lib.scan_workspace_bytes(2, 500, 192, d["x"].dtype))
    lib.conv1d_causal4(d["x"], d["conv_w"], d["conv_b"], d["conv_state"], u, None)
    lib.rglru_gates(u, d["W_a"], d["W_x"], d["b_a"], d["b_x"], d["lam"], a, beta, p["c"])
    lib.rglru_scan(d["x"], d["conv_w"], d["conv_b"], d["conv_state"], a, beta, d["h0"], y, hT, ws)
    torch.cuda.synchronize()
    o = oracle_forward(p)
    ok = oracle_forward(p, keep=True)
    assert err(host(a), ok["a"]) <= 1e-5 and err(host(beta), ok["m"] * ok["i"]) <= 1e-5
    ey, eh = err(host(y), o["y"]), err(host(hT), o["h_T"])
    print(f"split io={io} err(a)={err(host(a), ok['a']):.2e} err(y)={ey:.2e} err(h_T)={eh:.2e}")
    assert ey <= TOL[io] and eh <= TOL[io]


@pytest.mark.parametrize("io,B,T,D", [("bf16", 2, 700, 384), ("bf16", 3, 257, 192), ("bf16", 1, 1, 64),
                                      ("bf16", 2, 513, 320), ("f32", 2, 300, 128)])
def test_lru_layer_on_conv_output(lib, io, B, T, D):
    """conv1d_causal4 then rglru_lru (the RG-LRU layer alone) equals the full forward."""
    import torch
    from gpu_util import host
    p = make(workloads.TRAIN_FWD, B=B, T=T, D=D, io=io, h0="normal", history="normal")
    d = device_inputs(p)
    u = torch.empty_like(d["x"])
    y = torch.empty_like(d["x"])
    hT = torch.empty_like(d["h0"])
    ws = lib.workspace(lib.lru_workspace_bytes(B, T, D, d["x"].dtype))
    lib.conv1d_causal4(d["x"], d["conv_w"], d["conv_b"], d["conv_state"], u, None)
    lib.rglru_lru(u, d["W_a"], d["W_x"], d["b_a"], d["b_x"], d["lam"], d["h0"], y, hT, ws, p["c"])
    torch.cuda.synchronize()
    o = oracle_forward(p)
    ey, eh = err(host(y), o["y"]), err(host(hT), o["h_T"])
    print(f"lru io={io} shape={(B, T, D)} err(y)={ey:.2e} err(h_T)={eh:.2e}")
    assert ey <= TOL[io] and eh <= TOL[io]
