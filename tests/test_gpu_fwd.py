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


def _check(g, p, conv=True, channels=None, what=""):
    io = p["workload"].io
    d = device_inputs(p)
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


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_forward_with_conv_state_and_h0(lib, io):
    w = workloads.TRAIN_FWD.with_shape(B=2, T=333, D=128, io=io, h0="normal", history="normal")
    p = workloads.make_inputs(w)
    p["conv_b"] = np.random.default_rng(0).standard_normal(128).astype(np.float32) * 0.1
    _check(lib, p, what="state")


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_forward_without_conv(lib, io):
    p = make(workloads.TRAIN_FWD, B=2, T=200, D=128, io=io)
    _check(lib, p, conv=False, what="noconv")


def test_tiny_f32_workload_full(lib):
    p = workloads.make_inputs(workloads.TINY_F32)
    _check(lib, p, what="tiny")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("w", [workloads.TRAIN_FWD, workloads.LONG_FWD, workloads.TRAIN_BWD],
                         ids=lambda w: w.name)
def test_forward_full_size_channel_subset(lib, w):
    p = workloads.make_inputs(w)
    S = sample_channels(w.D, 40, seed=w.seed)
    _check(lib, p, channels=S, what=w.name)


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
