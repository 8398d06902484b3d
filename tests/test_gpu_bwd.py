"""Backward parity (rglru_bwd) with the oracle's chain-rule gradients, element by element,
at small shapes and at the full fwd+bwd training workload (4 x 2048 x 5376, bf16)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import TOL, device_inputs, err, host

pytestmark = pytest.mark.gpu

NAMES = ["dx", "dconv_w", "dconv_b", "dW_a", "dW_x", "db_a", "db_x", "dlambda", "dh0"]


def _check(g, p, dh_T=None, conv=True, what=""):
    w = p["workload"]
    d = device_inputs(p)
    dhT_d = None if dh_T is None else torch.from_numpy(dh_T.astype(np.float32)).cuda()
    got = g.backward(d["x"], d["conv_w"] if conv else None, d["conv_b"] if conv else None,
                     d["conv_state"] if conv else None, d["W_a"], d["W_x"], d["b_a"], d["b_x"],
                     d["lam"], d["h0"], d["dy"], dhT_d, p["c"])
    torch.cuda.synchronize()
    want = oracle.backward(p["x"], p["conv_w"] if conv else None, p["conv_b"] if conv else None,
                           p["conv_state"] if conv else None, p["W_a"], p["W_x"], p["b_a"],
                           p["b_x"], p["lam"], p["h0"], p["c"], w.io, p["dy"], dh_T)
    errs = {}
    for n in NAMES:
        if want[n] is None:
            continue
        errs[n] = err(host(got[n]), want[n])
    print(f"{what} io={w.io} shape={p['x'].shape} " +
          " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    for n, e in errs.items():
        assert e <= TOL[w.io], (n, e)
    return got


SMALL = [
    (workloads.TINY_F32, 1, 64, 64),
    (workloads.TINY_F32, 2, 200, 128),
    (workloads.TRAIN_BWD, 2, 300, 192),
    (workloads.TRAIN_BWD, 1, 130, 64),
    (workloads.TRAIN_BWD, 3, 1, 64),
]


@pytest.mark.parametrize("w,B,T,D", SMALL, ids=[f"{w.io}-{B}x{T}x{D}" for w, B, T, D in SMALL])
def test_backward_small_elementwise(lib, w, B, T, D):
    p = workloads.make_inputs(w.with_shape(B=B, T=T, D=D, with_dy=True))
    _check(lib, p, what="small")


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_backward_with_state_h0_and_dhT(lib, io):
    w = workloads.TRAIN_BWD.with_shape(B=2, T=257, D=128, io=io, h0="normal", history="normal")
    p = workloads.make_inputs(w)
    p["conv_b"] = np.random.default_rng(1).standard_normal(128).astype(np.float32) * 0.1
    dh_T = np.random.default_rng(2).standard_normal((2, 128))
    _check(lib, p, dh_T=dh_T, what="state")


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_backward_without_conv(lib, io):
    p = workloads.make_inputs(workloads.TRAIN_BWD.with_shape(B=2, T=150, D=128, io=io))
    _check(lib, p, conv=False, what="noconv")


def test_backward_is_bitwise_reproducible(lib):
    p = workloads.make_inputs(workloads.TRAIN_BWD.with_shape(B=2, T=300, D=192))
    d = device_inputs(p)
    args = (d["x"], d["conv_w"], d["conv_b"], None, d["W_a"], d["W_x"], d["b_a"], d["b_x"],
            d["lam"], None, d["dy"])
    g1 = lib.backward(*args, c=p["c"])
    g2 = lib.backward(*args, c=p["c"])
    torch.cuda.synchronize()
    for n in NAMES:
        assert torch.equal(g1[n], g2[n]), n


@pytest.mark.timeout(900)
def test_backward_full_training_workload(lib):
    p = workloads.make_inputs(workloads.TRAIN_BWD)
    _check(lib, p, what="full")


# ---------------------------------------------------------------- training forward + saved backward
def _train_pair(g, p, conv=True, dh_T=None):
    """rglru_fwd_train then rglru_bwd_saved, and rglru_bwd on the same inputs."""
    d = device_inputs(p)
    cw, cb, cs = (d["conv_w"], d["conv_b"], d["conv_state"]) if conv else (None, None, None)
    dhT_d = None if dh_T is None else torch.from_numpy(dh_T.astype(np.float32)).cuda()
    y, hT, cso, saved = g.forward_train(d["x"], cw, cb, cs, d["W_a"], d["W_x"], d["b_a"],
                                        d["b_x"], d["lam"], d["h0"], p["c"])
    got = g.backward(d["x"], cw, cb, cs, d["W_a"], d["W_x"], None, None, d["lam"], d["h0"],
                     d["dy"], dhT_d, p["c"], saved=saved)
    ref = g.backward(d["x"], cw, cb, cs, d["W_a"], d["W_x"], d["b_a"], d["b_x"], d["lam"],
                     d["h0"], d["dy"], dhT_d, p["c"])
    torch.cuda.synchronize()
    return (y, hT, cso), got, ref


TRAIN = [
    (workloads.TINY_F32, 2, 200, 128, True),
    (workloads.TRAIN_BWD, 2, 300, 192, True),
    (workloads.TRAIN_BWD, 1, 130, 64, False),
    (workloads.TRAIN_BWD, 3, 1, 64, True),
]


@pytest.mark.parametrize("w,B,T,D,conv", TRAIN,
                         ids=[f"{w.io}-{B}x{T}x{D}-{'conv' if cv else 'noconv'}" for w, B, T, D, cv in TRAIN])
def test_train_forward_matches_oracle_and_saved_backward_matches_bwd(lib, w, B, T, D, conv):
    wl = w.with_shape(B=B, T=T, D=D, with_dy=True, h0="normal", history="normal")
    p = workloads.make_inputs(wl)
    dh_T = np.random.default_rng(3).standard_normal((B, D))
    (y, hT, cso), got, ref = _train_pair(lib, p, conv=conv, dh_T=dh_T)
    from gpu_util import oracle_forward
    want = oracle_forward(p, conv=conv)
    e = {"y": err(host(y), want["y"]), "h_T": err(host(hT), want["h_T"])}
    if conv:
        e["conv_state"] = err(host(cso), want["conv_state_out"])
    print(f"train fwd io={w.io} shape={p['x'].shape} " + " ".join(f"{k}={v:.2e}" for k, v in e.items()),
          flush=True)
    for k, v in e.items():
        assert v <= TOL[w.io], (k, v)
    if conv:
        assert e["conv_state"] == 0.0
    for n in NAMES:
        if ref[n] is None:
            assert got[n] is None
            continue
        assert torch.equal(got[n], ref[n]), n


def test_saved_backward_rejects_short_saved_buffer(lib):
    p = workloads.make_inputs(workloads.TRAIN_BWD.with_shape(B=1, T=64, D=64, with_dy=True))
    d = device_inputs(p)
    _, _, _, saved = lib.forward_train(d["x"], d["conv_w"], d["conv_b"], None, d["W_a"], d["W_x"],
                                       d["b_a"], d["b_x"], d["lam"], None, p["c"])
    with pytest.raises(lib.RgluError):
        lib.backward(d["x"], d["conv_w"], d["conv_b"], None, d["W_a"], d["W_x"], None, None,
                     d["lam"], None, d["dy"], None, p["c"], saved=saved[:-16])


@pytest.mark.timeout(900)
def test_saved_backward_full_training_workload_equals_bwd(lib):
    """At 4 x 2048 x 5376: rglru_bwd_saved gives rglru_bwd's gradients bit for bit (those
    are checked against the oracle element by element above), and rglru_fwd_train's y on
    every channel of one sequence matches the oracle."""
    p = workloads.make_inputs(workloads.TRAIN_BWD)
    (y, hT, _), got, ref = _train_pair(lib, p)
    for n in NAMES:
        assert torch.equal(got[n], ref[n]), n
    from gpu_util import oracle_forward
    b = 3
    q = dict(p)
    q["x"] = p["x"][b:b + 1]
    q["conv_state"] = None if p["conv_state"] is None else p["conv_state"][b:b + 1]
    q["h0"] = None if p["h0"] is None else p["h0"][b:b + 1]
    want = oracle_forward(q)
    e_y = err(host(y)[b:b + 1], want["y"])
    e_h = err(host(hT)[b:b + 1], want["h_T"])
    print(f"train fwd full b={b} err(y)={e_y:.2e} err(h_T)={e_h:.2e}", flush=True)
    assert e_y <= TOL["bf16"] and e_h <= TOL["bf16"]
