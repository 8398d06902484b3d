"""Parity over seeded random shapes: the public forward (and, where small, the backward)
against the oracle on shapes drawn across both I/O dtypes, every workload recipe's gate
range, ragged and very short sequences (T = 1, 2, 3 and tile edges), one to twelve channel
tiles, with and without the conv, h0, the conv history, the conv bias and dh_T.

Each case is its own test id, so a failure names its shape; the draws are fixed by the case
index, so a failing case replays exactly.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import TOL, device_inputs, err, gpu_forward, host, oracle_forward

pytestmark = pytest.mark.gpu

NAMES = ["dx", "dconv_w", "dconv_b", "dW_a", "dW_x", "db_a", "db_x", "dlambda", "dh0"]
RECIPES = [workloads.TINY_F32, workloads.TRAIN_FWD, workloads.LONG_FWD, workloads.TRAIN_BWD]
N_CASES = 48


def _case(k):
    """Shape and options of case k (a pure function of k)."""
    rng = np.random.default_rng(1000 + k)
    io = ["f32", "bf16"][k % 2]
    B = int(rng.integers(1, 7))
    D = 64 * int(rng.integers(1, 13))
    T = int(rng.choice([1, 2, 3, 63, 64, 65, 255, 256, 257, 511, 700, 1025, 2049,
                        int(rng.integers(1, 3000))]))
    while B * T * D > 3_000_000:          # sizes the oracle finishes in about a second
        T = max(1, T // 2)
    return dict(io=io, B=B, T=T, D=D, recipe=RECIPES[int(rng.integers(0, 4))],
                h0=["zero", "normal"][int(rng.integers(0, 2))],
                history=["zero", "normal"][int(rng.integers(0, 2))],
                conv=bool(rng.integers(0, 4) > 0), bias=bool(rng.integers(0, 2)),
                dhT=bool(rng.integers(0, 2)), seed=int(rng.integers(0, 2 ** 31)))


def _id(k):
    c = _case(k)
    return f"{k}-{c['io']}-{c['B']}x{c['T']}x{c['D']}"


@pytest.mark.parametrize("k", range(N_CASES), ids=[_id(k) for k in range(N_CASES)])
def test_random_shape(lib, k):
    c = _case(k)
    io, B, T, D, conv = c["io"], c["B"], c["T"], c["D"], c["conv"]
    bwd = B * T * D <= 400_000
    w = c["recipe"].with_shape(B=B, T=T, D=D, io=io, h0=c["h0"], history=c["history"],
                               with_dy=bwd)
    p = workloads.make_inputs(w)
    rng = np.random.default_rng(c["seed"])
    if c["bias"]:
        p["conv_b"] = rng.standard_normal(D).astype(np.float32) * 0.1
    d = device_inputs(p)
    print(f"case {k}: {c}", flush=True)
    y, hT, cso = gpu_forward(lib, d, p["c"], conv=conv)
    o = oracle_forward(p, conv=conv)
    ey, eh = err(y, o["y"]), err(hT, o["h_T"])
    print(f"  forward err(y)={ey:.2e} err(h_T)={eh:.2e}", flush=True)
    assert ey <= TOL[io] and eh <= TOL[io]
    if conv:
        np.testing.assert_array_equal(cso, o["conv_state_out"])
    if not bwd:
        return
    dhT = rng.standard_normal((B, D)) if c["dhT"] else None
    dhT_d = None if dhT is None else torch.from_numpy(dhT.astype(np.float32)).cuda()
    got = lib.backward(d["x"], d["conv_w"] if conv else None, d["conv_b"] if conv else None,
                       d["conv_state"] if conv else None, d["W_a"], d["W_x"], d["b_a"], d["b_x"],
                       d["lam"], d["h0"], d["dy"], dhT_d, p["c"])
    torch.cuda.synchronize()
    want = oracle.backward(p["x"], p["conv_w"] if conv else None, p["conv_b"] if conv else None,
                           p["conv_state"] if conv else None, p["W_a"], p["W_x"], p["b_a"],
                           p["b_x"], p["lam"], p["h0"], p["c"], io, p["dy"], dhT)
    errs = {n: err(host(got[n]), want[n]) for n in NAMES if want[n] is not None}
    print("  backward " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()), flush=True)
    for n, e in errs.items():
        assert e <= TOL[io], (n, e)
