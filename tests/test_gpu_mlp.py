"""Parity of the gated MLP block (gated_mlp_fwd: the first layer's two branches on the
matrix cores with GeLU(q1) q2 formed in the GEMM epilogue, then the last linear; the
Griffin model-architecture page, section "MLP block", Fig. 2(b)) with the oracle.

Element by element at sizes the oracle finishes in seconds (ragged row tiles, hidden widths
that are not multiples of the 128-channel tile, the pages' expansion M = 3 and others), and
at the full training shape on a seeded subset of rows (rows are independent through the
block, so the oracle evaluates only those rows).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import TOL, TORCH_IO, dev, err, host

pytestmark = pytest.mark.gpu


def _gpu(g, p):
    io = TORCH_IO[p["workload"].io]
    out = g.mlp_forward(dev(p["x"], io), dev(p["W_1"], io), dev(p["W_2"], io), dev(p["W_3"], io))
    torch.cuda.synchronize()
    return host(out)


SMALL = [
    # (workload recipe, B, T, D, expansion)
    (workloads.TINY_F32, 1, 256, 256, 3),
    (workloads.TINY_F32, 2, 300, 64, 3),
    (workloads.TINY_F32, 1, 1, 64, 1),
    (workloads.TRAIN_FWD, 2, 700, 320, 3),
    (workloads.TRAIN_FWD, 3, 257, 192, 3),
    (workloads.TRAIN_FWD, 1, 1, 64, 3),
    (workloads.TRAIN_FWD, 1, 300, 128, 5),
    (workloads.TRAIN_FWD, 2, 100, 448, 2),
]


@pytest.mark.parametrize("w,B,T,D,M", SMALL, ids=[f"{w.io}-{B}x{T}-D{D}-M{M}" for w, B, T, D, M in SMALL])
def test_mlp_small_elementwise(lib, w, B, T, D, M):
    p = workloads.make_mlp_inputs(w.with_shape(B=B, T=T, D=D), expansion=M)
    out = _gpu(lib, p)
    o = oracle.gated_mlp_forward(p["x"], p["W_1"], p["W_2"], p["W_3"], w.io)
    e = err(out, o)
    print(f"{w.io} {B}x{T} D={D} M={M} err(out)={e:.3e}", flush=True)
    assert e <= TOL[w.io]


def test_mlp_repeat_is_bitwise_identical(lib):
    p = workloads.make_mlp_inputs(workloads.TRAIN_FWD.with_shape(B=2, T=300, D=256))
    first = _gpu(lib, p)
    for _ in range(2):
        np.testing.assert_array_equal(_gpu(lib, p), first)


@pytest.mark.timeout(600)
def test_mlp_full_training_shape_row_subset(lib):
    """B=8, T=2048, D=2560, M=3 (hidden 7680) in the launch configuration the benchmark
    times; 300 seeded rows (including both ends and tile edges) against the oracle."""
    w = workloads.TRAIN_FWD
    p = workloads.make_mlp_inputs(w)
    out = _gpu(lib, p).reshape(-1, w.D)
    rng = np.random.default_rng(23)
    M = w.B * w.T
    rows = np.unique(np.concatenate([[0, 1, 255, 256, M // 2, M - 257, M - 256, M - 1],
                                     rng.choice(M, 292, replace=False)]))
    x = p["x"].reshape(-1, w.D)[rows]
    o = oracle.gated_mlp_forward(x, p["W_1"], p["W_2"], p["W_3"], w.io)
    e = err(out[rows], o)
    print(f"full MLP rows={len(rows)} err(out)={e:.3e}", flush=True)
    assert e <= TOL["bf16"]
    assert np.all(np.isfinite(out))
