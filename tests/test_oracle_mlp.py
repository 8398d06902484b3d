"""Pins of the oracle's gated MLP block (the Griffin model-architecture page, section "MLP
block", Fig. 2(b): two width-M*D linears of the same input, GeLU on one, elementwise
product, a final linear back to D).

The expected values come from Python's own math.erf (not the oracle's scipy erf), from the
sign invariant of q^2 Phi(q), from single-entry weights that route one channel through every
operand, and from explicit per-element sums on a tiny input.
"""
import math

import numpy as np
import pytest

import oracle
import workloads


def _phi(q):
    return 0.5 * (1.0 + math.erf(q / math.sqrt(2.0)))


def test_mlp_single_channel_route_and_branch_order():
    """W_1 = 2 e(j, k1) (GeLU branch), W_2 = 3 e(j, k2), W_3 = e(n, j): only output channel n
    is non-zero and equals GeLU(2 x_k1) * 3 x_k2 (rounded); swapping W_1 and W_2 moves the
    GeLU to the other factor."""
    rng = np.random.default_rng(2)
    D, MD = 5, 9
    j, k1, k2, n = 7, 1, 3, 4
    x = rng.standard_normal((2, 6, D))
    W1 = np.zeros((MD, D)); W1[j, k1] = 2.0
    W2 = np.zeros((MD, D)); W2[j, k2] = 3.0
    W3 = np.zeros((D, MD)); W3[n, j] = 1.0
    out = oracle.gated_mlp_forward(x, W1, W2, W3, "f32")
    swapped = oracle.gated_mlp_forward(x, W2, W1, W3, "f32")
    assert np.all(out[..., [d for d in range(D) if d != n]] == 0)
    for b in range(2):
        for t in range(6):
            a1, a2 = 2.0 * x[b, t, k1], 3.0 * x[b, t, k2]
            want = float(oracle.round_io(np.float64(a1 * _phi(a1) * a2), "f32"))
            want_sw = float(oracle.round_io(np.float64(a2 * _phi(a2) * a1), "f32"))
            assert abs(out[b, t, n] - want) <= 1e-7 * max(1.0, abs(want))
            assert abs(swapped[b, t, n] - want_sw) <= 1e-7 * max(1.0, abs(want_sw))


def test_mlp_textbook_value():
    # q1 = 1, q2 = 2: h = 2 Phi(1) = 1.6826894921370859 (Phi(1) from normal tables)
    x = np.ones((1, 1, 1))
    out = oracle.gated_mlp_forward(x, np.ones((1, 1)), 2 * np.ones((1, 1)), np.ones((1, 1)), "f32")
    np.testing.assert_allclose(out[0, 0, 0], 2 * 0.8413447460685429, rtol=1e-7)


def test_mlp_equal_branches_are_nonnegative_and_zero_branch_is_zero():
    """With W_2 = W_1 every product is q * GeLU(q) = q^2 Phi(q) >= 0; with W_2 = 0 the block
    output is exactly zero."""
    p = workloads.make_mlp_inputs(workloads.TINY_F32.with_shape(B=2, T=30, D=16))
    r = oracle.gated_mlp_forward(p["x"], p["W_1"], p["W_1"], p["W_3"], "f32", keep=True)
    assert np.all(r["h"] >= 0) and np.any(r["h"] > 0)
    z = oracle.gated_mlp_forward(p["x"], p["W_1"], np.zeros_like(p["W_2"]), p["W_3"], "bf16")
    assert np.all(z == 0)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_mlp_explicit_elementwise_evaluation(io):
    p = workloads.make_mlp_inputs(workloads.TINY_F32.with_shape(B=1, T=3, D=4, io=io), expansion=3)
    x, W1, W2, W3 = p["x"], p["W_1"], p["W_2"], p["W_3"]
    out = oracle.gated_mlp_forward(x, W1, W2, W3, io)
    rnd = lambda v: float(oracle.round_io(np.float64(v), io))
    MD, D = W1.shape
    for t in range(3):
        h = []
        for j in range(MD):
            q1 = sum(float(W1[j, k]) * float(x[0, t, k]) for k in range(D))
            q2 = sum(float(W2[j, k]) * float(x[0, t, k]) for k in range(D))
            h.append(rnd(q1 * _phi(q1) * q2))
        for n in range(D):
            want = rnd(sum(float(W3[n, j]) * h[j] for j in range(MD)))
            # the same arithmetic in another summation order: identical after rounding
            assert abs(out[0, t, n] - want) <= 1e-12 * max(1.0, abs(want)), (t, n)
