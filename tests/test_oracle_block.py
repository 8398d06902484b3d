"""Pins of the oracle's recurrent block (the Griffin model-architecture page, section
"Recurrent block" and Fig. 2(c): two linear layers D -> D_RNN in parallel, Conv1D + RG-LRU
on the first branch, GeLU on the second, elementwise product, linear D_RNN -> D).

None of these compares the oracle with itself: textbook values and identities of the
normal distribution for GeLU, a numerical integral independent of erf, a closed form of
the whole block for constant gates, single-entry weights that fix every operand's
orientation, and an explicit per-element evaluation with the unrolled recurrence.
"""
import math

import numpy as np
import pytest

import oracle
import workloads


# ---------------------------------------------------------------- GeLU = q Phi(q)
def test_gelu_textbook_values():
    # Phi(1), Phi(2), Phi(-1) of the standard normal distribution (tables)
    assert oracle.gelu(0.0) == 0.0
    np.testing.assert_allclose(oracle.gelu(1.0), 0.8413447460685429, rtol=1e-15)
    np.testing.assert_allclose(oracle.gelu(2.0), 2 * 0.9772498680518208, rtol=1e-15)
    np.testing.assert_allclose(oracle.gelu(-1.0), -0.15865525393145707, rtol=1e-14)


def test_gelu_identities_and_limits():
    q = np.random.default_rng(3).standard_normal(10000) * 4
    # Phi(-q) = 1 - Phi(q)  =>  GeLU(-q) = GeLU(q) - q
    np.testing.assert_allclose(oracle.gelu(-q), oracle.gelu(q) - q, atol=1e-14)
    assert abs(oracle.gelu(12.0) - 12.0) < 1e-30
    assert abs(oracle.gelu(-12.0)) < 1e-30
    eps = 1e-6                                    # d/dq GeLU at 0 = Phi(0) = 1/2
    assert abs((oracle.gelu(eps) - oracle.gelu(-eps)) / (2 * eps) - 0.5) < 1e-10


def test_gelu_against_simpson_integral_of_the_normal_density():
    # Phi(x) = 1/2 + integral_0^x phi(t) dt, by composite Simpson (no erf involved)
    for x in (-3.0, -0.7, 0.4, 1.5, 2.9):
        n = 20000
        t = np.linspace(0.0, x, n + 1)
        f = np.exp(-0.5 * t * t) / math.sqrt(2 * math.pi)
        integral = (t[1] - t[0]) / 3 * (f[0] + f[-1] + 4 * f[1:-1:2].sum() + 2 * f[2:-1:2].sum())
        np.testing.assert_allclose(oracle.gelu(x), x * (0.5 + integral), rtol=1e-12, atol=1e-15)


# ---------------------------------------------------------------- the block
def _block_params(rng, B, T, D, R, io="f32"):
    w = workloads.TINY_F32.with_shape(B=B, T=T, D=R, io=io, h0="normal", history="normal",
                                      bias_std=0.3, seed=int(rng.integers(1 << 30)))
    return workloads.make_block_inputs(w, d_model=D)


def _block(p, **kw):
    args = dict(x=p["x_block"], W_in=p["W_in"], conv_w=p["conv_w"], conv_b=p["conv_b"],
                conv_state_in=p["conv_state"], W_a=p["W_a"], W_x=p["W_x"], b_a=p["b_a"],
                b_x=p["b_x"], lam=p["lam"], h0=p["h0"], W_out=p["W_out"], c=p["c"],
                io=p["workload"].io)
    args.update(kw)
    return oracle.block_forward(**args)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_block_constant_gates_closed_form(io):
    """W_a = W_x = 0, identity conv, no history, h0 = 0, x constant over time: r, i, a are
    constant per channel and h_t = (1 - a^t) / (1 - a) m i p with p = RNE(x W_in1^T); with
    D = R and W_out = I the block output is RNE(RNE(h_t g)) = RNE(h_t g), g = RNE(GeLU(q))."""
    rng = np.random.default_rng(7)
    B, T, R = 2, 40, 16
    D = R
    x1 = oracle.round_io(rng.standard_normal((B, 1, D)), io)
    x = np.repeat(x1, T, axis=1)
    W_in = oracle.round_io(rng.standard_normal((2 * R, D)) / 4, io)
    b_a, b_x = rng.normal(0, 0.5, R), rng.normal(0, 0.5, R)
    U = rng.uniform(0.9, 0.999, R)
    lam = np.log(U ** (1 / 8) / (1 - U ** (1 / 8)))
    conv_w = np.zeros((4, R))
    conv_w[0] = 1.0
    o = oracle.block_forward(x, W_in, conv_w, None, None, np.zeros((R, R)), np.zeros((R, R)),
                             b_a, b_x, lam, None, np.eye(D), 8.0, io)
    pin = oracle.round_io(x1[:, 0, :] @ W_in[:R].T, io)                 # [B, R]
    q = x1[:, 0, :] @ W_in[R:].T
    g = oracle.round_io(q * 0.5 * (1 + np.vectorize(math.erf)(q / math.sqrt(2))), io)
    sig = lambda v: 1 / (1 + np.exp(-v))
    a = sig(lam) ** (8.0 * sig(b_a))
    m = np.sqrt(1 - a * a)
    i = sig(b_x)
    t = np.arange(1, T + 1)[None, :, None]
    h = (1 - a ** t) / (1 - a) * (m * i * pin)[:, None, :]
    want = oracle.round_io(h * g[:, None, :], io)
    tol = 1e-13 if io == "f32" else 1e-12
    np.testing.assert_allclose(o["out"], want, rtol=tol if io == "f32" else 0, atol=1e-12)
    np.testing.assert_allclose(o["h_T"], h[:, -1], rtol=1e-12)


def test_block_operand_orientation_single_entries():
    """Single-entry weights route one channel through the block: W_in1 = e(j, k) feeds model
    channel k into branch channel j, W_in2 = 3 e(j, k') opens the GeLU gate from channel k',
    W_out = e(n, j) lands the product in output channel n.  Every other output is 0."""
    rng = np.random.default_rng(5)
    B, T, D, R = 1, 12, 6, 4
    j, k, k2, n = 2, 4, 1, 5
    x = rng.standard_normal((B, T, D))
    W_in = np.zeros((2 * R, D))
    W_in[j, k] = 1.0
    W_in[R + j, k2] = 3.0
    W_out = np.zeros((D, R))
    W_out[n, j] = 1.0
    conv_w = np.zeros((4, R))
    conv_w[0] = 1.0
    lam = np.full(R, 2.0)
    o = oracle.block_forward(x, W_in, conv_w, None, None, np.zeros((R, R)), np.zeros((R, R)),
                             np.zeros(R), np.zeros(R), lam, None, W_out, 8.0, "f32", keep=True)
    out = o["out"]
    assert np.all(out[:, :, [d for d in range(D) if d != n]] == 0)
    # channel n: the scalar recurrence of branch channel j on x[..., k], times GeLU(3 x[..., k2])
    a = (1 / (1 + math.exp(-2.0))) ** (8.0 * 0.5)
    m, i = math.sqrt(1 - a * a), 0.5
    h, want = 0.0, []
    for t in range(T):
        u = float(oracle.round_io(x[0, t, k], "f32"))
        h = a * h + m * i * u
        q = 3.0 * x[0, t, k2]
        gq = float(oracle.round_io(q * 0.5 * (1 + math.erf(q / math.sqrt(2))), "f32"))
        want.append(h * gq)
    np.testing.assert_allclose(out[0, :, n], oracle.round_io(np.array(want), "f32"), rtol=1e-6)


def test_block_explicit_elementwise_evaluation():
    """Every output of a tiny block evaluated element by element with explicit loops: the
    input linears and the output linear as sums, the recurrence as the unrolled sum
    h_t = (prod_{s<=t} a_s) h0 + sum_s (prod_{s<r<=t} a_r) m_s i_s u_s, the conv by its taps."""
    rng = np.random.default_rng(9)
    B, T, D, R = 2, 5, 3, 4
    p = _block_params(rng, B, T, D, R)
    o = _block(p)
    x, W_in, W_out = p["x_block"], p["W_in"], p["W_out"]
    f32 = lambda v: float(oracle.round_io(np.float64(v), "f32"))
    sig = lambda v: 1 / (1 + math.exp(-v))
    for b in range(B):
        P = [[f32(sum(x[b, t, d] * W_in[r, d] for d in range(D))) for r in range(R)] for t in range(T)]
        G = [[f32(oracle.gelu(sum(x[b, t, d] * W_in[R + r, d] for d in range(D)))) for r in range(R)]
             for t in range(T)]
        X = [list(p["conv_state"][b, s]) for s in range(3)] + P       # rows t-3 .. T-1
        U = [[f32(p["conv_b"][r] + sum(p["conv_w"][kk, r] * X[t + 3 - kk][r] for kk in range(4)))
              for r in range(R)] for t in range(T)]
        for t in range(T):
            z = []
            for r in range(R):
                def gate(s):
                    za = sum(p["W_a"][r, e] * U[s][e] for e in range(R)) + p["b_a"][r]
                    zx = sum(p["W_x"][r, e] * U[s][e] for e in range(R)) + p["b_x"][r]
                    a = sig(p["lam"][r]) ** (p["c"] * sig(za))
                    return a, math.sqrt(1 - a * a) * sig(zx)
                gs = [gate(s) for s in range(t + 1)]
                h = p["h0"][b, r] * math.prod(g[0] for g in gs)
                for s in range(t + 1):
                    h += math.prod(gs[q][0] for q in range(s + 1, t + 1)) * gs[s][1] * U[s][r]
                z.append(f32(h * G[t][r]))
            for dd in range(D):
                want = f32(sum(W_out[dd, r] * z[r] for r in range(R)))
                assert abs(o["out"][b, t, dd] - want) <= 2e-6 * max(1.0, abs(want)), (b, t, dd)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_block_decode_steps_equal_forward(io):
    """The block on a length-1 sequence with the carried (conv history, h) - a decode step -
    repeated over the tokens equals one block forward over them (the recurrence carries all
    of the past in the fixed-size state)."""
    rng = np.random.default_rng(13)
    p = _block_params(rng, 2, 9, 64, 128, io)
    full = _block(p)
    cs, h = p["conv_state"], p["h0"]
    for t in range(9):
        step = _block(p, x=p["x_block"][:, t:t + 1], conv_state_in=cs, h0=h)
        np.testing.assert_allclose(step["out"][:, 0], full["out"][:, t], rtol=1e-12, atol=1e-12)
        cs, h = step["conv_state_out"], step["h_T"]
    np.testing.assert_allclose(h, full["h_T"], rtol=1e-12)
    np.testing.assert_array_equal(cs, full["conv_state_out"])
