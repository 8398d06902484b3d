"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these compares the oracle with itself: each check is a closed form, an
invariant, a brute-force evaluation of a different formula, or a library routine.
Sources: the Griffin model-architecture page, sections "Recurrent block", "Real-Gated
Linear Recurrent Unit (RG-LRU)" (Eq. (1)-(4)) and "Gate behaviour"; the blog page
"Griffin's Compromise", sections "Hawk" and "Term explanation: Parallel scan".
"""
import math

import numpy as np
import pytest
import scipy.special as sps
import torch

import oracle
import workloads


def _params(rng, B, T, D, io="f32", bias_std=0.1, ac=(0.9, 0.999), c=8.0, h0=True, state=True):
    w = workloads.TINY_F32.with_shape(B=B, T=T, D=D, io=io, bias_std=bias_std, ac_lo=ac[0],
                                      ac_hi=ac[1], h0="normal" if h0 else "zero",
                                      history="normal" if state else "zero",
                                      seed=int(rng.integers(1 << 30)))
    return workloads.make_inputs(w, c)


def _fwd(p, **kw):
    args = dict(x=p["x"], conv_w=p["conv_w"], conv_b=p["conv_b"], conv_state_in=p["conv_state"],
                W_a=p["W_a"], W_x=p["W_x"], b_a=p["b_a"], b_x=p["b_x"], lam=p["lam"], h0=p["h0"],
                c=p["c"], io=p["workload"].io)
    args.update(kw)
    return oracle.forward(**args)


# ---------------------------------------------------------------- I/O rounding
def test_round_bf16_matches_torch_conversion():
    rng = np.random.default_rng(1)
    v = np.concatenate([rng.standard_normal(100000) * 10.0 ** rng.integers(-30, 30, 100000),
                        [0.0, -0.0, 1.0, -2.5, 3.0e38, 1e-39, -1e-40]]).astype(np.float32)
    want = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.round_io(v.astype(np.float64), "bf16")
    np.testing.assert_array_equal(got, want)


def test_round_bf16_ties_to_even_hand_cases():
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: ties go to the even significand (1).
    # 1 + 3*2^-8 lies halfway between 1 + 2^-7 (odd) and 1 + 2^-6 (even).
    v = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), 1 + 2.0 ** -8 + 2.0 ** -30])
    np.testing.assert_array_equal(oracle.round_io(v, "bf16"),
                                  [1.0, 1 + 2.0 ** -6, -1.0, 1 + 2.0 ** -7])


def test_round_f32_is_ieee_single():
    v = np.array([1 + 2.0 ** -24, 1 + 3 * 2.0 ** -24, 0.1])
    np.testing.assert_array_equal(oracle.round_io(v, "f32"),
                                  [1.0, 1 + 2.0 ** -22, float(np.float32(0.1))])


# ---------------------------------------------------------------- sigma, log sigma
def test_sigmoid_and_log_sigmoid_match_scipy():
    z = np.concatenate([np.linspace(-800, 800, 4001), [-np.inf, np.inf, 0.0, 1e-300, -1e-300]])
    np.testing.assert_allclose(oracle.sigmoid(z), sps.expit(z), rtol=1e-15, atol=1e-300)
    zf = z[np.isfinite(z)]
    np.testing.assert_allclose(oracle.log_sigmoid(zf), sps.log_expit(zf), rtol=1e-14, atol=1e-300)


def test_gates_equal_plain_power_form():
    """Eq. (3) as printed: a_t = a^{c r_t} with a = sigma(Lambda), m = sqrt(1 - a_t^2)."""
    rng = np.random.default_rng(2)
    zr, zi = rng.standard_normal(5000) * 4, rng.standard_normal(5000) * 4
    lam = rng.standard_normal(5000) * 3
    for c in (8.0, 1.0, 0.5):
        r, i, ell, a, m = oracle.gates(zr, zi, lam, c)
        a_plain = np.power(sps.expit(lam), c * sps.expit(zr))
        np.testing.assert_allclose(a, a_plain, rtol=1e-13)
        np.testing.assert_allclose(i, sps.expit(zi), rtol=1e-15)
        far = a < 0.99                       # away from cancellation in 1 - a^2
        np.testing.assert_allclose(m[far], np.sqrt(1 - a_plain[far] ** 2), rtol=1e-12)


def test_invariants_a_and_m():
    """0 <= a <= 1 guaranteed by a = sigma(Lambda) (RG-LRU section); a^2 + m^2 = 1."""
    rng = np.random.default_rng(3)
    zr = np.concatenate([rng.standard_normal(10000) * 30, [-np.inf, np.inf]])
    lam = np.concatenate([rng.standard_normal(10000) * 30, [0.0, 5.0]])
    _, _, ell, a, m = oracle.gates(zr, zr, lam, 8.0)
    assert np.all(ell <= 0)
    assert np.all((a >= 0) & (a <= 1)) and np.all((m >= 0) & (m <= 1))
    assert np.max(np.abs(a * a + m * m - 1)) <= 4e-16


# ---------------------------------------------------------------- conv
@pytest.mark.parametrize("k", [0, 1, 2, 3])
def test_conv_one_hot_tap_shifts(k):
    rng = np.random.default_rng(10 + k)
    B, T, D = 2, 9, 6
    x = rng.standard_normal((B, T, D))
    st = rng.standard_normal((B, 3, D))
    w = np.zeros((4, D)); w[k] = 1.0
    u, so = oracle.conv1d_causal4(x, w, None, st, "f64")
    X = np.concatenate([st, x], axis=1)              # X[tau + 3] = x_tau
    np.testing.assert_array_equal(u, X[:, 3 - k:3 - k + T])
    np.testing.assert_array_equal(so, x[:, T - 3:])
    u0, _ = oracle.conv1d_causal4(x, w, None, None, "f64")
    np.testing.assert_array_equal(u0[:, :k], 0.0)    # zero history before the first token


def test_conv_state_out_short_sequence_and_bias():
    x = np.arange(2 * 1 * 3, dtype=np.float64).reshape(2, 1, 3)
    st = 100 + np.arange(2 * 3 * 3, dtype=np.float64).reshape(2, 3, 3)
    w = np.zeros((4, 3))
    u, so = oracle.conv1d_causal4(x, w, np.array([1.5, -2.0, 0.25]), st, "f64")
    np.testing.assert_array_equal(u[0, 0], [1.5, -2.0, 0.25])
    np.testing.assert_array_equal(so, np.concatenate([st[:, 1:], x], axis=1))


# ---------------------------------------------------------------- P1: r = 0 keeps the state
@pytest.mark.parametrize("mode", ["b_a=-inf", "c=0"])
def test_recurrence_gate_closed_keeps_state_bit_exact(mode):
    """Gate behaviour: with r_t = 0 (or c = 0), a_t = 1 and sqrt(1-a_t^2) = 0, so
    h_t = h_{t-1} exactly and the input is discarded."""
    rng = np.random.default_rng(4)
    p = _params(rng, 3, 20, 8, h0=True)
    kw = {"b_a": np.full(8, -np.inf)} if mode == "b_a=-inf" else {"c": 0.0}
    o = _fwd(p, keep=True, **kw)
    assert np.all(o["a"] == 1.0) and np.all(o["m"] == 0.0)
    np.testing.assert_array_equal(o["h_T"], p["h0"].astype(np.float64))
    np.testing.assert_array_equal(o["y"], np.broadcast_to(
        p["h0"].astype(np.float32).astype(np.float64)[:, None, :], o["y"].shape))


# ---------------------------------------------------------------- P2: geometric closed form
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_constant_gates_geometric_closed_form(io):
    D, T = 7, 300
    rng = np.random.default_rng(5)
    lam = rng.uniform(1.0, 6.0, D)
    b_a, b_x = rng.standard_normal(D), rng.standard_normal(D)
    xi = oracle.round_io(rng.standard_normal(D), io)
    h0 = rng.standard_normal((1, D))
    x = np.broadcast_to(xi, (1, T, D)).copy()
    w = np.zeros((4, D)); w[0] = 1.0
    Z = np.zeros((D, D))
    o = oracle.forward(x, w, None, None, Z, Z, b_a, b_x, lam, h0, 8.0, io, keep=True)
    alpha = sps.expit(lam) ** (8.0 * sps.expit(b_a))
    s = sps.expit(b_x)
    t = np.arange(1, T + 1)[:, None]
    want = alpha ** t * h0 + (1 - alpha ** t) / (1 - alpha) * np.sqrt(1 - alpha ** 2) * s * xi
    np.testing.assert_allclose(o["y_exact"][0], want, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(o["h_T"][0], want[-1], rtol=1e-11)
    ulp = 2.0 ** -23 if io == "f32" else 2.0 ** -7
    np.testing.assert_allclose(o["y"][0], want, rtol=ulp, atol=0)
    # the long-time limit sqrt((1+alpha)/(1-alpha)) sigma(b_x) xi
    o2 = oracle.forward(np.broadcast_to(xi, (1, 20000, D)).copy(), w, None, None, Z, Z, b_a, b_x,
                        lam, None, 8.0, io)
    np.testing.assert_allclose(o2["h_T"][0], np.sqrt((1 + alpha) / (1 - alpha)) * s * xi,
                               rtol=1e-9)


# ---------------------------------------------------------------- P3: unrolled sum
def test_sequential_equals_unrolled_sum_brute_force():
    """h_T = (prod_j a_j) h0 + sum_k (prod_{j>k} a_j) m_k i_k u_k, written with scalar loops."""
    rng = np.random.default_rng(6)
    p = _params(rng, 2, 11, 5)
    o = _fwd(p, keep=True)
    a, m, i, u = o["a"], o["m"], o["i"], o["u"]
    h0 = p["h0"].astype(np.float64)
    B, T, D = a.shape
    for b in range(B):
        for d in range(D):
            tot = h0[b, d]
            for j in range(T):
                tot *= a[b, j, d]
            for k in range(T):
                term = m[b, k, d] * i[b, k, d] * u[b, k, d]
                for j in range(k + 1, T):
                    term *= a[b, j, d]
                tot += term
            assert math.isclose(tot, o["h_T"][b, d], rel_tol=1e-12, abs_tol=1e-14)


# ---------------------------------------------------------------- P5: stationary variance
def test_stationary_variance_is_one():
    """sqrt(1 - a^2) normalisation: with constant gates, i = 1 and i.i.d. unit-variance
    inputs, Var(h_t) = a^{2t} Var(h0) + 1 - a^{2t} = 1 for every t."""
    rng = np.random.default_rng(7)
    B, T, D = 800, 48, 256
    N = B * D
    x = rng.standard_normal((B, T, D))
    h0 = rng.standard_normal((B, D))
    lam = rng.uniform(0.0, 5.0, D)
    w = np.zeros((4, D)); w[0] = 1.0
    Z = np.zeros((D, D))
    o = oracle.forward(x, w, None, None, Z, Z, np.zeros(D), np.full(D, np.inf), lam, h0, 8.0,
                       "f64", keep=True)
    var = (o["y_exact"] ** 2).mean(axis=(0, 2))
    assert np.all(np.abs(var - 1.0) < 5 * math.sqrt(2.0 / N)), var


# ---------------------------------------------------------------- gate orientation z = W u
def test_gate_projection_orientation():
    """Eq. (1), (2) are matrix-vector products W x_t: output channel n reads W[n, :]."""
    rng = np.random.default_rng(8)
    B, T, D = 1, 6, 5
    x = rng.standard_normal((B, T, D))
    w = np.zeros((4, D)); w[0] = 1.0
    n0, k0 = 1, 3
    Wa = np.zeros((D, D)); Wa[n0, k0] = 0.7
    Wx = np.zeros((D, D)); Wx[k0, n0] = -1.3          # only channel k0 reads u[n0]
    b_a = rng.standard_normal(D); b_x = rng.standard_normal(D)
    o = oracle.forward(x, w, None, None, Wa, Wx, b_a, b_x, np.ones(D), None, 8.0, "f64", keep=True)
    want_r = np.tile(sps.expit(b_a), (T, 1)); want_r[:, n0] = sps.expit(0.7 * x[0, :, k0] + b_a[n0])
    want_i = np.tile(sps.expit(b_x), (T, 1)); want_i[:, k0] = sps.expit(-1.3 * x[0, :, n0] + b_x[k0])
    np.testing.assert_allclose(o["r"][0], want_r, rtol=1e-15)
    np.testing.assert_allclose(o["i"][0], want_i, rtol=1e-15)


# ---------------------------------------------------------------- P7: state consistency
def test_decode_steps_equal_forward():
    rng = np.random.default_rng(9)
    p = _params(rng, 3, 17, 16)
    o = _fwd(p)
    st, h = p["conv_state"], p["h0"]
    for t in range(p["x"].shape[1]):
        y, st, h = oracle.decode_step(p["x"][:, t], p["conv_w"], p["conv_b"], st, p["W_a"],
                                      p["W_x"], p["b_a"], p["b_x"], p["lam"], h, p["c"], "f32")
        np.testing.assert_allclose(y, o["y"][:, t], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(h, o["h_T"], rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(st, o["conv_state_out"])


def test_split_forward_equals_forward():
    """Streaming input: fwd(x1 || x2) == fwd(x2 | state after x1)."""
    rng = np.random.default_rng(11)
    p = _params(rng, 2, 40, 16)
    o = _fwd(p)
    t1 = 13
    o1 = _fwd(p, x=p["x"][:, :t1])
    o2 = _fwd(p, x=p["x"][:, t1:], conv_state_in=o1["conv_state_out"], h0=o1["h_T"])
    np.testing.assert_allclose(np.concatenate([o1["y"], o2["y"]], axis=1), o["y"], rtol=1e-12,
                               atol=1e-12)
    np.testing.assert_allclose(o2["h_T"], o["h_T"], rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- P9: chunked scan
def _chunked_scan(a, bu, h0, chunk):
    """A separate CPU scan: per-chunk (prod a, local h) summaries combined with
    (A1,H1) o (A2,H2) = (A1 A2, A2 H1 + H2), then each chunk re-run from its carry
    (the parallel-scan description: chunk subtotals, then pass each summary on)."""
    T = a.shape[0]
    starts = list(range(0, T, chunk))
    summ = []
    for s in starts:
        A, H = np.ones_like(h0), np.zeros_like(h0)
        for t in range(s, min(T, s + chunk)):
            A, H = A * a[t], a[t] * H + bu[t]
        summ.append((A, H))
    # tree (Hillis-Steele) inclusive scan of the summaries
    pref = list(summ)
    step = 1
    while step < len(pref):
        pref = [pref[j] if j < step else
                (pref[j - step][0] * pref[j][0], pref[j][0] * pref[j - step][1] + pref[j][1])
                for j in range(len(pref))]
        step *= 2
    out = np.empty_like(a)
    for ci, s in enumerate(starts):
        h = h0 if ci == 0 else pref[ci - 1][0] * h0 + pref[ci - 1][1]
        for t in range(s, min(T, s + chunk)):
            h = a[t] * h + bu[t]
            out[t] = h
    return out


@pytest.mark.parametrize("chunk", [1, 3, 8, 64])
def test_chunked_parallel_scan_equals_sequential(chunk):
    rng = np.random.default_rng(12)
    p = _params(rng, 1, 50, 12)
    o = _fwd(p, io="f64", keep=True)
    a, bu = o["a"][0], (o["m"] * o["i"] * o["u"])[0]
    got = _chunked_scan(a, bu, p["h0"][0].astype(np.float64), chunk)
    np.testing.assert_allclose(got, o["y_exact"][0], rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- P10: channel subset
def test_channel_subset_matches_full():
    rng = np.random.default_rng(13)
    p = _params(rng, 2, 30, 64)
    S = np.array([0, 5, 17, 63])
    full, sub = _fwd(p), _fwd(p, channels=S)
    np.testing.assert_allclose(sub["y"], full["y"][:, :, S], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(sub["h_T"], full["h_T"][:, S], rtol=1e-13, atol=1e-13)


def test_output_rounding_points():
    """R2: y is h rounded to the I/O dtype; R1: the rounded u feeds gates and scan."""
    rng = np.random.default_rng(14)
    p = _params(rng, 1, 20, 8, io="bf16")
    o = _fwd(p, keep=True)
    np.testing.assert_array_equal(o["y"], oracle.round_io(o["y_exact"], "bf16"))
    np.testing.assert_array_equal(o["u"], oracle.round_io(o["u"], "bf16"))


# ---------------------------------------------------------------- R1: the conv sum, rounded once
def _round_exact(fr, bits):
    """Nearest binary float with `bits` significant bits (ties to even) of an exact
    rational, by integer arithmetic; normal range only (fp32: 24 bits, bf16: 8 bits)."""
    from fractions import Fraction
    if fr == 0:
        return 0.0
    sign = -1.0 if fr < 0 else 1.0
    mag = abs(fr)
    e = mag.numerator.bit_length() - mag.denominator.bit_length()
    if Fraction(2) ** e > mag:
        e -= 1
    ulp = Fraction(2) ** (e - (bits - 1))
    q = mag / ulp
    n = q.numerator // q.denominator
    rem = q - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * float(n * ulp)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_conv_rounds_the_exact_sum_all_taps_and_bias(io):
    """R1 on the conv of the "Recurrent block" section: u = RNE_io(b + sum_k w_k x_{t-k}),
    the exact rational sum of all four taps and a non-zero bias, rounded once to the I/O
    dtype.  Inputs are I/O-dtype values (bf16 ones for bf16), the bias fp32, the history
    non-zero, and the magnitudes spread so that the terms do not share an exponent."""
    from fractions import Fraction
    rng = np.random.default_rng(41 if io == "f32" else 42)
    B, T, D = 2, 13, 24
    q = (lambda v: oracle.round_io(v, io))
    x = q(rng.standard_normal((B, T, D)) * 2.0 ** rng.integers(-6, 7, (B, T, D)))
    st = q(rng.standard_normal((B, 3, D)) * 2.0 ** rng.integers(-6, 7, (B, 3, D)))
    w = q(rng.standard_normal((4, D)) * 2.0 ** rng.integers(-4, 5, (4, D)))
    assert np.all(w != 0)
    cb = oracle.round_io(rng.standard_normal(D) * 2.0 ** rng.integers(-10, 3, D), "f32")
    u, _ = oracle.conv1d_causal4(x, w, cb, st, io)
    X = np.concatenate([st, x], axis=1)
    bits = 24 if io == "f32" else 8
    want = np.empty((B, T, D))
    for b in range(B):
        for t in range(T):
            for d in range(D):
                s = Fraction(float(cb[d]))
                for k in range(4):
                    s += Fraction(float(w[k, d])) * Fraction(float(X[b, t + 3 - k, d]))
                want[b, t, d] = _round_exact(s, bits)
    np.testing.assert_array_equal(u, want)
    # the taps matter one by one: dropping any tap, or the bias, changes u somewhere
    for k in range(4):
        w2 = w.copy()
        w2[k] = 0.0
        assert np.any(oracle.conv1d_causal4(x, w2, cb, st, io)[0] != u)
    assert np.any(oracle.conv1d_causal4(x, w, None, st, io)[0] != u)


def test_round_exact_helper_on_hand_cases():
    from fractions import Fraction
    assert _round_exact(Fraction(1) + Fraction(1, 2 ** 24), 24) == 1.0            # tie -> even
    assert _round_exact(Fraction(1) + Fraction(3, 2 ** 24), 24) == 1 + 2.0 ** -22
    assert _round_exact(Fraction(1) + Fraction(1, 2 ** 8), 8) == 1.0
    assert _round_exact(-(Fraction(1) + Fraction(3, 2 ** 8)), 8) == -(1 + 2.0 ** -6)
    assert _round_exact(Fraction(1) + Fraction(1, 2 ** 8) + Fraction(1, 2 ** 40), 8) == 1 + 2.0 ** -7


def test_conv_rounds_once_not_twice():
    """Constructed sums where rounding first to fp32 and then to the I/O dtype picks the
    other neighbour: taps give 1 + 2^-p (p = 8 for bf16, 24 for fp32: an exact halfway point
    of the I/O dtype) and a tap product of +-2^-40 moves the sum just above or below it, by
    far less than an fp32 ulp.  R1 rounds the exact sum once."""
    from fractions import Fraction
    for io, p in (("bf16", 8), ("f32", 24)):
        D = 4
        s1 = np.array([1.0, 1.0, -1.0, -1.0])
        s2 = np.array([1.0, -1.0, 1.0, -1.0])
        w = np.zeros((4, D)); w[3] = s1; w[2] = s1 * 2.0 ** -p; w[1] = s2 * 2.0 ** -20
        x = np.zeros((1, 4, D)); x[0, 0] = x[0, 1] = 1.0; x[0, 2] = 2.0 ** -20
        assert np.array_equal(oracle.round_io(w, io), w)
        u, _ = oracle.conv1d_causal4(x, w, None, None, io)
        want = [_round_exact(Fraction(int(a)) * (1 + Fraction(1, 2 ** p)) + Fraction(int(b), 2 ** 40),
                             8 if io == "bf16" else 24) for a, b in zip(s1, s2)]
        np.testing.assert_array_equal(u[0, 3], want)
        assert len(set(want)) == 4                      # the tiny tap decides the neighbour
