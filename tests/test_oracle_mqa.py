"""Pins of the oracle's local multi-query attention (the Griffin model-architecture page,
sections "Global multi-query attention" and "Local sliding-window attention").

RoPE against explicit 2x2 rotations with math.cos / math.sin and the relative-position
property that motivates it; the windowed attention against a per-element brute force with
math.exp, against its degenerate windows (W = 1 returns v_t, W >= T is causal attention),
against uniform weights (q = 0 averages the window) and one-hot weights; the block against
single-entry weights that route one head through every projection.
"""
import math

import numpy as np
import pytest

import oracle
import workloads


# ---------------------------------------------------------------- RoPE
def test_rope_explicit_rotation_and_identity_at_zero():
    rng = np.random.default_rng(1)
    v = rng.standard_normal((1, 4, 128))
    pos = np.array([0, 1, 7, 1000])
    r = oracle.rope(v, pos)
    np.testing.assert_array_equal(r[0, 0], v[0, 0])                     # angle 0
    for t in range(1, 4):
        for i in (0, 1, 17, 63):
            ang = pos[t] * 10000.0 ** (-2 * i / 128)
            c, s = math.cos(ang), math.sin(ang)
            e, o = v[0, t, 2 * i], v[0, t, 2 * i + 1]
            assert abs(r[0, t, 2 * i] - (e * c - o * s)) < 1e-12
            assert abs(r[0, t, 2 * i + 1] - (e * s + o * c)) < 1e-12


def test_rope_preserves_pair_norms_and_scores_depend_on_offset_only():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, 1, 3, 128))       # [B, T, H, d]
    k = rng.standard_normal((1, 1, 128))
    for t, s_, c in ((5, 2, 11), (100, 37, 900), (3, 3, 1)):
        qa, ka = oracle.rope(q, [t]), oracle.rope(k, [s_])
        qb, kb = oracle.rope(q, [t + c]), oracle.rope(k, [s_ + c])
        np.testing.assert_allclose(np.einsum("hd,d->h", qa[0, 0], ka[0, 0]),
                                   np.einsum("hd,d->h", qb[0, 0], kb[0, 0]), rtol=1e-9, atol=1e-9)
        pn = lambda a: a[..., 0::2] ** 2 + a[..., 1::2] ** 2
        np.testing.assert_allclose(pn(qa), pn(q), rtol=1e-12)


# ---------------------------------------------------------------- windowed attention
def _brute(q, k, v, window):
    B, T, H, d = q.shape
    out = np.zeros((B, T, H, d))
    for b in range(B):
        for t in range(T):
            keys = [s for s in range(k.shape[1]) if t - window < s <= t]
            for h in range(H):
                sc = [sum(float(q[b, t, h, j]) * float(k[b, s, j]) for j in range(d)) / math.sqrt(d)
                      for s in keys]
                m = max(sc)
                w = [math.exp(x - m) for x in sc]
                z = sum(w)
                for j in range(d):
                    out[b, t, h, j] = sum(wi * float(v[b, s, j]) for wi, s in zip(w, keys)) / z
    return out


@pytest.mark.parametrize("window", [1, 3, 6, 100])
def test_attention_against_per_element_brute_force(window):
    rng = np.random.default_rng(window)
    q = rng.standard_normal((2, 6, 2, 8)) * 2
    k = rng.standard_normal((2, 6, 8))
    v = rng.standard_normal((2, 6, 8))
    np.testing.assert_allclose(oracle.local_mqa_attention(q, k, v, window), _brute(q, k, v, window),
                               rtol=1e-12, atol=1e-12)


def test_attention_degenerate_windows():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, 40, 3, 16))
    k = rng.standard_normal((1, 40, 16))
    v = rng.standard_normal((1, 40, 16))
    one = oracle.local_mqa_attention(q, k, v, 1)
    np.testing.assert_allclose(one, np.broadcast_to(v[:, :, None, :], one.shape), rtol=1e-15)
    # q = 0: uniform weights over the window -> the mean of its values
    z = oracle.local_mqa_attention(np.zeros_like(q), k, v, 7)
    for t in range(40):
        lo = max(0, t - 6)
        np.testing.assert_allclose(z[0, t, 1], v[0, lo:t + 1].mean(axis=0), rtol=1e-12, atol=1e-14)


def test_attention_one_hot_weights_pick_the_matching_key():
    """Keys are one-hot vectors; a query equal to 240 * key s scores s above every other key
    by 240 / sqrt(16) = 60 in logits (weights e^-60 elsewhere), so the output is v_s."""
    d, T = 16, 12
    k = np.zeros((1, T, d))
    for s in range(T):
        k[0, s, s] = 1.0
    v = np.random.default_rng(4).standard_normal((1, T, d))
    q = np.zeros((1, T, 1, d))
    target = [max(0, t - 2) for t in range(T)]          # within a window of 4
    for t in range(T):
        q[0, t, 0, target[t]] = 240.0
    o = oracle.local_mqa_attention(q, k, v, 4)
    for t in range(T):
        np.testing.assert_allclose(o[0, t, 0], v[0, target[t]], rtol=1e-9, atol=1e-9)


def test_attention_positions_offset_matches_shifted_sequence():
    """Keys from an earlier chunk (kv positions before the queries') give the same result as
    attending within the concatenated sequence."""
    rng = np.random.default_rng(5)
    q = rng.standard_normal((1, 30, 2, 8))
    k = rng.standard_normal((1, 30, 8))
    v = rng.standard_normal((1, 30, 8))
    full = oracle.local_mqa_attention(q, k, v, 9)
    part = oracle.local_mqa_attention(q[:, 20:], k[:, 12:], v[:, 12:], 9, q_pos=np.arange(20, 30),
                                      kv_pos=np.arange(12, 30))
    np.testing.assert_allclose(part, full[:, 20:], rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------- the block
def test_block_single_head_routing():
    """D = 256 (two heads).  W_q routes x channel 5 into head 1 dimension 0, W_k routes x
    channel 7 into key dimension 0, W_v copies x channel 9 into value dimension 3, W_o reads
    head 1 dimension 3 into output channel 200.  With RoPE at dimension pair 0 the score of
    (t, s) is q0 k0 cos((t - s) theta_0) = x_t[5] x_s[7] cos(t - s), so the output channel
    200 is the softmax over the window of those scores applied to x_s[9]."""
    rng = np.random.default_rng(6)
    B, T, D = 1, 20, 256
    x = rng.standard_normal((B, T, D))
    Wq = np.zeros((D, D)); Wq[128 + 0, 5] = 1.0
    Wk = np.zeros((128, D)); Wk[0, 7] = 1.0
    Wv = np.zeros((128, D)); Wv[3, 9] = 1.0
    Wo = np.zeros((D, D)); Wo[200, 128 + 3] = 1.0
    out = oracle.local_mqa_forward(x, Wq, Wk, Wv, Wo, 5, "f32")
    assert np.all(out[..., [c for c in range(D) if c != 200]] == 0)
    for t in range(T):
        keys = [s for s in range(T) if t - 5 < s <= t]
        sc = [x[0, t, 5] * x[0, s, 7] * math.cos(t - s) / math.sqrt(128) for s in keys]
        m = max(sc)
        w = [math.exp(c - m) for c in sc]
        want = sum(wi * x[0, s, 9] for wi, s in zip(w, keys)) / sum(w)
        assert abs(out[0, t, 200] - want) <= 2e-6 * max(1.0, abs(want)), t


def test_block_rounding_points_bf16():
    """With bf16 I/O the returned q, k, v and attention output are bf16 values."""
    p = workloads.make_mqa_inputs(workloads.TRAIN_FWD.with_shape(B=1, T=40, D=256), window=16)
    r = oracle.local_mqa_forward(p["x"], p["W_q"], p["W_k"], p["W_v"], p["W_o"], 16, "bf16", keep=True)
    for name in ("q", "k", "v", "attn", "out"):
        np.testing.assert_array_equal(oracle.round_io(r[name], "bf16"), r[name])


@pytest.mark.parametrize("window", [4, 16])
def test_decode_steps_equal_forward_and_cache_stays_bounded(window):
    """T decode steps from an empty cache (T longer than the window, so slots are reused)
    give the forward's outputs for every position; the cache holds exactly the last
    `window` rotated keys and values, each in slot position % window."""
    w = workloads.TRAIN_FWD.with_shape(B=2, T=3 * window + 5, D=256, io="f32")
    p = workloads.make_mqa_inputs(w, window)
    f = oracle.local_mqa_forward(p["x"], p["W_q"], p["W_k"], p["W_v"], p["W_o"], window, "f32", keep=True)
    kc = np.zeros((2, window, 128))
    vc = np.zeros((2, window, 128))
    for t in range(w.T):
        out, kc, vc = oracle.local_mqa_decode_step(p["x"][:, t], p["W_q"], p["W_k"], p["W_v"], p["W_o"],
                                                   kc, vc, [t, t], window, "f32")
        np.testing.assert_allclose(out, f["out"][:, t], rtol=1e-9, atol=1e-12)
    for s in range(w.T - window, w.T):
        np.testing.assert_allclose(kc[:, s % window], f["k"][:, s], rtol=1e-12)
        np.testing.assert_allclose(vc[:, s % window], f["v"][:, s], rtol=1e-12)


def test_decode_ignores_slots_outside_the_window_and_before_zero():
    """Garbage in slots that hold no live position (before position 0, or evicted) does not
    change the step; distinct positions per sequence are honoured."""
    w = workloads.TRAIN_FWD.with_shape(B=2, T=3, D=128, io="f32")
    p = workloads.make_mqa_inputs(w, 8)
    rng = np.random.default_rng(9)
    kc = rng.standard_normal((2, 8, 128))
    vc = rng.standard_normal((2, 8, 128))
    pos = [2, 11]
    a, _, _ = oracle.local_mqa_decode_step(p["x"][:, 0], p["W_q"], p["W_k"], p["W_v"], p["W_o"], kc, vc,
                                           pos, 8, "f32")
    kc2, vc2 = kc.copy(), vc.copy()
    kc2[0, 3:] = 1e3          # sequence 0 at position 2: slots 3..7 hold no position yet
    vc2[0, 3:] = -1e3
    b, _, _ = oracle.local_mqa_decode_step(p["x"][:, 0], p["W_q"], p["W_k"], p["W_v"], p["W_o"], kc2, vc2,
                                           pos, 8, "f32")
    np.testing.assert_array_equal(a, b)
