"""CPU oracle for the RG-LRU temporal branch: causal depthwise Conv1D (width 4) -> RG-LRU.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import or run this module.  The HIP library never calls it, and it
shares no code with the HIP path (no kernels, headers, helpers or constants).

Plain, slow and sequential on purpose: NumPy, every operation in fp64, the recurrence a
Python loop over time vectorised over (batch, channel), the gate projections one
library matmul each.  No blocking, fusion or reordering beyond the definitions.

Sources (cited by page title and section; no other source is used):
  [ARCH]  "Griffin: Mixing Gated Linear Recurrences with Local Attention for Efficient
          Language Models" - model-architecture page (Chinese translation of the
          paper's Model Architecture section, downcodes.com):
            section "Recurrent block"   : Conv1D of temporal width 4 before the RG-LRU,
                                          only 4*D parameters (depthwise);
            section "Real-Gated Linear Recurrent Unit (RG-LRU)": Eq. (1)-(4), output
                                          y_t = h_t, a = sigma(Lambda), c = 8, a^{c r_t}
                                          computed in log space, diagonal recurrence;
            section "Gate behaviour"   : r_t -> 0 keeps the previous state.
  [BLOG]  "Griffin's Compromise: Combining Gated Linear Recurrence with Local Attention"
          (ql.gl): section "Hawk: Redesigning RNN State with Gates" (h_t = a_t h_{t-1} +
          b_t x_t; generation reads and writes only the current token and a fixed-size
          state) and "Term explanation: Parallel scan".

Readings where the pages leave a step open (each also listed in the design notes):
  * x_t in Eq. (1), (2) and (4) is the conv output u; the gates and the input term both
    use u.  W is stored [out, in]: z = W u + b.
  * "log space": log a_t = c * r_t * log sigma(Lambda), log sigma computed as
    -log1p(exp(-Lambda)) (stable form); sqrt(1 - a_t^2) = sqrt(-expm1(2 log a_t)).
  * Tap k of the conv multiplies x_{t-k}; history before the first token is the given
    conv state (x_{-3}, x_{-2}, x_{-1}) or zeros.
  * Rounding points of the I/O dtype: R1 - u is rounded to the I/O dtype (nearest-even)
    and that rounded u feeds both the gates and the scan; R2 - y_t is h_t rounded to the
    I/O dtype.  The state h and h_T stay unrounded.  R1 rounds the conv sum itself
    (taken in fp64); everything else is fp64 too.
  * Backward (not on the pages): chain rule through the same definitions, R1 and R2
    treated as identity; where m_t = sqrt(1 - a_t^2) = 0 the m-path term of d(log a_t)
    is defined as 0.

The recurrent block around the branch ([ARCH] "Recurrent block", Fig. 2(c)): two linear
layers D -> D_RNN in parallel, Conv1D + RG-LRU on the first branch, GeLU on the second,
elementwise product, linear D_RNN -> D.  Readings: the linears have no bias (the pages
give none); GeLU is the exact form q Phi(q); rounding points of the I/O dtype are the
branch input p = RNE(x W_in1^T), g = RNE(GeLU(x W_in2^T)), the product z = RNE(h_t g_t)
of the unrounded RG-LRU state and g, and the block output RNE(z W_out^T).

The gated MLP block ([ARCH] "MLP block", Fig. 2(b)): two linear layers D -> M*D on the
same input (M = 3 on the pages), GeLU on the first branch, elementwise product with the
second, a final linear M*D -> D.  Readings: no biases; exact GeLU; which branch carries
the GeLU is not fixed by the pages, W_1 (the first argument) is the GeLU branch; the two
branch outputs are not rounded on their own, the product h = RNE(GeLU(x W_1^T) (x W_2^T))
is (one rounding point, where the product is formed), and the output RNE(h W_3^T).

Local (sliding-window) multi-query attention ([ARCH] "Global multi-query attention" and
"Local sliding-window attention"; window 1024 from [BLOG] "Griffin: Attention for Recent
Memory"): H query heads of width 128 (H * 128 = D) share one key head and one value head;
no absolute position embedding, RoPE on queries and keys; each position attends only to a
fixed number W of the most recent positions.  Readings: RoPE is the original pairwise form
of Su et al. - pair (2i, 2i+1) of a head vector at position p is rotated by the angle
p * 10000^(-2i/128) - applied to every dimension of q and k, p the absolute token index;
the window holds W positions including the current one, keys s with t - W < s <= t; scores
are scaled by 1/sqrt(128); the projections carry no bias; with bf16 I/O the rotated q and
k, the values v, the attention output (heads concatenated) and the block output are
rounded to bf16.

Parity pins: every function here is pinned by a test against closed forms, invariants,
brute force or library routines (tests/test_oracle_pins.py, tests/test_oracle_grad.py,
tests/test_oracle_block.py, tests/test_oracle_mlp.py, tests/test_oracle_mqa.py).
"""
from __future__ import annotations

import numpy as np
from scipy.special import erf as _erf

_BF16_MAX = 3.3895313892515355e38   # largest finite bf16
_BF16_MIN_ULP_EXP = -133            # exponent of the smallest bf16 subnormal


# ----------------------------------------------------------------------------------
# I/O rounding (R1, R2)
# ----------------------------------------------------------------------------------
def round_io(v, io: str) -> np.ndarray:
    """Round fp64 values to the I/O dtype, nearest-even, and return them as fp64.

    bf16 keeps 8 significant bits and fp32's exponent range; fp32 is IEEE single.
    """
    v = np.asarray(v, dtype=np.float64)
    if io == "f64":                    # no rounding: used only by the gradient checks
        return v.copy()
    if io == "f32":
        return v.astype(np.float32).astype(np.float64)
    if io != "bf16":
        raise ValueError(f"unknown io dtype {io!r}")
    _, e = np.frexp(v)                              # |v| = m 2^e, 0.5 <= m < 1
    ulp_exp = np.maximum(e - 8, _BF16_MIN_ULP_EXP)  # 8 significant bits
    q = np.rint(np.ldexp(v, -ulp_exp))              # rint: ties to even
    r = np.ldexp(q, ulp_exp)
    return np.where(np.abs(r) > _BF16_MAX, np.copysign(np.inf, v), r)


# ----------------------------------------------------------------------------------
# Scalar functions of Eq. (1)-(3)
# ----------------------------------------------------------------------------------
def sigmoid(z) -> np.ndarray:
    """sigma(z) = 1 / (1 + e^{-z})  ([ARCH] RG-LRU: the nonlinearity is the sigmoid).

    Evaluated without overflow: 1/(1+e^{-z}) for z >= 0, e^{z}/(1+e^{z}) for z < 0.
    """
    z = np.asarray(z, dtype=np.float64)
    out = np.empty_like(z)
    pos = z >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-z[pos]))
    ez = np.exp(z[~pos])
    out[~pos] = ez / (1.0 + ez)
    return out


def log_sigmoid(lam) -> np.ndarray:
    """log sigma(Lambda), the log of the diagonal recurrent weight a = sigma(Lambda)
    ([ARCH] RG-LRU, the parametrisation of a in Eq. (3); computed in log space)."""
    lam = np.asarray(lam, dtype=np.float64)
    return np.where(lam >= 0,
                    -np.log1p(np.exp(-np.abs(lam))),
                    lam - np.log1p(np.exp(-np.abs(lam))))


def gates(zr, zi, lam, c):
    """Eq. (1)-(3) and the input scaling of Eq. (4) from the pre-activations.

    zr = W_a u + b_a, zi = W_x u + b_x  ->  r, i, log a, a, m = sqrt(1 - a^2).
    log a_t = c * r_t * log sigma(Lambda)  (log space);  a_t = exp(log a_t);
    m_t = sqrt(1 - a_t^2) = sqrt(-expm1(2 log a_t)).
    """
    r = sigmoid(zr)
    i = sigmoid(zi)
    L = log_sigmoid(lam)
    ell = c * r * L
    a = np.exp(ell)
    m = np.sqrt(-np.expm1(2.0 * ell))
    return r, i, ell, a, m


# ----------------------------------------------------------------------------------
# Conv1D of the recurrent block
# ----------------------------------------------------------------------------------
def _history(x, conv_state_in):
    """X = [x_{-3}, x_{-2}, x_{-1}, x_0 .. x_{T-1}] along time, fp64, shape [B, T+3, D]."""
    B, T, D = x.shape
    hist = (np.zeros((B, 3, D)) if conv_state_in is None
            else np.asarray(conv_state_in, dtype=np.float64))
    return np.concatenate([hist, np.asarray(x, dtype=np.float64)], axis=1)


def conv1d_causal4(x, conv_w, conv_b, conv_state_in, io):
    """Causal depthwise Conv1D with temporal width 4 ([ARCH] "Recurrent block").

    u[b,t,d] = conv_b[d] + sum_{k=0..3} conv_w[k,d] * X[b,t-k,d], then u is rounded to
    the I/O dtype (R1).  Returns (u [B,T,D] fp64, conv_state_out [B,3,D] = the last three
    time rows of [conv_state_in || x]).

    The sum is the plain definition in fp64: each product of two fp32 (or bf16) values is
    exact in fp64, and the fp64 additions (bias first, then taps k = 0..3) leave an error
    far below the I/O rounding, so R1 rounds the sum the definition names.
    """
    x = np.asarray(x, dtype=np.float64)
    B, T, D = x.shape
    X = _history(x, conv_state_in)
    w = np.asarray(conv_w, dtype=np.float64)
    u = np.zeros((B, T, D)) if conv_b is None else np.broadcast_to(
        np.asarray(conv_b, dtype=np.float64), (B, T, D)).copy()
    for k in range(4):
        u += w[k] * X[:, 3 - k:3 - k + T, :]
    return round_io(u, io), X[:, T:T + 3, :].copy()


# ----------------------------------------------------------------------------------
# Forward
# ----------------------------------------------------------------------------------
def forward(x, conv_w, conv_b, conv_state_in, W_a, W_x, b_a, b_x, lam, h0, c, io,
            channels=None, keep=False):
    """The temporal branch forward: conv (R1) -> Eq. (1)-(4) -> y_t = h_t (R2).

    x [B,T,D]; conv_w [4,D] or None (then x is already the RG-LRU input u); conv_b [D]
    or None; conv_state_in [B,3,D] or None; W_a, W_x [D,D] ([out,in]); b_a, b_x, lam [D];
    h0 [B,D] or None (zeros).  ``channels``: optional index array S of output channels;
    every output is then restricted to S (channels are independent through the
    diagonal recurrence, so the values on S do not depend on the other outputs).

    Returns dict with y [B,T,|S|] (I/O-rounded, fp64), h_T [B,|S|] (fp64),
    conv_state_out [B,3,D]; with keep=True also u, r, i, ell, a, m, h_prev.
    """
    x = np.asarray(x, dtype=np.float64)
    B, T, D = x.shape
    S = np.arange(D) if channels is None else np.asarray(channels)
    if conv_w is None:
        u = x.copy()
        cs_out = _history(x, conv_state_in)[:, T:T + 3, :].copy()
    else:
        u, cs_out = conv1d_causal4(x, conv_w, conv_b, conv_state_in, io)
    Wa = np.asarray(W_a, dtype=np.float64)[S]
    Wx = np.asarray(W_x, dtype=np.float64)[S]
    zr = np.empty((B, T, len(S)))
    zi = np.empty((B, T, len(S)))
    for b in range(B):                                  # z = W u + b   (Eq. (1), (2))
        zr[b] = u[b] @ Wa.T
        zi[b] = u[b] @ Wx.T
    zr += np.asarray(b_a, dtype=np.float64)[S]
    zi += np.asarray(b_x, dtype=np.float64)[S]
    r, i, ell, a, m = gates(zr, zi, np.asarray(lam, dtype=np.float64)[S], c)
    uS = u[:, :, S]
    h = np.zeros((B, len(S))) if h0 is None else np.asarray(h0, dtype=np.float64)[:, S].copy()
    y = np.empty((B, T, len(S)))
    h_prev = np.empty((B, T, len(S))) if keep else None
    for t in range(T):                                   # Eq. (4), sequential in t
        if keep:
            h_prev[:, t] = h
        h = a[:, t] * h + m[:, t] * (i[:, t] * uS[:, t])
        y[:, t] = h
    out = {"y": round_io(y, io), "h_T": h, "conv_state_out": cs_out}
    if keep:
        out.update(u=u, r=r, i=i, ell=ell, a=a, m=m, h_prev=h_prev, y_exact=y)
    return out


def decode_step(x_t, conv_w, conv_b, conv_state, W_a, W_x, b_a, b_x, lam, h, c, io):
    """One generation step with the fixed-size state ([BLOG] "Hawk": generation reads and
    writes only the current token and a fixed-size state).

    x_t [B,D]; conv_state [B,3,D] (x_{t-3}, x_{t-2}, x_{t-1}); h [B,D].  The step is the
    forward above on a length-1 sequence with the carried state.
    Returns (y_t [B,D], new conv_state [B,3,D], new h [B,D]).
    """
    o = forward(np.asarray(x_t, dtype=np.float64)[:, None, :], conv_w, conv_b, conv_state,
                W_a, W_x, b_a, b_x, lam, h, c, io)
    return o["y"][:, 0, :], o["conv_state_out"], o["h_T"]


# ----------------------------------------------------------------------------------
# Backward (chain rule through the same definitions; the pages state no backward)
# ----------------------------------------------------------------------------------
def backward(x, conv_w, conv_b, conv_state_in, W_a, W_x, b_a, b_x, lam, h0, c, io,
             dy, dh_T=None):
    """Gradients of sum(dy * y) + sum(dh_T * h_T) with respect to every input.

    R1 and R2 act as identity in the backward.  Let G_t be the total derivative with
    respect to h_t: G_t = dy_t + a_{t+1} G_{t+1}, G_{T-1} = dy_{T-1} + dh_T, dh0 = a_0 G_0.
      d(log a_t) = G_t (a_t h_{t-1} - (a_t^2 / m_t) i_t u_t)   [m-path term 0 where m_t=0]
      dr = c L d(log a), dL = sum c r d(log a), dLambda = dL * sigma(-Lambda)
      dzr = dr r (1-r), dzi = G m u i (1-i), db = sum dz, dW = sum dz (x) u
      du = G m i + W_a^T dzr + W_x^T dzi
      dconv_w[k] = sum du_t X_{t-k}, dconv_b = sum du, dx_tau = sum_k w[k] du_{tau+k}.
    Returns dict dx [B,T,D], dconv_w [4,D], dconv_b [D], dW_a, dW_x [D,D], db_a, db_x,
    dlambda [D], dh0 [B,D]; all fp64.
    """
    f = forward(x, conv_w, conv_b, conv_state_in, W_a, W_x, b_a, b_x, lam, h0, c, io,
                keep=True)
    u, r, i, a, m, hp = f["u"], f["r"], f["i"], f["a"], f["m"], f["h_prev"]
    B, T, D = u.shape
    dy = np.asarray(dy, dtype=np.float64)
    g = np.zeros((B, D)) if dh_T is None else np.asarray(dh_T, dtype=np.float64).copy()
    G = np.empty((B, T, D))
    for t in range(T - 1, -1, -1):                      # reverse-time recurrence
        g = g + dy[:, t]
        G[:, t] = g
        g = a[:, t] * g
    dh0 = g
    L = log_sigmoid(lam)
    safe_m = np.where(m > 0, m, 1.0)
    m_term = np.where(m > 0, (a * a / safe_m) * i * u, 0.0)
    dell = G * (a * hp - m_term)
    dr = c * L * dell
    dL = (c * r * dell).sum(axis=(0, 1))
    dlam = dL * sigmoid(-np.asarray(lam, dtype=np.float64))
    di = G * m * u
    dzr = dr * r * (1.0 - r)
    dzi = di * i * (1.0 - i)
    Wa = np.asarray(W_a, dtype=np.float64)
    Wx = np.asarray(W_x, dtype=np.float64)
    dW_a = np.zeros((D, D))
    dW_x = np.zeros((D, D))
    du = G * m * i
    for b in range(B):
        dW_a += dzr[b].T @ u[b]
        dW_x += dzi[b].T @ u[b]
        du[b] += dzr[b] @ Wa + dzi[b] @ Wx
    out = {"dW_a": dW_a, "dW_x": dW_x, "db_a": dzr.sum(axis=(0, 1)),
           "db_x": dzi.sum(axis=(0, 1)), "dlambda": dlam, "dh0": dh0}
    if conv_w is None:
        out.update(dx=du, dconv_w=None, dconv_b=None)
        return out
    X = _history(x, conv_state_in)
    w = np.asarray(conv_w, dtype=np.float64)
    dconv_w = np.empty((4, D))
    dx = np.zeros((B, T, D))
    for k in range(4):
        dconv_w[k] = (du * X[:, 3 - k:3 - k + T, :]).sum(axis=(0, 1))
        if k < T:                      # tap k reaches x_tau from u_{tau+k}, tau + k < T
            dx[:, :T - k, :] += w[k] * du[:, k:, :]
    out.update(dx=dx, dconv_w=dconv_w, dconv_b=du.sum(axis=(0, 1)))
    return out


# ----------------------------------------------------------------------------------
# The recurrent block around the branch ([ARCH] "Recurrent block", Fig. 2(c))
# ----------------------------------------------------------------------------------
def gelu(q) -> np.ndarray:
    """GeLU of the block's second branch, exact form: q Phi(q) = q (1 + erf(q / sqrt 2)) / 2."""
    q = np.asarray(q, dtype=np.float64)
    return 0.5 * q * (1.0 + _erf(q / np.sqrt(2.0)))


def block_forward(x, W_in, conv_w, conv_b, conv_state_in, W_a, W_x, b_a, b_x, lam, h0, W_out,
                  c, io, keep=False):
    """The recurrent block: out = W_out (RG-LRU(conv(W_in1 x)) * GeLU(W_in2 x)).

    x [B,T,D]; W_in [2R, D] ([out, in]: rows 0..R-1 the recurrence branch, rows R..2R-1
    the GeLU branch); conv and RG-LRU arguments as in forward() with width R; W_out [D, R].
    Rounding points (I/O dtype, nearest even): p = RNE(x W_in1^T), g = RNE(GeLU(x W_in2^T)),
    z = RNE(h_t * g_t) with h_t the unrounded RG-LRU state, out = RNE(z W_out^T).
    Returns dict with out [B,T,D], h_T [B,R], conv_state_out [B,3,R]; with keep=True also
    p, g, z.
    """
    x = np.asarray(x, dtype=np.float64)
    W_in = np.asarray(W_in, dtype=np.float64)
    R = W_in.shape[0] // 2
    pq = x @ W_in.T                                        # the two input linears
    p = round_io(pq[..., :R], io)
    g = round_io(gelu(pq[..., R:]), io)
    f = forward(p, conv_w, conv_b, conv_state_in, W_a, W_x, b_a, b_x, lam, h0, c, io, keep=True)
    z = round_io(f["y_exact"] * g, io)
    out = round_io(z @ np.asarray(W_out, dtype=np.float64).T, io)
    res = {"out": out, "h_T": f["h_T"], "conv_state_out": f["conv_state_out"]}
    if keep:
        res.update(p=p, g=g, z=z)
    return res


def gated_mlp_forward(x, W_1, W_2, W_3, io, keep=False):
    """The gated MLP block of [ARCH] "MLP block" (Fig. 2(b)): two branches of width M*D from
    the same input, GeLU on the first, merged by an elementwise product, then a linear layer
    back to width D.

    x [..., D]; W_1, W_2 [MD, D] and W_3 [D, MD], all [out, in].  Returns out [..., D]
    (rounded to io); with keep=True a dict that also holds h = RNE(GeLU(x W_1^T) (x W_2^T)).
    """
    x = np.asarray(x, dtype=np.float64)
    q1 = x @ np.asarray(W_1, dtype=np.float64).T
    q2 = x @ np.asarray(W_2, dtype=np.float64).T
    h = round_io(gelu(q1) * q2, io)
    out = round_io(h @ np.asarray(W_3, dtype=np.float64).T, io)
    if keep:
        return {"out": out, "h": h}
    return out


# ----------------------------------------------------------------------------------
# Local multi-query attention (the second temporal-mixing block)
# ----------------------------------------------------------------------------------
HEAD_DIM = 128          # [ARCH] "Global multi-query attention": fixed head width
ROPE_BASE = 10000.0     # RoPE frequency base of Su et al.


def rope(v, positions, base=ROPE_BASE) -> np.ndarray:
    """Rotary position embedding: for each head vector v[..., t, (h,) :] at absolute
    position positions[t], pair (2i, 2i+1) is rotated by the angle positions[t] * theta_i,
    theta_i = base^(-2i/d), d the last dimension.

    v [B, T, d] or [B, T, H, d]; positions [T] (integers).
    """
    v = np.asarray(v, dtype=np.float64)
    d = v.shape[-1]
    theta = base ** (-np.arange(0, d, 2, dtype=np.float64) / d)          # [d/2]
    ang = np.asarray(positions, dtype=np.float64)[:, None] * theta[None, :]   # [T, d/2]
    if v.ndim == 4:
        ang = ang[:, None, :]
    cos, sin = np.cos(ang), np.sin(ang)
    even, odd = v[..., 0::2], v[..., 1::2]
    out = np.empty_like(v)
    out[..., 0::2] = even * cos - odd * sin
    out[..., 1::2] = even * sin + odd * cos
    return out


def local_mqa_attention(q, k, v, window, q_pos=None, kv_pos=None) -> np.ndarray:
    """Sliding-window multi-query attention.

    q [B, T, H, d] (H heads); k, v [B, S, d] (the one shared key/value head).  q_pos [T] and
    kv_pos [S] are absolute positions (default 0..T-1 and 0..S-1).  Query t attends to the
    keys s with q_pos[t] - window < kv_pos[s] <= q_pos[t], with weights
    softmax_s(q_t . k_s / sqrt(d)).  Returns [B, T, H, d]; a query with no key in its window
    gets zeros.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, T, H, d = q.shape
    S = k.shape[1]
    qp = np.arange(T) if q_pos is None else np.asarray(q_pos)
    kp = np.arange(S) if kv_pos is None else np.asarray(kv_pos)
    allowed = (kp[None, :] <= qp[:, None]) & (kp[None, :] > qp[:, None] - window)   # [T, S]
    out = np.zeros((B, T, H, d))
    for b in range(B):
        scores = np.einsum("thd,sd->ths", q[b], k[b]) / np.sqrt(d)        # [T, H, S]
        scores = np.where(allowed[:, None, :], scores, -np.inf)
        mx = scores.max(axis=-1, keepdims=True)
        mx = np.where(np.isfinite(mx), mx, 0.0)
        w = np.exp(scores - mx)
        den = w.sum(axis=-1, keepdims=True)
        w = np.divide(w, den, out=np.zeros_like(w), where=den > 0)
        out[b] = np.einsum("ths,sd->thd", w, v[b])
    return out


def local_mqa_forward(x, W_q, W_k, W_v, W_o, window, io, pos0=0, keep=False):
    """The local-MQA temporal-mixing block on x [B, T, D] at absolute positions
    pos0 .. pos0+T-1: q = x W_q^T split into H = D/128 heads, k = x W_k^T, v = x W_v^T
    (one head each), RoPE on q and k, sliding-window attention, heads concatenated, then
    x_out = attn W_o^T.  W_q [D, D], W_k, W_v [128, D], W_o [D, D], all [out, in].
    Returns out [B, T, D]; with keep=True a dict with q, k (rotated), v and attn too.
    """
    x = np.asarray(x, dtype=np.float64)
    B, T, D = x.shape
    H = D // HEAD_DIM
    pos = pos0 + np.arange(T)
    q = (x @ np.asarray(W_q, dtype=np.float64).T).reshape(B, T, H, HEAD_DIM)
    k = x @ np.asarray(W_k, dtype=np.float64).T
    v = x @ np.asarray(W_v, dtype=np.float64).T
    qr = round_io(rope(q, pos), io)
    kr = round_io(rope(k, pos), io)
    vr = round_io(v, io)
    attn = round_io(local_mqa_attention(qr, kr, vr, window, pos, pos).reshape(B, T, D), io)
    out = round_io(attn @ np.asarray(W_o, dtype=np.float64).T, io)
    if keep:
        return {"out": out, "q": qr, "k": kr, "v": vr, "attn": attn}
    return out


def local_mqa_decode_step(x_t, W_q, W_k, W_v, W_o, k_cache, v_cache, pos, window, io):
    """One generation step of the local-MQA block with a bounded key/value cache ([ARCH]
    "Local sliding-window attention": the cache never holds more than the window).

    x_t [B, D] (the token of each sequence at absolute position pos[b]); k_cache, v_cache
    [B, window, 128]: slot j holds the rotated key and the value of the most recent
    position p <= pos[b] with p % window == j (slots of positions below 0 are never read).
    The step writes the new key and value into slot pos[b] % window, then attends over the
    cached positions (pos[b] - window, pos[b]].  Returns (out [B, D], new k_cache, new
    v_cache); the inputs are not modified.
    """
    x = np.asarray(x_t, dtype=np.float64)
    B, D = x.shape
    H = D // HEAD_DIM
    pos = np.asarray(pos, dtype=np.int64)
    kc = np.array(k_cache, dtype=np.float64, copy=True)
    vc = np.array(v_cache, dtype=np.float64, copy=True)
    attn = np.zeros((B, D))
    for b in range(B):
        p = int(pos[b])
        q = (x[b] @ np.asarray(W_q, dtype=np.float64).T).reshape(1, 1, H, HEAD_DIM)
        k = (x[b] @ np.asarray(W_k, dtype=np.float64).T).reshape(1, 1, HEAD_DIM)
        v = (x[b] @ np.asarray(W_v, dtype=np.float64).T).reshape(1, 1, HEAD_DIM)
        qr = round_io(rope(q, [p]), io)
        kc[b, p % window] = round_io(rope(k, [p]), io)[0, 0]
        vc[b, p % window] = round_io(v, io)[0, 0]
        slots = np.arange(window)
        slot_pos = p - ((p - slots) % window)          # the position each slot holds
        live = slot_pos >= 0
        a = local_mqa_attention(qr, kc[b:b + 1, live], vc[b:b + 1, live], window,
                                q_pos=[p], kv_pos=slot_pos[live])
        attn[b] = round_io(a.reshape(D), io)
    out = round_io(attn @ np.asarray(W_o, dtype=np.float64).T, io)
    return out, kc, vc
