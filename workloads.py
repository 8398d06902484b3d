"""Seeded synthetic inputs for the RG-LRU temporal branch (Conv1D width 4 -> RG-LRU) and
the recurrent block around it.

This module holds no arithmetic of the layer itself: it only draws the inputs that
both the CPU oracle and the HIP path consume, so that the two sides see the very same
host arrays.  Nothing here is trained or loaded from a dataset; every array is drawn
from ``numpy.random.default_rng(seed)`` (PCG64).

Sources for the recipe (the Griffin model-architecture page, "Recurrent block" and
"Real-Gated Linear Recurrent Unit (RG-LRU)" sections):
  * conv filter width 4, depthwise over the D_RNN-wide branch;
  * W_a and W_x use LeCun initialisation: N(0, 1/fan_in), fan_in = D_RNN;
  * Lambda is initialised so that a^c = sigma(Lambda)^c is uniform in [0.9, 0.999], c = 8.
The training shapes stand in for the 2048-token language-model training sequences and
the batched decode the pages describe; no public dataset is used.

Draw order (fixed, so a config is reproducible from its seed):
  x, conv_w, W_a, W_x, b_a, b_x, U_lambda, h0, conv_history, then dy or decode tokens.
Each draw is fp64, cast to fp32, and for bf16 I/O tensors rounded (nearest-even) to
bf16.  Arrays are returned as fp32 numpy arrays whose values are exactly representable
in the I/O dtype; Lambda, biases, h0 are always fp32.
"""
from __future__ import annotations

import dataclasses
import numpy as np

C_DEFAULT = 8.0  # the scalar constant c of the RG-LRU (set to 8 on the pages)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int                 # sequence length (decode: number of steps)
    D: int                 # D_RNN
    io: str                # "f32" or "bf16"
    seed: int
    bias_std: float        # std of b_a, b_x (0 means the biases are exactly zero)
    ac_lo: float           # a^c ~ U[ac_lo, ac_hi]
    ac_hi: float
    h0: str                # "zero" or "normal"
    history: str           # "zero" or "normal" (conv history before the first token)
    decode: bool = False
    with_dy: bool = False

    def with_shape(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads, each named by what it is and its sizes.
TINY_F32 = Workload("tiny_fwd_f32_B1_T256_D256", 1, 256, 256, "f32", 0, 0.0, 0.9, 0.999, "zero", "zero")
TRAIN_FWD = Workload("train_fwd_bf16_B8_T2048_D2560", 8, 2048, 2560, "bf16", 1, 0.1, 0.9, 0.999, "zero", "zero")
DECODE = Workload("decode_bf16_B256_D2560_steps1024", 256, 1024, 2560, "bf16", 2, 0.1, 0.9, 0.999,
                  "normal", "normal", decode=True)
LONG_FWD = Workload("long_fwd_bf16_B2_T32768_D4096", 2, 32768, 4096, "bf16", 3, 0.1, 0.999, 0.9999,
                    "normal", "zero")
TRAIN_BWD = Workload("train_fwdbwd_bf16_B4_T2048_D5376", 4, 2048, 5376, "bf16", 4, 0.1, 0.9, 0.999,
                     "zero", "zero", with_dy=True)

ALL = [TINY_F32, TRAIN_FWD, DECODE, LONG_FWD, TRAIN_BWD]


def bf16_round(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); returns fp32 holding them.

    Input preparation only (the draws of bf16 tensors); inputs are finite.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    bits = a.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    bits = (bits + 0x7FFF + lsb) & 0xFFFF0000
    return bits.astype(np.uint32).view(np.float32)


def _normal(rng, shape, std, io, block_rows=4096):
    """N(0, std^2) drawn in fp64 (in row blocks to bound memory), stored fp32 / bf16."""
    shape = tuple(int(s) for s in shape)
    out = np.empty(shape, dtype=np.float32)
    flat = out.reshape(-1, shape[-1]) if len(shape) > 1 else out.reshape(1, -1)
    for r0 in range(0, flat.shape[0], block_rows):
        r1 = min(flat.shape[0], r0 + block_rows)
        blk = rng.standard_normal((r1 - r0, flat.shape[1])) * std
        blk = blk.astype(np.float32)
        if io == "bf16":
            blk = bf16_round(blk)
        flat[r0:r1] = blk
    return out


def make_inputs(w: Workload, c: float = C_DEFAULT) -> dict:
    """Draw every input of workload ``w`` from ``default_rng(w.seed)``.

    Returns fp32 numpy arrays:
      x [B,T,D] (io-exact; decode: tokens [T,B,D]), conv_w [4,D] (io-exact), conv_b [D] (zeros),
      W_a, W_x [D,D] (io-exact, [out,in]), b_a, b_x [D], lam [D], h0 [B,D] or None,
      conv_state [B,3,D] (io-exact) or None, dy [B,T,D] (io-exact) or None.
    """
    rng = np.random.default_rng(w.seed)
    B, T, D, io = w.B, w.T, w.D, w.io
    out: dict = {"workload": w, "c": float(c)}
    if not w.decode:
        out["x"] = _normal(rng, (B, T, D), 1.0, io)
    out["conv_w"] = _normal(rng, (4, D), 0.5, io)          # N(0, 1/4): LeCun with fan_in 4
    out["conv_b"] = np.zeros(D, dtype=np.float32)
    out["W_a"] = _normal(rng, (D, D), 1.0 / np.sqrt(D), io)  # LeCun-normal, fan_in = D
    out["W_x"] = _normal(rng, (D, D), 1.0 / np.sqrt(D), io)
    if w.bias_std > 0:
        out["b_a"] = (rng.standard_normal(D) * w.bias_std).astype(np.float32)
        out["b_x"] = (rng.standard_normal(D) * w.bias_std).astype(np.float32)
    else:
        out["b_a"] = np.zeros(D, dtype=np.float32)
        out["b_x"] = np.zeros(D, dtype=np.float32)
    # a^c ~ U[lo, hi]  =>  a = U^(1/c),  Lambda = logit(a)   (computed in fp64, stored fp32)
    U = rng.uniform(w.ac_lo, w.ac_hi, size=D)
    a = U ** (1.0 / c)
    out["lam"] = (np.log(a) - np.log1p(-a)).astype(np.float32)
    out["h0"] = (rng.standard_normal((B, D)).astype(np.float32) if w.h0 == "normal" else None)
    out["conv_state"] = (_normal(rng, (B, 3, D), 1.0, io) if w.history == "normal" else None)
    if w.decode:
        out["x"] = _normal(rng, (T, B, D), 1.0, io)        # one token per sequence per step
    out["dy"] = _normal(rng, (B, T, D), 1.0, io) if w.with_dy else None
    return out


def extra_inputs_x(w: Workload, k: int) -> np.ndarray:
    """Input set k >= 1 of workload w for rotation in timing loops: x only, drawn the same
    way as x from default_rng(w.seed + 1000 k) (set 0 is make_inputs(w)["x"])."""
    rng = np.random.default_rng(w.seed + 1000 * k)
    return _normal(rng, (w.B, w.T, w.D), 1.0, w.io)


def make_block_inputs(w: Workload, d_model: int | None = None, c: float = C_DEFAULT) -> dict:
    """Inputs of the whole recurrent block around the branch of workload ``w`` (R = w.D is
    D_RNN, the branch width; d_model is the model width D, default D_RNN).

    The branch parameters are make_inputs(w)'s; the block's own arrays come from a second
    stream, default_rng(w.seed + 7919), in this order: x_block [B,T,D] ~ N(0,1),
    W_in [2R, D] ~ N(0, 1/D) (LeCun, fan_in = D; rows 0..R-1 feed the branch, rows R..2R-1
    the GeLU side), W_out [D, R] ~ N(0, 1/R) (LeCun, fan_in = R).  All io-exact fp32.
    """
    D = int(d_model or w.D)
    R = w.D
    out = make_inputs(w, c)
    rng = np.random.default_rng(w.seed + 7919)
    out["d_model"] = D
    out["x_block"] = _normal(rng, (w.B, w.T, D), 1.0, w.io)
    out["W_in"] = _normal(rng, (2 * R, D), 1.0 / np.sqrt(D), w.io)
    out["W_out"] = _normal(rng, (D, R), 1.0 / np.sqrt(R), w.io)
    return out


def make_mlp_inputs(w: Workload, expansion: int = 3) -> dict:
    """Inputs of the gated MLP block at model width D = w.D with hidden width
    expansion * D (M = 3 on the pages), from default_rng(w.seed + 104729) in this order:
    x [B,T,D] ~ N(0,1), W_1 and W_2 [MD, D] ~ N(0, 1/D), W_3 [D, MD] ~ N(0, 1/(MD))
    (LeCun, fan_in = D resp. MD).  All io-exact fp32."""
    D = w.D
    MD = expansion * D
    rng = np.random.default_rng(w.seed + 104729)
    return {"workload": w, "expansion": expansion,
            "x": _normal(rng, (w.B, w.T, D), 1.0, w.io),
            "W_1": _normal(rng, (MD, D), 1.0 / np.sqrt(D), w.io),
            "W_2": _normal(rng, (MD, D), 1.0 / np.sqrt(D), w.io),
            "W_3": _normal(rng, (D, MD), 1.0 / np.sqrt(MD), w.io)}


def make_mqa_inputs(w: Workload, window: int = 1024) -> dict:
    """Inputs of the local-MQA block at model width D = w.D (H = D / 128 heads) from
    default_rng(w.seed + 15485863) in this order: x [B,T,D] ~ N(0,1), W_q [D, D],
    W_k, W_v [128, D] ~ N(0, 1/D) (LeCun, fan_in = D), W_o [D, D] ~ N(0, 1/D).  All io-exact
    fp32; ``window`` is the attention window (1024 on the pages)."""
    D = w.D
    rng = np.random.default_rng(w.seed + 15485863)
    return {"workload": w, "window": int(window),
            "x": _normal(rng, (w.B, w.T, D), 1.0, w.io),
            "W_q": _normal(rng, (D, D), 1.0 / np.sqrt(D), w.io),
            "W_k": _normal(rng, (128, D), 1.0 / np.sqrt(D), w.io),
            "W_v": _normal(rng, (128, D), 1.0 / np.sqrt(D), w.io),
            "W_o": _normal(rng, (D, D), 1.0 / np.sqrt(D), w.io)}
