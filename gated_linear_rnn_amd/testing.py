"""Binding of the test-only entry points of librglru.so (declared in
csrc/rglru_testing.h, not in the public include/rglru.h).

Each rglru_testing_* call is the public call of the same name with the chained-scan settings
passed as an explicit first argument (the library keeps no state between calls).  Argument
marshalling only, like the public binding.
"""
from __future__ import annotations

import ctypes

import torch

from . import _binding as _b

_P, _I, _F, _Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t

EXPORTS = ("rglru_testing_default_knobs", "rglru_testing_fwd", "rglru_testing_scan",
           "rglru_testing_bwd", "rglru_testing_block_fwd")


class Knobs(ctypes.Structure):
    _fields_ = [("lru_ticket_guess", ctypes.c_int), ("scan_direct_polls", ctypes.c_int),
                ("lookback_polls", ctypes.c_int), ("lru_force_fused", ctypes.c_int)]


_declared = False


def _lib():
    global _declared
    lib = _b.load()
    if not _declared:
        kp = ctypes.POINTER(Knobs)
        lib.rglru_testing_default_knobs.argtypes = [kp]
        lib.rglru_testing_default_knobs.restype = None
        lib.rglru_testing_fwd.argtypes = [kp, _I, _I, _I, _I, _F] + [_P] * 13 + [_P, _Z, _P]
        lib.rglru_testing_fwd.restype = _I
        lib.rglru_testing_scan.argtypes = [kp, _I, _I, _I, _I] + [_P] * 9 + [_P, _Z, _P]
        lib.rglru_testing_scan.restype = _I
        lib.rglru_testing_bwd.argtypes = [kp, _I, _I, _I, _I, _F] + [_P] * 21 + [_P, _Z, _P]
        lib.rglru_testing_bwd.restype = _I
        lib.rglru_testing_block_fwd.argtypes = [kp, _I, _I, _I, _I, _I, _F] + [_P] * 15 + [_P, _Z, _P]
        lib.rglru_testing_block_fwd.restype = _I
        _declared = True
    return lib


def knobs(**over) -> Knobs:
    """The library's default settings with the named fields replaced."""
    k = Knobs()
    _lib().rglru_testing_default_knobs(ctypes.byref(k))
    for name, v in over.items():
        setattr(k, name, int(v))
    return k


def forward(k: Knobs, x, conv_w, conv_b, conv_state_in, W_a, W_x, b_a, b_x, lam, h0=None,
            c=8.0, ws=None, stream=None):
    """As gated_linear_rnn_amd.forward, through rglru_testing_fwd; returns (y, h_T, cs_out, ws)."""
    B, T, D = x.shape
    y = torch.empty_like(x)
    h_T = torch.empty((B, D), dtype=torch.float32, device=x.device)
    cs_out = torch.empty((B, 3, D), dtype=x.dtype, device=x.device) if conv_w is not None else None
    if ws is None:
        ws = _b.workspace(_b.fwd_workspace_bytes(B, T, D, x.dtype), x.device)
    P = _b._ptr
    _b._check(_lib().rglru_testing_fwd(
        ctypes.byref(k), B, T, D, _b.io_code(x.dtype), float(c), P(x), P(conv_w), P(conv_b),
        P(conv_state_in), P(W_a), P(W_x), P(b_a), P(b_x), P(lam), P(h0), P(y), P(h_T), P(cs_out),
        P(ws), ws.numel(), _b._stream(stream)), "rglru_testing_fwd")
    return y, h_T, cs_out, ws


def rglru_scan(k: Knobs, x, conv_w, conv_b, conv_state_in, a, beta, h0, y, h_T, ws, stream=None):
    B, T, D = x.shape
    P = _b._ptr
    _b._check(_lib().rglru_testing_scan(
        ctypes.byref(k), B, T, D, _b.io_code(x.dtype), P(x), P(conv_w), P(conv_b),
        P(conv_state_in), P(a), P(beta), P(h0), P(y), P(h_T), P(ws), ws.numel(),
        _b._stream(stream)), "rglru_testing_scan")


def backward(k: Knobs, x, conv_w, conv_b, conv_state_in, W_a, W_x, b_a, b_x, lam, h0, dy,
             dh_T=None, c=8.0, ws=None, stream=None):
    """As gated_linear_rnn_amd.backward, through rglru_testing_bwd; returns (grads, ws)."""
    B, T, D = x.shape
    f32 = dict(dtype=torch.float32, device=x.device)
    g = {"dx": torch.empty((B, T, D), **f32),
         "dconv_w": torch.empty((4, D), **f32) if conv_w is not None else None,
         "dconv_b": torch.empty((D,), **f32) if conv_w is not None else None,
         "dW_a": torch.empty((D, D), **f32), "dW_x": torch.empty((D, D), **f32),
         "db_a": torch.empty((D,), **f32), "db_x": torch.empty((D,), **f32),
         "dlambda": torch.empty((D,), **f32), "dh0": torch.empty((B, D), **f32)}
    if ws is None:
        ws = _b.workspace(_b.bwd_workspace_bytes(B, T, D, x.dtype), x.device)
    P = _b._ptr
    _b._check(_lib().rglru_testing_bwd(
        ctypes.byref(k), B, T, D, _b.io_code(x.dtype), float(c), P(x), P(conv_w), P(conv_b),
        P(conv_state_in), P(W_a), P(W_x), P(b_a), P(b_x), P(lam), P(h0), P(dy), P(dh_T),
        P(g["dx"]), P(g["dconv_w"]), P(g["dconv_b"]), P(g["dW_a"]), P(g["dW_x"]), P(g["db_a"]),
        P(g["db_x"]), P(g["dlambda"]), P(g["dh0"]), P(ws), ws.numel(), _b._stream(stream)),
        "rglru_testing_bwd")
    return g, ws


def block_forward(k: Knobs, x, W_in, conv_w, conv_b, conv_state_in, W_a, W_x, b_a, b_x, lam, h0,
                  W_out, c=8.0, ws=None, stream=None):
    """As gated_linear_rnn_amd.block_forward, through rglru_testing_block_fwd."""
    B, T, D = x.shape
    R = W_in.shape[0] // 2
    out = torch.empty_like(x)
    h_T = torch.empty((B, R), dtype=torch.float32, device=x.device)
    cs_out = torch.empty((B, 3, R), dtype=x.dtype, device=x.device) if conv_w is not None else None
    if ws is None:
        ws = _b.workspace(_b.block_fwd_workspace_bytes(B, T, D, R, x.dtype), x.device)
    P = _b._ptr
    _b._check(_lib().rglru_testing_block_fwd(
        ctypes.byref(k), B, T, D, R, _b.io_code(x.dtype), float(c), P(x), P(W_in), P(conv_w),
        P(conv_b), P(conv_state_in), P(W_a), P(W_x), P(b_a), P(b_x), P(lam), P(h0), P(W_out),
        P(out), P(h_T), P(cs_out), P(ws), ws.numel(), _b._stream(stream)),
        "rglru_testing_block_fwd")
    return out, h_T, cs_out
