"""ctypes binding of librglru.so: the same entry points as include/rglru.h.

Argument marshalling only: every step of the temporal branch runs in the HIP kernels of
librglru.so.  Tensors are torch tensors already on the GPU (torch provides device memory
and the stream); there is no fallback path: if the library is missing, load() raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librglru.so")

RGLRU_F32, RGLRU_BF16 = 0, 1
RGLRU_ESTALL = -7
_IO = {torch.float32: RGLRU_F32, torch.bfloat16: RGLRU_BF16}

# Symbols declared in include/rglru.h.
EXPORTS = ("rglru_status_string", "conv1d_causal4", "rglru_fwd_workspace_bytes", "rglru_fwd",
           "rglru_lru_workspace_bytes", "rglru_lru", "rglru_gates", "rglru_scan_workspace_bytes",
           "rglru_scan",
           "rglru_decode_workspace_bytes", "rglru_decode_step", "rglru_bwd_workspace_bytes",
           "rglru_bwd", "rglru_block_fwd_workspace_bytes", "rglru_block_fwd",
           "gated_mlp_fwd_workspace_bytes", "gated_mlp_fwd", "local_mqa_fwd_workspace_bytes",
           "local_mqa_fwd", "local_mqa_decode_workspace_bytes", "local_mqa_decode_step",
           "rglru_block_decode_workspace_bytes", "rglru_block_decode_step",
           "rglru_workspace_status", "rglru_decode_step_noalloc", "rglru_train_saved_bytes",
           "rglru_fwd_train_workspace_bytes", "rglru_fwd_train", "rglru_bwd_saved_workspace_bytes",
           "rglru_bwd_saved")

_lib = None
_P, _I, _F, _Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t


class RgluError(RuntimeError):
    pass


def load(path: str = LIB_PATH):
    """Load librglru.so (once) and declare every entry point's signature."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RgluError(f"{path} is not built; run `python -m gated_linear_rnn_amd.build`")
    lib = ctypes.CDLL(path)
    lib.rglru_status_string.argtypes = [_I]
    lib.rglru_status_string.restype = ctypes.c_char_p
    lib.conv1d_causal4.argtypes = [_I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P]
    lib.conv1d_causal4.restype = _I
    lib.rglru_fwd_workspace_bytes.argtypes = [_I, _I, _I, _I]
    lib.rglru_fwd_workspace_bytes.restype = _Z
    lib.rglru_fwd.argtypes = [_I, _I, _I, _I, _F] + [_P] * 13 + [_P, _Z, _P]
    lib.rglru_fwd.restype = _I
    lib.rglru_lru_workspace_bytes.argtypes = [_I, _I, _I, _I]
    lib.rglru_lru_workspace_bytes.restype = _Z
    lib.rglru_lru.argtypes = [_I, _I, _I, _I, _F] + [_P] * 9 + [_P, _Z, _P]
    lib.rglru_lru.restype = _I
    lib.rglru_gates.argtypes = [_I, _I, _I, _I, _F] + [_P] * 8 + [_P]
    lib.rglru_gates.restype = _I
    lib.rglru_scan_workspace_bytes.argtypes = [_I, _I, _I, _I]
    lib.rglru_scan_workspace_bytes.restype = _Z
    lib.rglru_scan.argtypes = [_I, _I, _I, _I] + [_P] * 9 + [_P, _Z, _P]
    lib.rglru_scan.restype = _I
    lib.rglru_workspace_status.argtypes = [_P, _Z, _P]
    lib.rglru_workspace_status.restype = _I
    lib.rglru_decode_workspace_bytes.argtypes = [_I, _I, _I]
    lib.rglru_decode_workspace_bytes.restype = _Z
    lib.rglru_decode_step.argtypes = [_I, _I, _I, _F] + [_P] * 11 + [_P, _Z, _P]
    lib.rglru_decode_step.restype = _I
    lib.rglru_decode_step_noalloc.argtypes = [_I, _I, _I, _F] + [_P] * 11 + [_P]
    lib.rglru_decode_step_noalloc.restype = _I
    lib.rglru_bwd_workspace_bytes.argtypes = [_I, _I, _I, _I]
    lib.rglru_bwd_workspace_bytes.restype = _Z
    lib.rglru_bwd.argtypes = [_I, _I, _I, _I, _F] + [_P] * 21 + [_P, _Z, _P]
    lib.rglru_bwd.restype = _I
    for q in ("rglru_train_saved_bytes", "rglru_fwd_train_workspace_bytes",
              "rglru_bwd_saved_workspace_bytes"):
        getattr(lib, q).argtypes = [_I, _I, _I, _I]
        getattr(lib, q).restype = _Z
    lib.rglru_fwd_train.argtypes = [_I, _I, _I, _I, _F] + [_P] * 13 + [_P, _Z, _P, _Z, _P]
    lib.rglru_fwd_train.restype = _I
    lib.rglru_bwd_saved.argtypes = [_I, _I, _I, _I, _F] + [_P] * 19 + [_P, _Z, _P, _Z, _P]
    lib.rglru_bwd_saved.restype = _I
    lib.rglru_block_fwd_workspace_bytes.argtypes = [_I, _I, _I, _I, _I]
    lib.rglru_block_fwd_workspace_bytes.restype = _Z
    lib.rglru_block_fwd.argtypes = [_I, _I, _I, _I, _I, _F] + [_P] * 15 + [_P, _Z, _P]
    lib.rglru_block_fwd.restype = _I
    lib.gated_mlp_fwd_workspace_bytes.argtypes = [_I, _I, _I, _I, _I]
    lib.gated_mlp_fwd_workspace_bytes.restype = _Z
    lib.gated_mlp_fwd.argtypes = [_I, _I, _I, _I, _I] + [_P] * 5 + [_P, _Z, _P]
    lib.gated_mlp_fwd.restype = _I
    lib.local_mqa_fwd_workspace_bytes.argtypes = [_I, _I, _I, _I]
    lib.local_mqa_fwd_workspace_bytes.restype = _Z
    lib.local_mqa_fwd.argtypes = [_I, _I, _I, _I, _I, _I] + [_P] * 6 + [_P, _Z, _P]
    lib.local_mqa_fwd.restype = _I
    lib.local_mqa_decode_workspace_bytes.argtypes = [_I, _I, _I]
    lib.local_mqa_decode_workspace_bytes.restype = _Z
    lib.local_mqa_decode_step.argtypes = [_I, _I, _I, _I] + [_P] * 7 + [_P, _Z, _P]
    lib.local_mqa_decode_step.restype = _I
    lib.rglru_block_decode_workspace_bytes.argtypes = [_I, _I, _I, _I]
    lib.rglru_block_decode_workspace_bytes.restype = _Z
    lib.rglru_block_decode_step.argtypes = [_I, _I, _I, _I, _F] + [_P] * 13 + [_P, _Z, _P]
    lib.rglru_block_decode_step.restype = _I
    _lib = lib
    return lib


def status_string(code: int) -> str:
    return load().rglru_status_string(int(code)).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(code: int, what: str):
    if code != 0:
        raise RgluError(f"{what} failed: {status_string(code)} ({code})")


def io_code(dtype) -> int:
    if dtype not in _IO:
        raise RgluError(f"unsupported I/O dtype {dtype}")
    return _IO[dtype]


# ------------------------------------------------------------------ workspace queries
def fwd_workspace_bytes(B, T, D, dtype) -> int:
    return int(load().rglru_fwd_workspace_bytes(B, T, D, io_code(dtype)))


def lru_workspace_bytes(B, T, D, dtype) -> int:
    return int(load().rglru_lru_workspace_bytes(B, T, D, io_code(dtype)))


def scan_workspace_bytes(B, T, D, dtype) -> int:
    return int(load().rglru_scan_workspace_bytes(B, T, D, io_code(dtype)))


def decode_workspace_bytes(B, D, dtype) -> int:
    return int(load().rglru_decode_workspace_bytes(B, D, io_code(dtype)))


def bwd_workspace_bytes(B, T, D, dtype) -> int:
    return int(load().rglru_bwd_workspace_bytes(B, T, D, io_code(dtype)))


def train_saved_bytes(B, T, D, dtype) -> int:
    return int(load().rglru_train_saved_bytes(B, T, D, io_code(dtype)))


def fwd_train_workspace_bytes(B, T, D, dtype) -> int:
    return int(load().rglru_fwd_train_workspace_bytes(B, T, D, io_code(dtype)))


def bwd_saved_workspace_bytes(B, T, D, dtype) -> int:
    return int(load().rglru_bwd_saved_workspace_bytes(B, T, D, io_code(dtype)))


def block_fwd_workspace_bytes(B, T, D, R, dtype) -> int:
    return int(load().rglru_block_fwd_workspace_bytes(B, T, D, R, io_code(dtype)))


def mlp_fwd_workspace_bytes(B, T, D, MD, dtype) -> int:
    return int(load().gated_mlp_fwd_workspace_bytes(B, T, D, MD, io_code(dtype)))


def mqa_fwd_workspace_bytes(B, T, D, dtype) -> int:
    return int(load().local_mqa_fwd_workspace_bytes(B, T, D, io_code(dtype)))


def mqa_decode_workspace_bytes(B, D, dtype) -> int:
    return int(load().local_mqa_decode_workspace_bytes(B, D, io_code(dtype)))


def block_decode_workspace_bytes(B, D, R, dtype) -> int:
    return int(load().rglru_block_decode_workspace_bytes(B, D, R, io_code(dtype)))


def workspace(nbytes: int, device="cuda") -> torch.Tensor:
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


# ------------------------------------------------------------------ entry points
def conv1d_causal4(x, w, b, state_in, u, state_out, stream=None):
    B, T, D = x.shape
    _check(load().conv1d_causal4(B, T, D, io_code(x.dtype), _ptr(x), _ptr(w), _ptr(b),
                                 _ptr(state_in), _ptr(u), _ptr(state_out), _stream(stream)),
           "conv1d_causal4")


def rglru_fwd(x, conv_w, conv_b, conv_state_in, W_a, W_x, b_a, b_x, lam, h0, y, h_T,
              conv_state_out, ws, c=8.0, stream=None):
    B, T, D = x.shape
    _check(load().rglru_fwd(B, T, D, io_code(x.dtype), float(c), _ptr(x), _ptr(conv_w),
                            _ptr(conv_b), _ptr(conv_state_in), _ptr(W_a), _ptr(W_x), _ptr(b_a),
                            _ptr(b_x), _ptr(lam), _ptr(h0), _ptr(y), _ptr(h_T),
                            _ptr(conv_state_out), _ptr(ws), ws.numel(), _stream(stream)),
           "rglru_fwd")


def rglru_lru(u, W_a, W_x, b_a, b_x, lam, h0, y, h_T, ws, c=8.0, stream=None):
    B, T, D = u.shape
    _check(load().rglru_lru(B, T, D, io_code(u.dtype), float(c), _ptr(u), _ptr(W_a), _ptr(W_x),
                            _ptr(b_a), _ptr(b_x), _ptr(lam), _ptr(h0), _ptr(y), _ptr(h_T),
                            _ptr(ws), ws.numel(), _stream(stream)),
           "rglru_lru")


def rglru_gates(u, W_a, W_x, b_a, b_x, lam, a, beta, c=8.0, stream=None):
    B, T, D = u.shape
    _check(load().rglru_gates(B, T, D, io_code(u.dtype), float(c), _ptr(u), _ptr(W_a), _ptr(W_x),
                              _ptr(b_a), _ptr(b_x), _ptr(lam), _ptr(a), _ptr(beta),
                              _stream(stream)),
           "rglru_gates")


def rglru_scan(x, conv_w, conv_b, conv_state_in, a, beta, h0, y, h_T, ws, stream=None):
    B, T, D = x.shape
    _check(load().rglru_scan(B, T, D, io_code(x.dtype), _ptr(x), _ptr(conv_w), _ptr(conv_b),
                             _ptr(conv_state_in), _ptr(a), _ptr(beta), _ptr(h0), _ptr(y),
                             _ptr(h_T), _ptr(ws), ws.numel(), _stream(stream)),
           "rglru_scan")


def rglru_workspace_status(ws, stream=None) -> int:
    """RGLRU_OK (0) or RGLRU_ESTALL (-7) for the chained scans of the last call on `ws`
    (synchronises the stream).  Other negative codes raise."""
    code = int(load().rglru_workspace_status(_ptr(ws), ws.numel(), _stream(stream)))
    if code not in (0, RGLRU_ESTALL):
        _check(code, "rglru_workspace_status")
    return code


def rglru_decode_step(x_t, conv_w, conv_b, conv_state, W_a, W_x, b_a, b_x, lam, h, y_t, ws,
                      c=8.0, stream=None):
    B, D = x_t.shape
    _check(load().rglru_decode_step(B, D, io_code(x_t.dtype), float(c), _ptr(x_t), _ptr(conv_w),
                                    _ptr(conv_b), _ptr(conv_state), _ptr(W_a), _ptr(W_x),
                                    _ptr(b_a), _ptr(b_x), _ptr(lam), _ptr(h), _ptr(y_t),
                                    _ptr(ws), ws.numel(), _stream(stream)),
           "rglru_decode_step")


def rglru_decode_step_noalloc(x_t, conv_w, conv_b, conv_state, W_a, W_x, b_a, b_x, lam, h, y_t,
                              c=8.0, stream=None):
    """rglru_decode_step without a workspace (the library's fixed per-GPU scratch)."""
    B, D = x_t.shape
    _check(load().rglru_decode_step_noalloc(B, D, io_code(x_t.dtype), float(c), _ptr(x_t),
                                            _ptr(conv_w), _ptr(conv_b), _ptr(conv_state),
                                            _ptr(W_a), _ptr(W_x), _ptr(b_a), _ptr(b_x), _ptr(lam),
                                            _ptr(h), _ptr(y_t), _stream(stream)),
           "rglru_decode_step_noalloc")


NOALLOC_SCRATCH_BYTES = 32 << 20


def rglru_bwd(x, conv_w, conv_b, conv_state_in, W_a, W_x, b_a, b_x, lam, h0, dy, dh_T, dx,
              dconv_w, dconv_b, dW_a, dW_x, db_a, db_x, dlam, dh0, ws, c=8.0, stream=None):
    B, T, D = x.shape
    _check(load().rglru_bwd(B, T, D, io_code(x.dtype), float(c), _ptr(x), _ptr(conv_w),
                            _ptr(conv_b), _ptr(conv_state_in), _ptr(W_a), _ptr(W_x), _ptr(b_a),
                            _ptr(b_x), _ptr(lam), _ptr(h0), _ptr(dy), _ptr(dh_T), _ptr(dx),
                            _ptr(dconv_w), _ptr(dconv_b), _ptr(dW_a), _ptr(dW_x), _ptr(db_a),
                            _ptr(db_x), _ptr(dlam), _ptr(dh0), _ptr(ws), ws.numel(),
                            _stream(stream)),
           "rglru_bwd")


def rglru_fwd_train(x, conv_w, conv_b, conv_state_in, W_a, W_x, b_a, b_x, lam, h0, y, h_T,
                    conv_state_out, saved, ws, c=8.0, stream=None):
    B, T, D = x.shape
    _check(load().rglru_fwd_train(B, T, D, io_code(x.dtype), float(c), _ptr(x), _ptr(conv_w),
                                  _ptr(conv_b), _ptr(conv_state_in), _ptr(W_a), _ptr(W_x),
                                  _ptr(b_a), _ptr(b_x), _ptr(lam), _ptr(h0), _ptr(y), _ptr(h_T),
                                  _ptr(conv_state_out), _ptr(saved), saved.numel(), _ptr(ws),
                                  ws.numel(), _stream(stream)),
           "rglru_fwd_train")


def rglru_bwd_saved(x, conv_w, conv_b, conv_state_in, W_a, W_x, lam, h0, dy, dh_T, dx, dconv_w,
                    dconv_b, dW_a, dW_x, db_a, db_x, dlam, dh0, saved, ws, c=8.0, stream=None):
    B, T, D = x.shape
    _check(load().rglru_bwd_saved(B, T, D, io_code(x.dtype), float(c), _ptr(x), _ptr(conv_w),
                                  _ptr(conv_b), _ptr(conv_state_in), _ptr(W_a), _ptr(W_x),
                                  _ptr(lam), _ptr(h0), _ptr(dy), _ptr(dh_T), _ptr(dx),
                                  _ptr(dconv_w), _ptr(dconv_b), _ptr(dW_a), _ptr(dW_x),
                                  _ptr(db_a), _ptr(db_x), _ptr(dlam), _ptr(dh0), _ptr(saved),
                                  saved.numel(), _ptr(ws), ws.numel(), _stream(stream)),
           "rglru_bwd_saved")


def rglru_block_fwd(x, W_in, conv_w, conv_b, conv_state_in, W_a, W_x, b_a, b_x, lam, h0, W_out,
                    out, h_T, conv_state_out, ws, c=8.0, stream=None):
    B, T, D = x.shape
    R = W_in.shape[0] // 2
    _check(load().rglru_block_fwd(B, T, D, R, io_code(x.dtype), float(c), _ptr(x), _ptr(W_in),
                                  _ptr(conv_w), _ptr(conv_b), _ptr(conv_state_in), _ptr(W_a),
                                  _ptr(W_x), _ptr(b_a), _ptr(b_x), _ptr(lam), _ptr(h0),
                                  _ptr(W_out), _ptr(out), _ptr(h_T), _ptr(conv_state_out),
                                  _ptr(ws), ws.numel(), _stream(stream)),
           "rglru_block_fwd")


def gated_mlp_fwd(x, W_1, W_2, W_3, out, ws, stream=None):
    B, T, D = x.shape
    MD = W_1.shape[0]
    _check(load().gated_mlp_fwd(B, T, D, MD, io_code(x.dtype), _ptr(x), _ptr(W_1), _ptr(W_2),
                                _ptr(W_3), _ptr(out), _ptr(ws), ws.numel(), _stream(stream)),
           "gated_mlp_fwd")


def local_mqa_fwd(x, W_qkv, W_o, out, k_out, v_out, ws, window=1024, pos0=0, stream=None):
    B, T, D = x.shape
    _check(load().local_mqa_fwd(B, T, D, io_code(x.dtype), int(window), int(pos0), _ptr(x),
                                _ptr(W_qkv), _ptr(W_o), _ptr(out), _ptr(k_out), _ptr(v_out),
                                _ptr(ws), ws.numel(), _stream(stream)),
           "local_mqa_fwd")


def local_mqa_decode_step(pos, x_t, W_qkv, W_o, k_cache, v_cache, out, ws, stream=None):
    """pos: int32 device tensor [B]; k_cache, v_cache [B, window, 128] (updated in place)."""
    B, D = x_t.shape
    window = k_cache.shape[1]
    _check(load().local_mqa_decode_step(B, D, io_code(x_t.dtype), int(window), _ptr(pos), _ptr(x_t),
                                        _ptr(W_qkv), _ptr(W_o), _ptr(k_cache), _ptr(v_cache),
                                        _ptr(out), _ptr(ws), ws.numel(), _stream(stream)),
           "local_mqa_decode_step")


def rglru_block_decode_step(x_t, W_in, conv_w, conv_b, conv_state, W_a, W_x, b_a, b_x, lam, h, W_out,
                            out_t, ws, c=8.0, stream=None):
    B, D = x_t.shape
    R = W_in.shape[0] // 2
    _check(load().rglru_block_decode_step(B, D, R, io_code(x_t.dtype), float(c), _ptr(x_t), _ptr(W_in),
                                          _ptr(conv_w), _ptr(conv_b), _ptr(conv_state), _ptr(W_a),
                                          _ptr(W_x), _ptr(b_a), _ptr(b_x), _ptr(lam), _ptr(h),
                                          _ptr(W_out), _ptr(out_t), _ptr(ws), ws.numel(),
                                          _stream(stream)),
           "rglru_block_decode_step")


# ------------------------------------------------------------------ allocating helpers
def forward(x, conv_w, conv_b, conv_state_in, W_a, W_x, b_a, b_x, lam, h0=None, c=8.0,
            ws=None, stream=None):
    """Allocate y, h_T, conv_state_out (and the workspace unless given), run rglru_fwd."""
    B, T, D = x.shape
    y = torch.empty_like(x)
    h_T = torch.empty((B, D), dtype=torch.float32, device=x.device)
    cs_out = torch.empty((B, 3, D), dtype=x.dtype, device=x.device) if conv_w is not None else None
    if ws is None:
        ws = workspace(fwd_workspace_bytes(B, T, D, x.dtype), x.device)
    rglru_fwd(x, conv_w, conv_b, conv_state_in, W_a, W_x, b_a, b_x, lam, h0, y, h_T, cs_out, ws,
              c, stream)
    return y, h_T, cs_out


def forward_train(x, conv_w, conv_b, conv_state_in, W_a, W_x, b_a, b_x, lam, h0=None, c=8.0,
                  ws=None, saved=None, stream=None):
    """Allocate y, h_T, conv_state_out and the saved activations (and the workspace unless
    given), run rglru_fwd_train; returns (y, h_T, conv_state_out, saved)."""
    B, T, D = x.shape
    y = torch.empty_like(x)
    h_T = torch.empty((B, D), dtype=torch.float32, device=x.device)
    cs_out = torch.empty((B, 3, D), dtype=x.dtype, device=x.device) if conv_w is not None else None
    if ws is None:
        ws = workspace(fwd_train_workspace_bytes(B, T, D, x.dtype), x.device)
    if saved is None:
        saved = workspace(train_saved_bytes(B, T, D, x.dtype), x.device)
    rglru_fwd_train(x, conv_w, conv_b, conv_state_in, W_a, W_x, b_a, b_x, lam, h0, y, h_T, cs_out,
                    saved, ws, c, stream)
    return y, h_T, cs_out, saved


def backward(x, conv_w, conv_b, conv_state_in, W_a, W_x, b_a, b_x, lam, h0, dy, dh_T=None,
             c=8.0, ws=None, stream=None, saved=None):
    """Allocate every gradient (fp32) and run rglru_bwd, or rglru_bwd_saved when `saved`
    (from forward_train) is given; returns a dict."""
    B, T, D = x.shape
    dev = x.device
    f32 = dict(dtype=torch.float32, device=dev)
    g = {"dx": torch.empty((B, T, D), **f32),
         "dconv_w": torch.empty((4, D), **f32) if conv_w is not None else None,
         "dconv_b": torch.empty((D,), **f32) if conv_w is not None else None,
         "dW_a": torch.empty((D, D), **f32), "dW_x": torch.empty((D, D), **f32),
         "db_a": torch.empty((D,), **f32), "db_x": torch.empty((D,), **f32),
         "dlambda": torch.empty((D,), **f32), "dh0": torch.empty((B, D), **f32)}
    if saved is not None:
        if ws is None:
            ws = workspace(bwd_saved_workspace_bytes(B, T, D, x.dtype), dev)
        rglru_bwd_saved(x, conv_w, conv_b, conv_state_in, W_a, W_x, lam, h0, dy, dh_T, g["dx"],
                        g["dconv_w"], g["dconv_b"], g["dW_a"], g["dW_x"], g["db_a"], g["db_x"],
                        g["dlambda"], g["dh0"], saved, ws, c, stream)
        return g
    if ws is None:
        ws = workspace(bwd_workspace_bytes(B, T, D, x.dtype), dev)
    rglru_bwd(x, conv_w, conv_b, conv_state_in, W_a, W_x, b_a, b_x, lam, h0, dy, dh_T, g["dx"],
              g["dconv_w"], g["dconv_b"], g["dW_a"], g["dW_x"], g["db_a"], g["db_x"],
              g["dlambda"], g["dh0"], ws, c, stream)
    return g


def block_forward(x, W_in, conv_w, conv_b, conv_state_in, W_a, W_x, b_a, b_x, lam, h0, W_out,
                  c=8.0, ws=None, stream=None):
    """Allocate out, h_T, conv_state_out (and the workspace unless given), run rglru_block_fwd."""
    B, T, D = x.shape
    R = W_in.shape[0] // 2
    out = torch.empty_like(x)
    h_T = torch.empty((B, R), dtype=torch.float32, device=x.device)
    cs_out = torch.empty((B, 3, R), dtype=x.dtype, device=x.device) if conv_w is not None else None
    if ws is None:
        ws = workspace(block_fwd_workspace_bytes(B, T, D, R, x.dtype), x.device)
    rglru_block_fwd(x, W_in, conv_w, conv_b, conv_state_in, W_a, W_x, b_a, b_x, lam, h0, W_out,
                    out, h_T, cs_out, ws, c, stream)
    return out, h_T, cs_out


def mlp_forward(x, W_1, W_2, W_3, ws=None, stream=None):
    """Allocate out (and the workspace unless given), run gated_mlp_fwd."""
    B, T, D = x.shape
    out = torch.empty_like(x)
    if ws is None:
        ws = workspace(mlp_fwd_workspace_bytes(B, T, D, W_1.shape[0], x.dtype), x.device)
    gated_mlp_fwd(x, W_1, W_2, W_3, out, ws, stream)
    return out


def mqa_forward(x, W_qkv, W_o, window=1024, pos0=0, with_kv=False, ws=None, stream=None):
    """Allocate out (and k, v when with_kv; the workspace unless given), run local_mqa_fwd."""
    B, T, D = x.shape
    out = torch.empty_like(x)
    k = torch.empty((B, T, 128), dtype=x.dtype, device=x.device) if with_kv else None
    v = torch.empty((B, T, 128), dtype=x.dtype, device=x.device) if with_kv else None
    if ws is None:
        ws = workspace(mqa_fwd_workspace_bytes(B, T, D, x.dtype), x.device)
    local_mqa_fwd(x, W_qkv, W_o, out, k, v, ws, window, pos0, stream)
    return (out, k, v) if with_kv else out
