"""Shared helpers of the GPU parity tests: seeded inputs to device tensors, the oracle on
the same host arrays, and the error metric.

Error metric per output tensor: e = max_i |g_i - o_i| / max(1, |o_i|) (absolute where
|o| <= 1, relative above).  Tolerances: 1e-5 for fp32 I/O, 2e-2 for bf16 I/O with fp32
state; gradients are fp32 outputs and use the tolerance of their I/O dtype.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import workloads

TOL = {"f32": 1e-5, "bf16": 2e-2}
TORCH_IO = {"f32": torch.float32, "bf16": torch.bfloat16}


def err(got, want) -> float:
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    if want.size == 0:
        return 0.0
    return float(np.max(np.abs(got - want) / np.maximum(1.0, np.abs(want))))


def dev(a, dtype=torch.float32):
    if a is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda").to(dtype).contiguous()


def host(t):
    return None if t is None else t.float().cpu().numpy().astype(np.float64)


def device_inputs(p: dict) -> dict:
    """The same host arrays as device tensors (io tensors in the I/O dtype, exact)."""
    io = TORCH_IO[p["workload"].io]
    return {
        "x": dev(p["x"], io), "conv_w": dev(p["conv_w"], io), "conv_b": dev(p["conv_b"]),
        "conv_state": dev(p["conv_state"], io), "W_a": dev(p["W_a"], io), "W_x": dev(p["W_x"], io),
        "b_a": dev(p["b_a"]), "b_x": dev(p["b_x"]), "lam": dev(p["lam"]), "h0": dev(p["h0"]),
        "dy": dev(p["dy"], io) if p.get("dy") is not None else None,
    }


def gpu_forward(g, d: dict, c: float, conv=True):
    y, hT, cso = g.forward(d["x"], d["conv_w"] if conv else None, d["conv_b"] if conv else None,
                           d["conv_state"] if conv else None, d["W_a"], d["W_x"], d["b_a"], d["b_x"],
                           d["lam"], d["h0"], c)
    torch.cuda.synchronize()
    return host(y), host(hT), host(cso)


def oracle_forward(p: dict, channels=None, conv=True, **over):
    args = dict(x=p["x"], conv_w=p["conv_w"] if conv else None,
                conv_b=p["conv_b"] if conv else None,
                conv_state_in=p["conv_state"] if conv else None, W_a=p["W_a"], W_x=p["W_x"],
                b_a=p["b_a"], b_x=p["b_x"], lam=p["lam"], h0=p["h0"], c=p["c"],
                io=p["workload"].io, channels=channels)
    args.update(over)
    return oracle.forward(**args)


def sample_channels(D: int, n: int, seed: int) -> np.ndarray:
    """A seeded channel subset that always includes the first and last tile edges."""
    rng = np.random.default_rng(seed)
    fixed = np.array([0, 1, 63, 64, D // 2, D - 65, D - 64, D - 1])
    rest = rng.choice(D, size=max(0, n - len(fixed)), replace=False)
    return np.unique(np.concatenate([fixed, rest]))


def make(w: workloads.Workload, **shape):
    return workloads.make_inputs(w.with_shape(**shape) if shape else w)
