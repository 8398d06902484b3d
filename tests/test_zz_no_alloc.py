"""The allocation-free decode step (rglru_decode_step_noalloc): the same step as
rglru_decode_step with its scratch in the library's fixed per-GPU array instead of a
caller workspace.  Checked against rglru_decode_step through the C ABI on two calls in a
row, the second with a smaller input (the array keeps the first call's contents), and a
shape too large for the fixed scratch is refused without launching anything."""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import TORCH_IO, dev

pytestmark = pytest.mark.gpu


def _state(p, io):
    return {"x": dev(p["x"][0], io), "cw": dev(p["conv_w"], io), "cb": dev(p["conv_b"]),
            "hist": dev(p["conv_state"], io), "Wa": dev(p["W_a"], io), "Wx": dev(p["W_x"], io),
            "ba": dev(p["b_a"]), "bx": dev(p["b_x"]), "lam": dev(p["lam"]), "h": dev(p["h0"])}


def _both(lib, p, io, steps=3):
    """`steps` steps from the same state through both entry points; returns the outputs."""
    a, b = _state(p, io), _state(p, io)
    B, D = a["x"].shape
    ws = lib.workspace(lib.decode_workspace_bytes(B, D, io))
    ya = torch.empty((B, D), dtype=io, device="cuda")
    yb = torch.empty_like(ya)
    outs = []
    for t in range(steps):
        xt = dev(p["x"][t], io)
        lib.rglru_decode_step(xt, a["cw"], a["cb"], a["hist"], a["Wa"], a["Wx"], a["ba"], a["bx"],
                              a["lam"], a["h"], ya, ws, p["c"])
        lib.rglru_decode_step_noalloc(xt, b["cw"], b["cb"], b["hist"], b["Wa"], b["Wx"], b["ba"],
                                      b["bx"], b["lam"], b["h"], yb, p["c"])
        torch.cuda.synchronize()
        outs.append((ya.clone(), yb.clone()))
    return a, b, outs


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_noalloc_decode_equals_workspace_decode(lib, io):
    tio = TORCH_IO[io]
    big = workloads.DECODE.with_shape(B=256, D=2560, T=3, io=io) if io == "bf16" else \
        workloads.DECODE.with_shape(B=64, D=1024, T=3, io=io)
    small = workloads.DECODE.with_shape(B=8, D=512, T=3, io=io)
    tiny = workloads.DECODE.with_shape(B=2, D=256, T=3, io=io)   # bf16: the one-launch step
    for w in (big, small, tiny):                # each call smaller than the one before
        p = workloads.make_inputs(w)
        a, b, outs = _both(lib, p, tio)
        for ya, yb in outs:
            assert torch.equal(ya, yb)
        assert torch.equal(a["h"], b["h"]) and torch.equal(a["hist"], b["hist"])


def test_noalloc_decode_refuses_a_shape_beyond_its_scratch(lib):
    B, D = 1024, 8192                           # u and the split sums: far over the 32 MiB
    assert lib.decode_workspace_bytes(B, D, torch.bfloat16) > lib.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((B, D), dtype=torch.bfloat16, device="cuda")
    h = torch.zeros((B, D), device="cuda")
    y = torch.zeros_like(x)
    W = torch.zeros((16, 16), dtype=torch.bfloat16, device="cuda")   # never read
    v = torch.zeros(D, device="cuda")
    with pytest.raises(lib.RgluError, match="ESCRATCH"):
        lib.rglru_decode_step_noalloc(x, None, None, None, W, W, v, v, v, h, y)
