"""The fused RG-LRU kernel's ticket guess.  Each workgroup takes its tile from an atomic
ticket counter (tiles of one chain must start in time order for the chained scan: the
blog page "Griffin's Compromise", "Term explanation: Parallel scan") and, while that
atomic is in flight, loads the first operand block of the tile it would get if tickets went
in launch order.  The test hook shifts the guess so that (nearly) every workgroup finds it
wrong, waits for those loads and loads its own tile: the results must be bitwise the same
as with the normal guess, and match the oracle.
"""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import TOL, TORCH_IO, dev, device_inputs, err, gpu_forward, host, make, oracle_forward

pytestmark = pytest.mark.gpu


def _with_guess(g, offset, fn):
    try:
        g.rglru_test_set_lru_ticket_guess(offset)
        return fn()
    finally:
        g.rglru_test_set_lru_ticket_guess(0)


@pytest.mark.parametrize("offset", [1, 5])
def test_forward_with_wrong_guesses_gives_the_same_bits(lib, offset):
    # 2 sequences x 3 channel tiles x 3 time tiles (the last one ragged)
    p = make(workloads.TRAIN_FWD, B=2, T=600, D=384, h0="normal", history="normal")
    d = device_inputs(p)
    y0, h0, _ = gpu_forward(lib, d, p["c"])
    y1, h1, _ = _with_guess(lib, offset, lambda: gpu_forward(lib, d, p["c"]))
    np.testing.assert_array_equal(y0, y1)
    np.testing.assert_array_equal(h0, h1)
    o = oracle_forward(p)
    ey, eh = err(y1, o["y"]), err(h1, o["h_T"])
    print(f"ticket guess +{offset}: err(y)={ey:.2e} err(h_T)={eh:.2e}", flush=True)
    assert ey <= TOL["bf16"] and eh <= TOL["bf16"]


def test_full_size_forward_with_wrong_guesses_gives_the_same_bits(lib):
    """B=8, T=2048, D=2560: 1280 tiles in 8 ticket groups."""
    p = workloads.make_inputs(workloads.TRAIN_FWD)
    d = device_inputs(p)
    y0, h0, _ = gpu_forward(lib, d, p["c"])
    y1, h1, _ = _with_guess(lib, 1, lambda: gpu_forward(lib, d, p["c"]))
    assert np.array_equal(y0, y1) and np.array_equal(h0, h1)


def test_gated_block_with_wrong_guesses_gives_the_same_bits(lib):
    """rglru_block_fwd runs the gated form of the kernel (output multiplied by the GeLU
    branch)."""
    w = workloads.TRAIN_FWD.with_shape(B=2, T=520, D=256)
    p = workloads.make_block_inputs(w)
    io = TORCH_IO[p["workload"].io]
    d = device_inputs(p)
    d.update(x_block=dev(p["x_block"], io), W_in=dev(p["W_in"], io), W_out=dev(p["W_out"], io))

    def run():
        out, hT, _ = lib.block_forward(d["x_block"], d["W_in"], d["conv_w"], d["conv_b"],
                                       d["conv_state"], d["W_a"], d["W_x"], d["b_a"], d["b_x"],
                                       d["lam"], d["h0"], d["W_out"], p["c"])
        torch.cuda.synchronize()
        return host(out), host(hT)

    o0, h0 = run()
    o1, h1 = _with_guess(lib, 3, run)
    np.testing.assert_array_equal(o0, o1)
    np.testing.assert_array_equal(h0, h1)
