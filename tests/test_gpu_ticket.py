"""The fused RG-LRU kernel's ticket guess.  Each workgroup takes its tile from an atomic
ticket counter (tiles of one chain must start in time order for the chained scan: the
blog page "Griffin's Compromise", "Term explanation: Parallel scan") and, while that
atomic is in flight, loads the first operand block of the tile it would get if tickets went
in launch order.  The test-only entry points (rglru_testing.h) shift the guess so that
(nearly) every workgroup finds it wrong, waits for those loads and loads its own tile: the
results must be bitwise the same as with the normal guess, and match the oracle.
"""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import TOL, TORCH_IO, dev, device_inputs, err, gpu_forward, host, make, oracle_forward

pytestmark = pytest.mark.gpu


def _fwd_with_guess(d, c, offset):
    """The forward with the fused kernel (forced: small shapes take the unfused form) and its
    ticket guess shifted by `offset`."""
    from gated_linear_rnn_amd import testing
    y, hT, _, _ = testing.forward(testing.knobs(lru_ticket_guess=offset, lru_force_fused=1), d["x"], d["conv_w"],
                                  d["conv_b"], d["conv_state"], d["W_a"], d["W_x"], d["b_a"],
                                  d["b_x"], d["lam"], d["h0"], c)
    torch.cuda.synchronize()
    return host(y), host(hT)


@pytest.mark.parametrize("offset", [1, 5])
def test_forward_with_wrong_guesses_gives_the_same_bits(lib, offset):
    # 2 sequences x 3 channel tiles x 3 time tiles (the last one ragged)
    p = make(workloads.TRAIN_FWD, B=2, T=600, D=384, h0="normal", history="normal")
    d = device_inputs(p)
    y0, h0 = _fwd_with_guess(d, p["c"], 0)
    y1, h1 = _fwd_with_guess(d, p["c"], offset)
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
    y1, h1 = _fwd_with_guess(d, p["c"], 1)
    assert np.array_equal(y0, y1) and np.array_equal(h0, h1)


def test_gated_block_with_wrong_guesses_gives_the_same_bits(lib):
    """rglru_block_fwd runs the gated form of the kernel (output multiplied by the GeLU
    branch)."""
    w = workloads.TRAIN_FWD.with_shape(B=2, T=520, D=256)
    p = workloads.make_block_inputs(w)
    io = TORCH_IO[p["workload"].io]
    d = device_inputs(p)
    d.update(x_block=dev(p["x_block"], io), W_in=dev(p["W_in"], io), W_out=dev(p["W_out"], io))

    from gated_linear_rnn_amd import testing
    args = (d["x_block"], d["W_in"], d["conv_w"], d["conv_b"], d["conv_state"], d["W_a"], d["W_x"],
            d["b_a"], d["b_x"], d["lam"], d["h0"], d["W_out"], p["c"])
    out, hT, _ = lib.block_forward(*args)
    torch.cuda.synchronize()
    o0, h0 = host(out), host(hT)
    out, hT, _ = testing.block_forward(testing.knobs(lru_ticket_guess=3), *args)
    torch.cuda.synchronize()
    o1, h1 = host(out), host(hT)
    np.testing.assert_array_equal(o0, o1)
    np.testing.assert_array_equal(h0, h1)


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_a_lookback_that_gives_up_is_reported(lib, io):
    """A look-back told to give up at once (lookback_polls < 0: the fused kernel's, and the
    reverse scan's in the backward) writes NaN where the carry was needed, every kernel still
    ends, and rglru_workspace_status reports RGLRU_ESTALL; the next ordinary call on the same
    workspace is clean again.  (fp32 I/O runs the forward scan, which never gives up: it
    computes a missing summary itself, so only its backward can stall.)"""
    from gated_linear_rnn_amd import testing
    p = make(workloads.TRAIN_BWD, B=2, T=600, D=128, io=io, h0="normal", history="normal")
    d = device_inputs(p)
    fargs = (d["x"], d["conv_w"], d["conv_b"], d["conv_state"], d["W_a"], d["W_x"], d["b_a"],
             d["b_x"], d["lam"], d["h0"])
    stop = testing.knobs(lookback_polls=-1, lru_force_fused=1)
    y, hT, _, ws = testing.forward(stop, *fargs, c=p["c"])
    st = lib.rglru_workspace_status(ws)
    if io == "bf16":
        assert st == lib.RGLRU_ESTALL
        yh = host(y)
        assert np.isnan(yh[:, 256:]).all() and np.isfinite(yh[:, :256]).all()
    else:
        assert st == 0
    y2, _, _ = lib.forward(*fargs, c=p["c"], ws=ws)
    assert lib.rglru_workspace_status(ws) == 0
    o = oracle_forward(p)
    assert err(host(y2), o["y"]) <= TOL[io]
    g, wsb = testing.backward(stop, *fargs, d["dy"], c=p["c"])
    assert lib.rglru_workspace_status(wsb) == lib.RGLRU_ESTALL
    assert np.isnan(host(g["dx"])).any()
    lib.backward(*fargs, d["dy"], c=p["c"], ws=wsb)
    assert lib.rglru_workspace_status(wsb) == 0
