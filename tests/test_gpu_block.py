"""Parity of the recurrent block (rglru_block_fwd: the two input linears, the GeLU branch,
the temporal branch, the product and the output linear of Fig. 2(c) on the Griffin
model-architecture page) with the oracle's block_forward.

Element by element at sizes the oracle finishes in seconds: ragged row tiles (M = B*T not
a multiple of 256), ragged column tiles of both linears (2R and D not multiples of 256,
the p/GeLU split inside a tile), an RG-LRU channel tile of 64 valid channels, T = 1, and
model width different from the branch width.  At the full training shape every output of
one whole sequence is compared (sequences are independent, so the oracle runs on that
sequence alone) together with its final state.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import TOL, TORCH_IO, dev, device_inputs, err, host

pytestmark = pytest.mark.gpu


def _device(p):
    io = TORCH_IO[p["workload"].io]
    d = device_inputs(p)
    d.update(x_block=dev(p["x_block"], io), W_in=dev(p["W_in"], io), W_out=dev(p["W_out"], io))
    return d


def _gpu(g, d, p, conv=True):
    out, hT, cso = g.block_forward(d["x_block"], d["W_in"], d["conv_w"] if conv else None,
                                   d["conv_b"] if conv else None, d["conv_state"] if conv else None,
                                   d["W_a"], d["W_x"], d["b_a"], d["b_x"], d["lam"], d["h0"],
                                   d["W_out"], p["c"])
    torch.cuda.synchronize()
    return host(out), host(hT), host(cso)


def _oracle(p, conv=True, rows=slice(None)):
    sel = lambda a: None if a is None else a[rows]
    return oracle.block_forward(
        x=p["x_block"][rows], W_in=p["W_in"], conv_w=p["conv_w"] if conv else None,
        conv_b=p["conv_b"] if conv else None, conv_state_in=sel(p["conv_state"]) if conv else None,
        W_a=p["W_a"], W_x=p["W_x"], b_a=p["b_a"], b_x=p["b_x"], lam=p["lam"], h0=sel(p["h0"]),
        W_out=p["W_out"], c=p["c"], io=p["workload"].io)


def _check(g, p, conv=True, what=""):
    io = p["workload"].io
    out, hT, cso = _gpu(g, _device(p), p, conv)
    o = _oracle(p, conv)
    eo, eh = err(out, o["out"]), err(hT, o["h_T"])
    print(f"{what} io={io} x={p['x_block'].shape} R={p['W_in'].shape[0] // 2} "
          f"err(out)={eo:.3e} err(h_T)={eh:.3e}", flush=True)
    assert eo <= TOL[io] and eh <= TOL[io]
    if conv:
        # the conv history is the last rows of p, the first linear's output: a GEMM result
        # rounded once to the I/O dtype, which may land on the neighbouring value where the
        # exact sum (the oracle's) sits next to a rounding boundary; compared to the bar
        ec = err(cso, o["conv_state_out"])
        print(f"{what} err(conv_state_out)={ec:.3e}", flush=True)
        assert ec <= TOL[io]


SMALL = [
    # (workload recipe, B, T, model width D, branch width R)
    (workloads.TINY_F32, 1, 256, 256, 256),
    (workloads.TINY_F32, 2, 300, 192, 320),
    (workloads.TINY_F32, 1, 1, 64, 64),
    (workloads.TRAIN_FWD, 2, 700, 320, 384),
    (workloads.TRAIN_FWD, 3, 257, 448, 192),
    (workloads.TRAIN_FWD, 1, 1, 64, 64),
    (workloads.TRAIN_FWD, 1, 300, 128, 640),
    (workloads.LONG_FWD, 1, 1500, 256, 256),
]


@pytest.mark.parametrize("w,B,T,D,R", SMALL, ids=[f"{w.io}-{B}x{T}-D{D}-R{R}" for w, B, T, D, R in SMALL])
def test_block_small_elementwise(lib, w, B, T, D, R):
    p = workloads.make_block_inputs(w.with_shape(B=B, T=T, D=R), d_model=D)
    _check(lib, p, what=w.name)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_block_with_conv_state_h0_and_bias(lib, io):
    w = workloads.TRAIN_FWD.with_shape(B=2, T=333, D=192, io=io, h0="normal", history="normal")
    p = workloads.make_block_inputs(w, d_model=256)
    p["conv_b"] = np.random.default_rng(0).standard_normal(192).astype(np.float32) * 0.1
    _check(lib, p, what="state")


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_block_without_conv(lib, io):
    # without the conv the branch input p is the layer input; the output must not overwrite
    # it while other channel tiles of the same rows still read it (R = 384: 3 channel tiles)
    w = workloads.TRAIN_FWD.with_shape(B=2, T=520, D=384, io=io)
    p = workloads.make_block_inputs(w, d_model=192)
    _check(lib, p, conv=False, what="noconv")


def test_block_repeat_is_bitwise_identical(lib):
    w = workloads.TRAIN_FWD.with_shape(B=2, T=600, D=256)
    p = workloads.make_block_inputs(w, d_model=320)
    d = _device(p)
    first = _gpu(lib, d, p)
    for _ in range(3):
        again = _gpu(lib, d, p)
        for a, b in zip(first, again):
            np.testing.assert_array_equal(a, b)


@pytest.mark.timeout(600)
def test_block_full_training_shape_one_sequence(lib):
    """B=8, T=2048, D = D_RNN = 2560 in the launch configuration the benchmark times; every
    output and the final state of the last sequence against the oracle on that sequence."""
    w = workloads.TRAIN_FWD
    p = workloads.make_block_inputs(w)
    out, hT, _ = _gpu(lib, _device(p), p)
    b = w.B - 1
    o = _oracle(p, rows=slice(b, b + 1))
    eo, eh = err(out[b:b + 1], o["out"]), err(hT[b:b + 1], o["h_T"])
    print(f"full block b={b} err(out)={eo:.3e} err(h_T)={eh:.3e}", flush=True)
    assert eo <= TOL["bf16"] and eh <= TOL["bf16"]
    assert np.all(np.isfinite(out))


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_block_prefill_then_decode(lib, io):
    """rglru_block_fwd over the first 300 tokens (its h_T and conv_state_out seed the
    state), then 24 rglru_block_decode_step calls: every output against one oracle block
    forward over the 324 tokens."""
    T0, steps = 300, 24
    w = workloads.TRAIN_FWD.with_shape(B=2, T=T0 + steps, D=192, io=io, h0="normal", history="normal")
    p = workloads.make_block_inputs(w, d_model=320)
    d = _device(p)
    x = d["x_block"]
    out0, hT, cso = lib.block_forward(x[:, :T0].contiguous(), d["W_in"], d["conv_w"], d["conv_b"],
                                      d["conv_state"], d["W_a"], d["W_x"], d["b_a"], d["b_x"], d["lam"],
                                      d["h0"], d["W_out"], p["c"])
    ws = lib.workspace(lib.block_decode_workspace_bytes(2, 320, 192, TORCH_IO[io]))
    outs = []
    for t in range(T0, T0 + steps):
        o = torch.empty((2, 320), dtype=TORCH_IO[io], device="cuda")
        lib.rglru_block_decode_step(x[:, t].contiguous(), d["W_in"], d["conv_w"], d["conv_b"], cso,
                                    d["W_a"], d["W_x"], d["b_a"], d["b_x"], d["lam"], hT, d["W_out"], o,
                                    ws, p["c"])
        outs.append(o)
    torch.cuda.synchronize()
    want = _oracle(p)
    e0 = err(host(out0), want["out"][:, :T0])
    e1 = err(host(torch.stack(outs, 1)), want["out"][:, T0:])
    eh = err(host(hT), want["h_T"])
    print(f"block prefill->decode io={io} err(prefill)={e0:.3e} err(decode)={e1:.3e} err(h)={eh:.3e}",
          flush=True)
    assert e0 <= TOL[io] and e1 <= TOL[io] and eh <= TOL[io]
    assert err(host(cso), want["conv_state_out"]) <= TOL[io]   # p rows: a rounded GEMM output


def test_block_decode_full_shape_sampled_sequences(lib):
    """B=256, D = R = 2560 (the decode workload's batch): 8 steps from its seeded state, the
    outputs of 4 sequences against the oracle block forward over those sequences' 8 tokens."""
    w = workloads.DECODE.with_shape(T=8, decode=False)
    p = workloads.make_block_inputs(w)
    d = _device(p)
    cs, h = d["conv_state"].clone(), d["h0"].clone()
    ws = lib.workspace(lib.block_decode_workspace_bytes(w.B, w.D, w.D, torch.bfloat16))
    outs = []
    for t in range(8):
        o = torch.empty((w.B, w.D), dtype=torch.bfloat16, device="cuda")
        lib.rglru_block_decode_step(d["x_block"][:, t].contiguous(), d["W_in"], d["conv_w"], d["conv_b"],
                                    cs, d["W_a"], d["W_x"], d["b_a"], d["b_x"], d["lam"], h, d["W_out"], o,
                                    ws, p["c"])
        outs.append(o)
    torch.cuda.synchronize()
    sel = np.array([0, 1, 128, 255])
    got = host(torch.stack(outs, 1))[sel]
    want = oracle.block_forward(x=p["x_block"][sel], W_in=p["W_in"], conv_w=p["conv_w"], conv_b=p["conv_b"],
                                conv_state_in=p["conv_state"][sel], W_a=p["W_a"], W_x=p["W_x"], b_a=p["b_a"],
                                b_x=p["b_x"], lam=p["lam"], h0=p["h0"][sel], W_out=p["W_out"], c=p["c"],
                                io="bf16")
    e = err(got, want["out"])
    print(f"block decode B=256 err(out)={e:.3e}", flush=True)
    assert e <= TOL["bf16"]
