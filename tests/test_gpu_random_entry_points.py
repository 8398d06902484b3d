"""Parity over seeded random shapes for the entry points around the RG-LRU forward: the
recurrent block, the gated MLP, local MQA, the decode step, the split path (rglru_gates then
rglru_scan), the training pair (rglru_fwd_train then rglru_bwd_saved, which must equal
rglru_bwd bit for bit), and the stateful paths: random prefill/decode schedules against one
forward, local MQA decode from an empty cache, and the block's prefill then decode.  Each
case reuses the element-by-element check of that entry point's own test module; the draws
are a pure function of (kind, case index), so a failing case replays exactly and its test
id names its shape.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import TOL, TORCH_IO, device_inputs, err, host, oracle_forward
import test_gpu_block as TB
import test_gpu_bwd as TW
import test_gpu_decode as TD
import test_gpu_mlp as TM
import test_gpu_mqa as TQ
import test_gpu_mqa_decode as TQD
import test_gpu_scan as TS
import test_gpu_streaming as TSt

pytestmark = pytest.mark.gpu

RECIPES = [workloads.TINY_F32, workloads.TRAIN_FWD, workloads.LONG_FWD, workloads.TRAIN_BWD]
KINDS = ["block", "mlp", "mqa", "decode", "split", "train", "stream", "mqa_decode", "block_decode"]
N_PER_KIND = 8


def _draw(kind, k):
    rng = np.random.default_rng([KINDS.index(kind), k])
    pick = lambda *xs: xs[int(rng.integers(0, len(xs)))]
    c = dict(io=["f32", "bf16"][k % 2], recipe=RECIPES[int(rng.integers(0, 4))],
             h0=pick("zero", "normal"), history=pick("zero", "normal"), seed=int(rng.integers(0, 2 ** 31)))
    if kind == "block":
        c.update(B=int(rng.integers(1, 4)), T=pick(1, 2, 3, 65, 257, 700, int(rng.integers(1, 1200))),
                 D=64 * int(rng.integers(1, 8)), R=64 * int(rng.integers(1, 8)), conv=bool(rng.integers(0, 4)))
    elif kind == "mlp":
        c.update(B=int(rng.integers(1, 4)), T=pick(1, 2, 3, 65, 257, int(rng.integers(1, 800))),
                 D=64 * int(rng.integers(1, 8)), M=int(rng.integers(1, 5)))
    elif kind == "mqa":
        c.update(B=int(rng.integers(1, 4)), T=pick(1, 2, 3, 5, 63, 130, int(rng.integers(1, 900))),
                 D=128 * int(rng.integers(1, 5)), W=pick(1, 3, 16, 64, 100, 1024),
                 sharp=bool(rng.integers(0, 2)), pos0=pick(0, 0, 7, 1000))
    elif kind == "decode":
        c.update(B=pick(1, 2, 3, 4, 5, 8, 17, 64, 300), D=64 * int(rng.integers(1, 11)),
                 steps=pick(1, 2, 7, 30), conv=bool(rng.integers(0, 4)))
    elif kind == "split":
        c.update(B=int(rng.integers(1, 5)), T=pick(1, 2, 3, 64, 65, 333, int(rng.integers(1, 1500))),
                 D=64 * int(rng.integers(1, 9)), conv=bool(rng.integers(0, 2)))
    elif kind == "train":
        c.update(B=int(rng.integers(1, 4)), T=pick(1, 2, 3, 65, 257, int(rng.integers(1, 400))),
                 D=64 * int(rng.integers(1, 5)), conv=bool(rng.integers(0, 3)))
    elif kind == "stream":
        sched = []
        for _ in range(int(rng.integers(1, 7))):
            if int(rng.integers(0, 3)) < 2:
                sched.append(("prefill", int(pick(1, 2, 3, 5, 64, 255, 256, 257, int(rng.integers(1, 600))))))
            else:
                sched.append(("decode", int(rng.integers(1, 9))))
        c.update(B=int(rng.integers(1, 5)), D=64 * int(rng.integers(1, 11)), sched=sched,
                 T=sum(n for _, n in sched))
    elif kind == "mqa_decode":
        W = pick(1, 2, 5, 16, 64)
        c.update(B=int(rng.integers(1, 4)), D=128 * int(rng.integers(1, 4)), W=W,
                 T=int(rng.integers(1, 2 * W + 10)))
    else:
        c.update(B=int(rng.integers(1, 4)), R=64 * int(rng.integers(1, 6)), D=64 * int(rng.integers(1, 6)),
                 T0=int(pick(1, 2, 3, 65, int(rng.integers(1, 400)))), steps=int(rng.integers(1, 12)))
        c["T"] = c["T0"] + c["steps"]
    return c


CASES = [(kind, k) for kind in KINDS for k in range(N_PER_KIND)]


def _id(kind, k):
    c = _draw(kind, k)
    shape = "x".join(str(c[n]) for n in ("B", "T", "D") if n in c)
    return f"{kind}-{k}-{c['io']}-{shape}"


@pytest.mark.parametrize("kind,k", CASES, ids=[_id(*c) for c in CASES])
def test_random_entry_point(lib, kind, k):
    c = _draw(kind, k)
    io = c["io"]
    print(f"{kind} case {k}: {c}", flush=True)
    if kind == "block":
        w = c["recipe"].with_shape(B=c["B"], T=c["T"], D=c["R"], io=io, h0=c["h0"], history=c["history"])
        TB._check(lib, workloads.make_block_inputs(w, d_model=c["D"]), conv=c["conv"], what="block")
    elif kind == "mlp":
        p = workloads.make_mlp_inputs(c["recipe"].with_shape(B=c["B"], T=c["T"], D=c["D"], io=io),
                                      expansion=c["M"])
        e = err(TM._gpu(lib, p), oracle.gated_mlp_forward(p["x"], p["W_1"], p["W_2"], p["W_3"], io))
        print(f"  err(out)={e:.2e}", flush=True)
        assert e <= TOL[io]
    elif kind == "mqa":
        p = TQ._inputs(c["recipe"].with_shape(B=c["B"], T=c["T"], D=c["D"], io=io), c["W"], c["sharp"])
        TQ._check(lib, p, pos0=c["pos0"], what="mqa")
    elif kind == "decode":
        p = workloads.make_inputs(workloads.DECODE.with_shape(B=c["B"], D=c["D"], T=c["steps"], io=io))
        TD._run(lib, p, c["steps"], conv=c["conv"])
    elif kind == "split":
        p = workloads.make_inputs(c["recipe"].with_shape(B=c["B"], T=c["T"], D=c["D"], io=io,
                                                         h0=c["h0"], history=c["history"]))
        y, hT = TS._split_scan(lib, p, device_inputs(p), c["conv"])
        o = oracle_forward(p, conv=c["conv"])
        ey, eh = err(y, o["y"]), err(hT, o["h_T"])
        print(f"  err(y)={ey:.2e} err(h_T)={eh:.2e}", flush=True)
        assert ey <= TOL[io] and eh <= TOL[io]
    elif kind == "stream":
        w = c["recipe"].with_shape(B=c["B"], T=c["T"], D=c["D"], io=io, h0="normal", history="normal")
        p = workloads.make_inputs(w)
        y, h, cs = TSt._run_schedule(lib, p, c["sched"])
        o = TSt._oracle(p)
        ey, eh = err(y, o["y"]), err(h, o["h_T"])
        print(f"  err(y)={ey:.2e} err(h)={eh:.2e}", flush=True)
        assert ey <= TOL[io] and eh <= TOL[io]
        np.testing.assert_array_equal(cs, o["conv_state_out"])   # a copy of x rows: exact
    elif kind == "mqa_decode":
        B, D, W, T = c["B"], c["D"], c["W"], c["T"]
        p = workloads.make_mqa_inputs(workloads.TRAIN_FWD.with_shape(B=B, T=T, D=D, io=io), W)
        got, kc, vc = TQD._decode_run(lib, p, W, T)
        f = oracle.local_mqa_forward(p["x"], p["W_q"], p["W_k"], p["W_v"], p["W_o"], W, io, keep=True)
        e = err(got, f["out"])
        print(f"  err(out)={e:.2e}", flush=True)
        assert e <= TOL[io]
        lo = max(0, T - W)
        slots = [s % W for s in range(lo, T)]
        assert err(kc[:, slots], f["k"][:, lo:]) <= TOL[io]
        assert err(vc[:, slots], f["v"][:, lo:]) <= TOL[io]
    elif kind == "block_decode":
        B, R, Dm, T0, steps = c["B"], c["R"], c["D"], c["T0"], c["steps"]
        w = c["recipe"].with_shape(B=B, T=T0 + steps, D=R, io=io, h0="normal", history="normal")
        p = workloads.make_block_inputs(w, d_model=Dm)
        d = TB._device(p)
        x = d["x_block"]
        out0, hT, cso = lib.block_forward(x[:, :T0].contiguous(), d["W_in"], d["conv_w"], d["conv_b"],
                                          d["conv_state"], d["W_a"], d["W_x"], d["b_a"], d["b_x"],
                                          d["lam"], d["h0"], d["W_out"], p["c"])
        ws = lib.workspace(lib.block_decode_workspace_bytes(B, Dm, R, TORCH_IO[io]))
        outs = []
        for t in range(T0, T0 + steps):
            o = torch.empty((B, Dm), dtype=TORCH_IO[io], device="cuda")
            lib.rglru_block_decode_step(x[:, t].contiguous(), d["W_in"], d["conv_w"], d["conv_b"], cso,
                                        d["W_a"], d["W_x"], d["b_a"], d["b_x"], d["lam"], hT,
                                        d["W_out"], o, ws, p["c"])
            outs.append(o)
        torch.cuda.synchronize()
        want = TB._oracle(p)
        e0 = err(host(out0), want["out"][:, :T0])
        e1 = err(host(torch.stack(outs, 1)), want["out"][:, T0:])
        eh = err(host(hT), want["h_T"])
        print(f"  err(prefill)={e0:.2e} err(decode)={e1:.2e} err(h)={eh:.2e}", flush=True)
        assert e0 <= TOL[io] and e1 <= TOL[io] and eh <= TOL[io]
    else:
        B, D, conv = c["B"], c["D"], c["conv"]
        p = workloads.make_inputs(c["recipe"].with_shape(B=B, T=c["T"], D=D, io=io, with_dy=True,
                                                         h0="normal", history="normal"))
        dh = np.random.default_rng(c["seed"]).standard_normal((B, D))
        (y, hT, cso), got, ref = TW._train_pair(lib, p, conv=conv, dh_T=dh)
        ey = err(host(y), oracle_forward(p, conv=conv)["y"])
        want = oracle.backward(p["x"], p["conv_w"] if conv else None, p["conv_b"] if conv else None,
                               p["conv_state"] if conv else None, p["W_a"], p["W_x"], p["b_a"],
                               p["b_x"], p["lam"], p["h0"], p["c"], io, p["dy"], dh)
        eg = max(err(host(got[n]), want[n]) for n in TW.NAMES if want[n] is not None)
        print(f"  err(y)={ey:.2e} worst gradient error={eg:.2e}", flush=True)
        assert ey <= TOL[io] and eg <= TOL[io]
        for n in TW.NAMES:
            assert (ref[n] is None and got[n] is None) or torch.equal(got[n], ref[n]), n
