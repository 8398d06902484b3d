"""Streaming input with the carried state (h, conv history): chunked prefill over many
launches, prefill -> decode -> prefill hand-offs, and a host checkpoint of the state
(the blog page "Griffin's Compromise": generation carries only a fixed-size state, section
"Hawk"; state consistency under streaming input and checkpoint recovery, "Limitations and a
Pre-Adoption Checklist").  Every output of every launch is compared with ONE oracle forward
over the whole sequence.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import TOL, TORCH_IO, dev, err, host, sample_channels

pytestmark = pytest.mark.gpu


def _dev_params(p):
    io = TORCH_IO[p["workload"].io]
    d = {k: dev(p[k], io) for k in ("x", "conv_w", "W_a", "W_x")}
    d.update({k: dev(p[k]) for k in ("conv_b", "b_a", "b_x", "lam")})
    d["conv_state"] = dev(p["conv_state"], io)
    d["h0"] = dev(p["h0"])
    return d


def _prefill(g, d, x, cs, h, c):
    """rglru_fwd on x [B, n, D] from state (cs, h); returns y and the new state."""
    y, hT, cso = g.forward(x.contiguous(), d["conv_w"], d["conv_b"], cs, d["W_a"], d["W_x"],
                           d["b_a"], d["b_x"], d["lam"], h, c)
    return y, cso, hT


def _decode(g, d, x, cs, h, c, ws):
    """rglru_decode_step on every token of x [B, n, D]; state (cs, h) updated in place."""
    B, n, D = x.shape
    ys = []
    for t in range(n):
        y_t = torch.empty((B, D), dtype=x.dtype, device="cuda")
        g.rglru_decode_step(x[:, t].contiguous(), d["conv_w"], d["conv_b"], cs, d["W_a"], d["W_x"],
                            d["b_a"], d["b_x"], d["lam"], h, y_t, ws, c)
        ys.append(y_t)
    return torch.stack(ys, 1)


def _oracle(p, channels=None):
    return oracle.forward(p["x"], p["conv_w"], p["conv_b"], p["conv_state"], p["W_a"], p["W_x"],
                          p["b_a"], p["b_x"], p["lam"], p["h0"], p["c"], p["workload"].io,
                          channels=channels)


def _run_schedule(g, p, schedule):
    """schedule: list of ("prefill" | "decode", n tokens) covering the sequence in order."""
    d = _dev_params(p)
    w = p["workload"]
    io = TORCH_IO[w.io]
    cs, h = d["conv_state"].clone(), d["h0"].clone()
    ws = g.workspace(g.decode_workspace_bytes(w.B, w.D, io))
    t, ys = 0, []
    for kind, n in schedule:
        x = d["x"][:, t:t + n]
        if kind == "prefill":
            y, cs, h = _prefill(g, d, x, cs, h, p["c"])
        else:
            y = _decode(g, d, x, cs, h, p["c"], ws)
        ys.append(y)
        t += n
    assert t == w.T
    torch.cuda.synchronize()
    return host(torch.cat(ys, 1)), host(h), host(cs)


SCHEDULES = {
    "chunks": [("prefill", n) for n in (1, 255, 256, 257, 3, 500, 228)],
    "prefill-decode-prefill": [("prefill", 300), ("decode", 20), ("prefill", 400), ("decode", 5),
                               ("prefill", 775)],
    "decode-first": [("decode", 7), ("prefill", 1), ("decode", 2), ("prefill", 1490)],
}


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("name", list(SCHEDULES))
def test_streaming_schedule_matches_one_forward(lib, io, name):
    w = workloads.TRAIN_FWD.with_shape(B=2, T=1500, D=192, io=io, h0="normal", history="normal")
    p = workloads.make_inputs(w)
    y, h, cs = _run_schedule(lib, p, SCHEDULES[name])
    o = _oracle(p)
    ey, eh = err(y, o["y"]), err(h, o["h_T"])
    print(f"{name} io={io} err(y)={ey:.3e} err(h)={eh:.3e}", flush=True)
    assert ey <= TOL[io] and eh <= TOL[io]
    np.testing.assert_array_equal(cs, o["conv_state_out"])


def test_state_checkpoint_through_host_is_bitwise(lib):
    """Stopping after a prefill, saving (h, history) to host memory and restoring it into
    fresh device buffers continues with exactly the bits of the uninterrupted run."""
    w = workloads.TRAIN_FWD.with_shape(B=3, T=900, D=256, h0="normal", history="normal")
    p = workloads.make_inputs(w)
    d = _dev_params(p)
    io = TORCH_IO[w.io]
    ws = lib.workspace(lib.decode_workspace_bytes(w.B, w.D, io))
    _, cs, h = _prefill(lib, d, d["x"][:, :600], d["conv_state"], d["h0"], p["c"])
    saved_cs = cs.view(torch.int16).cpu().numpy().copy()     # the bf16 bits
    saved_h = h.cpu().numpy().copy()
    y_a = _decode(lib, d, d["x"][:, 600:610], cs, h, p["c"], ws)
    y_a2, cs_a, h_a = _prefill(lib, d, d["x"][:, 610:], cs, h, p["c"])
    cs_r = torch.from_numpy(saved_cs).to("cuda").view(torch.bfloat16)
    h_r = torch.from_numpy(saved_h).to("cuda")
    y_b = _decode(lib, d, d["x"][:, 600:610], cs_r, h_r, p["c"], ws)
    y_b2, cs_b, h_b = _prefill(lib, d, d["x"][:, 610:], cs_r, h_r, p["c"])
    torch.cuda.synchronize()
    for a, b in ((y_a, y_b), (y_a2, y_b2), (cs_a, cs_b), (h_a, h_b)):
        assert torch.equal(a, b)


@pytest.mark.timeout(600)
def test_prefill_then_decode_at_decode_batch(lib):
    """The decode workload's batch (B=256, D=2560): prefill 64 tokens, then 16 decode steps,
    on a seeded channel subset of one oracle forward over the 80 tokens."""
    w = workloads.DECODE.with_shape(T=80, decode=False)
    p = workloads.make_inputs(w)
    y, h, cs = _run_schedule(lib, p, [("prefill", 64), ("decode", 16)])
    S = sample_channels(w.D, 32, seed=11)
    o = _oracle(p, channels=S)
    ey, eh = err(y[:, :, S], o["y"]), err(h[:, S], o["h_T"])
    print(f"B=256 prefill+decode err(y)={ey:.3e} err(h)={eh:.3e}", flush=True)
    assert ey <= TOL["bf16"] and eh <= TOL["bf16"]
    np.testing.assert_array_equal(cs, o["conv_state_out"])
