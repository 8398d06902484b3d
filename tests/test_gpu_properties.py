"""Properties the pages fix, re-checked on the HIP path itself.

* Gate behaviour (Griffin model-architecture page, "Gate behaviour" with Eq. (3)-(4)):
  r_t = 0 (b_a = -inf) or c = 0 gives a_t = 1 and sqrt(1 - a_t^2) = 0, so the state is
  kept bit-exactly: y_t = RNE(h0), h_T = h0.
* The sqrt(1 - a^2) normalisation: with constant gates, i = 1 and i.i.d. unit-variance
  input, Var(h_t) = 1 at every t (statistical, N >= 2e5 channels).
* Streaming input (the blog's checklist item on recurrent-state consistency): a forward
  split in two with the state handed over equals one forward.
* The stand-alone conv entry point against the oracle's conv, and bitwise determinism.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import TOL, TORCH_IO, dev, device_inputs, err, host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("mode", ["b_a=-inf", "c=0"])
def test_closed_recurrence_gate_keeps_state_bit_exact(lib, io, mode):
    w = workloads.TRAIN_FWD.with_shape(B=3, T=300, D=128, io=io, h0="normal", history="normal")
    p = workloads.make_inputs(w)
    d = device_inputs(p)
    c = p["c"]
    if mode == "b_a=-inf":
        d["b_a"] = torch.full((128,), -math.inf, device="cuda")
    else:
        c = 0.0
    y, hT, _ = lib.forward(d["x"], d["conv_w"], d["conv_b"], d["conv_state"], d["W_a"], d["W_x"],
                           d["b_a"], d["b_x"], d["lam"], d["h0"], c)
    torch.cuda.synchronize()
    assert torch.equal(hT, d["h0"])
    want = d["h0"].to(TORCH_IO[io])[:, None, :].expand_as(y)
    assert torch.equal(y, want)


def test_stationary_variance_is_one(lib):
    B, T, D = 64, 64, 4096
    N = B * D
    rng = np.random.default_rng(31)
    x = dev(rng.standard_normal((B, T, D)))
    h0 = dev(rng.standard_normal((B, D)))
    conv_w = torch.zeros((4, D), device="cuda"); conv_w[0] = 1.0
    Z = torch.zeros((D, D), device="cuda")
    lam = dev(rng.uniform(0.0, 5.0, D))
    y, _, _ = lib.forward(x, conv_w, None, None, Z, Z, torch.zeros(D, device="cuda"),
                          torch.full((D,), math.inf, device="cuda"), lam, h0, 8.0)
    torch.cuda.synchronize()
    var = (y.double() ** 2).mean(dim=(0, 2)).cpu().numpy()
    assert np.all(np.abs(var - 1.0) < 5 * math.sqrt(2.0 / N)), var


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_split_forward_equals_forward(lib, io):
    w = workloads.TRAIN_FWD.with_shape(B=2, T=700, D=192, io=io, h0="normal", history="normal")
    p = workloads.make_inputs(w)
    d = device_inputs(p)
    args = (d["W_a"], d["W_x"], d["b_a"], d["b_x"], d["lam"])
    y, hT, cso = lib.forward(d["x"], d["conv_w"], d["conv_b"], d["conv_state"], *args, d["h0"], p["c"])
    t1 = 333
    y1, h1, c1 = lib.forward(d["x"][:, :t1].contiguous(), d["conv_w"], d["conv_b"], d["conv_state"],
                             *args, d["h0"], p["c"])
    y2, h2, c2 = lib.forward(d["x"][:, t1:].contiguous(), d["conv_w"], d["conv_b"], c1, *args, h1,
                             p["c"])
    torch.cuda.synchronize()
    assert err(host(torch.cat([y1, y2], 1)), host(y)) <= TOL[io]
    assert err(host(h2), host(hT)) <= TOL[io]
    assert torch.equal(c2, cso)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_conv_entry_point_matches_oracle(lib, io):
    w = workloads.TRAIN_FWD.with_shape(B=3, T=77, D=192, io=io, history="normal")
    p = workloads.make_inputs(w)
    p["conv_b"] = np.random.default_rng(3).standard_normal(192).astype(np.float32)
    d = device_inputs(p)
    u = torch.empty_like(d["x"])
    so = torch.empty_like(d["conv_state"])
    lib.conv1d_causal4(d["x"], d["conv_w"], d["conv_b"], d["conv_state"], u, so)
    torch.cuda.synchronize()
    uo, soo = oracle.conv1d_causal4(p["x"], p["conv_w"], p["conv_b"], p["conv_state"], io)
    # the kernel takes the sum in fp64 in the definition's order and rounds it once
    np.testing.assert_array_equal(host(u), uo)
    np.testing.assert_array_equal(host(so), soo)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_conv_rounds_once_on_constructed_sums(lib, io):
    """Sums where rounding first to fp32 and then to the I/O dtype would pick the other
    neighbour, and sums in bf16's subnormal range; the kernel's u must equal the oracle's
    once-rounded sum bit for bit.  Channels 0..31, step 3: u = s (1 + 2^-p) + s' 2^-40 with
    p = 8 (bf16) or 24 (fp32), i.e. an exact halfway point of the I/O dtype moved by a tap
    product far below an fp32 ulp.  Channels 32..63, step 5: u = k 2^-140."""
    D, p = 64, (8 if io == "bf16" else 24)
    rng = np.random.default_rng(8)
    ch = np.arange(D)
    lo = ch < 32
    s1 = np.where(ch % 2 == 0, 1.0, -1.0)
    s2 = np.where(ch % 4 < 2, 1.0, -1.0)
    w = np.zeros((4, D))
    x = np.zeros((1, 6, D))
    w[3] = np.where(lo, s1, 0.0)                 # step 3, tap 3: x_0 = 1
    w[2] = np.where(lo, s1 * 2.0 ** -p, 0.0)     # tap 2: x_1 = 1
    w[1] = np.where(lo, s2 * 2.0 ** -20, 0.0)    # tap 1: x_2 = 2^-20
    x[0, 0] = x[0, 1] = np.where(lo, 1.0, 0.0)
    x[0, 2] = np.where(lo, 2.0 ** -20, 0.0)
    w[0] = np.where(lo, 0.0, 2.0 ** -70)         # step 5, tap 0: x_5 = k 2^-70
    x[0, 5] = np.where(lo, 0.0, rng.integers(1, 256, D) * 2.0 ** -70)
    d = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda().to(dt)
    dt = TORCH_IO[io]
    xd, wd = d(x, dt), d(w, dt)
    assert np.array_equal(host(xd), x) and np.array_equal(host(wd), w)
    u = torch.empty_like(xd)
    lib.conv1d_causal4(xd, wd, None, None, u, None)
    torch.cuda.synchronize()
    uo, _ = oracle.conv1d_causal4(x, w, None, None, io)
    np.testing.assert_array_equal(host(u), uo)
    assert len(np.unique(uo[0, 3, :32])) == 4         # the tiny taps decide the neighbour


def test_forward_is_bitwise_reproducible(lib):
    p = workloads.make_inputs(workloads.TRAIN_FWD.with_shape(B=4, T=1000, D=256))
    d = device_inputs(p)
    outs = [lib.forward(d["x"], d["conv_w"], d["conv_b"], None, d["W_a"], d["W_x"], d["b_a"],
                        d["b_x"], d["lam"], None, p["c"]) for _ in range(3)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o[0], outs[0][0]) and torch.equal(o[1], outs[0][1])


def test_bf16_rounding_of_halfway_sums_is_exact(lib):
    """R1 on halfway cases: with conv taps (1, 1, 0, 0) the fp32 sum x_t + x_{t-1} of two
    bf16 values lands exactly halfway between bf16 neighbours; the GPU's rounding must
    equal the oracle's round-to-nearest-even bit for bit."""
    D, T = 64, 48
    k = np.arange(T)[:, None] % 16
    x = np.zeros((1, T, D))
    x[0, 0::2] = 1.0 + (k[0::2] + np.arange(D)[None, :] % 8) * 2.0 ** -7   # even steps: 1 + j 2^-7
    x[0, 1::2] = 2.0 ** -8 * (1 + (np.arange(D)[None, :] % 3 == 0))         # odd: 2^-8 or 2^-7
    x[0, 1::2] *= np.where(np.arange(D) % 2 == 0, 1, -1)[None, :]
    w = np.zeros((4, D)); w[0] = 1.0; w[1] = 1.0
    xd = dev(x, torch.bfloat16)
    assert np.array_equal(host(xd), x)
    wd = dev(w, torch.bfloat16)
    u = torch.empty_like(xd)
    lib.conv1d_causal4(xd, wd, None, None, u, None)
    torch.cuda.synchronize()
    uo, _ = oracle.conv1d_causal4(x, w, None, None, "bf16")
    np.testing.assert_array_equal(host(u), uo)
    # and the ties really occur (half of the odd-step sums sit exactly between neighbours)
    s = x[0, 1:] + x[0, :-1]
    assert np.sum(oracle.round_io(s, "bf16") != s) > 100


def test_maximum_size_matches_geometric_closed_form(lib):
    """The largest shape the ABI accepts (B T D just under 2^31 elements, T ragged: 4096 tiles
    of 256 steps with 255 in the last) on the fused bf16 path.  With W_a = W_x = 0, an
    identity conv and x constant over time, r, i and a are constant per channel and Eq. (4)
    has the closed form h_t = (1 - a^t) / (1 - a) m i x (h0 = 0, t steps done), checked at
    sampled steps and for h_T."""
    B, T, D = 8, 1048575, 256
    assert B * T * D < 2 ** 31
    rng = np.random.default_rng(11)
    xi = torch.from_numpy(rng.standard_normal(D).astype(np.float32)).to(torch.bfloat16)
    b_a = rng.normal(0.0, 0.5, D).astype(np.float32)
    b_x = rng.normal(0.0, 0.5, D).astype(np.float32)
    U = rng.uniform(0.9, 0.999, D)
    c = 8.0
    lam = np.log(U ** (1 / c) / (1 - U ** (1 / c))).astype(np.float32)
    x = xi.cuda()[None, None, :].expand(B, T, D).contiguous()
    conv_w = torch.zeros((4, D), dtype=torch.bfloat16, device="cuda")
    conv_w[0] = 1.0
    Wz = torch.zeros((D, D), dtype=torch.bfloat16, device="cuda")
    y, hT, _ = lib.forward(x, conv_w, None, None, Wz, Wz, dev(b_a), dev(b_x), dev(lam), None, c)
    torch.cuda.synchronize()
    del x
    _, i, _, a, m = oracle.gates(b_a.astype(np.float64), b_x.astype(np.float64),
                                 lam.astype(np.float64), c)
    xv = xi.float().numpy().astype(np.float64)
    steady = m * i * xv / (1.0 - a)
    ts = np.array([0, 1, 2, 255, 256, 257, 4095, T // 2, T - 256, T - 255, T - 2, T - 1])
    want = (1.0 - a[None, :] ** (ts[:, None] + 1.0)) * steady[None, :]      # [len(ts), D]
    got = host(y[:, torch.from_numpy(ts).cuda(), :])                          # [B, len(ts), D]
    e_y = err(got, np.broadcast_to(want, got.shape))
    e_h = err(host(hT), np.broadcast_to(want[-1], (B, D)))
    print(f"max size B={B} T={T} D={D}: err(y)={e_y:.3e} err(h_T)={e_h:.3e}", flush=True)
    assert e_y <= TOL["bf16"] and e_h <= TOL["bf16"]


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_forward_graph_replays_match_eager(lib, io):
    """rglru_fwd captured in a hipGraph (its look-back status is initialised by kernels, not
    memset nodes), replayed several times with eager work and synchronisations in between;
    every replay equals the eager result bit for bit."""
    w = workloads.TRAIN_FWD.with_shape(B=2, T=700, D=320, io=io, h0="normal", history="normal")
    p = workloads.make_inputs(w)
    d = device_inputs(p)
    B, T, D = w.B, w.T, w.D
    y = torch.empty((B, T, D), dtype=TORCH_IO[io], device="cuda")
    hT = torch.empty((B, D), device="cuda")
    cso = torch.empty((B, 3, D), dtype=TORCH_IO[io], device="cuda")
    ws = lib.workspace(lib.fwd_workspace_bytes(B, T, D, TORCH_IO[io]))

    def run():
        lib.rglru_fwd(d["x"], d["conv_w"], d["conv_b"], d["conv_state"], d["W_a"], d["W_x"],
                      d["b_a"], d["b_x"], d["lam"], d["h0"], y, hT, cso, ws, p["c"])

    run()
    torch.cuda.synchronize()
    ref = (y.clone(), hT.clone(), cso.clone())
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            run()
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(4):
        y.zero_()
        hT.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ref[0]) and torch.equal(hT, ref[1]) and torch.equal(cso, ref[2]), rep
        _ = (d["x"].float() * 3).sum().item()       # unrelated eager work between replays


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_backward_graph_replays_match_eager(lib, io):
    """rglru_fwd_train + rglru_bwd_saved and rglru_bwd captured in one hipGraph (the reverse
    scan's tickets and look-back status are reset by kernels inside the calls, not memset
    nodes), replayed several times with eager work and synchronisations in between; every
    replay gives the eager gradients bit for bit."""
    w = workloads.TRAIN_BWD.with_shape(B=2, T=300, D=192, io=io, h0="normal", history="normal",
                                       with_dy=True)
    p = workloads.make_inputs(w)
    d = device_inputs(p)
    B, T, D = w.B, w.T, w.D
    t = TORCH_IO[io]
    f32 = dict(dtype=torch.float32, device="cuda")
    dh_T = torch.randn((B, D), generator=torch.Generator().manual_seed(5)).cuda()

    def grads():
        return [torch.empty((B, T, D), **f32), torch.empty((4, D), **f32), torch.empty(D, **f32),
                torch.empty((D, D), **f32), torch.empty((D, D), **f32), torch.empty(D, **f32),
                torch.empty(D, **f32), torch.empty(D, **f32), torch.empty((B, D), **f32)]
    g_bwd, g_saved = grads(), grads()
    y = torch.empty((B, T, D), dtype=t, device="cuda")
    hT = torch.empty((B, D), **f32)
    cso = torch.empty((B, 3, D), dtype=t, device="cuda")
    ws_b = lib.workspace(lib.bwd_workspace_bytes(B, T, D, t))
    ws_f = lib.workspace(lib.fwd_train_workspace_bytes(B, T, D, t))
    ws_s = lib.workspace(lib.bwd_saved_workspace_bytes(B, T, D, t))
    saved = lib.workspace(lib.train_saved_bytes(B, T, D, t))
    common = (d["x"], d["conv_w"], d["conv_b"], d["conv_state"], d["W_a"], d["W_x"])

    def run():
        lib.rglru_bwd(*common, d["b_a"], d["b_x"], d["lam"], d["h0"], d["dy"], dh_T, *g_bwd, ws_b,
                      p["c"])
        lib.rglru_fwd_train(*common, d["b_a"], d["b_x"], d["lam"], d["h0"], y, hT, cso, saved,
                            ws_f, p["c"])
        lib.rglru_bwd_saved(*common, d["lam"], d["h0"], d["dy"], dh_T, *g_saved, saved, ws_s,
                            p["c"])

    run()
    torch.cuda.synchronize()
    ref = [a.clone() for a in g_bwd + g_saved + [y, hT]]
    for a, b in zip(g_bwd, g_saved):       # the two routes give the same gradients
        assert torch.equal(a, b)
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            run()
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(3):
        for a in g_bwd + g_saved + [y, hT]:
            a.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (a, r) in enumerate(zip(g_bwd + g_saved + [y, hT], ref)):
            assert torch.equal(a, r), (rep, i)
        _ = (d["x"].float() * 3).sum().item()       # unrelated eager work between replays
