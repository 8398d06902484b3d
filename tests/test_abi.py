"""The C ABI of librglru.so, checked without a GPU: the library loads, exports every
symbol include/rglru.h declares, and rejects invalid arguments before any HIP call."""
import ctypes
import os
import re

import pytest

import gated_linear_rnn_amd as g

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rglru.h")
TEST_HEADER = os.path.join(ROOT, "gated_linear_rnn_amd", "csrc", "rglru_testing.h")


def _declared_functions(header=HEADER):
    src = open(header).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w ]*?[\s\*]+([a-z_][a-z0-9_]*)\s*\(", src, re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    return g.load()


def test_header_declares_the_expected_entry_points():
    assert _declared_functions() == sorted(g.EXPORTS)


def test_every_declared_symbol_is_exported(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_public_header_has_no_test_hooks():
    """The public interface takes no process-wide settings: test-only entry points live in
    their own header, take their settings as an argument, and the public names are disjoint
    from them."""
    public = _declared_functions()
    assert not [n for n in public if "test" in n], public
    src = open(HEADER).read()
    assert "rglru_testing" not in src and "test hook" not in src.lower()
    from gated_linear_rnn_amd import testing
    assert _declared_functions(TEST_HEADER) == sorted(testing.EXPORTS)


def test_test_only_symbols_are_exported_and_take_their_settings_per_call(lib):
    from gated_linear_rnn_amd import testing
    for name in testing.EXPORTS:
        assert hasattr(lib, name), name
    k = testing.knobs()
    assert (k.lru_ticket_guess, k.scan_direct_polls, k.lookback_polls) == (0, 2048, 1 << 20)
    assert testing.knobs(lookback_polls=-1).lookback_polls == -1
    assert testing.knobs().lookback_polls == 1 << 20          # nothing persists between calls


def test_status_strings_cover_every_code(lib):
    codes = {0: "RGLRU_OK", -1: "RGLRU_EINVAL", -2: "RGLRU_ESHAPE", -3: "RGLRU_EDTYPE",
             -4: "RGLRU_EWORKSPACE", -5: "RGLRU_EHIP", -6: "RGLRU_EINTERNAL", -7: "RGLRU_ESTALL"}
    for c, name in codes.items():
        assert g.status_string(c).startswith(name)
    assert "unknown" in g.status_string(7)


def test_workspace_queries(lib):
    assert lib.rglru_fwd_workspace_bytes(8, 2048, 2560, 1) >= 8 * 2048 * 2560 * 2          # u
    assert lib.rglru_fwd_workspace_bytes(8, 2048, 2560, 0) >= 8 * 2048 * 2560 * 12         # u, a, beta
    assert lib.rglru_lru_workspace_bytes(8, 2048, 2560, 1) < lib.rglru_fwd_workspace_bytes(8, 2048, 2560, 1)
    assert lib.rglru_fwd_workspace_bytes(1, 1, 63, 1) == 0          # D % 64
    assert lib.rglru_fwd_workspace_bytes(0, 1, 64, 1) == 0
    assert lib.rglru_fwd_workspace_bytes(1, 1, 64, 7) == 0          # dtype
    assert lib.rglru_bwd_workspace_bytes(4, 2048, 5376, 1) > lib.rglru_fwd_workspace_bytes(4, 2048, 5376, 1)
    assert lib.rglru_decode_workspace_bytes(256, 2560, 1) >= 256 * 2560 * 2
    assert lib.rglru_decode_workspace_bytes(256, 2560, 0) >= 3 * 256 * 2560 * 4


# Fake, 16-byte aligned "device" addresses: validation must reject the call before any HIP
# call would touch them.  These run only where no GPU is visible, so a validation bug can
# never hand a fake address to a kernel.
A = 1 << 20
no_gpu = pytest.mark.skipif(__import__("torch").cuda.is_available(),
                            reason="fake device addresses are only passed where no GPU exists")
BAD = A + 4


def _fwd(lib, B=1, T=4, D=64, io=1, c=8.0, **over):
    args = dict(x=A, conv_w=None, conv_b=None, cs=None, Wa=A, Wx=A, ba=A, bx=A, lam=A, h0=None,
                y=A, hT=None, cso=None, ws=A, wsb=1 << 40)
    args.update(over)
    return lib.rglru_fwd(B, T, D, io, c, *[args[k] for k in
                         ("x", "conv_w", "conv_b", "cs", "Wa", "Wx", "ba", "bx", "lam", "h0", "y",
                          "hT", "cso", "ws")], args["wsb"], None)


@no_gpu
def test_fwd_rejects_invalid_arguments(lib):
    assert _fwd(lib, B=0) == -1
    assert _fwd(lib, T=-3) == -1
    assert _fwd(lib, D=96) == -2
    assert _fwd(lib, B=1 << 12, T=1 << 12, D=1 << 7) == -2            # B*T*D >= 2^31
    assert _fwd(lib, io=2) == -3
    for k in ("x", "Wa", "Wx", "ba", "bx", "lam", "y"):
        assert _fwd(lib, **{k: None}) == -1, k
    assert _fwd(lib, x=BAD) == -1                                     # misaligned
    assert _fwd(lib, h0=BAD) == -1
    assert _fwd(lib, c=-1.0) == -1
    assert _fwd(lib, c=float("nan")) == -1
    assert _fwd(lib, ws=None) == -4
    assert _fwd(lib, wsb=10) == -4


@no_gpu
def test_decode_and_conv_and_bwd_reject_invalid_arguments(lib):
    r = lib.rglru_decode_step(1, 64, 1, 8.0, A, A, None, None, A, A, A, A, A, A, A, A, 1 << 40, None)
    assert r == -1                                                    # conv_w without state
    r = lib.rglru_decode_step(1, 64, 1, 8.0, A, None, None, None, A, A, A, A, A, None, A, A, 1 << 40, None)
    assert r == -1                                                    # h missing
    r = lib.rglru_decode_step(1, 64, 1, 8.0, A, None, None, None, A, A, A, A, A, A, A, A, 1, None)
    assert r == -4
    assert lib.conv1d_causal4(1, 4, 64, 1, None, A, None, None, A, None, None) == -1
    assert lib.conv1d_causal4(1, 4, 65, 1, A, A, None, None, A, None, None) == -2
    assert lib.conv1d_causal4(1, 4, 64, 5, A, A, None, None, A, None, None) == -3
    bwd = [A] * 21
    bwd[1] = None        # conv_w NULL
    r = lib.rglru_bwd(1, 4, 64, 1, 8.0, *bwd, A, 10, None)
    assert r == -4
    bwd[10] = None       # dy
    assert lib.rglru_bwd(1, 4, 64, 1, 8.0, *bwd, A, 1 << 40, None) == -1


def test_block_workspace_query(lib):
    n = 8 * 2048 * 2560
    assert lib.rglru_block_fwd_workspace_bytes(8, 2048, 2560, 2560, 1) >= 3 * n * 2   # p, g, u
    assert lib.rglru_block_fwd_workspace_bytes(8, 2048, 2560, 2560, 0) >= 6 * n * 4   # pq, p, g, y, u
    assert lib.rglru_block_fwd_workspace_bytes(1, 1, 64, 96, 1) == 0     # R % 64
    assert lib.rglru_block_fwd_workspace_bytes(1, 1, 96, 64, 1) == 0     # D % 64
    assert lib.rglru_block_fwd_workspace_bytes(1, 1, 64, 64, 3) == 0     # dtype
    assert lib.rglru_block_fwd_workspace_bytes(1 << 12, 1 << 12, 64, 128, 1) == 0   # B*T*R >= 2^31


def _block(lib, B=1, T=4, D=64, R=128, io=1, c=8.0, **over):
    names = ("x", "W_in", "conv_w", "conv_b", "cs", "Wa", "Wx", "ba", "bx", "lam", "h0", "W_out",
             "out", "hT", "cso", "ws")
    args = dict.fromkeys(names, A)
    args.update(conv_w=None, conv_b=None, cs=None, h0=None, hT=None, cso=None, wsb=1 << 40)
    args.update(over)
    return lib.rglru_block_fwd(B, T, D, R, io, c, *[args[k] for k in names], args["wsb"], None)


@no_gpu
def test_block_rejects_invalid_arguments(lib):
    assert _block(lib, B=0) == -1
    assert _block(lib, R=0) == -1
    assert _block(lib, R=96) == -2
    assert _block(lib, D=32) == -2
    assert _block(lib, B=1 << 12, T=1 << 12, D=1 << 7) == -2
    assert _block(lib, io=2) == -3
    for k in ("x", "W_in", "Wa", "Wx", "ba", "bx", "lam", "W_out", "out"):
        assert _block(lib, **{k: None}) == -1, k
    assert _block(lib, W_out=BAD) == -1
    assert _block(lib, c=-2.0) == -1
    assert _block(lib, ws=None) == -4
    assert _block(lib, wsb=100) == -4


def test_mlp_workspace_query(lib):
    assert lib.gated_mlp_fwd_workspace_bytes(8, 2048, 2560, 7680, 1) >= 8 * 2048 * 7680 * 2
    assert lib.gated_mlp_fwd_workspace_bytes(8, 2048, 2560, 7680, 0) >= 8 * 2048 * 7680 * 8
    assert lib.gated_mlp_fwd_workspace_bytes(1, 1, 64, 100, 1) == 0      # MD % 64
    assert lib.gated_mlp_fwd_workspace_bytes(1, 1, 100, 64, 1) == 0      # D % 64
    assert lib.gated_mlp_fwd_workspace_bytes(1 << 12, 1 << 10, 64, 1024, 1) == 0   # B*T*MD >= 2^31


@no_gpu
def test_mlp_rejects_invalid_arguments(lib):
    def call(B=1, T=4, D=64, MD=192, io=1, x=A, W1=A, W2=A, W3=A, out=A, ws=A, wsb=1 << 40):
        return lib.gated_mlp_fwd(B, T, D, MD, io, x, W1, W2, W3, out, ws, wsb, None)
    assert call(T=0) == -1
    assert call(MD=96) == -2
    assert call(io=4) == -3
    for k in ("x", "W1", "W2", "W3", "out"):
        assert call(**{k: None}) == -1, k
    assert call(W2=BAD) == -1
    assert call(ws=None) == -4
    assert call(wsb=5) == -4


def test_mqa_workspace_query(lib):
    assert lib.local_mqa_fwd_workspace_bytes(8, 2048, 2560, 1) >= 8 * 2048 * (2 * 2560 + 256) * 2
    assert lib.local_mqa_fwd_workspace_bytes(1, 1, 192, 1) == 0         # D % 128
    assert lib.local_mqa_fwd_workspace_bytes(1, 1, 128, 9) == 0         # dtype


@no_gpu
def test_mqa_rejects_invalid_arguments(lib):
    def call(B=1, T=4, D=128, io=1, window=16, pos0=0, x=A, Wqkv=A, Wo=A, out=A, k=None, v=None,
             ws=A, wsb=1 << 40):
        return lib.local_mqa_fwd(B, T, D, io, window, pos0, x, Wqkv, Wo, out, k, v, ws, wsb, None)
    assert call(window=0) == -1
    assert call(pos0=-1) == -1
    assert call(D=64) == -2
    assert call(io=3) == -3
    for kw in ("x", "Wqkv", "Wo", "out"):
        assert call(**{kw: None}) == -1, kw
    assert call(k=BAD) == -1
    assert call(ws=None) == -4
    assert call(wsb=7) == -4


def test_mqa_decode_workspace_query_and_validation(lib):
    assert lib.local_mqa_decode_workspace_bytes(256, 2560, 1) >= 2 * 256 * 2560 * 2
    assert lib.local_mqa_decode_workspace_bytes(4, 200, 1) == 0          # D % 128


@no_gpu
def test_mqa_decode_rejects_invalid_arguments(lib):
    def call(B=2, D=128, io=1, window=16, pos=A, x=A, Wqkv=A, Wo=A, kc=A, vc=A, out=A, ws=A,
             wsb=1 << 40):
        return lib.local_mqa_decode_step(B, D, io, window, pos, x, Wqkv, Wo, kc, vc, out, ws, wsb, None)
    assert call(window=0) == -1
    assert call(B=0) == -1
    assert call(D=96) == -2
    assert call(io=5) == -3
    for kw in ("pos", "x", "Wqkv", "Wo", "kc", "vc", "out"):
        assert call(**{kw: None}) == -1, kw
    assert call(vc=BAD) == -1
    assert call(ws=None) == -4


def test_block_decode_workspace_query(lib):
    assert lib.rglru_block_decode_workspace_bytes(256, 2560, 2560, 1) >= 4 * 256 * 2560 * 2
    assert lib.rglru_block_decode_workspace_bytes(1, 64, 96, 1) == 0


@no_gpu
def test_block_decode_rejects_invalid_arguments(lib):
    def call(B=2, D=64, R=128, io=1, c=8.0, **over):
        names = ("x", "W_in", "conv_w", "conv_b", "cs", "Wa", "Wx", "ba", "bx", "lam", "h", "W_out", "out", "ws")
        args = dict.fromkeys(names, A)
        args.update(conv_w=None, conv_b=None, cs=None)
        wsb = over.pop("wsb", 1 << 40)
        args.update(over)
        return lib.rglru_block_decode_step(B, D, R, io, c, *[args[k] for k in names[:-1]], args["ws"], wsb, None)
    assert call(B=0) == -1
    assert call(R=100) == -2
    assert call(io=2) == -3
    for k in ("x", "W_in", "Wa", "Wx", "ba", "bx", "lam", "h", "W_out", "out"):
        assert call(**{k: None}) == -1, k
    assert call(conv_w=A) == -1                                          # conv_w without state
    assert call(h=BAD) == -1
    assert call(ws=None) == -4
    assert call(wsb=3) == -4



@no_gpu
def test_layer_halves_and_training_pair_reject_invalid_arguments(lib):
    """rglru_lru, rglru_gates, rglru_scan, rglru_fwd_train and rglru_bwd_saved: bad shapes,
    dtypes, missing or misaligned pointers, short workspaces and short saved buffers are
    refused before any HIP call."""
    big = 1 << 40

    def lru(B=1, T=4, D=64, io=1, c=8.0, **o):
        a = dict(u=A, Wa=A, Wx=A, ba=A, bx=A, lam=A, h0=None, y=A, hT=None, ws=A, wsb=big)
        a.update(o)
        return lib.rglru_lru(B, T, D, io, c, a["u"], a["Wa"], a["Wx"], a["ba"], a["bx"], a["lam"],
                             a["h0"], a["y"], a["hT"], a["ws"], a["wsb"], None)
    assert lru(B=0) == -1 and lru(D=32) == -2 and lru(io=9) == -3 and lru(c=-2.0) == -1
    for k in ("u", "Wa", "Wx", "ba", "bx", "lam", "y"):
        assert lru(**{k: None}) == -1, k
    assert lru(y=BAD) == -1 and lru(ws=None) == -4 and lru(wsb=16) == -4

    def gates(B=1, T=4, D=64, io=1, c=8.0, **o):
        a = dict(u=A, Wa=A, Wx=A, ba=A, bx=A, lam=A, a=A, beta=A)
        a.update(o)
        return lib.rglru_gates(B, T, D, io, c, *[a[k] for k in ("u", "Wa", "Wx", "ba", "bx", "lam",
                                                                 "a", "beta")], None)
    assert gates(T=0) == -1 and gates(D=100) == -2 and gates(io=3) == -3
    for k in ("u", "Wa", "Wx", "ba", "bx", "lam", "a", "beta"):
        assert gates(**{k: None}) == -1, k
    assert gates(beta=BAD) == -1

    def scan(B=1, T=4, D=64, io=1, **o):
        a = dict(x=A, cw=None, cb=None, cs=None, a=A, beta=A, h0=None, y=A, hT=None, ws=A, wsb=big)
        a.update(o)
        return lib.rglru_scan(B, T, D, io, *[a[k] for k in ("x", "cw", "cb", "cs", "a", "beta", "h0",
                                                            "y", "hT", "ws")], a["wsb"], None)
    assert scan(B=-1) == -1 and scan(D=65) == -2 and scan(io=7) == -3
    for k in ("x", "a", "beta", "y"):
        assert scan(**{k: None}) == -1, k
    assert scan(a=BAD) == -1 and scan(ws=None) == -4 and scan(wsb=8) == -4

    def fwd_train(B=1, T=4, D=64, io=1, c=8.0, **o):
        a = dict(x=A, cw=None, cb=None, cs=None, Wa=A, Wx=A, ba=A, bx=A, lam=A, h0=None, y=A,
                 hT=None, cso=None, saved=A, sb=big, ws=A, wsb=big)
        a.update(o)
        return lib.rglru_fwd_train(B, T, D, io, c, *[a[k] for k in (
            "x", "cw", "cb", "cs", "Wa", "Wx", "ba", "bx", "lam", "h0", "y", "hT", "cso", "saved")],
            a["sb"], a["ws"], a["wsb"], None)
    assert fwd_train(B=0) == -1 and fwd_train(D=96) == -2 and fwd_train(io=4) == -3
    for k in ("x", "Wa", "Wx", "ba", "bx", "lam", "y", "saved"):
        assert fwd_train(**{k: None}) == -1, k
    assert fwd_train(saved=BAD) == -1
    assert fwd_train(sb=64) == -1                          # saved buffer too short
    assert fwd_train(ws=None) == -4 and fwd_train(wsb=64) == -4

    def bwd_saved(B=1, T=4, D=64, io=1, c=8.0, **o):
        names = ("x", "cw", "cb", "cs", "Wa", "Wx", "lam", "h0", "dy", "dhT", "dx", "dcw", "dcb",
                 "dWa", "dWx", "dba", "dbx", "dlam", "dh0", "saved")
        a = dict.fromkeys(names, A)
        a.update(cw=None, cb=None, cs=None, h0=None, dhT=None, dcw=None, dcb=None, dh0=None,
                 sb=big, ws=A, wsb=big)
        a.update(o)
        return lib.rglru_bwd_saved(B, T, D, io, c, *[a[k] for k in names], a["sb"], a["ws"],
                                   a["wsb"], None)
    assert bwd_saved(T=0) == -1 and bwd_saved(D=80) == -2 and bwd_saved(io=6) == -3
    for k in ("x", "Wa", "Wx", "lam", "dy", "dx", "dWa", "dWx", "dba", "dbx", "dlam"):
        assert bwd_saved(**{k: None}) == -1, k
    assert bwd_saved(cw=A) == -1                           # conv weights without their gradients
    assert bwd_saved(dx=BAD) == -1
    assert bwd_saved(sb=64) == -1                          # saved buffer too short
    assert bwd_saved(ws=None) == -4 and bwd_saved(wsb=64) == -4

@no_gpu
def test_workspace_status_rejects_invalid_arguments(lib):
    assert lib.rglru_workspace_status(None, 1 << 20, None) == -1
    assert lib.rglru_workspace_status(BAD, 1 << 20, None) == -1
    assert lib.rglru_workspace_status(A, 255, None) == -4


@no_gpu
def test_noalloc_decode_rejects_before_any_hip_call(lib):
    """rglru_decode_step_noalloc validates the shape and its fixed scratch size first."""
    f = lib.rglru_decode_step_noalloc
    args = lambda B, D, io=1: (B, D, io, 8.0, A, None, None, None, A, A, A, A, A, A, A, None)
    assert f(*args(0, 64)) == -1
    assert f(*args(2, 96)) == -2
    assert f(*args(2, 64, io=5)) == -3
    assert g.status_string(-8).startswith("RGLRU_ESCRATCH")
    assert f(*args(1024, 8192)) == -8                      # needs more than the fixed scratch


def test_bench_refuses_more_than_one_gpu():
    """bench.py runs on one GPU; --gpus N > 1 ends with a message and a nonzero status,
    before any device work."""
    import subprocess
    import sys
    from pathlib import Path
    root = Path(__file__).resolve().parents[1]
    r = subprocess.run([sys.executable, str(root / "bench.py"), "--gpus", "2"], cwd=root,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""
