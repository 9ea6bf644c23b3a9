"""CPU-only checks of the C ABI: the library loads, exports every declared symbol, and
rejects invalid arguments before touching HIP (no kernel is launched here)."""
import ctypes
import os
import re

import pytest

from gated_linear_recurrence_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rglru.h")

OK, NULL, SHAPE, UNSUP, WS, ALIAS = 0, 1, 2, 3, 4, 5


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_0-9]+)\s*\(", src)) - {"sizeof"})


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        pytest.skip("librglru.so not built")
    return binding.load_library()


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert set(names) >= {"rglru_prefill", "rglru_decode_step", "conv1d_state_update"}
    assert set(names) == set(binding.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version_and_strings(lib):
    assert lib.rglru_abi_version() == 7
    for st in range(7):
        assert lib.rglru_status_string(st)
    assert lib.rglru_status_string(99) == b"unknown status"


def _params(D=512, H=2, dtype=1, base=0x100000):
    p = binding.rglru_params()
    p.D, p.n_heads, p.dtype = D, H, dtype
    p.conv_w, p.conv_b = base + 0x0, base + 0x10000
    p.gate_a_w, p.gate_a_b = base + 0x20000, base + 0x220000
    p.gate_x_w, p.gate_x_b = base + 0x230000, base + 0x430000
    p.lambda_ = base + 0x440000
    return p


X, Y, OUT, H0, HL, C0, CL, WSP = (0x10000000 * k for k in range(1, 9))


def _prefill(lib, p, B=2, T=100, x=X, y=Y, out=OUT, h0=H0, hl=HL, c0=C0, cl=CL, ws=WSP,
             ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = lib.rglru_prefill_workspace_bytes(B, T, p.D, p.n_heads, p.dtype)
    return lib.rglru_prefill(ctypes.byref(p), B, T, x, y, out, h0, hl, c0, cl, ws, ws_bytes, None)


def test_workspace_bytes(lib):
    f = lib.rglru_prefill_workspace_bytes
    # header plus one word per (segment but the last, sequence, channel)
    assert f(8, 8192, 2560, 10, 1) == 4096 + 127 * 8 * 2560 * 8
    assert f(2, 65536, 4096, 16, 1) == 4096 + 1023 * 2 * 4096 * 8
    assert f(1, 65, 256, 2, 0) == 4096 + 1 * 1 * 256 * 8
    assert f(1, 64, 256, 2, 0) == 4096
    assert f(1, 1, 256, 2, 0) == 4096
    assert f(1, 0, 256, 2, 0) == 4096
    assert f(0, 10, 256, 2, 0) == 0
    assert f(1, -1, 256, 2, 0) == 0
    assert f(1, 10, 255, 2, 0) == 0
    assert f(1, 10, 256, 2, 7) == 0


def test_prefill_validation(lib):
    assert lib.rglru_prefill(None, 1, 1, X, Y, OUT, None, None, None, None, WSP, 1 << 20, None) == NULL
    p = _params()
    assert _prefill(lib, p, B=0) == SHAPE
    assert _prefill(lib, p, T=-1) == SHAPE
    assert _prefill(lib, p, x=None) == NULL
    assert _prefill(lib, p, out=None) == NULL
    assert _prefill(lib, _params(D=510, H=4)) == SHAPE       # D % H
    assert _prefill(lib, _params(D=512, H=8)) == UNSUP        # bs = 64
    assert _prefill(lib, _params(dtype=5)) == UNSUP
    assert _prefill(lib, p, x=X + 2) == UNSUP                 # alignment
    big = _params(D=4096, H=16)
    assert _prefill(lib, big, B=1, T=262144) == UNSUP         # one bf16 sequence of 2 GiB
    assert _prefill(lib, big, B=1, T=262143) != UNSUP         # just below (then other checks)
    assert _prefill(lib, big, B=87382, T=1) == UNSUP          # conv windows of 2 GiB
    assert _prefill(lib, big, B=87381, T=1) != UNSUP
    assert _prefill(lib, p, ws=None) == WS
    assert _prefill(lib, p, ws_bytes=1000) == WS
    assert _prefill(lib, p, out=X) == ALIAS
    assert _prefill(lib, p, out=Y + 64) == ALIAS
    assert _prefill(lib, p, hl=X + 16) == ALIAS
    assert _prefill(lib, p, hl=H0 + 16) == ALIAS               # partial overlap with h0
    assert _prefill(lib, p, cl=C0 + 16) == ALIAS
    assert _prefill(lib, p, ws=OUT) == ALIAS
    q = _params()
    q.gate_a_w = None
    assert _prefill(lib, q) == NULL
    q = _params()
    q.lambda_ = None
    assert _prefill(lib, q) == NULL


def test_decode_validation(lib):
    p = _params()
    f = lib.rglru_decode_step
    assert f(ctypes.byref(p), 0, X, 0, Y, 0, OUT, 0, H0, C0, None, 0, None) == SHAPE
    assert f(ctypes.byref(p), 4, None, 0, Y, 0, OUT, 0, H0, C0, None, 0, None) == NULL
    assert f(ctypes.byref(p), 4, X, 100, Y, 0, OUT, 0, H0, C0, None, 0, None) == SHAPE  # ld_x < D
    assert f(ctypes.byref(p), 4, X, 513, Y, 0, OUT, 0, H0, C0, None, 0, None) == UNSUP  # row alignment
    assert f(ctypes.byref(p), 4, X, 0, Y, 0, X, 0, H0, C0, None, 0, None) == ALIAS
    assert f(ctypes.byref(p), 4, X, 0, Y, 0, OUT, 0, X + 64, C0, None, 0, None) == ALIAS
    assert f(ctypes.byref(p), 4, X, 0, Y, 0, OUT, 0, H0, Y, None, 0, None) == ALIAS


def test_decode_workspace_validation(lib):
    p = _params()
    f = lib.rglru_decode_step
    need = lib.rglru_decode_workspace_bytes(4, 512, 1)
    assert need == 16 * 512 * 2                    # sequences in blocks of 16
    assert lib.rglru_decode_workspace_bytes(4, 512, 0) == 16 * 512 * 4
    assert lib.rglru_decode_workspace_bytes(17, 512, 1) == 32 * 512 * 2
    assert lib.rglru_decode_workspace_bytes(0, 512, 1) == 0
    assert f(ctypes.byref(p), 4, X, 0, Y, 0, OUT, 0, H0, C0, WSP, need - 2, None) == WS
    assert f(ctypes.byref(p), 4, X, 0, Y, 0, OUT, 0, H0, C0, WSP + 8, need, None) == UNSUP
    assert f(ctypes.byref(p), 4, X, 0, Y, 0, OUT, 0, H0, C0, OUT + 16, need, None) == ALIAS
    assert f(ctypes.byref(p), 4, X, 0, Y, 0, OUT, 0, H0, C0, C0, need, None) == ALIAS
    assert f(ctypes.byref(p), 4, X, 0, Y, 0, OUT, 0, H0, C0, H0 + 4096, need, None) == ALIAS


def test_conv_update_validation(lib):
    p = _params()
    f = lib.conv1d_state_update
    assert f(ctypes.byref(p), 0, 4, X, C0, OUT, None) == SHAPE
    assert f(ctypes.byref(p), 2, -1, X, C0, OUT, None) == SHAPE
    assert f(ctypes.byref(p), 2, 4, X, None, OUT, None) == NULL
    assert f(ctypes.byref(p), 2, 4, X, C0, X, None) == ALIAS
    assert f(ctypes.byref(p), 2, 0, None, C0, None, None) == OK   # nothing to do
    assert f(ctypes.byref(_params(D=100, H=1)), 2, 4, X, C0, None, None) == UNSUP  # D % 8


def test_linear_validation(lib):
    f = lib.rglru_linear
    W, B_ = 0x60000000, 0x70000000
    assert f(-1, 128, 256, X, W, B_, OUT, None) == SHAPE
    assert f(4, 0, 256, X, W, B_, OUT, None) == SHAPE
    assert f(4, 100, 256, X, W, B_, OUT, None) == UNSUP       # K % 128
    assert f(4, 128, 200, X, W, B_, OUT, None) == UNSUP       # N % 256
    assert f(4, 1 << 22, 256, X, W, B_, OUT, None) == UNSUP   # K bound
    assert f(4, 128, 256, None, W, B_, OUT, None) == NULL
    assert f(4, 128, 256, X, None, B_, OUT, None) == NULL
    assert f(4, 128, 256, X + 2, W, B_, OUT, None) == UNSUP   # alignment
    assert f(4, 128, 256, X, W, B_, X + 64, None) == ALIAS
    assert f(4, 128, 256, X, W, B_, W, None) == ALIAS
    assert f(0, 128, 256, None, W, None, None, None) == OK     # nothing to do, no launch


def _proj(Dm=512, base=0x90000000):
    q = binding.rglru_proj_params()
    q.D_model = Dm
    q.lin_x_w, q.lin_x_b = base, base + 0x100000
    q.lin_y_w, q.lin_y_b = base + 0x200000, base + 0x300000
    q.lin_out_w, q.lin_out_b = base + 0x400000, base + 0x500000
    return q


def _block(lib, p, q, B=2, T=100, x=X, out=OUT, h0=H0, hl=HL, c0=C0, cl=CL, ws=WSP, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = lib.rglru_block_prefill_workspace_bytes(B, T, p.D, p.n_heads, q.D_model, p.dtype)
    return lib.rglru_block_prefill(ctypes.byref(p), ctypes.byref(q), B, T, x, out, h0, hl, c0, cl,
                                   ws, ws_bytes, None)


def test_block_workspace_bytes(lib):
    f = lib.rglru_block_prefill_workspace_bytes
    pw = lib.rglru_prefill_workspace_bytes(8, 8192, 2560, 10, 1)
    assert f(8, 8192, 2560, 10, 2560, 1) == ((pw + 255) // 256) * 256 + 3 * 8 * 8192 * 2560 * 2
    assert f(8, 8192, 2560, 10, 0, 1) == 0
    assert f(0, 8192, 2560, 10, 2560, 1) == 0


def test_block_validation(lib):
    p, q = _params(), _proj()
    assert lib.rglru_block_prefill(ctypes.byref(p), None, 2, 10, X, OUT, H0, HL, C0, CL, WSP,
                                   1 << 30, None) == NULL
    assert _block(lib, _params(dtype=0), q) == UNSUP          # bf16 only
    assert _block(lib, _params(D=384, H=3), q) == UNSUP       # D % 256 (bs = 128 is fine)
    assert _block(lib, p, _proj(Dm=300)) == UNSUP             # D_model % 256
    assert _block(lib, p, _proj(Dm=0)) == SHAPE
    assert _block(lib, p, q, B=0) == SHAPE
    assert _block(lib, p, q, x=None) == NULL
    r = _proj()
    r.lin_out_w = None
    assert _block(lib, p, r) == NULL
    assert _block(lib, p, q, x=X + 2) == UNSUP
    assert _block(lib, p, q, ws=None) == WS
    assert _block(lib, p, q, ws_bytes=4096) == WS
    assert _block(lib, p, q, out=X + 64) == ALIAS
    assert _block(lib, p, q, out=H0) == ALIAS
    assert _block(lib, p, q, ws=X) == ALIAS
    assert _block(lib, p, q, ws=q.lin_y_w - 4096) == ALIAS
    # the path's own checks run before anything is launched
    assert _block(lib, p, q, hl=H0 + 16) == ALIAS
    assert _block(lib, p, q, c0=C0 + 2) == UNSUP
    big = _params(D=4096, H=16)
    far = [k << 40 for k in range(1, 8)]   # buffers of several GiB that do not overlap
    kw = dict(x=far[0], out=far[1], h0=far[2], hl=far[3], c0=far[4], cl=far[5], ws=far[6])
    assert _block(lib, big, _proj(), B=1, T=262144, **kw) == UNSUP   # one bf16 branch of 2 GiB


# ------------------------------------------------------------------------------------------
# local attention
# ------------------------------------------------------------------------------------------
AQ, AK, AV, AO, AW = (0x100000000 * k for k in range(1, 6))


def _attn(lib, B=2, T=300, Hq=4, window=64, base=10000.0, q=AQ, k=AK, v=AV, o=AO, ws=AW,
          ws_bytes=None, kc=None, vc=None):
    if ws_bytes is None:
        ws_bytes = lib.rglru_local_attention_workspace_bytes(B, T, Hq)
    return lib.rglru_local_attention(B, T, Hq, window, base, q, k, v, o, kc, vc, ws, ws_bytes,
                                     None)


def test_attention_workspace_bytes(lib):
    f = lib.rglru_local_attention_workspace_bytes
    # q, k after RoPE, then v regrouped in fours of keys (padded to a multiple of 4 tokens)
    assert f(2, 300, 4) == 2 * 300 * 4 * 512 + 2 * 300 * 512 + 2 * 75 * 2048
    assert f(1, 5, 1) == 5 * 512 + 5 * 512 + 2 * 2048
    assert f(1, 0, 3) == 0
    assert f(0, 5, 1) == 0 and f(1, -1, 1) == 0 and f(1, 5, 0) == 0


def test_attention_validation(lib):
    # every call here fails validation (or has T = 0), so nothing is launched
    assert _attn(lib, B=0) == SHAPE
    assert _attn(lib, T=-1) == SHAPE
    assert _attn(lib, Hq=0) == SHAPE and _attn(lib, Hq=65) == SHAPE
    assert _attn(lib, window=0) == SHAPE
    assert _attn(lib, base=1.0) == SHAPE and _attn(lib, base=float("nan")) == SHAPE
    assert _attn(lib, base=float("inf")) == SHAPE
    assert _attn(lib, T=1 << 22) == UNSUP                       # one sequence's k past 2 GiB
    assert _attn(lib, B=1 << 12, T=1 << 12) == UNSUP            # too many token rows per launch
    assert _attn(lib, q=None) == NULL and _attn(lib, o=None) == NULL
    assert _attn(lib, T=0, q=None, k=None, v=None, o=None, ws=None, ws_bytes=0) == OK
    assert _attn(lib, k=AK + 8) == UNSUP
    assert _attn(lib, ws=None) == WS
    assert _attn(lib, ws_bytes=lib.rglru_local_attention_workspace_bytes(2, 300, 4) - 1) == WS
    assert _attn(lib, o=AQ + 512) == ALIAS                       # o overlaps q
    assert _attn(lib, v=AO + 2 * 300 * 4 * 512 - 16) == ALIAS    # v's start inside o
    assert _attn(lib, ws=AV + 1024) == ALIAS                     # workspace overlaps v
    KC, VC = 0x700000000, 0x780000000
    assert _attn(lib, kc=KC) == NULL                             # one cache without the other
    assert _attn(lib, kc=KC + 8, vc=VC) == UNSUP
    assert _attn(lib, kc=AV, vc=VC) == ALIAS                     # a cache overlaps v
    assert _attn(lib, kc=KC, vc=KC + 4096) == ALIAS              # the caches overlap
    assert _attn(lib, window=1 << 22, kc=KC, vc=VC) == UNSUP


def test_attention_cache_and_decode_sizes(lib):
    # per sequence: ceil(window / 32) tiles of 32 slots x 256 dims, bf16
    assert lib.rglru_local_attention_cache_bytes(3, 2048) == 3 * 2048 * 512
    assert lib.rglru_local_attention_cache_bytes(1, 33) == 64 * 512
    assert lib.rglru_local_attention_cache_bytes(0, 64) == 0
    assert lib.rglru_local_attention_cache_bytes(1, 0) == 0
    f = lib.rglru_local_attention_decode_workspace_bytes
    # q after RoPE, then per split and head: max, normaliser and 256 outputs (fp32); a split is
    # 512 cache slots for N >= 64, 256 for 16 <= N < 64 and 128 below; the size is the largest
    # over batches up to N (so a buffer for N fits any smaller batch)
    def per(n, Hq=10, W=2048):
        slots = 512 if n >= 64 else (256 if n >= 16 else 128)
        return (n * Hq * 512 + 255) // 256 * 256 + n * (-(-W // slots)) * Hq * 258 * 4
    upto = lambda n: max(per(n), per(min(n, 15)), per(min(n, 63)))
    assert f(256, 10, 2048) == 256 * 10 * 512 + 256 * 4 * 10 * 258 * 4 == upto(256)
    assert f(64, 10, 2048) == 63 * 10 * 512 + 63 * 8 * 10 * 258 * 4 == upto(64)
    assert f(16, 10, 2048) == 15 * 10 * 512 + 15 * 16 * 10 * 258 * 4 == upto(16)
    assert f(1, 10, 2048) == 10 * 512 + 16 * 10 * 258 * 4
    assert f(1, 1, 1) == 512 + 258 * 4
    assert f(0, 1, 64) == 0 and f(1, 0, 64) == 0


DP, DQ, DK, DV, DKC, DVC, DO, DW = (0x1000000000 + k * 0x10000000 for k in range(8))


def _dec(lib, N=4, Hq=10, window=2048, base=10000.0, pos=DP, q=DQ, k=DK, v=DV, kc=DKC, vc=DVC,
         o=DO, ws=DW, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = lib.rglru_local_attention_decode_workspace_bytes(N, Hq, window)
    return lib.rglru_local_attention_decode(N, Hq, window, base, pos, q, k, v, kc, vc, o, ws,
                                            ws_bytes, None)


def test_attention_decode_validation(lib):
    # every call here fails validation, so nothing is launched
    assert _dec(lib, N=0) == SHAPE
    assert _dec(lib, Hq=0) == SHAPE and _dec(lib, Hq=17) == SHAPE
    assert _dec(lib, window=0) == SHAPE and _dec(lib, base=0.5) == SHAPE
    assert _dec(lib, window=1 << 22) == UNSUP
    assert _dec(lib, N=1 << 22, window=2048, ws_bytes=1 << 40) == UNSUP   # grid too large
    for name in ("pos", "q", "k", "v", "kc", "vc", "o"):
        assert _dec(lib, **{name: None}) == NULL, name
    assert _dec(lib, pos=DP + 4) == UNSUP
    assert _dec(lib, ws=None) == WS
    assert _dec(lib, ws_bytes=lib.rglru_local_attention_decode_workspace_bytes(4, 10, 2048) - 4) == WS
    assert _dec(lib, o=DQ) == ALIAS                  # output over q
    assert _dec(lib, kc=DV) == ALIAS                 # cache over v
    assert _dec(lib, vc=DKC + 4096) == ALIAS         # the caches overlap
    assert _dec(lib, ws=DO) == ALIAS                 # workspace over the output
    assert _dec(lib, pos=DKC) == ALIAS               # positions inside a cache


def _attn_params(Dm=512, Hq=2, dh=256, window=64, base=10000.0, b=True):
    a = binding.rglru_attn_params()
    a.D_model, a.n_heads, a.head_dim, a.window, a.rope_base = Dm, Hq, dh, window, base
    a.q_w, a.k_w, a.v_w, a.o_w = (0x200000000 + k * 0x1000000 for k in range(4))
    a.o_b = 0x200000000 + 4 * 0x1000000 if b else None
    return a


def _attn_block(lib, a, B=2, T=100, x=AQ, out=AO, ws=AW, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = lib.rglru_local_attention_block_workspace_bytes(ctypes.byref(a), B, T)
    return lib.rglru_local_attention_block(ctypes.byref(a), B, T, x, out, ws, ws_bytes, None)


def test_attention_block_workspace_bytes(lib):
    a = _attn_params(Hq=3)
    f = lib.rglru_local_attention_block_workspace_bytes
    core = lib.rglru_local_attention_workspace_bytes(2, 100, 3)
    # q and the attention output [M][Hq][256], k and v [M][256], then the attention's workspace
    assert f(ctypes.byref(a), 2, 100) == 2 * (200 * 3 * 512) + 2 * (200 * 512) + core
    assert f(None, 2, 100) == 0 and f(ctypes.byref(a), 0, 100) == 0


def test_attention_block_validation(lib):
    # every call here fails validation (or has T = 0), so nothing is launched
    assert lib.rglru_local_attention_block(None, 1, 1, AQ, AO, AW, 1 << 30, None) == NULL
    assert _attn_block(lib, _attn_params(dh=128)) == UNSUP
    assert _attn_block(lib, _attn_params(Dm=384)) == UNSUP
    assert _attn_block(lib, _attn_params(Hq=0)) == SHAPE
    assert _attn_block(lib, _attn_params(window=0)) == SHAPE
    assert _attn_block(lib, _attn_params(), B=0) == SHAPE
    a = _attn_params()
    a.k_w = None
    assert _attn_block(lib, a) == NULL
    a = _attn_params()
    a.o_b = a.o_b + 4
    assert _attn_block(lib, a) == UNSUP
    assert _attn_block(lib, _attn_params(), x=None) == NULL
    assert _attn_block(lib, _attn_params(), T=0, x=None, out=None, ws=None, ws_bytes=0) == OK
    assert _attn_block(lib, _attn_params(), ws=None) == WS
    assert _attn_block(lib, _attn_params(), out=AQ + 1024) == ALIAS     # out overlaps x_in
    a = _attn_params()
    assert _attn_block(lib, a, out=a.o_w) == ALIAS                      # out overlaps o_w
    assert _attn_block(lib, a, ws=a.q_w) == ALIAS                       # workspace overlaps q_w


# ------------------------------------------------------------------------------------------
# the residual layer (every call fails validation or has no rows, so nothing is launched)
# ------------------------------------------------------------------------------------------
NX, NR, NS, NH, NO = (0x2000000000 + k * 0x100000000 for k in range(5))


def test_rmsnorm_validation(lib):
    f = lib.rglru_rmsnorm
    assert f(-1, 2560, NX, None, NS, 1e-6, None, NO, None) == SHAPE
    assert f(10, 2560, NX, None, NS, -1.0, None, NO, None) == SHAPE
    assert f(10, 2564, NX, None, NS, 1e-6, None, NO, None) == UNSUP      # D % 8
    assert f(10, 8200, NX, None, NS, 1e-6, None, NO, None) == UNSUP      # D > 8192
    assert f(10, 2560, None, None, NS, 1e-6, None, NO, None) == NULL
    assert f(10, 2560, NX, None, NS, 1e-6, None, None, None) == NULL     # nothing to write
    assert f(10, 2560, NX, None, None, 1e-6, None, NO, None) == NULL     # norm without scale
    assert f(10, 2560, NX + 8, None, NS, 1e-6, None, NO, None) == UNSUP
    assert f(10, 2560, NX, None, NS, 1e-6, None, NX + 512, None) == ALIAS
    assert f(10, 2560, NX, NR, NS, 1e-6, NR, NO, None) == ALIAS          # h over the residual
    assert f(10, 2560, NX, NR, NS, 1e-6, NH, NH + 1024, None) == ALIAS   # out over h
    assert f(0, 2560, None, None, None, 1e-6, None, None, None) == OK


def _mlp(Dm=512, F=768, b=True):
    m = binding.rglru_mlp_params()
    m.D_model, m.F = Dm, F
    m.gate_w, m.up_w, m.down_w = (0x3000000000 + k * 0x10000000 for k in range(3))
    if b:
        m.gate_b, m.up_b, m.down_b = (0x3000000000 + k * 0x10000000 for k in range(3, 6))
    return m


def test_mlp_workspace_and_validation(lib):
    assert lib.rglru_mlp_workspace_bytes(300, 768) == 2 * 300 * 768 * 2
    assert lib.rglru_mlp_workspace_bytes(1, 256) == 2 * 512
    assert lib.rglru_mlp_workspace_bytes(-1, 256) == 0 and lib.rglru_mlp_workspace_bytes(5, 0) == 0
    ws = lib.rglru_mlp_workspace_bytes(300, 768)
    f = lambda m, M=300, x=NX, o=NO, w=NH, n=ws: lib.rglru_mlp(ctypes.byref(m), M, x, o, w, n, None)
    assert lib.rglru_mlp(None, 1, NX, NO, NH, ws, None) == NULL
    assert f(_mlp(Dm=384)) == UNSUP and f(_mlp(F=700)) == UNSUP
    m = _mlp()
    m.up_w = None
    assert f(m) == NULL
    assert f(_mlp(), M=-1) == SHAPE
    assert f(_mlp(), x=None) == NULL
    assert f(_mlp(), n=ws - 1) == WS
    assert f(_mlp(), o=NX + 256) == ALIAS                    # out over x
    assert f(_mlp(), w=0x3000000000) == ALIAS                # workspace over gate_w
    assert f(_mlp(), M=0, x=None, o=None, w=None, n=0) == OK


def _norms(eps=1e-6):
    n = binding.rglru_norm_params()
    n.temporal_scale, n.channel_scale, n.eps = 0x3800000000, 0x3800010000, eps
    return n


def test_layer_workspace_bytes(lib):
    B, T, D, H, Dm, F = 2, 100, 512, 2, 512, 768
    act = 2 * 100 * 512 * 2
    bw = lib.rglru_block_prefill_workspace_bytes(B, T, D, H, Dm, 1)
    r256 = lambda v: (v + 255) // 256 * 256
    assert lib.rglru_recurrent_layer_workspace_bytes(B, T, D, H, Dm, F) == \
        r256(bw) + 3 * r256(act) + lib.rglru_mlp_workspace_bytes(B * T, F)
    a = _attn_params(Dm=512, Hq=2)
    aw = lib.rglru_local_attention_block_workspace_bytes(ctypes.byref(a), B, T)
    assert lib.rglru_attention_layer_workspace_bytes(ctypes.byref(a), B, T, F) == \
        r256(aw) + 3 * r256(act) + lib.rglru_mlp_workspace_bytes(B * T, F)
    assert lib.rglru_recurrent_layer_workspace_bytes(B, T, D, H, Dm, 0) == 0


def test_layer_validation(lib):
    p = _params(D=512, H=2, dtype=1)
    q = _proj(Dm=512)
    a = _attn_params(Dm=512, Hq=2)
    m, n = _mlp(Dm=512), _norms()
    B, T = 2, 100
    ws = lib.rglru_attention_layer_workspace_bytes(ctypes.byref(a), B, T, 768)
    fa = lambda a=a, n=n, m=m, T=T, x=NX, o=NO, w=0x4000000000, nb=ws: \
        lib.rglru_attention_layer_prefill(ctypes.byref(a), n if n is None else ctypes.byref(n),
                                          ctypes.byref(m), B, T, x, o, None, None, w, nb, None)
    assert fa(n=None) == NULL
    assert fa(n=_norms(eps=-1.0)) == SHAPE
    assert fa(m=_mlp(Dm=768)) == SHAPE                        # MLP width != D_model
    assert fa(m=_mlp(Dm=512, F=700)) == UNSUP
    assert fa(x=None) == NULL
    assert fa(nb=ws - 1) == WS
    assert fa(o=NX + 1024) == ALIAS                           # out over x_in
    assert fa(w=0x3000000000) == ALIAS                        # workspace over the MLP weights
    assert fa(a=_attn_params(Dm=512, Hq=2, dh=128)) == UNSUP  # the block's own checks
    assert fa(T=0, x=None, o=None, w=None, nb=0) == OK
    if q is not None:
        wr = lib.rglru_recurrent_layer_workspace_bytes(B, T, 512, 2, 512, 768)
        fr = lambda n=n, x=NX, o=NO, nb=wr: lib.rglru_recurrent_layer_prefill(
            ctypes.byref(p), ctypes.byref(q), ctypes.byref(n), ctypes.byref(m), B, T, x, o,
            None, None, None, None, 0x4000000000, nb, None)
        assert fr(n=_norms(eps=float("nan"))) == SHAPE
        assert fr(nb=wr - 1) == WS
        assert fr(o=NX) == ALIAS


def test_layer_decode_validation(lib):
    p, q, m, n = _params(D=512, H=2, dtype=1), _proj(Dm=512), _mlp(Dm=512), _norms()
    N = 4
    wr = lib.rglru_recurrent_layer_decode_workspace_bytes(N, 512, 512, 768)
    r256 = lambda v: (v + 255) // 256 * 256
    base = r256(3 * r256(N * 512 * 2) + r256(lib.rglru_decode_workspace_bytes(N, 512, 1))) \
        + 3 * r256(N * 512 * 2) + lib.rglru_mlp_workspace_bytes(N, 768)
    # plus fp32 partial sums for the projections' split K (none at four rows or fewer, which take
    # the row kernel): at most 4 splits of K = 512 for the widest GEMM (gate|up, 1536 columns)
    # over N rows
    assert base <= wr <= base + r256(4 * N * 1536 * 4) and (wr - base) % 256 == 0
    fr = lambda n=n, x=NX, o=NO, hh=NH, c=NR, nb=wr: lib.rglru_recurrent_layer_decode(
        ctypes.byref(p), ctypes.byref(q), n if n is None else ctypes.byref(n), ctypes.byref(m),
        N, x, o, hh, c, 0x4000000000, nb, None)
    assert fr(n=None) == NULL
    assert fr(hh=None) == NULL
    assert fr(nb=wr - 1) == WS
    assert fr(o=NX) == ALIAS
    assert fr(c=0x3000000000) == ALIAS                       # conv state over gate_w
    a = _attn_params(Dm=512, Hq=2, window=64)
    wa = lib.rglru_attention_layer_decode_workspace_bytes(ctypes.byref(a), N, 768)
    assert wa > 0 and lib.rglru_attention_layer_decode_workspace_bytes(ctypes.byref(a), 0, 768) == 0
    fa = lambda a=a, pos=DP, o=NO, kc=DKC, vc=DVC, nb=wa: lib.rglru_attention_layer_decode(
        ctypes.byref(a), ctypes.byref(n), ctypes.byref(m), N, pos, NX, o, kc, vc, 0x4000000000,
        nb, None)
    assert fa(pos=None) == NULL
    assert fa(a=_attn_params(Dm=512, Hq=17)) == SHAPE           # decode takes 16 heads at most
    assert fa(nb=wa - 1) == WS
    assert fa(o=DKC) == ALIAS                                   # out over the key cache


def test_backward_workspace_and_validation(lib):
    f = lib.rglru_prefill_backward_workspace_bytes
    assert f(2, 128, 512, 2) > 0 and f(8, 8192, 2560, 10) > 0
    assert f(2, 100, 512, 2) == 0                      # T % 32
    assert f(1, 96, 512, 2) == 0                       # B * T % 256
    assert f(2, 128, 512, 4) == 0                      # block size 128
    p = _params(D=512, H=2, dtype=1)
    base = 0x5000000000
    ptr = [base + k * 0x10000000 for k in range(20)]
    ws = f(2, 128, 512, 2)

    def call(p=p, B=2, T=128, x=ptr[0], y=ptr[1], dout=ptr[2], outs=None, w=ptr[19], n=ws):
        o = outs or ptr[4:15]
        return lib.rglru_prefill_backward(ctypes.byref(p), B, T, x, y, None, None, dout, None, *o,
                                          w, n, None)
    assert call(T=100) == UNSUP
    assert call(p=_params(D=512, H=2, dtype=0)) == UNSUP   # fp32 storage
    assert call(x=None) == NULL
    assert call(outs=ptr[4:14] + [None]) == NULL
    assert call(n=ws - 1) == WS
    assert call(outs=ptr[4:14] + [ptr[0]]) == ALIAS        # dconv0 over x
    assert call(outs=[ptr[4]] + [ptr[4] + 0x100] + ptr[6:15]) == ALIAS   # dx and dy overlap
    assert call(w=ptr[1]) == ALIAS                          # workspace over y


def _noalloc(lib, p, B, T, base=1 << 36, step=1 << 36, **kw):
    ptr = {k: base + i * step for i, k in enumerate(("x", "y", "out", "h0", "hl", "c0", "cl"))}
    ptr.update(kw)
    return lib.rglru_prefill_noalloc(ctypes.byref(p), B, T, ptr["x"], ptr["y"], ptr["out"],
                                     ptr["h0"], ptr["hl"], ptr["c0"], ptr["cl"], None)


def test_prefill_noalloc_validation(lib):
    """The allocation-free prefill checks everything rglru_prefill checks, and rejects calls
    whose look-back state exceeds its static scratch, before any HIP call."""
    assert binding.PREFILL_NOALLOC_MAX_BYTES == 64 << 20
    p = _params()
    assert lib.rglru_prefill_noalloc(None, 1, 1, X, Y, OUT, None, None, None, None, None) == NULL
    assert _noalloc(lib, p, 0, 100) == SHAPE
    assert _noalloc(lib, p, 2, -1) == SHAPE
    assert _noalloc(lib, p, 2, 100, x=None) == NULL
    assert _noalloc(lib, p, 2, 100, x=(1 << 36) + 2) == UNSUP
    assert _noalloc(lib, p, 2, 100, out=(1 << 36) + 64) == ALIAS
    assert _noalloc(lib, _params(D=512, H=8), 2, 100) == UNSUP
    big = _params(D=4096, H=16)
    f = lib.rglru_prefill_workspace_bytes
    # the 9B long-context shape fits (1023 segments publish words) ...
    assert f(2, 65536, 4096, 16, 1) <= binding.PREFILL_NOALLOC_MAX_BYTES
    # ... one more segment does not, and is refused before anything is launched
    assert f(2, 65537, 4096, 16, 1) > binding.PREFILL_NOALLOC_MAX_BYTES
    assert _noalloc(lib, big, 2, 65537) == WS
    assert _noalloc(lib, big, 3, 65536) == WS


def test_decode_workspace_sizes_fit_smaller_batches(lib):
    """A decode workspace sized for N sequences also fits every smaller batch: the sizes never
    decrease with N, although the attention's window splits and the projections' K splits
    change with the batch."""
    fa = lib.rglru_local_attention_decode_workspace_bytes
    a = _attn_params(Dm=2560, Hq=10, window=2048)
    fl = lambda n: lib.rglru_attention_layer_decode_workspace_bytes(ctypes.byref(a), n, 7680)
    fr = lambda n: lib.rglru_recurrent_layer_decode_workspace_bytes(n, 2560, 2560, 7680)
    for f in (lambda n: fa(n, 10, 2048), lambda n: fa(n, 4, 100), fl, fr):
        sizes = [f(n) for n in list(range(1, 300)) + [511, 512, 513, 1000, 1024, 1025, 4096]]
        assert all(b >= a_ for a_, b in zip(sizes, sizes[1:])), sizes
    # the batches that used to shrink it: 63 -> 64 and 15 -> 16 sequences
    assert fa(64, 10, 2048) >= fa(63, 10, 2048) and fa(16, 10, 2048) >= fa(15, 10, 2048)
