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
    assert lib.rglru_abi_version() == 2
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
    assert f(8, 8192, 2560, 10, 1) == 4096 + 128 * 8 * 2560 * 8
    assert f(1, 1, 256, 2, 0) == 4096 + 1 * 1 * 256 * 8
    assert f(1, 0, 256, 2, 0) == 4096 + 256 * 8
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
