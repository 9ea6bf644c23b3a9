"""fp64 CPU oracle for the RG-LRU recurrent-block path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The HIP library never calls it, and it
shares no code with the HIP library: the arithmetic lives in
``rglru_oracle.c`` (plain C, fp64, sequential per (sequence, head) unit);
this module only compiles that file with gcc and marshals numpy arrays.

Storage conventions (the same as the library's inputs):
  * fp32 tensors are ``numpy.float32`` arrays;
  * bf16 tensors are ``numpy.uint16`` arrays holding the raw bf16 bits;
  * Lambda and h0 are always ``numpy.float32``.
Outputs are ``numpy.float64``.

What each function follows is stated in the C file's header; every function
is pinned in ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "rglru_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

F32 = 0
BF16 = 1
F64 = 2   # fp64 intermediates (inputs of a block inside a residual layer)


def build(src: str = _SRC, out: str = _LIB) -> str:
    """Compile the oracle with gcc (-O2, OpenMP).  Returns the library path."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-D_DEFAULT_SOURCE",
           src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _needs_build() -> bool:
    if not os.path.exists(_LIB):
        return True
    return os.path.getmtime(_LIB) < os.path.getmtime(_SRC)


def load(path: str | None = None):
    """Load (building first if needed) and return the ctypes library."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    with _lock:
        if _lib is None:
            if _needs_build():
                build()
            _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def _bind(lib):
    P = ctypes.c_void_p
    I = ctypes.c_int
    lib.oracle_prefill_unit.argtypes = [I, I, I, I, I, I, I] + [P] * 14
    lib.oracle_prefill_unit.restype = I
    lib.oracle_prefill.argtypes = [I, I, I, I, I] + [P] * 14 + [I]
    lib.oracle_prefill.restype = I
    lib.oracle_decode_step.argtypes = [I, I, I, I] + [P] * 12
    lib.oracle_decode_step.restype = I
    lib.oracle_conv1d_state_update.argtypes = [I, I, I, I] + [P] * 5
    lib.oracle_conv1d_state_update.restype = I
    lib.oracle_gate_preacts.argtypes = [I, I, I, I] + [P] * 7
    lib.oracle_gate_preacts.restype = I
    lib.oracle_gelu_tanh.argtypes = [ctypes.c_double]
    lib.oracle_gelu_tanh.restype = ctypes.c_double
    lib.oracle_rglru_step.argtypes = [ctypes.c_double] * 5
    lib.oracle_rglru_step.restype = ctypes.c_double
    lib.oracle_linear.argtypes = [I, I, I, I] + [P] * 4
    lib.oracle_linear.restype = I
    lib.oracle_block_prefill.argtypes = [I, I, I, I, I, I, I] + [P] * 19 + [I]
    lib.oracle_block_prefill.restype = I
    D_ = ctypes.c_double
    lib.oracle_rope.argtypes = [I, I, P, D_, P]
    lib.oracle_rope.restype = I
    lib.oracle_local_mqa.argtypes = [I, I, I, I, P, P, P, P]
    lib.oracle_local_mqa.restype = I
    lib.oracle_local_attention_block.argtypes = [I, I, I, I, I, I, I, I, D_] + [P] * 7 + [I]
    lib.oracle_local_attention_block.restype = I
    lib.oracle_prefill_backward.argtypes = [I, I, I, I, I] + [P] * 24
    lib.oracle_prefill_backward.restype = I
    lib.oracle_rmsnorm.argtypes = [I, I, I, I, P, P, D_, P]
    lib.oracle_rmsnorm.restype = I
    lib.oracle_mlp.argtypes = [I, I, I, I, I] + [P] * 8 + [I]
    lib.oracle_mlp.restype = I
    lib.oracle_max_threads.argtypes = []
    lib.oracle_max_threads.restype = I
    return lib


def _dtype_code(arr: np.ndarray) -> int:
    if arr.dtype == np.float32:
        return F32
    if arr.dtype == np.uint16:
        return BF16
    raise TypeError("storage arrays must be float32 or uint16 (bf16 bits), got %s" % arr.dtype)


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype=None):
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if dtype is not None and a.dtype != dtype:
        raise TypeError("expected %s, got %s" % (dtype, a.dtype))
    return a


class Params:
    """The block's parameters in storage form (see module docstring)."""

    def __init__(self, conv_w, conv_b, wa, ba, wx, bx, lam, n_heads):
        self.conv_w = _c(conv_w)
        self.dtype = _dtype_code(self.conv_w)
        sd = self.conv_w.dtype
        self.conv_b = _c(conv_b, sd)
        self.wa = _c(wa, sd)
        self.ba = _c(ba, sd)
        self.wx = _c(wx, sd)
        self.bx = _c(bx, sd)
        self.lam = _c(lam, np.float32)
        self.H = int(n_heads)
        self.D = int(self.lam.shape[0])

    def args(self):
        return [_ptr(self.conv_w), _ptr(self.conv_b), _ptr(self.wa), _ptr(self.ba),
                _ptr(self.wx), _ptr(self.bx), _ptr(self.lam)]


def _check(st, what):
    if st != 0:
        raise ValueError("%s: oracle status %d" % (what, st))


def prefill(p: Params, x, y, h0=None, conv0=None, nthreads: int = 0, lib=None):
    """Full prefill.  x, y [B, T, D].  Returns (out [B,T,D], h_last [B,D], conv_last [B,3,D])."""
    lib = lib or load()
    x = _c(x, p.conv_w.dtype)
    y = _c(y, p.conv_w.dtype)
    B, T, D = x.shape
    h0 = _c(h0, np.float32)
    conv0 = _c(conv0, p.conv_w.dtype)
    out = np.empty((B, T, D), np.float64)
    h_last = np.empty((B, D), np.float64)
    conv_last = np.empty((B, 3, D), np.float64)
    cw, cb, wa, ba, wx, bx, lam = p.args()
    st = lib.oracle_prefill(p.dtype, B, T, D, p.H, _ptr(x), _ptr(y), cw, cb, wa, ba, wx, bx, lam,
                            _ptr(h0), _ptr(conv0), _ptr(out), _ptr(h_last), _ptr(conv_last),
                            int(nthreads))
    _check(st, "oracle_prefill")
    return out, h_last, conv_last


def prefill_unit(p: Params, x, y, b: int, hd: int, t_use: int, h0=None, conv0=None, lib=None):
    """One (b, head) unit over the first t_use tokens.

    Returns (out [t_use, bs], h_end [bs], conv_end [3, bs]) for channels
    hd*bs .. hd*bs+bs-1.
    """
    lib = lib or load()
    x = _c(x, p.conv_w.dtype)
    y = _c(y, p.conv_w.dtype)
    B, T, D = x.shape
    bs = D // p.H
    out = np.empty((t_use, bs), np.float64)
    h_end = np.empty((bs,), np.float64)
    conv_end = np.empty((3, bs), np.float64)
    h0 = _c(h0, np.float32)
    conv0 = _c(conv0, p.conv_w.dtype)
    cw, cb, wa, ba, wx, bx, lam = p.args()
    st = lib.oracle_prefill_unit(p.dtype, T, D, p.H, int(b), int(hd), int(t_use), _ptr(x),
                                 _ptr(y), cw, cb, wa, ba, wx, bx, lam, _ptr(h0), _ptr(conv0),
                                 _ptr(out), _ptr(h_end), _ptr(conv_end))
    _check(st, "oracle_prefill_unit")
    return out, h_end, conv_end


def decode_step(p: Params, x_t, y_t, h, win, lib=None):
    """One decode step.  x_t, y_t [N, D] (storage); h [N, D] and win [N, 3, D] fp64, updated in place.

    Returns out_t [N, D] (fp64)."""
    lib = lib or load()
    x_t = _c(x_t, p.conv_w.dtype)
    y_t = _c(y_t, p.conv_w.dtype)
    N, D = x_t.shape
    assert h.dtype == np.float64 and h.flags.c_contiguous and h.shape == (N, D)
    assert win.dtype == np.float64 and win.flags.c_contiguous and win.shape == (N, 3, D)
    out = np.empty((N, D), np.float64)
    cw, cb, wa, ba, wx, bx, lam = p.args()
    st = lib.oracle_decode_step(p.dtype, N, D, p.H, _ptr(x_t), _ptr(y_t), cw, cb, wa, ba, wx, bx,
                                lam, _ptr(h), _ptr(win), _ptr(out))
    _check(st, "oracle_decode_step")
    return out


def conv1d_state_update(conv_w, conv_b, x_new, win, want_out=True, lib=None):
    """x_new [N, T_new, D] (storage); win [N, 3, D] fp64 updated in place.

    Returns conv_out [N, T_new, D] fp64 (or None)."""
    lib = lib or load()
    conv_w = _c(conv_w)
    dt = _dtype_code(conv_w)
    x_new = _c(x_new, conv_w.dtype)
    conv_b = _c(conv_b, conv_w.dtype)
    N, T_new, D = x_new.shape
    assert win.dtype == np.float64 and win.flags.c_contiguous and win.shape == (N, 3, D)
    out = np.empty((N, T_new, D), np.float64) if want_out else None
    st = lib.oracle_conv1d_state_update(dt, N, T_new, D, _ptr(x_new), _ptr(conv_w), _ptr(conv_b),
                                        _ptr(win), _ptr(out))
    _check(st, "oracle_conv1d_state_update")
    return out


def gate_preacts(wa, ba, wx, bx, u, n_heads: int, lib=None):
    """Gate pre-activations.  u [n, D] fp64 -> (ra, ri) [n, D] fp64."""
    lib = lib or load()
    wa = _c(wa)
    dt = _dtype_code(wa)
    wx = _c(wx, wa.dtype)
    ba = _c(ba, wa.dtype)
    bx = _c(bx, wa.dtype)
    u = _c(u, np.float64)
    n, D = u.shape
    ra = np.empty((n, D), np.float64)
    ri = np.empty((n, D), np.float64)
    st = lib.oracle_gate_preacts(dt, n, D, int(n_heads), _ptr(u), _ptr(wa), _ptr(ba), _ptr(wx),
                                 _ptr(bx), _ptr(ra), _ptr(ri))
    _check(st, "oracle_gate_preacts")
    return ra, ri


class ProjParams:
    """The block's dense projections in storage form: Linear weights [out][in], biases or None.

    lx_w, ly_w [D, Dm] (linear_x, linear_y); lo_w [Dm, D] (linear_out)."""

    def __init__(self, lx_w, lx_b, ly_w, ly_b, lo_w, lo_b):
        self.lx_w = _c(lx_w)
        sd = self.lx_w.dtype
        self.lx_b = _c(lx_b, sd)
        self.ly_w = _c(ly_w, sd)
        self.ly_b = _c(ly_b, sd)
        self.lo_w = _c(lo_w, sd)
        self.lo_b = _c(lo_b, sd)
        self.D, self.Dm = self.lx_w.shape

    def args(self):
        return [_ptr(self.lx_w), _ptr(self.lx_b), _ptr(self.ly_w), _ptr(self.ly_b),
                _ptr(self.lo_w), _ptr(self.lo_b)]


def linear(x, w, b=None, lib=None):
    """One Linear layer: x [M, K] (storage), w [N, K], b [N] or None -> [M, N] fp64."""
    lib = lib or load()
    x = _c(x)
    dt = _dtype_code(x)
    w = _c(w, x.dtype)
    b = _c(b, x.dtype)
    M, K = x.shape
    N = w.shape[0]
    assert w.shape == (N, K)
    out = np.empty((M, N), np.float64)
    _check(lib.oracle_linear(dt, M, K, N, _ptr(x), _ptr(w), _ptr(b), _ptr(out)), "oracle_linear")
    return out


def block_prefill(p: Params, q: ProjParams, x_in, h0=None, conv0=None, nthreads: int = 0, lib=None):
    """The recurrent block with its projections: x_in [B, T, Dm] (storage, or fp64 as inside a
    residual layer).

    Returns (out [B,T,Dm], h_last [B,D], conv_last [B,3,D]), all fp64."""
    lib = lib or load()
    x_in = _c(x_in)
    if x_in.dtype != np.float64:
        _c(x_in, p.conv_w.dtype)
    xdt = F64 if x_in.dtype == np.float64 else p.dtype
    B, T, Dm = x_in.shape
    assert q.Dm == Dm and q.D == p.D
    h0 = _c(h0, np.float32)
    conv0 = _c(conv0, p.conv_w.dtype)
    out = np.empty((B, T, Dm), np.float64)
    h_last = np.empty((B, p.D), np.float64)
    conv_last = np.empty((B, 3, p.D), np.float64)
    st = lib.oracle_block_prefill(p.dtype, xdt, B, T, Dm, p.D, p.H, _ptr(x_in), *q.args(),
                                  *p.args(),
                                  _ptr(h0), _ptr(conv0), _ptr(out), _ptr(h_last), _ptr(conv_last),
                                  int(nthreads))
    _check(st, "oracle_block_prefill")
    return out, h_last, conv_last


def prefill_backward(p: Params, x, y, dout, h0=None, conv0=None, dh_last=None, lib=None) -> dict:
    """Gradients of L = sum(dout * out) + sum(dh_last * h_last) for the path over x, y
    [B, T, D] (storage), dout [B, T, D] and dh_last [B, D] (fp64 or None).  Returns a dict of
    fp64 arrays: dx, dy, dconv_w [D,4], dconv_b, dwa, dwx [H,bs,bs], dba, dbx, dlambda [D],
    dh0 [B,D], dconv0 [B,3,D]."""
    lib = lib or load()
    x = _c(x, p.conv_w.dtype)
    y = _c(y, p.conv_w.dtype)
    B, T, D = x.shape
    h0 = _c(h0, np.float32)
    conv0 = _c(conv0, p.conv_w.dtype)
    dout = _c(np.asarray(dout, np.float64), np.float64)
    dh_last = _c(np.asarray(dh_last, np.float64), np.float64) if dh_last is not None else None
    bs = D // p.H
    g = {"dx": np.empty((B, T, D)), "dy": np.empty((B, T, D)), "dconv_w": np.empty((D, 4)),
         "dconv_b": np.empty(D), "dwa": np.empty((p.H, bs, bs)), "dba": np.empty(D),
         "dwx": np.empty((p.H, bs, bs)), "dbx": np.empty(D), "dlambda": np.empty(D),
         "dh0": np.empty((B, D)), "dconv0": np.empty((B, 3, D))}
    cw, cb, wa, ba, wx, bx, lam = p.args()
    st = lib.oracle_prefill_backward(p.dtype, B, T, D, p.H, _ptr(x), _ptr(y), cw, cb, wa, ba, wx,
                                     bx, lam, _ptr(h0), _ptr(conv0), _ptr(dout), _ptr(dh_last),
                                     *[_ptr(g[k]) for k in ("dx", "dy", "dconv_w", "dconv_b",
                                                            "dwa", "dba", "dwx", "dbx", "dlambda",
                                                            "dh0", "dconv0")])
    _check(st, "oracle_prefill_backward")
    return g


def rope(v, pos, base: float = 10000.0, lib=None):
    """Rotary position embedding of head vectors v [n, dh] (fp64) at positions pos [n]."""
    lib = lib or load()
    v = np.array(v, np.float64, copy=True, order="C")
    n, dh = v.shape
    pos = _c(np.asarray(pos, np.float64), np.float64)
    _check(lib.oracle_rope(n, dh, _ptr(pos), float(base), _ptr(v)), "oracle_rope")
    return v


def local_mqa(q, k, v, window: int, lib=None):
    """Sliding-window MQA over one sequence: q [T, Hq, dh], k, v [T, dh] (fp64, positions
    already encoded) -> o [T, Hq, dh]."""
    lib = lib or load()
    q = _c(np.asarray(q, np.float64), np.float64)
    k = _c(np.asarray(k, np.float64), np.float64)
    v = _c(np.asarray(v, np.float64), np.float64)
    T, Hq, dh = q.shape
    assert k.shape == (T, dh) and v.shape == (T, dh)
    o = np.empty((T, Hq, dh), np.float64)
    _check(lib.oracle_local_mqa(T, Hq, dh, int(window), _ptr(q), _ptr(k), _ptr(v), _ptr(o)),
           "oracle_local_mqa")
    return o


def local_attention_block(x_in, wq, wk, wv, wo, bo, n_heads: int, window: int,
                          base: float = 10000.0, nthreads: int = 0, lib=None):
    """The local-attention block: x_in [B, T, Dm] (storage, or fp64 as inside a residual layer)
    -> out [B, T, Dm] (fp64).
    wq [Hq*dh, Dm], wk, wv [dh, Dm], wo [Dm, Hq*dh] (storage, [out][in]), bo [Dm] or None."""
    lib = lib or load()
    x_in = _c(x_in)
    wq = _c(wq)
    dt = _dtype_code(wq)
    xdt = F64 if x_in.dtype == np.float64 else _dtype_code(x_in)
    if xdt != F64 and xdt != dt:
        raise TypeError("x_in must be fp64 or the weights' storage type")
    wk, wv, wo = (_c(a, wq.dtype) for a in (wk, wv, wo))
    bo = _c(bo, wq.dtype)
    B, T, Dm = x_in.shape
    dh = wk.shape[0]
    assert wq.shape == (n_heads * dh, Dm) and wv.shape == (dh, Dm) and wo.shape == (Dm, n_heads * dh)
    out = np.empty((B, T, Dm), np.float64)
    st = lib.oracle_local_attention_block(dt, xdt, B, T, Dm, int(n_heads), dh, int(window),
                                          float(base),
                                          _ptr(x_in), _ptr(wq), _ptr(wk), _ptr(wv), _ptr(wo),
                                          _ptr(bo), _ptr(out), int(nthreads))
    _check(st, "oracle_local_attention_block")
    return out


def rmsnorm(x, g, eps: float = 1e-6, lib=None):
    """RMSNorm over the last axis: x [..., D] (storage or fp64), g [D] (storage) -> fp64."""
    lib = lib or load()
    x = _c(x)
    g = _c(g)
    D = x.shape[-1]
    assert g.shape == (D,)
    rows = x.size // D if D else 0
    xdt = F64 if x.dtype == np.float64 else _dtype_code(x)
    out = np.empty(x.shape, np.float64)
    _check(lib.oracle_rmsnorm(xdt, _dtype_code(g), rows, D, _ptr(x), _ptr(g), float(eps),
                              _ptr(out)), "oracle_rmsnorm")
    return out


class MlpParams:
    """The gated MLP in storage form: gate_w, up_w [F, Dm], down_w [Dm, F] ([out][in]); biases
    [F], [F], [Dm] or None."""

    def __init__(self, gate_w, gate_b, up_w, up_b, down_w, down_b):
        self.gate_w = _c(gate_w)
        sd = self.gate_w.dtype
        self.gate_b, self.up_w, self.up_b = _c(gate_b, sd), _c(up_w, sd), _c(up_b, sd)
        self.down_w, self.down_b = _c(down_w, sd), _c(down_b, sd)
        self.F, self.Dm = self.gate_w.shape
        assert self.up_w.shape == (self.F, self.Dm) and self.down_w.shape == (self.Dm, self.F)

    def args(self):
        return [_ptr(a) for a in (self.gate_w, self.gate_b, self.up_w, self.up_b, self.down_w,
                                  self.down_b)]


def mlp(m: MlpParams, x, nthreads: int = 0, lib=None):
    """The gated MLP: x [..., Dm] (storage or fp64) -> down(gelu_tanh(gate(x)) * up(x)), fp64."""
    lib = lib or load()
    x = _c(x)
    assert x.shape[-1] == m.Dm
    rows = x.size // m.Dm
    xdt = F64 if x.dtype == np.float64 else _dtype_code(x)
    out = np.empty(x.shape, np.float64)
    _check(lib.oracle_mlp(xdt, _dtype_code(m.gate_w), rows, m.Dm, m.F, _ptr(x), *m.args(),
                          _ptr(out), int(nthreads)), "oracle_mlp")
    return out


def residual_layer(x_in, temporal, g1, g2, m: MlpParams, eps: float = 1e-6, lib=None):
    """One residual layer of the model (pre-norm, two residual additions):
        h = x + temporal(RMSNorm_1(x)),   out = h + MLP(RMSNorm_2(h))
    x_in [B, T, Dm] (storage); temporal maps an fp64 [B, T, Dm] array to fp64 [B, T, Dm] (the
    recurrent block or the local-attention block); g1, g2 [Dm] (storage).  Returns
    (out, h) in fp64."""
    x = widen_bf16(x_in).astype(np.float64) if np.asarray(x_in).dtype == np.uint16 \
        else np.asarray(x_in, np.float64)
    h = x + temporal(rmsnorm(x_in, g1, eps, lib=lib))
    return h + mlp(m, rmsnorm(h, g2, eps, lib=lib), lib=lib), h


def gelu_tanh(yv: float, lib=None) -> float:
    lib = lib or load()
    return lib.oracle_gelu_tanh(float(yv))


def rglru_step(lam: float, ra: float, ri: float, u: float, h_prev: float, lib=None) -> float:
    lib = lib or load()
    return lib.oracle_rglru_step(float(lam), float(ra), float(ri), float(u), float(h_prev))


def max_threads(lib=None) -> int:
    lib = lib or load()
    return lib.oracle_max_threads()


def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bits to float32 (the oracle's own converter, in numpy)."""
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)
