"""ctypes binding of librglru.so (argument marshalling only).

Every step of the path runs in the library's HIP kernels; this module checks
tensor dtype/device/contiguity/shape, passes ``data_ptr()`` values and
``torch.cuda.current_stream().cuda_stream``, and raises on a non-zero status.
PyTorch supplies device memory and streams, nothing else.

There is no fallback: if librglru.so is missing or fails to load, every call
raises ``RuntimeError``.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "librglru.so")

RGLRU_F32 = 0
RGLRU_BF16 = 1
STATUS = {0: "RGLRU_OK", 1: "RGLRU_ERR_NULL", 2: "RGLRU_ERR_SHAPE", 3: "RGLRU_ERR_UNSUPPORTED",
          4: "RGLRU_ERR_WORKSPACE", 5: "RGLRU_ERR_ALIAS", 6: "RGLRU_ERR_HIP"}
EXPORTS = ["rglru_prefill_workspace_bytes", "rglru_prefill_workspace_init", "rglru_prefill",
           "rglru_decode_workspace_bytes", "rglru_decode_step", "conv1d_state_update",
           "rglru_prefill_workspace_flags", "rglru_status_string", "rglru_last_hip_error",
           "rglru_abi_version", "rglru_linear", "rglru_block_prefill_workspace_bytes",
           "rglru_block_prefill", "rglru_local_attention_workspace_bytes", "rglru_local_attention",
           "rglru_local_attention_block_workspace_bytes", "rglru_local_attention_block",
           "rglru_local_attention_cache_bytes", "rglru_local_attention_decode_workspace_bytes",
           "rglru_local_attention_decode", "rglru_rmsnorm", "rglru_mlp_workspace_bytes",
           "rglru_mlp", "rglru_recurrent_layer_workspace_bytes", "rglru_recurrent_layer_prefill",
           "rglru_attention_layer_workspace_bytes", "rglru_attention_layer_prefill",
           "rglru_recurrent_layer_decode_workspace_bytes", "rglru_recurrent_layer_decode",
           "rglru_attention_layer_decode_workspace_bytes", "rglru_attention_layer_decode",
           "rglru_prefill_backward_workspace_bytes", "rglru_prefill_backward",
           "rglru_prefill_noalloc"]
PREFILL_NOALLOC_MAX_BYTES = 64 << 20  # RGLRU_PREFILL_NOALLOC_MAX_BYTES

_lock = threading.Lock()
_lib = None


class RglruError(RuntimeError):
    def __init__(self, status: int, where: str, hip_error: int = 0):
        msg = "%s failed: %s" % (where, STATUS.get(status, status))
        if status == 6:
            msg += " (hipError %d)" % hip_error
        super().__init__(msg)
        self.status = status


class rglru_params(ctypes.Structure):
    _fields_ = [("D", ctypes.c_int32), ("n_heads", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("conv_w", ctypes.c_void_p), ("conv_b", ctypes.c_void_p),
                ("gate_a_w", ctypes.c_void_p), ("gate_a_b", ctypes.c_void_p),
                ("gate_x_w", ctypes.c_void_p), ("gate_x_b", ctypes.c_void_p),
                ("lambda_", ctypes.c_void_p)]


class rglru_proj_params(ctypes.Structure):
    _fields_ = [("D_model", ctypes.c_int32),
                ("lin_x_w", ctypes.c_void_p), ("lin_x_b", ctypes.c_void_p),
                ("lin_y_w", ctypes.c_void_p), ("lin_y_b", ctypes.c_void_p),
                ("lin_out_w", ctypes.c_void_p), ("lin_out_b", ctypes.c_void_p)]


class rglru_attn_params(ctypes.Structure):
    _fields_ = [("D_model", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("window", ctypes.c_int32),
                ("rope_base", ctypes.c_float),
                ("q_w", ctypes.c_void_p), ("k_w", ctypes.c_void_p), ("v_w", ctypes.c_void_p),
                ("o_w", ctypes.c_void_p), ("o_b", ctypes.c_void_p)]


class rglru_norm_params(ctypes.Structure):
    _fields_ = [("temporal_scale", ctypes.c_void_p), ("channel_scale", ctypes.c_void_p),
                ("eps", ctypes.c_float)]


class rglru_mlp_params(ctypes.Structure):
    _fields_ = [("D_model", ctypes.c_int32), ("F", ctypes.c_int32),
                ("gate_w", ctypes.c_void_p), ("gate_b", ctypes.c_void_p),
                ("up_w", ctypes.c_void_p), ("up_b", ctypes.c_void_p),
                ("down_w", ctypes.c_void_p), ("down_b", ctypes.c_void_p)]


def load_library(path: str = LIB_PATH):
    """Load librglru.so (no build, no fallback)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise RuntimeError("librglru.so not found at %s: build it with "
                               "`python -c 'import __graft_entry__ as g; g.build()'`" % path)
        lib = ctypes.CDLL(path)
        P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        PP = ctypes.POINTER(rglru_params)
        lib.rglru_prefill_workspace_bytes.argtypes = [I32, I32, I32, I32, I32]
        lib.rglru_prefill_workspace_bytes.restype = SZ
        lib.rglru_prefill_workspace_init.argtypes = [P, SZ, P]
        lib.rglru_prefill_workspace_init.restype = ctypes.c_int
        lib.rglru_prefill.argtypes = [PP, I32, I32, P, P, P, P, P, P, P, P, SZ, P]
        lib.rglru_prefill.restype = ctypes.c_int
        lib.rglru_prefill_noalloc.argtypes = [PP, I32, I32, P, P, P, P, P, P, P, P]
        lib.rglru_prefill_noalloc.restype = ctypes.c_int
        lib.rglru_decode_workspace_bytes.argtypes = [I32, I32, I32]
        lib.rglru_decode_workspace_bytes.restype = SZ
        lib.rglru_decode_step.argtypes = [PP, I32, P, I64, P, I64, P, I64, P, P, P, SZ, P]
        lib.rglru_decode_step.restype = ctypes.c_int
        lib.conv1d_state_update.argtypes = [PP, I32, I32, P, P, P, P]
        lib.conv1d_state_update.restype = ctypes.c_int
        lib.rglru_prefill_workspace_flags.argtypes = [P, SZ, ctypes.POINTER(ctypes.c_uint32), P]
        lib.rglru_prefill_workspace_flags.restype = ctypes.c_int
        lib.rglru_status_string.argtypes = [ctypes.c_int]
        lib.rglru_status_string.restype = ctypes.c_char_p
        lib.rglru_last_hip_error.argtypes = []
        lib.rglru_last_hip_error.restype = ctypes.c_int
        lib.rglru_linear.argtypes = [I32, I32, I32, P, P, P, P, P]
        lib.rglru_linear.restype = ctypes.c_int
        lib.rglru_block_prefill_workspace_bytes.argtypes = [I32, I32, I32, I32, I32, I32]
        lib.rglru_block_prefill_workspace_bytes.restype = SZ
        lib.rglru_block_prefill.argtypes = [PP, ctypes.POINTER(rglru_proj_params), I32, I32, P, P,
                                            P, P, P, P, P, SZ, P]
        lib.rglru_block_prefill.restype = ctypes.c_int
        lib.rglru_local_attention_workspace_bytes.argtypes = [I32, I32, I32]
        lib.rglru_local_attention_workspace_bytes.restype = SZ
        lib.rglru_local_attention.argtypes = [I32, I32, I32, I32, ctypes.c_float, P, P, P, P, P,
                                              P, P, SZ, P]
        lib.rglru_local_attention_cache_bytes.argtypes = [I32, I32]
        lib.rglru_local_attention_cache_bytes.restype = SZ
        lib.rglru_local_attention_decode_workspace_bytes.argtypes = [I32, I32, I32]
        lib.rglru_local_attention_decode_workspace_bytes.restype = SZ
        lib.rglru_local_attention_decode.argtypes = [I32, I32, I32, ctypes.c_float, P, P, P, P, P,
                                                     P, P, P, SZ, P]
        lib.rglru_local_attention_decode.restype = ctypes.c_int
        lib.rglru_local_attention.restype = ctypes.c_int
        AP = ctypes.POINTER(rglru_attn_params)
        lib.rglru_local_attention_block_workspace_bytes.argtypes = [AP, I32, I32]
        lib.rglru_local_attention_block_workspace_bytes.restype = SZ
        lib.rglru_local_attention_block.argtypes = [AP, I32, I32, P, P, P, SZ, P]
        lib.rglru_local_attention_block.restype = ctypes.c_int
        NP, MP = ctypes.POINTER(rglru_norm_params), ctypes.POINTER(rglru_mlp_params)
        lib.rglru_rmsnorm.argtypes = [I32, I32, P, P, P, ctypes.c_float, P, P, P]
        lib.rglru_rmsnorm.restype = ctypes.c_int
        lib.rglru_mlp_workspace_bytes.argtypes = [I32, I32]
        lib.rglru_mlp_workspace_bytes.restype = SZ
        lib.rglru_mlp.argtypes = [MP, I32, P, P, P, SZ, P]
        lib.rglru_mlp.restype = ctypes.c_int
        lib.rglru_recurrent_layer_workspace_bytes.argtypes = [I32, I32, I32, I32, I32, I32]
        lib.rglru_recurrent_layer_workspace_bytes.restype = SZ
        lib.rglru_recurrent_layer_prefill.argtypes = [PP, ctypes.POINTER(rglru_proj_params), NP, MP,
                                                      I32, I32, P, P, P, P, P, P, P, SZ, P]
        lib.rglru_recurrent_layer_prefill.restype = ctypes.c_int
        lib.rglru_attention_layer_workspace_bytes.argtypes = [AP, I32, I32, I32]
        lib.rglru_attention_layer_workspace_bytes.restype = SZ
        lib.rglru_attention_layer_prefill.argtypes = [AP, NP, MP, I32, I32, P, P, P, P, P, SZ, P]
        lib.rglru_attention_layer_prefill.restype = ctypes.c_int
        lib.rglru_recurrent_layer_decode_workspace_bytes.argtypes = [I32, I32, I32, I32]
        lib.rglru_recurrent_layer_decode_workspace_bytes.restype = SZ
        lib.rglru_recurrent_layer_decode.argtypes = [PP, ctypes.POINTER(rglru_proj_params), NP, MP,
                                                     I32, P, P, P, P, P, SZ, P]
        lib.rglru_recurrent_layer_decode.restype = ctypes.c_int
        lib.rglru_attention_layer_decode_workspace_bytes.argtypes = [AP, I32, I32]
        lib.rglru_attention_layer_decode_workspace_bytes.restype = SZ
        lib.rglru_attention_layer_decode.argtypes = [AP, NP, MP, I32, P, P, P, P, P, P, SZ, P]
        lib.rglru_attention_layer_decode.restype = ctypes.c_int
        lib.rglru_prefill_backward_workspace_bytes.argtypes = [I32, I32, I32, I32]
        lib.rglru_prefill_backward_workspace_bytes.restype = SZ
        lib.rglru_prefill_backward.argtypes = [PP, I32, I32] + [P] * 18 + [SZ, P]
        lib.rglru_prefill_backward.restype = ctypes.c_int
        lib.rglru_abi_version.argtypes = []
        lib.rglru_abi_version.restype = ctypes.c_int
        _lib = lib
        return lib


def _check(lib, st: int, where: str):
    if st != 0:
        raise RglruError(st, where, lib.rglru_last_hip_error() if st == 6 else 0)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(dt) -> int:
    if dt == torch.bfloat16:
        return RGLRU_BF16
    if dt == torch.float32:
        return RGLRU_F32
    raise TypeError("storage dtype must be torch.bfloat16 or torch.float32, got %s" % dt)


def _need(t, name, dtype, shape=None, device=None):
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s: expected %s, got %s" % (name, dtype, t.dtype))
    if device is not None and t.device != device:
        raise ValueError("%s: expected device %s, got %s" % (name, device, t.device))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s: expected shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


class Params:
    """Block parameters on one device (storage dtype bf16 or fp32; Lambda fp32).

    conv_w [D, 4]; conv_b [D] or None; gate_a_w, gate_x_w [H, bs, bs] stored like Linear
    weights ([out, in]); gate_a_b, gate_x_b [D] or None; lam [D] fp32.
    """

    def __init__(self, conv_w, conv_b, gate_a_w, gate_a_b, gate_x_w, gate_x_b, lam):
        self.dtype = conv_w.dtype
        self.code = _dtype_code(self.dtype)
        self.device = conv_w.device
        D = conv_w.shape[0]
        H = gate_a_w.shape[0]
        bs = gate_a_w.shape[1]
        _need(conv_w, "conv_w", self.dtype, (D, 4), self.device)
        _need(conv_b, "conv_b", self.dtype, (D,), self.device)
        _need(gate_a_w, "gate_a_w", self.dtype, (H, bs, bs), self.device)
        _need(gate_x_w, "gate_x_w", self.dtype, (H, bs, bs), self.device)
        _need(gate_a_b, "gate_a_b", self.dtype, (D,), self.device)
        _need(gate_x_b, "gate_x_b", self.dtype, (D,), self.device)
        _need(lam, "lam", torch.float32, (D,), self.device)
        if H * bs != D:
            raise ValueError("gate blocks %d x %d do not tile D=%d" % (H, bs, D))
        self.D, self.H, self.bs = D, H, bs
        self.tensors = (conv_w, conv_b, gate_a_w, gate_a_b, gate_x_w, gate_x_b, lam)
        self.c = rglru_params(D, H, self.code, *[t.data_ptr() if t is not None else None
                                                 for t in self.tensors])


def rglru_prefill_workspace_bytes(B: int, T: int, D: int, n_heads: int, dtype) -> int:
    lib = load_library()
    return int(lib.rglru_prefill_workspace_bytes(B, T, D, n_heads, _dtype_code(dtype)))


def rglru_prefill_workspace_init(ws: torch.Tensor):
    lib = load_library()
    _check(lib, lib.rglru_prefill_workspace_init(_ptr(ws), ws.numel(), _stream()),
           "rglru_prefill_workspace_init")


class Workspace:
    """A reusable prefill workspace (uint8 device tensor; the library prepares it at each call,
    so its contents never matter)."""

    def __init__(self, nbytes: int, device):
        self.t = torch.empty(max(int(nbytes), 4096), dtype=torch.uint8, device=device)

    @property
    def nbytes(self) -> int:
        return self.t.numel()

    def flags(self) -> int:
        lib = load_library()
        v = ctypes.c_uint32(0)
        _check(lib, lib.rglru_prefill_workspace_flags(_ptr(self.t), self.t.numel(),
                                                      ctypes.byref(v), _stream()),
               "rglru_prefill_workspace_flags")
        return int(v.value)


def make_workspace(p: Params, B: int, T: int) -> Workspace:
    return Workspace(rglru_prefill_workspace_bytes(B, T, p.D, p.H, p.dtype), p.device)


def rglru_prefill(p: Params, x, y, h0=None, conv0=None, *, out=None, h_last=None, conv_last=None,
                  workspace: Workspace | None = None, want_state: bool = True):
    """out = prefill(x, y); returns (out, h_last, conv_last) (state tensors None if not wanted)."""
    lib = load_library()
    B, T, D = x.shape
    _need(x, "x", p.dtype, (B, T, p.D), p.device)
    _need(y, "y", p.dtype, (B, T, p.D), p.device)
    _need(h0, "h0", torch.float32, (B, D), p.device)
    _need(conv0, "conv0", p.dtype, (B, 3, D), p.device)
    if out is None:
        out = torch.empty_like(x)
    _need(out, "out", p.dtype, (B, T, D), p.device)
    if want_state:
        if h_last is None:
            h_last = torch.empty((B, D), dtype=torch.float32, device=p.device)
        if conv_last is None:
            conv_last = torch.empty((B, 3, D), dtype=p.dtype, device=p.device)
    _need(h_last, "h_last", torch.float32, (B, D), p.device)
    _need(conv_last, "conv_last", p.dtype, (B, 3, D), p.device)
    if workspace is None:
        workspace = make_workspace(p, B, T)
    st = lib.rglru_prefill(ctypes.byref(p.c), B, T, _ptr(x), _ptr(y), _ptr(out), _ptr(h0),
                           _ptr(h_last), _ptr(conv0), _ptr(conv_last), _ptr(workspace.t),
                           workspace.nbytes, _stream())
    _check(lib, st, "rglru_prefill")
    return out, h_last, conv_last


def rglru_prefill_noalloc(p: Params, x, y, h0=None, conv0=None, *, out=None, h_last=None,
                          conv_last=None, want_state: bool = True):
    """rglru_prefill without a workspace: the library's static scratch holds the look-back
    state (no device allocation by the library; outputs are allocated here when not given)."""
    lib = load_library()
    B, T, D = x.shape
    _need(x, "x", p.dtype, (B, T, p.D), p.device)
    _need(y, "y", p.dtype, (B, T, p.D), p.device)
    _need(h0, "h0", torch.float32, (B, D), p.device)
    _need(conv0, "conv0", p.dtype, (B, 3, D), p.device)
    if out is None:
        out = torch.empty_like(x)
    _need(out, "out", p.dtype, (B, T, D), p.device)
    if want_state:
        if h_last is None:
            h_last = torch.empty((B, D), dtype=torch.float32, device=p.device)
        if conv_last is None:
            conv_last = torch.empty((B, 3, D), dtype=p.dtype, device=p.device)
    _need(h_last, "h_last", torch.float32, (B, D), p.device)
    _need(conv_last, "conv_last", p.dtype, (B, 3, D), p.device)
    st = lib.rglru_prefill_noalloc(ctypes.byref(p.c), B, T, _ptr(x), _ptr(y), _ptr(out),
                                   _ptr(h0), _ptr(h_last), _ptr(conv0), _ptr(conv_last), _stream())
    _check(lib, st, "rglru_prefill_noalloc")
    return out, h_last, conv_last


def rglru_decode_workspace_bytes(N: int, D: int, dtype) -> int:
    lib = load_library()
    return int(lib.rglru_decode_workspace_bytes(N, D, _dtype_code(dtype)))


def make_decode_workspace(p: Params, N: int):
    """Device buffer for the split decode step (uint8; needs no initialisation)."""
    return torch.empty(max(rglru_decode_workspace_bytes(N, p.D, p.dtype), 16), dtype=torch.uint8,
                       device=p.device)


def rglru_decode_step(p: Params, x_t, y_t, h, conv_state, out_t=None, workspace=None):
    """One token for N sequences.  x_t, y_t [N, D] (rows may be strided, e.g. x[:, t]);
    h [N, D] fp32 and conv_state [N, 3, D] are updated in place.  Returns out_t [N, D].
    workspace: None (fused kernel) or a buffer from make_decode_workspace (split step)."""
    lib = load_library()
    N, D = x_t.shape
    for t, name in ((x_t, "x_t"), (y_t, "y_t")):
        if t.dtype != p.dtype or t.device != p.device or t.shape != (N, p.D) or t.stride(1) != 1:
            raise ValueError("%s must be [N, D] %s rows with unit channel stride" % (name, p.dtype))
    _need(h, "h", torch.float32, (N, D), p.device)
    _need(conv_state, "conv_state", p.dtype, (N, 3, D), p.device)
    if out_t is None:
        out_t = torch.empty((N, D), dtype=p.dtype, device=p.device)
    if out_t.shape != (N, D) or out_t.stride(1) != 1 or out_t.dtype != p.dtype:
        raise ValueError("out_t must be [N, D] rows with unit channel stride")
    if workspace is not None and (workspace.device != p.device or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous buffer on %s" % p.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.rglru_decode_step(ctypes.byref(p.c), N, _ptr(x_t), x_t.stride(0), _ptr(y_t),
                               y_t.stride(0), _ptr(out_t), out_t.stride(0), _ptr(h),
                               _ptr(conv_state), _ptr(workspace), ws_bytes, _stream())
    _check(lib, st, "rglru_decode_step")
    return out_t


def conv1d_state_update(p: Params, x_new, conv_state, want_out: bool = True, out=None):
    """x_new [N, T_new, D]; conv_state [N, 3, D] updated in place.  Returns conv_out (written
    into `out` when given) or None when want_out is False."""
    lib = load_library()
    N, T_new, D = x_new.shape
    _need(x_new, "x_new", p.dtype, (N, T_new, p.D), p.device)
    _need(conv_state, "conv_state", p.dtype, (N, 3, D), p.device)
    if out is not None:
        _need(out, "out", p.dtype, (N, T_new, D), p.device)
    elif want_out:
        out = torch.empty_like(x_new)
    st = lib.conv1d_state_update(ctypes.byref(p.c), N, T_new, _ptr(x_new), _ptr(conv_state),
                                 _ptr(out), _stream())
    _check(lib, st, "conv1d_state_update")
    return out


def rglru_linear(x, w, b=None, out=None):
    """One Linear layer (bf16): out [M, N] = x [M, K] @ w [N, K]^T + b [N]."""
    lib = load_library()
    M, K = x.shape
    N = w.shape[0]
    _need(x, "x", torch.bfloat16, (M, K))
    _need(w, "w", torch.bfloat16, (N, K), x.device)
    _need(b, "b", torch.bfloat16, (N,), x.device)
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _need(out, "out", torch.bfloat16, (M, N), x.device)
    _check(lib, lib.rglru_linear(M, K, N, _ptr(x), _ptr(w), _ptr(b), _ptr(out), _stream()),
           "rglru_linear")
    return out


class ProjParams:
    """The block's dense projections on one device (bf16, Linear weights [out, in]).

    lin_x_w, lin_y_w [D, D_model]; lin_out_w [D_model, D]; biases [D], [D], [D_model] or None.
    """

    def __init__(self, lin_x_w, lin_x_b, lin_y_w, lin_y_b, lin_out_w, lin_out_b):
        D, Dm = lin_x_w.shape
        dev = lin_x_w.device
        _need(lin_x_w, "lin_x_w", torch.bfloat16, (D, Dm), dev)
        _need(lin_y_w, "lin_y_w", torch.bfloat16, (D, Dm), dev)
        _need(lin_out_w, "lin_out_w", torch.bfloat16, (Dm, D), dev)
        _need(lin_x_b, "lin_x_b", torch.bfloat16, (D,), dev)
        _need(lin_y_b, "lin_y_b", torch.bfloat16, (D,), dev)
        _need(lin_out_b, "lin_out_b", torch.bfloat16, (Dm,), dev)
        self.D, self.Dm, self.device = D, Dm, dev
        self.tensors = (lin_x_w, lin_x_b, lin_y_w, lin_y_b, lin_out_w, lin_out_b)
        self.c = rglru_proj_params(Dm, *[t.data_ptr() if t is not None else None
                                         for t in self.tensors])


def rglru_block_prefill_workspace_bytes(B: int, T: int, D: int, n_heads: int, D_model: int,
                                        dtype) -> int:
    lib = load_library()
    return int(lib.rglru_block_prefill_workspace_bytes(B, T, D, n_heads, D_model,
                                                       _dtype_code(dtype)))


def make_block_workspace(p: Params, q: ProjParams, B: int, T: int) -> Workspace:
    return Workspace(rglru_block_prefill_workspace_bytes(B, T, p.D, p.H, q.Dm, p.dtype), p.device)


def rglru_block_prefill(p: Params, q: ProjParams, x_in, h0=None, conv0=None, *, out=None,
                        h_last=None, conv_last=None, workspace: Workspace | None = None,
                        want_state: bool = True):
    """The whole temporal-mixing block: out [B, T, D_model] = linear_out(path(linear_x(x_in),
    linear_y(x_in))).  Returns (out, h_last, conv_last)."""
    lib = load_library()
    B, T, Dm = x_in.shape
    D = p.D
    if q.D != D or q.Dm != Dm:
        raise ValueError("projection shapes (%d, %d) do not match D=%d, D_model=%d"
                         % (q.D, q.Dm, D, Dm))
    _need(x_in, "x_in", p.dtype, (B, T, Dm), p.device)
    _need(h0, "h0", torch.float32, (B, D), p.device)
    _need(conv0, "conv0", p.dtype, (B, 3, D), p.device)
    if out is None:
        out = torch.empty_like(x_in)
    _need(out, "out", p.dtype, (B, T, Dm), p.device)
    if want_state:
        if h_last is None:
            h_last = torch.empty((B, D), dtype=torch.float32, device=p.device)
        if conv_last is None:
            conv_last = torch.empty((B, 3, D), dtype=p.dtype, device=p.device)
    _need(h_last, "h_last", torch.float32, (B, D), p.device)
    _need(conv_last, "conv_last", p.dtype, (B, 3, D), p.device)
    if workspace is None:
        workspace = make_block_workspace(p, q, B, T)
    st = lib.rglru_block_prefill(ctypes.byref(p.c), ctypes.byref(q.c), B, T, _ptr(x_in), _ptr(out),
                                 _ptr(h0), _ptr(h_last), _ptr(conv0), _ptr(conv_last),
                                 _ptr(workspace.t), workspace.nbytes, _stream())
    _check(lib, st, "rglru_block_prefill")
    return out, h_last, conv_last


# ------------------------------------------------------------------------------------------
# local sliding-window multi-query attention
# ------------------------------------------------------------------------------------------
ATTN_HEAD_DIM = 256


class DeviceBuffer:
    """Scratch device memory for one call (uint8 tensor); needs no initialisation."""

    def __init__(self, nbytes: int, device):
        self.t = torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)

    @property
    def nbytes(self) -> int:
        return self.t.numel()


def rglru_local_attention_workspace_bytes(B: int, T: int, n_heads: int) -> int:
    return int(load_library().rglru_local_attention_workspace_bytes(B, T, n_heads))


class AttnCache:
    """The ring KV cache of the local attention for N sequences (two device buffers in the
    library's tile layout; slot t % window holds position t)."""

    def __init__(self, N: int, window: int, device):
        nbytes = int(load_library().rglru_local_attention_cache_bytes(N, window))
        if nbytes == 0:
            raise ValueError("invalid cache shape N=%d window=%d" % (N, window))
        self.N, self.window = N, window
        self.k = torch.empty(nbytes // 2, dtype=torch.bfloat16, device=device)
        self.v = torch.empty(nbytes // 2, dtype=torch.bfloat16, device=device)


def rglru_local_attention(q, k, v, window: int, rope_base: float = 10000.0, *, out=None,
                          cache: AttnCache | None = None, workspace: DeviceBuffer | None = None):
    """Sliding-window MQA with RoPE (bf16): q [B, T, Hq, 256], k, v [B, T, 256] (before RoPE)
    -> o [B, T, Hq, 256].  With a cache, the last `window` positions are written into it."""
    lib = load_library()
    B, T, Hq, dh = q.shape
    dev = q.device
    _need(q, "q", torch.bfloat16, (B, T, Hq, ATTN_HEAD_DIM))
    _need(k, "k", torch.bfloat16, (B, T, ATTN_HEAD_DIM), dev)
    _need(v, "v", torch.bfloat16, (B, T, ATTN_HEAD_DIM), dev)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.bfloat16, (B, T, Hq, ATTN_HEAD_DIM), dev)
    if workspace is None:
        workspace = DeviceBuffer(rglru_local_attention_workspace_bytes(B, T, Hq), dev)
    if cache is not None and (cache.N != B or cache.window != window):
        raise ValueError("cache is for N=%d window=%d" % (cache.N, cache.window))
    kc = _ptr(cache.k) if cache is not None else None
    vc = _ptr(cache.v) if cache is not None else None
    st = lib.rglru_local_attention(B, T, Hq, int(window), float(rope_base), _ptr(q), _ptr(k),
                                   _ptr(v), _ptr(out), kc, vc, _ptr(workspace.t), workspace.nbytes,
                                   _stream())
    _check(lib, st, "rglru_local_attention")
    return out


def rglru_local_attention_decode_workspace_bytes(N: int, n_heads: int, window: int) -> int:
    return int(load_library().rglru_local_attention_decode_workspace_bytes(N, n_heads, window))


def rglru_local_attention_decode(pos, q, k, v, cache: AttnCache, rope_base: float = 10000.0, *,
                                 out=None, workspace: DeviceBuffer | None = None):
    """One decode step: pos [N] int32 (device), q [N, Hq, 256], k, v [N, 256] (before RoPE);
    writes position pos[n] into the cache and returns o [N, Hq, 256]."""
    lib = load_library()
    N, Hq, _ = q.shape
    dev = q.device
    _need(pos, "pos", torch.int32, (N,), dev)
    _need(q, "q", torch.bfloat16, (N, Hq, ATTN_HEAD_DIM))
    _need(k, "k", torch.bfloat16, (N, ATTN_HEAD_DIM), dev)
    _need(v, "v", torch.bfloat16, (N, ATTN_HEAD_DIM), dev)
    if cache.N != N:
        raise ValueError("cache is for N=%d, got %d sequences" % (cache.N, N))
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.bfloat16, (N, Hq, ATTN_HEAD_DIM), dev)
    if workspace is None:
        workspace = DeviceBuffer(rglru_local_attention_decode_workspace_bytes(N, Hq, cache.window),
                                 dev)
    st = lib.rglru_local_attention_decode(N, Hq, cache.window, float(rope_base), _ptr(pos),
                                          _ptr(q), _ptr(k), _ptr(v), _ptr(cache.k), _ptr(cache.v),
                                          _ptr(out), _ptr(workspace.t), workspace.nbytes,
                                          _stream())
    _check(lib, st, "rglru_local_attention_decode")
    return out


class AttnParams:
    """The local-attention block's weights on one device (bf16, Linear weights [out, in]).

    q_w [n_heads * 256, D_model]; k_w, v_w [256, D_model]; o_w [D_model, n_heads * 256];
    o_b [D_model] or None.
    """

    def __init__(self, q_w, k_w, v_w, o_w, o_b, n_heads: int, window: int,
                 rope_base: float = 10000.0):
        HD, Dm = q_w.shape
        dev = q_w.device
        if HD != n_heads * ATTN_HEAD_DIM:
            raise ValueError("q_w has %d rows, expected n_heads * 256 = %d"
                             % (HD, n_heads * ATTN_HEAD_DIM))
        _need(q_w, "q_w", torch.bfloat16, (HD, Dm), dev)
        _need(k_w, "k_w", torch.bfloat16, (ATTN_HEAD_DIM, Dm), dev)
        _need(v_w, "v_w", torch.bfloat16, (ATTN_HEAD_DIM, Dm), dev)
        _need(o_w, "o_w", torch.bfloat16, (Dm, HD), dev)
        _need(o_b, "o_b", torch.bfloat16, (Dm,), dev)
        self.Dm, self.H, self.window, self.device = Dm, n_heads, window, dev
        self.tensors = (q_w, k_w, v_w, o_w, o_b)
        self.c = rglru_attn_params(Dm, n_heads, ATTN_HEAD_DIM, int(window), float(rope_base),
                                   *[t.data_ptr() if t is not None else None
                                     for t in self.tensors])


def rglru_local_attention_block_workspace_bytes(a: AttnParams, B: int, T: int) -> int:
    return int(load_library().rglru_local_attention_block_workspace_bytes(ctypes.byref(a.c), B, T))


def rglru_local_attention_block(a: AttnParams, x_in, *, out=None,
                                workspace: DeviceBuffer | None = None):
    """The whole local-attention block: out [B, T, D_model] = o_proj(attention(q_proj(x_in),
    k_proj(x_in), v_proj(x_in)))."""
    lib = load_library()
    B, T, Dm = x_in.shape
    if Dm != a.Dm:
        raise ValueError("x_in width %d does not match D_model=%d" % (Dm, a.Dm))
    _need(x_in, "x_in", torch.bfloat16, (B, T, Dm), a.device)
    if out is None:
        out = torch.empty_like(x_in)
    _need(out, "out", torch.bfloat16, (B, T, Dm), a.device)
    if workspace is None:
        workspace = DeviceBuffer(rglru_local_attention_block_workspace_bytes(a, B, T), a.device)
    st = lib.rglru_local_attention_block(ctypes.byref(a.c), B, T, _ptr(x_in), _ptr(out),
                                         _ptr(workspace.t), workspace.nbytes, _stream())
    _check(lib, st, "rglru_local_attention_block")
    return out


# ------------------------------------------------------------------------------------------
# the residual layer
# ------------------------------------------------------------------------------------------
class NormParams:
    """The layer's two RMSNorm scales ([D_model] bf16 each) and eps."""

    def __init__(self, temporal_scale, channel_scale, eps: float = 1e-6):
        Dm = temporal_scale.shape[0]
        dev = temporal_scale.device
        _need(temporal_scale, "temporal_scale", torch.bfloat16, (Dm,), dev)
        _need(channel_scale, "channel_scale", torch.bfloat16, (Dm,), dev)
        self.Dm, self.device = Dm, dev
        self.tensors = (temporal_scale, channel_scale)
        self.c = rglru_norm_params(temporal_scale.data_ptr(), channel_scale.data_ptr(), float(eps))


class MlpParams:
    """The MLP (bf16, Linear weights [out, in]): gate_w, up_w [F, D_model], down_w [D_model, F];
    biases [F], [F], [D_model] or None."""

    def __init__(self, gate_w, gate_b, up_w, up_b, down_w, down_b):
        F, Dm = gate_w.shape
        dev = gate_w.device
        _need(gate_w, "gate_w", torch.bfloat16, (F, Dm), dev)
        _need(up_w, "up_w", torch.bfloat16, (F, Dm), dev)
        _need(down_w, "down_w", torch.bfloat16, (Dm, F), dev)
        _need(gate_b, "gate_b", torch.bfloat16, (F,), dev)
        _need(up_b, "up_b", torch.bfloat16, (F,), dev)
        _need(down_b, "down_b", torch.bfloat16, (Dm,), dev)
        self.F, self.Dm, self.device = F, Dm, dev
        self.tensors = (gate_w, gate_b, up_w, up_b, down_w, down_b)
        self.c = rglru_mlp_params(Dm, F, *[t.data_ptr() if t is not None else None
                                           for t in self.tensors])


def rglru_rmsnorm(x, scale=None, residual=None, eps: float = 1e-6, *, want_norm: bool = True,
                  want_h: bool = False, out=None, h_out=None):
    """h = x (+ residual) and RMSNorm(h) * scale over the last axis (bf16).  Returns
    (out, h_out) with None for what was not asked for."""
    lib = load_library()
    D = x.shape[-1]
    M = x.numel() // D if D else 0
    _need(x, "x", torch.bfloat16)
    _need(residual, "residual", torch.bfloat16, tuple(x.shape), x.device)
    _need(scale, "scale", torch.bfloat16, (D,), x.device)
    if want_norm and out is None:
        out = torch.empty_like(x)
    if want_h and h_out is None:
        h_out = torch.empty_like(x)
    _need(out, "out", torch.bfloat16, tuple(x.shape), x.device)
    _need(h_out, "h_out", torch.bfloat16, tuple(x.shape), x.device)
    st = lib.rglru_rmsnorm(M, D, _ptr(x), _ptr(residual), _ptr(scale), float(eps), _ptr(h_out),
                           _ptr(out), _stream())
    _check(lib, st, "rglru_rmsnorm")
    return out, h_out


def rglru_mlp(m: MlpParams, x, *, out=None, workspace: DeviceBuffer | None = None):
    """The gated MLP over the rows of x [..., D_model] (bf16)."""
    lib = load_library()
    M = x.numel() // m.Dm
    _need(x, "x", torch.bfloat16, None, m.device)
    if x.shape[-1] != m.Dm:
        raise ValueError("x width %d, MLP width %d" % (x.shape[-1], m.Dm))
    if out is None:
        out = torch.empty_like(x)
    _need(out, "out", torch.bfloat16, tuple(x.shape), m.device)
    if workspace is None:
        workspace = DeviceBuffer(int(lib.rglru_mlp_workspace_bytes(M, m.F)), m.device)
    st = lib.rglru_mlp(ctypes.byref(m.c), M, _ptr(x), _ptr(out), _ptr(workspace.t),
                       workspace.nbytes, _stream())
    _check(lib, st, "rglru_mlp")
    return out


def make_recurrent_layer_workspace(p: Params, q: ProjParams, m: MlpParams, B: int,
                                   T: int) -> Workspace:
    lib = load_library()
    return Workspace(int(lib.rglru_recurrent_layer_workspace_bytes(B, T, p.D, p.H, q.Dm, m.F)),
                     p.device)


def rglru_recurrent_layer_prefill(p: Params, q: ProjParams, n: NormParams, m: MlpParams, x_in,
                                  h0=None, conv0=None, *, out=None, h_last=None, conv_last=None,
                                  workspace: Workspace | None = None):
    """The residual layer around the recurrent block.  Returns (out, h_last, conv_last)."""
    lib = load_library()
    B, T, Dm = x_in.shape
    _need(x_in, "x_in", torch.bfloat16, (B, T, q.Dm), p.device)
    _need(h0, "h0", torch.float32, (B, p.D), p.device)
    _need(conv0, "conv0", torch.bfloat16, (B, 3, p.D), p.device)
    if out is None:
        out = torch.empty_like(x_in)
    if h_last is None:
        h_last = torch.empty((B, p.D), dtype=torch.float32, device=p.device)
    if conv_last is None:
        conv_last = torch.empty((B, 3, p.D), dtype=torch.bfloat16, device=p.device)
    if workspace is None:
        workspace = make_recurrent_layer_workspace(p, q, m, B, T)
    st = lib.rglru_recurrent_layer_prefill(ctypes.byref(p.c), ctypes.byref(q.c), ctypes.byref(n.c),
                                           ctypes.byref(m.c), B, T, _ptr(x_in), _ptr(out),
                                           _ptr(h0), _ptr(h_last), _ptr(conv0), _ptr(conv_last),
                                           _ptr(workspace.t), workspace.nbytes, _stream())
    _check(lib, st, "rglru_recurrent_layer_prefill")
    return out, h_last, conv_last


def rglru_attention_layer_prefill(a: AttnParams, n: NormParams, m: MlpParams, x_in, *,
                                  cache: AttnCache | None = None, out=None,
                                  workspace: DeviceBuffer | None = None):
    """The residual layer around the local-attention block (optionally filling a ring cache)."""
    lib = load_library()
    B, T, Dm = x_in.shape
    _need(x_in, "x_in", torch.bfloat16, (B, T, a.Dm), a.device)
    if out is None:
        out = torch.empty_like(x_in)
    if workspace is None:
        workspace = DeviceBuffer(int(lib.rglru_attention_layer_workspace_bytes(
            ctypes.byref(a.c), B, T, m.F)), a.device)
    if cache is not None and (cache.N != B or cache.window != a.window):
        raise ValueError("cache is for N=%d window=%d" % (cache.N, cache.window))
    st = lib.rglru_attention_layer_prefill(
        ctypes.byref(a.c), ctypes.byref(n.c), ctypes.byref(m.c), B, T, _ptr(x_in), _ptr(out),
        _ptr(cache.k) if cache is not None else None, _ptr(cache.v) if cache is not None else None,
        _ptr(workspace.t), workspace.nbytes, _stream())
    _check(lib, st, "rglru_attention_layer_prefill")
    return out


def rglru_recurrent_layer_decode(p: Params, q: ProjParams, n: NormParams, m: MlpParams, x_t, h,
                                 conv_state, *, out=None, workspace: DeviceBuffer | None = None):
    """One decode step of the residual layer around the recurrent block: x_t [N, D_model];
    h [N, D] fp32 and conv_state [N, 3, D] are updated in place."""
    lib = load_library()
    N, Dm = x_t.shape
    _need(x_t, "x_t", torch.bfloat16, (N, q.Dm), p.device)
    _need(h, "h", torch.float32, (N, p.D), p.device)
    _need(conv_state, "conv_state", torch.bfloat16, (N, 3, p.D), p.device)
    if out is None:
        out = torch.empty_like(x_t)
    if workspace is None:
        workspace = DeviceBuffer(int(lib.rglru_recurrent_layer_decode_workspace_bytes(
            N, p.D, q.Dm, m.F)), p.device)
    st = lib.rglru_recurrent_layer_decode(ctypes.byref(p.c), ctypes.byref(q.c), ctypes.byref(n.c),
                                          ctypes.byref(m.c), N, _ptr(x_t), _ptr(out), _ptr(h),
                                          _ptr(conv_state), _ptr(workspace.t), workspace.nbytes,
                                          _stream())
    _check(lib, st, "rglru_recurrent_layer_decode")
    return out


def rglru_attention_layer_decode(a: AttnParams, n: NormParams, m: MlpParams, pos, x_t,
                                 cache: AttnCache, *, out=None,
                                 workspace: DeviceBuffer | None = None):
    """One decode step of the residual layer around the local-attention block."""
    lib = load_library()
    N, Dm = x_t.shape
    _need(x_t, "x_t", torch.bfloat16, (N, a.Dm), a.device)
    _need(pos, "pos", torch.int32, (N,), a.device)
    if out is None:
        out = torch.empty_like(x_t)
    if workspace is None:
        workspace = DeviceBuffer(int(lib.rglru_attention_layer_decode_workspace_bytes(
            ctypes.byref(a.c), N, m.F)), a.device)
    st = lib.rglru_attention_layer_decode(ctypes.byref(a.c), ctypes.byref(n.c), ctypes.byref(m.c),
                                          N, _ptr(pos), _ptr(x_t), _ptr(out), _ptr(cache.k),
                                          _ptr(cache.v), _ptr(workspace.t), workspace.nbytes,
                                          _stream())
    _check(lib, st, "rglru_attention_layer_decode")
    return out


def rglru_prefill_backward_workspace_bytes(B: int, T: int, D: int, n_heads: int) -> int:
    return int(load_library().rglru_prefill_backward_workspace_bytes(B, T, D, n_heads))


BACKWARD_GRADS = ("dx", "dy", "dconv_w", "dconv_b", "dwa", "dba", "dwx", "dbx", "dlambda", "dh0",
                  "dconv0")


def rglru_prefill_backward(p: Params, x, y, dout, h0=None, conv0=None, dh_last=None, *,
                           workspace: DeviceBuffer | None = None) -> dict:
    """Gradients of sum(dout * out) + sum(dh_last * h_last) for rglru_prefill (bf16, block
    size 256).  Returns a dict of tensors: dx, dy (bf16, like x); the rest fp32."""
    lib = load_library()
    B, T, D = x.shape
    dev = p.device
    _need(x, "x", torch.bfloat16, (B, T, p.D), dev)
    _need(y, "y", torch.bfloat16, (B, T, p.D), dev)
    _need(dout, "dout", torch.bfloat16, (B, T, p.D), dev)
    _need(h0, "h0", torch.float32, (B, D), dev)
    _need(conv0, "conv0", torch.bfloat16, (B, 3, D), dev)
    _need(dh_last, "dh_last", torch.float32, (B, D), dev)
    bs = D // p.H
    f32 = dict(dtype=torch.float32, device=dev)
    g = {"dx": torch.empty_like(x), "dy": torch.empty_like(y),
         "dconv_w": torch.empty((D, 4), **f32), "dconv_b": torch.empty((D,), **f32),
         "dwa": torch.empty((p.H, bs, bs), **f32), "dba": torch.empty((D,), **f32),
         "dwx": torch.empty((p.H, bs, bs), **f32), "dbx": torch.empty((D,), **f32),
         "dlambda": torch.empty((D,), **f32), "dh0": torch.empty((B, D), **f32),
         "dconv0": torch.empty((B, 3, D), **f32)}
    if workspace is None:
        workspace = DeviceBuffer(rglru_prefill_backward_workspace_bytes(B, T, D, p.H), dev)
    st = lib.rglru_prefill_backward(ctypes.byref(p.c), B, T, _ptr(x), _ptr(y), _ptr(h0),
                                    _ptr(conv0), _ptr(dout), _ptr(dh_last),
                                    *[_ptr(g[k]) for k in BACKWARD_GRADS], _ptr(workspace.t),
                                    workspace.nbytes, _stream())
    _check(lib, st, "rglru_prefill_backward")
    return g
