"""Seeded synthetic inputs shaped like RecurrentGemma's recurrent block.

This module only draws random numbers; it holds none of the method's
arithmetic.  The oracle tests, the GPU parity tests and the benchmark all take
their inputs from here, so both sides of a comparison read the same bits.

Storage form: fp32 tensors are ``float32`` arrays; bf16 tensors are ``uint16``
arrays of raw bf16 bits, rounded from fp32 draws with round-to-nearest-even.
Lambda and h0 are always ``float32``.

Streams: every tensor has its own ``numpy.random.Generator(PCG64(...))``
seeded by ``SeedSequence([seed, tensor_id, ...])``.  Activations (x, y) are
drawn in blocks of 1024 tokens per sequence, each block from its own stream,
so a time prefix of one sequence can be regenerated without the rest.

The widths follow the RecurrentGemma pages (2B: width 2560 for both branches,
conv kernel 4); the 9B width (4096, 16 heads of 256), the gate block sizes and
the value distributions are those of the five workloads below.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

F32 = "f32"
BF16 = "bf16"
ACT_BLOCK = 1024  # tokens per activation stream block

# tensor ids for SeedSequence (fixed order: Lambda, W_a, W_x, b_a, b_x, conv_w, conv_b, h0, x, y)
_TID = {"lambda": 0, "wa": 1, "wx": 2, "ba": 3, "bx": 4, "conv_w": 5, "conv_b": 6, "h0": 7,
        "x": 8, "y": 9,
        # the block's dense projections and its input (x_in feeds linear_x and linear_y)
        "lx_w": 10, "lx_b": 11, "ly_w": 12, "ly_b": 13, "lo_w": 14, "lo_b": 15, "x_in": 16,
        # the local-attention block's projections and the attention's own inputs
        "q_w": 17, "k_w": 18, "v_w": 19, "o_w": 20, "o_b": 21, "q": 22, "k": 23, "v": 24,
        # the residual layer: the two norm scales and the MLP
        "norm_t": 25, "norm_c": 26, "gate_w": 27, "gate_b": 28, "up_w": 29, "up_b": 30,
        "down_w": 31, "down_b": 32}

MLP_EXPANSION = 3      # MLP width = 3 x model width (7680 at width 2560)
NORM_EPS = 1e-6

# local attention of the 2B model: 10 query heads of width 256 sharing one key/value head,
# a window of 2048 tokens, RoPE base 10000
ATTN_HEAD_DIM = 256
ATTN_HEADS_2B = 10
ATTN_WINDOW = 2048
ROPE_BASE = 10000.0


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int            # sequences (decode: concurrent sequences N)
    T: int            # tokens per sequence (decode: number of single-token steps)
    D: int            # channels (RNN width)
    H: int            # gate heads; block size bs = D // H
    dtype: str        # storage type of activations and weights
    sig_lo: float     # sigmoid(Lambda) ~ U[sig_lo, sig_hi]
    sig_hi: float
    h0_std: float     # 0 -> h0 = 0
    seed: int
    decode: bool = False

    @property
    def bs(self) -> int:
        return self.D // self.H

    @property
    def w_std(self) -> float:
        return 1.0 / math.sqrt(self.bs)


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny-fp32-B1-T256-D256-H2", 1, 256, 256, 2, F32, 0.9, 0.999, 0.0, 1000),
        Workload("2b-prefill-B1-T2048-D2560-H10", 1, 2048, 2560, 10, BF16, 0.9, 0.999, 0.0, 1001),
        Workload("2b-batched-B8-T8192-D2560-H10", 8, 8192, 2560, 10, BF16, 0.9, 0.999, 0.1, 1002),
        Workload("2b-decode-N256-S1024-D2560-H10", 256, 1024, 2560, 10, BF16, 0.9, 0.999, 0.0, 1003,
                 decode=True),
        Workload("9b-long-B2-T65536-D4096-H16", 2, 65536, 4096, 16, BF16, 0.99, 0.9999, 0.0, 1004),
    ]
}
TINY, PREFILL_2B, BATCHED_2B, DECODE_2B, LONG_9B = list(WORKLOADS)


def round_bf16(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bits, round to nearest even (inputs are finite draws)."""
    a = np.ascontiguousarray(a, np.float32)
    bits = a.view(np.uint32).astype(np.uint64)
    bits = (bits + 0x7FFF + ((bits >> 16) & 1)) >> 16
    return bits.astype(np.uint16)


def to_storage(a: np.ndarray, dtype: str) -> np.ndarray:
    a = np.asarray(a, np.float32)
    return round_bf16(a) if dtype == BF16 else np.ascontiguousarray(a)


def _rng(*key) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def make_params(w: Workload, biases: bool = False, seed: int | None = None) -> dict:
    """Parameters in storage form.

    Lambda: s ~ U[sig_lo, sig_hi], Lambda = log(s / (1 - s)), so sigmoid(Lambda) = s.
    W_a, W_x [H, bs, bs] ~ N(0, std 1/sqrt(bs)); conv_w [D, 4] ~ N(0, std 0.5).
    biases=False: b_a = b_x = conv_b = 0 (the measured workloads);
    biases=True:  b_a, b_x, conv_b ~ N(0, std 0.5) (extra parity coverage).
    """
    s0 = w.seed if seed is None else seed
    D, H, bs = w.D, w.H, w.bs
    s = _rng(s0, _TID["lambda"]).uniform(w.sig_lo, w.sig_hi, D)
    lam = np.log(s / (1.0 - s)).astype(np.float32)
    wa = _rng(s0, _TID["wa"]).standard_normal((H, bs, bs), dtype=np.float32) * np.float32(w.w_std)
    wx = _rng(s0, _TID["wx"]).standard_normal((H, bs, bs), dtype=np.float32) * np.float32(w.w_std)
    if biases:
        ba = _rng(s0, _TID["ba"]).standard_normal(D, dtype=np.float32) * np.float32(0.5)
        bx = _rng(s0, _TID["bx"]).standard_normal(D, dtype=np.float32) * np.float32(0.5)
        cb = _rng(s0, _TID["conv_b"]).standard_normal(D, dtype=np.float32) * np.float32(0.5)
    else:
        ba = np.zeros(D, np.float32)
        bx = np.zeros(D, np.float32)
        cb = np.zeros(D, np.float32)
    cw = _rng(s0, _TID["conv_w"]).standard_normal((D, 4), dtype=np.float32) * np.float32(0.5)
    st = lambda a: to_storage(a, w.dtype)
    return {"conv_w": st(cw), "conv_b": st(cb), "wa": st(wa), "ba": st(ba), "wx": st(wx),
            "bx": st(bx), "lambda": lam}


def make_h0(w: Workload, B: int | None = None, seed: int | None = None) -> np.ndarray | None:
    """h0 [B, D] fp32 ~ N(0, h0_std), or None when the workload starts from zero."""
    if w.h0_std == 0.0:
        return None
    s0 = w.seed if seed is None else seed
    B = w.B if B is None else B
    return _rng(s0, _TID["h0"]).standard_normal((B, w.D), dtype=np.float32) * np.float32(w.h0_std)


def make_conv0(w: Workload, B: int, seed: int | None = None) -> np.ndarray:
    """A random conv state [B, 3, D] ~ N(0, 1) in storage form (edge-case coverage only)."""
    s0 = w.seed if seed is None else seed
    return to_storage(_rng(s0, _TID["conv_b"], 77).standard_normal((B, 3, w.D), dtype=np.float32),
                      w.dtype)


def make_act(w: Workload, which: str, B: int | None = None, T: int | None = None,
             seed: int | None = None) -> np.ndarray:
    """x or y [B, T, D] ~ N(0, 1) in storage form; blocks of 1024 tokens per stream."""
    assert which in ("x", "y")
    s0 = w.seed if seed is None else seed
    B = w.B if B is None else B
    T = w.T if T is None else T
    st_dtype = np.uint16 if w.dtype == BF16 else np.float32
    out = np.empty((B, T, w.D), st_dtype)
    for b in range(B):
        for blk in range((T + ACT_BLOCK - 1) // ACT_BLOCK):
            t0 = blk * ACT_BLOCK
            n = min(ACT_BLOCK, T - t0)
            a = _rng(s0, _TID[which], b, blk).standard_normal((ACT_BLOCK, w.D), dtype=np.float32)
            out[b, t0:t0 + n] = to_storage(a[:n], w.dtype)
    return out


def small(w: Workload, B: int | None = None, T: int | None = None) -> Workload:
    """The same distributions with other sizes (test cases)."""
    return dataclasses.replace(w, B=w.B if B is None else B, T=w.T if T is None else T)


def make_proj(w: Workload, Dm: int | None = None, biases: bool = False,
              seed: int | None = None) -> dict:
    """The block's dense projections in storage form (Linear weights [out][in]).

    linear_x, linear_y [D, Dm] ~ N(0, std 1/sqrt(Dm)) and linear_out [Dm, D] ~ N(0, std
    1/sqrt(D)), so unit-variance block inputs give unit-variance branch inputs.
    biases=False: zero biases (the measured workloads); True: N(0, std 0.1) (parity coverage).
    """
    s0 = w.seed if seed is None else seed
    D = w.D
    Dm = D if Dm is None else Dm
    out = {}
    for name, shape, fan_in in (("lx_w", (D, Dm), Dm), ("ly_w", (D, Dm), Dm), ("lo_w", (Dm, D), D)):
        a = _rng(s0, _TID[name]).standard_normal(shape, dtype=np.float32)
        out[name] = to_storage(a * np.float32(1.0 / math.sqrt(fan_in)), w.dtype)
    for name, n in (("lx_b", D), ("ly_b", D), ("lo_b", Dm)):
        a = (_rng(s0, _TID[name]).standard_normal(n, dtype=np.float32) * np.float32(0.1)
             if biases else np.zeros(n, np.float32))
        out[name] = to_storage(a, w.dtype)
    return out


def make_block_input(w: Workload, Dm: int | None = None, B: int | None = None,
                     T: int | None = None, seed: int | None = None) -> np.ndarray:
    """The block input x_in [B, T, Dm] ~ N(0, 1) in storage form; blocks of 1024 tokens."""
    s0 = w.seed if seed is None else seed
    Dm = w.D if Dm is None else Dm
    B = w.B if B is None else B
    T = w.T if T is None else T
    st_dtype = np.uint16 if w.dtype == BF16 else np.float32
    out = np.empty((B, T, Dm), st_dtype)
    for b in range(B):
        for blk in range((T + ACT_BLOCK - 1) // ACT_BLOCK):
            t0 = blk * ACT_BLOCK
            n = min(ACT_BLOCK, T - t0)
            a = _rng(s0, _TID["x_in"], b, blk).standard_normal((ACT_BLOCK, Dm), dtype=np.float32)
            out[b, t0:t0 + n] = to_storage(a[:n], w.dtype)
    return out


def make_attn(w: Workload, Dm: int | None = None, n_heads: int = ATTN_HEADS_2B,
              bias: bool = False, seed: int | None = None) -> dict:
    """The local-attention block's projections in storage form (Linear weights [out][in]).

    q_w [n_heads*256, Dm], k_w, v_w [256, Dm] ~ N(0, std 1/sqrt(Dm)); o_w [Dm, n_heads*256] ~
    N(0, std 1/sqrt(n_heads*256)); o_b zero, or N(0, std 0.1) with bias=True.
    """
    s0 = w.seed if seed is None else seed
    Dm = w.D if Dm is None else Dm
    HD = n_heads * ATTN_HEAD_DIM
    out = {}
    for name, shape, fan_in in (("q_w", (HD, Dm), Dm), ("k_w", (ATTN_HEAD_DIM, Dm), Dm),
                                ("v_w", (ATTN_HEAD_DIM, Dm), Dm), ("o_w", (Dm, HD), HD)):
        a = _rng(s0, _TID[name]).standard_normal(shape, dtype=np.float32)
        out[name] = to_storage(a * np.float32(1.0 / math.sqrt(fan_in)), w.dtype)
    a = (_rng(s0, _TID["o_b"]).standard_normal(Dm, dtype=np.float32) * np.float32(0.1)
         if bias else np.zeros(Dm, np.float32))
    out["o_b"] = to_storage(a, w.dtype)
    return out


def make_qkv(w: Workload, n_heads: int = ATTN_HEADS_2B, B: int | None = None,
             T: int | None = None, seed: int | None = None):
    """The attention's inputs before RoPE, ~ N(0, 1) in storage form, blocks of 1024 tokens:
    q [B, T, n_heads, 256], k and v [B, T, 256]."""
    s0 = w.seed if seed is None else seed
    B = w.B if B is None else B
    T = w.T if T is None else T
    st_dtype = np.uint16 if w.dtype == BF16 else np.float32
    res = []
    for name, tail in (("q", (n_heads, ATTN_HEAD_DIM)), ("k", (ATTN_HEAD_DIM,)),
                       ("v", (ATTN_HEAD_DIM,))):
        out = np.empty((B, T) + tail, st_dtype)
        for b in range(B):
            for blk in range((T + ACT_BLOCK - 1) // ACT_BLOCK):
                t0 = blk * ACT_BLOCK
                n = min(ACT_BLOCK, T - t0)
                a = _rng(s0, _TID[name], b, blk).standard_normal((ACT_BLOCK,) + tail,
                                                                 dtype=np.float32)
                out[b, t0:t0 + n] = to_storage(a[:n], w.dtype)
        res.append(out)
    return tuple(res)


def make_layer(w: Workload, Dm: int | None = None, F: int | None = None, biases: bool = False,
               seed: int | None = None) -> dict:
    """The residual layer's own weights in storage form: the two RMSNorm scales
    (temporal_scale, channel_scale) ~ 1 + N(0, 0.1); the MLP's gate_w, up_w [F, Dm] ~
    N(0, 1/sqrt(Dm)) and down_w [Dm, F] ~ N(0, 1/sqrt(F)); biases zero, or N(0, 0.1)."""
    s0 = w.seed if seed is None else seed
    Dm = w.D if Dm is None else Dm
    F = MLP_EXPANSION * Dm if F is None else F
    out = {}
    for name in ("norm_t", "norm_c"):
        a = 1.0 + _rng(s0, _TID[name]).standard_normal(Dm, dtype=np.float32) * np.float32(0.1)
        out[name] = to_storage(a, w.dtype)
    for name, shape, fan_in in (("gate_w", (F, Dm), Dm), ("up_w", (F, Dm), Dm),
                                ("down_w", (Dm, F), F)):
        a = _rng(s0, _TID[name]).standard_normal(shape, dtype=np.float32)
        out[name] = to_storage(a * np.float32(1.0 / math.sqrt(fan_in)), w.dtype)
    for name, n in (("gate_b", F), ("up_b", F), ("down_b", Dm)):
        a = (_rng(s0, _TID[name]).standard_normal(n, dtype=np.float32) * np.float32(0.1)
             if biases else np.zeros(n, np.float32))
        out[name] = to_storage(a, w.dtype)
    return out
