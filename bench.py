#!/usr/bin/env python3
"""Benchmark of the RG-LRU recurrent-block path on one MI355X.

A step is one rglru_prefill call over the 2B-shaped batched workload (B=8, T=8192, D=2560,
10 gate heads of 256, bf16 storage, fp32 state): conv, gates, scan, GELU merge and all
stores, inputs resident in HBM.  Prints one JSON line.  Besides the headline prefill figure
the line carries the dominant kernel's roofline, the oracle's CPU throughput on a bounded
sample, the 2B single-sequence prefill, the decode step time (256 sequences, D=2560), the
conv-state update and the whole block with its dense projections.

  python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline] [--no-extras]
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from gated_linear_recurrence_amd import synth  # noqa: E402

METRIC = "RG-LRU prefill tokens·channels/s + decode step µs; % of MI355X HBM peak"
HBM_PEAK_GBS = 8000.0
PREFILL_KERNEL = "prefill_bf16_kernel<256>"
# sources that define the measured prefill kernel; counter summaries name their hash
KERNEL_SOURCES = ["gated_linear_recurrence_amd/csrc/rglru_prefill.hip",
                  "gated_linear_recurrence_amd/csrc/rglru_device.h",
                  "gated_linear_recurrence_amd/csrc/rglru_internal.h",
                  "gated_linear_recurrence_amd/build.py"]
COUNTERS_JSON = os.path.join(ROOT, "profiles", "prefill_bf16_kernel-2b-batched-counters.json")


def algorithmic_bytes(w: synth.Workload, B: int, T: int, state: bool = True) -> int:
    """Minimum HBM bytes of one prefill: x, y read and out written once, weights, state."""
    e = 2 if w.dtype == synth.BF16 else 4
    D, Hh, bs = w.D, w.H, w.bs
    act = 3 * B * T * D * e
    weights = 2 * Hh * bs * bs * e + D * 4 * e + D * 4  # gate blocks, conv taps, Lambda
    st = (B * D * 4 * (2 if w.h0_std else 1) + B * 3 * D * e) if state else 0
    return act + weights + st


def decode_bytes(w: synth.Workload, N: int) -> int:
    """HBM bytes of one decode step in the ABI's layout: x_t, y_t, out_t, h (r+w),
    conv window (r+w), gate blocks, conv taps, Lambda."""
    e = 2 if w.dtype == synth.BF16 else 4
    D = w.D
    return 3 * N * D * e + 2 * N * D * 4 + 2 * N * 3 * D * e + 2 * w.H * w.bs * w.bs * e + \
        D * 4 * e + D * 4


def conv_update_bytes(w: synth.Workload, N: int, T: int) -> int:
    """HBM bytes of one conv1d_state_update with outputs: x read and u written once, the
    window read and written, the taps and bias."""
    e = 2 if w.dtype == synth.BF16 else 4
    return 2 * N * T * w.D * e + 2 * N * 3 * w.D * e + w.D * 5 * e


def time_conv_update(w, steps, torch, binding):
    """ms per conv1d_state_update (outputs for all T tokens, window update) on w's shape."""
    p = synth.make_params(w)
    P = binding.Params(*[_to_dev(p[k], torch) for k in ("conv_w", "conv_b", "wa", "ba", "wx",
                                                          "bx", "lambda")])
    x = _to_dev(synth.make_act(w, "x"), torch)
    cs = torch.zeros((w.B, 3, w.D), dtype=x.dtype, device="cuda")
    out = torch.empty_like(x)
    for _ in range(2):
        binding.conv1d_state_update(P, x, cs, out=out)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        binding.conv1d_state_update(P, x, cs, out=out)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def _to_dev(a, torch):
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


FLUSH_BYTES = 512 << 20  # twice the 256 MB Infinity Cache


def flushed_median_ms(torch, call, reps):
    """Median GPU time of call() when a FLUSH_BYTES write precedes each rep, so that the call's
    working set is no longer held in the L2 or the Infinity Cache."""
    buf = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
    ev = []
    for _ in range(reps):
        buf.zero_()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        call()
        e1.record()
        ev.append((e0, e1))
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in ev)
    del buf
    return ms[len(ms) // 2]


def prepare_prefill(w, B, T, torch, binding):
    """Device-resident parameters, inputs, outputs and workspace of one prefill workload."""
    p = synth.make_params(w)
    P = binding.Params(*[_to_dev(p[k], torch) for k in ("conv_w", "conv_b", "wa", "ba", "wx",
                                                          "bx", "lambda")])
    wb = synth.small(w, B=B, T=T)
    x = _to_dev(synth.make_act(wb, "x"), torch)
    y = _to_dev(synth.make_act(wb, "y"), torch)
    h0 = _to_dev(synth.make_h0(wb), torch)
    out = torch.empty_like(x)
    hl = torch.empty((B, w.D), dtype=torch.float32, device="cuda")
    cl = torch.empty((B, 3, w.D), dtype=x.dtype, device="cuda")
    ws = binding.make_workspace(P, B, T)
    torch.cuda.synchronize()
    return P, x, y, h0, out, hl, cl, ws


def time_prefill(w, B, T, steps, warmup, torch, binding, flush=False, prepared=None):
    """Mean ms per rglru_prefill call over `steps` back-to-back calls after `warmup` untimed
    ones (or, with flush=True, the median of single calls after a cache-flushing write)."""
    P, x, y, h0, out, hl, cl, ws = prepared or prepare_prefill(w, B, T, torch, binding)
    for _ in range(warmup):
        binding.rglru_prefill(P, x, y, h0, out=out, h_last=hl, conv_last=cl, workspace=ws)
    torch.cuda.synchronize()
    if flush:
        ms = flushed_median_ms(torch, lambda: binding.rglru_prefill(
            P, x, y, h0, out=out, h_last=hl, conv_last=cl, workspace=ws), steps)
        if ws.flags():
            raise RuntimeError("prefill workspace reported error flags %#x" % ws.flags())
        return ms
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        binding.rglru_prefill(P, x, y, h0, out=out, h_last=hl, conv_last=cl, workspace=ws)
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    flags = ws.flags()
    if flags:
        raise RuntimeError("prefill workspace reported error flags %#x" % flags)
    return ms


def time_decode(w, N, steps, torch, binding, split=True, flush=False):
    """Per-step time of `steps` decode steps: (eager us, graph us), or with flush=True the median
    of single steps each preceded by a cache-flushing write (eager, us)."""
    p = synth.make_params(w)
    P = binding.Params(*[_to_dev(p[k], torch) for k in ("conv_w", "conv_b", "wa", "ba", "wx",
                                                          "bx", "lambda")])
    wb = synth.small(w, B=N, T=steps)
    x = _to_dev(synth.make_act(wb, "x"), torch)
    y = _to_dev(synth.make_act(wb, "y"), torch)
    h = torch.zeros((N, w.D), dtype=torch.float32, device="cuda")
    cs = torch.zeros((N, 3, w.D), dtype=x.dtype, device="cuda")
    outs = torch.empty_like(x)

    ws = binding.make_decode_workspace(P, N) if split else None

    def run():
        for t in range(steps):
            binding.rglru_decode_step(P, x[:, t], y[:, t], h, cs, out_t=outs[:, t], workspace=ws)

    run()  # warm-up
    torch.cuda.synchronize()
    if flush:
        t = [0]

        def one():
            k = t[0] % steps
            binding.rglru_decode_step(P, x[:, k], y[:, k], h, cs, out_t=outs[:, k], workspace=ws)
            t[0] += 1
        return flushed_median_ms(torch, one, 25) * 1e3
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    run()
    e1.record()
    torch.cuda.synchronize()
    eager_us = e0.elapsed_time(e1) * 1e3 / steps
    # the same loop captured once as a graph and replayed (no host launch cost per step)
    graph_us = None
    try:
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            run()
        torch.cuda.current_stream().wait_stream(s)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            run()
        g.replay()
        torch.cuda.synchronize()
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        graph_us = e0.elapsed_time(e1) * 1e3 / steps
    except Exception as exc:  # graph capture is optional for the figure
        print("decode graph capture skipped: %s" % exc, file=sys.stderr)
    return eager_us, graph_us


MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA


def time_block(w, steps, warmup, torch, binding):
    """The whole temporal-mixing block (linear_x | linear_y, the path, linear_out) at the
    workload's shape, plus each projection GEMM on its own (rglru_linear) and, for context, the
    same GEMMs through torch.nn.functional.linear (hipBLASLt)."""
    p = synth.make_params(w)
    q = synth.make_proj(w)
    P = binding.Params(*[_to_dev(p[k], torch) for k in ("conv_w", "conv_b", "wa", "ba", "wx",
                                                          "bx", "lambda")])
    qd = {k: _to_dev(v, torch) for k, v in q.items()}
    Q = binding.ProjParams(qd["lx_w"], qd["lx_b"], qd["ly_w"], qd["ly_b"], qd["lo_w"], qd["lo_b"])
    x_in = _to_dev(synth.make_block_input(w), torch)
    h0 = _to_dev(synth.make_h0(w), torch)
    out = torch.empty_like(x_in)
    hl = torch.empty((w.B, w.D), dtype=torch.float32, device="cuda")
    cl = torch.empty((w.B, 3, w.D), dtype=x_in.dtype, device="cuda")
    ws = binding.make_block_workspace(P, Q, w.B, w.T)

    def timed(call, n):
        for _ in range(warmup):
            call()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            call()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    ms_block = timed(lambda: binding.rglru_block_prefill(P, Q, x_in, h0, out=out, h_last=hl,
                                                         conv_last=cl, workspace=ws), steps)
    if ws.flags():
        raise RuntimeError("block workspace reported error flags %#x" % ws.flags())
    M = w.B * w.T
    x2 = x_in.view(M, w.D)
    w_in = torch.cat([qd["lx_w"], qd["ly_w"]], 0).contiguous()     # [2D, D_model]
    b_in = torch.cat([qd["lx_b"], qd["ly_b"]], 0).contiguous()
    y_in = torch.empty((M, 2 * w.D), dtype=x_in.dtype, device="cuda")
    mg = out.view(M, w.D)                                          # any [M, D] bf16 operand
    y_out = torch.empty((M, w.D), dtype=x_in.dtype, device="cuda")
    gemms = {}
    for name, (a, wt, b, o) in {"in_proj": (x2, w_in, b_in, y_in),
                                "out_proj": (mg, qd["lo_w"], qd["lo_b"], y_out)}.items():
        ms = timed(lambda: binding.rglru_linear(a, wt, b, out=o), steps)
        ms_lib = timed(lambda: torch.nn.functional.linear(a, wt, b), steps)
        fl = 2.0 * M * a.shape[1] * wt.shape[0]
        gemms[name] = {"M": M, "K": a.shape[1], "N": wt.shape[0], "ms": ms,
                       "tflops": fl / (ms * 1e-3) / 1e12,
                       "mfma_frac": fl / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                       "hipblaslt_ms": ms_lib,
                       "hipblaslt_tflops": fl / (ms_lib * 1e-3) / 1e12}
    flops = 2.0 * M * w.D * (2 * w.D) + 2.0 * M * w.D * w.D
    return {"workload": w.name + " (block input width 2560 = D)", "ms": ms_block,
            "tokens/s": M / (ms_block * 1e-3),
            "projection_tflop": flops / 1e12,
            "roofline": {"bound": "mfma", "kernel": "proj_gemm_kernel (in_proj)",
                         "achieved": gemms["in_proj"]["tflops"], "peak": MFMA_BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s",
                         "frac": gemms["in_proj"]["tflops"] / MFMA_BF16_PEAK_TFLOPS},
            "gemms": gemms,
            "note": "hipblaslt_* is torch.nn.functional.linear on the same operands, for context"}


def attention_flops(B: int, T: int, Hq: int, W: int) -> float:
    """Algorithmic flops of local attention: per (query, head, key in its window) a 256-long dot
    product and a 256-long update, 4 * 256 flops."""
    keys = sum(min(t + 1, W) for t in range(T))
    return 4.0 * synth.ATTN_HEAD_DIM * keys * B * Hq


def time_attention(w, steps, warmup, torch, binding):
    """Local sliding-window MQA (the model's other temporal-mixing block) at the batched 2B
    shape: the attention alone (RoPE prep + flash kernel), the block with its projections, and
    a decode step for 256 sequences with a full 2048-slot ring cache."""
    Hq, W = synth.ATTN_HEADS_2B, synth.ATTN_WINDOW

    def timed(call, n):
        for _ in range(warmup):
            call()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            call()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    q, k, v = (_to_dev(a, torch) for a in synth.make_qkv(w, Hq))
    o = torch.empty_like(q)
    ws = binding.DeviceBuffer(binding.rglru_local_attention_workspace_bytes(w.B, w.T, Hq), "cuda")
    ms = timed(lambda: binding.rglru_local_attention(q, k, v, W, out=o, workspace=ws), steps)
    fl = attention_flops(w.B, w.T, Hq, W)
    tf = fl / (ms * 1e-3) / 1e12
    # torch's scaled_dot_product_attention with the same band as a boolean mask, one sequence
    # (the shared key/value head expanded to the ten query heads), for context
    i = torch.arange(w.T, device="cuda")
    band = (i[None, :] <= i[:, None]) & (i[None, :] > i[:, None] - W)
    qq = q[:1].transpose(1, 2).contiguous()
    kk = k[:1, :, None].expand(1, w.T, Hq, 256).transpose(1, 2).contiguous()
    vv = v[:1, :, None].expand(1, w.T, Hq, 256).transpose(1, 2).contiguous()
    ms_sdpa = timed(lambda: torch.nn.functional.scaled_dot_product_attention(
        qq, kk, vv, attn_mask=band), max(steps // 4, 2))
    del qq, kk, vv, band

    a = synth.make_attn(w)
    ad = {n: _to_dev(t, torch) for n, t in a.items()}
    A = binding.AttnParams(ad["q_w"], ad["k_w"], ad["v_w"], ad["o_w"], ad["o_b"], Hq, W)
    x_in = _to_dev(synth.make_block_input(w), torch)
    out = torch.empty_like(x_in)
    wsb = binding.DeviceBuffer(binding.rglru_local_attention_block_workspace_bytes(A, w.B, w.T),
                               "cuda")
    ms_block = timed(lambda: binding.rglru_local_attention_block(A, x_in, out=out, workspace=wsb),
                     max(steps // 2, 3))
    M, Dm, HD = w.B * w.T, w.D, Hq * synth.ATTN_HEAD_DIM
    fl_proj = 2.0 * M * Dm * (HD + 2 * synth.ATTN_HEAD_DIM) + 2.0 * M * HD * Dm
    del x_in, out, wsb, q, k, v, o, ws

    N, pos0 = 256, 5000
    cache = binding.AttnCache(N, W, "cuda")
    cache.k.normal_()
    cache.v.normal_()
    g = torch.Generator(device="cuda").manual_seed(w.seed)
    qd = torch.randn((N, Hq, 256), generator=g, device="cuda").to(torch.bfloat16)
    kd = torch.randn((N, 256), generator=g, device="cuda").to(torch.bfloat16)
    vd = torch.randn((N, 256), generator=g, device="cuda").to(torch.bfloat16)
    pos = torch.full((N,), pos0, dtype=torch.int32, device="cuda")
    od = torch.empty_like(qd)
    wsd = binding.DeviceBuffer(binding.rglru_local_attention_decode_workspace_bytes(N, Hq, W),
                               "cuda")
    us_dec = 1e3 * timed(lambda: binding.rglru_local_attention_decode(
        pos, qd, kd, vd, cache, out=od, workspace=wsd), max(steps, 20))
    dec_bytes = 2 * N * W * 256 * 2 + 2 * N * Hq * 256 * 2 + 2 * N * 256 * 2 * 2
    return {
        "workload": "%s shape: %d x %d tokens, %d query heads x 256 sharing one key/value head, "
                    "window %d, RoPE base %g" % (w.name, w.B, w.T, Hq, W, synth.ROPE_BASE),
        "ms": ms, "tflop": fl / 1e12, "tflops": tf,
        "roofline": {"bound": "mfma", "kernel": "attn_prep_kernel + attn_fwd_kernel (whole call)",
                     "achieved": tf, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": tf / MFMA_BF16_PEAK_TFLOPS},
        "torch_sdpa_band_mask_ms_per_sequence": ms_sdpa,
        "torch_sdpa_band_mask_ms_x_sequences": ms_sdpa * w.B,
        "block_ms": ms_block, "block_tokens/s": M / (ms_block * 1e-3),
        "block_projection_tflop": fl_proj / 1e12,
        "decode": {"sequences": N, "position": pos0, "window": W, "us_per_step": us_dec,
                   "bytes_per_step": dec_bytes,
                   "roofline": {"bound": "hbm", "kernel": "attn_dec_kernel (whole step)",
                                "achieved": dec_bytes / (us_dec * 1e-6) / 1e9,
                                "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                "frac": dec_bytes / (us_dec * 1e-6) / 1e9 / HBM_PEAK_GBS}},
        "note": "torch_sdpa_* is torch.nn.functional.scaled_dot_product_attention with the "
                "window as a boolean mask, for context"}


STACK_LAYERS = 26   # layers 0-1 recurrent, 2 attention, and so on (two recurrent to one attention)


def _dev_randn(torch, g, shape, std):
    return (torch.randn(shape, generator=g, device="cuda") * std).to(torch.bfloat16)


def _stack_weights(torch, binding, w, g):
    """Seeded random weights of one layer of each kind at the 2B widths, on the device."""
    D, Dm, F, Hq = w.D, w.D, synth.MLP_EXPANSION * w.D, synth.ATTN_HEADS_2B
    HD = Hq * synth.ATTN_HEAD_DIM

    def norms():
        return binding.NormParams(1 + _dev_randn(torch, g, (Dm,), 0.1),
                                  1 + _dev_randn(torch, g, (Dm,), 0.1), synth.NORM_EPS)

    def mlp():
        return binding.MlpParams(_dev_randn(torch, g, (F, Dm), Dm ** -0.5), None,
                                 _dev_randn(torch, g, (F, Dm), Dm ** -0.5), None,
                                 _dev_randn(torch, g, (Dm, F), F ** -0.5), None)

    def recurrent():
        bs = D // w.H
        lam = torch.log(torch.rand((D,), generator=g, device="cuda") * 0.099 + 0.9)
        lam = lam - torch.log1p(-torch.exp(lam))          # sigmoid(Lambda) ~ U[0.9, 0.999]
        P = binding.Params(_dev_randn(torch, g, (D, 4), 0.5), None,
                           _dev_randn(torch, g, (w.H, bs, bs), bs ** -0.5), None,
                           _dev_randn(torch, g, (w.H, bs, bs), bs ** -0.5), None,
                           lam.float().contiguous())
        Q = binding.ProjParams(_dev_randn(torch, g, (D, Dm), Dm ** -0.5), None,
                               _dev_randn(torch, g, (D, Dm), Dm ** -0.5), None,
                               _dev_randn(torch, g, (Dm, D), D ** -0.5), None)
        return ("recurrent", P, Q, norms(), mlp())

    def attention():
        A = binding.AttnParams(_dev_randn(torch, g, (HD, Dm), Dm ** -0.5),
                               _dev_randn(torch, g, (256, Dm), Dm ** -0.5),
                               _dev_randn(torch, g, (256, Dm), Dm ** -0.5),
                               _dev_randn(torch, g, (Dm, HD), HD ** -0.5), None, Hq,
                               synth.ATTN_WINDOW)
        return ("attention", A, None, norms(), mlp())

    return [attention() if i % 3 == 2 else recurrent() for i in range(STACK_LAYERS)]


def time_layers(w, steps, warmup, torch, binding):
    """The residual layers at the batched 2B shape (width 2560, MLP 7680): each layer alone, the
    MLP alone, and the 26-layer stack (two recurrent layers to one attention layer) on seeded
    random weights: a prefill of the whole 8 x 8192-token batch, and decode steps for 256 and
    for 1 sequences."""

    def timed(call, n, warm=warmup):
        for _ in range(warm):
            call()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            call()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    g = torch.Generator(device="cuda").manual_seed(w.seed + 7)
    layers = _stack_weights(torch, binding, w, g)
    B, T, Dm, D = w.B, w.T, w.D, w.D
    F = synth.MLP_EXPANSION * Dm
    M = B * T
    x = _to_dev(synth.make_block_input(w), torch)
    y = torch.empty_like(x)
    _, P, Q, Nn, Mm = layers[0]
    _, A, _, _, _ = layers[2]
    ws_r = binding.make_recurrent_layer_workspace(P, Q, Mm, B, T)
    ws_a = binding.DeviceBuffer(binding.load_library().rglru_attention_layer_workspace_bytes(
        __import__("ctypes").byref(A.c), B, T, F), "cuda")
    hl = torch.empty((B, D), dtype=torch.float32, device="cuda")
    cl = torch.empty((B, 3, D), dtype=torch.bfloat16, device="cuda")

    def rec_layer(P, Q, Nn, Mm, xi, yo):
        binding.rglru_recurrent_layer_prefill(P, Q, Nn, Mm, xi, out=yo, h_last=hl, conv_last=cl,
                                              workspace=ws_r)

    def att_layer(A, Nn, Mm, xi, yo):
        binding.rglru_attention_layer_prefill(A, Nn, Mm, xi, out=yo, workspace=ws_a)

    n = max(steps // 4, 2)
    ms_rec = timed(lambda: rec_layer(P, Q, Nn, Mm, x, y), n)
    ms_att = timed(lambda: att_layer(A, layers[2][3], layers[2][4], x, y), n)
    ws_m = binding.DeviceBuffer(binding.load_library().rglru_mlp_workspace_bytes(M, F), "cuda")
    xm = x.view(M, Dm)
    ms_mlp = timed(lambda: binding.rglru_mlp(Mm, xm, out=y.view(M, Dm), workspace=ws_m), n)
    del ws_m
    fl_mlp = 2.0 * M * Dm * F * 3
    z = torch.empty_like(xm)
    ms_norm = timed(lambda: binding.rglru_rmsnorm(xm, Nn.tensors[0], y.view(M, Dm), out=z),
                    max(steps, 10))
    del z
    norm_bytes = 3 * M * Dm * 2

    def stack_prefill():
        xi, yo = x, y
        for kind, Pa, Qa, Na, Ma in layers:
            if kind == "recurrent":
                rec_layer(Pa, Qa, Na, Ma, xi, yo)
            else:
                att_layer(Pa, Na, Ma, xi, yo)
            xi, yo = yo, xi

    ms_stack = timed(stack_prefill, 2, warm=1)
    del ws_r, ws_a, hl, cl

    def decode_stack(N):
        xs = _dev_randn(torch, g, (N, Dm), 1.0)
        ys = torch.empty_like(xs)
        pos = torch.full((N,), 4096, dtype=torch.int32, device="cuda")
        state = []
        lib = binding.load_library()
        import ctypes
        for kind, Pa, Qa, Na, Ma in layers:
            if kind == "recurrent":
                state.append((torch.zeros((N, D), dtype=torch.float32, device="cuda"),
                              _dev_randn(torch, g, (N, 3, D), 1.0),
                              binding.DeviceBuffer(lib.rglru_recurrent_layer_decode_workspace_bytes(
                                  N, D, Dm, F), "cuda")))
            else:
                c = binding.AttnCache(N, synth.ATTN_WINDOW, "cuda")
                c.k.normal_(generator=g)
                c.v.normal_(generator=g)
                state.append((c, None, binding.DeviceBuffer(
                    lib.rglru_attention_layer_decode_workspace_bytes(ctypes.byref(Pa.c), N, F),
                    "cuda")))

        def step():
            xi, yo = xs, ys
            for (kind, Pa, Qa, Na, Ma), (s0, s1, wsd) in zip(layers, state):
                if kind == "recurrent":
                    binding.rglru_recurrent_layer_decode(Pa, Qa, Na, Ma, xi, s0, s1, out=yo,
                                                         workspace=wsd)
                else:
                    binding.rglru_attention_layer_decode(Pa, Na, Ma, pos, xi, s0, out=yo,
                                                         workspace=wsd)
                xi, yo = yo, xi

        us = 1e3 * timed(step, max(steps // 2, 5), warm=2)
        graph_us = None
        try:
            gr = torch.cuda.CUDAGraph()
            st = torch.cuda.Stream()
            st.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(st):
                step()
                torch.cuda.synchronize()
                with torch.cuda.graph(gr, stream=st):
                    step()
            torch.cuda.current_stream().wait_stream(st)
            graph_us = 1e3 * timed(gr.replay, max(steps // 2, 5), warm=2)
        except Exception as ex:          # graph capture is an optimisation; eager stays valid
            print("stack decode graph capture failed: %s" % ex, file=sys.stderr)
        return us, graph_us

    dec256, dec256_g = decode_stack(256)
    dec1, dec1_g = decode_stack(1)
    n_params = sum(sum(t.numel() for t in (l[1].tensors if hasattr(l[1], "tensors") else ())
                       if t is not None) +
                   sum(t.numel() for t in (l[2].tensors if l[2] is not None else ()) if t is not None) +
                   sum(t.numel() for t in l[4].tensors if t is not None) for l in layers)
    return {
        "workload": "%s shape, width 2560, MLP 7680, residual layers with seeded random weights"
                    % w.name,
        "recurrent_layer_ms": ms_rec, "attention_layer_ms": ms_att,
        "mlp": {"ms": ms_mlp, "tflops": fl_mlp / (ms_mlp * 1e-3) / 1e12,
                "roofline": {"bound": "mfma", "achieved": fl_mlp / (ms_mlp * 1e-3) / 1e12,
                             "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                             "frac": fl_mlp / (ms_mlp * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS}},
        "add_rmsnorm": {"ms": ms_norm, "bytes": norm_bytes,
                        "roofline": {"bound": "hbm",
                                     "achieved": norm_bytes / (ms_norm * 1e-3) / 1e9,
                                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                     "frac": norm_bytes / (ms_norm * 1e-3) / 1e9 / HBM_PEAK_GBS}},
        "stack": {"layers": STACK_LAYERS, "pattern": "recurrent, recurrent, attention",
                  "parameters": n_params,
                  "prefill_ms": ms_stack, "prefill_tokens/s": M / (ms_stack * 1e-3),
                  "decode_256_us_per_step": dec256, "decode_256_us_per_step_graph": dec256_g,
                  "decode_1_us_per_step": dec1, "decode_1_us_per_step_graph": dec1_g,
                  "note": "no embedding or final norm; decode at position 4096 with full "
                          "attention windows; weight bytes per decode step %d"
                          % (2 * n_params)}}


def time_backward(w, steps, warmup, torch, binding):
    """The path's backward pass (rglru_prefill_backward) over the batched 2B workload."""
    p = synth.make_params(w)
    P = binding.Params(*[_to_dev(p[k], torch) for k in ("conv_w", "conv_b", "wa", "ba", "wx",
                                                          "bx", "lambda")])
    x, y = _to_dev(synth.make_act(w, "x"), torch), _to_dev(synth.make_act(w, "y"), torch)
    h0 = _to_dev(synth.make_h0(w), torch)
    g = torch.Generator(device="cuda").manual_seed(w.seed + 11)
    dout = torch.randn(tuple(x.shape), generator=g, device="cuda").to(torch.bfloat16)
    ws = binding.DeviceBuffer(binding.rglru_prefill_backward_workspace_bytes(w.B, w.T, w.D, w.H),
                              "cuda")
    call = lambda: binding.rglru_prefill_backward(P, x, y, dout, h0, workspace=ws)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        call()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    n = w.B * w.T * w.D
    byts = 10 * n               # x, y, dout read and dx, dy written, bf16
    flops = 3 * 2 * 2.0 * w.B * w.T * w.D * w.bs   # three block-diagonal products, two gates
    return {"workload": w.name, "ms": ms, "tokens·channels/s": n / (ms * 1e-3),
            "algorithmic_bytes": byts, "algorithmic_flop": flops,
            "roofline": {"bound": "hbm", "kernel": "whole backward call",
                         "achieved": byts / (ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": byts / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS},
            "mfma_frac": flops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
            "workspace_bytes": ws.nbytes}


def cpu_baseline(w):
    """The oracle on the whole headline workload (all 8 sequences x 8192 tokens x 10 heads),
    one OpenMP thread per (sequence, head) unit; inputs are generated before the clock starts."""
    import oracle
    x = synth.make_act(w, "x")
    y = synth.make_act(w, "y")
    h0 = synth.make_h0(w)
    p = synth.make_params(w)
    P = oracle.Params(p["conv_w"], p["conv_b"], p["wa"], p["ba"], p["wx"], p["bx"], p["lambda"], w.H)
    lib = oracle.load()
    threads = min(lib.oracle_max_threads(), w.B * w.H)
    t = time.perf_counter()
    oracle.prefill(P, x, y, h0=h0, nthreads=threads, lib=lib)
    dt = time.perf_counter() - t
    # one thread on one sequence of the same workload (all heads)
    t = time.perf_counter()
    oracle.prefill(P, x[:1], y[:1], h0=None if h0 is None else h0[:1], nthreads=1, lib=lib)
    dt1 = time.perf_counter() - t
    return {"value": w.B * w.T * w.D / dt, "unit": "tokens·channels/s", "cores": threads,
            "kind": "oracle", "seconds": round(dt, 3),
            "sample": "the whole workload: B=%d x T=%d x D=%d (all %d heads), fp64 sequential "
                      "oracle, OpenMP over (sequence, head) units" % (w.B, w.T, w.D, w.H),
            "single_core": {"value": w.T * w.D / dt1, "seconds": round(dt1, 3),
                            "sample": "sequence 0 only (T=%d x D=%d, all heads), one thread"
                                      % (w.T, w.D)}}


def copy_probe(torch, nbytes: int = 1 << 30, reps: int = 5):
    """A plain copy of known size: reads and writes nbytes per launch."""
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").normal_()
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    print(json.dumps({"copy_probe_bytes_each_way": nbytes, "ms": ms,
                      "GBs_read_plus_write": 2 * nbytes / (ms * 1e-3) / 1e9}), flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(rel.encode() + b"\0" + f.read() + b"\0")
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch of the prefill kernel from the committed counter summary, or None
    when the summary is missing or was taken on other kernel sources."""
    try:
        with open(COUNTERS_JSON) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("kernel_source_hash") != kernel_source_hash():
        return None
    return c.get("traffic_bytes_per_launch")


def _rows(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _mean_counter(path, name_part, counter, min_value=0.0):
    vals = [float(r["Counter_Value"]) for r in _rows(path)
            if name_part in r["Kernel_Name"] and r["Counter_Name"] == counter
            and float(r["Counter_Value"]) >= min_value]
    if not vals:
        raise SystemExit("no %s rows for %r in %s" % (counter, name_part, path))
    return sum(vals) / len(vals), len(vals)


def counter_summary(args):
    """Turn rocprofv3 CSV output into the committed summaries under profiles/."""
    kt = _rows(args.kernel_stats)
    pre = [r for r in kt if "prefill_bf16_kernel" in r["Name"]]
    if not pre:
        raise SystemExit("prefill_bf16_kernel not in %s" % args.kernel_stats)
    r = pre[0]
    avg_ns = float(r["AverageNs"])
    if args.kernel_trace:
        # the headline's timed steps are the run's last prefill dispatches (the other legs,
        # which also launch this kernel at other shapes, run before it)
        tr = [t for t in _rows(args.kernel_trace) if "prefill_bf16_kernel" in t["Kernel_Name"]]
        tr.sort(key=lambda t: int(t["Start_Timestamp"]))
        last = tr[-args.last:]
        avg_ns = sum(int(t["End_Timestamp"]) - int(t["Start_Timestamp"]) for t in last) / len(last)
    f_kib, nf = _mean_counter(args.fetch, "prefill_bf16_kernel", "FETCH_SIZE")
    w_kib, nw = _mean_counter(args.write, "prefill_bf16_kernel", "WRITE_SIZE")
    # calibration: a plain copy of 1 GiB reads and writes 1 GiB per dispatch
    cf_kib, _ = _mean_counter(args.copy_fetch, "copyBuffer", "FETCH_SIZE", 1e5)
    cw_kib, _ = _mean_counter(args.copy_write, "copyBuffer", "WRITE_SIZE", 1e5)
    gib_kib = float(1 << 20)
    fs, ws = gib_kib / cf_kib, gib_kib / cw_kib
    traffic = (f_kib * fs + w_kib * ws) * 1024.0
    w = synth.WORKLOADS[synth.BATCHED_2B]
    alg = algorithmic_bytes(w, w.B, w.T)
    out = {
        "kernel": PREFILL_KERNEL, "workload": w.name,
        "kernel_source_hash": kernel_source_hash(),
        "avg_duration_ns": avg_ns, "calls": int(r["Calls"]),
        "avg_over": ("the last %d dispatches (the headline's timed steps)" % args.last)
                    if args.kernel_trace else "all dispatches",
        "fetch_kib_per_dispatch": f_kib, "write_kib_per_dispatch": w_kib,
        "fetch_dispatches": nf, "write_dispatches": nw,
        "copy_probe_fetch_kib_per_gib": cf_kib, "copy_probe_write_kib_per_gib": cw_kib,
        "fetch_scale": fs, "write_scale": ws,
        "traffic_bytes_per_launch": traffic, "algorithmic_bytes_per_launch": alg,
        "traffic_over_algorithmic": traffic / alg,
        "commands": args.commands,
    }
    with open(COUNTERS_JSON, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    txt = os.path.join(ROOT, "profiles", "prefill_bf16_kernel-2b-batched-kernel-trace.txt")
    with open(txt, "w") as f:
        f.write("rocprofv3 kernel statistics, prefill on 2b-batched-B8-T8192-D2560-H10 (bf16)\n")
        f.write("kernel source hash %s\n\n" % out["kernel_source_hash"])
        f.write("commands (from the repository root):\n")
        for c in args.commands:
            f.write("  %s\n" % c)
        f.write("\n%-60s %6s %14s %14s %14s\n" % ("kernel", "calls", "avg ns", "min ns", "max ns"))
        for row in kt:
            f.write("%-60s %6s %14.0f %14.0f %14.0f\n" % (row["Name"][:60], row["Calls"],
                    float(row["AverageNs"]), float(row["MinNs"]), float(row["MaxNs"])))
        f.write("\nprefill_bf16_kernel per dispatch: FETCH_SIZE %.0f KiB (x%.3f), WRITE_SIZE %.0f KiB "
                "(x%.3f)\n" % (f_kib, fs, w_kib, ws))
        f.write("calibration (plain 1 GiB copy): FETCH_SIZE %.0f KiB, WRITE_SIZE %.0f KiB per GiB\n"
                % (cf_kib, cw_kib))
        f.write("HBM traffic per launch %.0f B = %.3f x algorithmic %d B\n"
                % (traffic, traffic / alg, alg))
        f.write("prefill_bf16_kernel average over %s: %.0f ns\n" % (out["avg_over"], avg_ns))
        f.write("algorithmic GB/s at that average duration: %.1f\n" % (alg / (avg_ns * 1e-9) / 1e9))
    print(json.dumps(out))


BACKWARD_TXT = os.path.join(ROOT, "profiles", "prefill_backward-2b-batched-kernel-trace.txt")


def backward_summary(args):
    """Per-kernel time and HBM traffic of the path's backward (rglru_prefill_backward) from
    rocprofv3 CSVs of the `--legs backward` run: a kernel trace and one FETCH_SIZE and one
    WRITE_SIZE pass, scaled by the copy-probe calibration; written to profiles/."""
    stats = _rows(args.kernel_stats)
    cf_kib, _ = _mean_counter(args.copy_fetch, "copyBuffer", "FETCH_SIZE", 1e5)
    cw_kib, _ = _mean_counter(args.copy_write, "copyBuffer", "WRITE_SIZE", 1e5)
    fs, ws = float(1 << 20) / cf_kib, float(1 << 20) / cw_kib
    per = {}
    for path, ctr in ((args.fetch, "FETCH_SIZE"), (args.write, "WRITE_SIZE")):
        acc = {}
        for r in _rows(path):
            if r["Counter_Name"] == ctr:
                acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        for name, v in acc.items():
            per.setdefault(name, {})[ctr] = sum(v) / len(v)
    w = synth.WORKLOADS[synth.BATCHED_2B]
    alg = 10 * w.B * w.T * w.D
    # kernels of the backward: everything but the forward prefill and torch's own set-up kernels
    keep = lambda n: ("bwd_" in n or "proj_" in n) and "prefill_bf16" not in n
    rows, tot_ns, tot_b = [], 0.0, 0.0
    for r in stats:
        n = r["Name"]
        if not keep(n):
            continue
        c = per.get(n, {})
        b = (c.get("FETCH_SIZE", 0.0) * fs + c.get("WRITE_SIZE", 0.0) * ws) * 1024.0
        calls = int(r["Calls"])
        short = n.replace("(anonymous namespace)", "").split("(")[0].split("::")[-1]
        rows.append((short, calls, float(r["AverageNs"]), b))
    # calls per backward: the bwd_ kernels run once per call
    n_bwd = max(c for name, c, _, _ in rows if name == "bwd_grad_kernel")
    with open(BACKWARD_TXT, "w") as f:
        f.write("rocprofv3 kernel trace and HBM traffic, the path's backward pass "
                "(rglru_prefill_backward) on\n%s (bf16, 10 heads of 256)\n\n" % w.name)
        f.write("commands (from the repository root):\n")
        for c in args.commands:
            f.write("  %s\n" % c)
        f.write("\n%-28s %6s %12s %14s %10s\n" % ("kernel", "calls", "avg us", "MB per call",
                                                  "GB/s"))
        for short, calls, ns, b in sorted(rows, key=lambda t: -t[1] * t[2]):
            k = calls / n_bwd   # launches per backward
            tot_ns += ns * k
            tot_b += b * k
            f.write("%-28s %6d %12.1f %14.1f %10.0f\n" % (short, calls, ns / 1e3, b / 1e6,
                                                          b / ns if ns else 0.0))
        f.write("\nper backward (launches per call weighted): %.0f us of kernels, %.2f GB of HBM "
                "traffic = %.2f x the algorithmic %.2f GB (x, y, dout read; dx, dy written)\n"
                % (tot_ns / 1e3, tot_b / 1e9, tot_b / alg, alg / 1e9))
        f.write("traffic = FETCH_SIZE x %.3f + WRITE_SIZE x %.3f (KiB per dispatch, scaled by a "
                "plain 1 GiB copy)\n" % (fs, ws))
    print(open(BACKWARD_TXT).read())


LAYERS_TXT = os.path.join(ROOT, "profiles", "residual-layers-2b-batched-kernel-trace.txt")
PROJ_TXT = os.path.join(ROOT, "profiles", "proj_gemm_kernel-2b-batched-kernel-trace.txt")


def _kernel_short(name):
    """'void rglru::(anonymous namespace)::proj_gemm_kernel<false, true>(rglru::ProjGemmArgs)'
    -> 'proj_gemm_kernel<false, true>'."""
    n = name.replace("(anonymous namespace)::", "")
    if n.startswith("void "):
        n = n[5:]
    depth, end = 0, len(n)
    for i, ch in enumerate(n):          # the argument list starts at the first '(' outside <>
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            end = i
            break
    return n[:end].replace("rglru::", "").replace("unsigned short", "uint16_t")


def _trace_dispatches(path):
    """(start ns, duration ns, kernel short name, workgroups) of this library's dispatches."""
    out = []
    for r in _rows(path):
        if "rglru::" not in r["Kernel_Name"]:
            continue
        wg = int(r["Workgroup_Size_X"]) * int(r["Workgroup_Size_Y"]) * int(r["Workgroup_Size_Z"])
        grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
        t0, t1 = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
        out.append((t0, t1 - t0, _kernel_short(r["Kernel_Name"]), grid // max(wg, 1)))
    out.sort()
    return out


def _stack_decode_steps(disp, anchor_groups):
    """Per-kernel time per decode step of the 26-layer stack: the dispatches between the first
    and the last-but-one step's first attention decode (anchor: attn_dec_kernel, any tile
    count, with `anchor_groups` workgroups, eight per step) span whole steps."""
    idx = [i for i, d in enumerate(disp)
           if d[2].startswith("attn_dec_kernel") and d[3] == anchor_groups]
    per_step = sum(1 for i in range(STACK_LAYERS) if i % 3 == 2)   # attention layers per step
    steps = len(idx) // per_step
    if steps < 2:
        return 0, {}
    lo, hi = idx[0], idx[(steps - 1) * per_step]
    acc = {}
    for _, ns, k, g in disp[lo:hi]:
        e = acc.setdefault((k, g), [0, 0.0])
        e[0] += 1
        e[1] += ns
    return steps - 1, acc


def trace_summary(args):
    """Kernel-trace summaries of the residual layers and the projection GEMMs from a rocprofv3
    --kernel-trace CSV of `bench.py --legs residual_layers` (no GPU): every kernel of this
    library grouped by name and grid, and the per-step kernel time of the stack's decode steps
    for 256 and for 1 sequences; written to profiles/."""
    disp = _trace_dispatches(args.kernel_trace)
    groups = {}
    for _, ns, k, g in disp:
        groups.setdefault((k, g), []).append(ns)
    w = synth.WORKLOADS[synth.BATCHED_2B]
    M, Dm = w.B * w.T, w.D
    F = synth.MLP_EXPANSION * Dm
    # large-M projections: 256 x 256 tiles over M = B T rows; the gated gate|up tiles take 128
    # features of both halves
    big = {("proj_gemm_kernel<false, false>", (M // 256) * (2 * w.D // 256)): ("x | y", 2 * w.D, Dm),
           ("proj_gemm_kernel<false, false>", (M // 256) * ((Dm + 512) // 256)): ("q | k | v", Dm + 512, Dm),
           ("proj_gemm_kernel<false, true>", (M // 256) * (F // 128)): ("MLP gate | up, gated", 2 * F, Dm)}

    def table(f, keep):
        f.write("%-44s %8s %7s %11s %11s %11s %10s\n" % ("kernel", "groups", "calls", "avg us",
                                                          "min us", "max us", "total ms"))
        for (k, g), v in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
            if keep(k):
                f.write("%-44s %8d %7d %11.1f %11.1f %11.1f %10.2f\n" % (
                    k, g, len(v), sum(v) / len(v) / 1e3, min(v) / 1e3, max(v) / 1e3, sum(v) / 1e6))

    def steps_table(f, n_seq, anchor):
        steps, acc = _stack_decode_steps(disp, anchor)
        if not steps:
            f.write("(no decode steps for %d sequences in this trace)\n" % n_seq)
            return
        tot = sum(v[1] for v in acc.values()) / steps
        f.write("\n26-layer stack, one decode step for %d sequences: kernel time per step over %d "
                "whole steps = %.0f us\n" % (n_seq, steps, tot / 1e3))
        f.write("%-44s %8s %10s %12s %12s\n" % ("kernel", "groups", "per step", "avg us",
                                                 "us per step"))
        for (k, g), (c, ns) in sorted(acc.items(), key=lambda kv: -kv[1][1]):
            f.write("%-44s %8d %10.2f %12.1f %12.1f\n" % (k, g, c / steps, ns / c / 1e3,
                                                          ns / steps / 1e3))

    def hdr(f):
        f.write("commands (from the repository root):\n")
        for c in args.commands:
            f.write("  %s\n" % c)
    with open(LAYERS_TXT, "w") as f:
        f.write("rocprofv3 kernel trace, the residual layers at the 2B widths (bf16, width %d, MLP "
                "%d)\non the %s shape (prefill of %d rows) and decode steps of the 26-layer stack\n\n"
                % (Dm, F, w.name, M))
        hdr(f)
        f.write("\nkernel_trace.csv, End - Start, every kernel of this library grouped by kernel and "
                "grid (the\nprefill leg's own rglru_prefill calls included):\n")
        table(f, lambda k: True)
        steps_table(f, 256, 256 * attn_nsplit(256))
        steps_table(f, 1, attn_nsplit(1))
        f.write("\nadd_rmsnorm_kernel (four rows per workgroup) serves a layer's first norm, the residual "
                "add fused\nwith the second norm, and the final residual add; for one decode row the "
                "norms ride in the\nrow kernel's input (gemv_rows_kernel<1, *, true>).  "
                "proj_splitk_rows_kernel (one workgroup per\nrow) adds a decode projection's split "
                "partials with the bias and the residual and writes the\nsecond norm.  The MLP's "
                "gating runs in the gate|up launch at every row count (the <*, true>\nkernels).\n")
    with open(PROJ_TXT, "w") as f:
        f.write("rocprofv3 kernel trace, the projection GEMMs at the 2B widths (bf16)\n\n")
        hdr(f)
        f.write("\nLarge M (M = %d rows): 256 x 256 tiles, proj_gemm_kernel<split K, gated>\n" % M)
        f.write("%-28s %6s %6s %7s %11s %9s\n" % ("launch", "K", "N", "calls", "avg us", "TFLOP/s"))
        for (k, g), (label, N, K) in big.items():
            v = groups.get((k, g))
            if v:
                avg = sum(v) / len(v)
                f.write("%-28s %6d %6d %7d %11.1f %9.0f\n" % (label, K, N, len(v), avg / 1e3,
                                                            2.0 * M * N * K / avg / 1e3))
        f.write("(the out-projection, o_proj and the MLP's down projection share the N = %d grid; "
                "down has\nthree times the K, so that grid's average is not one shape's)\n\n" % Dm)
        f.write("Every projection kernel (large M above; decode rows: the row kernel for one to "
                "four rows,\nthe mid-size 128 x 128 tiles for 5 to 1024, their split-K reductions):\n")
        table(f, lambda k: k.startswith("proj_") or k.startswith("gemv_rows"))
    print(open(LAYERS_TXT).read())
    print(open(PROJ_TXT).read())


def attn_nsplit(N, window=None):
    """Window splits per sequence of the attention decode (one workgroup each)."""
    W = synth.ATTN_WINDOW if window is None else window
    slots = 128 * (4 if N >= 64 else (2 if N >= 16 else 1))
    return (W + slots - 1) // slots


CENSUS_JSON = os.path.join(ROOT, "profiles", "prefill_bf16_kernel-2b-batched-census.json")
CENSUS_PASSES = [
    # (derived or base counters of one rocprofv3 --pmc pass; each fits the SQ/GRBM limits)
    ["VALUBusy", "MfmaUtil", "SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_BUSY_CYCLES"],
    ["SQ_INSTS_VALU", "SQ_INSTS_VALU_TRANS_F32", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_INSTS_SALU",
     "SQ_INSTS_VMEM", "SQ_WAVES", "SQ_LDS_BANK_CONFLICT"],
    ["SQ_WAVE_CYCLES", "SQ_ACTIVE_INST_ANY", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_WAIT_INST_LDS",
     "SQ_ACTIVE_INST_LDS", "SQ_ACTIVE_INST_VALU", "GRBM_GUI_ACTIVE"],
]


def census_summary(args):
    """Per-launch SQ counters of the prefill kernel (from rocprofv3 --pmc CSVs of the passes in
    CENSUS_PASSES) turned into per-element instruction counts, unit utilisations and the wave
    state split; written to profiles/ with the commands that produced the CSVs."""
    vals = {}
    for path in args.census:
        names = {r["Counter_Name"] for r in _rows(path) if "prefill_bf16_kernel" in r["Kernel_Name"]}
        for n in names:
            vals[n] = _mean_counter(path, "prefill_bf16_kernel", n)[0]
    w = synth.WORKLOADS[synth.BATCHED_2B]
    elems = w.B * w.T * w.D
    per_elem = lambda n: vals[n] * 64.0 / elems if n in vals else None  # wave instr x 64 lanes
    ratio = lambda a, b: vals[a] / vals[b] if a in vals and b in vals and vals[b] else None
    out = {
        "kernel": PREFILL_KERNEL, "workload": w.name, "kernel_source_hash": kernel_source_hash(),
        "elements_per_launch": elems,
        "counters_per_launch": vals,
        "valu_busy_pct": vals.get("VALUBusy"), "mfma_util_pct": vals.get("MfmaUtil"),
        "mfma_coexec_over_mfma_busy": ratio("SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_VALU_MFMA_BUSY_CYCLES"),
        "valu_instructions_per_element": per_elem("SQ_INSTS_VALU"),
        "transcendental_f32_per_element": per_elem("SQ_INSTS_VALU_TRANS_F32"),
        "mfma_instructions_per_element": per_elem("SQ_INSTS_MFMA"),
        "lds_instructions_per_element": per_elem("SQ_INSTS_LDS"),
        "salu_instructions_per_element": per_elem("SQ_INSTS_SALU"),
        "vmem_instructions_per_element": per_elem("SQ_INSTS_VMEM"),
        "wave_state": {"issuing": ratio("SQ_ACTIVE_INST_ANY", "SQ_WAVE_CYCLES"),
                       "waiting_any": ratio("SQ_WAIT_ANY", "SQ_WAVE_CYCLES"),
                       "waiting_to_issue": ratio("SQ_WAIT_INST_ANY", "SQ_WAVE_CYCLES"),
                       "waiting_lds": ratio("SQ_WAIT_INST_LDS", "SQ_WAVE_CYCLES"),
                       "valu_active": ratio("SQ_ACTIVE_INST_VALU", "SQ_WAVE_CYCLES")},
        "lds_bank_conflict_cycles_per_lds_instruction": ratio("SQ_LDS_BANK_CONFLICT", "SQ_INSTS_LDS"),
        "passes": CENSUS_PASSES, "commands": args.commands,
        "definitions": "per element = wave instructions x 64 lanes / (B T D); VALUBusy and MfmaUtil "
                       "are rocprofv3's derived counters; wave_state ratios are over SQ_WAVE_CYCLES",
    }
    with open(CENSUS_JSON, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    txt = CENSUS_JSON.replace(".json", ".txt")
    with open(txt, "w") as f:
        f.write("rocprofv3 --pmc counter census, %s on %s (bf16)\n" % (PREFILL_KERNEL, w.name))
        f.write("kernel source hash %s\n\ncommands (from the repository root):\n" %
                out["kernel_source_hash"])
        for c in args.commands:
            f.write("  %s\n" % c)
        f.write("\nper launch (mean over the profiled dispatches):\n")
        for k in sorted(vals):
            f.write("  %-30s %16.1f\n" % (k, vals[k]))
        f.write("\nderived:\n")
        for k in ("valu_busy_pct", "mfma_util_pct", "mfma_coexec_over_mfma_busy",
                  "valu_instructions_per_element", "transcendental_f32_per_element",
                  "mfma_instructions_per_element", "lds_instructions_per_element",
                  "salu_instructions_per_element", "vmem_instructions_per_element",
                  "lds_bank_conflict_cycles_per_lds_instruction"):
            v = out[k]
            f.write("  %-46s %s\n" % (k, "n/a" if v is None else "%.4g" % v))
        for k, v in out["wave_state"].items():
            f.write("  wave_state.%-36s %s\n" % (k, "n/a" if v is None else "%.3f" % v))
    print(json.dumps(out))


BACKWARD_CENSUS_TXT = os.path.join(ROOT, "profiles", "prefill_backward-2b-batched-census.txt")
BACKWARD_CENSUS_KERNELS = ("bwd_grad_kernel", "bwd_front_kernel", "bwd_conv_kernel", "bwd_wgrad_kernel",
                           "bwd_dgate_kernel")


def backward_census(args):
    """Per-launch SQ counters of the backward's largest kernels (from rocprofv3 --pmc CSVs of the
    passes in CENSUS_PASSES over `bench.py --legs backward`): per-element instruction counts, unit
    utilisations and the wave-state split of each; written to profiles/ with the commands."""
    w = synth.WORKLOADS[synth.BATCHED_2B]
    elems = w.B * w.T * w.D
    rows = []
    for kern in BACKWARD_CENSUS_KERNELS:
        vals = {}
        for path in args.census:
            names = {r["Counter_Name"] for r in _rows(path) if kern in r["Kernel_Name"]}
            for n in names:
                vals[n] = _mean_counter(path, kern, n)[0]
        per_elem = lambda n: vals[n] * 64.0 / elems if n in vals else None
        ratio = lambda a, b: vals[a] / vals[b] if a in vals and b in vals and vals[b] else None
        rows.append((kern, [
            ("VALUBusy %", vals.get("VALUBusy")), ("MfmaUtil %", vals.get("MfmaUtil")),
            ("VALU instructions per element", per_elem("SQ_INSTS_VALU")),
            ("  of them transcendental f32", per_elem("SQ_INSTS_VALU_TRANS_F32")),
            ("LDS instructions per element", per_elem("SQ_INSTS_LDS")),
            ("VMEM instructions per element", per_elem("SQ_INSTS_VMEM")),
            ("SALU instructions per element", per_elem("SQ_INSTS_SALU")),
            ("waves per launch", vals.get("SQ_WAVES")),
            ("wave state: issuing", ratio("SQ_ACTIVE_INST_ANY", "SQ_WAVE_CYCLES")),
            ("wave state: waiting at s_waitcnt", ratio("SQ_WAIT_ANY", "SQ_WAVE_CYCLES")),
            ("wave state: ready, not issued", ratio("SQ_WAIT_INST_ANY", "SQ_WAVE_CYCLES")),
            ("wave state: VALU active", ratio("SQ_ACTIVE_INST_VALU", "SQ_WAVE_CYCLES")),
            ("LDS bank-conflict cycles per LDS instruction", ratio("SQ_LDS_BANK_CONFLICT", "SQ_INSTS_LDS")),
        ]))
    with open(BACKWARD_CENSUS_TXT, "w") as f:
        f.write("rocprofv3 --pmc counter census, the path's backward kernels on %s (bf16)\n\n" % w.name)
        f.write("commands (from the repository root):\n")
        for c in args.commands:
            f.write("  %s\n" % c)
        f.write("\nper launch, mean over the profiled dispatches; per element = wave instructions x 64 "
                "lanes / (B T D) = %d elements;\nwave-state ratios over SQ_WAVE_CYCLES\n\n" % elems)
        f.write("%-46s" % "" + "".join("%18s" % k for k, _ in rows) + "\n")
        for i in range(len(rows[0][1])):
            label = rows[0][1][i][0]
            f.write("%-46s" % label)
            for _, r in rows:
                v = r[i][1]
                f.write("%18s" % ("n/a" if v is None else "%.3g" % v))
            f.write("\n")
    print(open(BACKWARD_CENSUS_TXT).read())


def measured_census():
    """MFMA and VALU utilisation of the prefill kernel from the committed census, or None when
    it was taken on other kernel sources."""
    try:
        with open(CENSUS_JSON) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("kernel_source_hash") != kernel_source_hash():
        return None
    return {"valu_busy_pct": c.get("valu_busy_pct"), "mfma_util_pct": c.get("mfma_util_pct"),
            "valu_instructions_per_element": c.get("valu_instructions_per_element"),
            "source": "profiles/" + os.path.basename(CENSUS_JSON)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="prefill headline only")
    ap.add_argument("--legs", default="all",
                    help="comma-separated extras to run (default all): prefill_2b_single, "
                         "prefill_9b_long, prefill_tiny_fp32, decode, conv1d_state_update, "
                         "block_prefill, local_attention, residual_layers, backward")
    ap.add_argument("--copy-probe", action="store_true",
                    help="time a plain 1 GiB device-to-device copy instead (counter calibration)")
    ap.add_argument("--counter-summary", action="store_true",
                    help="write profiles/ summaries from rocprofv3 CSV output (no GPU)")
    ap.add_argument("--kernel-stats")
    ap.add_argument("--kernel-trace", help="rocprofv3 kernel trace CSV: average the prefill "
                    "kernel over its last --last dispatches")
    ap.add_argument("--last", type=int, default=20)
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--copy-fetch")
    ap.add_argument("--copy-write")
    ap.add_argument("--commands", nargs="*", default=[])
    ap.add_argument("--census-summary", action="store_true",
                    help="write the SQ counter census under profiles/ from rocprofv3 CSVs (no GPU)")
    ap.add_argument("--census", nargs="*", default=[])
    ap.add_argument("--backward-census", action="store_true",
                    help="write the backward kernels' counter census from --census CSVs (no GPU)")
    ap.add_argument("--backward-summary", action="store_true",
                    help="write the backward's kernel-trace and traffic summary under profiles/ "
                         "from rocprofv3 CSVs (no GPU; --kernel-stats, --fetch, --write, "
                         "--copy-fetch, --copy-write)")
    ap.add_argument("--trace-summary", action="store_true",
                    help="write the residual-layer and projection kernel-trace summaries under "
                         "profiles/ from a rocprofv3 kernel trace CSV (--kernel-trace) of "
                         "`--legs residual_layers` (no GPU)")
    args = ap.parse_args()
    if args.trace_summary:
        trace_summary(args)
        return
    if args.backward_summary:
        backward_summary(args)
        return
    if args.backward_census:
        backward_census(args)
        return
    if args.counter_summary:
        counter_summary(args)
        return
    if args.census_summary:
        census_summary(args)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (--gpus %d "
              "requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_probe:
        copy_probe(torch)
        return
    from gated_linear_recurrence_amd import binding
    binding.load_library()
    w = synth.WORKLOADS[synth.BATCHED_2B]
    # The headline's buffers are built first and the other legs run before it, so that its W
    # warm-up and K timed calls follow GPU work directly. Started from an idle GPU (such as the
    # seconds of host-side input generation), calls 3-25 of a back-to-back prefill run at a
    # shader clock that the power management drops from 2.4 to 1.9-2.2 GHz (measured per call
    # with a clock probe); right after another leg the clock stays at ~2.43 GHz.
    headline = prepare_prefill(w, w.B, w.T, torch, binding)
    extra = {}
    legs = None if args.legs == "all" else set(args.legs.split(","))
    want = lambda leg: not args.no_extras and (legs is None or leg in legs)
    if want("prefill_2b_single"):
        w2 = synth.WORKLOADS[synth.PREFILL_2B]
        ms2 = time_prefill(w2, w2.B, w2.T, max(args.steps, 50), args.warmup, torch, binding)
        ms2f = time_prefill(w2, w2.B, w2.T, 25, args.warmup, torch, binding, flush=True)
        b2 = algorithmic_bytes(w2, w2.B, w2.T)
        extra["prefill_2b_single"] = {
            "workload": w2.name, "ms": ms2, "tokens·channels/s": w2.B * w2.T * w2.D / (ms2 * 1e-3),
            "algorithmic_GBs": b2 / (ms2 * 1e-3) / 1e9, "hbm_frac": b2 / (ms2 * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "ms_flushed": ms2f, "hbm_frac_flushed": b2 / (ms2f * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "note": "34 MB working set fits the 256 MB Infinity Cache: 'ms' is back-to-back "
                    "launches, 'ms_flushed' the median single launch after a 512 MB write"}
    # the 9B-scale long-context prefill (B=2, T=65536, D=4096, 16 heads) and the tiny fp32
    # block (B=1, T=256, D=256): same call, same roofline arithmetic.  Their inputs are built on
    # the host just before, so the GPU starts them idle: 30 warm-up calls carry the 9B leg past
    # the clock dip of the first ~25 back-to-back calls.
    for key, wk, reps, warm in (("prefill_9b_long", synth.WORKLOADS[synth.LONG_9B], max(args.steps // 2, 5), 30),
                                ("prefill_tiny_fp32", synth.WORKLOADS[synth.TINY], max(args.steps, 50), args.warmup)):
        if want(key):
            msk = time_prefill(wk, wk.B, wk.T, reps, max(warm, args.warmup), torch, binding)
            bk = algorithmic_bytes(wk, wk.B, wk.T)
            gbs = bk / (msk * 1e-3) / 1e9
            extra[key] = {
                "workload": wk.name, "ms": msk, "warmup_calls": max(warm, args.warmup),
                "tokens·channels/s": wk.B * wk.T * wk.D / (msk * 1e-3),
                "dtype": "bf16" if wk.dtype == synth.BF16 else "f32",
                "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": gbs / HBM_PEAK_GBS, "algorithmic_bytes": bk,
                             "kernel": "one rglru_prefill call (look-back reset + scan kernel)"}}
    if want("decode"):
        wd = synth.WORKLOADS[synth.DECODE_2B]
        eager_us, graph_us = time_decode(wd, wd.B, wd.T, torch, binding, split=True)
        f_eager, f_graph = time_decode(wd, wd.B, wd.T, torch, binding, split=False)
        flushed_us = time_decode(wd, wd.B, wd.T, torch, binding, split=True, flush=True)
        db = decode_bytes(wd, wd.B)
        best = graph_us if graph_us is not None else eager_us
        extra["decode"] = {"workload": wd.name, "form": "split (conv pass + gate pass, workspace)",
                          "us_per_step_graph": graph_us, "us_per_step_eager": eager_us,
                          "fused_us_per_step_graph": f_graph, "fused_us_per_step_eager": f_eager,
                          "us_per_step_flushed": flushed_us,
                          "bytes_per_step": db,
                          "hbm_frac": db / (best * 1e-6) / 1e9 / HBM_PEAK_GBS}
    if want("conv1d_state_update"):
        msc = time_conv_update(w, max(args.steps, 10), torch, binding)
        cb = conv_update_bytes(w, w.B, w.T)
        extra["conv1d_state_update"] = {
            "workload": w.name + " (conv outputs for every token, window update)", "ms": msc,
            "algorithmic_bytes": cb, "algorithmic_GBs": cb / (msc * 1e-3) / 1e9,
            "hbm_frac": cb / (msc * 1e-3) / 1e9 / HBM_PEAK_GBS}
    if want("block_prefill"):
        extra["block_prefill"] = time_block(w, max(args.steps // 2, 5), args.warmup, torch, binding)
    if want("local_attention"):
        extra["local_attention"] = time_attention(w, max(args.steps // 2, 5), args.warmup, torch,
                                                 binding)
    if want("residual_layers"):
        extra["residual_layers"] = time_layers(w, args.steps, args.warmup, torch, binding)
    if want("backward"):
        extra["backward"] = time_backward(w, max(args.steps // 4, 3), args.warmup, torch, binding)
    ms = time_prefill(w, w.B, w.T, args.steps, args.warmup, torch, binding, prepared=headline)
    tokch = w.B * w.T * w.D
    nbytes = algorithmic_bytes(w, w.B, w.T)
    achieved = nbytes / (ms * 1e-3) / 1e9
    line = {
        "metric": METRIC, "value": tokch / (ms * 1e-3), "unit": "tokens·channels/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded; x, y ~ N(0,1); random-init gate and conv weights)",
        "config": {"workload": w.name, "B": w.B, "T": w.T, "D": w.D, "gate_heads": w.H,
                   "block": w.bs, "state": "fp32", "h0_std": w.h0_std},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic(),
                     "kernel": PREFILL_KERNEL, "algorithmic_bytes": nbytes,
                     "timed": "whole rglru_prefill calls on the launch stream (HIP events): the "
                              "look-back reset kernel and the scan kernel; inputs built before "
                              "the other legs, timed right after them",
                     "census": measured_census()},
    }
    line.update(extra)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
