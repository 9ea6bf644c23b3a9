"""Pins for the fp64 oracle (CPU only).

The pages print no worked numeric example for this path, so the oracle is
pinned by what mathematics fixes: closed forms with exactly known values,
library routines for the sub-steps (numpy.convolve, a dense block-diagonal
matmul, torch's tanh-GELU), exact rational brute force for the scan algebra,
and invariants of the recurrence (decode == prefill, causality, head
independence, state hand-over).  Each ``_pin_*`` function takes an oracle
library handle so that ``test_planted_mistakes_are_caught`` can run the same
pins against deliberately broken copies of the oracle and show that each
plausible mistake fails at least one of them.
"""
from __future__ import annotations

import fractions
import itertools
import math
import os
import re
import shutil
import subprocess
import tempfile

import numpy as np
import pytest
import scipy.linalg

import oracle
from gated_linear_recurrence_amd import synth

F = fractions.Fraction


# ----------------------------------------------------------------------------------------------
# small helpers (input construction only; no arithmetic of the method)
# ----------------------------------------------------------------------------------------------
def _params(D, H, dtype="f32", seed=0, biases=True, **over):
    rng = np.random.default_rng(seed)
    bs = D // H
    p = {
        "conv_w": rng.normal(0, 0.5, (D, 4)).astype(np.float32),
        "conv_b": rng.normal(0, 0.5, D).astype(np.float32) if biases else np.zeros(D, np.float32),
        "wa": rng.normal(0, 1 / math.sqrt(bs), (H, bs, bs)).astype(np.float32),
        "ba": rng.normal(0, 0.5, D).astype(np.float32) if biases else np.zeros(D, np.float32),
        "wx": rng.normal(0, 1 / math.sqrt(bs), (H, bs, bs)).astype(np.float32),
        "bx": rng.normal(0, 0.5, D).astype(np.float32) if biases else np.zeros(D, np.float32),
        "lambda": np.log(1 / (1 / rng.uniform(0.9, 0.999, D) - 1)).astype(np.float32),
    }
    p.update(over)
    if dtype == "bf16":
        for k in ("conv_w", "conv_b", "wa", "ba", "wx", "bx"):
            p[k] = synth.round_bf16(p[k])
    return p


def _P(p, H):
    return oracle.Params(p["conv_w"], p["conv_b"], p["wa"], p["ba"], p["wx"], p["bx"], p["lambda"], H)


def _acts(B, T, D, dtype="f32", seed=1):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, T, D)).astype(np.float32)
    y = rng.standard_normal((B, T, D)).astype(np.float32)
    if dtype == "bf16":
        return synth.round_bf16(x), synth.round_bf16(y)
    return x, y


def _wide(a):
    a = np.asarray(a)
    return oracle.widen_bf16(a).astype(np.float64) if a.dtype == np.uint16 else a.astype(np.float64)


# ----------------------------------------------------------------------------------------------
# widening
# ----------------------------------------------------------------------------------------------
def test_widen_bf16_exact():
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0000, 0x8000, 0x7F7F], np.uint16)
    want = np.array([1.0, -2.0, 1.0078125, 0.0, -0.0, 3.3895313892515355e38])
    np.testing.assert_array_equal(oracle.widen_bf16(bits).astype(np.float64), want)


def test_round_bf16_is_rne():
    # ties go to even; values chosen on exact bf16 midpoints
    f = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 1.0 + 2 ** -8 + 2 ** -20],
                 np.float32)
    got = oracle.widen_bf16(synth.round_bf16(f)).astype(np.float64)
    np.testing.assert_array_equal(got, [1.0, 1.0 + 2 ** -6, -1.0, 1.0 + 2 ** -7])


# ----------------------------------------------------------------------------------------------
# conv (depthwise, causal, kernel 4)
# ----------------------------------------------------------------------------------------------
def _pin_conv_matches_numpy_convolve(lib):
    rng = np.random.default_rng(5)
    N, T, D = 2, 11, 6
    w = rng.normal(0, 0.5, (D, 4)).astype(np.float32)
    b = rng.normal(0, 0.5, D).astype(np.float32)
    x = rng.standard_normal((N, T, D)).astype(np.float32)
    c0 = rng.standard_normal((N, 3, D)).astype(np.float32)
    win = c0.astype(np.float64).copy()
    u = oracle.conv1d_state_update(w, b, x, win, lib=lib)
    for n in range(N):
        for c in range(D):
            seq = np.concatenate([c0[n, :, c], x[n, :, c]]).astype(np.float64)
            want = np.convolve(seq, w[c, ::-1].astype(np.float64))[3:3 + T] + float(b[c])
            np.testing.assert_allclose(u[n, :, c], want, rtol=1e-13, atol=1e-13)
    # the state is the last three inputs, oldest first
    np.testing.assert_array_equal(win, x[:, T - 3:, :].astype(np.float64))


def _pin_conv_unit_taps(lib):
    # w = e_j moves x by 3-j tokens; the first 3-j outputs come from the carried state
    rng = np.random.default_rng(6)
    T, D = 9, 4
    x = rng.standard_normal((1, T, D)).astype(np.float32)
    c0 = rng.standard_normal((1, 3, D)).astype(np.float32)
    for j in range(4):
        w = np.zeros((D, 4), np.float32)
        w[:, j] = 1.0
        win = c0.astype(np.float64).copy()
        u = oracle.conv1d_state_update(w, None, x, win, lib=lib)
        full = np.concatenate([c0[0], x[0]]).astype(np.float64)  # index 3 is token 0
        np.testing.assert_array_equal(u[0], full[j:j + T])


def _pin_conv_short_update(lib):
    # fewer than 3 new tokens: the window shifts and keeps older state
    rng = np.random.default_rng(7)
    D = 5
    c0 = rng.standard_normal((2, 3, D)).astype(np.float32)
    for t_new in (0, 1, 2):
        x = rng.standard_normal((2, t_new, D)).astype(np.float32)
        win = c0.astype(np.float64).copy()
        oracle.conv1d_state_update(np.ones((D, 4), np.float32), None, x, win, lib=lib)
        want = np.concatenate([c0, x], axis=1)[:, -3:, :]
        np.testing.assert_array_equal(win, want.astype(np.float64))


def test_conv_matches_numpy_convolve(oracle_lib):
    _pin_conv_matches_numpy_convolve(oracle_lib)


def test_conv_unit_taps(oracle_lib):
    _pin_conv_unit_taps(oracle_lib)


def test_conv_short_update(oracle_lib):
    _pin_conv_short_update(oracle_lib)


def test_conv_bf16_widening():
    rng = np.random.default_rng(8)
    D, T = 8, 7
    w = synth.round_bf16(rng.normal(0, 0.5, (D, 4)).astype(np.float32))
    x = synth.round_bf16(rng.standard_normal((1, T, D)).astype(np.float32))
    win = np.zeros((1, 3, D))
    u = oracle.conv1d_state_update(w, None, x, win)
    wf, xf = _wide(w), _wide(x)
    for c in range(D):
        want = np.convolve(np.concatenate([np.zeros(3), xf[0, :, c]]), wf[c, ::-1])[3:3 + T]
        np.testing.assert_allclose(u[0, :, c], want, rtol=1e-14, atol=1e-14)


# ----------------------------------------------------------------------------------------------
# gates: block-diagonal projections
# ----------------------------------------------------------------------------------------------
def _pin_gates_block_diagonal(lib):
    rng = np.random.default_rng(9)
    D, H, n = 12, 3, 5
    bs = D // H
    wa = rng.standard_normal((H, bs, bs)).astype(np.float32)  # not symmetric
    wx = rng.standard_normal((H, bs, bs)).astype(np.float32)
    ba = rng.standard_normal(D).astype(np.float32)
    bx = rng.standard_normal(D).astype(np.float32)
    u = rng.standard_normal((n, D))
    ra, ri = oracle.gate_preacts(wa, ba, wx, bx, u, H, lib=lib)
    # each head block is a Linear weight [out][in]: pre = u @ block_diag(W_h^T) + b
    Ma = scipy.linalg.block_diag(*[wa[h].astype(np.float64).T for h in range(H)])
    Mx = scipy.linalg.block_diag(*[wx[h].astype(np.float64).T for h in range(H)])
    np.testing.assert_allclose(ra, u @ Ma + ba, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(ri, u @ Mx + bx, rtol=1e-12, atol=1e-12)


def test_gates_block_diagonal(oracle_lib):
    _pin_gates_block_diagonal(oracle_lib)


# ----------------------------------------------------------------------------------------------
# decay and normaliser: exactly known values
# ----------------------------------------------------------------------------------------------
def _pin_step_exact_values(lib):
    ln3 = math.log(3.0)
    # Lambda = 0 -> sigmoid = 1/2; ra = ln 3 -> r = 3/4 -> a = (1/2)^6 = 1/64; ri = ln 3 -> i = 3/4
    h, u = 0.37, -1.3
    a = 1 / 64
    m = math.sqrt(4095) / 64
    want = a * h + m * 0.75 * u
    got = oracle.rglru_step(0.0, ln3, ln3, u, h, lib=lib)
    assert abs(got - want) <= 1e-14 * max(1.0, abs(want)), (got, want)
    # Lambda = ln 3 -> sigmoid = 3/4; ra = 0 -> r = 1/2 -> a = (3/4)^4 = 81/256; ri = -ln 3 -> i = 1/4
    a = 81 / 256
    m = math.sqrt(65536 - 6561) / 256
    want = a * h + m * 0.25 * u
    got = oracle.rglru_step(ln3, 0.0, -ln3, u, h, lib=lib)
    assert abs(got - want) <= 1e-14 * max(1.0, abs(want)), (got, want)


def _pin_step_limits(lib):
    # r -> 0: a = sigmoid(Lambda)^0 = 1 and sqrt(1 - a^2) = 0, so the state is held exactly
    for lam in (-3.0, 0.5, 6.9):
        assert oracle.rglru_step(lam, -200.0, 0.3, 2.5, 0.8125, lib=lib) == 0.8125
    # a -> 0 (Lambda = -100, r ~ 1): the state is the gated input i*u
    i = 1.0 / (1.0 + math.exp(-0.7))
    got = oracle.rglru_step(-100.0, 20.0, 0.7, -1.75, 123.0, lib=lib)
    assert abs(got - i * -1.75) <= 1e-15, got


def test_step_exact_values(oracle_lib):
    _pin_step_exact_values(oracle_lib)


def test_step_limits(oracle_lib):
    _pin_step_limits(oracle_lib)


# ----------------------------------------------------------------------------------------------
# GELU (tanh form)
# ----------------------------------------------------------------------------------------------
def _pin_gelu(lib):
    import torch

    assert oracle.gelu_tanh(0.0, lib=lib) == 0.0
    ys = np.linspace(-7.0, 7.0, 57)
    for v in ys:
        # exact identity of the tanh form: gelu(y) - gelu(-y) = y
        d = oracle.gelu_tanh(v, lib=lib) - oracle.gelu_tanh(-v, lib=lib)
        assert abs(d - v) <= 1e-14 * max(1.0, abs(v)), (v, d)
    got = np.array([oracle.gelu_tanh(v, lib=lib) for v in ys])
    want = torch.nn.functional.gelu(torch.tensor(ys, dtype=torch.float64), approximate="tanh").numpy()
    np.testing.assert_allclose(got, want, rtol=1e-14, atol=1e-15)


def test_gelu(oracle_lib):
    _pin_gelu(oracle_lib)


# ----------------------------------------------------------------------------------------------
# scan: geometric series (closed form) through the whole prefill
# ----------------------------------------------------------------------------------------------
def _pin_geometric_series(lib):
    # W = 0 and constant biases make every gate constant; identity conv taps make u = x;
    # constant x then gives h_t = a^(t+1) h0 + v (1 - a^(t+1)) / (1 - a), v = sqrt(1-a^2) i X.
    D, H, T = 4, 2, 60
    bs = D // H
    ln3 = math.log(3.0)
    sig = np.array([0.99, 0.9, 0.5, 0.75])
    p = {
        "conv_w": np.tile(np.array([0, 0, 0, 1], np.float32), (D, 1)),
        "conv_b": np.zeros(D, np.float32),
        "wa": np.zeros((H, bs, bs), np.float32), "wx": np.zeros((H, bs, bs), np.float32),
        "ba": np.full(D, ln3, np.float32), "bx": np.full(D, -ln3, np.float32),
        "lambda": np.log(sig / (1 - sig)).astype(np.float32),
    }
    X = 0.625
    x = np.full((1, T, D), X, np.float32)
    yv = np.full((1, T, D), 1.5, np.float32)
    h0 = np.array([[0.5, -2.0, 1.0, 0.25]], np.float32)
    out, h_last, _ = oracle.prefill(_P(p, H), x, yv, h0=h0, lib=lib)
    # the biases are stored in fp32, so r and i are 3/4 and 1/4 up to that rounding
    r = 1.0 / (1.0 + math.exp(-float(p["ba"][0])))
    i = 1.0 / (1.0 + math.exp(-float(p["bx"][0])))
    assert abs(r - 0.75) < 1e-7 and abs(i - 0.25) < 1e-7
    # Lambda is stored in fp32, so use the stored value's sigmoid
    s = 1.0 / (1.0 + np.exp(-p["lambda"].astype(np.float64)))
    a = s ** (8 * r)
    v = np.sqrt(1 - a * a) * i * X
    t = np.arange(T)[:, None] + 1
    h = a ** t * h0[0].astype(np.float64) + v * (1 - a ** t) / (1 - a)
    g = 0.5 * 1.5 * (1 + math.tanh(math.sqrt(2 / math.pi) * (1.5 + 0.044715 * 1.5 ** 3)))
    np.testing.assert_allclose(out[0], h * g, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(h_last[0], h[-1], rtol=1e-12, atol=1e-13)


def test_geometric_series(oracle_lib):
    _pin_geometric_series(oracle_lib)


def test_exact_special_case_values():
    """Rational s, r, i whose decay a = s**(8r) is exact (tests/golden/closed_forms.txt)."""
    u, h = -1.3, 0.37
    for s, r, i, a in _read_golden("closed_forms.txt"):
        s, r, i, a = (float(F(v)) for v in (s, r, i, a))
        lam, ra, ri = (math.log(q / (1 - q)) for q in (s, r, i))
        want = a * h + math.sqrt(1 - a * a) * i * u
        got = oracle.rglru_step(lam, ra, ri, u, h)
        assert abs(got - want) <= 1e-13 * max(1.0, abs(want)), (s, r, i, a, got, want)


def _read_golden(name):
    path = os.path.join(os.path.dirname(__file__), "golden", name)
    rows = []
    with open(path) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


# ----------------------------------------------------------------------------------------------
# associative scan == sequential scan, exactly, for every bracketing (T <= 6)
# ----------------------------------------------------------------------------------------------
def _combine(e1, e2):
    """(A1, B1) then (A2, B2): h -> A2 (A1 h + B1) + B2."""
    return (e1[0] * e2[0], e2[0] * e1[1] + e2[1])


def _all_bracketings(elems):
    if len(elems) == 1:
        yield elems[0]
        return
    for k in range(1, len(elems)):
        for left in _all_bracketings(elems[:k]):
            for right in _all_bracketings(elems[k:]):
                yield _combine(left, right)


def test_associative_scan_brute_force():
    rng = np.random.default_rng(11)
    for T in range(1, 7):
        a = [F(int(rng.integers(1, 30)), 31) for _ in range(T)]
        v = [F(int(rng.integers(-20, 20)), int(rng.integers(1, 9))) for _ in range(T)]
        h0 = F(3, 7)
        h = h0
        for t in range(T):
            h = a[t] * h + v[t]
        elems = [(a[t], v[t]) for t in range(T)]
        results = {_combine((F(0), h0), e) for e in _all_bracketings(elems)}
        assert results == {(F(0), h)}, T
        # chunked: local scans from zero, then carry-in fix-up h_t = b_t + p_t * carry
        for chunk in range(1, T + 1):
            carry = h0
            for c0 in range(0, T, chunk):
                bl, pl = F(0), F(1)
                for t in range(c0, min(T, c0 + chunk)):
                    bl, pl = a[t] * bl + v[t], pl * a[t]
                carry = bl + pl * carry
            assert carry == h


# ----------------------------------------------------------------------------------------------
# whole-path invariants
# ----------------------------------------------------------------------------------------------
def _pin_decode_equals_prefill(lib):
    D, H, T, B = 16, 2, 13, 3
    for dtype in ("f32", "bf16"):
        p = _params(D, H, dtype, seed=21)
        P = _P(p, H)
        x, y = _acts(B, T, D, dtype, seed=22)
        h0 = np.random.default_rng(23).normal(0, 0.3, (B, D)).astype(np.float32)
        c0 = _acts(B, 3, D, dtype, seed=24)[0]
        out, h_last, conv_last = oracle.prefill(P, x, y, h0=h0, conv0=c0, lib=lib)
        h = h0.astype(np.float64).copy()
        win = _wide(c0).copy()
        for t in range(T):
            o = oracle.decode_step(P, x[:, t], y[:, t], h, win, lib=lib)
            np.testing.assert_array_equal(o, out[:, t])
        np.testing.assert_array_equal(h, h_last)
        np.testing.assert_array_equal(win, conv_last)
        np.testing.assert_array_equal(conv_last, _wide(x[:, T - 3:]))


def _pin_causality_and_heads(lib):
    D, H, T = 16, 2, 12
    bs = D // H
    p = _params(D, H, seed=31)
    P = _P(p, H)
    x, y = _acts(1, T, D, seed=32)
    out, _, _ = oracle.prefill(P, x, y, lib=lib)
    t0 = 7
    x2 = x.copy()
    x2[0, t0] += 1.0
    out2, _, _ = oracle.prefill(P, x2, y, lib=lib)
    np.testing.assert_array_equal(out2[0, :t0], out[0, :t0])
    assert np.all(np.abs(out2[0, t0] - out[0, t0]) > 0)
    x3 = x.copy()
    x3[0, :, bs:] += 0.5   # perturb head 1 only
    out3, _, _ = oracle.prefill(P, x3, y, lib=lib)
    np.testing.assert_array_equal(out3[0, :, :bs], out[0, :, :bs])
    assert np.all(np.abs(out3[0, 3:, bs:] - out[0, 3:, bs:]) > 0)


def _pin_unit_matches_full(lib):
    D, H, T, B = 16, 2, 10, 2
    bs = D // H
    p = _params(D, H, "bf16", seed=41)
    P = _P(p, H)
    x, y = _acts(B, T, D, "bf16", seed=42)
    h0 = np.random.default_rng(43).normal(0, 0.3, (B, D)).astype(np.float32)
    out, h_last, _ = oracle.prefill(P, x, y, h0=h0, lib=lib)
    for b in range(B):
        for hd in range(H):
            ou, he, ce = oracle.prefill_unit(P, x, y, b, hd, 6, h0=h0, lib=lib)
            np.testing.assert_array_equal(ou, out[b, :6, hd * bs:(hd + 1) * bs])
            ou, he, ce = oracle.prefill_unit(P, x, y, b, hd, T, h0=h0, lib=lib)
            np.testing.assert_array_equal(he, h_last[b, hd * bs:(hd + 1) * bs])
            np.testing.assert_array_equal(ce, _wide(x[b, T - 3:, hd * bs:(hd + 1) * bs]))


def _pin_empty_sequence(lib):
    D, H = 8, 2
    P = _P(_params(D, H, seed=51), H)
    x = np.zeros((2, 0, D), np.float32)
    h0 = np.arange(2 * D, dtype=np.float32).reshape(2, D)
    c0 = np.arange(2 * 3 * D, dtype=np.float32).reshape(2, 3, D)
    out, h_last, conv_last = oracle.prefill(P, x, x, h0=h0, conv0=c0, lib=lib)
    assert out.shape == (2, 0, D)
    np.testing.assert_array_equal(h_last, h0)
    np.testing.assert_array_equal(conv_last, c0)


# ----------------------------------------------------------------------------------------------
# the dense projections around the path (Linear layers) and the composed block
# ----------------------------------------------------------------------------------------------
def _shift(n):
    """Cyclic shift as a Linear weight [out][in]: output j takes input (j + 1) mod n."""
    w = np.zeros((n, n), np.float32)
    w[np.arange(n), (np.arange(n) + 1) % n] = 1.0
    return w


def _pin_linear_library(lib):
    """A Linear layer equals numpy's fp64 matmul x @ W^T + b (W stored [out][in])."""
    rng = np.random.default_rng(71)
    x = rng.standard_normal((6, 40)).astype(np.float32)
    w = rng.standard_normal((24, 40)).astype(np.float32)
    b = rng.standard_normal(24).astype(np.float32)
    ref = x.astype(np.float64) @ w.astype(np.float64).T + b.astype(np.float64)
    np.testing.assert_allclose(oracle.linear(x, w, b, lib=lib), ref, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(oracle.linear(x, w, None, lib=lib), ref - b, rtol=1e-13, atol=1e-13)
    xb = synth.round_bf16(x)
    wb = synth.round_bf16(w)
    refb = _wide(xb) @ _wide(wb).T
    np.testing.assert_allclose(oracle.linear(xb, wb, None, lib=lib), refb, rtol=1e-13, atol=1e-13)


def _pin_linear_exact(lib):
    """Exact special cases: identity, a cyclic shift (orientation), a zero weight (bias only)."""
    x = np.arange(-12, 12, dtype=np.float32).reshape(3, 8) * 0.25
    n = x.shape[1]
    np.testing.assert_array_equal(oracle.linear(x, np.eye(n, dtype=np.float32), lib=lib), x)
    np.testing.assert_array_equal(oracle.linear(x, _shift(n), lib=lib), np.roll(x, -1, axis=1))
    b = np.linspace(-1, 1, 5).astype(np.float32)
    np.testing.assert_array_equal(oracle.linear(x, np.zeros((5, n), np.float32), b, lib=lib),
                                  np.broadcast_to(b.astype(np.float64), (3, 5)))


def _proj(lx_w, ly_w, lo_w, lx_b=None, ly_b=None, lo_b=None):
    return oracle.ProjParams(lx_w, lx_b, ly_w, ly_b, lo_w, lo_b)


def _pin_block_composition(lib):
    """With linear_x = I, linear_y = 2 I and linear_out = a cyclic shift plus a bias, the block
    is exactly the path on (x, 2x), shifted, plus the bias."""
    D, H, B, T = 16, 2, 2, 11
    P = _P(_params(D, H, seed=81), H)
    x, _ = _acts(B, T, D, seed=82)
    h0 = np.random.default_rng(83).normal(0, 0.3, (B, D)).astype(np.float32)
    c0 = np.random.default_rng(84).normal(0, 1.0, (B, 3, D)).astype(np.float32)
    c = np.linspace(-2, 2, D).astype(np.float32)
    q = _proj(np.eye(D, dtype=np.float32), 2 * np.eye(D, dtype=np.float32), _shift(D), lo_b=c)
    out, h_last, conv_last = oracle.block_prefill(P, q, x, h0=h0, conv0=c0, lib=lib)
    po, ph, pc = oracle.prefill(P, x, 2 * x, h0=h0, conv0=c0, lib=lib)
    np.testing.assert_array_equal(out, np.roll(po, -1, axis=2) + c.astype(np.float64))
    np.testing.assert_array_equal(h_last, ph)
    np.testing.assert_array_equal(conv_last, pc)


def _pin_block_rectangular(lib):
    """Block width Dm != path width D, random small-integer projections (every intermediate of
    the projections is exact in fp32): the block equals numpy's matmuls around the path."""
    D, H, Dm, B, T = 16, 2, 24, 2, 9
    rng = np.random.default_rng(91)
    P = _P(_params(D, H, seed=92), H)
    x = rng.integers(-2, 3, (B, T, Dm)).astype(np.float32)
    lx_w = rng.integers(-1, 2, (D, Dm)).astype(np.float32)
    ly_w = rng.integers(-1, 2, (D, Dm)).astype(np.float32) * 0.25
    lo_w = rng.standard_normal((Dm, D)).astype(np.float32)
    lx_b = rng.integers(-3, 4, D).astype(np.float32)
    ly_b = rng.integers(-3, 4, D).astype(np.float32) * 0.5
    lo_b = rng.standard_normal(Dm).astype(np.float32)
    q = _proj(lx_w, ly_w, lo_w, lx_b, ly_b, lo_b)
    out, h_last, conv_last = oracle.block_prefill(P, q, x, lib=lib)
    xw = x.astype(np.float64)
    xb = (xw @ lx_w.astype(np.float64).T + lx_b).astype(np.float32)
    yb = (xw @ ly_w.astype(np.float64).T + ly_b).astype(np.float32)
    po, ph, pc = oracle.prefill(P, xb, yb, lib=lib)
    ref = po @ lo_w.astype(np.float64).T + lo_b.astype(np.float64)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(h_last, ph)
    np.testing.assert_array_equal(conv_last, pc)


def test_linear_matches_numpy(oracle_lib):
    _pin_linear_library(oracle_lib)


def test_linear_exact_cases(oracle_lib):
    _pin_linear_exact(oracle_lib)


def test_block_composition(oracle_lib):
    _pin_block_composition(oracle_lib)


def test_block_rectangular(oracle_lib):
    _pin_block_rectangular(oracle_lib)


def test_block_empty_sequence(oracle_lib):
    D, H, Dm = 8, 2, 16
    P = _P(_params(D, H, seed=95), H)
    rng = np.random.default_rng(96)
    q = _proj(rng.standard_normal((D, Dm)).astype(np.float32),
              rng.standard_normal((D, Dm)).astype(np.float32),
              rng.standard_normal((Dm, D)).astype(np.float32))
    h0 = np.arange(2 * D, dtype=np.float32).reshape(2, D)
    c0 = np.arange(2 * 3 * D, dtype=np.float32).reshape(2, 3, D)
    out, h_last, conv_last = oracle.block_prefill(P, q, np.zeros((2, 0, Dm), np.float32), h0=h0,
                                                  conv0=c0, lib=oracle_lib)
    assert out.shape == (2, 0, Dm)
    np.testing.assert_array_equal(h_last, h0)
    np.testing.assert_array_equal(conv_last, c0)


# ----------------------------------------------------------------------------------------------
# local sliding-window multi-query attention and the rotary position embedding
# ----------------------------------------------------------------------------------------------
def _pin_rope_complex(lib):
    """RoPE turns the pair (v_i, v_{i+dh/2}) as the complex number v_i + j v_{i+dh/2} times
    exp(j pos 10000^(-2i/dh)) (numpy's complex exponential, not the oracle's cos/sin loop)."""
    rng = np.random.default_rng(101)
    dh, half = 16, 8
    v = rng.standard_normal((5, dh))
    pos = np.array([0.0, 1.0, 7.0, 100.0, 2047.0])
    z = (v[:, :half] + 1j * v[:, half:]) * np.exp(
        1j * pos[:, None] * 10000.0 ** (-2.0 * np.arange(half) / dh))
    ref = np.concatenate([z.real, z.imag], axis=1)
    np.testing.assert_allclose(oracle.rope(v, pos, lib=lib), ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(oracle.rope(v[:1], [0.0], lib=lib), v[:1])


def _pin_rope_relative(lib):
    """After RoPE, q_m . k_n depends on m - n only."""
    rng = np.random.default_rng(102)
    q, k = rng.standard_normal((1, 32)), rng.standard_normal((1, 32))
    d1 = float((oracle.rope(q, [10.0], lib=lib) @ oracle.rope(k, [3.0], lib=lib).T)[0, 0])
    d2 = float((oracle.rope(q, [1007.0], lib=lib) @ oracle.rope(k, [1000.0], lib=lib).T)[0, 0])
    assert abs(d1 - d2) < 1e-9 * (1.0 + abs(d1))
    d3 = float((oracle.rope(q, [11.0], lib=lib) @ oracle.rope(k, [3.0], lib=lib).T)[0, 0])
    assert abs(d3 - d1) > 1e-6


def _pin_mqa_closed_forms(lib):
    rng = np.random.default_rng(103)
    T, Hq, dh, W = 12, 3, 8, 4
    q = rng.standard_normal((T, Hq, dh))
    k = rng.standard_normal((T, dh))
    v = rng.standard_normal((T, dh))
    # window 1: every query sees only its own token
    np.testing.assert_array_equal(oracle.local_mqa(q, k, v, 1, lib=lib),
                                  np.broadcast_to(v[:, None, :], (T, Hq, dh)))
    # zero queries: equal weights over the window, so the mean of the window's values
    o = oracle.local_mqa(np.zeros_like(q), k, v, W, lib=lib)
    ref = np.stack([v[max(0, t - W + 1):t + 1].mean(0) for t in range(T)])
    np.testing.assert_allclose(o[:, 1], ref, rtol=1e-13, atol=1e-13)
    # two tokens: the newer one's weight is the logistic of the scaled score difference
    q2 = rng.standard_normal((2, 1, dh))
    o2 = oracle.local_mqa(q2, k[:2], v[:2], 2, lib=lib)
    w1 = 1.0 / (1.0 + math.exp(-float(q2[1, 0] @ (k[1] - k[0])) / math.sqrt(dh)))
    np.testing.assert_allclose(o2[1, 0], v[0] + w1 * (v[1] - v[0]), rtol=1e-12, atol=1e-12)


def _pin_mqa_invariants(lib):
    rng = np.random.default_rng(104)
    T, Hq, dh, W = 20, 2, 8, 5
    q = rng.standard_normal((T, Hq, dh))
    k = rng.standard_normal((T, dh))
    v = rng.standard_normal((T, dh))
    o = oracle.local_mqa(q, k, v, W, lib=lib)
    t0 = 9
    # tokens after t0, and tokens older than its window, do not change o[t0]
    for s_ in (t0 + 1, t0 - W):
        k2, v2 = k.copy(), v.copy()
        k2[s_] += 3.0
        v2[s_] -= 2.0
        np.testing.assert_array_equal(oracle.local_mqa(q, k2, v2, W, lib=lib)[t0], o[t0])
    # the oldest token inside the window does
    k3 = k.copy()
    k3[t0 - W + 1] += 3.0
    assert np.all(np.abs(oracle.local_mqa(q, k3, v, W, lib=lib)[t0] - o[t0]) > 0)
    # a component shared by every key shifts all scores of a query alike: no change
    u = rng.standard_normal(dh)
    np.testing.assert_allclose(oracle.local_mqa(q, k + u, v, W, lib=lib), o, rtol=1e-11,
                               atol=1e-12)
    # the heads share keys and values: equal queries give equal outputs
    q4 = q.copy()
    q4[:, 1] = q4[:, 0]
    o4 = oracle.local_mqa(q4, k, v, W, lib=lib)
    np.testing.assert_array_equal(o4[:, 1], o4[:, 0])


def _pin_attention_block_composition(lib):
    """Two heads, block width != head width, small-integer projections (exact in fp32): the
    block equals numpy's projections around the pinned RoPE and attention."""
    rng = np.random.default_rng(105)
    B, T, Dm, Hq, dh, W = 2, 11, 24, 2, 8, 4
    x = rng.integers(-2, 3, (B, T, Dm)).astype(np.float32)
    wq = rng.integers(-1, 2, (Hq * dh, Dm)).astype(np.float32)
    wk = rng.integers(-1, 2, (dh, Dm)).astype(np.float32)
    wv = rng.integers(-1, 2, (dh, Dm)).astype(np.float32)
    wo = rng.standard_normal((Dm, Hq * dh)).astype(np.float32)
    bo = rng.standard_normal(Dm).astype(np.float32)
    out = oracle.local_attention_block(x, wq, wk, wv, wo, bo, Hq, W, lib=lib)
    pos = np.arange(T, dtype=np.float64)
    for b in range(B):
        xb = x[b].astype(np.float64)
        q = xb @ wq.astype(np.float64).T
        k = oracle.rope(xb @ wk.astype(np.float64).T, pos, lib=lib)
        v = xb @ wv.astype(np.float64).T
        qr = np.stack([oracle.rope(q[:, h * dh:(h + 1) * dh], pos, lib=lib) for h in range(Hq)], 1)
        o = oracle.local_mqa(qr, k, v, W, lib=lib).reshape(T, Hq * dh)
        np.testing.assert_allclose(out[b], o @ wo.astype(np.float64).T + bo, rtol=1e-11, atol=1e-11)


def test_rope_complex(oracle_lib):
    _pin_rope_complex(oracle_lib)


def test_rope_relative(oracle_lib):
    _pin_rope_relative(oracle_lib)


def test_mqa_closed_forms(oracle_lib):
    _pin_mqa_closed_forms(oracle_lib)


def test_mqa_invariants(oracle_lib):
    _pin_mqa_invariants(oracle_lib)


def test_attention_block_composition(oracle_lib):
    _pin_attention_block_composition(oracle_lib)


def test_decode_equals_prefill(oracle_lib):
    _pin_decode_equals_prefill(oracle_lib)


def test_causality_and_head_independence(oracle_lib):
    _pin_causality_and_heads(oracle_lib)


def test_unit_matches_full(oracle_lib):
    _pin_unit_matches_full(oracle_lib)


def test_empty_sequence(oracle_lib):
    _pin_empty_sequence(oracle_lib)


def test_split_prefill_hands_over_state(oracle_lib):
    D, H, T1, T2 = 16, 2, 9, 8
    P = _P(_params(D, H, seed=61), H)
    x, y = _acts(2, T1 + T2, D, seed=62)
    out, h_last, conv_last = oracle.prefill(P, x, y)
    o1, h1, c1 = oracle.prefill(P, x[:, :T1], y[:, :T1])
    o2, h2, c2 = oracle.prefill(P, x[:, T1:], y[:, T1:], h0=h1.astype(np.float32),
                                conv0=c1.astype(np.float32))
    np.testing.assert_array_equal(o1, out[:, :T1])
    # the hand-over rounds the state to fp32 (the library's state type)
    np.testing.assert_allclose(o2, out[:, T1:], rtol=1e-6, atol=1e-6)
    np.testing.assert_allclose(h2, h_last, rtol=1e-6, atol=1e-6)
    np.testing.assert_array_equal(c2, conv_last)


def test_variance_is_sane():
    """Sanity (not a pin): unit-variance inputs keep the state's variance O(1)."""
    w = synth.small(synth.WORKLOADS[synth.TINY], T=512)
    p = synth.make_params(w)
    x = synth.make_act(w, "x")
    y = synth.make_act(w, "y")
    P = _P(p, w.H)
    lib = oracle.load()
    _, h_end, _ = oracle.prefill_unit(P, x, y, 0, 0, 512, lib=lib)
    assert 0.05 < float(np.var(h_end)) < 20.0


# ----------------------------------------------------------------------------------------------
# the residual layer: RMSNorm, gated MLP, composition
# ----------------------------------------------------------------------------------------------
def _pin_rmsnorm_closed_forms(lib):
    """RMSNorm against closed forms (eps = 0 unless stated):
    - alternating +a, -a: the root mean square is |a|, so the output is +-g exactly;
    - one nonzero entry v of D: the root mean square is |v| / sqrt(D), so that entry becomes
      sign(v) sqrt(D) g_j and the rest stay 0;
    - a constant row c with eps: c / sqrt(c^2 + eps) g (0.5 and eps 0.25 give g / sqrt(2));
    - scaling a row by a power of two changes nothing, and with g = 1 the output's mean square
      is 1; bf16 inputs give the same as their exact fp64 values."""
    D = 8
    g = np.array([1.0, 2.0, 0.5, -1.0, 3.0, 1.5, 0.25, 4.0], np.float32)
    x = np.array([[3.0, -3.0] * 4, [-0.5, 0.5] * 4])
    out = oracle.rmsnorm(x, g, 0.0, lib=lib)
    assert np.array_equal(out, np.sign(x) * g.astype(np.float64))
    x = np.zeros((1, D))
    x[0, 5] = -7.0
    out = oracle.rmsnorm(x, g, 0.0, lib=lib)
    want = np.zeros((1, D))
    want[0, 5] = -np.sqrt(D) * 1.5
    assert np.allclose(out, want, rtol=1e-15, atol=0)
    out = oracle.rmsnorm(np.full((1, D), 0.5), g, 0.25, lib=lib)
    assert np.allclose(out, g / np.sqrt(2.0), rtol=1e-15, atol=0)
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 64))
    ones = np.ones(64, np.float32)
    a = oracle.rmsnorm(x, ones, 0.0, lib=lib)
    b = oracle.rmsnorm(x * 4.0, ones, 0.0, lib=lib)
    assert np.array_equal(a, b)
    assert np.allclose((a * a).mean(axis=1), 1.0, rtol=1e-13, atol=0)
    xb = synth.round_bf16(x.astype(np.float32))
    assert np.array_equal(oracle.rmsnorm(xb, ones, 1e-6, lib=lib),
                          oracle.rmsnorm(oracle.widen_bf16(xb).astype(np.float64), ones, 1e-6,
                                         lib=lib))


def _pin_mlp_integer_exact(lib):
    """The gated MLP on integers where GELU-tanh is exactly the identity (pre-activations of 10
    or more: tanh rounds to 1 in fp64, which the pin checks first): then
    out = b_d + W_d ((W_g x + b_g) * (W_u x + b_u)) exactly, against numpy's integer matmul.
    The up branch takes small values of both signs, on which GELU is far from the identity.
    With the up branch zero, the output is the down bias alone."""
    assert oracle.gelu_tanh(10.0, lib=lib) == 10.0 and oracle.gelu_tanh(17.0, lib=lib) == 17.0
    rng = np.random.default_rng(4)
    rows, Dm, F = 6, 8, 12
    x = rng.integers(0, 3, (rows, Dm)).astype(np.float32)
    wg = rng.integers(0, 2, (F, Dm)).astype(np.float32)
    bg = np.full(F, 10.0, np.float32)
    wu = rng.integers(-2, 3, (F, Dm)).astype(np.float32)
    bu = rng.integers(-3, 4, F).astype(np.float32)
    wd = rng.integers(-2, 3, (Dm, F)).astype(np.float32)
    bd = rng.integers(-5, 6, Dm).astype(np.float32)
    m = oracle.MlpParams(wg, bg, wu, bu, wd, bd)
    out = oracle.mlp(m, x, lib=lib)
    xi = x.astype(np.int64)
    gate = xi @ wg.astype(np.int64).T + bg.astype(np.int64)
    up = xi @ wu.astype(np.int64).T + bu.astype(np.int64)
    assert gate.min() >= 10 and up.min() < 0 < up.max()
    want = (gate * up) @ wd.astype(np.int64).T + bd.astype(np.int64)
    assert np.array_equal(out, want.astype(np.float64))
    z = oracle.MlpParams(wg, bg, np.zeros_like(wu), np.zeros_like(bu), wd, bd)
    assert np.array_equal(oracle.mlp(z, x, lib=lib), np.broadcast_to(bd.astype(np.float64), x.shape))


def _pin_residual_layer_composition(lib):
    """The residual layer around a temporal block whose output is known exactly: with the
    recurrent block's linear_out weights zero and its bias c, the block gives c for every token,
    so h = x + c exactly, and out must be h + MLP(RMSNorm_2(h)) with the pinned MLP and RMSNorm
    applied to that h (not to x).  The same holds for the local-attention block with o_proj
    zero.  The blocks also take fp64 inputs (as inside the layer) exactly like storage ones."""
    rng = np.random.default_rng(6)
    w = synth.small(synth.WORKLOADS[synth.TINY], B=2, T=9)
    Dm, F = 256, 64
    p = synth.make_params(w, biases=True)
    q = synth.make_proj(w, Dm=Dm, biases=True)
    c = rng.standard_normal(Dm).astype(np.float32)
    P = oracle.Params(p["conv_w"], p["conv_b"], p["wa"], p["ba"], p["wx"], p["bx"], p["lambda"], w.H)
    Qz = oracle.ProjParams(q["lx_w"], q["lx_b"], q["ly_w"], q["ly_b"], np.zeros_like(q["lo_w"]), c)
    x = rng.standard_normal((2, 9, Dm)).astype(np.float32)
    g1 = (1.0 + 0.1 * rng.standard_normal(Dm)).astype(np.float32)
    g2 = (1.0 + 0.1 * rng.standard_normal(Dm)).astype(np.float32)
    m = oracle.MlpParams(*(rng.standard_normal(s).astype(np.float32) / 8
                           for s in ((F, Dm), F, (F, Dm), F, (Dm, F), Dm)))
    out, h = oracle.residual_layer(x, lambda xn: oracle.block_prefill(P, Qz, xn, lib=lib)[0],
                                   g1, g2, m, lib=lib)
    hw = x.astype(np.float64) + c.astype(np.float64)
    assert np.array_equal(h, hw)
    assert np.array_equal(out, hw + oracle.mlp(m, oracle.rmsnorm(hw, g2, lib=lib), lib=lib))
    # the attention block with o_proj zero and bias c
    Hq, dh = 1, 16
    wq, wk, wv = (rng.standard_normal((n, Dm)).astype(np.float32) / 16 for n in (Hq * dh, dh, dh))
    out2, h2 = oracle.residual_layer(
        x, lambda xn: oracle.local_attention_block(xn, wq, wk, wv, np.zeros((Dm, Hq * dh), np.float32),
                                                   c, Hq, 4, lib=lib), g1, g2, m, lib=lib)
    assert np.array_equal(h2, hw) and np.array_equal(out2, out)
    # fp64 inputs to the blocks equal their storage inputs
    Q = oracle.ProjParams(q["lx_w"], q["lx_b"], q["ly_w"], q["ly_b"], q["lo_w"], q["lo_b"])
    a = oracle.block_prefill(P, Q, x, lib=lib)[0]
    b = oracle.block_prefill(P, Q, x.astype(np.float64), lib=lib)[0]
    assert np.array_equal(a, b)
    wo = rng.standard_normal((Dm, Hq * dh)).astype(np.float32) / 4
    a = oracle.local_attention_block(x, wq, wk, wv, wo, c, Hq, 4, lib=lib)
    b = oracle.local_attention_block(x.astype(np.float64), wq, wk, wv, wo, c, Hq, 4, lib=lib)
    assert np.array_equal(a, b)


# ----------------------------------------------------------------------------------------------
# backward pass of the path
# ----------------------------------------------------------------------------------------------
def _pin_backward_finite_differences(lib):
    """The backward oracle against central differences of the (pinned) forward oracle, for
    L = sum(dout * out) + sum(dh_last * h_last), on a tiny block (D = 8, two heads of 4, six
    tokens, with state), at three sampled elements of each of the eleven inputs.  fp32
    storage; the step is 1e-3 and the difference is divided by the exact step between the two
    fp32 values, so the truncation error (~1e-7 relative) stays far below the bar (2e-5).
    Also: the gradients are linear in (dout, dh_last), exactly so under doubling, and vanish
    with them."""
    rng = np.random.default_rng(11)
    B, T, D, H = 2, 6, 8, 2
    bs = D // H

    def f(*s, sc=1.0):
        return (rng.standard_normal(s) * sc).astype(np.float32)

    lam = np.log(rng.uniform(0.9, 0.99, D) / (1 - rng.uniform(0.9, 0.99, D))).astype(np.float32)
    ins = {"conv_w": f(D, 4, sc=0.5), "conv_b": f(D, sc=0.3), "wa": f(H, bs, bs, sc=0.5),
           "ba": f(D, sc=0.3), "wx": f(H, bs, bs, sc=0.5), "bx": f(D, sc=0.3), "lambda": lam,
           "x": f(B, T, D), "y": f(B, T, D), "h0": f(B, D, sc=0.3), "conv0": f(B, 3, D)}
    dout = rng.standard_normal((B, T, D))
    dhl = rng.standard_normal((B, D))

    def params(v):
        return oracle.Params(v["conv_w"], v["conv_b"], v["wa"], v["ba"], v["wx"], v["bx"],
                             v["lambda"], H)

    def loss(v):
        o, hl, _ = oracle.prefill(params(v), v["x"], v["y"], h0=v["h0"], conv0=v["conv0"], lib=lib)
        return float((o * dout).sum() + (hl * dhl).sum())

    g = oracle.prefill_backward(params(ins), ins["x"], ins["y"], dout, h0=ins["h0"],
                                conv0=ins["conv0"], dh_last=dhl, lib=lib)
    names = {"conv_w": "dconv_w", "conv_b": "dconv_b", "wa": "dwa", "ba": "dba", "wx": "dwx",
             "bx": "dbx", "lambda": "dlambda", "x": "dx", "y": "dy", "h0": "dh0",
             "conv0": "dconv0"}
    for name, gname in names.items():
        a = ins[name]
        for idx in [tuple(rng.integers(0, n) for n in a.shape) for _ in range(3)]:
            vp = {k: v.copy() for k, v in ins.items()}
            vm = {k: v.copy() for k, v in ins.items()}
            vp[name][idx] += np.float32(1e-3)
            vm[name][idx] -= np.float32(1e-3)
            step = float(vp[name][idx]) - float(vm[name][idx])
            fd = (loss(vp) - loss(vm)) / step
            an = g[gname][idx]
            assert abs(fd - an) <= 2e-5 * abs(an) + 1e-6, (name, idx, fd, an)
    g2 = oracle.prefill_backward(params(ins), ins["x"], ins["y"], 2 * dout, h0=ins["h0"],
                                 conv0=ins["conv0"], dh_last=2 * dhl, lib=lib)
    for k in g:
        assert np.array_equal(g2[k], 2 * g[k]), k
    g0 = oracle.prefill_backward(params(ins), ins["x"], ins["y"], np.zeros_like(dout),
                                 h0=ins["h0"], conv0=ins["conv0"], lib=lib)
    for k in g0:
        assert not np.any(g0[k]), k


# ----------------------------------------------------------------------------------------------
# planted mistakes: each plausible error in the oracle must fail at least one pin
# ----------------------------------------------------------------------------------------------
PINS = [
    _pin_conv_matches_numpy_convolve, _pin_conv_unit_taps, _pin_conv_short_update,
    _pin_gates_block_diagonal, _pin_step_exact_values, _pin_step_limits, _pin_gelu,
    _pin_geometric_series, _pin_decode_equals_prefill, _pin_causality_and_heads,
    _pin_unit_matches_full, _pin_empty_sequence,
    _pin_linear_library, _pin_linear_exact, _pin_block_composition, _pin_block_rectangular,
    _pin_rope_complex, _pin_rope_relative, _pin_mqa_closed_forms, _pin_mqa_invariants,
    _pin_attention_block_composition,
    _pin_rmsnorm_closed_forms, _pin_mlp_integer_exact, _pin_residual_layer_composition,
    _pin_backward_finite_differences,
]

MUTANTS = {
    "transposed gate weight": ("const size_t widx = ((size_t)hd * bs + j) * bs + k;",
                               "const size_t widx = ((size_t)hd * bs + k) * bs + j;"),
    "reversed conv taps": ("(size_t)c * 4 + 0, p->dtype) * win[0]", "(size_t)c * 4 + 3, p->dtype) * win[0]"),
    "tap on the wrong input": ("(size_t)c * 4 + 3, p->dtype) * xt", "(size_t)c * 4 + 3, p->dtype) * win[2]"),
    "dropped sqrt": ("const double m = sqrt(1.0 - a * a);", "const double m = 1.0 - a * a;"),
    "dropped normaliser": ("return a * h_prev + m * (i * u);", "return a * h_prev + (i * u);"),
    "dropped input gate": ("return a * h_prev + m * (i * u);", "return a * h_prev + m * u;"),
    "c = 1": ("pow(sigmoid(lambda), 8.0 * r)", "pow(sigmoid(lambda), 1.0 * r)"),
    "sigmoid sign": ("return 1.0 / (1.0 + exp(-z));", "return 1.0 / (1.0 + exp(z));"),
    "gelu cubic coefficient": ("0.044715 * y * y * y", "0.04715 * y * y * y"),
    "gelu half": ("return 0.5 * y * (1.0 +", "return y * (1.0 +"),
    "window shift": ("win[0] = win[1];\n    win[1] = win[2];", "win[0] = win[2];\n    win[1] = win[1];"),
    "gate bias dropped": ("double sa = p->ba ? widen(p->ba, ch, p->dtype) : 0.0;", "double sa = 0.0;"),
    "conv bias dropped": ("double acc = p->conv_b ? widen(p->conv_b, (size_t)c, p->dtype) : 0.0;",
                          "double acc = 0.0;"),
    "state not carried": ("h[c] = rglru_step((double)p->lambda[ch], ra[c], ri[c], u[c], h[c]);",
                          "h[c] = rglru_step((double)p->lambda[ch], ra[c], ri[c], u[c], 0.0);"),
    "gelu on the wrong branch": ("out[(size_t)t * bs + c] = h[c] * oracle_gelu_tanh(yt);",
                                 "out[(size_t)t * bs + c] = h[c] * oracle_gelu_tanh(u[c]);"),
    "lambda index": ("rglru_step((double)p->lambda[ch]", "rglru_step((double)p->lambda[c]"),
    "bf16 widening": ("uint32_t bits = (uint32_t)((const uint16_t *)base)[idx] << 16;",
                      "uint32_t bits = (uint32_t)((const uint16_t *)base)[idx] << 15;"),
    "h0 ignored": ("h[c] = h0 ? (double)h0[(size_t)b * D + ch] : 0.0;", "h[c] = 0.0;"),
    "linear weight transposed": ("widen(w, (size_t)n * K + k, wdtype)", "widen(w, (size_t)k * N + n, wdtype)"),
    "linear bias dropped": ("double s = b ? widen(b, (size_t)n, wdtype) : 0.0;", "double s = 0.0;"),
    "linear input row": ("widen(in, (size_t)m * K + k, xdtype)", "widen(in, (size_t)k, xdtype)"),
    "branches swapped": ("linear_rows(B * T, Dm, D, x_in, xdtype, lx_w, lx_b, dtype, xb);",
                         "linear_rows(B * T, Dm, D, x_in, xdtype, ly_w, ly_b, dtype, xb);"),
    "output projection skips the path": (
        "linear_rows(B * T, D, Dm, mg, ORACLE_F64, lo_w, lo_b, dtype, out);",
        "linear_rows(B * T, D, Dm, xb, ORACLE_F64, lo_w, lo_b, dtype, out);"),
    "rope pairs neighbours": ("const double a = v[i], b = v[i + half];",
                              "const double a = v[2 * i], b = v[2 * i + 1];"),
    "rope sign": ("v[i] = a * c - b * s;", "v[i] = a * c + b * s;"),
    "rope frequency": ("pow(base, -2.0 * (double)i / (double)dh)",
                       "pow(base, -1.0 * (double)i / (double)dh)"),
    "rope position of k": ("rope_head(k + (size_t)t * dh, dh, (double)t, base);",
                           "rope_head(k + (size_t)t * dh, dh, (double)(t + 1), base);"),
    "window one too wide": ("const int s0 = t - W + 1 > 0 ? t - W + 1 : 0;",
                            "const int s0 = t - W > 0 ? t - W : 0;"),
    "scores not scaled": ("score[s] = d * scale;", "score[s] = d;"),
    "output projection on q": ("linear_rows(T, DQ, Dm, o, ORACLE_F64, wo, bo, dtype, out + xoff);",
                               "linear_rows(T, DQ, Dm, q, ORACLE_F64, wo, bo, dtype, out + xoff);"),
    "rmsnorm sum instead of mean": ("sqrt(ss / (double)D + eps)", "sqrt(ss + eps)"),
    "rmsnorm eps outside the root": ("1.0 / sqrt(ss / (double)D + eps)", "1.0 / (sqrt(ss / (double)D) + eps)"),
    "rmsnorm scale dropped": ("* inv * widen(g, d, wdtype)", "* inv"),
    "mlp activation on the up branch": ("gt[i] = oracle_gelu_tanh(gt[i]) * up[i];",
                                        "gt[i] = gt[i] * oracle_gelu_tanh(up[i]);"),
    "mlp up branch dropped": ("gt[i] = oracle_gelu_tanh(gt[i]) * up[i];",
                              "gt[i] = oracle_gelu_tanh(gt[i]);"),
    "mlp down bias dropped": ("linear_rows(rows, F, Dm, gt, ORACLE_F64, dw, db, wdtype, out);",
                              "linear_rows(rows, F, Dm, gt, ORACLE_F64, dw, NULL, wdtype, out);"),
    "backward carry without the decay": ("dh[c] = g * a[k];", "dh[c] = g;"),
    "backward drops the normaliser's decay term": ("const double da = g * h[k] - dm * a[k] / m[k];",
                                                   "const double da = g * h[k];"),
    "backward lambda factor": ("dlambda[ch] += da * a[k] * 8.0 * r[k] * (1.0 - sg);",
                               "dlambda[ch] += da * a[k] * 8.0 * r[k] * sg;"),
    "backward gate weights not transposed": (
        "duv[kk] += widen(p.wa, widx, p.dtype) * dra[j] +",
        "duv[kk] += widen(p.wa, ((size_t)hd * bs + kk) * bs + j, p.dtype) * dra[j] +"),
    "backward conv position": ("const int pos = t - 3 + j;", "const int pos = t - j;"),
    "backward gelu derivative": ("(1.0 + 3.0 * 0.044715 * y * y)", "(1.0 + 0.044715 * y * y)"),
    "block input type ignored": ("linear_rows(T, Dm, DQ, xb, xdtype, wq, NULL, dtype, q);",
                                 "linear_rows(T, Dm, DQ, xb, dtype, wq, NULL, dtype, q);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes_are_caught(name, tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    src = open(oracle._SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) >= 1, "mutant pattern not found: %s" % name
    mutated = src.replace(old, new)
    path = tmp_path / "mutant.c"
    path.write_text(mutated)
    so = str(tmp_path / "libmutant.so")
    oracle.build(str(path), so)
    lib = oracle.load(so)
    failed = []
    for pin in PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError):
            failed.append(pin.__name__)
    assert failed, "no pin caught the planted mistake '%s'" % name


def test_workloads_follow_printed_shapes():
    """The 2B workloads use the widths and conv shape printed on the RecurrentGemma page."""
    kv = {k: v for k, v in _read_golden("recurrent_block_shapes.txt")}
    for name in (synth.PREFILL_2B, synth.BATCHED_2B, synth.DECODE_2B):
        w = synth.WORKLOADS[name]
        assert w.D == int(kv["rnn_width"]) == int(kv["conv_channels"]) == int(kv["conv_groups"])
    # kernel 4 with padding 3 on both sides gives T + 3 outputs; keeping the first T is causal
    assert int(kv["conv_kernel"]) - 1 == int(kv["conv_padding"]) == 3
    assert kv["gelu"] == "tanh"
