"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Bars: rel-L2 <= 1e-5 for fp32 storage and <= 2e-2 for bf16 storage (fp32 state), per tensor,
for out and h_last; conv_last is a copy and must be bit-exact.  Full-size workloads are
checked on sampled (sequence, head) units, which the oracle can compute one by one because
heads are independent and outputs are causal.
"""
from __future__ import annotations

import os

import numpy as np
import pytest

import helpers as H
from gated_linear_recurrence_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_linear_recurrence_amd import binding
    binding.load_library()  # no fallback: a missing library fails here


def _run_prefill(w, p, x, y, h0=None, conv0=None, ws=None):
    from gated_linear_recurrence_amd import binding
    P = H.dev_params(p, w.H)
    xd, yd = H.to_dev(x), H.to_dev(y)
    out, h_last, conv_last = binding.rglru_prefill(P, xd, yd, H.to_dev(h0), H.to_dev(conv0),
                                                   workspace=ws)
    torch.cuda.synchronize()
    return P, out, h_last, conv_last


def _check_full(w, p, x, y, h0=None, conv0=None, label=""):
    """Whole-tensor comparison with the oracle (small and medium sizes)."""
    P, out, h_last, conv_last = _run_prefill(w, p, x, y, h0, conv0)
    ro, rh, rc = H.oracle.prefill(H.oracle_params(p, w.H), x, y, h0=h0, conv0=conv0)
    e_out = H.rel_l2(H.wide(H.to_host(out)), ro)
    e_h = H.rel_l2(H.to_host(h_last).astype(np.float64), rh)
    print("%s rel-L2 out %.3e h_last %.3e" % (label or w.name, e_out, e_h))
    tol = H.TOL[w.dtype]
    assert e_out <= tol and e_h <= tol, (e_out, e_h)
    np.testing.assert_array_equal(H.wide(H.to_host(conv_last)), rc)
    return e_out, e_h


# ------------------------------------------------------------------------------------------
# the five workloads
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("biases", [False, True])
def test_tiny_fp32_full(biases):
    w = synth.WORKLOADS[synth.TINY]
    p = synth.make_params(w, biases=biases)
    x, y = synth.make_act(w, "x"), synth.make_act(w, "y")
    _check_full(w, p, x, y, label="tiny-fp32 biases=%s" % biases)


def test_tiny_fp32_with_state():
    w = synth.WORKLOADS[synth.TINY]
    p = synth.make_params(w, biases=True)
    x, y = synth.make_act(w, "x"), synth.make_act(w, "y")
    h0 = np.random.default_rng(3).normal(0, 0.5, (w.B, w.D)).astype(np.float32)
    c0 = synth.make_conv0(w, w.B)
    _check_full(w, p, x, y, h0, c0, label="tiny-fp32 with h0, conv0")


def test_2b_prefill_full():
    w = synth.WORKLOADS[synth.PREFILL_2B]
    p = synth.make_params(w)
    x, y = synth.make_act(w, "x"), synth.make_act(w, "y")
    _check_full(w, p, x, y)


def _check_sampled(w, p, x, y, units, t_use, h0=None, label=""):
    P, out, h_last, conv_last = _run_prefill(w, p, x, y, h0)
    ref = H.oracle_units(H.oracle_params(p, w.H), x, y, units, t_use, h0=h0)
    bs = w.bs
    outh = out[:, :t_use].float().cpu().numpy() if w.dtype == synth.BF16 else \
        out[:, :t_use].cpu().numpy()
    hl = H.to_host(h_last)
    cl = H.wide(H.to_host(conv_last))
    xw = x
    worst = 0.0
    worst_seg = 0.0
    for (b, hd), (ro, rh, rc) in ref.items():
        sl = slice(hd * bs, (hd + 1) * bs)
        e = H.rel_l2(outh[b, :, sl], ro)
        worst = max(worst, e)
        assert e <= H.TOL[w.dtype], ((b, hd), e)
        # and per 64-token segment, so that one segment with a wrong carry (whose error decays
        # over the following tokens) cannot hide inside the norm over the whole sequence
        for t0 in range(0, t_use, 64):
            es = H.rel_l2(outh[b, t0:t0 + 64, sl], ro[t0:t0 + 64])
            worst_seg = max(worst_seg, es)
            assert es <= H.TOL[w.dtype], ((b, hd), t0, es)
        if t_use == w.T:
            eh = H.rel_l2(hl[b, sl].astype(np.float64), rh)
            assert eh <= H.TOL[w.dtype], ((b, hd), eh)
            np.testing.assert_array_equal(cl[b, :, sl], rc)
    print("%s sampled units %d x %d tokens: worst rel-L2 out %.3e, worst 64-token segment %.3e"
          % (label or w.name, len(units), t_use, worst, worst_seg))
    # conv_last everywhere is the last three inputs
    np.testing.assert_array_equal(cl, H.wide(xw[:, w.T - 3:]))


def test_2b_batched_full_size_sampled():
    w = synth.WORKLOADS[synth.BATCHED_2B]
    p = synth.make_params(w)
    x, y = synth.make_act(w, "x"), synth.make_act(w, "y")
    h0 = synth.make_h0(w)
    units = [(0, 0), (3, 4), (5, 9), (7, 7)]
    _check_sampled(w, p, x, y, units, w.T, h0=h0)


def test_9b_long_full_size_sampled():
    w = synth.WORKLOADS[synth.LONG_9B]
    p = synth.make_params(w)
    x, y = synth.make_act(w, "x"), synth.make_act(w, "y")
    units = [(0, 5), (1, 15)]
    _check_sampled(w, p, x, y, units, w.T)


@pytest.fixture(scope="module")
def c4_inputs():
    """The 256-sequence 2B decode workload in full: 1024 steps of x and y [256, 1024, 2560]
    (bf16), on the host and on the device, with the prefill of the same tokens."""
    from gated_linear_recurrence_amd import binding
    w = synth.WORKLOADS[synth.DECODE_2B]
    p = synth.make_params(w)
    x, y = synth.make_act(w, "x"), synth.make_act(w, "y")
    P = H.dev_params(p, w.H)
    xd, yd = H.to_dev(x), H.to_dev(y)
    pout, ph, pc = binding.rglru_prefill(P, xd, yd)
    torch.cuda.synchronize()
    return w, p, x, y, P, xd, yd, pout, ph, pc


@pytest.mark.parametrize("form", ["split", "fused"])
def test_decode_workload_matches_prefill_and_oracle(c4_inputs, form):
    """The whole 2B decode workload (256 sequences, 1024 single-token steps fed as strided
    slices, state from zero) in both decode forms: the split step with a workspace (the form
    the benchmark times) and the fused kernel.  Against the prefill of the same tokens on the
    GPU, and against the oracle on sampled (sequence, head) units: out and h within the bf16
    bar, per unit and per 64-step window; the conv window bit-exact for every sequence."""
    from gated_linear_recurrence_amd import binding
    w, p, x, y, P, xd, yd, pout, ph, pc = c4_inputs
    N, T, D = x.shape
    h = torch.zeros((N, D), dtype=torch.float32, device="cuda")
    cs = torch.zeros((N, 3, D), dtype=xd.dtype, device="cuda")
    outs = torch.empty_like(xd)
    ws = binding.make_decode_workspace(P, N) if form == "split" else None
    if ws is not None:
        ws.fill_(0x5A)  # the workspace's contents never matter
    for t in range(T):
        binding.rglru_decode_step(P, xd[:, t], yd[:, t], h, cs, out_t=outs[:, t], workspace=ws)
    torch.cuda.synchronize()
    # decode vs prefill on the GPU: same math, different fp32 evaluation order (the norms are
    # summed in fp64 on the device: the tensors are 671 M elements each)
    def rel_dev(got, ref):
        g, r = got.double(), ref.double()
        return float(torch.linalg.vector_norm(g - r) / torch.linalg.vector_norm(r))
    e = rel_dev(outs, pout)
    eh = rel_dev(h, ph)
    print("decode (%s) vs prefill, %d sequences x %d steps: rel-L2 out %.3e h %.3e"
          % (form, N, T, e, eh))
    assert e <= 1e-2 and eh <= 1e-4
    assert torch.equal(cs, pc)
    np.testing.assert_array_equal(H.to_host(cs), x[:, T - 3:])
    units = [(0, 0), (17, 3), (128, 5), (255, 9)]
    ref = H.oracle_units(H.oracle_params(p, w.H), x, y, units, T)
    hd_ = h.cpu().numpy()
    worst, worst_win = 0.0, 0.0
    for (b, hd), (ro, rh, rc) in ref.items():
        sl = slice(hd * w.bs, (hd + 1) * w.bs)
        od = outs[b, :, sl].float().cpu().numpy()
        eo = H.rel_l2(od, ro)
        assert eo <= H.TOL[w.dtype], ((b, hd), eo)
        assert H.rel_l2(hd_[b, sl], rh) <= H.TOL[w.dtype], (b, hd)
        np.testing.assert_array_equal(H.wide(H.to_host(cs[b, :, sl])), rc)
        for t0 in range(0, T, 64):
            ew = H.rel_l2(od[t0:t0 + 64], ro[t0:t0 + 64])
            assert ew <= H.TOL[w.dtype], ((b, hd), t0, ew)
            worst_win = max(worst_win, ew)
        worst = max(worst, eo)
    print("decode (%s) vs oracle on %d units: worst rel-L2 out %.3e, worst 64-step window %.3e"
          % (form, len(units), worst, worst_win))


def test_decode_fp32_against_oracle():
    from gated_linear_recurrence_amd import binding
    w = synth.small(synth.WORKLOADS[synth.TINY], B=40, T=20)
    p = synth.make_params(w, biases=True)
    x, y = synth.make_act(w, "x"), synth.make_act(w, "y")
    P = H.dev_params(p, w.H)
    xd, yd = H.to_dev(x), H.to_dev(y)
    N, T, D = x.shape
    h0 = np.random.default_rng(4).normal(0, 0.5, (N, D)).astype(np.float32)
    c0 = synth.make_conv0(w, N)
    h = H.to_dev(h0).clone()
    cs = H.to_dev(c0).clone()
    outs = torch.empty_like(xd)
    for t in range(T):
        binding.rglru_decode_step(P, xd[:, t], yd[:, t], h, cs, out_t=outs[:, t])
    torch.cuda.synchronize()
    ro, rh, rc = H.oracle.prefill(H.oracle_params(p, w.H), x, y, h0=h0, conv0=c0)
    assert H.rel_l2(outs.cpu().numpy(), ro) <= 1e-5
    assert H.rel_l2(h.cpu().numpy(), rh) <= 1e-5
    np.testing.assert_array_equal(H.to_host(cs).astype(np.float64), rc)


@pytest.mark.parametrize("split", [False, True])
@pytest.mark.parametrize("D,nh,N", [(512, 2, 45), (384, 3, 33), (2560, 10, 70), (256, 1, 1)])
def test_decode_bf16_ragged_against_oracle(D, nh, N, split):
    """bf16 decode with biases, a carried state and N not a multiple of the 32-sequence tile,
    for both gate block sizes (256 and 128): every element against the oracle, the conv window
    bit-exact, and canary bands around h, the conv window and the outputs untouched."""
    from gated_linear_recurrence_amd import binding
    T = 12
    w = synth.Workload("dec-ragged", N, T, D, nh, synth.BF16, 0.9, 0.999, 0.0, 21)
    p = synth.make_params(w, biases=True)
    x, y = synth.make_act(w, "x"), synth.make_act(w, "y")
    P = H.dev_params(p, w.H)
    xd, yd = H.to_dev(x), H.to_dev(y)
    h0 = np.random.default_rng(5).normal(0, 0.5, (N, D)).astype(np.float32)
    c0 = synth.make_conv0(w, N)
    pad = 4096
    hb = torch.full((N * D + 2 * pad,), float("nan"), device="cuda")
    cb = torch.full((3 * N * D + 2 * pad,), float("nan"), dtype=torch.bfloat16, device="cuda")
    ob = torch.full((N * T * D + 2 * pad,), float("nan"), dtype=torch.bfloat16, device="cuda")
    h = hb[pad:pad + N * D].view(N, D)
    cs = cb[pad:pad + 3 * N * D].view(N, 3, D)
    outs = ob[pad:pad + N * T * D].view(N, T, D)
    h.copy_(H.to_dev(h0))
    cs.copy_(H.to_dev(c0))
    ws, wsb = None, None
    if split:
        need = binding.rglru_decode_workspace_bytes(N, D, torch.bfloat16)
        wsb = torch.full((need + 2 * pad,), 0x5A, dtype=torch.uint8, device="cuda")
        ws = wsb[pad:pad + need]
    for t in range(T):
        binding.rglru_decode_step(P, xd[:, t], yd[:, t], h, cs, out_t=outs[:, t], workspace=ws)
    torch.cuda.synchronize()
    if split:
        assert (wsb[:pad] == 0x5A).all() and (wsb[pad + need:] == 0x5A).all()
    ro, rh, rc = H.oracle.prefill(H.oracle_params(p, w.H), x, y, h0=h0, conv0=c0)
    e_out = H.rel_l2(outs.float().cpu().numpy(), ro)
    e_h = H.rel_l2(h.cpu().numpy().astype(np.float64), rh)
    print("decode bf16 D=%d H=%d N=%d split=%s rel-L2 out %.3e h %.3e" % (D, nh, N, split, e_out, e_h))
    assert e_out <= H.TOL[synth.BF16] and e_h <= H.TOL[synth.BF16]
    np.testing.assert_array_equal(H.wide(H.to_host(cs)), rc)
    for t_, m in ((hb, N * D), (cb, 3 * N * D), (ob, N * T * D)):
        assert torch.isnan(t_[:pad].float()).all() and torch.isnan(t_[pad + m:].float()).all()


# the gate pass picks 6, 3, 1, 1, 8 and 3 waves per workgroup for these shapes on a 256-CU part
@pytest.mark.parametrize("D,nh,N", [(2560, 10, 256), (2560, 10, 100), (384, 3, 70), (512, 2, 1),
                                    (2560, 10, 1024), (1280, 10, 256)])
def test_decode_split_matches_fused(D, nh, N):
    """The split step (conv pass into the workspace, then the gate pass) and the fused kernel
    compute the same expressions on the same bf16 operands; only the order in which the MFMA
    tiles sum the K = block-width products differs (16x16x32 tiles against 32x32x16).  So over
    several steps, with biases and a carried state: the conv window is bit-identical, h agrees
    to fp32 rounding, and each output differs by at most one bf16 rounding step."""
    from gated_linear_recurrence_amd import binding
    T = 6
    w = synth.Workload("dec-split", N, T, D, nh, synth.BF16, 0.9, 0.999, 0.0, 23)
    p = synth.make_params(w, biases=True)
    x, y = synth.make_act(w, "x"), synth.make_act(w, "y")
    P = H.dev_params(p, w.H)
    xd, yd = H.to_dev(x), H.to_dev(y)
    h0 = H.to_dev(np.random.default_rng(6).normal(0, 0.5, (N, D)).astype(np.float32))
    c0 = H.to_dev(synth.make_conv0(w, N))
    ws = binding.make_decode_workspace(P, N)
    runs = []
    for workspace in (None, ws):
        h, cs = h0.clone(), c0.clone()
        outs = torch.empty_like(xd)
        for t in range(T):
            binding.rglru_decode_step(P, xd[:, t], yd[:, t], h, cs, out_t=outs[:, t],
                                      workspace=workspace)
        runs.append((outs, h, cs))
    torch.cuda.synchronize()
    (o1, h1, c1), (o2, h2, c2) = runs
    assert torch.equal(c1, c2)
    torch.testing.assert_close(h2, h1, rtol=1e-5, atol=1e-5)
    a, b = o1.float(), o2.float()
    # one bf16 step is 2^-8 of the leading power of two, at most 2^-7 of the value
    assert bool(((a - b).abs() <= a.abs() * 2.0 ** -7 + 1e-6).all())
    assert float((a != b).float().mean()) < 0.01


def test_decode_workspace_reused_across_batch_sizes():
    """One workspace, never initialised (random bytes), serves split steps of several batch
    sizes in turn (the gate pass's waves per workgroup, and so its blocks of u, change with
    the batch).  Every step must match the fused kernel (no workspace) on the same state:
    windows bit-identical, h to fp32 rounding, outputs within one bf16 step."""
    from gated_linear_recurrence_amd import binding
    D, nh, Nmax = 2560, 10, 300
    w = synth.Workload("dec-reuse", Nmax, 4, D, nh, synth.BF16, 0.9, 0.999, 0.0, 31)
    p = synth.make_params(w, biases=True)
    x, y = synth.make_act(w, "x"), synth.make_act(w, "y")
    P = H.dev_params(p, w.H)
    xd, yd = H.to_dev(x), H.to_dev(y)
    need = binding.rglru_decode_workspace_bytes(Nmax, D, torch.bfloat16)
    g = torch.Generator(device="cuda").manual_seed(5)
    ws = torch.randint(0, 256, (need,), generator=g, dtype=torch.uint8, device="cuda")
    h0 = H.to_dev(np.random.default_rng(8).normal(0, 0.5, (Nmax, D)).astype(np.float32))
    c0 = H.to_dev(synth.make_conv0(w, Nmax))
    state = {k: (h0.clone(), c0.clone()) for k in ("fused", "ws")}
    for t, N in enumerate((300, 40, 300, 1, 129)):
        outs = {}
        for k, workspace in (("fused", None), ("ws", ws)):
            h, cs = state[k]
            o = torch.empty((N, D), dtype=torch.bfloat16, device="cuda")
            binding.rglru_decode_step(P, xd[:N, t % 4], yd[:N, t % 4], h[:N], cs[:N], out_t=o,
                                      workspace=workspace)
            outs[k] = o
        torch.cuda.synchronize()
        assert torch.equal(state["fused"][1], state["ws"][1]), "window, step %d N=%d" % (t, N)
        torch.testing.assert_close(state["ws"][0], state["fused"][0], rtol=1e-5, atol=1e-5)
        a, b = outs["fused"].float(), outs["ws"].float()
        assert bool(((a - b).abs() <= a.abs() * 2.0 ** -7 + 1e-6).all()), "out, step %d N=%d" % (t, N)
        # keep both paths on the same state (their h differ by fp32 rounding)
        state["ws"] = (state["fused"][0].clone(), state["fused"][1].clone())


# ------------------------------------------------------------------------------------------
# conv-state update
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("storage,t_new", [(synth.BF16, 1), (synth.BF16, 2), (synth.BF16, 37),
                                           (synth.F32, 5), (synth.F32, 100)])
def test_conv1d_state_update(storage, t_new):
    from gated_linear_recurrence_amd import binding
    base = synth.WORKLOADS[synth.PREFILL_2B if storage == synth.BF16 else synth.TINY]
    w = synth.small(base, B=3, T=t_new)
    p = synth.make_params(w, biases=True)
    x = synth.make_act(w, "x")
    c0 = synth.make_conv0(w, 3)
    P = H.dev_params(p, w.H)
    cs = H.to_dev(c0).clone()
    u = binding.conv1d_state_update(P, H.to_dev(x), cs)
    torch.cuda.synchronize()
    win = H.wide(c0).copy()
    ru = H.oracle.conv1d_state_update(p["conv_w"], p["conv_b"], x, win)
    np.testing.assert_array_equal(H.wide(H.to_host(cs)), win)
    got = H.wide(H.to_host(u))
    if storage == synth.BF16:
        # one rounding of an fp32 sum to bf16: within one bf16 ulp of the exact value
        ulp = np.abs(ru) * 2.0 ** -7 + 1e-30
        assert np.all(np.abs(got - ru) <= ulp)
    else:
        assert H.rel_l2(got, ru) <= 1e-6


# ------------------------------------------------------------------------------------------
# edges, invariants, robustness
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("T", [1, 2, 3, 4, 5, 31, 32, 33, 63, 64, 65, 127, 128, 129, 200])
@pytest.mark.parametrize("storage", [synth.BF16, synth.F32])
def test_edge_lengths(T, storage):
    base = synth.WORKLOADS[synth.PREFILL_2B if storage == synth.BF16 else synth.TINY]
    D, nh = (512, 2) if storage == synth.BF16 else (256, 2)
    w = synth.Workload("edge", 2, T, D, nh, storage, 0.9, 0.999, 0.0, 77)
    p = synth.make_params(w, biases=True)
    x, y = synth.make_act(w, "x"), synth.make_act(w, "y")
    h0 = np.random.default_rng(T).normal(0, 0.5, (2, D)).astype(np.float32)
    c0 = synth.make_conv0(w, 2)
    _check_full(w, p, x, y, h0, c0, label="edge T=%d %s" % (T, storage))


def test_empty_sequence_passes_state_through():
    from gated_linear_recurrence_amd import binding
    w = synth.Workload("edge", 2, 0, 512, 2, synth.BF16, 0.9, 0.999, 0.0, 5)
    p = synth.make_params(w)
    P = H.dev_params(p, w.H)
    x = torch.empty((2, 0, 512), dtype=torch.bfloat16, device="cuda")
    h0 = torch.randn((2, 512), device="cuda")
    c0 = torch.randn((2, 3, 512), device="cuda").to(torch.bfloat16)
    out, hl, cl = binding.rglru_prefill(P, x, x, h0, c0)
    torch.cuda.synchronize()
    assert out.shape == (2, 0, 512)
    assert torch.equal(hl, h0) and torch.equal(cl, c0)


def test_bs128_bf16():
    w = synth.Workload("bs128", 2, 300, 384, 3, synth.BF16, 0.9, 0.999, 0.0, 8)
    p = synth.make_params(w, biases=True)
    x, y = synth.make_act(w, "x"), synth.make_act(w, "y")
    _check_full(w, p, x, y)


def test_bs256_fp32():
    w = synth.Workload("bs256f", 1, 150, 512, 2, synth.F32, 0.9, 0.999, 0.0, 9)
    p = synth.make_params(w, biases=True)
    x, y = synth.make_act(w, "x"), synth.make_act(w, "y")
    _check_full(w, p, x, y)


def test_split_prefill_hands_over_state():
    from gated_linear_recurrence_amd import binding
    w = synth.small(synth.WORKLOADS[synth.TINY], B=2, T=300)
    p = synth.make_params(w, biases=True)
    x, y = synth.make_act(w, "x"), synth.make_act(w, "y")
    P = H.dev_params(p, w.H)
    xd, yd = H.to_dev(x), H.to_dev(y)
    out, hl, cl = binding.rglru_prefill(P, xd, yd)
    o1, h1, c1 = binding.rglru_prefill(P, xd[:, :130].contiguous(), yd[:, :130].contiguous())
    o2, h2, c2 = binding.rglru_prefill(P, xd[:, 130:].contiguous(), yd[:, 130:].contiguous(), h1, c1)
    torch.cuda.synchronize()
    assert H.rel_l2(torch.cat([o1, o2], 1).cpu().numpy(), out.cpu().numpy()) <= 1e-6
    assert H.rel_l2(h2.cpu().numpy(), hl.cpu().numpy()) <= 1e-6
    assert torch.equal(c2, cl)


def test_in_place_state():
    from gated_linear_recurrence_amd import binding
    for T in (2, 200):
        w = synth.Workload("inplace", 2, T, 512, 2, synth.BF16, 0.9, 0.999, 0.0, 10)
        p = synth.make_params(w, biases=True)
        x, y = synth.make_act(w, "x"), synth.make_act(w, "y")
        h0 = np.random.default_rng(1).normal(0, 0.5, (2, 512)).astype(np.float32)
        c0 = synth.make_conv0(w, 2)
        P = H.dev_params(p, w.H)
        xd, yd = H.to_dev(x), H.to_dev(y)
        ref_out, ref_h, ref_c = binding.rglru_prefill(P, xd, yd, H.to_dev(h0), H.to_dev(c0))
        hs, cs = H.to_dev(h0).clone(), H.to_dev(c0).clone()
        out, _, _ = binding.rglru_prefill(P, xd, yd, hs, cs, h_last=hs, conv_last=cs)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(hs, ref_h) and torch.equal(cs, ref_c)


def test_deterministic_and_workspace_reuse():
    """Bitwise repeatable; one workspace reused across shapes gives the fresh-workspace bits."""
    from gated_linear_recurrence_amd import binding
    w = synth.WORKLOADS[synth.PREFILL_2B]
    p = synth.make_params(w)
    x, y = synth.make_act(w, "x"), synth.make_act(w, "y")
    P = H.dev_params(p, w.H)
    xd, yd = H.to_dev(x), H.to_dev(y)
    ws = binding.make_workspace(P, 1, w.T)
    a1, h1, _ = binding.rglru_prefill(P, xd, yd, workspace=ws)
    s1, hs1, _ = binding.rglru_prefill(P, xd[:, :700].contiguous(), yd[:, :700].contiguous(),
                                       workspace=ws)
    a2, h2, _ = binding.rglru_prefill(P, xd, yd, workspace=ws)
    s2, hs2, _ = binding.rglru_prefill(P, xd[:, :700].contiguous(), yd[:, :700].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(a1, a2) and torch.equal(h1, h2)
    assert torch.equal(s1, s2) and torch.equal(hs1, hs2)
    assert ws.flags() == 0


@pytest.mark.parametrize("storage", [synth.BF16, synth.F32])
def test_workspace_needs_no_initialisation(storage):
    """Every prefill call prepares its own look-back state on the stream, so the workspace's
    previous contents never matter: buffers filled with 0x5A, 0x00 (every word reads as a ready
    aggregate A = B = 0), 0x3F (ready aggregates A = B = 0.75) or 0xFF, and one left by calls
    of other lengths, all give the oracle's result and bitwise the fresh-workspace output, with
    no error flag."""
    from gated_linear_recurrence_amd import binding
    D, nh = (512, 2) if storage == synth.BF16 else (256, 2)
    w = synth.Workload("wsfresh", 4, 1000, D, nh, storage, 0.9, 0.999, 0.0, 12)
    p = synth.make_params(w, biases=True)
    x, y = synth.make_act(w, "x"), synth.make_act(w, "y")
    P = H.dev_params(p, w.H)
    xd, yd = H.to_dev(x), H.to_dev(y)
    ws = binding.make_workspace(P, w.B, w.T)
    ws.t.fill_(0x5A)
    ref, ref_h, _ = binding.rglru_prefill(P, xd, yd, workspace=ws)
    torch.cuda.synchronize()
    ro, rh, _ = H.oracle.prefill(H.oracle_params(p, w.H), x, y)
    assert H.rel_l2(H.wide(H.to_host(ref)), ro) <= H.TOL[w.dtype]
    assert H.rel_l2(H.to_host(ref_h).astype(np.float64), rh) <= H.TOL[w.dtype]
    for fill in (0x00, 0x3F, 0xFF):
        ws.t.fill_(fill)
        out, hl, _ = binding.rglru_prefill(P, xd, yd, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(out, ref) and torch.equal(hl, ref_h), "fill 0x%02X" % fill
    for rep in range(6):
        T = w.T if rep % 2 == 0 else 700
        out, _, _ = binding.rglru_prefill(P, xd[:, :T].contiguous(), yd[:, :T].contiguous(),
                                          workspace=ws)
        torch.cuda.synchronize()
        if T == w.T:
            assert torch.equal(out, ref)
    assert ws.flags() == 0


def test_outputs_stay_in_bounds():
    """Canary bands around out/h_last/conv_last are untouched; the workspace gets no errors."""
    from gated_linear_recurrence_amd import binding
    w = synth.Workload("canary", 3, 150, 512, 2, synth.BF16, 0.9, 0.999, 0.0, 11)
    p = synth.make_params(w)
    x, y = synth.make_act(w, "x"), synth.make_act(w, "y")
    P = H.dev_params(p, w.H)
    pad = 4096
    n = 3 * 150 * 512
    buf = torch.full((n + 2 * pad,), float("nan"), dtype=torch.bfloat16, device="cuda")
    hb = torch.full((3 * 512 + 2 * pad,), float("nan"), device="cuda")
    cb = torch.full((9 * 512 + 2 * pad,), float("nan"), dtype=torch.bfloat16, device="cuda")
    out = buf[pad:pad + n].view(3, 150, 512)
    hl = hb[pad:pad + 3 * 512].view(3, 512)
    cl = cb[pad:pad + 9 * 512].view(3, 3, 512)
    ws = binding.make_workspace(P, 3, 150)
    binding.rglru_prefill(P, H.to_dev(x), H.to_dev(y), out=out, h_last=hl, conv_last=cl,
                          workspace=ws)
    torch.cuda.synchronize()
    for t, m in ((buf, n), (hb, 3 * 512), (cb, 9 * 512)):
        assert torch.isnan(t[:pad].float()).all() and torch.isnan(t[pad + m:].float()).all()
        assert not torch.isnan(t[pad:pad + m].float()).any()
    assert ws.flags() == 0
