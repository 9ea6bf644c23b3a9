"""The allocation-free prefill (rglru_prefill_noalloc, for callers that cannot allocate device
memory) through the C ABI against rglru_prefill with a caller workspace: same kernels on the
same inputs, so the outputs must be bitwise equal; two calls in a row, the second smaller, so
state the first left in the library's static scratch cannot leak into the second; the second
also against the oracle."""
from __future__ import annotations

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
    binding.load_library()


def _case(name, B, T, D, nh, storage, seed, h0=True):
    w = synth.Workload(name, B, T, D, nh, storage, 0.9, 0.999, 0.0, seed)
    p = synth.make_params(w, biases=True)
    x, y = synth.make_act(w, "x"), synth.make_act(w, "y")
    h = np.random.default_rng(seed).normal(0, 0.5, (B, D)).astype(np.float32) if h0 else None
    c0 = synth.make_conv0(w, B)
    return w, p, x, y, h, c0


@pytest.mark.parametrize("storage", [synth.BF16, synth.F32])
def test_noalloc_matches_workspace_prefill(storage):
    from gated_linear_recurrence_amd import binding
    D, nh = (2560, 10) if storage == synth.BF16 else (256, 2)
    big = _case("noalloc-a", 4, 2000, D, nh, storage, 31)
    small = _case("noalloc-b", 2, 300, D, nh, storage, 32)
    results = []
    for w, p, x, y, h0, c0 in (big, small):
        P = H.dev_params(p, w.H)
        xd, yd, hd, cd = H.to_dev(x), H.to_dev(y), H.to_dev(h0), H.to_dev(c0)
        print("noalloc %s B=%d T=%d D=%d" % (storage, w.B, w.T, w.D), flush=True)
        got = binding.rglru_prefill_noalloc(P, xd, yd, hd, cd)
        torch.cuda.synchronize()
        ws = binding.make_workspace(P, w.B, w.T)
        ws.t.fill_(0x5A)
        ref = binding.rglru_prefill(P, xd, yd, hd, cd, workspace=ws)
        torch.cuda.synchronize()
        for g, r, what in zip(got, ref, ("out", "h_last", "conv_last")):
            assert torch.equal(g, r), (storage, w.B, w.T, what)
        results.append((w, p, x, y, h0, c0, got))
    # the second (smaller) call against the oracle as well
    w, p, x, y, h0, c0, (out, hl, cl) = results[1]
    ro, rh, rc = H.oracle.prefill(H.oracle_params(p, w.H), x, y, h0=h0, conv0=c0)
    assert H.rel_l2(H.wide(H.to_host(out)), ro) <= H.TOL[w.dtype]
    assert H.rel_l2(H.to_host(hl).astype(np.float64), rh) <= H.TOL[w.dtype]
    np.testing.assert_array_equal(H.wide(H.to_host(cl)), rc)


def test_noalloc_refuses_oversize_and_passes_empty_state():
    from gated_linear_recurrence_amd import binding
    w, p, x, y, h0, c0 = _case("noalloc-c", 2, 0, 512, 2, synth.BF16, 33)
    P = H.dev_params(p, w.H)
    xd = torch.empty((2, 0, 512), dtype=torch.bfloat16, device="cuda")
    hd, cd = H.to_dev(h0), H.to_dev(c0)
    out, hl, cl = binding.rglru_prefill_noalloc(P, xd, xd, hd, cd)
    torch.cuda.synchronize()
    assert torch.equal(hl, hd) and torch.equal(cl, cd)
    # more carry words than the static scratch holds: refused, nothing written
    wb = synth.Workload("noalloc-d", 8, 64 * 411, 2560, 10, synth.BF16, 0.9, 0.999, 0.0, 34)
    Pb = H.dev_params(synth.make_params(wb), wb.H)
    # 410 segments x 8 sequences x 2560 channels x 8 bytes > 64 MiB - 4 KiB
    assert binding.rglru_prefill_workspace_bytes(wb.B, wb.T, wb.D, wb.H, torch.bfloat16) > \
        binding.PREFILL_NOALLOC_MAX_BYTES
    xs = torch.zeros((wb.B, wb.T, wb.D), dtype=torch.bfloat16, device="cuda")
    o = torch.full_like(xs, 7.0)
    with pytest.raises(binding.RglruError, match="WORKSPACE"):
        binding.rglru_prefill_noalloc(Pb, xs, xs, out=o)
    torch.cuda.synchronize()
    assert bool((o == 7.0).all())
