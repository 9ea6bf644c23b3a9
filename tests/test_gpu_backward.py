"""GPU parity of the path's backward pass (rglru_prefill_backward) through the C ABI against the
fp64 oracle (itself pinned by finite differences of the forward oracle).

Bar: every gradient tensor meets the bf16 bar, rel-L2 <= 2e-2.  The kernels round u, the gate
pre-activations and their gradients to bf16 where they feed the matrix cores (as the forward
rounds u); sums over tokens (weights, biases, Lambda) are fp32 in a fixed order.  At full size the
output gradient is nonzero only on the first 512 tokens of one sequence: every gradient then
comes from that sequence's first 512 tokens, which the oracle computes.
"""
from __future__ import annotations

import dataclasses

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


def _compare(g, ref, label):
    worst = 0.0
    for k, r in ref.items():
        got = H.to_host(g[k])
        got = H.wide(got) if got.dtype == np.uint16 else got.astype(np.float64)
        e = H.rel_l2(got.reshape(r.shape), r)
        print("%s %-8s rel-L2 %.3e" % (label, k, e))
        worst = max(worst, e)
        assert e <= H.TOL[synth.BF16], (k, e)
    return worst


@pytest.mark.parametrize("D,nh,B,T,state", [
    (512, 2, 2, 128, True),      # two heads, with h0, conv0 and dh_last
    (256, 1, 4, 64, False),      # one chunk per sequence
    (2560, 10, 1, 256, True),    # the 2B widths
    (256, 1, 8, 96, True),       # T = 96: the front pass's last unit of each sequence has 32 tokens
    (256, 1, 8, 32, False),      # one 32-token unit per sequence
])
def test_backward_matches_oracle(D, nh, B, T, state):
    from gated_linear_recurrence_amd import binding
    w = dataclasses.replace(synth.small(synth.WORKLOADS[synth.PREFILL_2B], B=B, T=T), D=D, H=nh)
    p = synth.make_params(w, biases=True)
    x, y = synth.make_act(w, "x"), synth.make_act(w, "y")
    rng = np.random.default_rng(D + B + T)
    dout = synth.round_bf16(rng.standard_normal((B, T, D)).astype(np.float32))
    h0 = c0 = dhl = None
    if state:
        h0 = rng.normal(0, 0.3, (B, D)).astype(np.float32)
        c0 = synth.make_conv0(w, B)
        dhl = rng.standard_normal((B, D)).astype(np.float32)
    g = binding.rglru_prefill_backward(H.dev_params(p, w.H), H.to_dev(x), H.to_dev(y),
                                       H.to_dev(dout), H.to_dev(h0), H.to_dev(c0), H.to_dev(dhl))
    torch.cuda.synchronize()
    ref = H.oracle.prefill_backward(H.oracle_params(p, w.H), x, y, H.wide(dout), h0=h0, conv0=c0,
                                    dh_last=None if dhl is None else dhl.astype(np.float64))
    _compare(g, ref, "backward D=%d B=%d T=%d" % (D, B, T))


def test_backward_deterministic():
    from gated_linear_recurrence_amd import binding
    w = dataclasses.replace(synth.small(synth.WORKLOADS[synth.PREFILL_2B], B=2, T=128), D=512, H=2)
    p = synth.make_params(w, biases=True)
    P = H.dev_params(p, w.H)
    x, y = H.to_dev(synth.make_act(w, "x")), H.to_dev(synth.make_act(w, "y"))
    dout = torch.randn((2, 128, 512), device="cuda").to(torch.bfloat16)
    g1 = binding.rglru_prefill_backward(P, x, y, dout)
    g2 = binding.rglru_prefill_backward(P, x, y, dout)
    torch.cuda.synchronize()
    for k in g1:
        assert torch.equal(g1[k], g2[k]), k


def test_backward_2b_batched_full_size_one_window():
    """The batched 2B shape (8 x 8192 tokens, width 2560) at full size, with the output gradient
    nonzero only on tokens 0..511 of sequence 5: gradients of the other sequences and of later
    tokens vanish, and the rest matches the oracle over that sequence's first 512 tokens."""
    from gated_linear_recurrence_amd import binding
    w = synth.WORKLOADS[synth.BATCHED_2B]
    p = synth.make_params(w)
    x, y, h0 = synth.make_act(w, "x"), synth.make_act(w, "y"), synth.make_h0(w)
    b0, n = 5, 512
    dout = np.zeros((w.B, w.T, w.D), np.uint16)
    dout[b0, :n] = synth.round_bf16(np.random.default_rng(3).standard_normal((n, w.D)).astype(np.float32))
    g = binding.rglru_prefill_backward(H.dev_params(p, w.H), H.to_dev(x), H.to_dev(y),
                                       H.to_dev(dout), H.to_dev(h0))
    torch.cuda.synchronize()
    for k in ("dx", "dy"):
        t = g[k].float()
        assert not bool(t[b0, n:].any()) and not bool(t[:b0].any()) and not bool(t[b0 + 1:].any()), k
    assert not bool(g["dh0"][:b0].any()) and not bool(g["dh0"][b0 + 1:].any())
    ref = H.oracle.prefill_backward(H.oracle_params(p, w.H), x[b0:b0 + 1, :n], y[b0:b0 + 1, :n],
                                    H.wide(dout[b0:b0 + 1, :n]), h0=h0[b0:b0 + 1])
    sub = {k: v for k, v in g.items()}
    sub["dx"], sub["dy"] = g["dx"][b0:b0 + 1, :n], g["dy"][b0:b0 + 1, :n]
    sub["dh0"], sub["dconv0"] = g["dh0"][b0:b0 + 1], g["dconv0"][b0:b0 + 1]
    _compare(sub, ref, "backward full size, sequence %d, first %d tokens" % (b0, n))
