"""GPU parity of the dense projections around the path (Linear layers, bf16 MFMA GEMM) and of
the whole temporal-mixing block (projections + path), through the C ABI, against the fp64
oracle.

Bars: a Linear layer's output is one bf16 rounding of an fp32 sum, so every element is within
one bf16 step (2^-8 relative) of the exact value plus a small absolute term for the fp32
accumulation (K terms of size |x||w|); the block's out and h_last meet the path's bf16 bar,
rel-L2 <= 2e-2.  The conv window holds linear_x outputs, which the GPU rounds to bf16 and the
oracle keeps in fp64: it is compared to within one bf16 step.  Full-size workloads are checked
on sampled rows (a Linear layer's rows are independent) and on time prefixes of sampled
sequences (the block is causal).
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


def _bf(a):
    return synth.round_bf16(np.asarray(a, np.float32))


def _check_linear(got_bits, ref, x_bits, w_bits, label):
    got = H.wide(got_bits)
    # fp32 accumulation bound: K * 2^-23 * sum_k |x_k w_k| per element (generous)
    K = x_bits.shape[1]
    mag = np.abs(H.wide(x_bits)) @ np.abs(H.wide(w_bits)).T
    bound = 2.0 ** -8 * np.abs(ref) + K * 2.0 ** -23 * mag + 1e-30
    err = np.abs(got - ref)
    worst = float(np.max(err / bound))
    print("%s: rel-L2 %.3e, worst error / bound %.3f" % (label, H.rel_l2(got, ref), worst))
    assert worst <= 1.0


@pytest.mark.parametrize("M,K,N,bias", [
    (1, 128, 256, True),          # one row
    (300, 256, 512, True),        # ragged M on the 128-row tiles: two full tiles and a partial one
    (257, 2560, 2560, False),     # the 2B widths, one row past a 128-row tile pair
    (256, 2560, 5120, True),      # decode of 256 sequences, the branch projections' shape
    (65, 7680, 256, False),       # the fewest rows of the 128-row tiles, a long K
    (513, 384, 768, True),        # K = 384: six k-steps through the four-stage ring
    (1025, 384, 768, True),       # past 1024 rows: the 256 x 256 tiles, a ragged last row tile
    (1, 2560, 2560, True),        # decode of one sequence: the row kernel (M <= 4, K % 512 == 0)
    (2, 7680, 512, False),        # row kernel, two rows, the MLP down projection's K
    (3, 1024, 768, True),         # row kernel, a ragged row count (held as four)
    (4, 512, 256, True),          # row kernel, one 512-wide step of K
    (5, 512, 512, True),          # five rows: the MFMA skinny kernel
    (4, 768, 512, True),          # K % 512 != 0: the MFMA skinny kernel
    (64, 256, 256, False),        # the MFMA skinny kernel's largest row count
])
def test_linear_matches_oracle(M, K, N, bias):
    from gated_linear_recurrence_amd import binding
    rng = np.random.default_rng(M * 7 + K + N)
    x = _bf(rng.standard_normal((M, K)))
    w = _bf(rng.standard_normal((N, K)) / np.sqrt(K))
    b = _bf(rng.standard_normal(N) * 0.5) if bias else None
    out = binding.rglru_linear(H.to_dev(x), H.to_dev(w), H.to_dev(b))
    torch.cuda.synchronize()
    ref = H.oracle.linear(x, w, b)
    _check_linear(H.to_host(out), ref, x, w, "linear M=%d K=%d N=%d" % (M, K, N))


def test_linear_empty_and_stays_in_bounds():
    """M = 0 launches nothing; a ragged M writes no row past M (canary rows stay intact)."""
    from gated_linear_recurrence_amd import binding
    rng = np.random.default_rng(5)
    K, N, M = 256, 256, 37
    x = _bf(rng.standard_normal((M, K)))
    w = _bf(rng.standard_normal((N, K)) / 16)
    buf = torch.full((M + 64, N), 7.0, dtype=torch.bfloat16, device="cuda")
    binding.rglru_linear(H.to_dev(x), H.to_dev(w), None, out=buf[:M])
    binding.rglru_linear(torch.empty((0, K), dtype=torch.bfloat16, device="cuda"), H.to_dev(w))
    torch.cuda.synchronize()
    assert bool((buf[M:] == 7.0).all())
    _check_linear(H.to_host(buf[:M]), H.oracle.linear(x, w), x, w, "linear M=37 in canary buffer")


def test_linear_full_size_sampled_rows():
    """The out-projection's shape at the batched 2B workload (65536 x 2560 x 2560), checked on
    sampled rows against the oracle."""
    from gated_linear_recurrence_amd import binding
    w_ = synth.WORKLOADS[synth.BATCHED_2B]
    M, K, N = w_.B * w_.T, w_.D, w_.D
    g = torch.Generator(device="cuda").manual_seed(11)
    xd = torch.randn((M, K), generator=g, device="cuda").to(torch.bfloat16)
    wd = (torch.randn((N, K), generator=g, device="cuda") / 50.0).to(torch.bfloat16)
    bd = torch.randn((N,), generator=g, device="cuda").to(torch.bfloat16)
    out = binding.rglru_linear(xd, wd, bd)
    torch.cuda.synchronize()
    rows = np.concatenate([np.arange(0, 3), np.random.default_rng(1).integers(0, M, 120),
                           np.arange(M - 3, M)])
    x = H.to_host(xd[torch.as_tensor(rows, device="cuda")])
    w, b = H.to_host(wd), H.to_host(bd)
    ref = H.oracle.linear(x, w, b)
    _check_linear(H.to_host(out[torch.as_tensor(rows, device="cuda")]), ref, x, w,
                  "linear 65536x2560x2560, 126 sampled rows")


# ------------------------------------------------------------------------------------------
# the whole block
# ------------------------------------------------------------------------------------------
def _block_setup(w, Dm, B, T, biases, seed_state=None):
    p = synth.make_params(w, biases=biases)
    q = synth.make_proj(w, Dm=Dm, biases=biases)
    x_in = synth.make_block_input(w, Dm=Dm, B=B, T=T)
    h0 = c0 = None
    if seed_state is not None:
        rng = np.random.default_rng(seed_state)
        h0 = rng.normal(0, 0.3, (B, w.D)).astype(np.float32)
        c0 = synth.make_conv0(w, B)
    return p, q, x_in, h0, c0


def _run_block(w, p, q, x_in, h0, c0):
    from gated_linear_recurrence_amd import binding
    P = H.dev_params(p, w.H)
    Q = binding.ProjParams(*[H.to_dev(q[k]) for k in ("lx_w", "lx_b", "ly_w", "ly_b",
                                                      "lo_w", "lo_b")])
    out, h_last, conv_last = binding.rglru_block_prefill(P, Q, H.to_dev(x_in), H.to_dev(h0),
                                                         H.to_dev(c0))
    torch.cuda.synchronize()
    return out, h_last, conv_last


def _oracle_block(w, p, q, x_in, h0, c0):
    Po = H.oracle_params(p, w.H)
    Qo = H.oracle.ProjParams(q["lx_w"], q["lx_b"], q["ly_w"], q["ly_b"], q["lo_w"], q["lo_b"])
    return H.oracle.block_prefill(Po, Qo, x_in, h0=h0, conv0=c0)


def _compare_block(out, h_last, conv_last, ro, rh, rc, label):
    e_out = H.rel_l2(H.wide(H.to_host(out)), ro)
    e_h = H.rel_l2(H.to_host(h_last).astype(np.float64), rh)
    cw = H.wide(H.to_host(conv_last))
    e_c = float(np.max(np.abs(cw - rc) / (np.abs(rc) * 2.0 ** -8 + 1e-3)))
    print("%s: rel-L2 out %.3e h_last %.3e; conv window worst %.3f of one bf16 step"
          % (label, e_out, e_h, e_c))
    assert e_out <= H.TOL[synth.BF16] and e_h <= H.TOL[synth.BF16], (e_out, e_h)
    assert e_c <= 1.0


@pytest.mark.parametrize("D,nh,Dm,B,T,biases,state", [
    (512, 2, 768, 2, 200, True, 7),      # D != D_model, ragged rows (M = 400), with state
    (512, 4, 512, 1, 130, False, None),  # bs = 128
    (2560, 10, 2560, 1, 96, True, 9),    # the 2B widths
])
def test_block_prefill_matches_oracle(D, nh, Dm, B, T, biases, state):
    w = synth.small(synth.WORKLOADS[synth.PREFILL_2B], B=B, T=T)
    w = dataclasses.replace(w, D=D, H=nh)
    p, q, x_in, h0, c0 = _block_setup(w, Dm, B, T, biases, state)
    out, h_last, conv_last = _run_block(w, p, q, x_in, h0, c0)
    ro, rh, rc = _oracle_block(w, p, q, x_in, h0, c0)
    _compare_block(out, h_last, conv_last, ro, rh, rc,
                   "block D=%d H=%d Dm=%d B=%d T=%d" % (D, nh, Dm, B, T))


def test_block_empty_sequence_passes_state_through():
    from gated_linear_recurrence_amd import binding
    w = dataclasses.replace(synth.small(synth.WORKLOADS[synth.PREFILL_2B], B=2, T=0),
                                  D=512, H=2)
    p, q, x_in, h0, c0 = _block_setup(w, 256, 2, 0, True, 3)
    out, h_last, conv_last = _run_block(w, p, q, x_in, h0, c0)
    assert tuple(out.shape) == (2, 0, 256)
    np.testing.assert_array_equal(H.to_host(h_last), h0)
    np.testing.assert_array_equal(H.to_host(conv_last), c0)


def test_block_2b_batched_full_size_sampled():
    """The batched 2B block (8 x 8192 tokens, widths 2560) at full size; the oracle checks time
    prefixes of sampled sequences (the block is causal and its sequences independent)."""
    w = synth.WORKLOADS[synth.BATCHED_2B]
    p = synth.make_params(w)
    q = synth.make_proj(w)
    x_in = synth.make_block_input(w)
    h0 = synth.make_h0(w)
    out, h_last, conv_last = _run_block(w, p, q, x_in, h0, None)
    t_use = 160
    for b in (0, w.B - 1):
        ro, rh, rc = _oracle_block(synth.small(w, B=1, T=t_use), p, q, x_in[b:b + 1, :t_use],
                                   h0[b:b + 1], None)
        e_out = H.rel_l2(H.wide(H.to_host(out[b:b + 1, :t_use])), ro)
        print("block 2b-batched full size, sequence %d, first %d tokens: rel-L2 out %.3e"
              % (b, t_use, e_out))
        assert e_out <= H.TOL[synth.BF16]
    assert bool(torch.isfinite(out.float()).all()) and bool(torch.isfinite(h_last).all())
