"""GPU parity of the residual layer (RMSNorm, gated MLP, both layers) through the C ABI against
the fp64 oracle.

Bars: the layer rounds each step's result to bf16 as a bf16 model does (normalised rows, block
output, h, the MLP's gate, up, their product and its output) while the oracle keeps fp64, so
outputs meet the bf16 bar, rel-L2 <= 2e-2; every row of an RMSNorm is also held to 2e-2, and
h = x + residual to one bf16 rounding (2^-8 relative) of the exact sum.  Full-size layers are checked on time
prefixes of sampled sequences (both layers are causal and their sequences independent).
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


@pytest.mark.parametrize("M,D,residual", [
    (37, 2560, True),     # the 2B width, with the residual addition
    (5, 8, False),        # one chunk per row, most lanes idle
    (64, 8192, True),     # the widest row
    (300, 512, False),
])
def test_rmsnorm_matches_oracle(M, D, residual):
    from gated_linear_recurrence_amd import binding
    rng = np.random.default_rng(M + D)
    x = _bf(rng.standard_normal((M, D)) * 2)
    r = _bf(rng.standard_normal((M, D))) if residual else None
    g = _bf(1 + 0.1 * rng.standard_normal(D))
    out, h = binding.rglru_rmsnorm(H.to_dev(x), H.to_dev(g), H.to_dev(r), 1e-6, want_h=True)
    torch.cuda.synchronize()
    exact = H.wide(x) + (H.wide(r) if residual else 0.0)
    hg = H.wide(H.to_host(h))
    assert np.all(np.abs(hg - exact) <= 2.0 ** -8 * np.abs(exact) + 1e-30)
    ref = H.oracle.rmsnorm(exact, g, 1e-6)
    got = H.wide(H.to_host(out))
    e = H.rel_l2(got, ref)
    rows = np.linalg.norm(got - ref, axis=1) / np.linalg.norm(ref, axis=1)
    print("rmsnorm M=%d D=%d: rel-L2 %.3e, worst row %.3e" % (M, D, e, rows.max()))
    assert e <= H.TOL[synth.BF16] and rows.max() <= H.TOL[synth.BF16]


def test_rmsnorm_in_place_add_and_empty():
    """h_out may be x itself (in-place residual addition); M = 0 launches nothing."""
    from gated_linear_recurrence_amd import binding
    rng = np.random.default_rng(2)
    x = _bf(rng.standard_normal((20, 256)))
    r = _bf(rng.standard_normal((20, 256)))
    xd = H.to_dev(x)
    binding.rglru_rmsnorm(xd, None, H.to_dev(r), want_norm=False, h_out=xd)
    e = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    binding.rglru_rmsnorm(e, torch.ones(256, dtype=torch.bfloat16, device="cuda"))
    torch.cuda.synchronize()
    exact = H.wide(x) + H.wide(r)
    assert np.all(np.abs(H.wide(H.to_host(xd)) - exact) <= 2.0 ** -8 * np.abs(exact) + 1e-30)


def _mlp_dev(L):
    from gated_linear_recurrence_amd import binding
    return binding.MlpParams(*[H.to_dev(L[k]) for k in ("gate_w", "gate_b", "up_w", "up_b",
                                                       "down_w", "down_b")])


def _mlp_oracle(L):
    return H.oracle.MlpParams(L["gate_w"], L["gate_b"], L["up_w"], L["up_b"], L["down_w"],
                              L["down_b"])


@pytest.mark.parametrize("M,Dm,F,biases", [
    (300, 512, 768, True),     # ragged rows
    (130, 2560, 7680, False),  # the 2B widths
    (1, 2560, 7680, True),     # one row: gating in the gate|up row kernel's epilogue
    (3, 512, 768, True),       # gated row kernel, then the down projection on the MFMA kernel
    (40, 512, 768, True),      # no workspace for partial sums: gated mid-size tiles, skinny down
    (2048, 512, 768, True),    # past 1024 rows: gating in the 256 x 256 tiles' epilogue
])
def test_mlp_matches_oracle(M, Dm, F, biases):
    from gated_linear_recurrence_amd import binding
    w = synth.small(synth.WORKLOADS[synth.PREFILL_2B], B=1, T=M)
    L = synth.make_layer(w, Dm=Dm, F=F, biases=biases)
    x = synth.make_block_input(w, Dm=Dm, B=1, T=M)[0]
    out = binding.rglru_mlp(_mlp_dev(L), H.to_dev(x))
    torch.cuda.synchronize()
    ref = H.oracle.mlp(_mlp_oracle(L), x)
    e = H.rel_l2(H.wide(H.to_host(out)), ref)
    print("mlp M=%d Dm=%d F=%d: rel-L2 %.3e" % (M, Dm, F, e))
    assert e <= H.TOL[synth.BF16]


# ------------------------------------------------------------------------------------------
# the two layers
# ------------------------------------------------------------------------------------------
def _norms_dev(L):
    from gated_linear_recurrence_amd import binding
    return binding.NormParams(H.to_dev(L["norm_t"]), H.to_dev(L["norm_c"]), synth.NORM_EPS)


def _run_recurrent_layer(w, p, q, L, x_in, h0, c0):
    from gated_linear_recurrence_amd import binding
    P = H.dev_params(p, w.H)
    Q = binding.ProjParams(*[H.to_dev(q[k]) for k in ("lx_w", "lx_b", "ly_w", "ly_b",
                                                      "lo_w", "lo_b")])
    out, hl, cl = binding.rglru_recurrent_layer_prefill(P, Q, _norms_dev(L), _mlp_dev(L),
                                                        H.to_dev(x_in), H.to_dev(h0), H.to_dev(c0))
    torch.cuda.synchronize()
    return out, hl, cl


def _oracle_recurrent_layer(w, p, q, L, x_in, h0, c0):
    Po = H.oracle_params(p, w.H)
    Qo = H.oracle.ProjParams(q["lx_w"], q["lx_b"], q["ly_w"], q["ly_b"], q["lo_w"], q["lo_b"])
    state = {}

    def temporal(xn):
        o, state["h"], state["c"] = H.oracle.block_prefill(Po, Qo, xn, h0=h0, conv0=c0)
        return o

    out, _ = H.oracle.residual_layer(x_in, temporal, L["norm_t"], L["norm_c"], _mlp_oracle(L),
                                     synth.NORM_EPS)
    return out, state["h"], state["c"]


@pytest.mark.parametrize("D,nh,Dm,F,B,T,biases,state", [
    (512, 2, 512, 768, 2, 150, True, 3),       # ragged rows (M = 300), with state
    (2560, 10, 2560, 7680, 1, 96, False, None),  # the 2B widths
])
def test_recurrent_layer_matches_oracle(D, nh, Dm, F, B, T, biases, state):
    w = dataclasses.replace(synth.small(synth.WORKLOADS[synth.PREFILL_2B], B=B, T=T), D=D, H=nh)
    p = synth.make_params(w, biases=biases)
    q = synth.make_proj(w, Dm=Dm, biases=biases)
    L = synth.make_layer(w, Dm=Dm, F=F, biases=biases)
    x_in = synth.make_block_input(w, Dm=Dm, B=B, T=T)
    h0 = c0 = None
    if state is not None:
        h0 = np.random.default_rng(state).normal(0, 0.3, (B, D)).astype(np.float32)
        c0 = synth.make_conv0(w, B)
    out, hl, cl = _run_recurrent_layer(w, p, q, L, x_in, h0, c0)
    ro, rh, rc = _oracle_recurrent_layer(w, p, q, L, x_in, h0, c0)
    e = H.rel_l2(H.wide(H.to_host(out)), ro)
    eh = H.rel_l2(H.to_host(hl).astype(np.float64), rh)
    ec = H.rel_l2(H.wide(H.to_host(cl)), rc)
    print("recurrent layer D=%d Dm=%d F=%d B=%d T=%d: rel-L2 out %.3e h_last %.3e conv %.3e"
          % (D, Dm, F, B, T, e, eh, ec))
    assert max(e, eh, ec) <= H.TOL[synth.BF16]


def _run_attention_layer(a, L, x_in, Hq, W, cache=None):
    from gated_linear_recurrence_amd import binding
    A = binding.AttnParams(H.to_dev(a["q_w"]), H.to_dev(a["k_w"]), H.to_dev(a["v_w"]),
                           H.to_dev(a["o_w"]), H.to_dev(a["o_b"]), Hq, W)
    out = binding.rglru_attention_layer_prefill(A, _norms_dev(L), _mlp_dev(L), H.to_dev(x_in),
                                                cache=cache)
    torch.cuda.synchronize()
    return out


def _oracle_attention_layer(a, L, x_in, Hq, W):
    out, _ = H.oracle.residual_layer(
        x_in, lambda xn: H.oracle.local_attention_block(xn, a["q_w"], a["k_w"], a["v_w"],
                                                        a["o_w"], a["o_b"], Hq, W,
                                                        synth.ROPE_BASE),
        L["norm_t"], L["norm_c"], _mlp_oracle(L), synth.NORM_EPS)
    return out


@pytest.mark.parametrize("Dm,Hq,F,B,T,W,biases", [
    (512, 2, 512, 2, 200, 64, True),          # ragged rows, window edges
    (2560, 10, 7680, 1, 130, 2048, False),    # the 2B widths and window
])
def test_attention_layer_matches_oracle(Dm, Hq, F, B, T, W, biases):
    w = synth.small(synth.WORKLOADS[synth.PREFILL_2B], B=B, T=T)
    a = synth.make_attn(w, Dm=Dm, n_heads=Hq, bias=biases)
    L = synth.make_layer(w, Dm=Dm, F=F, biases=biases)
    x_in = synth.make_block_input(w, Dm=Dm, B=B, T=T)
    out = _run_attention_layer(a, L, x_in, Hq, W)
    ref = _oracle_attention_layer(a, L, x_in, Hq, W)
    e = H.rel_l2(H.wide(H.to_host(out)), ref)
    print("attention layer Dm=%d Hq=%d F=%d B=%d T=%d W=%d: rel-L2 %.3e" % (Dm, Hq, F, B, T, W, e))
    assert e <= H.TOL[synth.BF16]


def test_layers_empty_sequence():
    from gated_linear_recurrence_amd import binding
    w = dataclasses.replace(synth.small(synth.WORKLOADS[synth.PREFILL_2B], B=2, T=0), D=512, H=2)
    p, q = synth.make_params(w), synth.make_proj(w, Dm=256)
    L = synth.make_layer(w, Dm=256, F=512)
    h0 = np.random.default_rng(1).normal(0, 0.3, (2, 512)).astype(np.float32)
    out, hl, _ = _run_recurrent_layer(w, p, q, L, np.zeros((2, 0, 256), np.uint16), h0, None)
    assert tuple(out.shape) == (2, 0, 256)
    np.testing.assert_array_equal(H.to_host(hl), h0)
    a = synth.make_attn(w, Dm=256, n_heads=1)
    out = _run_attention_layer(a, L, np.zeros((2, 0, 256), np.uint16), 1, 64)
    assert tuple(out.shape) == (2, 0, 256)
    del binding


def test_layers_2b_batched_full_size_sampled():
    """Both layers at the batched 2B size (8 x 8192 tokens, width 2560, MLP 7680); the oracle
    checks the first 96 tokens of two sequences."""
    w = synth.WORKLOADS[synth.BATCHED_2B]
    x_in = synth.make_block_input(w)
    L = synth.make_layer(w)
    p, q = synth.make_params(w), synth.make_proj(w)
    h0 = synth.make_h0(w)
    out, _, _ = _run_recurrent_layer(w, p, q, L, x_in, h0, None)
    a = synth.make_attn(w)
    out_a = _run_attention_layer(a, L, x_in, synth.ATTN_HEADS_2B, synth.ATTN_WINDOW)
    t_use = 96
    for b in (0, w.B - 1):
        ro, _, _ = _oracle_recurrent_layer(synth.small(w, B=1, T=t_use), p, q, L,
                                           x_in[b:b + 1, :t_use], h0[b:b + 1], None)
        e = H.rel_l2(H.wide(H.to_host(out[b:b + 1, :t_use])), ro)
        ra = _oracle_attention_layer(a, L, x_in[b:b + 1, :t_use], synth.ATTN_HEADS_2B,
                                     synth.ATTN_WINDOW)
        ea = H.rel_l2(H.wide(H.to_host(out_a[b:b + 1, :t_use])), ra)
        print("layers full size, sequence %d, first %d tokens: recurrent %.3e, attention %.3e"
              % (b, t_use, e, ea))
        assert e <= H.TOL[synth.BF16] and ea <= H.TOL[synth.BF16]
    assert bool(torch.isfinite(out.float()).all()) and bool(torch.isfinite(out_a.float()).all())


# ------------------------------------------------------------------------------------------
# decode steps of the layers: a prefill of T0 tokens, then single-token steps, must give the
# oracle layer's rows over the whole sequence (the layers are causal)
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("D,nh,Dm,F,N,T0,steps", [
    (512, 2, 512, 768, 3, 40, 6),
    (2560, 10, 2560, 7680, 2, 20, 3),     # the 2B widths
    (2560, 10, 2560, 7680, 1, 20, 3),     # one row: the row GEMV with the residual epilogue
    (2560, 10, 2560, 7680, 4, 20, 3),     # four rows: the row GEMV's widest case
    (512, 2, 512, 768, 40, 6, 2),         # 5..64 rows: mid-size tiles with split K, add-and-norm in their sums
    (2560, 10, 2560, 7680, 16, 4, 2),     # the same at the 2B widths
    (512, 2, 768, 1536, 130, 6, 2),       # 128-row tiles with split K (gate|up: 12 k-steps in 5)
    (512, 2, 512, 768, 1100, 2, 1),       # past 1024 rows: 256-row tiles; add-and-norm in their sums
])
def test_recurrent_layer_decode_continues_prefill(D, nh, Dm, F, N, T0, steps):
    from gated_linear_recurrence_amd import binding
    T = T0 + steps
    w = dataclasses.replace(synth.small(synth.WORKLOADS[synth.PREFILL_2B], B=N, T=T), D=D, H=nh)
    p, q = synth.make_params(w, biases=True), synth.make_proj(w, Dm=Dm, biases=True)
    L = synth.make_layer(w, Dm=Dm, F=F, biases=True)
    x_in = synth.make_block_input(w, Dm=Dm, B=N, T=T)
    P = H.dev_params(p, w.H)
    Q = binding.ProjParams(*[H.to_dev(q[k]) for k in ("lx_w", "lx_b", "ly_w", "ly_b",
                                                      "lo_w", "lo_b")])
    Nd, Md = _norms_dev(L), _mlp_dev(L)
    _, h, conv = binding.rglru_recurrent_layer_prefill(P, Q, Nd, Md, H.to_dev(x_in[:, :T0]))
    outs = []
    for t in range(T0, T):
        o = binding.rglru_recurrent_layer_decode(P, Q, Nd, Md, H.to_dev(x_in[:, t].copy()), h, conv)
        outs.append(H.wide(H.to_host(o)))
    torch.cuda.synchronize()
    ref, _, _ = _oracle_recurrent_layer(w, p, q, L, x_in, None, None)
    got = np.stack(outs, axis=1)
    e = H.rel_l2(got, ref[:, T0:])
    print("recurrent layer decode D=%d Dm=%d F=%d N=%d, %d steps after %d: rel-L2 %.3e"
          % (D, Dm, F, N, steps, T0, e))
    assert e <= H.TOL[synth.BF16]


@pytest.mark.parametrize("Dm,Hq,F,N,W,T0,steps", [
    (512, 2, 512, 3, 32, 40, 6),          # the ring wraps
    (2560, 10, 7680, 2, 2048, 20, 3),     # the 2B widths and window
    (2560, 10, 7680, 1, 2048, 20, 3),     # one row
    (2560, 10, 7680, 4, 2048, 20, 3),     # four rows
    (512, 2, 768, 40, 32, 20, 2),         # 5..64 rows: mid-size tiles with split K
    (512, 2, 768, 130, 32, 40, 2),        # 128-row tiles with split K
])
def test_attention_layer_decode_continues_prefill(Dm, Hq, F, N, W, T0, steps):
    from gated_linear_recurrence_amd import binding
    T = T0 + steps
    w = synth.small(synth.WORKLOADS[synth.PREFILL_2B], B=N, T=T)
    a = synth.make_attn(w, Dm=Dm, n_heads=Hq, bias=True)
    L = synth.make_layer(w, Dm=Dm, F=F, biases=True)
    x_in = synth.make_block_input(w, Dm=Dm, B=N, T=T)
    A = binding.AttnParams(H.to_dev(a["q_w"]), H.to_dev(a["k_w"]), H.to_dev(a["v_w"]),
                           H.to_dev(a["o_w"]), H.to_dev(a["o_b"]), Hq, W)
    Nd, Md = _norms_dev(L), _mlp_dev(L)
    cache = binding.AttnCache(N, W, "cuda")
    binding.rglru_attention_layer_prefill(A, Nd, Md, H.to_dev(x_in[:, :T0]), cache=cache)
    outs = []
    for t in range(T0, T):
        pos = torch.full((N,), t, dtype=torch.int32, device="cuda")
        o = binding.rglru_attention_layer_decode(A, Nd, Md, pos, H.to_dev(x_in[:, t].copy()), cache)
        outs.append(H.wide(H.to_host(o)))
    torch.cuda.synchronize()
    ref = _oracle_attention_layer(a, L, x_in, Hq, W)
    got = np.stack(outs, axis=1)
    e = H.rel_l2(got, ref[:, T0:])
    print("attention layer decode Dm=%d Hq=%d F=%d N=%d W=%d, %d steps after %d: rel-L2 %.3e"
          % (Dm, Hq, F, N, W, steps, T0, e))
    assert e <= H.TOL[synth.BF16]


def test_one_row_decode_folds_the_norms_bitwise():
    """One sequence takes the layers' folded path (each RMSNorm formed inside the projection
    that consumes it); two copies of the same sequence take the separate norm kernel.  The
    folded norm repeats the norm kernel's arithmetic in its order, so the outputs and the
    updated states of the one sequence must equal those of either copy bit for bit."""
    from gated_linear_recurrence_amd import binding
    D, Dm, F, Hq, W = 2560, 2560, 7680, 10, 64
    w = dataclasses.replace(synth.small(synth.WORKLOADS[synth.PREFILL_2B], B=2, T=8), D=D, H=10)
    p, q = synth.make_params(w, biases=True), synth.make_proj(w, Dm=Dm, biases=True)
    L = synth.make_layer(w, Dm=Dm, F=F, biases=True)
    a = synth.make_attn(w, Dm=Dm, n_heads=Hq, bias=True)
    P = H.dev_params(p, w.H)
    Q = binding.ProjParams(*[H.to_dev(q[k]) for k in ("lx_w", "lx_b", "ly_w", "ly_b",
                                                      "lo_w", "lo_b")])
    A = binding.AttnParams(H.to_dev(a["q_w"]), H.to_dev(a["k_w"]), H.to_dev(a["v_w"]),
                           H.to_dev(a["o_w"]), H.to_dev(a["o_b"]), Hq, W)
    Nd, Md = _norms_dev(L), _mlp_dev(L)
    g = torch.Generator(device="cuda").manual_seed(11)
    x1 = torch.randn((1, Dm), generator=g, device="cuda").to(torch.bfloat16)
    h1 = torch.randn((1, D), generator=g, device="cuda") * 0.3
    c1 = torch.randn((1, 3, D), generator=g, device="cuda").to(torch.bfloat16)
    x2, h2, c2 = x1.repeat(2, 1), h1.repeat(2, 1), c1.repeat(2, 1, 1)
    o1 = binding.rglru_recurrent_layer_decode(P, Q, Nd, Md, x1, h1, c1)
    o2 = binding.rglru_recurrent_layer_decode(P, Q, Nd, Md, x2, h2, c2)
    torch.cuda.synchronize()
    for r in range(2):
        assert torch.equal(o1[0], o2[r]) and torch.equal(h1[0], h2[r]) and torch.equal(c1[0], c2[r]), r
    k1, k2 = binding.AttnCache(1, W, "cuda"), binding.AttnCache(2, W, "cuda")
    per = k1.k.numel()                       # the cache is sequence-major
    assert k2.k.numel() == 2 * per
    k1.k.normal_(generator=g)
    k1.v.normal_(generator=g)
    for r in range(2):
        k2.k.view(2, per)[r].copy_(k1.k)
        k2.v.view(2, per)[r].copy_(k1.v)
    pos1 = torch.full((1,), 40, dtype=torch.int32, device="cuda")
    pos2 = torch.full((2,), 40, dtype=torch.int32, device="cuda")
    y1 = binding.rglru_attention_layer_decode(A, Nd, Md, pos1, o1, k1)
    y2 = binding.rglru_attention_layer_decode(A, Nd, Md, pos2, o2, k2)
    torch.cuda.synchronize()
    for r in range(2):
        assert torch.equal(y1[0], y2[r]), r
        assert torch.equal(k1.k, k2.k.view(2, per)[r]) and torch.equal(k1.v, k2.v.view(2, per)[r]), r


def test_layer_decode_steps_replay_from_a_graph():
    """Decode steps of both layers captured in one HIP graph and replayed three times (eager
    work in between) give bitwise the eager steps' outputs and states."""
    from gated_linear_recurrence_amd import binding
    N, D, Dm, F, Hq, W = 3, 512, 512, 768, 2, 32
    w = dataclasses.replace(synth.small(synth.WORKLOADS[synth.PREFILL_2B], B=N, T=8), D=D, H=2)
    p, q = synth.make_params(w, biases=True), synth.make_proj(w, Dm=Dm, biases=True)
    L = synth.make_layer(w, Dm=Dm, F=F, biases=True)
    a = synth.make_attn(w, Dm=Dm, n_heads=Hq, bias=True)
    P = H.dev_params(p, w.H)
    Q = binding.ProjParams(*[H.to_dev(q[k]) for k in ("lx_w", "lx_b", "ly_w", "ly_b",
                                                      "lo_w", "lo_b")])
    A = binding.AttnParams(H.to_dev(a["q_w"]), H.to_dev(a["k_w"]), H.to_dev(a["v_w"]),
                           H.to_dev(a["o_w"]), H.to_dev(a["o_b"]), Hq, W)
    Nd, Md = _norms_dev(L), _mlp_dev(L)
    lib = binding.load_library()
    import ctypes
    ws_r = binding.DeviceBuffer(lib.rglru_recurrent_layer_decode_workspace_bytes(N, D, Dm, F), "cuda")
    ws_a = binding.DeviceBuffer(lib.rglru_attention_layer_decode_workspace_bytes(
        ctypes.byref(A.c), N, F), "cuda")
    g = torch.Generator(device="cuda").manual_seed(4)
    x = torch.randn((N, Dm), generator=g, device="cuda").to(torch.bfloat16)
    h0 = torch.randn((N, D), generator=g, device="cuda") * 0.3
    c0 = torch.randn((N, 3, D), generator=g, device="cuda").to(torch.bfloat16)
    cache0 = binding.AttnCache(N, W, "cuda")
    cache0.k.normal_(generator=g)
    cache0.v.normal_(generator=g)
    # state and output buffers the graph owns
    h, conv = h0.clone(), c0.clone()
    cache = binding.AttnCache(N, W, "cuda")
    pos = torch.full((N,), 40, dtype=torch.int32, device="cuda")
    y1, y2 = torch.empty_like(x), torch.empty_like(x)

    def step():
        binding.rglru_recurrent_layer_decode(P, Q, Nd, Md, x, h, conv, out=y1, workspace=ws_r)
        binding.rglru_attention_layer_decode(A, Nd, Md, pos, y1, cache, out=y2, workspace=ws_a)

    def reset():
        h.copy_(h0)
        conv.copy_(c0)
        cache.k.copy_(cache0.k)
        cache.v.copy_(cache0.v)

    reset()
    eager = []
    for _ in range(3):
        step()
        eager.append((y2.clone(), h.clone(), conv.clone(), cache.k.clone()))
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        reset()
        step()                        # warm-up outside the capture
        torch.cuda.synchronize()
        with torch.cuda.graph(gr, stream=st):
            step()
    torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    reset()
    torch.cuda.synchronize()
    for r in range(3):
        gr.replay()
        torch.cuda.synchronize()
        got = (y2, h, conv, cache.k)
        for i, (e, t) in enumerate(zip(eager[r], got)):
            assert torch.equal(e, t), (r, i)
        _ = (x.float() * 2).sum().item()   # eager work between replays
