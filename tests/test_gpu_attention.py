"""GPU parity of local sliding-window multi-query attention (RoPE, MQA, window) and of the
whole local-attention block, through the C ABI, against the fp64 oracle.

Bars: the kernel rounds q and k to bf16 after RoPE, and the probabilities to bf16 before the
P.V product, so the output meets the bf16 bar, rel-L2 <= 2e-2, over each call; every (token,
head) row is also held to 5e-2 (1e-1 where the scores are sharp, inputs x3, where the bf16
rounding of q and k moves large logits by ~2^-8 of their size).  A mask that is off by one key
is caught where it matters: window 1 is bit-exact (the output row is v itself), and windows of
2 and 3 with zero queries give the mean of two or three rows, which one key more or less
changes by a large fraction.  Full-size workloads are checked on sampled rows: the first tokens
of sampled sequences, and single queries whose whole window is handed to the oracle.
"""
from __future__ import annotations

import numpy as np
import pytest

import helpers as H
from gated_linear_recurrence_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

DH = synth.ATTN_HEAD_DIM


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_linear_recurrence_amd import binding
    binding.load_library()


def _inputs(B, T, Hq, qk_scale, seed):
    rng = np.random.default_rng(seed)
    q = synth.round_bf16(rng.standard_normal((B, T, Hq, DH)).astype(np.float32) * qk_scale)
    k = synth.round_bf16(rng.standard_normal((B, T, DH)).astype(np.float32) * max(qk_scale, 1))
    v = synth.round_bf16(rng.standard_normal((B, T, DH)).astype(np.float32))
    return q, k, v


def _oracle_seq(q, k, v, window, base=synth.ROPE_BASE, t0=0):
    """One sequence (or a slice of one starting at position t0): q [T, Hq, dh], k, v [T, dh]
    (bf16 bits) -> o [T, Hq, dh] fp64."""
    T, Hq, _ = q.shape
    pos = np.arange(t0, t0 + T, dtype=np.float64)
    qr = H.oracle.rope(H.wide(q).reshape(T * Hq, DH), np.repeat(pos, Hq), base).reshape(T, Hq, DH)
    kr = H.oracle.rope(H.wide(k), pos, base)
    return H.oracle.local_mqa(qr, kr, H.wide(v), window)


def _compare(got, ref, label, row_bar=5e-2):
    e = H.rel_l2(got, ref)
    rows = np.linalg.norm((got - ref).reshape(-1, DH), axis=1) / \
        np.maximum(np.linalg.norm(ref.reshape(-1, DH), axis=1), 1e-30)
    print("%s: rel-L2 %.3e, worst row %.3e" % (label, e, rows.max()))
    assert e <= H.TOL[synth.BF16], e
    assert rows.max() <= row_bar, rows.max()


@pytest.mark.parametrize("B,T,Hq,W,qk_scale", [
    (2, 300, 2, 64, 1.0),      # ragged T: two full query blocks and 44 rows; window edges
    (2, 517, 2, 129, 1.0),     # window not a multiple of the key tile
    (1, 130, 3, 1000, 1.0),    # T < window: plain causal attention
    (1, 2100, 1, 2048, 1.0),   # the 2B window, crossed by the last 52 queries
    (1, 5, 10, 2048, 1.0),     # fewer tokens than a key tile, the 2B head count
    (1, 300, 2, 64, 3.0),      # sharp scores: lazy rescaling of the running output
])
def test_attention_matches_oracle(B, T, Hq, W, qk_scale):
    from gated_linear_recurrence_amd import binding
    q, k, v = _inputs(B, T, Hq, qk_scale, B * 1000 + T + Hq + W)
    o = binding.rglru_local_attention(H.to_dev(q), H.to_dev(k), H.to_dev(v), W)
    torch.cuda.synchronize()
    got = H.wide(H.to_host(o))
    ref = np.stack([_oracle_seq(q[b], k[b], v[b], W) for b in range(B)])
    _compare(got, ref, "attention B=%d T=%d Hq=%d W=%d scale %g" % (B, T, Hq, W, qk_scale),
             row_bar=5e-2 if qk_scale <= 1 else 1e-1)


def test_attention_window_one_is_v():
    """Window 1: every query sees only its own token, so o[t, h] = v[t] bit for bit."""
    from gated_linear_recurrence_amd import binding
    q, k, v = _inputs(2, 200, 2, 1.0, 21)
    o = H.to_host(binding.rglru_local_attention(H.to_dev(q), H.to_dev(k), H.to_dev(v), 1))
    ref = _oracle_seq(q[0], k[0], v[0], 1)
    np.testing.assert_array_equal(H.wide(v[0]), ref[:, 0])          # the oracle agrees
    for h in range(2):
        np.testing.assert_array_equal(o[:, :, h], v)


@pytest.mark.parametrize("W", [2, 3])
def test_attention_zero_queries_average_the_window(W):
    """q = 0: uniform weights, so each output is the mean of the (up to) W newest v rows."""
    from gated_linear_recurrence_amd import binding
    q, k, v = _inputs(1, 170, 1, 1.0, 30 + W)
    q[:] = 0
    o = binding.rglru_local_attention(H.to_dev(q), H.to_dev(k), H.to_dev(v), W)
    got = H.wide(H.to_host(o))
    ref = _oracle_seq(q[0], k[0], v[0], W)[None]
    _compare(got, ref, "attention zero queries W=%d" % W, row_bar=1e-2)


def test_attention_empty_and_stays_in_bounds():
    """T = 0 launches nothing; a ragged T writes no row past T (canary rows stay intact)."""
    from gated_linear_recurrence_amd import binding
    q, k, v = _inputs(1, 45, 2, 1.0, 7)
    buf = torch.full((1, 45 + 100, 2, DH), 7.0, dtype=torch.bfloat16, device="cuda")
    binding.rglru_local_attention(H.to_dev(q), H.to_dev(k), H.to_dev(v), 16, out=buf[:, :45])
    e = torch.empty((1, 0, 2, DH), dtype=torch.bfloat16, device="cuda")
    binding.rglru_local_attention(e, e[:, :, 0], e[:, :, 0].clone(), 16)
    torch.cuda.synchronize()
    assert bool((buf[:, 45:] == 7.0).all())
    _compare(H.wide(H.to_host(buf[:, :45])), _oracle_seq(q[0], k[0], v[0], 16)[None],
             "attention T=45 in canary buffer")


def test_attention_full_size_sampled():
    """The 2B attention at the batched workload's size (8 x 8192 tokens, 10 heads, window
    2048), checked on the first 256 tokens of two sequences (all heads) and on full-window
    queries (their 2048-token windows handed to the oracle) for two heads."""
    from gated_linear_recurrence_amd import binding
    w = synth.WORKLOADS[synth.BATCHED_2B]
    B, T, Hq, W = w.B, w.T, synth.ATTN_HEADS_2B, synth.ATTN_WINDOW
    g = torch.Generator(device="cuda").manual_seed(12)
    qd = torch.randn((B, T, Hq, DH), generator=g, device="cuda").to(torch.bfloat16)
    kd = torch.randn((B, T, DH), generator=g, device="cuda").to(torch.bfloat16)
    vd = torch.randn((B, T, DH), generator=g, device="cuda").to(torch.bfloat16)
    o = binding.rglru_local_attention(qd, kd, vd, W)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o.float()).all())
    for b in (0, B - 1):
        n = 256
        ref = _oracle_seq(H.to_host(qd[b, :n]), H.to_host(kd[b, :n]), H.to_host(vd[b, :n]), W)
        _compare(H.wide(H.to_host(o[b, :n])), ref, "attention full size, seq %d, first %d" % (b, n))
    for b, t in ((0, T - 1), (B - 1, 4097), (3, 2047 + 32 * 37 + 5)):
        s0 = t - W + 1
        for h in (0, Hq - 1):
            ref = _oracle_seq(H.to_host(qd[b, s0:t + 1, h:h + 1]), H.to_host(kd[b, s0:t + 1]),
                              H.to_host(vd[b, s0:t + 1]), W, t0=s0)[-1:]
            _compare(H.wide(H.to_host(o[b, t:t + 1, h:h + 1])), ref,
                     "attention full size, seq %d, query %d, head %d" % (b, t, h))


# ------------------------------------------------------------------------------------------
# the whole local-attention block
# ------------------------------------------------------------------------------------------
def _run_block(a, x_in, Hq, W):
    from gated_linear_recurrence_amd import binding
    P = binding.AttnParams(H.to_dev(a["q_w"]), H.to_dev(a["k_w"]), H.to_dev(a["v_w"]),
                           H.to_dev(a["o_w"]), H.to_dev(a["o_b"]), Hq, W)
    out = binding.rglru_local_attention_block(P, H.to_dev(x_in))
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("Dm,Hq,B,T,W,bias", [
    (512, 2, 2, 300, 64, True),       # ragged rows (M = 600), window edges
    (2560, 10, 1, 160, 2048, False),  # the 2B widths and window
    (768, 1, 1, 70, 16, True),        # one query head
])
def test_attention_block_matches_oracle(Dm, Hq, B, T, W, bias):
    w = synth.small(synth.WORKLOADS[synth.PREFILL_2B], B=B, T=T)
    a = synth.make_attn(w, Dm=Dm, n_heads=Hq, bias=bias)
    x_in = synth.make_block_input(w, Dm=Dm, B=B, T=T)
    out = _run_block(a, x_in, Hq, W)
    ref = H.oracle.local_attention_block(x_in, a["q_w"], a["k_w"], a["v_w"], a["o_w"], a["o_b"],
                                         Hq, W, synth.ROPE_BASE)
    e = H.rel_l2(H.wide(H.to_host(out)), ref)
    print("attention block Dm=%d Hq=%d B=%d T=%d W=%d: rel-L2 %.3e" % (Dm, Hq, B, T, W, e))
    assert e <= H.TOL[synth.BF16]


def test_attention_block_empty_sequence():
    w = synth.small(synth.WORKLOADS[synth.PREFILL_2B], B=2, T=0)
    a = synth.make_attn(w, Dm=256, n_heads=1)
    out = _run_block(a, np.zeros((2, 0, 256), np.uint16), 1, 64)
    assert tuple(out.shape) == (2, 0, 256)


def test_attention_block_2b_batched_full_size_sampled():
    """The 2B local-attention block at the batched workload's size (8 x 8192 tokens, width
    2560); the oracle checks time prefixes of sampled sequences (the block is causal and its
    sequences independent)."""
    w = synth.WORKLOADS[synth.BATCHED_2B]
    a = synth.make_attn(w)
    x_in = synth.make_block_input(w)
    out = _run_block(a, x_in, synth.ATTN_HEADS_2B, synth.ATTN_WINDOW)
    t_use = 160
    for b in (0, w.B - 1):
        ref = H.oracle.local_attention_block(x_in[b:b + 1, :t_use], a["q_w"], a["k_w"], a["v_w"],
                                             a["o_w"], a["o_b"], synth.ATTN_HEADS_2B,
                                             synth.ATTN_WINDOW, synth.ROPE_BASE)
        e = H.rel_l2(H.wide(H.to_host(out[b:b + 1, :t_use])), ref)
        print("attention block 2b-batched full size, sequence %d, first %d tokens: rel-L2 %.3e"
              % (b, t_use, e))
        assert e <= H.TOL[synth.BF16]
    assert bool(torch.isfinite(out.float()).all())


# ------------------------------------------------------------------------------------------
# decode with the ring KV cache
# ------------------------------------------------------------------------------------------
def _decode_run(N, Hq, W, T0, steps, pause=None, seed=0):
    """Prefill T0 tokens of N sequences into the cache (none when T0 = 0), then decode `steps`
    tokens; sequence n skips the steps listed in pause.get(n, ()) (position -1: no cache write,
    o = 0), so positions become ragged.  Returns the per-step outputs with each sequence's
    positions, and the whole sequences' inputs for the oracle."""
    from gated_linear_recurrence_amd import binding
    total = T0 + steps
    q, k, v = _inputs(N, total, Hq, 1.0, seed)
    cache = binding.AttnCache(N, W, "cuda")
    if T0 > 0:
        binding.rglru_local_attention(H.to_dev(q[:, :T0]), H.to_dev(k[:, :T0]),
                                      H.to_dev(v[:, :T0]), W, cache=cache)
    nxt = [T0] * N          # next position of each sequence
    outs = []
    pause = pause or {}
    for j in range(steps):
        pos = np.array([-1 if j in pause.get(n, ()) else nxt[n] for n in range(N)], np.int32)
        idx = np.maximum(pos, 0)
        qs = np.stack([q[n, idx[n]] for n in range(N)])
        ks = np.stack([k[n, idx[n]] for n in range(N)])
        vs = np.stack([v[n, idx[n]] for n in range(N)])
        o = binding.rglru_local_attention_decode(torch.as_tensor(pos, device="cuda"), H.to_dev(qs),
                                                 H.to_dev(ks), H.to_dev(vs), cache)
        outs.append((pos, H.wide(H.to_host(o))))
        for n in range(N):
            nxt[n] += pos[n] >= 0
    torch.cuda.synchronize()
    return outs, (q, k, v)


def _check_decode(outs, inputs, W, label):
    q, k, v = inputs
    N = q.shape[0]
    refs = [_oracle_seq(q[n], k[n], v[n], W) for n in range(N)]
    got, ref = [], []
    for pos, o in outs:
        for n in range(N):
            if pos[n] < 0:
                assert not o[n].any(), "a paused sequence must give zeros"
            else:
                got.append(o[n])
                ref.append(refs[n][pos[n]])
    _compare(np.stack(got), np.stack(ref), label)


@pytest.mark.parametrize("N,Hq,W,T0,steps", [
    (3, 10, 64, 50, 40),      # the ring wraps during decoding; window not a multiple of 512
    (2, 4, 2048, 2040, 20),   # the 2B window, crossed at position 2048
    (2, 16, 100, 0, 45),      # from an empty cache, 16 heads, window not a multiple of 32
    (20, 4, 600, 590, 12),    # 16 <= N < 64: 256-slot splits, the last one ragged
    (1, 1, 1, 5, 6),          # window 1
])
def test_attention_decode_matches_oracle(N, Hq, W, T0, steps):
    outs, inputs = _decode_run(N, Hq, W, T0, steps, seed=N * 100 + W + T0)
    _check_decode(outs, inputs, W, "decode N=%d Hq=%d W=%d from %d, %d steps" % (N, Hq, W, T0, steps))


def test_attention_decode_ragged_positions():
    """Sequences at different positions in one call: sequence 1 pauses for five steps (position
    -1 leaves its cache alone and gives zeros), sequence 2 for one."""
    outs, inputs = _decode_run(3, 10, 48, 30, 30, pause={1: range(8, 13), 2: (0,)}, seed=5)
    _check_decode(outs, inputs, 48, "decode with ragged positions")


def test_attention_prefill_fills_cache_past_window():
    """A prefill longer than the window leaves the last `window` positions in the cache; the
    next decode step sees exactly those."""
    outs, inputs = _decode_run(2, 10, 128, 300, 3, seed=9)
    _check_decode(outs, inputs, 128, "decode after a prefill past the window")


def test_attention_decode_full_size_sampled():
    """One decode step of the 2B attention for 256 sequences at window 2048, with the ring
    wrapped (prefill of 2100 tokens); sampled sequences and heads against the oracle on their
    2048-token windows."""
    from gated_linear_recurrence_amd import binding
    N, Hq, W, T0 = 256, synth.ATTN_HEADS_2B, synth.ATTN_WINDOW, 2100
    g = torch.Generator(device="cuda").manual_seed(21)
    qd = torch.randn((N, T0 + 1, Hq, DH), generator=g, device="cuda").to(torch.bfloat16)
    kd = torch.randn((N, T0 + 1, DH), generator=g, device="cuda").to(torch.bfloat16)
    vd = torch.randn((N, T0 + 1, DH), generator=g, device="cuda").to(torch.bfloat16)
    cache = binding.AttnCache(N, W, "cuda")
    binding.rglru_local_attention(qd[:, :T0].contiguous(), kd[:, :T0].contiguous(),
                                  vd[:, :T0].contiguous(), W, cache=cache)
    pos = torch.full((N,), T0, dtype=torch.int32, device="cuda")
    o = binding.rglru_local_attention_decode(pos, qd[:, T0].contiguous(), kd[:, T0].contiguous(),
                                             vd[:, T0].contiguous(), cache)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o.float()).all())
    s0 = T0 - W + 1
    for n in (0, 137, N - 1):
        for h in (0, Hq - 1):
            ref = _oracle_seq(H.to_host(qd[n, s0:, h:h + 1]), H.to_host(kd[n, s0:]),
                              H.to_host(vd[n, s0:]), W, t0=s0)[-1:]
            _compare(H.wide(H.to_host(o[n:n + 1, h:h + 1])), ref,
                     "decode full size, sequence %d, head %d" % (n, h))
