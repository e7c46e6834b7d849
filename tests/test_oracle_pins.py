"""Pins of the CPU oracle against things other than itself.

Attention: library routines for the special cases the pages fix (no prefix ->
plain bidirectional attention; a one-token block -> causal single-token decode;
the block rows of a block-causal full-sequence attention), GQA against MHA with
repeated KV heads, closed forms, invariants (block permutation, prefix
independence, split invariance) and brute force on tiny inputs.
Unmasking: closed forms, a library softmax, exact ties, special gammas.
Loop: the invariants the commit rule implies.

Each pin is chosen so that a plausible slip in the oracle (a dropped key set, a
wrong scale, a transposed operand, a wrong GQA mapping, a missing max
subtraction, ``>=`` for ``>``, a last-index tie-break, a wrong merge weight)
fails at least one of them; ``test_planted_mistakes_are_caught`` plants several
such slips in a copy of the oracle and checks that the pins catch them.
"""
import itertools
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import bd_oracle as O


def rnd(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def make_case(B=2, S=4, Hq=4, Hkv=2, D=16, lens=(5, 0), seed=0, lcap=None):
    lcap = lcap or max(1, max(lens))
    q = rnd((B, S, Hq, D), seed)
    kb = rnd((B, S, Hkv, D), seed + 1)
    vb = rnd((B, S, Hkv, D), seed + 2)
    kc = rnd((B, Hkv, lcap, D), seed + 3)
    vc = rnd((B, Hkv, lcap, D), seed + 4)
    return q, kb, vb, kc, vc, np.array(lens, dtype=np.int32)


def sdpa(q, k, v, mask=None, is_causal=False, scale=None):
    """torch's float64 CPU scaled_dot_product_attention on [H, N, D] tensors."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(torch.float64)
    return F.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=None if mask is None else torch.from_numpy(mask),
                                          is_causal=is_causal, scale=scale).numpy()


# ------------------------------------------------------------------------------------ attention
def test_no_prefix_is_plain_bidirectional_attention():
    # L = 0: the block attends only to itself, bidirectionally (no mask).
    q, kb, vb, kc, vc, lens = make_case(B=2, S=5, Hq=4, Hkv=4, D=8, lens=(0, 0))
    Oo, _ = O.attn_step(q, kb, vb, kc, vc, lens)
    for b in range(2):
        ref = sdpa(q[b].transpose(1, 0, 2), kb[b].transpose(1, 0, 2), vb[b].transpose(1, 0, 2),
                   scale=O.default_scale(8))
        np.testing.assert_allclose(Oo[b], ref.transpose(1, 0, 2), rtol=1e-12, atol=1e-13)


def test_default_scale_is_inverse_sqrt_d():
    q, kb, vb, kc, vc, lens = make_case(B=1, S=3, Hq=2, Hkv=2, D=16, lens=(0,))
    Oo, _ = O.attn_step(q, kb, vb, kc, vc, lens)
    ref = sdpa(q[0].transpose(1, 0, 2), kb[0].transpose(1, 0, 2), vb[0].transpose(1, 0, 2))  # torch default 1/sqrt(D)
    np.testing.assert_allclose(Oo[0], ref.transpose(1, 0, 2), rtol=1e-7, atol=1e-9)


@pytest.mark.parametrize("Hq,Hkv", [(4, 2), (8, 2), (6, 3), (4, 1)])
def test_gqa_equals_mha_with_repeated_kv_heads(Hq, Hkv):
    q, kb, vb, kc, vc, lens = make_case(B=2, S=3, Hq=Hq, Hkv=Hkv, D=8, lens=(7, 2), seed=3)
    Oo, Lo = O.attn_step(q, kb, vb, kc, vc, lens)
    g = Hq // Hkv
    for b in range(2):
        n = lens[b]
        K = np.concatenate([kc[b, :, :n], kb[b].transpose(1, 0, 2)], axis=1)   # [Hkv, n+S, D]
        V = np.concatenate([vc[b, :, :n], vb[b].transpose(1, 0, 2)], axis=1)
        K = np.repeat(K, g, axis=0)   # head h reads KV head h // g (repeat_interleave)
        V = np.repeat(V, g, axis=0)
        ref = sdpa(q[b].transpose(1, 0, 2), K, V, scale=O.default_scale(8))
        np.testing.assert_allclose(Oo[b], ref.transpose(1, 0, 2), rtol=1e-11, atol=1e-12)
        tq = torch.from_numpy(q[b].transpose(1, 0, 2).copy())
        scores = torch.einsum("hsd,hjd->hsj", tq, torch.from_numpy(K)) * O.default_scale(8)
        np.testing.assert_allclose(Lo[b], torch.logsumexp(scores, dim=-1).numpy(), rtol=1e-12)


def test_one_token_block_is_causal_decode():
    # S = 1 (AR mode): the step equals causal single-token decode at position L.
    rng = np.random.default_rng(11)
    for L in (0, 1, 9, 31):
        H, D = 3, 8
        x_k, x_v, x_q = (rng.standard_normal((H, L + 1, D)) for _ in range(3))
        causal = sdpa(x_q, x_k, x_v, is_causal=True, scale=O.default_scale(D))
        q = x_q[:, L:L + 1].transpose(1, 0, 2)[None]          # [1,1,H,D]
        kb = x_k[:, L:L + 1].transpose(1, 0, 2)[None]
        vb = x_v[:, L:L + 1].transpose(1, 0, 2)[None]
        kc = x_k[None, :, :max(L, 1)] if L else np.zeros((1, H, 1, D))
        vc = x_v[None, :, :max(L, 1)] if L else np.zeros((1, H, 1, D))
        Oo, _ = O.attn_step(q, kb, vb, kc, vc, np.array([L]))
        np.testing.assert_allclose(Oo[0, 0], causal[:, L], rtol=1e-12, atol=1e-13)


def test_block_rows_of_block_causal_full_sequence():
    # Full sequence [prefix ; block] with a block-causal mask: prefix rows are causal over the
    # prefix, block rows see everything. Block rows equal the step; prefix rows do not change
    # when the block content changes (the cached prefix is a function of the prefix only).
    rng = np.random.default_rng(5)
    H, D, L, S = 2, 8, 6, 4
    xk, xv, xq = (rng.standard_normal((H, L + S, D)) for _ in range(3))
    mask = np.zeros((L + S, L + S), dtype=bool)
    for i in range(L + S):
        for j in range(L + S):
            mask[i, j] = (j <= i) if i < L else True
    full = sdpa(xq, xk, xv, mask=mask, scale=O.default_scale(D))
    q = xq[:, L:].transpose(1, 0, 2)[None]
    kb = xk[:, L:].transpose(1, 0, 2)[None]
    vb = xv[:, L:].transpose(1, 0, 2)[None]
    Oo, _ = O.attn_step(q, kb, vb, xk[None, :, :L], xv[None, :, :L], np.array([L]))
    np.testing.assert_allclose(Oo[0], full[:, L:].transpose(1, 0, 2), rtol=1e-12, atol=1e-13)
    xk2, xv2 = xk.copy(), xv.copy()
    xk2[:, L:] = rng.standard_normal((H, S, D))
    xv2[:, L:] = rng.standard_normal((H, S, D))
    full2 = sdpa(xq, xk2, xv2, mask=mask, scale=O.default_scale(D))
    np.testing.assert_array_equal(full2[:, :L], full[:, :L])


def test_block_permutation_permutes_outputs():
    q, kb, vb, kc, vc, lens = make_case(B=2, S=6, Hq=4, Hkv=2, D=8, lens=(4, 9), seed=7)
    Oo, Lo = O.attn_step(q, kb, vb, kc, vc, lens)
    perm = np.random.default_rng(1).permutation(6)
    Op, Lp = O.attn_step(q[:, perm], kb[:, perm], vb[:, perm], kc, vc, lens)
    np.testing.assert_allclose(Op, Oo[:, perm], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(Lp, Lo[:, :, perm], rtol=1e-12)


def test_closed_forms():
    B, S, Hq, Hkv, D, L = 1, 3, 2, 1, 8, 5
    q, kb, vb, kc, vc, lens = make_case(B, S, Hq, Hkv, D, (L,), seed=9)
    # all keys identical -> uniform weights: O = mean of the visible V rows, LSE = s + ln(n)
    k = rnd(D, 99)
    kb1, kc1 = np.broadcast_to(k, kb.shape).copy(), np.broadcast_to(k, kc.shape).copy()
    Oo, Lo = O.attn_step(q, kb1, vb, kc1, vc, lens)
    Vall = np.concatenate([vc[0, 0, :L], vb[0, :, 0]], axis=0)
    for s, h in itertools.product(range(S), range(Hq)):
        np.testing.assert_allclose(Oo[0, s, h], Vall.mean(axis=0), rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(Lo[0, h, s], O.default_scale(D) * q[0, s, h] @ k + math.log(L + S), rtol=1e-12)
    # all V rows equal -> O = v
    v = rnd(D, 98)
    Oo, _ = O.attn_step(q, kb, np.broadcast_to(v, vb.shape).copy(), kc, np.broadcast_to(v, vc.shape).copy(), lens)
    np.testing.assert_allclose(Oo, np.broadcast_to(v, Oo.shape), rtol=1e-12, atol=1e-13)
    # one key with a huge score gap -> O = its V row, with no overflow
    q2 = np.zeros_like(q)
    q2[..., 0] = 4000.0
    kc2 = np.zeros_like(kc)
    kb2 = np.zeros_like(kb)
    kc2[0, 0, 2, 0] = 1.0        # score 4000/sqrt(8) ~ 1414 for prefix key 2 (exp overflows without the max shift)
    Oo, Lo = O.attn_step(q2, kb2, vb, kc2, vc, lens)
    assert np.all(np.isfinite(Oo))
    np.testing.assert_allclose(Oo[0, :, :], np.broadcast_to(vc[0, 0, 2], (S, Hq, D)), rtol=0, atol=1e-40)


@pytest.mark.parametrize("seed", range(4))
def test_split_invariance(seed):
    q, kb, vb, kc, vc, lens = make_case(B=2, S=5, Hq=4, Hkv=2, D=8, lens=(40, 3), seed=seed, lcap=40)
    Oo, Lo = O.attn_step(q, kb, vb, kc, vc, lens)
    rng = np.random.default_rng(seed + 100)

    def split(n):
        k = rng.integers(1, 7)
        cuts = sorted(rng.integers(0, n + 1, size=k))   # may create empty chunks
        return [0] + list(cuts) + [n]

    Oc, Lc = O.attn_step_chunked(q, kb, vb, kc, vc, lens, split)
    np.testing.assert_allclose(Oc, Oo, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(Lc, Lo, rtol=1e-12)


def test_tiny_brute_force():
    # pure-Python enumeration on tiny shapes: explicit exp / sums, no max subtraction
    for seed in range(3):
        rng = np.random.default_rng(seed)
        B, S, Hq, Hkv, D = 2, 3, 4, 2, 8
        lens = rng.integers(0, 6, size=B)
        q, kb, vb, kc, vc, _ = make_case(B, S, Hq, Hkv, D, tuple(lens), seed=seed + 20, lcap=5)
        Oo, Lo = O.attn_step(q, kb, vb, kc, vc, lens)
        tau = 1.0 / math.sqrt(D)
        for b, s, h in itertools.product(range(B), range(S), range(Hq)):
            g = h // (Hq // Hkv)
            keys = [(kc[b, g, j], vc[b, g, j]) for j in range(lens[b])] + [(kb[b, j, g], vb[b, j, g]) for j in range(S)]
            w = [math.exp(tau * sum(q[b, s, h, d] * k[d] for d in range(D))) for k, _ in keys]
            z = sum(w)
            for d in range(D):
                assert abs(Oo[b, s, h, d] - sum(wi * v[d] for wi, (_, v) in zip(w, keys)) / z) < 1e-6
            assert abs(Lo[b, h, s] - math.log(z)) < 1e-6


def test_sampled_rows_match_full():
    q, kb, vb, kc, vc, lens = make_case(B=2, S=4, Hq=8, Hkv=2, D=16, lens=(30, 11), seed=4, lcap=30)
    Oo, Lo = O.attn_step(q, kb, vb, kc, vc, lens)
    rows = [(0, 1, 3), (1, 3, 7), (1, 0, 0)]
    got = O.attn_rows(q, kb, vb, kc, vc, lens, rows)
    for (b, s, h) in rows:
        np.testing.assert_allclose(got[(b, s, h)][0], Oo[b, s, h], rtol=1e-13, atol=1e-15)
        assert abs(got[(b, s, h)][1] - Lo[b, h, s]) < 1e-12


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_sampled_rows_on_bf16_bits_match_decoded_full(D, causal):
    """attn_rows' bf16 branch (uint16 bit patterns decoded one (sequence, KV head) slab at a time,
    as the full-size GPU checks use it) gives the rows of attn_step run on the whole decoded
    tensors: every (b, s, h), ragged prefix lengths including 0, both attention modes."""
    from block_diffusion_lm_amd import inputs as I
    w = I.small_workload("rows-bits", B=3, Hq=8, Hkv=2, D=D, S=5, prefix_len=70, wid=900 + D + int(causal))
    lens = np.array([70, 0, 33], np.int32)
    inp = I.attn_inputs(w, lens=lens)
    assert inp["q"].dtype == np.uint16
    f = {k: O.bf16_to_f64(inp[k]) for k in ("q", "k_blk", "v_blk", "k_cache", "v_cache")}
    Oo, Lo = O.attn_step(f["q"], f["k_blk"], f["v_blk"], f["k_cache"], f["v_cache"], lens, causal=causal)
    rows = [(b, s, h) for b in range(3) for s in range(5) for h in range(8)]
    got = O.attn_rows(inp["q"], inp["k_blk"], inp["v_blk"], inp["k_cache"], inp["v_cache"], lens, rows, causal=causal)
    assert set(got) == set(rows)
    for (b, s, h) in rows:
        np.testing.assert_allclose(got[(b, s, h)][0], Oo[b, s, h], rtol=1e-12, atol=1e-14)
        assert abs(got[(b, s, h)][1] - Lo[b, h, s]) < 1e-12


def test_inactive_sequences_are_skipped():
    q, kb, vb, kc, vc, lens = make_case(B=2, S=2, Hq=2, Hkv=1, D=4, lens=(3, 3), seed=2)
    Oo, _ = O.attn_step(q, kb, vb, kc, vc, lens, active=[1, 0])
    assert np.all(np.isfinite(Oo[0])) and np.all(np.isnan(Oo[1]))


def test_bf16_decoding_and_scale():
    bits = np.array([0x3F80, 0xBF80, 0x4000, 0x0000, 0x3FC0, 0x7F7F], dtype=np.uint16)
    np.testing.assert_array_equal(O.bf16_to_f64(bits), [1.0, -1.0, 2.0, 0.0, 1.5, 3.3895313892515355e38])
    assert O.default_scale(128) == float(np.float32(1 / math.sqrt(128)))
    assert O.default_scale(64) == 0.125


# ------------------------------------------------------------------------------------ unmasking
def test_constant_row():
    m, a, Z, p = O.vocab_reduce(np.full(4096, 1.25))
    assert a == 0 and Z == 4096.0 and p == 1.0 / 4096


@pytest.mark.parametrize("V,delta", [(4096, 3.0), (131072, 14.0), (1000, -2.0)])
def test_single_peak_closed_form(V, delta):
    row = np.zeros(V)
    row[V // 3] = delta
    _, a, _, p = O.vocab_reduce(row)
    expect_a = V // 3 if delta > 0 else 0
    assert a == expect_a
    if delta > 0:
        assert abs(p - math.exp(delta) / (math.exp(delta) + V - 1)) <= 1e-15
    else:
        assert abs(p - 1.0 / (math.exp(delta) + V - 1)) <= 1e-15


def test_vs_library_softmax():
    x = np.random.default_rng(3).standard_normal((6, 777)) * 3
    for r in range(6):
        _, a, _, p = O.vocab_reduce(x[r])
        sm = torch.softmax(torch.from_numpy(x[r]), dim=0)
        assert a == int(np.argmax(x[r]))   # numpy: first occurrence
        assert abs(p - float(sm.max())) < 1e-15


def test_reduction_is_shift_invariant():
    # adding a constant to every logit of a row changes neither the argmax nor the softmax maximum
    # (the maximum is subtracted before exponentiating; +-1000 overflows exp otherwise)
    row = np.random.default_rng(11).standard_normal(4099) * 4
    _, a0, _, p0 = O.vocab_reduce(row)
    for c in (1000.0, -1000.0, 1e6):
        _, a, _, p = O.vocab_reduce(row + c)
        assert a == a0
        assert abs(p - p0) <= 1e-9 * p0


def test_argmax_ties_lowest_index():
    row = np.random.default_rng(0).standard_normal(500)
    row[[37, 101, 499]] = 9.0
    assert O.vocab_reduce(row)[1] == 37
    row[[5]] = 9.0
    assert O.vocab_reduce(row)[1] == 5


def _p_rows(ps):
    """Logit rows with a prescribed max probability: V = 2 rows [ln(p/(1-p)), 0]."""
    rows = []
    for p in ps:
        rows.append([math.log(p / (1 - p)), 0.0] if p != 0.5 else [0.0, 0.0])
    return np.array(rows)


def test_commit_threshold_is_strict():
    logits = np.array([[0.0, 0.0], [1.0, 0.0], [0.0, 0.0], [0.0, 0.0]])   # p = 0.5, 0.731, 0.5, 0.5
    res = O.confidence_unmask(logits, np.array([1, 1, 1, 1], np.uint8), np.zeros(4, np.int32), S=4, gamma=0.5)
    np.testing.assert_array_equal(res["mask"], [1, 0, 1, 1])
    res = O.confidence_unmask(logits[[0, 2, 3, 0]], np.array([1, 1, 1, 1], np.uint8), np.zeros(4, np.int32), S=4, gamma=0.5)
    np.testing.assert_array_equal(res["mask"], [0, 1, 1, 1])      # nobody > 0.5 -> fallback, tie -> lowest s
    assert list(res["n_commit"]) == [1]


def test_commit_rule_cases():
    S = 4
    p = np.array([0.2, 0.95, 0.91, 0.3,   0.5, 0.6, 0.55, 0.1,   0.99, 0.99, 0.0, 0.0])
    a = np.arange(12) + 100
    mask = np.array([1, 1, 1, 1,   1, 1, 0, 1,   0, 0, 0, 0], np.uint8)
    tok = np.full(12, -7, np.int32)
    m2, t2, n = O.commit(p, a, mask, tok, S, gamma=0.9)
    np.testing.assert_array_equal(m2, [1, 0, 0, 1,   1, 0, 0, 1,   0, 0, 0, 0])
    np.testing.assert_array_equal(t2, [-7, 101, 102, -7,   -7, 105, -7, -7,   -7, -7, -7, -7])
    np.testing.assert_array_equal(n, [2, 1, 0])
    # without min_commit the middle sequence commits nothing
    m3, _, n3 = O.commit(p, a, mask, tok, S, gamma=0.9, min_commit=False)
    np.testing.assert_array_equal(n3, [2, 0, 0])
    # commit_all commits every masked position regardless of p
    m4, t4, n4 = O.commit(p, a, mask, tok, S, gamma=0.9, commit_all=True)
    assert m4.sum() == 0 and list(n4) == [4, 3, 0]
    # gamma promoted from float32: p equal to float64(0.9) is above float32(0.9) = 0.899999976...
    m5, _, _ = O.commit(np.array([0.9, 0.1]), np.array([1, 2]), np.array([1, 1], np.uint8), np.zeros(2, np.int32), 2, 0.9)
    np.testing.assert_array_equal(m5, [0, 1])


def test_gamma_zero_and_one():
    x = np.random.default_rng(8).standard_normal((12, 300))
    mask = np.array([1] * 12, np.uint8)
    r0 = O.confidence_unmask(x, mask, np.zeros(12, np.int32), S=4, gamma=0.0)
    assert r0["mask"].sum() == 0                         # one-step parallel greedy decode
    np.testing.assert_array_equal(r0["tokens"], np.argmax(x, axis=1))
    r1 = O.confidence_unmask(x, mask, np.zeros(12, np.int32), S=4, gamma=1.0)
    assert list(r1["n_commit"]) == [1, 1, 1]             # only the fallback fires
    for b in range(3):
        pb = [torch.softmax(torch.from_numpy(x[b * 4 + s]), 0).max().item() for s in range(4)]
        assert r1["mask"][b * 4 + int(np.argmax(pb))] == 0


def test_bf16_logits_path():
    from block_diffusion_lm_amd.inputs import f32_to_bf16_bits
    x = (np.random.default_rng(4).standard_normal((3, 64)) * 3).astype(np.float32)
    bits = f32_to_bf16_bits(x)
    p, a = O.confidences(bits, np.ones(3, np.uint8), decode=O.bf16_to_f64)
    dec = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    for r in range(3):
        assert a[r] == int(np.argmax(dec[r]))
        assert abs(p[r] - float(torch.softmax(torch.from_numpy(dec[r]), 0).max())) < 1e-15


def test_margins_report_near_ties():
    g = float(np.float32(0.9))
    p = np.array([g * (1 + 5e-5), 0.1, 0.5, 0.5 * (1 - 2e-5)])
    nt = O.near_ties(p, np.array([1, 1, 1, 1], np.uint8), S=2, gamma=0.9)
    kinds = sorted(k for k, _, _ in nt)
    assert kinds == ["fallback", "gamma"]


# ------------------------------------------------------------------------------------ loop
def _loop_case(seed, B=3, S=8, V=50, T=6, gamma=0.6, Hq=4, Hkv=2, D=8, L=5, scale=3.0):
    rng = np.random.default_rng(seed)
    mask0 = (rng.random(B * S) < 0.8).astype(np.uint8)
    mask0[:S] = 1
    kc = rng.standard_normal((B, Hkv, L, D))
    vc = rng.standard_normal((B, Hkv, L, D))
    lens = np.full(B, L, np.int32)
    step = {}
    for t in range(T):
        r = np.random.default_rng([seed, t])
        step[t] = {"q": r.standard_normal((B, S, Hq, D)), "k_blk": r.standard_normal((B, S, Hkv, D)),
                   "v_blk": r.standard_normal((B, S, Hkv, D)), "logits": r.standard_normal((B * S, V)) * scale}
    return mask0, kc, vc, lens, step


@pytest.mark.parametrize("seed", range(5))
def test_loop_invariants(seed):
    B, S, T = 3, 8, 6
    mask0, kc, vc, lens, step = _loop_case(seed, B=B, S=S, T=T)
    res = O.denoise_block(T, 0, B, S, mask0, np.full(B * S, -1, np.int32), lambda t: step[t], kc, vc, lens, 0.6)
    ts = sorted(res["outs"])
    for i, t in enumerate(ts):
        m = res["masks"][t]
        m_next = res["masks"][ts[i + 1]] if i + 1 < len(ts) else res["mask"]
        assert np.all(m_next <= m)                                   # mask never increases
        act = m.reshape(B, S).any(axis=1)
        np.testing.assert_array_equal(act, res["active"][t])
        for b in range(B):
            assert (res["commits"][t, b] >= 1) if act[b] else (res["commits"][t, b] == 0)
        turned = (m == 1) & (m_next == 0)
        np.testing.assert_array_equal(turned.reshape(B, S).sum(axis=1), res["commits"][t])
        # committed tokens equal that step's argmax of the logits (library argmax: first maximum)
        np.testing.assert_array_equal(res["tokens"][turned], np.argmax(step[t]["logits"][turned], axis=1))
    assert res["mask"].sum() == 0                              # commit_all at t = T-1
    assert res["commits"].sum() == mask0.sum()
    nm = mask0.reshape(B, S).sum(axis=1)
    assert np.all(res["steps_used"] <= np.minimum(T, nm))
    assert np.all(res["steps_used"] >= 1)


def test_loop_mask_monotone_and_tokens_are_argmax():
    B, S, T = 2, 6, 5
    mask0, kc, vc, lens, step = _loop_case(42, B=B, S=S, T=T, gamma=0.7)
    mask = mask0.copy()
    tokens = np.full(B * S, -1, np.int32)
    for t in range(T):
        res = O.confidence_unmask(step[t]["logits"], mask, tokens, S, 0.7, commit_all=(t == T - 1))
        assert np.all(res["mask"] <= mask)
        turned = (mask == 1) & (res["mask"] == 0)
        assert np.all(res["tokens"][turned] == np.argmax(step[t]["logits"][turned], axis=1))
        assert np.all(res["tokens"][~turned] == tokens[~turned])
        mask, tokens = res["mask"], res["tokens"]
    full = O.denoise_block(T, 0, B, S, mask0, np.full(B * S, -1, np.int32), lambda t: step[t], kc, vc, lens, 0.7)
    np.testing.assert_array_equal(full["tokens"], tokens)


def test_loop_sequential_decode_with_gamma_one():
    # gamma = 1 never passes: exactly one commit per active sequence per step (sequential
    # top-confidence decoding); steps_used = number of masked positions.
    B, S, T = 2, 5, 5
    mask0, kc, vc, lens, step = _loop_case(7, B=B, S=S, T=T, gamma=1.0)
    res = O.denoise_block(T, 0, B, S, mask0, np.zeros(B * S, np.int32), lambda t: step[t], kc, vc, lens, 1.0,
                          final_commit_all=False)
    nm = mask0.reshape(B, S).sum(axis=1)
    np.testing.assert_array_equal(res["steps_used"], nm)
    for t in range(T):
        for b in range(B):
            assert res["commits"][t, b] == (1 if t < nm[b] else 0)


def test_loop_resume_from_t0():
    B, S, T = 2, 6, 6
    mask0, kc, vc, lens, step = _loop_case(3, B=B, S=S, T=T, gamma=0.8)
    full = O.denoise_block(T, 0, B, S, mask0, np.zeros(B * S, np.int32), lambda t: step[t], kc, vc, lens, 0.8)
    first = O.denoise_block(2, 0, B, S, mask0, np.zeros(B * S, np.int32), lambda t: step[t], kc, vc, lens, 0.8,
                            final_commit_all=False)
    rest = O.denoise_block(T, 2, B, S, first["mask"], first["tokens"], lambda t: step[t], kc, vc, lens, 0.8)
    np.testing.assert_array_equal(rest["tokens"], full["tokens"])
    np.testing.assert_array_equal(np.maximum(first["steps_used"], rest["steps_used"]), full["steps_used"])


def test_gamma_zero_loop_finishes_in_one_step():
    B, S, T = 2, 6, 4
    mask0, kc, vc, lens, step = _loop_case(9, B=B, S=S, T=T)
    res = O.denoise_block(T, 0, B, S, mask0, np.zeros(B * S, np.int32), lambda t: step[t], kc, vc, lens, 0.0)
    assert list(res["steps_used"]) == [1, 1] and sorted(res["outs"]) == [0]


# ------------------------------------------------------------------------------------ planted slips
def _fails(fn, *a):
    try:
        fn(*a)
    except (AssertionError, IndexError, ValueError, FloatingPointError):
        return True
    return False


# ------------------------------------------------------------ context-tower pass, append, LinearSpec
def test_causal_pass_without_prefix_is_causal_attention():
    # L = 0: block position s sees block keys 0..s -- torch's causal SDPA on the block alone.
    q, kb, vb, kc, vc, lens = make_case(B=2, S=6, Hq=4, Hkv=4, D=8, lens=(0, 0), seed=21)
    Oo, _ = O.attn_step(q, kb, vb, kc, vc, lens, causal=True)
    for b in range(2):
        ref = sdpa(q[b].transpose(1, 0, 2), kb[b].transpose(1, 0, 2), vb[b].transpose(1, 0, 2), is_causal=True,
                   scale=O.default_scale(8))
        np.testing.assert_allclose(Oo[b], ref.transpose(1, 0, 2), rtol=1e-12, atol=1e-13)


def test_causal_pass_with_prefix_is_the_full_causal_sequence():
    # [prefix ; block] under one causal mask: the block's rows are the causal pass over the block.
    rng = np.random.default_rng(22)
    H, D, L, S = 3, 8, 7, 5
    xk, xv, xq = (rng.standard_normal((H, L + S, D)) for _ in range(3))
    full = sdpa(xq, xk, xv, is_causal=True, scale=O.default_scale(D))
    Oo, _ = O.attn_step(xq[:, L:].transpose(1, 0, 2)[None], xk[:, L:].transpose(1, 0, 2)[None],
                        xv[:, L:].transpose(1, 0, 2)[None], xk[None, :, :L], xv[None, :, :L], np.array([L]),
                        causal=True)
    np.testing.assert_allclose(Oo[0], full[:, L:].transpose(1, 0, 2), rtol=1e-12, atol=1e-13)


def test_causal_pass_is_incremental_decode_over_the_appended_cache():
    # Row s of the causal pass equals a one-token step at position len + s over the cache into
    # which block rows 0..s-1 were appended: appending the block is exact for what follows.
    q, kb, vb, kc, vc, lens = make_case(B=2, S=5, Hq=4, Hkv=2, D=8, lens=(6, 3), seed=23, lcap=12)
    Oc, Lc = O.attn_step(q, kb, vb, kc, vc, lens, causal=True)
    for s in range(5):
        kc2, vc2, ln2 = kc, vc, lens
        if s:
            kc2, vc2, ln2 = O.kv_append(kc, vc, lens, kb[:, :s], vb[:, :s])
        o1, l1 = O.attn_step(q[:, s:s + 1], kb[:, s:s + 1], vb[:, s:s + 1], kc2, vc2, ln2)
        np.testing.assert_allclose(o1[:, 0], Oc[:, s], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(l1[:, :, 0], Lc[:, :, s], rtol=1e-12, atol=1e-13)


def test_last_causal_row_is_the_bidirectional_row():
    q, kb, vb, kc, vc, lens = make_case(B=2, S=4, Hq=4, Hkv=2, D=8, lens=(5, 0), seed=24)
    Oc, _ = O.attn_step(q, kb, vb, kc, vc, lens, causal=True)
    Ob, _ = O.attn_step(q, kb, vb, kc, vc, lens)
    np.testing.assert_array_equal(Oc[:, -1], Ob[:, -1])
    assert not np.allclose(Oc[:, 0], Ob[:, 0])


def test_kv_append_rows_and_lengths():
    rng = np.random.default_rng(25)
    B, Hkv, Lcap, D, S = 3, 2, 10, 4, 3
    kc = rng.integers(0, 1 << 16, (B, Hkv, Lcap, D)).astype(np.uint16)
    vc = rng.integers(0, 1 << 16, (B, Hkv, Lcap, D)).astype(np.uint16)
    kn = rng.integers(0, 1 << 16, (B, S, Hkv, D)).astype(np.uint16)
    vn = rng.integers(0, 1 << 16, (B, S, Hkv, D)).astype(np.uint16)
    lens = np.array([0, 4, 7], dtype=np.int32)
    k2, v2, l2 = O.kv_append(kc, vc, lens, kn, vn, active=[1, 0, 1])
    np.testing.assert_array_equal(l2, [3, 4, 10])
    for b, n in ((0, 0), (2, 7)):
        for g in range(Hkv):
            np.testing.assert_array_equal(k2[b, g, n:n + S], kn[b, :, g])
            np.testing.assert_array_equal(v2[b, g, n:n + S], vn[b, :, g])
            np.testing.assert_array_equal(k2[b, g, :n], kc[b, g, :n])
            np.testing.assert_array_equal(k2[b, g, n + S:], kc[b, g, n + S:])
    np.testing.assert_array_equal(k2[1], kc[1])
    with pytest.raises(ValueError):
        O.kv_append(kc, vc, np.array([8, 0, 0], dtype=np.int32), kn, vn)


def test_spec_accept_cases():
    S = 4
    draft = np.array([5, 6, 7, 8,   1, 2, 3, 4,   3, 3, 3, 3])
    first = np.array([5, 9, 3])
    pa = np.array([6, 7, 8, 2,      2, 3, 4, 5,   3, 3, 3, 1])
    r = O.spec_accept(draft, first, pa, S)
    # seq 0: every draft token is AR's choice -> all commit, next choice from the last position
    # seq 1: position 0 differs -> AR's own choice (9) commits alone
    # seq 2: all equal -> all commit
    np.testing.assert_array_equal(r["n_commit"], [4, 1, 4])
    np.testing.assert_array_equal(r["tokens"], [5, 6, 7, 8, 9, -1, -1, -1, 3, 3, 3, 3])
    np.testing.assert_array_equal(r["next_choice"], [2, -1, 1])
    r = O.spec_accept(np.array([5, 6, 0, 8]), np.array([5]), np.array([6, 7, 8, 2]), S)
    np.testing.assert_array_equal(r["tokens"], [5, 6, 7, -1])
    assert r["n_commit"][0] == 3 and r["next_choice"][0] == -1


def test_spec_accept_is_lossless_against_ar_decoding():
    # A toy deterministic AR model (next token = hash of the last three tokens). Drafts with
    # random corruptions, checked block by block with the causal pass simulated from the model,
    # reproduce the model's own greedy decode exactly, and every check commits >= 1 token.
    V, S, N = 11, 5, 60

    def f(ctx):
        return (7 * ctx[-1] + 3 * ctx[-2] + ctx[-3] * ctx[-1] + 5) % V

    rng = np.random.default_rng(26)
    ar = [1, 2, 3]
    while len(ar) < 3 + N + S:
        ar.append(f(ar))
    out = [1, 2, 3]
    while len(out) < 3 + N:
        pos = len(out)
        truth = ar[pos:pos + S]
        draft = [t if rng.random() < 0.7 else int(rng.integers(V)) for t in truth]
        ctx = list(out)
        pa = []
        for i in range(S):        # causal pass over the draft: the model's choice after draft[:i+1]
            pa.append(f(ctx + draft[:i + 1]))
        r = O.spec_accept(np.array(draft), np.array([f(ctx)]), np.array(pa), S)
        n = int(r["n_commit"][0])
        assert n >= 1
        out += [int(t) for t in r["tokens"][:n]]
        if draft == truth:
            assert n == S and r["next_choice"][0] == f(out)
    assert out[:3 + N] == ar[:3 + N]


# -------------------------------------------------------------------------------- loop halting
def test_loop_halt_closed_forms_and_library_norm():
    rng = np.random.default_rng(31)
    hp = rng.standard_normal((4, 7, 16))
    a = np.array([0.5, -0.01, 0.0, 2.0])
    hc = hp * (1 + a)[:, None, None]                         # scaled copy: rel = |a|
    rel, halt = O.loop_halt(hp, hc, 0.05, 3, 10)
    np.testing.assert_allclose(rel, np.abs(a), rtol=1e-12, atol=1e-15)
    np.testing.assert_array_equal(halt, [0, 1, 1, 0])
    d = rng.standard_normal((4, 7, 16))
    hc2 = hp + d
    rel2, _ = O.loop_halt(hp, hc2, 0.05, 3, 10)
    ref = np.linalg.norm(d.reshape(4, -1), axis=1) / np.linalg.norm(hp.reshape(4, -1), axis=1)
    np.testing.assert_allclose(rel2, ref, rtol=1e-12)
    # the change is per sequence: perturbing one sequence moves only its value
    hc3 = hc2.copy()
    hc3[2] += 1.0
    rel3, _ = O.loop_halt(hp, hc3, 0.05, 3, 10)
    np.testing.assert_array_equal(rel3[[0, 1, 3]], rel2[[0, 1, 3]])
    assert rel3[2] != rel2[2]


def test_loop_halt_budget_and_degenerate_states():
    hp = np.zeros((3, 5))
    hc = np.zeros((3, 5))
    hc[1, 0] = 1.0
    hp[2] = 1.0
    hc[2] = 1.0
    rel, halt = O.loop_halt(hp, hc, 1e-3, 1, 4)
    assert rel[0] == 0 and np.isinf(rel[1]) and rel[2] == 0
    np.testing.assert_array_equal(halt, [1, 0, 1])
    _, halt = O.loop_halt(hp, hc, 1e-3, 4, 4)                 # budget reached: every sequence halts
    np.testing.assert_array_equal(halt, [1, 1, 1])
    # strict comparison at a float32 epsilon
    hp = np.ones((1, 4))
    hc = hp * (1 + 0.25)
    _, halt = O.loop_halt(hp, hc, 0.25, 1, 9)
    assert halt[0] == 0


def test_planted_mistakes_are_caught(monkeypatch):
    """Plant plausible slips in the oracle (on the CPU) and check that some pin fails."""
    orig = {k: getattr(O, k) for k in ("kv_head_of", "default_scale", "vocab_reduce", "keys_values",
                                       "softmax_attention", "merge_partials", "commit", "causal_visible",
                                       "kv_append", "spec_accept", "loop_halt")}

    def check(name, bad, pins):
        monkeypatch.setattr(O, name, bad)
        with np.errstate(all="ignore"):
            assert any(_fails(*p) for p in pins), f"no pin caught a slip in {name}"
        monkeypatch.setattr(O, name, orig[name])

    check("kv_head_of", lambda h, Hq, Hkv: h % Hkv, [(test_gqa_equals_mha_with_repeated_kv_heads, 8, 2)])
    check("default_scale", lambda D: 1.0 / D, [(test_default_scale_is_inverse_sqrt_d,)])

    def no_block_keys(k_blk, v_blk, k_cache, v_cache, prefix_len, b, g):
        n = int(prefix_len[b])
        return k_cache[b, g, :max(n, 1)], v_cache[b, g, :max(n, 1)]
    check("keys_values", no_block_keys, [(test_no_prefix_is_plain_bidirectional_attention,)])

    def no_prefix(k_blk, v_blk, k_cache, v_cache, prefix_len, b, g):
        return k_blk[b, :, g], v_blk[b, :, g]
    check("keys_values", no_prefix, [(test_one_token_block_is_causal_decode,)])

    def transposed(Qr, K, V, tau, visible=None):
        o, l = orig["softmax_attention"](Qr, K, V, tau, visible)
        return o[:, ::-1].copy(), l
    check("softmax_attention", transposed, [(test_no_prefix_is_plain_bidirectional_attention,)])

    def no_max_sub(Qr, K, V, tau, visible=None):
        e = np.exp(tau * (Qr @ K.T))
        if visible is not None:
            e = np.where(visible, e, 0.0)
        z = e.sum(axis=1, keepdims=True)
        return (e / z) @ V, np.log(z[:, 0])
    check("softmax_attention", no_max_sub, [(test_closed_forms,)])

    def bad_merge(parts):
        M = np.max(np.stack([p[0] for p in parts]), axis=0)
        num = sum(p[2] for p in parts)
        den = sum(p[1] for p in parts)
        return num / den[:, None], M + np.log(den)
    check("merge_partials", bad_merge, [(test_split_invariance, 0)])

    def last_index(row):
        m, a, Z, p = orig["vocab_reduce"](row)
        return m, int(np.flatnonzero(row == m)[-1]), Z, p
    check("vocab_reduce", last_index, [(test_argmax_ties_lowest_index,)])

    def ge_commit(p, a, mask, tokens, S, gamma, min_commit=True, commit_all=False):
        return orig["commit"](p, a, mask, tokens, S, float(np.nextafter(np.float32(gamma), np.float32(-1))),
                              min_commit, commit_all)
    check("commit", ge_commit, [(test_commit_threshold_is_strict,)])

    def last_fallback(p, a, mask, tokens, S, gamma, min_commit=True, commit_all=False):
        return orig["commit"](p, a, mask, tokens, S, gamma, min_commit, commit_all) if commit_all else \
            orig["commit"](p[::-1].copy(), a[::-1].copy(), mask[::-1].copy(), tokens[::-1].copy(), S, gamma,
                           min_commit, commit_all)
    check("commit", last_fallback, [(test_commit_threshold_is_strict,), (test_commit_rule_cases,)])

    def strict_causal(S, n_prefix, rows_s):
        j = np.arange(n_prefix + S)
        return np.stack([(j < n_prefix) | (j - n_prefix < max(s, 1)) for s in rows_s])
    check("causal_visible", strict_causal, [(test_causal_pass_without_prefix_is_causal_attention,)])

    def append_one_late(k_cache, v_cache, prefix_len, k_new, v_new, active=None):
        kc, vc, ln = orig["kv_append"](k_cache, v_cache, np.asarray(prefix_len) + 1, k_new, v_new, active)
        return kc, vc, ln - 1
    check("kv_append", append_one_late, [(test_kv_append_rows_and_lengths,)])

    def no_correction(draft, first_choice, pass_argmax, S):
        r = orig["spec_accept"](draft, first_choice, pass_argmax, S)
        for b in range(len(r["n_commit"])):
            if r["n_commit"][b] < S or r["next_choice"][b] < 0:
                r["n_commit"][b] -= 1
        return r
    check("spec_accept", no_correction, [(test_spec_accept_cases,)])

    def unshifted(draft, first_choice, pass_argmax, S):
        pa = np.asarray(pass_argmax).reshape(-1, S)
        shifted = np.concatenate([pa[:, 1:], pa[:, -1:]], axis=1).reshape(-1)
        return orig["spec_accept"](draft, first_choice, shifted, S)
    check("spec_accept", unshifted, [(test_spec_accept_is_lossless_against_ar_decoding,)])

    def halt_le(h_prev, h_cur, eps, iteration, max_iter):
        rel, halt = orig["loop_halt"](h_prev, h_cur, eps, iteration, max_iter)
        return rel, (halt | (rel <= float(np.float32(eps)))).astype(np.uint8)
    check("loop_halt", halt_le, [(test_loop_halt_budget_and_degenerate_states,)])

    def halt_squared(h_prev, h_cur, eps, iteration, max_iter):
        rel, halt = orig["loop_halt"](h_prev, h_cur, eps, iteration, max_iter)
        return rel ** 2, halt
    check("loop_halt", halt_squared, [(test_loop_halt_closed_forms_and_library_norm,)])

    # the commit rule's flags and mask: commit_all ignored, the at-least-one fallback dropped,
    # unmasked positions committed too
    def no_commit_all(p, a, mask, tokens, S, gamma, min_commit=True, commit_all=False):
        return orig["commit"](p, a, mask, tokens, S, gamma, min_commit, False)
    check("commit", no_commit_all, [(test_commit_rule_cases,), (test_gamma_zero_loop_finishes_in_one_step,)])

    def no_fallback(p, a, mask, tokens, S, gamma, min_commit=True, commit_all=False):
        return orig["commit"](p, a, mask, tokens, S, gamma, False, commit_all)
    check("commit", no_fallback, [(test_commit_rule_cases,), (test_gamma_zero_and_one,)])

    def no_shift(row):
        z = float(np.sum(np.exp(row)))
        m = float(np.max(row))
        return m, int(np.flatnonzero(row == m)[0]), z, float(np.exp(m)) / z
    check("vocab_reduce", no_shift, [(test_reduction_is_shift_invariant,)])

    def ignores_mask(p, a, mask, tokens, S, gamma, min_commit=True, commit_all=False):
        return orig["commit"](p, a, np.ones_like(mask), tokens, S, gamma, min_commit, commit_all)
    check("commit", ignores_mask, [(test_commit_rule_cases,), (test_loop_invariants, 0)])

    # a causal mask inside the block in the bidirectional step; sequence 0's cache for every sequence
    def causal_inside(Qr, K, V, tau, visible=None):
        if visible is None:
            S, n = Qr.shape[0], K.shape[0]
            visible = O.causal_visible(S, n - S, range(S))
        return orig["softmax_attention"](Qr, K, V, tau, visible)
    check("softmax_attention", causal_inside, [(test_block_permutation_permutes_outputs,),
                                               (test_no_prefix_is_plain_bidirectional_attention,)])

    def first_cache(k_blk, v_blk, k_cache, v_cache, prefix_len, b, g):
        return orig["keys_values"](k_blk, v_blk, k_cache[:1].repeat(k_cache.shape[0], 0),
                                   v_cache[:1].repeat(v_cache.shape[0], 0), prefix_len, b, g)
    check("keys_values", first_cache, [(test_tiny_brute_force,)])

    # the loop commits everything at every step instead of at the last one
    orig_cu = O.confidence_unmask
    monkeypatch.setattr(O, "confidence_unmask", lambda *args, **kw: orig_cu(*args, **{**kw, "commit_all": True}))
    with np.errstate(all="ignore"):
        assert _fails(test_loop_sequential_decode_with_gamma_one), "no pin caught commit-all at every step"
    monkeypatch.setattr(O, "confidence_unmask", orig_cu)
