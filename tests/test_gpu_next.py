"""GPU parity of the rows after the denoise step: the context tower's causal pass over a committed
block (bd_attn_step in causal mode), the append of the block to the prefix cache (bd_kv_append)
and the self-speculation check (bd_spec_verify), each against the float64 oracle through the C
ABI. Attention within the bf16 tolerance; cache rows, lengths, committed tokens and counts
bit-exact."""
import numpy as np
import pytest
import torch

import block_diffusion_lm_amd as bd
from block_diffusion_lm_amd import inputs as I
from oracle import bd_oracle as O
from tests.gpu_util import LSE_ATOL, assert_attn_close, bf16_f64, dev, dev_bf16, host_f64, oracle_attn_all

pytestmark = pytest.mark.gpu


def causal_case(name, B, Hq, Hkv, D, S, L, wid):
    w = I.small_workload(name, B=B, Hq=Hq, Hkv=Hkv, D=D, S=S, prefix_len=L, wid=wid)
    return w, I.attn_inputs(w)


def run_attn(inp, **kw):
    t = {k: dev_bf16(inp[k]) for k in ("q", "k_blk", "v_blk", "k_cache", "v_cache")}
    ln = dev(inp["prefix_len"])
    out, lse = bd.attn_step(t["q"], t["k_blk"], t["v_blk"], t["k_cache"], t["v_cache"], ln, **kw)
    torch.cuda.synchronize()
    return host_f64(out), lse.cpu().numpy().astype(np.float64)


def oracle_attn(inp, causal):
    f = {k: bf16_f64(inp[k]) for k in ("q", "k_blk", "v_blk", "k_cache", "v_cache")}
    return O.attn_step(f["q"], f["k_blk"], f["v_blk"], f["k_cache"], f["v_cache"], inp["prefix_len"], causal=causal)


CAUSAL = [
    # name, B, Hq, Hkv, D, S, prefix_len
    ("no-prefix-S16", 2, 8, 2, 64, 16, 0),
    ("ragged-d128", 3, 32, 2, 128, 16, (1, 700)),
    ("S64-g4", 1, 16, 4, 128, 64, 190),
    # a chunk that starts inside the block: rows before it see no key of that chunk
    ("S64-late-chunk", 2, 8, 8, 128, 64, 100),
    ("S1", 2, 32, 8, 128, 1, (60, 300)),
    ("S32-two-row-tiles", 1, 32, 2, 128, 32, 333),
]


@pytest.mark.parametrize("case", CAUSAL, ids=[c[0] for c in CAUSAL])
@pytest.mark.parametrize("num_splits", [0, 1, 3])
def test_causal_pass_matches_oracle(case, num_splits):
    name, B, Hq, Hkv, D, S, L = case
    w, inp = causal_case(name, B, Hq, Hkv, D, S, L, 300 + CAUSAL.index(case))
    print(f"[causal] {name} splits={num_splits} lens={inp['prefix_len'].tolist()}", flush=True)
    got, lse = run_attn(inp, num_splits=num_splits, causal=True)
    ref, ref_lse = oracle_attn(inp, causal=True)
    assert_attn_close(got, ref, name)
    np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=LSE_ATOL)


def test_causal_last_row_equals_bidirectional_and_first_rows_differ():
    w, inp = causal_case("last-row", 2, 32, 2, 128, 16, 500, 310)
    gc, _ = run_attn(inp, causal=True)
    gb, _ = run_attn(inp)
    np.testing.assert_array_equal(gc[:, -1], gb[:, -1])   # same keys, same kernel path: same bits
    assert np.abs(gc[:, 0] - gb[:, 0]).max() > 1e-3


@pytest.mark.parametrize("name", ["decode", "long"])
def test_causal_full_size(name):
    """The context tower's pass at full size (the decode and long workloads' shapes in causal mode):
    every element of out and lse against the oracle."""
    w = I.WORKLOADS[name]
    lens = I.prefix_lengths(w)
    inp = I.attn_inputs(w, lens=lens)
    print(f"[causal] full-size {name}", flush=True)
    got, lse = run_attn(inp, causal=True)
    ref, ref_lse = oracle_attn_all(inp, causal=True)
    assert_attn_close(got, ref, f"{name} causal")
    np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=LSE_ATOL)


def capacity_cache(w, lens, extra):
    c = I.prefix_cache(w, lens)
    out = {}
    for k, v in c.items():
        big = np.zeros(v.shape[:2] + (v.shape[2] + extra,) + v.shape[3:], dtype=np.uint16)
        big[:, :, :v.shape[2]] = v
        out[k] = big
    return out


APPEND_SHAPES = [
    # B, Hq, Hkv, D, S: one launch per call up to 2048 16-byte units of K per sequence (one to
    # eight per thread of the sequence's workgroup), two launches above
    (3, 8, 2, 128, 16),
    (3, 4, 1, 64, 5),
    (3, 16, 8, 128, 16),
    (3, 16, 8, 128, 32),
]


@pytest.mark.parametrize("shape", APPEND_SHAPES, ids=[f"B{s[0]}-Hkv{s[2]}-D{s[3]}-S{s[4]}" for s in APPEND_SHAPES])
@pytest.mark.parametrize("active", [None, [1, 0, 1]])
def test_kv_append_bit_exact(active, shape):
    B, Hq, Hkv, D, S = shape
    w = I.small_workload("append", B=B, Hq=Hq, Hkv=Hkv, D=D, S=S, prefix_len=(0, 300),
                         wid=320 + APPEND_SHAPES.index(shape))
    lens = I.prefix_lengths(w)
    cache = capacity_cache(w, lens, 40)
    print(f"[append] shape={shape} active={active} lens={lens.tolist()}", flush=True)
    new = I.attn_inputs(w, lens=lens, cache=False)
    kc, vc, ln = dev_bf16(cache["k_cache"]), dev_bf16(cache["v_cache"]), dev(lens.copy())
    act = None if active is None else dev(np.array(active, np.uint8))
    bd.kv_append(dev_bf16(new["k_blk"]), dev_bf16(new["v_blk"]), kc, vc, ln, active=act,
                 max_prefix_len=int(lens.max()))
    torch.cuda.synchronize()
    rk, rv, rl = O.kv_append(cache["k_cache"], cache["v_cache"], lens, new["k_blk"], new["v_blk"], active)
    np.testing.assert_array_equal(kc.view(torch.int16).cpu().numpy().view(np.uint16), rk)
    np.testing.assert_array_equal(vc.view(torch.int16).cpu().numpy().view(np.uint16), rv)
    np.testing.assert_array_equal(ln.cpu().numpy(), rl)


def test_kv_append_fills_the_cache_exactly():
    """The longest sequence's block lands in the last S rows of the cache (max_prefix_len + S equals
    the capacity); nothing past the cache is written (the tensors are exactly that size)."""
    w = I.small_workload("append-full", B=2, Hq=8, Hkv=2, D=128, S=16, prefix_len=(100, 300), wid=328)
    lens = I.prefix_lengths(w)
    cap = int(lens.max()) + w.S
    full = I.prefix_cache(w, lens)
    assert cap <= full["k_cache"].shape[2]
    cache = {k: np.ascontiguousarray(v[:, :, :cap]) for k, v in full.items()}   # rows past each prefix are 0
    new = I.attn_inputs(w, lens=lens, cache=False)
    kc, vc, ln = dev_bf16(cache["k_cache"]), dev_bf16(cache["v_cache"]), dev(lens.copy())
    bd.kv_append(dev_bf16(new["k_blk"]), dev_bf16(new["v_blk"]), kc, vc, ln, max_prefix_len=int(lens.max()))
    torch.cuda.synchronize()
    rk, rv, rl = O.kv_append(cache["k_cache"], cache["v_cache"], lens, new["k_blk"], new["v_blk"])
    np.testing.assert_array_equal(kc.view(torch.int16).cpu().numpy().view(np.uint16), rk)
    np.testing.assert_array_equal(vc.view(torch.int16).cpu().numpy().view(np.uint16), rv)
    np.testing.assert_array_equal(ln.cpu().numpy(), rl)


@pytest.mark.parametrize("S,Hkv", [(16, 2), (64, 4)], ids=["one-launch", "two-launches"])
def test_kv_append_skips_a_length_past_the_capacity(S, Hkv):
    """A stale host bound: sequence 0's device length leaves fewer than S free rows. Its slab and
    length stay as they were (nothing lands in sequence 1's slab), the other sequences append as
    usual. Both the one-launch and the two-launch path."""
    w = I.small_workload("append-guard", B=3, Hq=4 * Hkv, Hkv=Hkv, D=128, S=S, prefix_len=(20, 100), wid=329 + S)
    lens = I.prefix_lengths(w)
    cache = capacity_cache(w, lens, S)   # capacity: longest prefix + S
    cap = cache["k_cache"].shape[2]
    lens = lens.copy()
    lens[0] = cap - S + 1                # one row short
    new = I.attn_inputs(w, lens=lens, cache=False)
    kc, vc, ln = dev_bf16(cache["k_cache"]), dev_bf16(cache["v_cache"]), dev(lens.copy())
    bd.kv_append(dev_bf16(new["k_blk"]), dev_bf16(new["v_blk"]), kc, vc, ln, max_prefix_len=cap - S)
    torch.cuda.synchronize()
    act = np.array([0, 1, 1], np.uint8)   # what must have happened: sequence 0 skipped
    rk, rv, rl = O.kv_append(cache["k_cache"], cache["v_cache"], lens, new["k_blk"], new["v_blk"], act)
    np.testing.assert_array_equal(kc.view(torch.int16).cpu().numpy().view(np.uint16), rk)
    np.testing.assert_array_equal(vc.view(torch.int16).cpu().numpy().view(np.uint16), rv)
    np.testing.assert_array_equal(ln.cpu().numpy(), rl)


def test_commit_then_next_step_sees_the_appended_block():
    # causal pass + append of block 1, then the next block's denoise-step attention over the grown
    # cache equals the oracle's (its prefix now ends with block 1).
    w = I.small_workload("commit", B=2, Hq=32, Hkv=2, D=128, S=16, prefix_len=(70, 400), wid=330)
    lens = I.prefix_lengths(w)
    cache = capacity_cache(w, lens, 16)
    blk1 = I.attn_inputs(w, step=0, lens=lens, cache=False)
    blk2 = I.attn_inputs(w, step=1, lens=lens, cache=False)
    kc, vc, ln = dev_bf16(cache["k_cache"]), dev_bf16(cache["v_cache"]), dev(lens.copy())
    q1, k1, v1 = (dev_bf16(blk1[k]) for k in ("q", "k_blk", "v_blk"))
    o1, _ = bd.attn_step(q1, k1, v1, kc, vc, ln, causal=True, max_prefix_len=int(lens.max()))
    bd.kv_append(k1, v1, kc, vc, ln, max_prefix_len=int(lens.max()))
    q2, k2, v2 = (dev_bf16(blk2[k]) for k in ("q", "k_blk", "v_blk"))
    o2, _ = bd.attn_step(q2, k2, v2, kc, vc, ln, max_prefix_len=int(lens.max()) + 16)
    torch.cuda.synchronize()
    f = lambda a: bf16_f64(a)
    r1, _ = O.attn_step(f(blk1["q"]), f(blk1["k_blk"]), f(blk1["v_blk"]), f(cache["k_cache"]), f(cache["v_cache"]),
                        lens, causal=True)
    rk, rv, rl = O.kv_append(f(cache["k_cache"]), f(cache["v_cache"]), lens, f(blk1["k_blk"]), f(blk1["v_blk"]))
    r2, _ = O.attn_step(f(blk2["q"]), f(blk2["k_blk"]), f(blk2["v_blk"]), rk, rv, rl)
    assert_attn_close(host_f64(o1), r1, "context pass")
    assert_attn_close(host_f64(o2), r2, "next step")
    np.testing.assert_array_equal(ln.cpu().numpy(), rl)


def spec_case(B, S, V, dtype, seed, ties=False):
    rng = np.random.default_rng(seed)
    lg = rng.standard_normal((B * S, V)).astype(np.float32) * 3
    if ties:   # duplicate each row's maximum at a later index: lowest index must win
        for r in range(B * S):
            j = int(np.argmax(lg[r]))
            lg[r, min(V - 1, j + 1 + int(rng.integers(V - j - 1 if V - j - 1 > 0 else 1)))] = lg[r, j]
    if dtype == "bf16":
        bits = I.f32_to_bf16_bits(lg)
        dec = bf16_f64(bits)
    else:
        bits, dec = lg, lg.astype(np.float64)
    amax = np.array([O.vocab_reduce(dec[r])[1] for r in range(B * S)], dtype=np.int32)
    first = rng.integers(0, V, B).astype(np.int32)
    # drafts: AR's own choices up to a random first mismatch per sequence (every k in 0..S)
    draft = np.zeros(B * S, dtype=np.int32)
    for b in range(B):
        k = int(rng.integers(0, S + 1)) if b >= 2 else (S if b == 0 else 0)
        for i in range(S):
            ar = first[b] if i == 0 else amax[b * S + i - 1]
            draft[b * S + i] = ar if i < k else (ar + 1 + int(rng.integers(V - 1))) % V if i == k else int(rng.integers(V))
    return bits, dec, amax, first, draft


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", [(6, 16, 4096), (3, 64, 1000), (4, 1, 131072)])
def test_spec_verify_matches_oracle(dtype, shape):
    B, S, V = shape
    bits, dec, amax, first, draft = spec_case(B, S, V, dtype, seed=B * 1000 + S + V, ties=True)
    lg = dev_bf16(bits) if dtype == "bf16" else dev(bits)
    r = bd.spec_verify(lg, dev(draft), dev(first), S)
    torch.cuda.synchronize()
    ref = O.spec_accept(draft, first, amax, S)
    np.testing.assert_array_equal(r["n_commit"].cpu().numpy(), ref["n_commit"])
    np.testing.assert_array_equal(r["tokens"].cpu().numpy(), ref["tokens"])
    np.testing.assert_array_equal(r["next_choice"].cpu().numpy(), ref["next_choice"])
    assert (r["n_commit"].cpu().numpy() >= 1).all()


def test_spec_verify_full_vocab_padded_rows():
    # row stride > vocab (padded rows): only the first V logits of a row count
    B, S, V, stride = 4, 16, 131000, 131072
    bits, dec, amax, first, draft = spec_case(B, S, V, "bf16", seed=7)
    padded = np.zeros((B * S, stride), dtype=np.uint16)
    padded[:, :V] = bits
    padded[:, V:] = I.f32_to_bf16_bits(np.full((B * S, stride - V), 100.0, np.float32))   # would win if read
    r = bd.spec_verify(dev_bf16(padded), dev(draft), dev(first), S, vocab=V)
    torch.cuda.synchronize()
    ref = O.spec_accept(draft, first, amax, S)
    np.testing.assert_array_equal(r["tokens"].cpu().numpy(), ref["tokens"])
    np.testing.assert_array_equal(r["n_commit"].cpu().numpy(), ref["n_commit"])
