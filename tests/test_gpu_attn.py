"""GPU parity of bd_attn_step against the float64 oracle (through the C ABI).

Small shapes (whole tensors compared) span several key tiles, several splits, ragged tails,
padded row tiles, S = 1 (AR decode), L = 0 and head_dim 64/128. The official workloads run at
full size in the launch configuration the benchmark uses, every output element compared with the
oracle, plus properties that hold at any size (determinism, the cache is never written, inactive
sequences untouched, canaries around the output intact)."""
import numpy as np
import pytest
import torch

import block_diffusion_lm_amd as bd
from block_diffusion_lm_amd import inputs as I
from oracle import bd_oracle as O
from tests.gpu_util import (LSE_ATOL, assert_attn_close, bf16_f64, dev, dev_bf16, guarded, guards_intact, host_f64,
                             oracle_attn_all)

pytestmark = pytest.mark.gpu


def run_gpu(inp, **kw):
    t = {k: dev_bf16(inp[k]) for k in ("q", "k_blk", "v_blk", "k_cache", "v_cache")}
    t["prefix_len"] = dev(inp["prefix_len"])
    out, lse = bd.attn_step(t["q"], t["k_blk"], t["v_blk"], t["k_cache"], t["v_cache"], t["prefix_len"], **kw)
    torch.cuda.synchronize()
    return host_f64(out), lse.cpu().numpy().astype(np.float64), t


def oracle_full(inp, active=None):
    f = {k: bf16_f64(inp[k]) for k in ("q", "k_blk", "v_blk", "k_cache", "v_cache")}
    return O.attn_step(f["q"], f["k_blk"], f["v_blk"], f["k_cache"], f["v_cache"], inp["prefix_len"], active=active)


SMALL = [
    # name, B, Hq, Hkv, D, S, prefix_len
    ("tiny-like", 1, 8, 2, 64, 16, 256),
    ("ragged-d128", 3, 32, 2, 128, 16, (1, 700)),
    ("no-prefix", 2, 8, 2, 64, 16, 0),
    ("ar-decode-S1", 2, 32, 8, 128, 1, (60, 300)),
    ("S32-two-row-tiles", 1, 32, 2, 128, 32, 333),
    ("padded-rows", 2, 6, 3, 64, 5, (0, 129)),
    ("S64-g4", 1, 16, 4, 128, 64, 190),
    ("mha-D64", 2, 4, 4, 64, 16, 77),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
@pytest.mark.parametrize("num_splits", [0, 1, 2, 7])
def test_small_shapes_match_oracle(case, num_splits):
    name, B, Hq, Hkv, D, S, L = case
    w = I.small_workload(name, B=B, Hq=Hq, Hkv=Hkv, D=D, S=S, prefix_len=L, wid=200 + SMALL.index(case))
    inp = I.attn_inputs(w)
    print(f"[attn] {name} splits={num_splits} lens={inp['prefix_len'].tolist()}", flush=True)
    got, lse, _ = run_gpu(inp, num_splits=num_splits)
    ref, ref_lse = oracle_full(inp)
    assert_attn_close(got, ref, name)
    np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=LSE_ATOL)


def test_tiny_workload_and_planted_large_scores():
    w = I.WORKLOADS["tiny"]
    inp = I.attn_inputs(w)
    got, lse, _ = run_gpu(inp)
    ref, ref_lse = oracle_full(inp)
    assert_attn_close(got, ref, "tiny")
    np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=LSE_ATOL)
    # planted large scores: one prefix key per KV head aligned with every query -> O ~ its V row (O(1))
    inp2 = {k: v.copy() for k, v in inp.items()}
    qf = bf16_f64(inp2["q"])
    kc = bf16_f64(inp2["k_cache"])
    kc[:, :, 17, :] = 0.0
    kc[:, :, 17, 0] = 8.0
    qf[..., 0] = 16.0
    inp2["q"] = I.f32_to_bf16_bits(qf.astype(np.float32))
    inp2["k_cache"] = I.f32_to_bf16_bits(kc.astype(np.float32))
    got2, _, _ = run_gpu(inp2)
    ref2, _ = oracle_full(inp2)
    assert np.abs(ref2).max() > 0.5
    assert_attn_close(got2, ref2, "planted")


def test_block_permutation_on_gpu():
    w = I.small_workload("perm", B=2, Hq=32, Hkv=2, D=128, S=16, prefix_len=(100, 500), wid=230)
    inp = I.attn_inputs(w)
    perm = np.random.default_rng(0).permutation(16)
    inp2 = dict(inp)
    for k in ("q", "k_blk", "v_blk"):
        inp2[k] = np.ascontiguousarray(inp[k][:, perm])
    a, _, _ = run_gpu(inp)
    b, _, _ = run_gpu(inp2)
    np.testing.assert_allclose(b, a[:, perm], atol=4e-3)


def test_determinism_and_cache_untouched():
    w = I.small_workload("det", B=2, Hq=32, Hkv=2, D=128, S=16, prefix_len=(3000, 5000), wid=231)
    inp = I.attn_inputs(w)
    t = {k: dev_bf16(inp[k]) for k in ("q", "k_blk", "v_blk", "k_cache", "v_cache")}
    t["prefix_len"] = dev(inp["prefix_len"])
    before = {k: v.clone() for k, v in t.items()}
    o1, l1 = bd.attn_step(t["q"], t["k_blk"], t["v_blk"], t["k_cache"], t["v_cache"], t["prefix_len"])
    o2, l2 = bd.attn_step(t["q"], t["k_blk"], t["v_blk"], t["k_cache"], t["v_cache"], t["prefix_len"])
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
    for k in t:
        assert torch.equal(t[k].view(torch.uint8) if t[k].dtype != torch.int32 else t[k],
                           before[k].view(torch.uint8) if before[k].dtype != torch.int32 else before[k]), k


def test_inactive_sequences_and_canaries():
    w = I.small_workload("act", B=3, Hq=8, Hkv=2, D=64, S=16, prefix_len=(10, 900), wid=232)
    inp = I.attn_inputs(w)
    t = {k: dev_bf16(inp[k]) for k in ("q", "k_blk", "v_blk", "k_cache", "v_cache")}
    t["prefix_len"] = dev(inp["prefix_len"])
    active = torch.tensor([1, 0, 1], dtype=torch.uint8, device="cuda")
    for splits in (0, 3):
        big, out, g = guarded(tuple(inp["q"].shape), torch.bfloat16)
        lbig, lse, lg = guarded((3, 8, 16), torch.float32)
        b0, l0 = big.clone(), lbig.clone()
        bd.attn_step(t["q"], t["k_blk"], t["v_blk"], t["k_cache"], t["v_cache"], t["prefix_len"], active=active,
                     out=out, lse=lse, num_splits=splits)
        torch.cuda.synchronize()
        assert guards_intact(big, g, out.numel(), b0) and guards_intact(lbig, lg, lse.numel(), l0)
        assert torch.equal(out[1].view(torch.int16), b0[g:g + out.numel()].view(out.shape)[1].view(torch.int16))
        ref, _ = oracle_full(inp, active=[1, 0, 1])
        got = host_f64(out[[0, 2]])
        assert_attn_close(got, ref[[0, 2]], "active")


@pytest.mark.parametrize("name", ["decode", "batched16", "batched32", "long", "stress_a", "stress_b"])
def test_official_workloads_full_size(name):
    """Every element of out and lse at full size, in the launch configuration the benchmark uses,
    against the oracle computed row by row (one (sequence, KV head) slab at a time)."""
    w = I.WORKLOADS[name]
    print(f"[attn] full-size {name}", flush=True)
    inp = I.attn_inputs(w)
    got, lse, t = run_gpu(inp)
    ref, ref_lse = oracle_attn_all(inp)
    assert_attn_close(got, ref, name)
    np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=LSE_ATOL)
    # the cache was not written
    assert torch.equal(t["k_cache"].view(torch.int16).cpu(), torch.from_numpy(inp["k_cache"].view(np.int16)))
    assert torch.equal(t["v_cache"].view(torch.int16).cpu(), torch.from_numpy(inp["v_cache"].view(np.int16)))


EDGE = [
    # name, Hq, Hkv, D, S, lengths (tile edges: 64-key tiles, chunks of whole tiles)
    ("edges-8w-d128", 32, 2, 128, 16, (64, 127, 128, 129, 0, 191)),
    ("edges-4w-d64", 8, 2, 64, 16, (64, 65, 256, 63, 1, 320)),
    ("edges-8w-S64", 16, 4, 128, 64, (0, 64, 100, 192)),
]


@pytest.mark.parametrize("case", EDGE, ids=[c[0] for c in EDGE])
@pytest.mark.parametrize("num_splits", [0, 1, 2, 5])
@pytest.mark.parametrize("causal", [False, True])
def test_tile_edge_lengths(case, num_splits, causal):
    """Prefix lengths on and next to tile edges, so that chunks hold zero, one or several tiles
    wholly inside the prefix before the ones holding its end or the block's keys."""
    name, Hq, Hkv, D, S, lens = case
    lens = np.asarray(lens, np.int32)
    w = I.small_workload(name, B=len(lens), Hq=Hq, Hkv=Hkv, D=D, S=S, prefix_len=int(lens.max()),
                         wid=260 + EDGE.index(case))
    inp = I.attn_inputs(w, lens=lens)
    print(f"[attn] {name} splits={num_splits} causal={causal} lens={lens.tolist()}", flush=True)
    got, lse, _ = run_gpu(inp, num_splits=num_splits, causal=causal)
    f = {k: bf16_f64(inp[k]) for k in ("q", "k_blk", "v_blk", "k_cache", "v_cache")}
    ref, ref_lse = O.attn_step(f["q"], f["k_blk"], f["v_blk"], f["k_cache"], f["v_cache"], inp["prefix_len"],
                               causal=causal)
    assert_attn_close(got, ref, name)
    np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=LSE_ATOL)


WIDE_EDGE_LENS = [(4096, 4097), (4031, 4161), (4095, 4160), (4159, 4033), (4032, 4096)]


@pytest.mark.parametrize("lens", WIDE_EDGE_LENS, ids=[f"L{a}-{b}" for a, b in WIDE_EDGE_LENS])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("num_splits", [0, 1, 3])
@pytest.mark.parametrize("causal", [False, True])
def test_tile_edges_of_the_long_prefix_kernel(lens, D, num_splits, causal):
    """Tile-edge prefix lengths (a multiple of 64 keys and +-1 around it) in shapes that plan the
    long-prefix kernel -- one 256-row work-group per (sequence, KV head, chunk), the launch the
    long, batched and stress workloads use -- asserted through the plan query so a planner change
    cannot silently move these cases to another kernel. Both modes, both head dims, forced splits."""
    lens = np.asarray(lens, np.int32)
    w = I.small_workload(f"wide-edge-{D}", B=2, Hq=128, Hkv=8, D=D, S=16, prefix_len=int(lens.max()),
                         wid=330 + D // 64)
    desc = bd.attn_desc(w.B, w.Hq, w.Hkv, w.D, w.S, int(lens.max()), int(lens.max()), num_splits=num_splits,
                        causal=causal)
    plan = bd.attn_plan(desc)
    assert plan["waves"] * plan["rows_per_wave"] == 256 and plan["row_tiles"] == 1, plan
    inp = I.attn_inputs(w, lens=lens)
    print(f"[attn] wide-edge D={D} splits={num_splits} causal={causal} lens={lens.tolist()} plan={plan}", flush=True)
    got, lse, _ = run_gpu(inp, num_splits=num_splits, causal=causal)
    ref, ref_lse = oracle_attn_all(inp, causal=causal)
    assert_attn_close(got, ref, f"wide-edge-{D}")
    np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=LSE_ATOL)


RAGGED = [
    # name, Hq, Hkv, D, lengths: one long sequence among very short ones (the plan sizes chunks
    # from the actual lengths: the long one takes most of the slots), empty prefixes, tile edges
    ("ragged-wave-plan", 8, 2, 128, (32768, 1, 0, 5, 4097, 64, 63, 20000, 2)),
    ("ragged-d64", 16, 4, 64, (0, 0, 9000, 0, 1, 129)),
]


@pytest.mark.parametrize("case", RAGGED, ids=[c[0] for c in RAGGED])
@pytest.mark.parametrize("num_splits", [0, 3, 7])
@pytest.mark.parametrize("causal", [False, True])
def test_length_balanced_plan(case, num_splits, causal):
    """Split launches plan their chunks from the actual prefix lengths on the device: every row of
    a very ragged batch against the oracle (forced and automatic split counts, both modes)."""
    name, Hq, Hkv, D, lens = case
    lens = np.asarray(lens, np.int32)
    w = I.small_workload(name, B=len(lens), Hq=Hq, Hkv=Hkv, D=D, S=16, prefix_len=int(lens.max()),
                         wid=370 + RAGGED.index(case))
    plan = bd.attn_plan(bd.attn_desc(w.B, Hq, Hkv, D, 16, int(lens.max()), int(lens.max()), num_splits=num_splits,
                                     causal=causal))
    assert plan["num_splits"] > 1, plan
    inp = I.attn_inputs(w, lens=lens)
    print(f"[attn] {name} splits={num_splits} causal={causal} plan={plan}", flush=True)
    got, lse, _ = run_gpu(inp, num_splits=num_splits, causal=causal)
    ref, ref_lse = oracle_attn_all(inp, causal=causal)
    assert_attn_close(got, ref, name)
    np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=LSE_ATOL)


@pytest.mark.parametrize("B", [64, 65, 1024], ids=["wave-plan-edge-64", "group-plan-65", "group-plan-limit-1024"])
def test_balanced_plan_at_its_batch_edges(B):
    """The batch sizes where the device plan changes hands: 64 sequences (the last per-wave plan),
    65 (the first per-work-group one) and 1024 (the largest balanced batch), ragged lengths and a
    scattered active mask, every active row against the oracle."""
    rng = np.random.default_rng(390 + B)
    lens = rng.integers(0, 400, size=B).astype(np.int32)
    w = I.small_workload(f"edge-{B}", B=B, Hq=4, Hkv=1, D=64, S=4, prefix_len=400, wid=391 + B)
    inp = I.attn_inputs(w, lens=lens)
    act = (rng.random(B) < 0.6).astype(np.uint8)
    act[-1] = 1
    plan = bd.attn_plan(bd.attn_desc(B, 4, 1, 64, 4, 400, 400, num_splits=3))
    assert plan["num_splits"] > 1, plan
    t = {k: dev_bf16(inp[k]) for k in ("q", "k_blk", "v_blk", "k_cache", "v_cache")}
    print(f"[attn] balanced-plan edge B={B} active={int(act.sum())} plan={plan}", flush=True)
    out, _ = bd.attn_step(t["q"], t["k_blk"], t["v_blk"], t["k_cache"], t["v_cache"], dev(inp["prefix_len"]),
                          active=dev(act), num_splits=3, max_prefix_len=400)
    torch.cuda.synchronize()
    ref, _ = oracle_attn_all(inp, active=act)
    assert_attn_close(host_f64(out[torch.from_numpy(act == 1).cuda()]), ref[act == 1], f"edge-{B}")


@pytest.mark.parametrize("B,num_splits", [(5, 2), (5, 4), (80, 2), (80, 3), (5, 1), (80, 1), (1100, 2)],
                         ids=["wave-plan-2", "wave-plan-4", "group-plan-2", "group-plan-3", "one-chunk-5",
                              "one-chunk-80", "uniform-plan-1100"])
def test_lengths_above_the_host_bound(B, num_splits):
    """prefix_len above the descriptor's max_prefix_len (but within the cache): the device plan (per
    wave up to 64 sequences, per work-group up to 1024), the uniform plan beyond (its last chunk runs
    to the sequence's end) and the one-chunk plan still take every key of every sequence, so the
    output matches the oracle over the true lengths."""
    rng = np.random.default_rng(380 + B + num_splits)
    lens = rng.integers(0, 1500, size=B).astype(np.int32)
    lens[0] = 1500
    w = I.small_workload(f"over-bound-{B}", B=B, Hq=8, Hkv=2, D=64, S=16, prefix_len=2048, wid=381 + B)
    inp = I.attn_inputs(w, lens=lens)
    bound = 100   # the host's (stale) bound: far below the true lengths
    plan = bd.attn_plan(bd.attn_desc(B, 8, 2, 64, 16, 2048, bound, num_splits=num_splits))
    assert (plan["num_splits"] > 1) == (num_splits > 1), plan
    print(f"[attn] over-bound B={B} splits={num_splits} plan={plan}", flush=True)
    got, lse, _ = run_gpu(inp, num_splits=num_splits, max_prefix_len=bound)
    ref, ref_lse = oracle_attn_all(inp)
    assert_attn_close(got, ref, f"over-bound-{B}")
    np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=LSE_ATOL)


MANY = [
    # name, Hq, Hkv, D, num_splits, waves: 512 sequences; 64 and 128 rows per KV head plan the
    # four-wave kernel (with 64 rows half its waves hold no rows), 256 rows the eight-wave one;
    # forced splits run the merge and the device re-plan over the active sequences
    ("many-4w-64rows", 8, 2, 64, 0, 4),
    ("many-4w", 16, 2, 64, 2, 4),
    ("many-8w", 32, 2, 128, 0, 8),
    ("many-8w-split3", 32, 2, 128, 3, 8),
]


@pytest.mark.parametrize("case", MANY, ids=[c[0] for c in MANY])
def test_many_sequences_with_a_ragged_active_mask(case):
    """512 sequences, a seeded ragged active mask (first inactive, last active): the split
    work-groups find their sequence through the length-balanced plan over the active sequences
    (derived per work-group), the merge its partial rows through the plan's stored prefix sums.
    Active rows match the oracle; inactive rows keep the canary fill."""
    name, Hq, Hkv, D, num_splits, waves = case
    B = 512
    w = I.small_workload(name, B=B, Hq=Hq, Hkv=Hkv, D=D, S=16, prefix_len=(60, 700), wid=340 + MANY.index(case))
    inp = I.attn_inputs(w)
    act = (np.random.default_rng(341).random(B) < 0.45).astype(np.uint8)
    act[0], act[-1] = 0, 1
    plan = bd.attn_plan(bd.attn_desc(B, Hq, Hkv, D, 16, inp["k_cache"].shape[2], int(inp["prefix_len"].max()),
                                     num_splits=num_splits))
    assert plan["waves"] == waves, plan
    print(f"[attn] {name} active={int(act.sum())} plan={plan}", flush=True)
    t = {k: dev_bf16(inp[k]) for k in ("q", "k_blk", "v_blk", "k_cache", "v_cache")}
    big, out, gd = guarded(tuple(inp["q"].shape), torch.bfloat16)
    b0 = big.clone()
    bd.attn_step(t["q"], t["k_blk"], t["v_blk"], t["k_cache"], t["v_cache"], dev(inp["prefix_len"]), active=dev(act),
                 out=out, want_lse=False, num_splits=num_splits, max_prefix_len=int(inp["prefix_len"].max()))
    torch.cuda.synchronize()
    assert guards_intact(big, gd, out.numel(), b0)
    keep = b0[gd:gd + out.numel()].view(out.shape)
    ina = torch.from_numpy(act == 0).cuda()
    assert torch.equal(out[ina].view(torch.int16), keep[ina].view(torch.int16))
    got = host_f64(out[torch.from_numpy(act == 1).cuda()])
    ref, _ = oracle_attn_all(inp, active=act)
    assert_attn_close(got, ref[act == 1], name)


@pytest.mark.parametrize("Hq,waves", [(4, 4), (16, 8)], ids=["4w-64rows", "8w-256rows"])
def test_uniform_plan_beyond_the_balanced_batch(Hq, waves):
    """1100 sequences, above the largest balanced batch (1024), keep the uniform plan: under a
    scattered active mask every split work-group finds its sequence, and the merge the partial rows
    of its own, by counting the active flags in passes of one work-group's width (three passes of
    512 flags, five of 256); active rows match the oracle, inactive rows keep the canary fill."""
    B = 1100
    rng = np.random.default_rng(395 + Hq)
    lens = rng.integers(0, 400, size=B).astype(np.int32)
    w = I.small_workload(f"uniform-{Hq}", B=B, Hq=Hq, Hkv=1, D=64, S=16, prefix_len=400, wid=396 + Hq)
    inp = I.attn_inputs(w, lens=lens)
    act = (rng.random(B) < 0.5).astype(np.uint8)
    act[0], act[-1] = 0, 1
    act[512:530] = 1   # a run of active flags across the first pass boundary of the wide kernel
    plan = bd.attn_plan(bd.attn_desc(B, Hq, 1, 64, 16, 400, 400, num_splits=3))
    assert plan["num_splits"] == 3 and plan["waves"] == waves, plan
    print(f"[attn] uniform plan B={B} Hq={Hq} active={int(act.sum())} plan={plan}", flush=True)
    t = {k: dev_bf16(inp[k]) for k in ("q", "k_blk", "v_blk", "k_cache", "v_cache")}
    big, out, gd = guarded(tuple(inp["q"].shape), torch.bfloat16)
    b0 = big.clone()
    bd.attn_step(t["q"], t["k_blk"], t["v_blk"], t["k_cache"], t["v_cache"], dev(inp["prefix_len"]), active=dev(act),
                 out=out, want_lse=False, num_splits=3, max_prefix_len=400)
    torch.cuda.synchronize()
    assert guards_intact(big, gd, out.numel(), b0)
    keep = b0[gd:gd + out.numel()].view(out.shape)
    ina = torch.from_numpy(act == 0).cuda()
    assert torch.equal(out[ina].view(torch.int16), keep[ina].view(torch.int16))
    ref, _ = oracle_attn_all(inp, active=act)
    assert_attn_close(host_f64(out[torch.from_numpy(act == 1).cuda()]), ref[act == 1], f"uniform-{Hq}")


@pytest.mark.parametrize("num_splits", [0, 1, 3])
def test_largest_query_group(num_splits):
    """The largest row count per KV head the descriptor allows in one group: S = 64 block positions
    times 64 query heads on one KV head (4096 rows, many row tiles)."""
    w = I.small_workload("rows4096", B=1, Hq=64, Hkv=1, D=128, S=64, prefix_len=900, wid=289)
    inp = I.attn_inputs(w)
    print(f"[attn] rows4096 splits={num_splits}", flush=True)
    got, lse, _ = run_gpu(inp, num_splits=num_splits)
    ref, ref_lse = oracle_full(inp)
    assert_attn_close(got, ref, "rows4096")
    np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=LSE_ATOL)


RISE = ["ramp", "jumps", "wide"]
RISE_SHAPES = [
    # name, B, Hq, Hkv, D, S, prefix_len: the first plans eight-wave workgroups (the full-tile loop of
    # the long-prefix kernel), the second four-wave ones with head_dim 64 (the same loop)
    ("8w-d128", 2, 128, 8, 128, 16, (4000, 4200)),
    ("4w-d64", 2, 32, 2, 64, 16, (1100, 1300)),
]


@pytest.mark.parametrize("shape", RISE_SHAPES, ids=[s[0] for s in RISE_SHAPES])
@pytest.mark.parametrize("pattern", RISE)
@pytest.mark.parametrize("num_splits", [0, 1, 3])
def test_running_max_rises_inside_the_prefix(shape, pattern, num_splits):
    """Scores that keep rising across the cached prefix, so that blocks of wholly cached keys raise
    the running max again and again: a ramp (every 32-key block ~4 log2 units above the one before,
    so its P sum per lane passes 256, mostly with no key above the max by 8), single keys at ~12,
    ~98 and ~255 log2 units (the last ~157 above the max: its P overflows float32 until the max is
    raised), and a wide case where half of a block's keys sit ~5 units above the max (figures for
    head_dim 128; 1.4 times as many units at 64)."""
    sname, B, Hq, Hkv, D, S, L = shape
    w = I.small_workload(f"rise-{pattern}-{sname}", B=B, Hq=Hq, Hkv=Hkv, D=D, S=S, prefix_len=L,
                         wid=290 + 3 * RISE_SHAPES.index(shape) + RISE.index(pattern))
    inp = I.attn_inputs(w)
    q = bf16_f64(inp["q"])
    kc = bf16_f64(inp["k_cache"])
    q[..., 0] = 8.0
    nk = kc.shape[2]
    blk = np.arange(nk) // 32
    if pattern == "ramp":
        kc[:, :, :, 0] = 4.0 * blk                            # +32 raw = +4.08 log2 units a block
    elif pattern == "jumps":
        kc[:, :, :, 0] = 0.0
        for b0, v in ((5, 12.0), (14, 96.0), (26, 250.0)):   # ~12, ~98 and ~255 log2 units
            kc[:, :, 32 * b0 + 7, 0] = v
    else:
        kc[:, :, :, 0] = 0.0
        kc[:, :, 32 * 9:32 * 9 + 32:2, 0] = 5.0             # 16 keys of one block at ~+5 units
    inp["q"] = I.f32_to_bf16_bits(q.astype(np.float32))
    inp["k_cache"] = I.f32_to_bf16_bits(kc.astype(np.float32))
    print(f"[attn] rise-{pattern}-{sname} splits={num_splits} lens={inp['prefix_len'].tolist()}", flush=True)
    got, lse, _ = run_gpu(inp, num_splits=num_splits)
    ref, ref_lse = oracle_full(inp)
    assert np.isfinite(got).all()
    assert_attn_close(got, ref, f"rise-{pattern}-{sname}")
    np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=LSE_ATOL * max(1.0, np.abs(ref_lse).max() / 64))


def _random_cases(n=40, seed=2026):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        D = int(rng.choice([64, 128]))
        Hkv = int(rng.choice([1, 2, 4, 8]))
        g = int(rng.choice([1, 2, 4, 8, 16]))
        S = int(rng.choice([1, 2, 5, 16, 32, 64]))
        B = int(rng.integers(1, 5))
        lmax = int(rng.choice([0, 63, 64, 200, 777, 2100]))
        lens = rng.integers(0, lmax + 1, size=B).astype(np.int32)
        splits = int(rng.choice([0, 0, 1, 3, 9]))
        causal = bool(rng.integers(0, 2))
        cases.append((f"r{i}-B{B}-g{g}x{Hkv}-D{D}-S{S}-L{lmax}-s{splits}-{'c' if causal else 'b'}",
                      B, g * Hkv, Hkv, D, S, lens, splits, causal))
    return cases


RANDOM = _random_cases()


@pytest.mark.parametrize("case", RANDOM, ids=[c[0] for c in RANDOM])
def test_random_shapes_match_oracle(case):
    """A seeded sweep over head dims, GQA groups, block lengths, ragged prefix lengths (on and off
    tile edges, zero included), forced split counts and both attention modes."""
    name, B, Hq, Hkv, D, S, lens, splits, causal = case
    w = I.small_workload(name, B=B, Hq=Hq, Hkv=Hkv, D=D, S=S, prefix_len=max(int(lens.max()), 1),
                         wid=400 + RANDOM.index(case))
    inp = I.attn_inputs(w, lens=lens)
    print(f"[attn] {name} lens={lens.tolist()}", flush=True)
    got, lse, _ = run_gpu(inp, num_splits=splits, causal=causal)
    f = {k: bf16_f64(inp[k]) for k in ("q", "k_blk", "v_blk", "k_cache", "v_cache")}
    ref, ref_lse = O.attn_step(f["q"], f["k_blk"], f["v_blk"], f["k_cache"], f["v_cache"], inp["prefix_len"],
                               causal=causal)
    assert_attn_close(got, ref, name)
    np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=LSE_ATOL)
