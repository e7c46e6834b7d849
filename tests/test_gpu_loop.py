"""GPU parity of bd_denoise_block (the T-step loop) against the oracle's loop.

The hooks hand the library seeded per-step q / k_blk / v_blk and logits (the logits do not
depend on the attention output: no LM head is in scope), and snapshot every step's attention
output so each step can be checked. Masks, tokens, steps used and per-step commit counts are
bit-exact; the attention of every executed step matches within the bf16 tolerance."""
import numpy as np
import pytest
import torch

import block_diffusion_lm_amd as bd
from block_diffusion_lm_amd import inputs as I
from oracle import bd_oracle as O
from tests.gpu_util import assert_attn_close, bf16_f64, dev, dev_bf16, host_f64, oracle_attn_all

pytestmark = pytest.mark.gpu


def run_loop(w, t0=0, mask0=None, tokens0=None, T=None, full_oracle=True, trace=None):
    T = w.T if T is None else T
    lens = I.prefix_lengths(w)
    cache = I.prefix_cache(w, lens)
    steps = {t: I.attn_inputs(w, step=t, lens=lens, cache=False) for t in range(T)}
    logits = {t: I.logits(w, step=t) for t in range(T)}
    mask0 = I.initial_mask(w) if mask0 is None else mask0
    tokens0 = np.full(w.B * w.S, -1, np.int32) if tokens0 is None else tokens0
    dsteps = {t: tuple(dev_bf16(steps[t][k]) for k in ("q", "k_blk", "v_blk")) for t in range(T)}
    is_bf16 = w.logits_dtype == "bf16"
    dlogits = {t: (dev_bf16(logits[t]) if is_bf16 else dev(logits[t])) for t in range(T)}
    snaps = {}

    def get_qkv(step, mask, tokens):
        return dsteps[step]

    def get_logits(step, out):
        snaps[step] = out.clone()
        return dlogits[step]

    kc, vc = dev_bf16(cache["k_cache"]), dev_bf16(cache["v_cache"])
    m_d, t_d = dev(mask0.copy()), dev(tokens0.copy())
    if trace is not None:
        trace.__enter__()
    try:
        res = bd.denoise_block(get_qkv, get_logits, kc, vc, dev(lens), m_d, t_d, T, w.Hq, w.gamma, w.S, w.V,
                               logits_bf16=is_bf16, t0=t0, min_commit=bool(w.min_commit))
        torch.cuda.synchronize()
    finally:
        if trace is not None:
            trace.__exit__(None, None, None)

    f_cache = {k: bf16_f64(v) for k, v in cache.items()}

    def step_inputs(t):
        d = {k: bf16_f64(steps[t][k]) for k in ("q", "k_blk", "v_blk")} if full_oracle else \
            {k: np.zeros(1) for k in ("q", "k_blk", "v_blk")}
        d["logits"] = logits[t]
        return d

    if full_oracle:
        ref = O.denoise_block(T, t0, w.B, w.S, mask0, tokens0, step_inputs, f_cache["k_cache"], f_cache["v_cache"],
                              lens, w.gamma, bool(w.min_commit), True,
                              logits_decode=O.bf16_to_f64 if is_bf16 else None)
    else:
        # control flow only (the logits do not depend on the attention); every row of every
        # executed step's attention is checked below, one (sequence, KV head) slab at a time
        mask, tokens = mask0.copy(), tokens0.copy()
        ref = {"steps_used": np.zeros(w.B, np.int32), "commits": np.zeros((T, w.B), np.int32), "active": {},
               "masks": {}}
        for t in range(t0, T):
            act = mask.reshape(w.B, w.S).any(axis=1)
            if not act.any():
                break
            ref["active"][t] = act
            ref["masks"][t] = mask.copy()
            r = O.confidence_unmask(logits[t], mask, tokens, w.S, w.gamma, bool(w.min_commit), t == T - 1,
                                    decode=O.bf16_to_f64 if is_bf16 else None)
            assert not O.near_ties(r["conf"], mask, w.S, w.gamma, bool(w.min_commit), t == T - 1)
            mask, tokens = r["mask"], r["tokens"]
            ref["commits"][t] = r["n_commit"]
            ref["steps_used"][act] = t + 1
        ref["mask"], ref["tokens"] = mask, tokens

    np.testing.assert_array_equal(m_d.cpu().numpy(), ref["mask"])
    np.testing.assert_array_equal(t_d.cpu().numpy(), ref["tokens"])
    np.testing.assert_array_equal(res["steps_used"].cpu().numpy(), ref["steps_used"])
    np.testing.assert_array_equal(res["commits_per_step"].cpu().numpy()[t0:], ref["commits"][t0:])
    executed = sorted(ref["active"])
    for t in executed:
        act = ref["active"][t]
        got = host_f64(snaps[t])
        if full_oracle:
            assert_attn_close(got[act], ref["outs"][t][act], f"step {t}")
        else:
            step_inp = dict(steps[t], k_cache=cache["k_cache"], v_cache=cache["v_cache"], prefix_len=lens)
            ref_o, _ = oracle_attn_all(step_inp, active=act)
            assert_attn_close(got[act], ref_o[act], f"step {t}")
    return res, ref


def test_small_loop_matches_oracle():
    w = I.small_workload("loop", B=3, Hq=8, Hkv=2, D=64, S=16, prefix_len=(50, 400), V=3000, logits_dtype="bf16",
                         sigma=3.0, gamma=0.9, mask_rule="frac", peaks=True, T=6, wid=250)
    run_loop(w)


@pytest.mark.parametrize("B,S", [(4, 16), (2, 32), (1, 64), (5, 8), (6, 16), (3, 32)],
                         ids=["4x16", "2x32", "1x64", "five-seqs-40-rows", "96-rows", "3x32-rows"])
def test_loop_over_block_shapes(B, S):
    """Loops over block lengths 8 to 64 and one to six sequences (masked rows found by a ballot up
    to 64 rows, by the work-group scan above) match the oracle's loop bit for bit, through steps
    where some or all sequences have finished: every step runs one reduction and one commit
    launch, the commit of an empty step included (n_commit = 0, nothing left active)."""
    w = I.small_workload(f"shape{B}x{S}", B=B, Hq=8, Hkv=2, D=64, S=S, prefix_len=(40, 300), V=2504,
                         logits_dtype="bf16", sigma=3.0, gamma=0.9, mask_rule="frac", peaks=True, T=9, wid=260 + B * S)
    tr = bd.Trace(capacity=256)
    try:
        res, ref = run_loop(w, trace=tr)
        names = [n for n, _ in tr.records()]
    finally:
        tr.close()
    assert names.count("vocab_reduce") == w.T and names.count("commit") == w.T
    assert ref["steps_used"].max() < w.T, ref["steps_used"]


def test_loop_resume_from_t0():
    w = I.small_workload("loop2", B=2, Hq=32, Hkv=2, D=128, S=16, prefix_len=(200, 900), V=2000, logits_dtype="f32",
                         sigma=2.0, gamma=0.5, mask_rule="all", peaks=True, T=5, wid=251)
    mask = I.initial_mask(w)
    mask[:5] = 0
    run_loop(w, t0=2, mask0=mask, tokens0=np.arange(w.B * w.S, dtype=np.int32))


def test_long_workload_full_loop():
    w = I.WORKLOADS["long"]
    res, ref = run_loop(w, full_oracle=False)
    assert ref["steps_used"].max() >= 2      # the loop runs several steps before every position commits


def test_native_step_table_matches_python_hooks():
    w = I.small_workload("loop3", B=2, Hq=32, Hkv=2, D=128, S=16, prefix_len=(300, 1200), V=2048, logits_dtype="bf16",
                         sigma=3.0, gamma=0.9, mask_rule="all", peaks=True, T=4, wid=252)
    lens = I.prefix_lengths(w)
    cache = I.prefix_cache(w, lens)
    steps = [I.attn_inputs(w, step=t, lens=lens, cache=False) for t in range(w.T)]
    qkv = [tuple(dev_bf16(steps[t][k]) for k in ("q", "k_blk", "v_blk")) for t in range(w.T)]
    lg = [dev_bf16(I.logits(w, step=t)) for t in range(w.T)]
    kc, vc, ln = dev_bf16(cache["k_cache"]), dev_bf16(cache["v_cache"]), dev(lens)
    results = []
    for mode in ("python", "table"):
        m_d, t_d = dev(I.initial_mask(w)), dev(np.zeros(w.B * w.S, np.int32))
        kw = {"step_table": ([x[0] for x in qkv], [x[1] for x in qkv], [x[2] for x in qkv], lg)} if mode == "table" else {}
        res = bd.denoise_block((lambda t, m, tk: qkv[t]) if mode == "python" else None,
                               (lambda t, o: lg[t]) if mode == "python" else None,
                               kc, vc, ln, m_d, t_d, w.T, w.Hq, w.gamma, w.S, w.V, **kw)
        torch.cuda.synchronize()
        results.append((m_d.cpu(), t_d.cpu(), res["steps_used"].cpu(), res["commits_per_step"].cpu(),
                        res["out"].view(torch.int16).cpu()))
    for a, b in zip(*results):
        assert torch.equal(a, b)


def test_denoise_block_captured_in_a_graph_replays_like_eager():
    """The whole T-step loop (table hooks: no host callback into Python, no allocation, no memset,
    no host synchronisation) can be captured into a HIP graph; every replay -- with eager work and
    synchronisations between the replays -- gives the eager call's bytes."""
    w = I.small_workload("loopg", B=2, Hq=32, Hkv=2, D=128, S=16, prefix_len=(300, 1200), V=2048, logits_dtype="bf16",
                         sigma=3.0, gamma=0.9, mask_rule="all", peaks=True, T=4, wid=253)
    lens = I.prefix_lengths(w)
    cache = I.prefix_cache(w, lens)
    steps = [I.attn_inputs(w, step=t, lens=lens, cache=False) for t in range(w.T)]
    qkv = [tuple(dev_bf16(steps[t][k]) for k in ("q", "k_blk", "v_blk")) for t in range(w.T)]
    lg = [dev_bf16(I.logits(w, step=t)) for t in range(w.T)]
    table = ([x[0] for x in qkv], [x[1] for x in qkv], [x[2] for x in qkv], lg)
    kc, vc, ln = dev_bf16(cache["k_cache"]), dev_bf16(cache["v_cache"]), dev(lens)
    mask_src = dev(I.initial_mask(w))
    m_d = torch.empty_like(mask_src)
    t_d = torch.zeros(w.B * w.S, dtype=torch.int32, device="cuda")
    out = torch.empty((w.B, w.S, w.Hq, w.D), dtype=torch.bfloat16, device="cuda")
    su = torch.zeros(w.B, dtype=torch.int32, device="cuda")
    cps = torch.zeros((w.T, w.B), dtype=torch.int32, device="cuda")
    ad = bd.attn_desc(w.B, w.Hq, w.Hkv, w.D, w.S, kc.shape[2])
    ud = bd.unmask_desc(w.B, w.S, w.V, None, True, w.gamma)
    ws = torch.empty(bd.denoise_workspace_bytes(ad, ud), dtype=torch.uint8, device="cuda")

    def call():
        m_d.copy_(mask_src)
        bd.denoise_block(None, None, kc, vc, ln, m_d, t_d, w.T, w.Hq, w.gamma, w.S, w.V, out=out, workspace=ws,
                         step_table=table, steps_used=su, commits_per_step=cps)

    call()
    torch.cuda.synchronize()
    ref = [x.clone() for x in (m_d, t_d, out.view(torch.int16), su, cps)]
    s = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        call()
    torch.cuda.synchronize()
    for rep in range(3):
        for x in (t_d, out, su, cps):
            x.zero_()
        graph.replay()
        torch.cuda.synchronize()
        got = (m_d, t_d, out.view(torch.int16), su, cps)
        assert all(torch.equal(a, b) for a, b in zip(got, ref)), f"replay {rep}"
        call()   # eager work between the replays
        torch.cuda.synchronize()
        assert torch.equal(t_d, ref[1])
