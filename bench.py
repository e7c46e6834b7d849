"""Benchmark of the block-diffusion denoise step on one MI355X.

A step is one pass of the whole hot path: one bd_denoise_block call that runs the T-step loop
over a block -- per step the block+prefix attention (split and merge kernels), then the
confidence unmasking (vocabulary reduction and commit kernels) -- on seeded synthetic inputs
already resident in HBM.

Default workload: the long-context loop -- B=4 sequences, 32 query / 2 KV heads, head_dim 128,
block S=16, prefix L=65536, vocabulary 131072 (bf16 logits, planted peaks), T=8 steps, gamma=0.9,
commit-at-least-one, every remaining position committed at the last step. Other workloads can be
selected with --workload (single-step ones run T=1).

Prints ONE JSON line. `value` is attention TFLOP/s over the whole step (all attention FLOPs the
loop executes divided by the wall time of the loop, unmasking included); the per-kernel figures
come from HIP events recorded around every kernel launch inside the timed region (libbd's
kernel trace, on the launch stream). The CPU baseline times the float64 oracle on a bounded
sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA


def attn_units(w, lens, active):
    """Algorithmic work of one attention launch over the active sequences.

    flops = sum_b 4 * Hq * S * (len_b + S) * D (Q K^T and P V);
    kv_bytes = sum_b 2 * Hkv * (len_b + S) * D * 2 (prefix and block K and V, bf16, read once);
    q_bytes = sum_b S * Hq * D * 2; o_bytes the same (written by the merge)."""
    fl = kv = qb = 0
    for b in range(w.B):
        if not active[b]:
            continue
        n = int(lens[b]) + w.S
        fl += 4 * w.Hq * w.S * n * w.D
        kv += 2 * w.Hkv * n * w.D * 2
        qb += w.S * w.Hq * w.D * 2
    return fl, kv, qb


def cpu_baseline(w, inputs, logits0, mask0, budget_s=20.0):
    """Time the oracle as it stands on a bounded sample of the workload: the attention of
    whole (sequence, KV head) groups of step 0 and the vocabulary reduction of masked rows."""
    from oracle import bd_oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([int(i.get("num_threads", 1)) for i in threadpool_info()] + [1])
    except Exception:
        cores = len(os.sched_getaffinity(0))
    lens = inputs["prefix_len"]
    # whole passes over step 0's attention (every (sequence, KV head) group), repeated until about
    # 70 % of the budget is spent (at least one pass), then the vocabulary reduction of the masked
    # rows, repeated for the rest
    t0 = time.perf_counter()
    fl = 0
    pairs = 0
    passes = 0
    while passes == 0 or time.perf_counter() - t0 < budget_s * 0.7:
        for b in range(w.B):
            for g in range(w.Hkv):
                rows = [(b, s, h) for s in range(w.S) for h in range(g * w.group, (g + 1) * w.group)]
                O.attn_rows(inputs["q"], inputs["k_blk"], inputs["v_blk"], inputs["k_cache"], inputs["v_cache"], lens,
                            rows)
                fl += 4 * len(rows) * (int(lens[b]) + w.S) * w.D
                pairs += 1
        passes += 1
    t_attn = time.perf_counter() - t0
    t1 = time.perf_counter()
    masked = np.flatnonzero(mask0)
    dec = O.bf16_to_f64 if w.logits_dtype == "bf16" else None
    n = 0
    while n == 0 or time.perf_counter() - t1 < budget_s * 0.3:
        for r in masked:
            O.confidences(logits0[r:r + 1], np.ones(1, np.uint8), dec)
            n += 1
    t_um = time.perf_counter() - t1
    return {"value": fl / t_attn / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"float64 oracle: {passes} pass(es) over step 0's attention ({w.B * w.Hkv} (sequence, KV head) "
                      f"groups, {w.B * w.S * w.Hq} query rows over {int(lens[0]) + w.S} keys each) in {t_attn:.1f} s; "
                      f"vocabulary reduction of {n} masked rows ({len(masked)} distinct) in {t_um:.1f} s",
            "unmask_positions_per_s": n / t_um if t_um > 0 else None}


def row_figures(args, w, bd, torch, dev, recs, steps_used, commits, mask0, lens, ad, ws, dq, dlog, caches, lens_d,
                is_bf16, T):
    """Per-row kernel durations (trace events) with their algorithmic bytes and HBM fraction.

    Rows of the step, from the traced loop region, over the steps in which every sequence is
    active: attn_split (K, V, Q read), attn_merge (the split partials read back, the output
    written), vocab_reduce (the masked rows' logits), commit (latency only). Rows after the step,
    each timed on its own with the same trace (5 launches, first dropped): the context tower's
    causal pass over the block (bd_attn_step, causal), the append of the block to a cache
    (bd_kv_append), the self-speculation check of a drafted block (bd_spec_verify) and adaptive
    loop halting (bd_loop_halt) on two hidden states of 32 x 1024 positions x 4096 units, bf16."""
    per = {}
    for name, ms in recs:
        per.setdefault(name, []).append(ms)
    # the loop enqueues all T steps (the early exit happens on the device), so every kernel of the
    # step has T launches per call; step t is full when every sequence is still active at t
    full = [t for t in range(T) if (steps_used > t).all()]
    lg_bytes = 2 if is_bf16 else 4
    out_bytes = w.B * w.S * w.Hq * w.D * 2
    fl, kv, qb = attn_units(w, lens, np.ones(w.B, bool))
    remaining = mask0.reshape(w.B, w.S).sum(axis=1).astype(np.int64)
    masked_at = []
    for t in range(T):
        masked_at.append(int(remaining.sum()))
        remaining -= commits[t]
    part_bytes = bd.attn_workspace_bytes(ad)

    def pick(name, ts):
        v = per.get(name, [])
        return [v[c * T + t] for c in range(len(v) // T) for t in ts]

    def fig(ms_list, nbytes):
        if not ms_list:
            return None
        avg = float(np.mean(ms_list))
        r = {"avg_us": round(avg * 1e3, 2), "launches": len(ms_list)}
        if nbytes:
            gbs = nbytes / (avg * 1e-3) / 1e9
            r.update({"bytes_per_launch": int(nbytes), "gbs": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)})
        return r

    rows = {"attn_split": fig(pick("attn_split", full), kv + qb),
            "attn_merge": fig(pick("attn_merge", full), part_bytes + out_bytes),
            "vocab_reduce": fig(pick("vocab_reduce", [0]), masked_at[0] * w.V * lg_bytes),
            "commit": fig(pick("commit", full), None)}

    # rows after the step, each on its own
    kc, vc = caches[0]
    q, kb, vb = dq[0]
    tr = bd.Trace(capacity=64)
    with tr:
        for _ in range(5):
            bd.attn_step(q, kb, vb, kc, vc, lens_d, max_prefix_len=w.max_prefix_len, causal=True, want_lse=False,
                         workspace=ws)
    cp = {}
    for name, ms in tr.records():
        cp.setdefault(name, []).append(ms)
    tr.clear()
    ctx = [a + b for a, b in zip(cp.get("attn_split", [])[1:], cp.get("attn_merge", [0] * 5)[1:])]
    rows["context_pass"] = fig(ctx, kv + qb + out_bytes)
    kc_s = torch.zeros((w.B, w.Hkv, w.S, w.D), dtype=torch.bfloat16, device=dev)
    vc_s = torch.zeros_like(kc_s)
    len_s = torch.zeros(w.B, dtype=torch.int32, device=dev)
    with tr:
        for _ in range(5):
            len_s.zero_()
            bd.kv_append(kb, vb, kc_s, vc_s, len_s, max_prefix_len=0)
    ap = {}
    for name, ms in tr.records():
        ap.setdefault(name, []).append(ms)
    tr.clear()
    # one launch per call for small blocks (copy and length advance together), else two
    app = ap.get("kv_append", [])[1:]
    if ap.get("len_advance"):
        app = [a + b for a, b in zip(app, ap["len_advance"][1:])]
    rows["kv_append"] = fig(app, 2 * 2 * w.B * w.S * w.Hkv * w.D * 2)
    draft = torch.zeros(w.B * w.S, dtype=torch.int32, device=dev)
    first = torch.zeros(w.B, dtype=torch.int32, device=dev)
    ws_u = torch.empty(max(bd.unmask_workspace_bytes(bd.unmask_desc(w.B, w.S, w.V, None, is_bf16)), 1),
                       dtype=torch.uint8, device=dev)
    with tr:
        for _ in range(5):
            bd.spec_verify(dlog[0], draft, first, w.S, vocab=w.V, workspace=ws_u)
    sv = {}
    for name, ms in tr.records():
        sv.setdefault(name, []).append(ms)
    tr.close()
    spec = [a + b for a, b in zip(sv.get("vocab_reduce", [])[1:], sv.get("spec_accept", [])[1:])]
    rows["spec_verify"] = fig(spec, w.B * w.S * w.V * lg_bytes)
    hb, hn = 32, 1024 * 4096
    g = torch.Generator(device=dev)
    g.manual_seed(20261203)
    h_prev = torch.randn((hb, hn), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    h_cur = (h_prev.float() + 1e-2 * torch.randn((hb, hn), generator=g, device=dev)).to(torch.bfloat16)
    ws_h = torch.empty(bd.loop_halt_workspace_bytes(bd.halt_desc(hb, hn)), dtype=torch.uint8, device=dev)
    tr = bd.Trace(capacity=64)
    with tr:
        for _ in range(5):
            bd.loop_halt(h_prev, h_cur, 2, 1e-3, 12, workspace=ws_h)
    lh = {}
    for name, ms in tr.records():
        lh.setdefault(name, []).append(ms)
    tr.close()
    halt = [a + b for a, b in zip(lh.get("halt_reduce", [])[1:], lh.get("halt_final", [])[1:])]
    rows["loop_halt"] = fig(halt, 2 * hb * hn * 2)
    del h_prev, h_cur
    torch.cuda.synchronize()
    return rows


def config_rows(bd, dev):
    """One row per workload besides the loop's: the attention step (split + merge kernels) and the
    confidence unmasking (vocabulary reduction + commit kernels) at full size -- single-sequence
    decode (L 4096), the batched step at S = 16 and S = 32 (32 sequences, L 8192), one 262144-token
    prefix, and the ragged batch (16 sequences, 8 KV heads, the workload's seeded lengths in
    [1024, 32768]). Attention inputs are seeded N(0,1) bf16 and logits N(0,3) bf16 drawn on the
    device (the workload's shapes, lengths and masked positions); three independent cache and
    logits sets rotate so consecutive launches do not find their bytes in the 256 MB Infinity
    Cache. 7 launches of each with the kernel trace, the first dropped.

    Attention: TFLOP/s and K/V/Q GB/s over split + merge, with their fractions of the dense bf16
    MFMA peak and of HBM; unmask: masked positions per second over reduction + commit, against the
    HBM roofline 8e12 / (V * 2) positions/s."""
    import torch
    from block_diffusion_lm_amd import inputs as I
    out_rows = {}
    g = torch.Generator(device=dev)
    g.manual_seed(20261205)
    for name in ("decode", "batched16", "batched32", "stress_a", "stress_b"):
        w = I.WORKLOADS[name]
        print(f"[bench] row {name}", file=sys.stderr, flush=True)
        lens_np = I.prefix_lengths(w)
        lcap = int(lens_np.max())
        rnd = lambda *shape: torch.randn(shape, generator=g, device=dev).to(torch.bfloat16)
        sets = [(rnd(w.B, w.Hkv, lcap, w.D), rnd(w.B, w.Hkv, lcap, w.D)) for _ in range(3)]
        q, kb, vb = rnd(w.B, w.S, w.Hq, w.D), rnd(w.B, w.S, w.Hkv, w.D), rnd(w.B, w.S, w.Hkv, w.D)
        lens = torch.from_numpy(lens_np).to(dev)
        ad = bd.attn_desc(w.B, w.Hq, w.Hkv, w.D, w.S, lcap, lcap)
        ws = torch.empty(max(bd.attn_workspace_bytes(ad), 1), dtype=torch.uint8, device=dev)
        out = torch.empty_like(q)
        tr = bd.Trace(capacity=64)
        with tr:
            for i in range(7):
                kc, vc = sets[i % 3]
                bd.attn_step(q, kb, vb, kc, vc, lens, out=out, want_lse=False, max_prefix_len=lcap, workspace=ws)
        per = {}
        for n, ms in tr.records():
            per.setdefault(n, []).append(ms)
        tr.clear()
        split = float(np.mean(per["attn_split"][1:])) * 1e3
        merge = float(np.mean(per["attn_merge"][1:])) * 1e3 if per.get("attn_merge") else 0.0
        fl, kv, qb = attn_units(w, lens_np, np.ones(w.B, bool))
        at = split + merge
        del sets
        torch.cuda.synchronize()
        logit_sets = [(torch.randn((w.B * w.S, w.V), generator=g, device=dev) * 3.0).to(torch.bfloat16)
                      for _ in range(3)]
        mask_np = I.initial_mask(w)
        mask0 = torch.from_numpy(mask_np).to(dev)
        mask = mask0.clone()
        tok = torch.zeros(w.B * w.S, dtype=torch.int32, device=dev)
        ud = bd.unmask_desc(w.B, w.S, w.V, None, True, w.gamma, True, False)
        uws = torch.empty(max(bd.unmask_workspace_bytes(ud), 1), dtype=torch.uint8, device=dev)
        with tr:
            for i in range(7):
                mask.copy_(mask0)
                bd.confidence_unmask(logit_sets[i % 3], mask, tok, w.S, w.gamma, outputs=False, workspace=uws)
        per = {}
        for n, ms in tr.records():
            per.setdefault(n, []).append(ms)
        tr.close()
        red = float(np.mean(per["vocab_reduce"][1:])) * 1e3
        com = float(np.mean(per["commit"][1:])) * 1e3
        nm = int(mask_np.sum())
        pos_s = nm / ((red + com) * 1e-6)
        roof = HBM_PEAK_GBS * 1e9 / (w.V * 2)
        out_rows[name] = {
            "workload": f"{name}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} D={w.D} S={w.S} L={w.prefix_len} V={w.V}",
            "attn": {"split_us": round(split, 2), "merge_us": round(merge, 2),
                     "tflops": round(fl / (at * 1e-6) / 1e12, 1),
                     "mfma_frac": round(fl / (at * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4),
                     "gbs": round((kv + qb) / (at * 1e-6) / 1e9, 1),
                     "frac_hbm": round((kv + qb) / (at * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                     "frac_hbm_split_only": round((kv + qb) / (split * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                     "bytes": int(kv + qb), "flops": int(fl)},
            "unmask": {"masked_rows": nm, "reduce_us": round(red, 2), "commit_us": round(com, 2),
                       "positions_per_s": round(pos_s, 1), "frac_roofline": round(pos_s / roof, 4),
                       "reduce_gbs": round(nm * w.V * 2 / (red * 1e-6) / 1e9, 1)},
        }
        del logit_sets, q, kb, vb, ws, out
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return out_rows


def mamba_row(bd, dev):
    """The block-local bidirectional Mamba scan at its measured shape (32 sequences x 64 heads x
    P 64, N 128 in 8 groups, S 16): a denoising step (y only: the cached boundary state is read,
    not advanced) and the committing pass (y and the new boundary state). Inputs seeded on the
    device (x, B, C ~ N(0,1) bf16 with B, C scaled by N^-1/2; dt ~ U[0.01, 0.2]; A ~ -U[1, 16]);
    three state sets rotate so that no launch finds h0 in the Infinity Cache. Algorithmic bytes:
    h0 read (+ h_out written), x and dt of both directions, B and C of both directions, y written,
    A, A_r and D."""
    import torch
    B, S, H, G, N, P = 32, 16, 64, 8, 128, 64
    g = torch.Generator(device=dev)
    g.manual_seed(20261206)
    bf = lambda *shape, sc=1.0: (torch.randn(shape, generator=g, device=dev) * sc).to(torch.bfloat16)
    uni = lambda *shape, lo, hi: torch.rand(shape, generator=g, device=dev) * (hi - lo) + lo
    sides = [(bf(B, S, H, P), uni(B, S, H, lo=0.01, hi=0.2), bf(B, S, G, N, sc=N ** -0.5), bf(B, S, G, N, sc=N ** -0.5))
             for _ in range(2)]
    A, Ar = -uni(H, lo=1.0, hi=16.0), -uni(H, lo=1.0, hi=16.0)
    D = torch.randn(H, generator=g, device=dev)
    states = [torch.randn((B, H, N, P), generator=g, device=dev) for _ in range(3)]
    y = torch.empty((B, S, H, P), dtype=torch.bfloat16, device=dev)
    h_out = torch.empty_like(states[0])
    inputs = 2 * (B * S * H * P * 2 + B * S * H * 4 + 2 * B * S * G * N * 2) + B * S * H * P * 2 + 3 * H * 4
    state = B * H * N * P * 4
    res = {"workload": f"mamba_h: B={B} H={H} P={P} N={N} G={G} S={S}"}
    for name, want in (("step", False), ("commit", True)):
        tr = bd.Trace(capacity=64)
        with tr:
            for i in range(7):
                bd.mamba_block_scan(states[i % 3], sides[0], sides[1], A, Ar, D, y=y, h_out=h_out if want else None,
                                    want_h_out=want)
        ms = [m for n, m in tr.records() if n == "mamba_block"]
        tr.close()
        us = float(np.mean(ms[1:])) * 1e3
        nbytes = inputs + state * (2 if want else 1)
        res[name] = {"us": round(us, 2), "bytes": int(nbytes), "gbs": round(nbytes / (us * 1e-6) / 1e9, 1),
                     "frac_hbm": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    del states, sides, y, h_out
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def per_step_kernel_us(recs, T: int, names=("attn_split", "attn_merge", "vocab_reduce", "commit")) -> dict:
    """Median duration (us) of each loop kernel at each step t, over the traced calls: records are
    (kernel, ms) in launch order and every call launches each kernel once per step; a kernel whose
    launch count is not a multiple of T is left out."""
    out = {}
    for name in names:
        ms = [m for n, m in recs if n == name]
        if not ms or len(ms) % T:
            continue
        a = np.asarray(ms, np.float64).reshape(len(ms) // T, T)
        out[name] = [round(float(v) * 1e3, 2) for v in np.median(a, axis=0)]
    return out


def code_sha256(source: str) -> str:
    """SHA-256 of a source file's code: every line with its // comment and surrounding blanks
    removed, blank lines dropped (comment edits leave it unchanged; any code change alters it)."""
    import hashlib
    import re
    lines = []
    with open(source) as f:
        for line in f:
            code = re.sub(r"//.*$", "", line).strip()
            if code:
                lines.append(code)
    return hashlib.sha256("\n".join(lines).encode()).hexdigest()


def measured_traffic(kernel_source: str):
    """HBM traffic per launch of the attention split kernel from the committed counter summary
    (rocprofv3 FETCH_SIZE / WRITE_SIZE, scaled by a plain copy kernel), or None when the summary
    is missing or was taken on different kernel code."""
    path = os.path.join(ROOT, "profiles", "attn_split_long_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("code_sha256") != code_sha256(kernel_source):
        return None
    return rec.get("traffic_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="long")
    ap.add_argument("--sets", type=int, default=3, help="independent prefix caches rotated between steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-config-rows", action="store_true", help="skip the per-workload attention/unmask rows")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 512 MiB device copy (5 times): the reference for HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (one MI355X per process); "
              "use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.calibrate_copy:
        src = torch.empty(512 << 20, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "device copy", "bytes_read_per_launch": 512 << 20,
                          "bytes_written_per_launch": 512 << 20}))
        return

    import block_diffusion_lm_amd as bd
    from block_diffusion_lm_amd import inputs as I

    w = I.WORKLOADS[args.workload]
    T = w.T
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def d16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    print(f"[bench] generating inputs for {w.name}", file=sys.stderr, flush=True)
    lens = I.prefix_lengths(w)
    inp0 = I.attn_inputs(w, step=0, lens=lens)
    steps = [I.attn_inputs(w, step=t, lens=lens, cache=False) if t else inp0 for t in range(T)]
    dq = [tuple(d16(steps[t][k]) for k in ("q", "k_blk", "v_blk")) for t in range(T)]
    logits_np = [I.logits(w, step=t) for t in range(T)]
    is_bf16 = w.logits_dtype == "bf16"
    dlog = [d16(x) if is_bf16 else torch.from_numpy(x).to(dev) for x in logits_np]
    mask0 = I.initial_mask(w)
    caches = [(d16(inp0["k_cache"]), d16(inp0["v_cache"]))]
    g = torch.Generator(device=dev)
    g.manual_seed(20261203)
    for _ in range(1, args.sets):   # same distribution (bf16 N(0,1)), distinct bytes
        caches.append(tuple(torch.randn(inp0["k_cache"].shape, generator=g, device=dev).to(torch.bfloat16)
                            for _ in range(2)))
    lens_d = torch.from_numpy(lens).to(dev)
    mask_d = torch.from_numpy(mask0).to(dev)
    tok_d = torch.zeros(w.B * w.S, dtype=torch.int32, device=dev)
    out = torch.empty((w.B, w.S, w.Hq, w.D), dtype=torch.bfloat16, device=dev)

    ad = bd.attn_desc(w.B, w.Hq, w.Hkv, w.D, w.S, inp0["k_cache"].shape[2], w.max_prefix_len)
    ud = bd.unmask_desc(w.B, w.S, w.V, None, is_bf16, w.gamma, True, False)
    ws = torch.empty(max(bd.denoise_workspace_bytes(ad, ud), 1), dtype=torch.uint8, device=dev)

    table = ([x[0] for x in dq], [x[1] for x in dq], [x[2] for x in dq], dlog)
    steps_used_d = torch.zeros(w.B, dtype=torch.int32, device=dev)
    cps_d = torch.zeros((T, w.B), dtype=torch.int32, device=dev)

    def step(i):
        kc, vc = caches[i % len(caches)]
        mask_d.copy_(mask_src)   # every step denoises the same fresh block
        return bd.denoise_block(None, None, kc, vc, lens_d, mask_d, tok_d, T, w.Hq, w.gamma, w.S, w.V,
                                logits_bf16=is_bf16, out=out, workspace=ws, step_table=table,
                                steps_used=steps_used_d, commits_per_step=cps_d)

    mask_src = torch.from_numpy(mask0).to(dev)
    for i in range(args.warmup):
        r = step(i)
    torch.cuda.synchronize()
    steps_used = r["steps_used"].cpu().numpy()
    commits = r["commits_per_step"].cpu().numpy()

    # Timed region: K steps, no tracing (the per-step mask reset, a 64-byte device copy, is part of
    # every step). A second region of K steps runs with libbd's kernel trace attached: HIP events
    # recorded around every kernel launch on the launch stream give the per-kernel durations.
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    trace = bd.Trace(capacity=args.steps * (4 * T + 1) + 16)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    with trace:
        for i in range(args.steps):
            step(i)
    torch.cuda.synchronize()
    wall_traced = time.perf_counter() - t1
    recs = trace.records()
    trace.close()

    # control flow is deterministic: sequences active at step t are those with steps_used > t
    per_kernel = {}
    for name, ms in recs:
        per_kernel.setdefault(name, []).append(ms)
    split_ms = per_kernel.get("attn_split", [])
    merge_ms = per_kernel.get("attn_merge", [])
    red_ms = per_kernel.get("vocab_reduce", [])
    com_ms = per_kernel.get("commit", [])
    fl_step = kv_step = q_step = 0
    masked_rows_step = 0
    m = mask0.reshape(w.B, w.S).copy()
    per_launch_bytes = []
    for t in range(T):
        active = steps_used > t
        fl, kv, qb = attn_units(w, lens, active)
        fl_step += fl
        kv_step += kv
        q_step += qb
        per_launch_bytes.append(kv + qb)
    # masked rows read by the vocabulary reduction, step by step (from the commit counts)
    remaining = mask0.reshape(w.B, w.S).sum(axis=1).astype(np.int64)
    for t in range(T):
        masked_rows_step += int(remaining.sum())
        remaining -= commits[t]
    K = args.steps
    ms_per_step = wall / K * 1e3
    attn_ms = (sum(split_ms) + sum(merge_ms)) / K
    unmask_ms = (sum(red_ms) + sum(com_ms)) / K
    split_avg = float(np.mean(split_ms))
    bytes_per_launch = float(np.mean(per_launch_bytes))
    achieved_gbs = bytes_per_launch / (split_avg * 1e-3) / 1e9
    value = fl_step / (ms_per_step * 1e-3) / 1e12
    line = {
        "metric": "denoise-step attn TFLOP/s & KV GB/s (% roofline); unmask positions/s",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "ms_per_step_traced": round(wall_traced / K * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: denoise loop B={w.B} Hq={w.Hq} Hkv={w.Hkv} D={w.D} S={w.S} "
                               f"L={w.prefix_len} V={w.V} T={T} gamma={w.gamma}",
                   "global_batch": w.B, "block_len": w.S, "prefix_len": w.max_prefix_len, "T": T,
                   "vocab": w.V, "parallelism": "none (1 GPU)"},
        "attention": {
            "ms_per_step": round(attn_ms, 4),
            "tflops": round(fl_step / (attn_ms * 1e-3) / 1e12, 3),
            "tflops_frac_bf16_peak": round(fl_step / (attn_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "kv_gbs": round(kv_step / (attn_ms * 1e-3) / 1e9, 1),
            "kv_frac_hbm_peak": round(kv_step / (attn_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "split_avg_ms": round(split_avg, 5),
            "merge_avg_ms": round(float(np.mean(merge_ms)), 5) if merge_ms else 0.0,
        },
        "unmask": {
            "ms_per_step": round(unmask_ms, 4),
            "positions_per_s": round(masked_rows_step / (unmask_ms * 1e-3), 1),
            "frac_roofline": round(masked_rows_step / (unmask_ms * 1e-3) / (HBM_PEAK_GBS * 1e9 / (w.V * (2 if is_bf16 else 4))), 4),
            "reduce_avg_ms": round(float(np.mean(red_ms)), 5),
        },
        "loop": {"steps_used": steps_used.tolist(), "commits_per_step": commits.sum(axis=1).tolist(),
                 "tokens_per_step": round(float(mask0.sum()) / max(1, int(steps_used.max())), 3),
                 # where the loop's time goes, step by step (full, partly active and empty steps)
                 "kernel_us_per_step": per_step_kernel_us(recs, T)},
        "roofline": {"kernel": "attn_split", "bound": "hbm", "achieved": round(achieved_gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved_gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(os.path.join(ROOT, "block_diffusion_lm_amd", "csrc", "bd_attn.hip")),
                     "algorithmic_bytes_per_launch": round(bytes_per_launch),
                     # the same launches against the dense bf16 MFMA peak (the kernel sits near the ridge)
                     "mfma_frac": round(fl_step / T / (split_avg * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)},
    }
    line["rows"] = row_figures(args, w, bd, torch, dev, recs, steps_used, commits, mask0, lens, ad, ws, dq, dlog,
                               caches, lens_d, is_bf16, T)
    # the same kernel over the launches of full steps only (every sequence active)
    line["roofline"]["frac_full_step_launches"] = line["rows"]["attn_split"]["frac_hbm"]
    if not args.no_config_rows:
        del caches, dq, dlog
        torch.cuda.empty_cache()
        line["configs"] = config_rows(bd, dev)
        print("[bench] row mamba_h", file=sys.stderr, flush=True)
        line["configs"]["mamba_h"] = mamba_row(bd, dev)
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle sample", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(w, inp0, logits_np[0], mask0, args.cpu_budget)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
