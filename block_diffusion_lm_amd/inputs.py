"""Seeded synthetic inputs for the block-diffusion denoise step.

This module only *draws* inputs: random normals, masks, prefix lengths and
planted logit peaks. It holds none of the step's arithmetic (no attention, no
softmax, no commit rule), so the CPU oracle and the HIP path can both consume
exactly the same bytes without sharing any code of the method.

Shapes and value distributions follow the workloads the pages describe:

* block sizes S = 16 (TwoTower default) and S = 32 (Nemotron-Labs Diffusion
  "FastDiffuser" blocks) -- Nemotron-TwoTower technical summary, §Results
  (block-size sensitivity); Nemotron-Labs Diffusion blog, generation modes;
* context lengths 8192 / 65K / 262K tokens -- Hybrid Block Diffusion with
  Partial Bidirectionality summary, technical §Results (throughput);
* bf16 tensors (the released TwoTower checkpoint is BF16 -- Nemotron-Labs-
  TwoTower blog note, reference 2).

They stand in for the public suites the pages evaluate on; no item of any
suite is reproduced.

Every tensor is drawn from ``numpy.random.default_rng([SEED_BASE, workload_id,
tensor_id, step])`` (PCG64). Floating-point tensors are drawn as float32
``standard_normal * sigma`` and rounded to bf16 with round-to-nearest-even;
bf16 tensors are returned as ``uint16`` bit patterns.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

SEED_BASE = 20261203

TENSOR_IDS = {
    "q": 0, "k_blk": 1, "v_blk": 2, "k_cache": 3, "v_cache": 4,
    "logits": 5, "mask": 6, "peaks": 7, "lens": 8, "ties": 9,
    "h_prev": 10, "h_delta": 11,
    "m_h0": 12, "m_x": 13, "m_dt": 14, "m_B": 15, "m_C": 16, "m_A": 17, "m_D": 18,
}


def rng(workload_id: int, tensor: str, step: int = 0) -> np.random.Generator:
    return np.random.default_rng([SEED_BASE, workload_id, TENSOR_IDS[tensor], step])


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round-to-nearest-even); return uint16 bits.

    Inputs must be finite (this module never draws anything else)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + (np.uint32(0x7FFF) + lsb)) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32 (used to plant peaks)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16(g: np.random.Generator, shape, sigma: float = 1.0) -> np.ndarray:
    x = g.standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return f32_to_bf16_bits(x)


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload of the denoise step.

    ``prefix_len`` is an int (every sequence) or a ``(lo, hi)`` range drawn
    uniformly per sequence (inclusive). ``mask_rule`` is ``"half"`` (exactly
    S/2 seeded positions masked), ``"all"`` or ``"frac"`` (fraction
    f_b ~ U[0.25, 1] per sequence, round(f_b * S) seeded positions).
    ``peaks`` plants ``logit = rowmax + 8`` at a seeded token on a seeded half
    of each sequence's positions; ``ties`` additionally plants exact ties.
    """
    name: str
    wid: int
    B: int
    Hq: int
    Hkv: int
    D: int
    S: int
    prefix_len: object
    V: int
    logits_dtype: str          # "bf16" | "f32"
    logit_sigma: float
    gamma: float
    mask_rule: str
    peaks: bool
    ties: bool = False
    T: int = 1                 # denoise steps (the loop workload uses 8)
    min_commit: int = 1

    @property
    def group(self) -> int:
        return self.Hq // self.Hkv

    @property
    def max_prefix_len(self) -> int:
        return self.prefix_len[1] if isinstance(self.prefix_len, tuple) else int(self.prefix_len)


WORKLOADS = {
    # tiny parity case: B1, 8q/2kv, D64, S16, L256; fp32 logits [16,4096] sigma 2, 8 of 16 masked
    "tiny": Workload("tiny", 0, 1, 8, 2, 64, 16, 256, 4096, "f32", 2.0, 0.9, "half", False),
    # single-sequence decode step: B1, 32q/2kv, D128, S16, L4096; bf16 logits, peaks, all masked
    "decode": Workload("decode", 1, 1, 32, 2, 128, 16, 4096, 131072, "bf16", 3.0, 0.9, "all", True),
    # batched step: B32, L8192, S16 and S32; mask fraction U[0.25,1]; gamma 0.8
    "batched16": Workload("batched16", 2, 32, 32, 2, 128, 16, 8192, 131072, "bf16", 3.0, 0.8, "frac", True),
    "batched32": Workload("batched32", 2, 32, 32, 2, 128, 32, 8192, 131072, "bf16", 3.0, 0.8, "frac", True),
    # long context: B4, L65536, S16, T=8 denoise loop with per-step q/k/v/logits
    "long": Workload("long", 3, 4, 32, 2, 128, 16, 65536, 131072, "bf16", 3.0, 0.9, "all", True, T=8),
    # stress (a): one 262144-token prefix
    "stress_a": Workload("stress_a", 4, 1, 32, 2, 128, 16, 262144, 131072, "bf16", 3.0, 0.95, "frac", True, True),
    # stress (b): ragged B16, 32q/8kv, lengths U{1024..32768}
    "stress_b": Workload("stress_b", 5, 16, 32, 8, 128, 16, (1024, 32768), 131072, "bf16", 3.0, 0.95, "frac", True, True),
}


def prefix_lengths(w: Workload) -> np.ndarray:
    if isinstance(w.prefix_len, tuple):
        lo, hi = w.prefix_len
        return rng(w.wid, "lens").integers(lo, hi + 1, size=w.B, dtype=np.int64).astype(np.int32)
    return np.full(w.B, int(w.prefix_len), dtype=np.int32)


def attn_inputs(w: Workload, step: int = 0, lens: Optional[np.ndarray] = None,
                cache: bool = True) -> dict:
    """Q / block K,V (per step) and the prefix cache (step independent).

    Layouts: q [B,S,Hq,D]; k_blk, v_blk [B,S,Hkv,D]; k_cache, v_cache
    [B,Hkv,Lcap,D] with Lcap = max prefix length; rows past prefix_len[b] are
    zero. All bf16 bits (uint16)."""
    if lens is None:
        lens = prefix_lengths(w)
    out = {
        "q": normal_bf16(rng(w.wid, "q", step), (w.B, w.S, w.Hq, w.D)),
        "k_blk": normal_bf16(rng(w.wid, "k_blk", step), (w.B, w.S, w.Hkv, w.D)),
        "v_blk": normal_bf16(rng(w.wid, "v_blk", step), (w.B, w.S, w.Hkv, w.D)),
        "prefix_len": lens.astype(np.int32),
    }
    if cache:
        out.update(prefix_cache(w, lens))
    return out


def prefix_cache(w: Workload, lens: np.ndarray) -> dict:
    lcap = max(1, w.max_prefix_len)
    res = {}
    for name in ("k_cache", "v_cache"):
        g = rng(w.wid, name)
        arr = np.zeros((w.B, w.Hkv, lcap, w.D), dtype=np.uint16)
        for b in range(w.B):
            n = int(lens[b])
            if n:
                arr[b, :, :n, :] = normal_bf16(g, (w.Hkv, n, w.D))
        res[name] = arr
    return res


def initial_mask(w: Workload) -> np.ndarray:
    """uint8 [B*S], 1 = masked."""
    g = rng(w.wid, "mask")
    m = np.zeros((w.B, w.S), dtype=np.uint8)
    for b in range(w.B):
        if w.mask_rule == "all":
            n = w.S
        elif w.mask_rule == "half":
            n = w.S // 2
        elif w.mask_rule == "frac":
            f = g.uniform(0.25, 1.0)
            n = int(np.rint(f * w.S))
        else:
            raise ValueError(w.mask_rule)
        pos = g.permutation(w.S)[:n]
        m[b, pos] = 1
    return m.reshape(-1)


def logits(w: Workload, step: int = 0, additive_peaks: bool = False) -> np.ndarray:
    """Logits [B*S, V]: float32, or bf16 bits (uint16).

    Noise is N(0, sigma) (sigma = standard deviation). With peaks, a seeded
    half of each sequence's positions gets one seeded token set to
    ``rowmax + 8`` (or ``+= 8`` with ``additive_peaks``, an extra input set).

    With ties, a seeded quarter of the rows gets an exact tie for the maximum:
    a row with a planted peak at j gets the same value at a second seeded
    token; a row without one gets two seeded tokens j1 < j2 both set to
    ``rowmax + 2``. Sequence 0 also gets a fallback tie: its rows carry no
    peak, its first masked row gets one token at ``rowmax + 4`` and its last
    masked row becomes a verbatim copy of that row, so the two most confident
    positions of the sequence are bit-identical and the earlier must win."""
    rows = w.B * w.S
    x = rng(w.wid, "logits", step).standard_normal(size=(rows, w.V), dtype=np.float32)
    x *= np.float32(w.logit_sigma)
    bf = w.logits_dtype == "bf16"
    if bf:
        x = bf16_bits_to_f32(f32_to_bf16_bits(x))
    mask = initial_mask(w).reshape(w.B, w.S)
    fb_seq = w.ties and int(mask[0].sum()) >= 2
    peak_at = np.full(rows, -1, dtype=np.int64)
    if w.peaks:
        gp = rng(w.wid, "peaks", step)
        for b in range(w.B):
            pos = gp.permutation(w.S)[: w.S // 2]
            for s in pos:
                r = b * w.S + int(s)
                j = int(gp.integers(0, w.V))
                if fb_seq and b == 0:
                    continue
                if additive_peaks:
                    x[r, j] = x[r, j] + np.float32(8.0)
                else:
                    x[r, j] = x[r].max() + np.float32(8.0)
                peak_at[r] = j
    if w.ties:
        gt = rng(w.wid, "ties", step)
        for r in gt.permutation(rows)[: rows // 4]:
            r = int(r)
            if fb_seq and r < w.S:
                continue
            if peak_at[r] >= 0:
                j2 = int(gt.integers(0, w.V - 1))
                j2 += int(j2 >= peak_at[r])          # any token but the peak
                x[r, j2] = x[r, peak_at[r]]
            else:
                j1, j2 = sorted(int(v) for v in gt.choice(w.V, size=2, replace=False))
                x[r, j1] = x[r, j2] = x[r].max() + np.float32(2.0)
        if fb_seq:
            masked = np.flatnonzero(mask[0])
            s1, s2 = int(masked[0]), int(masked[-1])
            j = int(gt.integers(0, w.V))
            x[s1, j] = x[s1].max() + np.float32(4.0)
            x[s2] = x[s1]
    if bf:
        return f32_to_bf16_bits(x)
    return np.ascontiguousarray(x, dtype=np.float32)


def small_workload(name: str = "small", B: int = 2, Hq: int = 8, Hkv: int = 2, D: int = 64,
                   S: int = 16, prefix_len=200, V: int = 1000, logits_dtype: str = "f32",
                   sigma: float = 2.0, gamma: float = 0.9, mask_rule: str = "frac",
                   peaks: bool = True, ties: bool = False, T: int = 1, wid: int = 100) -> Workload:
    """Ad-hoc small workloads for parity sweeps (shapes spanning several tiles and a ragged tail)."""
    return Workload(name, wid, B, Hq, Hkv, D, S, prefix_len, V, logits_dtype, sigma, gamma,
                    mask_rule, peaks, ties, T)


def loop_states(wid: int, B: int, n: int, scales, bf16: bool = True, zero_prev=(), same=()):
    """Hidden states of a looped mid-block after two consecutive iterations, [B, n] each.

    h_prev ~ N(0, 1); h_cur = h_prev + scales[b] * N(0, 1), drawn in float32 and then rounded
    to bf16 (uint16 bits) when ``bf16``. Sequences listed in ``zero_prev`` get h_prev = 0;
    those in ``same`` get h_cur = h_prev (no change). No hidden size is given for the looped
    model, so n (positions x hidden units) is the caller's choice."""
    x = rng(wid, "h_prev").standard_normal(size=(B, n), dtype=np.float32)
    y = rng(wid, "h_delta").standard_normal(size=(B, n), dtype=np.float32)
    y *= np.asarray(scales, np.float32).reshape(B, 1)
    y += x
    for b in zero_prev:
        x[b] = 0
    for b in same:
        y[b] = x[b]
    if bf16:
        return f32_to_bf16_bits(x).reshape(B, n), f32_to_bf16_bits(y).reshape(B, n)
    return x, y


def mamba_inputs(wid: int, B: int, S: int, H: int, G: int, N: int, P: int = 64) -> dict:
    """Inputs of one block-local bidirectional Mamba scan: the cached boundary state h0 ~ N(0,1)
    float32 [B,H,N,P]; per direction (forward = step 0, reverse = step 1 of the seeds) x ~ N(0,1)
    bf16 [B,S,H,P], B and C ~ N(0,1)/sqrt(N) bf16 [B,S,G,N], step sizes dt ~ U[0.01, 0.2] float32
    [B,S,H] and decay rates A = -U[1, 16] float32 [H] (the range of Mamba-2's initialisation);
    skip D ~ N(0,1) float32 [H]. bf16 tensors are uint16 bit patterns."""
    def side(step):
        x = normal_bf16(rng(wid, "m_x", step), (B, S, H, P))
        sc = np.float32(1.0 / np.sqrt(N))
        Bm = f32_to_bf16_bits(rng(wid, "m_B", step).standard_normal((B, S, G, N), dtype=np.float32) * sc)
        Cm = f32_to_bf16_bits(rng(wid, "m_C", step).standard_normal((B, S, G, N), dtype=np.float32) * sc)
        dt = rng(wid, "m_dt", step).uniform(0.01, 0.2, size=(B, S, H)).astype(np.float32)
        A = (-rng(wid, "m_A", step).uniform(1.0, 16.0, size=H)).astype(np.float32)
        return {"x": x, "dt": dt, "Bm": Bm, "Cm": Cm, "A": A}
    return {"h0": rng(wid, "m_h0").standard_normal((B, H, N, P), dtype=np.float32),
            "fwd": side(0), "rev": side(1),
            "D": rng(wid, "m_D").standard_normal(H, dtype=np.float32)}
