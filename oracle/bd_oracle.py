"""CPU float64 oracle of the block-diffusion denoise step.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, links or calls
this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it. It shares no code with the
HIP library (no kernels, headers, helpers, tables or pre/post-processing);
both sides only consume the same seeded input bytes.

Every quantity is computed in numpy float64 from the plain definition of the
step, without blocking, fusion or reordering beyond what the definition
states. Sources (page title, section):

* Attention of the active block -- Nemotron-TwoTower technical summary,
  §Architecture (the denoiser uses bidirectional attention inside the noisy
  block and causal cross-attention into the frozen context tower) and
  §Generation (at every layer the denoiser attends to the context tower's KV
  cache of past blocks and to the current block's bidirectional KV).
* Exact prefix caching -- Hybrid Block Diffusion with Partial Bidirectionality
  summary, technical §Method: the cached prefix state depends on the clean
  prefix only, never on the diffusion step or on the active block.
* Confidence unmasking (Algorithm 2) -- Nemotron-TwoTower technical summary,
  §Training and conditioning, sampling bullet: all masked positions are
  predicted in parallel, those whose confidence is above gamma are committed,
  the others stay masked for further refinement.
* Block loop (Algorithm 1) -- Nemotron-TwoTower technical summary,
  §Generation: a block of S masked tokens is refined for T steps and then
  committed.
* Context-tower update after a commit -- Nemotron-TwoTower technical summary,
  §Architecture (the frozen context tower is a causal autoregressive model
  over the prompt and the committed tokens, producing the KV cache) and
  §Generation (once a block commits, the context tower takes in the new clean
  tokens before the next block): a causal pass over the block (each new token
  sees the prefix and the new tokens up to itself) and the append of the
  block's keys and values to the cache.
* Self-speculation (LinearSpec) -- Nemotron-Labs Diffusion page, decoding
  modes: the same model drafts a block bidirectionally, then checks it
  causally; the matching prefix is committed; lossless against AR decoding at
  temperature 0.
* Adaptive loop halting -- Technical summary: LoopMDM, §Adaptive inference:
  the looped mid-block stops when the relative change of the hidden state
  between consecutive loop iterations falls below epsilon, or when the
  iteration budget is reached.
* Block-local bidirectional Mamba scan (BDLM Mamba-H) -- Hybrid Block Diffusion
  with Partial Bidirectionality summary, technical §Method: completed prefix
  blocks keep only the forward scan's boundary (recurrent) state; the reverse
  scan is confined to the active block, so the cached prefix state is a
  function of the clean prefix alone.

Readings where the pages are silent:
one softmax over prefix keys followed by block keys; every prefix key visible
to every block query; no mask inside the block; scale tau = float32(1/sqrt(D))
unless given; GQA head h reads KV head floor(h * Hkv / Hq); confidence = the
maximum softmax probability at temperature 1; argmax ties -> lowest token
index; commit iff p > gamma (strict) with gamma promoted from float32; when no
masked position passes, the single most confident masked position commits
(ties -> lowest position); at the last step every masked position commits;
commits are final. Causal pass: block key j is visible to block position s iff
j <= s (all prefix keys stay visible). KV append: the block's rows go to cache
positions len .. len+S-1 and len grows by S. Self-speculation: AR's choice for
block position i is the argmax of the causal pass at position i-1 (for i = 0:
the choice carried from the pass before); the committed run is the longest
prefix of the draft equal to AR's choices, followed, when it is shorter than
the block, by AR's own choice at the first mismatch (the token AR decoding
would emit there, so the output stays identical to AR decoding and every
verification commits at least one token). Loop halting: per sequence, the
relative change is ||h_cur - h_prev||_2 / ||h_prev||_2 over all its positions and
hidden units (0/0 counts as no change); the loop halts after iteration k
(1-based) when that change is below epsilon or k has reached the budget.
Mamba-H scan (the pages name the Mamba mixer but print no recurrence): the
Mamba-2 selective scan per head -- a scalar decay exp(dt A) per position, an
input dt B x^T, an output C^T H -- forward from the cached boundary state over
the block, reverse from a zero state over the block only, the two outputs
summed with a skip term D x; the step sizes, decay rates and the B, C, x
projections are inputs, as q, k, v are for the attention.

Pins: every function here is checked in ``tests/test_oracle_pins.py`` against
things other than itself (library routines for special cases, closed forms,
invariants, brute-force enumeration); see the docstrings below.
"""
from __future__ import annotations

import math
from typing import Callable, Iterable, Optional, Sequence

import numpy as np

NEAR_TIE_REL = 1e-4   # decisions closer than this (relative) are reported as near-ties


# ----------------------------------------------------------------------------------------------
# input decoding
# ----------------------------------------------------------------------------------------------
def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly (bf16 is the top half of a float32)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def f32_to_f64(x: np.ndarray) -> np.ndarray:
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def default_scale(D: int) -> float:
    """Softmax scale tau: 1/sqrt(D) evaluated in float32, promoted exactly to float64."""
    return float(np.float32(1.0) / np.sqrt(np.float32(D)))


def kv_head_of(h: int, Hq: int, Hkv: int) -> int:
    """Contiguous GQA groups: query head h reads KV head floor(h * Hkv / Hq)."""
    return (h * Hkv) // Hq


# ----------------------------------------------------------------------------------------------
# attention of the active block over [prefix ; block]
# ----------------------------------------------------------------------------------------------
def keys_values(k_blk, v_blk, k_cache, v_cache, prefix_len, b: int, g: int):
    """Key/value rows visible to the block of sequence b through KV head g:
    prefix rows 0..len_b-1 of the cache, then the S rows of the block (float64)."""
    n = int(prefix_len[b])
    K = np.concatenate([k_cache[b, g, :n, :], k_blk[b, :, g, :]], axis=0)
    V = np.concatenate([v_cache[b, g, :n, :], v_blk[b, :, g, :]], axis=0)
    return K, V


def softmax_attention(Qr: np.ndarray, K: np.ndarray, V: np.ndarray, tau: float, visible=None):
    """O = softmax(tau * Qr K^T) V and LSE = ln sum exp(tau * Qr K^T), row-wise, float64.
    ``visible`` (rows x keys, bool) removes the invisible keys from each row's softmax."""
    s = tau * (Qr @ K.T)
    if visible is not None:
        s = np.where(visible, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    z = e.sum(axis=1, keepdims=True)
    O = (e / z) @ V
    lse = m[:, 0] + np.log(z[:, 0])
    return O, lse


def causal_visible(S: int, n_prefix: int, rows_s: Sequence[int]):
    """Visibility of the causal pass: rows at block positions rows_s see every prefix key and the
    block keys j <= s."""
    j = np.arange(n_prefix + S)
    return np.stack([(j < n_prefix) | (j - n_prefix <= s) for s in rows_s])


def attn_step(q, k_blk, v_blk, k_cache, v_cache, prefix_len, scale: Optional[float] = None,
              active: Optional[Sequence[int]] = None, causal: bool = False):
    """One denoise-step attention for every (b, s, h).

    q [B,S,Hq,D]; k_blk, v_blk [B,S,Hkv,D]; k_cache, v_cache [B,Hkv,Lcap,D];
    prefix_len [B] -- all float64 (decode bf16 first). Returns O [B,S,Hq,D] and
    LSE [B,Hq,S] (float64). Sequences with ``active[b] == 0`` get NaN rows
    (the step does not touch them). ``causal``: the context tower's pass over a
    committed block (block key j visible to block position s iff j <= s)."""
    B, S, Hq, D = q.shape
    Hkv = k_blk.shape[2]
    tau = default_scale(D) if scale is None else float(np.float32(scale))
    O = np.full((B, S, Hq, D), np.nan)
    L = np.full((B, Hq, S), np.nan)
    for b in range(B):
        if active is not None and not active[b]:
            continue
        for h in range(Hq):
            K, V = keys_values(k_blk, v_blk, k_cache, v_cache, prefix_len, b, kv_head_of(h, Hq, Hkv))
            vis = causal_visible(S, int(prefix_len[b]), range(S)) if causal else None
            o, lse = softmax_attention(q[b, :, h, :], K, V, tau, vis)
            O[b, :, h, :] = o
            L[b, h, :] = lse
    return O, L


def attn_rows(q, k_blk, v_blk, k_cache, v_cache, prefix_len, rows: Iterable, scale=None, causal: bool = False):
    """Same definition for selected (b, s, h) triples only (full-size sampled checks).

    Inputs may be bf16 bit arrays (uint16) or float64; only the slabs needed
    are decoded. Returns {(b, s, h): (o[D], lse)}."""
    dec = (lambda a: bf16_to_f64(a)) if np.asarray(q).dtype == np.uint16 else (lambda a: np.asarray(a, np.float64))
    B, S, Hq, D = q.shape
    Hkv = k_blk.shape[2]
    tau = default_scale(D) if scale is None else float(np.float32(scale))
    out = {}
    by_bg = {}
    for (b, s, h) in rows:
        by_bg.setdefault((b, kv_head_of(h, Hq, Hkv)), []).append((b, s, h))
    for (b, g), lst in by_bg.items():
        n = int(prefix_len[b])
        K = np.concatenate([dec(k_cache[b, g, :n, :]), dec(k_blk[b, :, g, :])], axis=0)
        V = np.concatenate([dec(v_cache[b, g, :n, :]), dec(v_blk[b, :, g, :])], axis=0)
        Qr = np.stack([dec(q[b, s, h, :]) for (_, s, h) in lst])
        vis = causal_visible(S, n, [s for (_, s, _) in lst]) if causal else None
        o, lse = softmax_attention(Qr, K, V, tau, vis)
        for i, key in enumerate(lst):
            out[key] = (o[i], float(lse[i]))
    return out


def chunk_partials(Qr: np.ndarray, K: np.ndarray, V: np.ndarray, tau: float, bounds: Sequence[int]):
    """Per key chunk [bounds[i], bounds[i+1]): running max m_c, l_c = sum exp(s - m_c) and
    acc_c = sum exp(s - m_c) v. Empty chunks give m = -inf, l = 0, acc = 0."""
    parts = []
    s_all = tau * (Qr @ K.T)
    for c0, c1 in zip(bounds[:-1], bounds[1:]):
        if c1 <= c0:
            parts.append((np.full(Qr.shape[0], -np.inf), np.zeros(Qr.shape[0]), np.zeros((Qr.shape[0], V.shape[1]))))
            continue
        s = s_all[:, c0:c1]
        m = s.max(axis=1)
        e = np.exp(s - m[:, None])
        parts.append((m, e.sum(axis=1), e @ V[c0:c1]))
    return parts


def merge_partials(parts):
    """Combine chunk partials: M = max_c m_c; O = sum_c acc_c e^(m_c - M) / sum_c l_c e^(m_c - M);
    LSE = M + ln sum_c l_c e^(m_c - M). Chunks are combined in index order."""
    M = np.max(np.stack([p[0] for p in parts]), axis=0)
    num = np.zeros_like(parts[0][2])
    den = np.zeros_like(parts[0][1])
    for m, l, acc in parts:
        w = np.where(np.isfinite(m), np.exp(m - M), 0.0)
        num += acc * w[:, None]
        den += l * w
    return num / den[:, None], M + np.log(den)


def attn_step_chunked(q, k_blk, v_blk, k_cache, v_cache, prefix_len, split_fn: Callable, scale=None):
    """attn_step computed by splitting each (b, KV head) key sequence into chunks and merging.

    ``split_fn(n_keys) -> bounds`` returns chunk boundaries 0 = c0 <= ... <= c_k = n_keys."""
    B, S, Hq, D = q.shape
    Hkv = k_blk.shape[2]
    tau = default_scale(D) if scale is None else float(np.float32(scale))
    O = np.zeros((B, S, Hq, D))
    L = np.zeros((B, Hq, S))
    for b in range(B):
        for h in range(Hq):
            K, V = keys_values(k_blk, v_blk, k_cache, v_cache, prefix_len, b, kv_head_of(h, Hq, Hkv))
            bounds = list(split_fn(K.shape[0]))
            assert bounds[0] == 0 and bounds[-1] == K.shape[0]
            o, lse = merge_partials(chunk_partials(q[b, :, h, :], K, V, tau, bounds))
            O[b, :, h, :] = o
            L[b, h, :] = lse
    return O, L


# ----------------------------------------------------------------------------------------------
# confidence unmasking
# ----------------------------------------------------------------------------------------------
def vocab_reduce(logits_row: np.ndarray):
    """For one row l (float64): m = max_j l_j, a = min{j : l_j = m}, Z = sum_j exp(l_j - m),
    p = 1 / Z (the maximum softmax probability)."""
    m = float(np.max(logits_row))
    a = int(np.flatnonzero(logits_row == m)[0])
    Z = float(np.sum(np.exp(logits_row - m)))
    return m, a, Z, 1.0 / Z


def confidences(logits: np.ndarray, mask: np.ndarray, decode: Optional[Callable] = None):
    """p and argmax for every masked row (unmasked rows: p = 0, argmax = -1).

    ``logits`` is [rows, V] float32 or bf16 bits (uint16, with ``decode=bf16_to_f64``);
    rows are decoded one at a time to keep memory bounded."""
    rows = logits.shape[0]
    p = np.zeros(rows)
    a = np.full(rows, -1, dtype=np.int64)
    for r in range(rows):
        if mask[r]:
            row = decode(logits[r]) if decode is not None else np.asarray(logits[r], np.float64)
            _, a[r], _, p[r] = vocab_reduce(row)
    return p, a


def commit(p: np.ndarray, a: np.ndarray, mask: np.ndarray, tokens: np.ndarray, S: int,
           gamma: float, min_commit: bool = True, commit_all: bool = False):
    """Commit rule per sequence b (positions b*S .. b*S+S-1), in this order:
    1. commit_all: C = every masked position;
    2. else C = {s masked : p_s > gamma64}, gamma64 = float64(float32(gamma));
    3. if C is empty, min_commit is set and some position is masked: C = {the masked s with
       the largest p_s, ties -> lowest s}.
    For s in C: tokens[s] = a_s, mask[s] = 0. Returns (mask, tokens, n_commit[B]) as new arrays."""
    g64 = float(np.float32(gamma))
    mask = np.array(mask, dtype=np.uint8, copy=True)
    tokens = np.array(tokens, dtype=np.int32, copy=True)
    B = mask.shape[0] // S
    n_commit = np.zeros(B, dtype=np.int32)
    for b in range(B):
        idx = [b * S + s for s in range(S) if mask[b * S + s]]
        if commit_all:
            C = list(idx)
        else:
            C = [r for r in idx if p[r] > g64]
            if not C and min_commit and idx:
                best = idx[0]
                for r in idx[1:]:
                    if p[r] > p[best]:
                        best = r
                C = [best]
        for r in C:
            tokens[r] = a[r]
            mask[r] = 0
        n_commit[b] = len(C)
    return mask, tokens, n_commit


def confidence_unmask(logits, mask, tokens, S, gamma, min_commit=True, commit_all=False, decode=None):
    """Vocabulary reduction of every masked row, then the commit rule.
    Returns dict(mask, tokens, n_commit, conf, argmax)."""
    p, a = confidences(logits, mask, decode)
    m2, t2, n = commit(p, a, mask, tokens, S, gamma, min_commit, commit_all)
    return {"mask": m2, "tokens": t2, "n_commit": n, "conf": p, "argmax": a}


def margins(p: np.ndarray, mask: np.ndarray, S: int, gamma: float, min_commit=True, commit_all=False):
    """Decision margins of the commit rule, to flag outcomes that float32 rounding could flip.

    Returns a list of (kind, position or sequence, relative margin): 'gamma' for every masked row
    (|p - gamma64| / gamma64) and 'fallback' for every sequence where the fallback fires (relative
    gap between its two largest p; inf with a single masked position). Decisions with margin
    < NEAR_TIE_REL are near-ties. Exactly equal p (bit-identical rows) are not near-ties: the
    rule breaks them by position, deterministically on both sides."""
    g64 = float(np.float32(gamma))
    out = []
    if commit_all:
        return out
    B = mask.shape[0] // S
    for b in range(B):
        idx = [b * S + s for s in range(S) if mask[b * S + s]]
        for r in idx:
            out.append(("gamma", r, abs(p[r] - g64) / g64 if g64 > 0 else math.inf))
        if min_commit and idx and not any(p[r] > g64 for r in idx):
            ps = sorted((p[r] for r in idx), reverse=True)
            if len(ps) < 2 or ps[0] == ps[1]:
                gap = math.inf
            else:
                gap = (ps[0] - ps[1]) / ps[0]
            out.append(("fallback", b, gap))
    return out


def near_ties(p, mask, S, gamma, min_commit=True, commit_all=False, rel=NEAR_TIE_REL):
    return [m for m in margins(p, mask, S, gamma, min_commit, commit_all) if m[2] < rel]


# ----------------------------------------------------------------------------------------------
# the T-step block loop
# ----------------------------------------------------------------------------------------------
# ----------------------------------------------------------------------------------------------
# context-tower update after a commit, and self-speculation
# ----------------------------------------------------------------------------------------------
def kv_append(k_cache, v_cache, prefix_len, k_new, v_new, active: Optional[Sequence[int]] = None):
    """Append the committed block: for every active sequence b and KV head g, rows
    prefix_len[b] .. prefix_len[b]+S-1 of the cache become k_new[b, :, g, :] / v_new[b, :, g, :],
    then prefix_len[b] += S. Returns new (k_cache, v_cache, prefix_len); inputs are not modified
    (any dtype: the rows are copied bit for bit)."""
    kc, vc, ln = np.array(k_cache, copy=True), np.array(v_cache, copy=True), np.array(prefix_len, copy=True)
    B, S, Hkv, D = k_new.shape
    for b in range(B):
        if active is not None and not active[b]:
            continue
        n = int(ln[b])
        if n + S > kc.shape[2]:
            raise ValueError("append past the cache capacity")
        for g in range(Hkv):
            kc[b, g, n:n + S, :] = k_new[b, :, g, :]
            vc[b, g, n:n + S, :] = v_new[b, :, g, :]
        ln[b] = n + S
    return kc, vc, ln


def spec_accept(draft, first_choice, pass_argmax, S: int):
    """Self-speculation check of drafted blocks against the causal pass over them.

    draft [B*S] drafted tokens; first_choice [B] AR's choice for block position 0 (carried from
    the pass before); pass_argmax [B*S] argmax of the causal pass at each block position (the
    choice for the next position). AR's choice for position i: first_choice[b] for i = 0, else
    pass_argmax[b*S + i - 1]. Returns dict(tokens [B*S] (committed positions filled, others
    -1), n_commit [B], next_choice [B]: AR's choice for the position after the committed run when
    the pass has seen every committed token (the whole draft accepted), else -1)."""
    draft = np.asarray(draft, dtype=np.int64)
    pa = np.asarray(pass_argmax, dtype=np.int64)
    B = draft.size // S
    tokens = np.full(B * S, -1, dtype=np.int32)
    n_commit = np.zeros(B, dtype=np.int32)
    next_choice = np.full(B, -1, dtype=np.int32)
    for b in range(B):
        k = 0
        while k < S:
            ar = int(first_choice[b]) if k == 0 else int(pa[b * S + k - 1])
            if int(draft[b * S + k]) != ar:
                break
            tokens[b * S + k] = draft[b * S + k]
            k += 1
        if k < S:
            tokens[b * S + k] = int(first_choice[b]) if k == 0 else int(pa[b * S + k - 1])
            n_commit[b] = k + 1
        else:
            n_commit[b] = S
            next_choice[b] = int(pa[b * S + S - 1])
    return {"tokens": tokens, "n_commit": n_commit, "next_choice": next_choice}


# ----------------------------------------------------------------------------------------------
# adaptive loop halting
# ----------------------------------------------------------------------------------------------
def loop_halt(h_prev, h_cur, eps: float, iteration: int, max_iter: int):
    """Relative hidden-state change of every sequence between two consecutive loop iterations
    and the halting decision after 1-based iteration ``iteration``.

    h_prev, h_cur [B, ...] float64. rel[b] = ||h_cur[b] - h_prev[b]||_2 / ||h_prev[b]||_2 (both
    zero -> 0; h_prev zero, h_cur not -> inf). halt[b] = rel[b] < eps (eps promoted from float32)
    or iteration >= max_iter. Returns (rel [B] float64, halt [B] uint8)."""
    B = h_prev.shape[0]
    dp = np.asarray(h_prev, np.float64).reshape(B, -1)
    dc = np.asarray(h_cur, np.float64).reshape(B, -1)
    num = np.sqrt(((dc - dp) ** 2).sum(axis=1))
    den = np.sqrt((dp ** 2).sum(axis=1))
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = np.where(num == 0, 0.0, num / den)
    e = float(np.float32(eps))
    halt = ((rel < e) | (iteration >= max_iter)).astype(np.uint8)
    return rel, halt


def denoise_block(T: int, t0: int, B: int, S: int, mask0, tokens0, step_inputs: Callable,
                  k_cache, v_cache, prefix_len, gamma: float, min_commit: bool = True,
                  final_commit_all: bool = True, logits_decode=None, scale=None):
    """Algorithm 1's inner loop for one block of every sequence.

    For t = t0 .. T-1: a sequence is active iff it still has a masked position; if none is
    active the loop stops. Active sequences get the attention of the step (q/k/v from
    ``step_inputs(t)`` -> dict(q, k_blk, v_blk, logits), float64 q/k/v), then the confidence
    unmasking of the step's logits with commit_all at t = T-1 (when ``final_commit_all``).
    Returns dict(mask, tokens, steps_used[B], commits[T][B], and per executed step t: outs[t] (O),
    conf[t], argmax[t], active[t], masks[t] (the mask at the start of step t))."""
    mask = np.array(mask0, dtype=np.uint8, copy=True)
    tokens = np.array(tokens0, dtype=np.int32, copy=True)
    steps_used = np.zeros(B, dtype=np.int32)
    commits = np.zeros((T, B), dtype=np.int32)
    outs, confs, argmaxes, actives, masks = {}, {}, {}, {}, {}
    for t in range(t0, T):
        active = mask.reshape(B, S).any(axis=1)
        if not active.any():
            break
        masks[t] = mask.copy()
        inp = step_inputs(t)
        O, _ = attn_step(inp["q"], inp["k_blk"], inp["v_blk"], k_cache, v_cache, prefix_len,
                         scale=scale, active=active)
        outs[t] = O
        actives[t] = active.copy()
        res = confidence_unmask(inp["logits"], mask, tokens, S, gamma, min_commit,
                                commit_all=(final_commit_all and t == T - 1), decode=logits_decode)
        confs[t], argmaxes[t] = res["conf"], res["argmax"]
        mask, tokens = res["mask"], res["tokens"]
        commits[t] = res["n_commit"]
        steps_used[active] = t + 1
    return {"mask": mask, "tokens": tokens, "steps_used": steps_used, "commits": commits,
            "outs": outs, "conf": confs, "argmax": argmaxes, "active": actives, "masks": masks}


# ----------------------------------------------------------------------------------------------
# block-local bidirectional Mamba scan (BDLM Mamba-H)
# ----------------------------------------------------------------------------------------------
def _group_of(h: int, H: int, G: int) -> int:
    """Head h reads B and C of group floor(h * G / H) (contiguous groups, as for GQA)."""
    return (h * G) // H


def mamba_block_scan(h0, fwd, rev, A, A_r, D_skip):
    """One Mamba-H mixer pass over the active block of every sequence, float64.

    h0 [B, H, N, P]: the cached forward boundary state (the forward scan's state after the clean
    prefix). fwd and rev: the block's per-position inputs of the forward and of the reverse
    direction, dicts with x [B, S, H, P], dt [B, S, H] (step sizes > 0), Bm and Cm [B, S, G, N].
    A, A_r [H]: decay rates (< 0); D_skip [H].

    Forward, state F_{-1} = h0:   F_s = exp(dt_s A) F_{s-1} + dt_s Bm_s x_s^T,   yf_s = Cm_s^T F_s
    Reverse, state R_S = 0:       R_s = exp(dtr_s A_r) R_{s+1} + dtr_s Bmr_s xr_s^T,  yr_s = Cmr_s^T R_s
    (s = S-1 down to 0: the reverse scan sees the block's positions only)
    y_s = yf_s + yr_s + D_skip x_s.
    Returns y [B, S, H, P] and h_out [B, H, N, P] = F_{S-1}, the forward state after the block
    (the cache entry once the block is committed)."""
    B, S, H, P = fwd["x"].shape
    G = fwd["Bm"].shape[2]
    y = np.zeros((B, S, H, P))
    h_out = np.zeros(np.shape(h0))
    for b in range(B):
        for h in range(H):
            g = _group_of(h, H, G)
            F = np.array(h0[b, h], dtype=np.float64)
            for s in range(S):
                F = np.exp(fwd["dt"][b, s, h] * A[h]) * F + fwd["dt"][b, s, h] * np.outer(fwd["Bm"][b, s, g],
                                                                                          fwd["x"][b, s, h])
                y[b, s, h] += fwd["Cm"][b, s, g] @ F
            h_out[b, h] = F
            R = np.zeros_like(F)
            for s in range(S - 1, -1, -1):
                R = np.exp(rev["dt"][b, s, h] * A_r[h]) * R + rev["dt"][b, s, h] * np.outer(rev["Bm"][b, s, g],
                                                                                             rev["x"][b, s, h])
                y[b, s, h] += rev["Cm"][b, s, g] @ R
            y[b, :, h] += D_skip[h] * fwd["x"][b, :, h]
    return y, h_out


def mamba_sequence(fwd, rev, A, A_r, D_skip, S: int, h_init=None):
    """A whole sequence of blocks of S positions the way BDLM Mamba-H runs it: one forward scan
    over every position from h_init (zero by default), and a reverse scan restarted from zero in
    every block. fwd / rev hold x [B, L, H, P], dt [B, L, H], Bm / Cm [B, L, G, N] with L a
    multiple of S. Returns (y [B, L, H, P], the forward boundary states after every block
    [B, L/S, H, N, P])."""
    B, L, H, P = fwd["x"].shape
    N = fwd["Bm"].shape[3]
    state = np.zeros((B, H, N, P)) if h_init is None else np.array(h_init, dtype=np.float64)
    ys, bounds = [], []
    for k in range(L // S):
        sl = slice(k * S, (k + 1) * S)
        blk_f = {n: v[:, sl] for n, v in fwd.items()}
        blk_r = {n: v[:, sl] for n, v in rev.items()}
        y, state = mamba_block_scan(state, blk_f, blk_r, A, A_r, D_skip)
        ys.append(y)
        bounds.append(state)
    return np.concatenate(ys, axis=1), np.stack(bounds, axis=1)
