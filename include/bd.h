/*
 * bd.h -- C ABI of the block-diffusion denoise step for AMD MI355X (gfx950).
 *
 * One denoise step of a block-diffusion language model: the S positions of
 * the active block attend bidirectionally to each other and to a read-only
 * cache of the clean prefix's keys and values, then a confidence-unmasking
 * pass commits the masked positions whose maximum softmax probability is
 * above gamma. A T-step loop wraps the two.
 *
 * Sources (page title, section):
 *  - Nemotron-TwoTower technical summary, §Architecture: the denoiser tower
 *    uses bidirectional attention inside the noisy block and causal
 *    cross-attention into the frozen context tower's layer-aligned KV cache.
 *  - same page, §Generation (Algorithm 1): a block starts as S masked tokens
 *    and is refined over T denoiser steps; at every layer the denoiser
 *    attends to the context tower's KV cache of past blocks and to the
 *    current block's bidirectional KV; the refined block is committed.
 *  - same page, §Training and conditioning, sampling bullet (Algorithm 2):
 *    every step predicts all masked positions in parallel and commits those
 *    whose confidence exceeds gamma; the rest stay masked.
 *  - Hybrid Block Diffusion with Partial Bidirectionality summary, technical
 *    §Method: the prefix cache is a function of the clean prefix only, so the
 *    step never writes it.
 *  - Nemotron-TwoTower technical summary, §Architecture and §Generation: the
 *    frozen context tower is a causal AR model over the committed tokens;
 *    after a block commits it takes in the new clean tokens (bd_attn_desc's
 *    causal mode, bd_kv_append).
 *  - Nemotron-Labs Diffusion page, decoding modes (self-speculation,
 *    LinearSpec): a block drafted bidirectionally is checked causally and its
 *    matching prefix commits (bd_spec_verify).
 *  - Technical summary: LoopMDM, §Adaptive inference: the looped mid-block
 *    stops once the relative hidden-state change between iterations falls
 *    below epsilon or the iteration budget is spent (bd_loop_halt).
 *  - Hybrid Block Diffusion with Partial Bidirectionality summary, technical
 *    §Method: the reverse Mamba scan stays inside the active block and the
 *    forward scan's boundary state is the prefix cache (bd_mamba_block_scan).
 *
 * Conventions (every entry point):
 *  - Pointers are DEVICE pointers unless marked (host). The caller owns every
 *    buffer; the library never allocates or frees device memory on these
 *    paths and keeps no pointer after returning.
 *  - Calls are asynchronous on `stream` (a hipStream_t passed as void*; NULL
 *    is the null stream). Results are valid once the stream is synchronised.
 *    No entry point synchronises the stream.
 *  - Arguments are validated on the host before anything is enqueued. On a
 *    non-OK status nothing has been enqueued (BD_EHIP: a launch failed) and
 *    bd_last_error() describes the cause.
 *  - Alignment: every tensor base pointer must be 16-byte aligned; row
 *    strides must be multiples of 16 bytes.
 *  - Inputs must be finite, except logits, which may hold -inf (each
 *    evaluated row must hold at least one finite value).
 *  - Calls that share a workspace, or overlapping output buffers, must not
 *    run concurrently.
 */
#ifndef BD_H
#define BD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  BD_OK = 0,
  BD_EINVAL = 1,        /* invalid argument (null pointer, shape, range, alignment) */
  BD_EUNSUPPORTED = 2,  /* valid but not supported by the library (e.g. head_dim 96) */
  BD_EWORKSPACE = 3,    /* workspace smaller than the *_workspace_bytes query */
  BD_EHIP = 4           /* a HIP runtime call or kernel launch failed */
} bd_status;

typedef enum { BD_BF16 = 0, BD_F32 = 1 } bd_dtype;

/* ------------------------------------------------------------------------------------------
 * Attention of the active block over [prefix ; block]
 *
 * For sequence b, block position s and query head h (GQA: KV head
 * g = floor(h * Hkv / Hq), contiguous groups), with keys/values
 *   K_b,g = [ k_cache[b, g, 0 .. prefix_len[b]-1, :] ; k_blk[b, 0 .. S-1, g, :] ]
 * (likewise V) and tau = softmax_scale:
 *   out[b, s, h, :] = softmax_j(tau * q[b,s,h,:] . K_b,g[j,:]) V_b,g
 *   lse[b, h, s]    = ln sum_j exp(tau * q[b,s,h,:] . K_b,g[j,:])
 * One softmax runs over every prefix key and every block key; there is no
 * mask inside the block (every block position sees every other) and every
 * prefix key is visible to every block query. Positions are not applied here
 * (rotary embeddings, if any, are already in q and k).
 *
 * Causal mode (desc.causal = 1): the context tower's pass over a committed
 * block, or the causal check of a drafted block -- block key j is visible to
 * block position s only when j <= s (prefix keys stay visible to all).
 * ---------------------------------------------------------------------------------------- */
typedef struct {
  int32_t batch;            /* B >= 1 */
  int32_t n_q_heads;        /* Hq >= 1, Hq % Hkv == 0 */
  int32_t n_kv_heads;       /* Hkv >= 1 */
  int32_t head_dim;         /* D: 64 or 128 */
  int32_t block_len;        /* S: 1 .. 64 */
  int64_t prefix_capacity;  /* Lcap >= 1: token stride of k_cache / v_cache; Lcap * D * 2 bytes < 2 GiB
                               (one (sequence, KV head) slab), else BD_EUNSUPPORTED */
  int64_t max_prefix_len;   /* host upper bound on every prefix_len[b]; 0 .. Lcap; used to plan the split */
  float softmax_scale;      /* tau; <= 0 selects 1/sqrt(D) computed in float32 */
  int32_t num_splits;       /* 0 = automatic; > 0 forces the number of key chunks per (b, KV head) */
  int32_t causal;           /* 0: bidirectional block (denoiser); 1: causal within the block */
} bd_attn_desc;

/* Workspace bytes bd_attn_step needs for this descriptor (0 on an invalid descriptor, or on one
 * too large for one launch: see bd_attn_step). */
size_t bd_attn_workspace_bytes(const bd_attn_desc* desc);

/* How bd_attn_step will run a descriptor (host-side query; nothing is enqueued): work-group shape,
 * row tiles and key chunks per (sequence, KV head). For diagnostics and tests. */
typedef struct {
  int32_t waves;            /* waves (of 64 lanes) per work-group */
  int32_t rows_per_wave;    /* query rows a wave owns (32-row MFMA blocks x 32) */
  int32_t row_tiles;        /* work-groups per (sequence, KV head, chunk) along the query rows */
  int32_t num_splits;       /* key chunks per (sequence, KV head) */
  int64_t chunk_keys;       /* keys per chunk (a multiple of 64) */
  int64_t workgroups;       /* work-groups of the split launch */
} bd_attn_plan_info;

/* BD_OK and *info filled (host pointer), or the descriptor's validation error. */
bd_status bd_attn_plan(const bd_attn_desc* desc, bd_attn_plan_info* info);

/* q:        bf16 [B, S, Hq, D]            (read only)
 * k_blk:    bf16 [B, S, Hkv, D]           (read only)  keys of the active block
 * v_blk:    bf16 [B, S, Hkv, D]           (read only)
 * k_cache:  bf16 [B, Hkv, Lcap, D]        (read only)  prefix keys; rows >= prefix_len[b] are never read
 * v_cache:  bf16 [B, Hkv, Lcap, D]        (read only)
 * prefix_len: int32 [B], 0 <= prefix_len[b] <= max_prefix_len (device-side precondition)
 * active:   uint8 [B] or NULL (all active). Sequences with active[b] == 0 are skipped: their rows
 *           of out and lse are left untouched.
 * out:      bf16 [B, S, Hq, D]  (written; rounded to nearest even)
 * lse:      float32 [B, Hq, S] or NULL
 * workspace: device scratch of at least bd_attn_workspace_bytes(desc) bytes.
 * Errors (all before anything is enqueued): BD_EINVAL for an invalid descriptor, NULL or misaligned
 * pointer; BD_EWORKSPACE for a workspace below the query; BD_EUNSUPPORTED for an unsupported
 * head_dim or capacity, and for a problem too large for one launch (B * Hkv * S * Hq / Hkv query
 * rows at or above 2^31, or a split launch beyond 2^32 - 1 work-items, e.g. with a large forced
 * num_splits). The output is a convex combination of per-chunk outputs kept in bf16, so it carries
 * up to twice the rounding of one bf16 result. */
bd_status bd_attn_step(const bd_attn_desc* desc,
                       const void* q, const void* k_blk, const void* v_blk,
                       const void* k_cache, const void* v_cache,
                       const int32_t* prefix_len, const uint8_t* active,
                       void* out, float* lse,
                       void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------------------------
 * Context-tower update after a commit: append the committed block to the prefix cache
 *
 * For every active sequence b and KV head g:
 *   k_cache[b, g, prefix_len[b] + s, :] = k_new[b, s, g, :]   (s = 0 .. S-1; likewise v)
 * then prefix_len[b] += S. The rows are copied bit for bit; nothing else in the caches is
 * written. k_new / v_new are the committed block's keys and values from the context tower's
 * causal pass (bd_attn_step with desc.causal = 1 over the same block).
 * desc: the attention descriptor (batch, n_kv_heads, head_dim, block_len = S, prefix_capacity,
 *       max_prefix_len); max_prefix_len + S must not exceed prefix_capacity (BD_EINVAL otherwise),
 *       and prefix_len[b] <= max_prefix_len is the device-side precondition as for bd_attn_step.
 *       Afterwards max_prefix_len + S bounds the new lengths. A sequence that breaks the device
 *       precondition so far that prefix_len[b] + S would pass prefix_capacity (or whose length is
 *       negative) is left untouched: no row written, prefix_len[b] not advanced (the caller sees it
 *       in prefix_len).
 * k_new, v_new: bf16 [B, S, Hkv, D] (read only); k_cache, v_cache: bf16 [B, Hkv, Lcap, D] (rows
 *       prefix_len[b] .. prefix_len[b]+S-1 written); prefix_len: int32 [B] (read, then advanced);
 * active: uint8 [B] or NULL (all). Inactive sequences are untouched. No workspace. */
bd_status bd_kv_append(const bd_attn_desc* desc, const void* k_new, const void* v_new,
                       void* k_cache, void* v_cache, int32_t* prefix_len, const uint8_t* active,
                       void* stream);

/* ------------------------------------------------------------------------------------------
 * Confidence unmasking
 *
 * For every masked row r (mask[r] == 1) of the logits:
 *   m_r = max_j l_rj,  a_r = min{ j : l_rj = m_r } (lowest index wins ties),
 *   p_r = 1 / sum_j exp(l_rj - m_r)   (the maximum softmax probability).
 * Rows with mask[r] == 0 are not read. Then, per sequence b (rows b*S .. b*S+S-1):
 *   C = every masked position                        if commit_all,
 *   C = { masked s : p_s > gamma }  (strict, float32)  otherwise;
 *   if C is empty, min_commit is set and a position is masked, C = { the masked position with
 *   the largest p, lowest position on ties };
 *   for s in C: tokens[s] = a_s, mask[s] = 0.  Commits are final.
 * ---------------------------------------------------------------------------------------- */
typedef struct {
  int32_t batch;         /* B >= 1 */
  int32_t block_len;     /* S: 1 .. 64 */
  int32_t vocab;         /* V >= 1 */
  int64_t row_stride;    /* elements between consecutive logit rows, >= V */
  bd_dtype logits_dtype; /* BD_BF16 or BD_F32 */
  float gamma;           /* threshold in [0, 1]; commit iff p > gamma */
  int32_t min_commit;    /* 1: commit the most confident masked position when none passes */
  int32_t commit_all;    /* 1: commit every masked position (last step of a block) */
} bd_unmask_desc;

size_t bd_unmask_workspace_bytes(const bd_unmask_desc* desc);

/* logits:   [B*S, row_stride] of logits_dtype (read only)
 * mask:     uint8 [B*S], 1 = masked (read, then updated in place)
 * tokens:   int32 [B*S] (committed positions are written)
 * conf:     float32 [B*S] or NULL: p_r of masked rows, 0 for rows that were not masked
 * argmax:   int32 [B*S] or NULL: a_r of masked rows, -1 for rows that were not masked
 * n_commit: int32 [B] or NULL: |C| per sequence */
bd_status bd_confidence_unmask(const bd_unmask_desc* desc, const void* logits,
                               uint8_t* mask, int32_t* tokens,
                               float* conf, int32_t* argmax, int32_t* n_commit,
                               void* workspace, size_t workspace_bytes, void* stream);

/* The same operation with no workspace and no allocation of any kind, for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops, harnesses that forbid
 * hipMalloc). The slice partials live in a static scratch array inside the library: 4 MiB per
 * device, held until the process ends, which bounds the problem to B*S <= 349525 rows (larger
 * descriptors return BD_EUNSUPPORTED before anything is enqueued). The first call on a device
 * resolves that array's address (hipGetSymbolAddress); make it once outside any capture. Calls
 * that overlap on one device share the array and race: serialise them (one stream, or events).
 * Arguments and results otherwise exactly as bd_confidence_unmask. */
bd_status bd_confidence_unmask_noalloc(const bd_unmask_desc* desc, const void* logits,
                                       uint8_t* mask, int32_t* tokens,
                                       float* conf, int32_t* argmax, int32_t* n_commit, void* stream);

/* ------------------------------------------------------------------------------------------
 * Self-speculation check (LinearSpec): commit the prefix of a drafted block that AR decoding
 * would produce
 *
 * logits are the causal pass over the drafted block (bd_attn_step with desc.causal = 1, then
 * the model's head): row b*S + i predicts block position i + 1. For every row,
 * c_r = min{ j : l_rj = max_j l_rj } (lowest index on ties). AR's choice for block position i of
 * sequence b is first_choice[b] for i = 0 (carried from the pass before) and c_{b*S+i-1} for
 * i >= 1. With k = the length of the longest prefix of draft[b*S ..] equal to AR's choices:
 *   tokens[b*S + i] = draft[b*S + i] for i < k; tokens[b*S + k] = AR's choice at k if k < S;
 *   every other position of the block gets -1;
 *   n_commit[b] = min(k + 1, S)  (>= 1: AR's own choice at the first mismatch commits, so the
 *                                 output is exactly AR decoding's at temperature 0);
 *   next_choice[b] = c_{b*S+S-1} if k == S (AR's choice after the block), else -1 (the pass has
 *                    not seen the corrected token; the next pass provides it).
 * desc: batch, block_len (S), vocab, row_stride, logits_dtype (gamma, min_commit, commit_all are
 *       not used). draft, first_choice: int32 [B*S], [B] (read only); tokens: int32 [B*S],
 *       n_commit, next_choice: int32 [B] (written). workspace: >= bd_unmask_workspace_bytes(desc).
 * Every row of the logits is read once (HBM-bound like the confidence pass). */
bd_status bd_spec_verify(const bd_unmask_desc* desc, const void* logits, const int32_t* draft,
                         const int32_t* first_choice, int32_t* tokens, int32_t* n_commit,
                         int32_t* next_choice, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------------------------
 * Adaptive loop halting (LoopMDM)
 *
 * For every sequence b, with h_prev / h_cur its hidden state after loop iterations k-1 and k
 * (n_per_seq values each, all positions and hidden units):
 *   rel[b]  = ||h_cur[b] - h_prev[b]||_2 / ||h_prev[b]||_2   (0 when both norms are 0; +inf when
 *             only h_prev's is), sums of squares in float32, in a fixed order;
 *   halt[b] = rel[b] < eps (strict) or iteration >= max_iter  (iteration is 1-based: k).
 * ---------------------------------------------------------------------------------------- */
typedef struct {
  int32_t batch;            /* B >= 1 */
  int64_t n_per_seq;        /* values per sequence (positions x hidden units), >= 1 */
  bd_dtype dtype;           /* BD_BF16 or BD_F32 */
  float eps;                /* >= 0, finite */
  int32_t max_iter;         /* >= 1 */
} bd_halt_desc;

/* Workspace bytes bd_loop_halt needs (0 on an invalid descriptor). */
size_t bd_loop_halt_workspace_bytes(const bd_halt_desc* desc);

/* h_prev, h_cur: [B, n_per_seq] in desc.dtype (read only, rows contiguous, 16-byte aligned);
 * iteration: k >= 1; rel: float32 [B] or NULL; halt: uint8 [B] (written). */
bd_status bd_loop_halt(const bd_halt_desc* desc, const void* h_prev, const void* h_cur, int32_t iteration,
                       float* rel, uint8_t* halt, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------------------------
 * Block-local bidirectional Mamba scan (BDLM Mamba-H)
 *
 * Hybrid Block Diffusion with Partial Bidirectionality summary, technical §Method: completed
 * prefix blocks keep only the forward scan's boundary (recurrent) state, and the reverse scan is
 * confined to the active block, so the cached prefix state is a function of the clean prefix
 * alone. The pages print no recurrence; this is the Mamba-2 selective scan. For sequence b, head
 * h (B and C of group g = floor(h G / H)) and block position s (0 .. S-1):
 *   forward, F_{-1} = h0[b,h]:  F_s = exp(dt_s A_h) F_{s-1} + dt_s B_s x_s^T   (N x P state)
 *   reverse, R_S = 0:           R_s = exp(dtr_s Ar_h) R_{s+1} + dtr_s Br_s xr_s^T (s = S-1 .. 0)
 *   y[b,s,h,:] = C_s^T F_s + Cr_s^T R_s + D_h x_s,     h_out[b,h] = F_{S-1}
 * (B_s, C_s, x_s, dt_s of the forward inputs; Br, Cr, xr, dtr of the reverse inputs). h_out is the
 * boundary state the block leaves, the cache entry once the block is committed. Computed in
 * float32 (float32 MFMA) from the closed form of the two recurrences.
 * ---------------------------------------------------------------------------------------- */
typedef struct {
  int32_t batch;        /* B >= 1 */
  int32_t n_heads;      /* H >= 1, H % G == 0 */
  int32_t n_groups;     /* G >= 1 */
  int32_t head_dim;     /* P: 64 */
  int32_t state_dim;    /* N: 64 or 128 */
  int32_t block_len;    /* S: 1 .. 32 */
} bd_mamba_desc;

typedef struct {        /* one direction's inputs for the block (device pointers, read only) */
  const void* x;        /* bf16 [B, S, H, P] */
  const float* dt;      /* float32 [B, S, H], step sizes (> 0) */
  const void* Bm;       /* bf16 [B, S, G, N] */
  const void* Cm;       /* bf16 [B, S, G, N] */
  const float* A;       /* float32 [H], decay rates (< 0) */
} bd_mamba_dir;

/* h0: float32 [B, H, N, P]; fwd, rev: host structs of device pointers; D: float32 [H]; active:
 * uint8 [B] or NULL (inactive sequences are skipped: their y and h_out untouched); y: bf16
 * [B, S, H, P] (written); h_out: float32 [B, H, N, P] or NULL (written). h_out may be h0 itself
 * (the cache entry advanced in place: every state element is read before it is written, by the
 * thread that writes it); otherwise h0 is not written and the buffers must not overlap. Every
 * pointer 16-byte aligned. No workspace, no allocation. BD_EINVAL: NULL descriptor or pointer,
 * misalignment, a count < 1, H not a multiple of G, S outside 1 .. 32; BD_EUNSUPPORTED: P != 64,
 * N not 64 or 128, B * H above 2^31 - 1; launch errors as BD_EHIP. */
bd_status bd_mamba_block_scan(const bd_mamba_desc* desc, const float* h0, const bd_mamba_dir* fwd,
                              const bd_mamba_dir* rev, const float* D, const uint8_t* active,
                              void* y, float* h_out, void* stream);

/* ------------------------------------------------------------------------------------------
 * The T-step block loop (Algorithm 1's inner loop)
 *
 * For t = t0 .. T-1: sequences with a masked position are active; the model hooks provide the
 * step's q / k_blk / v_blk, bd_attn_step runs for the active sequences into `out`, the hooks
 * turn `out` into logits, and bd_confidence_unmask runs with commit_all = (t == T-1). Sequences
 * without a masked position skip all work on the device; there is no host synchronisation
 * inside the loop (every step is enqueued, inactive work exits at once).
 * ---------------------------------------------------------------------------------------- */
typedef struct {
  /* Return device pointers (valid until the next hook call) to the step's q [B,S,Hq,D],
   * k_blk and v_blk [B,S,Hkv,D] (bf16). May enqueue work on `stream`. Non-OK aborts the loop. */
  bd_status (*get_qkv)(void* user, int32_t step, const uint8_t* mask, const int32_t* tokens,
                       const void** q, const void** k_blk, const void** v_blk, void* stream);
  /* Return a device pointer to the step's logits [B*S, row_stride] computed from attn_out. */
  bd_status (*get_logits)(void* user, int32_t step, const void* attn_out, const void** logits,
                          void* stream);
  void* user;
} bd_step_hooks;

/* Hooks that replay precomputed per-step device pointers (no host callback into the caller).
 * step t uses q[t], k_blk[t], v_blk[t] and logits[t]; the table (host arrays of n_steps device
 * pointers each) must stay alive while the loop is being enqueued. A step outside
 * [0, n_steps) makes the hook return BD_EINVAL. */
typedef struct {
  const void* const* q;
  const void* const* k_blk;
  const void* const* v_blk;
  const void* const* logits;
  int32_t n_steps;
} bd_step_table;

bd_status bd_table_hooks(const bd_step_table* table, bd_step_hooks* hooks_out);

size_t bd_denoise_workspace_bytes(const bd_attn_desc* attn, const bd_unmask_desc* unmask);

/* attn / unmask: descriptors as above (unmask->commit_all is ignored; the loop sets it).
 * T >= 1 steps, 0 <= t0 < T (resume from step t0 with the caller's mask and tokens).
 * out:        bf16 [B,S,Hq,D], rewritten every step for the active sequences.
 * mask/tokens: as in bd_confidence_unmask, updated step by step.
 * steps_used: int32 [B] (required): t+1 of the last step at which b was active, 0 if never.
 * commits_per_step: int32 [T, B] or NULL: rows t0 .. T-1 receive n_commit of each step.
 * The call only enqueues kernels on `stream` (no allocation, memset or host synchronisation while
 * no trace is attached), so with hooks that do not synchronise either (bd_table_hooks) the whole
 * loop can be captured into a HIP graph and replayed. */
bd_status bd_denoise_block(const bd_attn_desc* attn, const bd_unmask_desc* unmask,
                           int32_t T, int32_t t0, const bd_step_hooks* hooks,
                           const void* k_cache, const void* v_cache, const int32_t* prefix_len,
                           void* out, uint8_t* mask, int32_t* tokens,
                           int32_t* steps_used, int32_t* commits_per_step,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Thread-local message describing this thread's last non-OK status ("" if none). */
const char* bd_last_error(void);

/* ------------------------------------------------------------------------------------------
 * Kernel tracing (observability; off unless a trace is attached)
 *
 * While a trace is attached to the calling thread, every kernel the library enqueues from that
 * thread carries two HIP events that its dispatch stamps at kernel start and end
 * (hipExtLaunchKernelGGL), and the launch first waits for its stream to drain, so that a recorded
 * duration is the kernel's own and not the queueing behind its predecessor (tracing serializes
 * the host with the stream; do not attach a trace while capturing a graph). bd_trace_get waits
 * for the events of record i and returns the kernel name and its duration.
 * ---------------------------------------------------------------------------------------- */
typedef struct bd_trace bd_trace;

bd_status bd_trace_create(int32_t capacity, bd_trace** out);   /* capacity: records kept */
void bd_trace_destroy(bd_trace* trace);
bd_status bd_trace_attach(bd_trace* trace);                     /* NULL detaches */
bd_status bd_trace_clear(bd_trace* trace);
int32_t bd_trace_count(const bd_trace* trace);                  /* records taken (<= capacity) */
bd_status bd_trace_get(const bd_trace* trace, int32_t i, const char** kernel, float* ms);

/* Library version string, e.g. "bd 0.1.0 gfx950". */
const char* bd_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BD_H */
