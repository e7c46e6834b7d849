// Host side of the block-diffusion denoise-step library: argument validation, split planning,
// workspace layout, kernel launches, the T-step loop and kernel tracing. The public ABI and the
// definitions of the three operations are in include/bd.h.
#include "bd.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "bd_internal.h"

struct bd_trace {
  struct Rec {
    const char* name;
    hipEvent_t start, stop;
  };
  std::vector<Rec> recs;
  int32_t count = 0;
};

namespace {

thread_local std::string g_error;
thread_local bd_trace* g_trace = nullptr;

bd_status fail(bd_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_error = buf;
  return st;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// A C caller may store any int in a bd_dtype field; reading an out-of-range value through the C++
// enum type is undefined, so validation reads the field's bytes as the int the ABI passes.
static_assert(sizeof(bd_dtype) == sizeof(int32_t), "bd_dtype is passed as a 32-bit int");
int32_t dtype_value(const bd_dtype& f) {
  int32_t v;
  std::memcpy(&v, &f, sizeof(v));
  return v;
}

constexpr int kCUs = 256;                  // MI355X compute units
constexpr size_t kLdsPerCU = 160 * 1024;   // bytes of LDS per compute unit
constexpr int64_t kMinChunk = 256;         // keys per split below which splitting does not pay

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Launch wrapper: when a trace is attached, the kernel's dispatch stamps the record's events.
template <typename F>
bd_status traced(const char* name, hipStream_t stream, F&& launch) {
  bd_trace* tr = g_trace;
  bd::Launch l{stream};
  if (tr && tr->count < (int32_t)tr->recs.size()) {
    bd_trace::Rec* rec = &tr->recs[tr->count++];
    rec->name = name;
    l.start = rec->start;
    l.stop = rec->stop;
    // let the stream drain first: the start stamp is taken when the dispatch is processed, which
    // would otherwise include the wait for the previous kernel
    if (hipStreamSynchronize(stream) != hipSuccess) return fail(BD_EHIP, "hipStreamSynchronize failed");
  }
  hipError_t e = launch(l);
  if (e != hipSuccess) return fail(BD_EHIP, "launch of %s failed: %s", name, hipGetErrorString(e));
  return BD_OK;
}

// ------------------------------------------------------------------------------------------
// attention
// ------------------------------------------------------------------------------------------
bd_status check_attn_desc(const bd_attn_desc* d) {
  if (!d) return fail(BD_EINVAL, "attention descriptor is NULL");
  if (d->batch < 1) return fail(BD_EINVAL, "batch must be >= 1 (got %d)", d->batch);
  if (d->n_kv_heads < 1 || d->n_q_heads < 1) return fail(BD_EINVAL, "head counts must be >= 1");
  if (d->n_q_heads % d->n_kv_heads != 0)
    return fail(BD_EINVAL, "n_q_heads (%d) must be a multiple of n_kv_heads (%d)", d->n_q_heads, d->n_kv_heads);
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(BD_EUNSUPPORTED, "head_dim %d is not supported (64 or 128)", d->head_dim);
  if (d->block_len < 1 || d->block_len > 64) return fail(BD_EINVAL, "block_len must be in [1, 64] (got %d)", d->block_len);
  if (d->prefix_capacity < 1) return fail(BD_EINVAL, "prefix_capacity must be >= 1");
  // the kernels address one (sequence, KV head) slab of the cache with 32-bit buffer offsets
  if (d->prefix_capacity > (int64_t)0x7fffffff / (2 * d->head_dim))
    return fail(BD_EUNSUPPORTED, "prefix_capacity %lld too large: a (sequence, KV head) slab of the cache must stay "
                "below 2 GiB", (long long)d->prefix_capacity);
  if (d->max_prefix_len < 0 || d->max_prefix_len > d->prefix_capacity)
    return fail(BD_EINVAL, "max_prefix_len must be in [0, prefix_capacity]");
  if (!std::isfinite(d->softmax_scale)) return fail(BD_EINVAL, "softmax_scale must be finite");
  if (d->num_splits < 0) return fail(BD_EINVAL, "num_splits must be >= 0");
  if (d->causal != 0 && d->causal != 1) return fail(BD_EINVAL, "causal must be 0 or 1");
  const int64_t rows = (int64_t)d->block_len * (d->n_q_heads / d->n_kv_heads);
  if (rows > (1 << 20)) return fail(BD_EUNSUPPORTED, "too many query rows per KV head");
  return BD_OK;
}

// Plans the attention launches for a validated descriptor. Fails when they would not fit their
// grids (HIP: at most 2^32 - 1 work-items in x) or the merge's 32-bit row indices.
bd_status plan_attn(const bd_attn_desc* d, bd::AttnPlan* p) {
  const int group = d->n_q_heads / d->n_kv_heads;
  p->head_dim = d->head_dim;
  p->rows = d->block_len * group;
  // 32 query rows per wave, two waves per SIMD; eight waves (one workgroup per CU) share each LDS
  // key tile when the group has more than 128 rows and such workgroups, over chunks of at least
  // kMinChunk keys, can fill the chip; otherwise four (two workgroups per CU, twice as many row
  // tiles: short prefixes of few sequences, e.g. single-sequence decode).
  p->rows_per_wave = 32;
  {
    const int64_t nk = d->max_prefix_len + d->block_len;
    const int64_t wide_items = (int64_t)d->batch * d->n_kv_heads * ((p->rows + 255) / 256) * (nk / kMinChunk);
    p->waves = p->rows > 128 && wide_items >= kCUs ? 8 : 4;
  }
  p->key_tile = bd::kAttnKeyTile;
  const int tile_rows = p->waves * p->rows_per_wave;
  p->row_tiles = (p->rows + tile_rows - 1) / tile_rows;
  const int64_t nkeys = d->max_prefix_len + d->block_len;
  const int64_t base = (int64_t)d->batch * d->n_kv_heads * p->row_tiles;
  int64_t nsplit;
  if (d->num_splits > 0) {
    nsplit = d->num_splits;
  } else {
    // fill every workgroup slot of the chip once, without chunks shorter than kMinChunk keys
    const int row_blocks = p->waves * p->rows_per_wave / 32;
    const size_t lds = (size_t)bd::attn_stages(d->head_dim, row_blocks) * bd::attn_stage_bytes(d->head_dim);
    const int by_regs = 8 / row_blocks;   // 512 registers per SIMD lane: 2 waves of 32 rows or 1 of 64
    const int by_lds = (int)(kLdsPerCU / lds);
    const int64_t slots = (int64_t)kCUs * (by_regs < by_lds ? by_regs : by_lds);
    nsplit = (slots + base - 1) / base;
    const int64_t cap = nkeys / kMinChunk;   // chunks of at least kMinChunk keys
    if (nsplit > cap) nsplit = cap;
    if (nsplit < 1) nsplit = 1;
  }
  int64_t chunk = (nkeys + nsplit - 1) / nsplit;
  chunk = (chunk + 63) / 64 * 64;
  p->chunk = chunk;
  p->nsplit = (int)((nkeys + chunk - 1) / chunk);
  p->n_items = base * p->nsplit;
  p->direct = p->nsplit == 1;
  p->wide_merge = p->nsplit > 16;
  if (p->direct) {
    p->part_o_off = p->part_ml_off = p->plan_off = p->bytes = 0;
  } else {
    const size_t prow = (size_t)p->n_items * tile_rows;
    p->part_o_off = 0;
    p->part_ml_off = align_up(prow * d->head_dim * sizeof(uint16_t), 256);
    p->plan_off = align_up(p->part_ml_off + prow * 2 * sizeof(float), 256);
    p->bytes = align_up(p->plan_off + ((size_t)d->batch + 1) * sizeof(int32_t), 256);
  }
  const int64_t merge_rows = (int64_t)d->batch * d->n_kv_heads * p->rows;
  if (merge_rows > 0x7fffffff || p->n_items * p->waves * 64 > (int64_t)0xffffffff)
    return fail(BD_EUNSUPPORTED, "problem too large for one launch: %lld query rows, %lld workgroups",
                (long long)merge_rows, (long long)p->n_items);
  return BD_OK;
}

bd_status check_attn_ptrs(const bd_attn_desc* d, const void* q, const void* kb, const void* vb, const void* kc,
                          const void* vc, const int32_t* len, const void* out, const float* lse) {
  struct {
    const void* p;
    const char* n;
  } req[] = {{q, "q"}, {kb, "k_blk"}, {vb, "v_blk"}, {kc, "k_cache"}, {vc, "v_cache"}, {len, "prefix_len"}, {out, "out"}};
  for (auto& r : req) {
    if (!r.p) return fail(BD_EINVAL, "%s is NULL", r.n);
    const size_t al = (r.p == len) ? 4 : 16;
    if (!aligned(r.p, al)) return fail(BD_EINVAL, "%s is not %zu-byte aligned", r.n, al);
  }
  if (lse && !aligned(lse, 4)) return fail(BD_EINVAL, "lse is not 4-byte aligned");
  (void)d;
  return BD_OK;
}

bd_status run_attn(const bd_attn_desc* d, const bd::AttnPlan& plan, const void* q, const void* k_blk,
                   const void* v_blk, const void* k_cache, const void* v_cache, const int32_t* prefix_len,
                   const uint8_t* active, void* out, float* lse, void* ws, hipStream_t stream) {
  bd::AttnArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k_blk = static_cast<const uint16_t*>(k_blk);
  a.v_blk = static_cast<const uint16_t*>(v_blk);
  a.k_cache = static_cast<const uint16_t*>(k_cache);
  a.v_cache = static_cast<const uint16_t*>(v_cache);
  a.prefix_len = prefix_len;
  a.active = active;
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  char* w = static_cast<char*>(ws);
  a.part_o = plan.direct ? nullptr : reinterpret_cast<uint16_t*>(w + plan.part_o_off);
  a.part_ml = plan.direct ? nullptr : reinterpret_cast<float*>(w + plan.part_ml_off);
  a.plan_pfx = plan.direct ? nullptr : reinterpret_cast<int*>(w + plan.plan_off);
  a.B = d->batch;
  a.S = d->block_len;
  a.Hq = d->n_q_heads;
  a.Hkv = d->n_kv_heads;
  a.group = d->n_q_heads / d->n_kv_heads;
  a.rows = plan.rows;
  a.rows_pad = plan.waves * plan.rows_per_wave;
  a.lcap = d->prefix_capacity;
  a.chunk = plan.chunk;
  a.max_keys = d->max_prefix_len + d->block_len;
  a.nsplit = plan.nsplit;
  a.row_tiles = plan.row_tiles;
  const float tau = d->softmax_scale > 0.f ? d->softmax_scale : 1.0f / std::sqrt((float)d->head_dim);
  a.scale_log2 = tau * 1.4426950408889634f;
  a.direct = plan.direct ? 1 : 0;
  a.balanced = !plan.direct && d->batch <= bd::kMaxBalancedBatch ? 1 : 0;
  a.stream_kv = (double)d->batch * d->n_kv_heads * (double)a.max_keys * d->head_dim * 4 > (double)bd::kStreamKvBytes;
  a.causal = d->causal;
  bd_status st = traced("attn_split", stream, [&](const bd::Launch& l) { return bd::launch_attn_split(plan, a, l); });
  if (st != BD_OK || plan.direct) return st;
  return traced("attn_merge", stream, [&](const bd::Launch& l) { return bd::launch_attn_merge(plan, a, l); });
}

// ------------------------------------------------------------------------------------------
// unmasking
// ------------------------------------------------------------------------------------------
bd_status check_unmask_desc(const bd_unmask_desc* d) {
  if (!d) return fail(BD_EINVAL, "unmask descriptor is NULL");
  if (d->batch < 1) return fail(BD_EINVAL, "batch must be >= 1");
  if (d->block_len < 1 || d->block_len > 64) return fail(BD_EINVAL, "block_len must be in [1, 64] (got %d)", d->block_len);
  if (d->vocab < 1) return fail(BD_EINVAL, "vocab must be >= 1");
  if (d->row_stride < d->vocab) return fail(BD_EINVAL, "row_stride must be >= vocab");
  const int32_t dt = dtype_value(d->logits_dtype);
  if (dt != BD_BF16 && dt != BD_F32) return fail(BD_EINVAL, "logits_dtype must be BD_BF16 or BD_F32");
  const int elt = dt == BD_BF16 ? 2 : 4;
  if ((d->row_stride * elt) % 16 != 0) return fail(BD_EINVAL, "row_stride * element size must be a multiple of 16 bytes");
  if (!(d->gamma >= 0.f && d->gamma <= 1.f)) return fail(BD_EINVAL, "gamma must be in [0, 1]");
  if ((d->min_commit != 0 && d->min_commit != 1) || (d->commit_all != 0 && d->commit_all != 1))
    return fail(BD_EINVAL, "min_commit and commit_all must be 0 or 1");
  return BD_OK;
}

void plan_unmask(const bd_unmask_desc* d, bd::UnmaskPlan* p) {
  const int64_t rows = (int64_t)d->batch * d->block_len;
  // ~2048 workgroups of 256 threads keep every CU streaming; slices of >= 8192 logits amortise
  // the per-slice merge.
  int64_t vs = (2048 + rows - 1) / rows;
  const int64_t cap = (d->vocab + 8191) / 8192;
  if (vs > cap) vs = cap;
  if (vs < 1) vs = 1;
  int64_t slice = ((int64_t)d->vocab + vs - 1) / vs;
  slice = (slice + 7) / 8 * 8;
  p->slice = slice;
  p->vsplit = (int)((d->vocab + slice - 1) / slice);
  p->bytes = align_up((size_t)rows * p->vsplit * 3 * sizeof(float), 256);
}

bd_status check_unmask_ptrs(const void* logits, const uint8_t* mask, const int32_t* tokens, const float* conf,
                            const int32_t* argmax, const int32_t* n_commit) {
  if (!logits) return fail(BD_EINVAL, "logits is NULL");
  if (!aligned(logits, 16)) return fail(BD_EINVAL, "logits is not 16-byte aligned");
  if (!mask) return fail(BD_EINVAL, "mask is NULL");
  if (!tokens) return fail(BD_EINVAL, "tokens is NULL");
  if (!aligned(tokens, 4) || (conf && !aligned(conf, 4)) || (argmax && !aligned(argmax, 4)) ||
      (n_commit && !aligned(n_commit, 4)))
    return fail(BD_EINVAL, "int32/float32 outputs must be 4-byte aligned");
  return BD_OK;
}

bd_status run_unmask(const bd_unmask_desc* d, const bd::UnmaskPlan& plan, const void* logits, uint8_t* mask,
                     int32_t* tokens, float* conf, int32_t* argmax, int32_t* n_commit, void* ws, int commit_all,
                     int step, int32_t* steps_used, uint8_t* active_next, hipStream_t stream) {
  bd::UnmaskArgs a{};
  a.logits = logits;
  a.is_bf16 = d->logits_dtype == BD_BF16;
  a.row_stride = d->row_stride;
  a.vocab = d->vocab;
  a.B = d->batch;
  a.S = d->block_len;
  a.mask = mask;
  a.tokens = tokens;
  a.conf = conf;
  a.argmax = argmax;
  a.n_commit = n_commit;
  a.gamma = d->gamma;
  a.min_commit = d->min_commit;
  a.commit_all = commit_all;
  a.part = static_cast<float*>(ws);
  a.compact = (int64_t)d->batch * d->block_len <= bd::kCompactRows ? 1 : 0;
  a.vsplit = plan.vsplit;
  a.slice = plan.slice;
  a.step = step;
  a.steps_used = steps_used;
  a.active_next = active_next;
  bd_status st = traced("vocab_reduce", stream, [&](const bd::Launch& l) { return bd::launch_vocab_reduce(a, l); });
  if (st != BD_OK) return st;
  return traced("commit", stream, [&](const bd::Launch& l) { return bd::launch_commit(a, l); });
}

// denoise-loop workspace: [attention partials][unmask partials][active flags]
size_t loop_bytes(const bd::AttnPlan& ap, const bd::UnmaskPlan& up, int B) {
  return ap.bytes + up.bytes + align_up((size_t)B, 256);
}

bd_status check_ws(void* ws, size_t have, size_t need) {
  if (have < need) return fail(BD_EWORKSPACE, "workspace too small: %zu bytes given, %zu needed", have, need);
  if (need && !ws) return fail(BD_EINVAL, "workspace is NULL");
  if (ws && !aligned(ws, 256)) return fail(BD_EINVAL, "workspace must be 256-byte aligned");
  return BD_OK;
}

// ------------------------------------------------------------------------------------------
// adaptive loop halting
// ------------------------------------------------------------------------------------------
bd_status check_halt_desc(const bd_halt_desc* d) {
  if (!d) return fail(BD_EINVAL, "halting descriptor is NULL");
  if (d->batch < 1) return fail(BD_EINVAL, "batch must be >= 1");
  if (d->n_per_seq < 1) return fail(BD_EINVAL, "n_per_seq must be >= 1");
  const int32_t dt = dtype_value(d->dtype);
  if (dt != BD_BF16 && dt != BD_F32) return fail(BD_EINVAL, "dtype must be BD_BF16 or BD_F32");
  const int elt = dt == BD_BF16 ? 2 : 4;
  if ((d->n_per_seq * elt) % 16 != 0) return fail(BD_EINVAL, "n_per_seq * element size must be a multiple of 16 bytes");
  if (!(d->eps >= 0.f) || !std::isfinite(d->eps)) return fail(BD_EINVAL, "eps must be finite and >= 0");
  if (d->max_iter < 1) return fail(BD_EINVAL, "max_iter must be >= 1");
  return BD_OK;
}

void plan_halt(const bd_halt_desc* d, int* nslice, int64_t* slice, size_t* bytes) {
  // ~2048 workgroups of 256 threads, slices of >= 16384 values
  int64_t ns = (2048 + d->batch - 1) / d->batch;
  const int64_t cap = (d->n_per_seq + 16383) / 16384;
  if (ns > cap) ns = cap;
  if (ns < 1) ns = 1;
  int64_t sl = (d->n_per_seq + ns - 1) / ns;
  sl = (sl + 7) / 8 * 8;
  *slice = sl;
  *nslice = (int)((d->n_per_seq + sl - 1) / sl);
  *bytes = align_up((size_t)d->batch * *nslice * 2 * sizeof(float), 256);
}

}  // namespace

extern "C" {

const char* bd_last_error(void) { return g_error.c_str(); }

const char* bd_version(void) { return "bd 0.1.0 gfx950"; }

size_t bd_attn_workspace_bytes(const bd_attn_desc* desc) {
  if (check_attn_desc(desc) != BD_OK) return 0;
  bd::AttnPlan p;
  if (plan_attn(desc, &p) != BD_OK) return 0;
  return p.bytes;
}

bd_status bd_attn_plan(const bd_attn_desc* desc, bd_attn_plan_info* info) {
  bd_status st = check_attn_desc(desc);
  if (st != BD_OK) return st;
  if (!info) return fail(BD_EINVAL, "info is NULL");
  bd::AttnPlan p;
  st = plan_attn(desc, &p);
  if (st != BD_OK) return st;
  info->waves = p.waves;
  info->rows_per_wave = p.rows_per_wave;
  info->row_tiles = p.row_tiles;
  info->num_splits = p.nsplit;
  info->chunk_keys = p.chunk;
  info->workgroups = p.n_items;
  return BD_OK;
}

bd_status bd_attn_step(const bd_attn_desc* desc, const void* q, const void* k_blk, const void* v_blk,
                       const void* k_cache, const void* v_cache, const int32_t* prefix_len, const uint8_t* active,
                       void* out, float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  bd_status st = check_attn_desc(desc);
  if (st != BD_OK) return st;
  st = check_attn_ptrs(desc, q, k_blk, v_blk, k_cache, v_cache, prefix_len, out, lse);
  if (st != BD_OK) return st;
  bd::AttnPlan plan;
  st = plan_attn(desc, &plan);
  if (st != BD_OK) return st;
  st = check_ws(workspace, workspace_bytes, plan.bytes);
  if (st != BD_OK) return st;
  return run_attn(desc, plan, q, k_blk, v_blk, k_cache, v_cache, prefix_len, active, out, lse, workspace,
                  static_cast<hipStream_t>(stream));
}

size_t bd_unmask_workspace_bytes(const bd_unmask_desc* desc) {
  if (check_unmask_desc(desc) != BD_OK) return 0;
  bd::UnmaskPlan p;
  plan_unmask(desc, &p);
  return p.bytes;
}

bd_status bd_confidence_unmask(const bd_unmask_desc* desc, const void* logits, uint8_t* mask, int32_t* tokens,
                               float* conf, int32_t* argmax, int32_t* n_commit, void* workspace,
                               size_t workspace_bytes, void* stream) {
  bd_status st = check_unmask_desc(desc);
  if (st != BD_OK) return st;
  st = check_unmask_ptrs(logits, mask, tokens, conf, argmax, n_commit);
  if (st != BD_OK) return st;
  bd::UnmaskPlan plan;
  plan_unmask(desc, &plan);
  st = check_ws(workspace, workspace_bytes, plan.bytes);
  if (st != BD_OK) return st;
  return run_unmask(desc, plan, logits, mask, tokens, conf, argmax, n_commit, workspace, desc->commit_all, 0,
                    nullptr, nullptr, static_cast<hipStream_t>(stream));
}

bd_status bd_confidence_unmask_noalloc(const bd_unmask_desc* desc, const void* logits, uint8_t* mask,
                                       int32_t* tokens, float* conf, int32_t* argmax, int32_t* n_commit,
                                       void* stream) {
  bd_status st = check_unmask_desc(desc);
  if (st != BD_OK) return st;
  st = check_unmask_ptrs(logits, mask, tokens, conf, argmax, n_commit);
  if (st != BD_OK) return st;
  bd::UnmaskPlan plan;
  plan_unmask(desc, &plan);
  if (plan.bytes > bd::kUnmaskStaticScratchBytes)
    return fail(BD_EUNSUPPORTED, "bd_confidence_unmask_noalloc: %lld rows need %zu bytes of scratch; the static "
                "scratch holds %zu (at most %zu rows: use bd_confidence_unmask with a workspace)",
                (long long)desc->batch * desc->block_len, plan.bytes, bd::kUnmaskStaticScratchBytes,
                bd::kUnmaskStaticScratchBytes / (3 * sizeof(float)));
  void* ws = nullptr;
  const hipError_t e = bd::unmask_static_scratch(&ws);
  if (e != hipSuccess) return fail(BD_EHIP, "static scratch address: %s", hipGetErrorString(e));
  return run_unmask(desc, plan, logits, mask, tokens, conf, argmax, n_commit, ws, desc->commit_all, 0, nullptr,
                    nullptr, static_cast<hipStream_t>(stream));
}

bd_status bd_kv_append(const bd_attn_desc* desc, const void* k_new, const void* v_new, void* k_cache,
                       void* v_cache, int32_t* prefix_len, const uint8_t* active, void* stream) {
  bd_status st = check_attn_desc(desc);
  if (st != BD_OK) return st;
  if (desc->max_prefix_len + desc->block_len > desc->prefix_capacity)
    return fail(BD_EINVAL, "append would pass the cache capacity: max_prefix_len (%lld) + block_len (%d) > "
                "prefix_capacity (%lld)", (long long)desc->max_prefix_len, desc->block_len,
                (long long)desc->prefix_capacity);
  const void* req[] = {k_new, v_new, k_cache, v_cache};
  const char* names[] = {"k_new", "v_new", "k_cache", "v_cache"};
  for (int i = 0; i < 4; ++i) {
    if (!req[i]) return fail(BD_EINVAL, "%s is NULL", names[i]);
    if (!aligned(req[i], 16)) return fail(BD_EINVAL, "%s is not 16-byte aligned", names[i]);
  }
  if (!prefix_len || !aligned(prefix_len, 4)) return fail(BD_EINVAL, "prefix_len is NULL or not 4-byte aligned");
  bd::AppendArgs a{};
  a.k_new = static_cast<const uint16_t*>(k_new);
  a.v_new = static_cast<const uint16_t*>(v_new);
  a.k_cache = static_cast<uint16_t*>(k_cache);
  a.v_cache = static_cast<uint16_t*>(v_cache);
  a.prefix_len = prefix_len;
  a.active = active;
  a.B = desc->batch;
  a.S = desc->block_len;
  a.Hkv = desc->n_kv_heads;
  a.D = desc->head_dim;
  a.lcap = desc->prefix_capacity;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (bd::kv_append_one_launch(a))
    return traced("kv_append", s, [&](const bd::Launch& l) { return bd::launch_kv_append_seq(a, l); });
  st = traced("kv_append", s, [&](const bd::Launch& l) { return bd::launch_kv_append(a, l); });
  if (st != BD_OK) return st;
  return traced("len_advance", s, [&](const bd::Launch& l) { return bd::launch_len_advance(a, l); });
}

bd_status bd_spec_verify(const bd_unmask_desc* desc, const void* logits, const int32_t* draft,
                         const int32_t* first_choice, int32_t* tokens, int32_t* n_commit, int32_t* next_choice,
                         void* workspace, size_t workspace_bytes, void* stream) {
  bd_status st = check_unmask_desc(desc);
  if (st != BD_OK) return st;
  if (!logits || !aligned(logits, 16)) return fail(BD_EINVAL, "logits is NULL or not 16-byte aligned");
  const void* req[] = {draft, first_choice, tokens, n_commit, next_choice};
  const char* names[] = {"draft", "first_choice", "tokens", "n_commit", "next_choice"};
  for (int i = 0; i < 5; ++i)
    if (!req[i] || !aligned(req[i], 4)) return fail(BD_EINVAL, "%s is NULL or not 4-byte aligned", names[i]);
  bd::UnmaskPlan plan;
  plan_unmask(desc, &plan);
  st = check_ws(workspace, workspace_bytes, plan.bytes);
  if (st != BD_OK) return st;
  bd::UnmaskArgs a{};
  a.logits = logits;
  a.is_bf16 = desc->logits_dtype == BD_BF16;
  a.row_stride = desc->row_stride;
  a.vocab = desc->vocab;
  a.B = desc->batch;
  a.S = desc->block_len;
  a.mask = nullptr;   // every row
  a.tokens = tokens;
  a.n_commit = n_commit;
  a.part = static_cast<float*>(workspace);
  a.vsplit = plan.vsplit;
  a.slice = plan.slice;
  a.draft = draft;
  a.first_choice = first_choice;
  a.next_choice = next_choice;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = traced("vocab_reduce", s, [&](const bd::Launch& l) { return bd::launch_vocab_reduce(a, l); });
  if (st != BD_OK) return st;
  return traced("spec_accept", s, [&](const bd::Launch& l) { return bd::launch_spec_accept(a, l); });
}

size_t bd_loop_halt_workspace_bytes(const bd_halt_desc* desc) {
  if (check_halt_desc(desc) != BD_OK) return 0;
  int ns;
  int64_t sl;
  size_t bytes;
  plan_halt(desc, &ns, &sl, &bytes);
  return bytes;
}

bd_status bd_loop_halt(const bd_halt_desc* desc, const void* h_prev, const void* h_cur, int32_t iteration,
                       float* rel, uint8_t* halt, void* workspace, size_t workspace_bytes, void* stream) {
  bd_status st = check_halt_desc(desc);
  if (st != BD_OK) return st;
  if (!h_prev || !h_cur || !aligned(h_prev, 16) || !aligned(h_cur, 16))
    return fail(BD_EINVAL, "h_prev / h_cur must be non-NULL and 16-byte aligned");
  if (!halt) return fail(BD_EINVAL, "halt is NULL");
  if (rel && !aligned(rel, 4)) return fail(BD_EINVAL, "rel is not 4-byte aligned");
  if (iteration < 1) return fail(BD_EINVAL, "iteration must be >= 1 (1-based)");
  bd::HaltArgs a{};
  size_t need;
  plan_halt(desc, &a.nslice, &a.slice, &need);
  st = check_ws(workspace, workspace_bytes, need);
  if (st != BD_OK) return st;
  a.h_prev = h_prev;
  a.h_cur = h_cur;
  a.is_bf16 = desc->dtype == BD_BF16;
  a.B = desc->batch;
  a.n = desc->n_per_seq;
  a.part = static_cast<float*>(workspace);
  a.eps = desc->eps;
  a.iteration = iteration;
  a.max_iter = desc->max_iter;
  a.rel = rel;
  a.halt = halt;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = traced("halt_reduce", s, [&](const bd::Launch& l) { return bd::launch_halt_reduce(a, l); });
  if (st != BD_OK) return st;
  return traced("halt_final", s, [&](const bd::Launch& l) { return bd::launch_halt_final(a, l); });
}

bd_status bd_mamba_block_scan(const bd_mamba_desc* desc, const float* h0, const bd_mamba_dir* fwd,
                              const bd_mamba_dir* rev, const float* D, const uint8_t* active, void* y, float* h_out,
                              void* stream) {
  if (!desc) return fail(BD_EINVAL, "Mamba descriptor is NULL");
  if (desc->batch < 1 || desc->n_heads < 1 || desc->n_groups < 1) return fail(BD_EINVAL, "batch, heads and groups must be >= 1");
  if (desc->n_heads % desc->n_groups != 0)
    return fail(BD_EINVAL, "n_heads (%d) must be a multiple of n_groups (%d)", desc->n_heads, desc->n_groups);
  if (desc->head_dim != 64) return fail(BD_EUNSUPPORTED, "head_dim %d is not supported (64)", desc->head_dim);
  if (desc->state_dim != 64 && desc->state_dim != 128)
    return fail(BD_EUNSUPPORTED, "state_dim %d is not supported (64 or 128)", desc->state_dim);
  if (desc->block_len < 1 || desc->block_len > 32) return fail(BD_EINVAL, "block_len must be in [1, 32] (got %d)", desc->block_len);
  if ((int64_t)desc->batch * desc->n_heads > 0x7fffffff) return fail(BD_EUNSUPPORTED, "batch * n_heads too large");
  if (!fwd || !rev) return fail(BD_EINVAL, "direction inputs are NULL");
  const bd_mamba_dir* dirs[2] = {fwd, rev};
  for (int d = 0; d < 2; ++d) {
    const bd_mamba_dir* r = dirs[d];
    const void* req[] = {r->x, r->dt, r->Bm, r->Cm, r->A};
    const char* names[] = {"x", "dt", "Bm", "Cm", "A"};
    for (int i = 0; i < 5; ++i)
      if (!req[i] || !aligned(req[i], 16))
        return fail(BD_EINVAL, "%s %s is NULL or not 16-byte aligned", d ? "reverse" : "forward", names[i]);
  }
  const void* req[] = {h0, D, y};
  const char* names[] = {"h0", "D", "y"};
  for (int i = 0; i < 3; ++i)
    if (!req[i] || !aligned(req[i], 16)) return fail(BD_EINVAL, "%s is NULL or not 16-byte aligned", names[i]);
  if (h_out && !aligned(h_out, 16)) return fail(BD_EINVAL, "h_out is not 16-byte aligned");
  bd::MambaArgs a{};
  a.h0 = h0;
  a.x = static_cast<const uint16_t*>(fwd->x);
  a.dt = fwd->dt;
  a.Bm = static_cast<const uint16_t*>(fwd->Bm);
  a.Cm = static_cast<const uint16_t*>(fwd->Cm);
  a.A = fwd->A;
  a.x_r = static_cast<const uint16_t*>(rev->x);
  a.dt_r = rev->dt;
  a.Bm_r = static_cast<const uint16_t*>(rev->Bm);
  a.Cm_r = static_cast<const uint16_t*>(rev->Cm);
  a.A_r = rev->A;
  a.D = D;
  a.active = active;
  a.y = static_cast<uint16_t*>(y);
  a.h_out = h_out;
  a.B = desc->batch;
  a.S = desc->block_len;
  a.H = desc->n_heads;
  a.G = desc->n_groups;
  a.N = desc->state_dim;
  return traced("mamba_block", static_cast<hipStream_t>(stream),
                [&](const bd::Launch& l) { return bd::launch_mamba_block(a, l); });
}

size_t bd_denoise_workspace_bytes(const bd_attn_desc* attn, const bd_unmask_desc* unmask) {
  if (check_attn_desc(attn) != BD_OK || check_unmask_desc(unmask) != BD_OK) return 0;
  if (attn->batch != unmask->batch || attn->block_len != unmask->block_len) return 0;
  bd::AttnPlan ap;
  bd::UnmaskPlan up;
  if (plan_attn(attn, &ap) != BD_OK) return 0;
  plan_unmask(unmask, &up);
  return loop_bytes(ap, up, attn->batch);
}

bd_status bd_denoise_block(const bd_attn_desc* attn, const bd_unmask_desc* unmask, int32_t T, int32_t t0,
                           const bd_step_hooks* hooks, const void* k_cache, const void* v_cache,
                           const int32_t* prefix_len, void* out, uint8_t* mask, int32_t* tokens, int32_t* steps_used,
                           int32_t* commits_per_step, void* workspace, size_t workspace_bytes, void* stream) {
  bd_status st = check_attn_desc(attn);
  if (st != BD_OK) return st;
  st = check_unmask_desc(unmask);
  if (st != BD_OK) return st;
  if (attn->batch != unmask->batch || attn->block_len != unmask->block_len)
    return fail(BD_EINVAL, "attention and unmask descriptors disagree on batch / block_len");
  if (T < 1) return fail(BD_EINVAL, "T must be >= 1");
  if (t0 < 0 || t0 >= T) return fail(BD_EINVAL, "t0 must be in [0, T)");
  if (!hooks || !hooks->get_qkv || !hooks->get_logits) return fail(BD_EINVAL, "hooks and both callbacks are required");
  if (!steps_used || !aligned(steps_used, 4)) return fail(BD_EINVAL, "steps_used is NULL or misaligned");
  if (commits_per_step && !aligned(commits_per_step, 4)) return fail(BD_EINVAL, "commits_per_step is misaligned");
  if (!mask || !tokens || !aligned(tokens, 4)) return fail(BD_EINVAL, "mask / tokens NULL or misaligned");
  if (!k_cache || !v_cache || !prefix_len || !out || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(out, 16) || !aligned(prefix_len, 4))
    return fail(BD_EINVAL, "k_cache / v_cache / prefix_len / out NULL or misaligned");
  bd::AttnPlan ap;
  bd::UnmaskPlan up;
  st = plan_attn(attn, &ap);
  if (st != BD_OK) return st;
  plan_unmask(unmask, &up);
  const size_t need = loop_bytes(ap, up, attn->batch);
  st = check_ws(workspace, workspace_bytes, need);
  if (st != BD_OK) return st;
  char* w = static_cast<char*>(workspace);
  void* ws_attn = w;
  void* ws_unmask = w + ap.bytes;
  uint8_t* active = reinterpret_cast<uint8_t*>(w + ap.bytes + up.bytes);
  hipStream_t s = static_cast<hipStream_t>(stream);

  st = traced("loop_init", s, [&](const bd::Launch& l) { return bd::launch_loop_init(mask, attn->batch, attn->block_len, active, steps_used, l); });
  if (st != BD_OK) return st;
  for (int32_t t = t0; t < T; ++t) {
    const void *q = nullptr, *kb = nullptr, *vb = nullptr;
    st = hooks->get_qkv(hooks->user, t, mask, tokens, &q, &kb, &vb, stream);
    if (st != BD_OK) return fail(st, "get_qkv hook failed at step %d", t);
    if (!q || !kb || !vb || !aligned(q, 16) || !aligned(kb, 16) || !aligned(vb, 16))
      return fail(BD_EINVAL, "get_qkv returned NULL or misaligned pointers at step %d", t);
    st = run_attn(attn, ap, q, kb, vb, k_cache, v_cache, prefix_len, active, out, nullptr, ws_attn, s);
    if (st != BD_OK) return st;
    const void* logits = nullptr;
    st = hooks->get_logits(hooks->user, t, out, &logits, stream);
    if (st != BD_OK) return fail(st, "get_logits hook failed at step %d", t);
    if (!logits || !aligned(logits, 16)) return fail(BD_EINVAL, "get_logits returned NULL or misaligned logits at step %d", t);
    int32_t* nc = commits_per_step ? commits_per_step + (int64_t)t * attn->batch : nullptr;
    st = run_unmask(unmask, up, logits, mask, tokens, nullptr, nullptr, nc, ws_unmask, t == T - 1 ? 1 : 0, t, steps_used,
                    active, s);
    if (st != BD_OK) return st;
  }
  return BD_OK;
}

static bd_status table_get_qkv(void* user, int32_t step, const uint8_t*, const int32_t*, const void** q,
                               const void** kb, const void** vb, void*) {
  const bd_step_table* t = static_cast<const bd_step_table*>(user);
  if (!t || step < 0 || step >= t->n_steps) return fail(BD_EINVAL, "step %d outside the step table", step);
  *q = t->q[step];
  *kb = t->k_blk[step];
  *vb = t->v_blk[step];
  return BD_OK;
}

static bd_status table_get_logits(void* user, int32_t step, const void*, const void** logits, void*) {
  const bd_step_table* t = static_cast<const bd_step_table*>(user);
  if (!t || step < 0 || step >= t->n_steps) return fail(BD_EINVAL, "step %d outside the step table", step);
  *logits = t->logits[step];
  return BD_OK;
}

bd_status bd_table_hooks(const bd_step_table* table, bd_step_hooks* hooks_out) {
  if (!table || !hooks_out || !table->q || !table->k_blk || !table->v_blk || !table->logits || table->n_steps < 1)
    return fail(BD_EINVAL, "bd_table_hooks: incomplete step table");
  hooks_out->get_qkv = table_get_qkv;
  hooks_out->get_logits = table_get_logits;
  hooks_out->user = const_cast<bd_step_table*>(table);
  return BD_OK;
}

// ------------------------------------------------------------------------------------------
// tracing
// ------------------------------------------------------------------------------------------
bd_status bd_trace_create(int32_t capacity, bd_trace** out) {
  if (!out || capacity < 1) return fail(BD_EINVAL, "bd_trace_create: bad arguments");
  bd_trace* t = new bd_trace();
  t->recs.resize(capacity);
  for (auto& r : t->recs) {
    r.name = "";
    if (hipEventCreate(&r.start) != hipSuccess || hipEventCreate(&r.stop) != hipSuccess) {
      bd_trace_destroy(t);
      return fail(BD_EHIP, "hipEventCreate failed");
    }
  }
  *out = t;
  return BD_OK;
}

void bd_trace_destroy(bd_trace* t) {
  if (!t) return;
  if (g_trace == t) g_trace = nullptr;
  for (auto& r : t->recs) {
    if (r.start) (void)hipEventDestroy(r.start);
    if (r.stop) (void)hipEventDestroy(r.stop);
  }
  delete t;
}

bd_status bd_trace_attach(bd_trace* t) {
  g_trace = t;
  return BD_OK;
}

bd_status bd_trace_clear(bd_trace* t) {
  if (!t) return fail(BD_EINVAL, "trace is NULL");
  t->count = 0;
  return BD_OK;
}

int32_t bd_trace_count(const bd_trace* t) { return t ? t->count : 0; }

bd_status bd_trace_get(const bd_trace* t, int32_t i, const char** kernel, float* ms) {
  if (!t || i < 0 || i >= t->count) return fail(BD_EINVAL, "bd_trace_get: index out of range");
  const auto& r = t->recs[i];
  if (hipEventSynchronize(r.stop) != hipSuccess) return fail(BD_EHIP, "hipEventSynchronize failed");
  float v = 0.f;
  if (hipEventElapsedTime(&v, r.start, r.stop) != hipSuccess) return fail(BD_EHIP, "hipEventElapsedTime failed");
  if (kernel) *kernel = r.name;
  if (ms) *ms = v;
  return BD_OK;
}

}  // extern "C"
