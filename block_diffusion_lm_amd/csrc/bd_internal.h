// Internal interface between the host side of the library (bd_api.cpp) and the HIP kernels
// (bd_attn.hip, bd_unmask.hip, bd_cache.hip, bd_halt.hip, bd_mamba.hip). Not installed; the public ABI is
// include/bd.h.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace bd {

// Where a kernel goes: its stream and, when a trace is attached, the events that the dispatch
// itself stamps at kernel start and end (hipExtLaunchKernelGGL), so a traced duration is the
// kernel's own, without the gaps of separately recorded events.
struct Launch {
  hipStream_t stream;
  hipEvent_t start = nullptr, stop = nullptr;
};

template <typename K, typename... Args>
hipError_t launch_kernel(K kernel, dim3 grid, dim3 block, const Launch& l, Args... args) {
  hipExtLaunchKernelGGL(kernel, grid, block, 0, l.stream, l.start, l.stop, 0, args...);
  return hipGetLastError();
}

// Work item of this work-group such that the work-groups of one XCD take consecutive items. The
// dispatcher hands work-groups to the eight XCDs in turn (work-group i to XCD i mod 8) and each XCD
// has its own L2, so items that share data (heads of one B/C group, rows sharing a cache sector)
// are fetched once per XCD instead of once per work-group. A bijection of [0, n): the first
// 8 * floor(n / 8) work-groups are regrouped, the rest keep their index.
constexpr unsigned kXcds = 8;
__device__ __forceinline__ unsigned xcd_local_item(unsigned i, unsigned n) {
  const unsigned per = n / kXcds;
  return i < per * kXcds ? (i % kXcds) * per + i / kXcds : i;
}

// ---------------------------------------------------------------------------------------------
// attention
// ---------------------------------------------------------------------------------------------

// LDS ring of the attention split kernel, shared by the kernel and the host planner: a stage holds
// one tile of kAttnKeyTile keys (K rows, then V rows; D values each, 16-byte chunks or 64-byte blocks swizzled).
constexpr int kAttnKeyTile = 64;
constexpr int attn_stage_bytes(int head_dim) { return 2 * kAttnKeyTile * head_dim * 2; }
// stages in the ring: 256-row workgroups (one per CU) prefetch three tiles ahead; 128-row
// workgroups (two per CU) one, except at head_dim 64 where four stages still fit twice.
constexpr int attn_stages(int head_dim, int row_blocks) { return (row_blocks == 8 || head_dim == 64) ? 4 : 2; }

struct AttnPlan {
  int head_dim;       // D
  int waves;          // waves per workgroup (4 or 8)
  int rows_per_wave;  // 32 or 64 (one or two 32-row MFMA blocks); a workgroup owns waves*rows_per_wave rows
  int rows;           // R = S * (Hq / Hkv): query rows per (sequence, KV head)
  int row_tiles;      // ceil(R / (waves * rows_per_wave))
  int key_tile;       // keys staged through LDS per iteration (kAttnKeyTile)
  int64_t chunk;      // keys per split (multiple of 64)
  int nsplit;         // splits per (sequence, KV head)
  int64_t n_items;    // B * Hkv * nsplit * row_tiles workgroups
  bool direct;        // nsplit == 1: the split kernel writes the final output itself
  bool wide_merge;    // many splits: the merge spreads each row's chunks over eight thread groups
  size_t part_o_off, part_ml_off, plan_off, bytes;   // workspace layout
};

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k_blk;
  const uint16_t* v_blk;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const int32_t* prefix_len;
  const uint8_t* active;
  uint16_t* out;
  float* lse;
  uint16_t* part_o;   // [n_items][rows_pad][D] bf16: the chunk's normalized output acc / l
  float* part_ml;     // [n_items][rows_pad][2]: running max (log2 units) and sum
  int* plan_pfx;      // [B + 1] balanced plan: first chunk slot of every sequence, then the total
                      // (written by the split launch's first work-group, read by the merge)
  int B, S, Hq, Hkv, group, rows, rows_pad;
  int64_t lcap;
  int64_t chunk;
  int64_t max_keys;   // max_prefix_len + S: the longest key sequence the plan covers
  int nsplit, row_tiles;
  float scale_log2;   // tau * log2(e)
  int direct;
  int balanced;       // split launch over at most kMaxBalancedBatch sequences: chunks sized on the
                      // device from the actual lengths (see balanced_plan in bd_attn.hip)
  int causal;         // 1: block key j is visible to block position s only when j <= s
  int stream_kv;      // 1: the cached K/V of one launch exceed kStreamKvBytes; loaded non-temporally
};

// K/V bytes of one launch (B Hkv (max_prefix_len + S) D, K and V, bf16) above which the split
// kernel streams the cache past the caches: half the MI355X's 256 MB last-level cache.
constexpr int64_t kStreamKvBytes = (int64_t)128 << 20;

// Largest batch whose split launches plan their chunks from the actual prefix lengths on the device
// (the work-groups keep one prefix-sum entry per sequence in LDS).
constexpr int kMaxBalancedBatch = 1024;

hipError_t launch_attn_split(const AttnPlan& plan, const AttnArgs& a, const Launch& l);
hipError_t launch_attn_merge(const AttnPlan& plan, const AttnArgs& a, const Launch& l);

// ---------------------------------------------------------------------------------------------
// confidence unmasking
// ---------------------------------------------------------------------------------------------
struct UnmaskPlan {
  int vsplit;          // vocabulary slices per row
  int64_t slice;       // elements per slice (multiple of 8)
  size_t bytes;
};

struct UnmaskArgs {
  const void* logits;
  int is_bf16;
  int64_t row_stride;
  int vocab;
  int B, S;
  uint8_t* mask;
  int32_t* tokens;
  float* conf;
  int32_t* argmax;
  int32_t* n_commit;
  float gamma;
  int min_commit, commit_all;
  float* part;         // [B*S][vsplit][3]: max, index (as int bits), sum of exp
  int compact;         // the reduction's work-groups take the masked rows in order (B*S <= kCompactRows)
  int vsplit;
  int64_t slice;
  // loop bookkeeping (all optional)
  int step;
  int32_t* steps_used;          // [B]: set to step+1 where the sequence had a masked position
  uint8_t* active_next;         // [B]: whether a masked position remains after the commit
  // self-speculation check (mask == nullptr: every row is reduced)
  const int32_t* draft;         // [B*S]
  const int32_t* first_choice;  // [B]
  int32_t* next_choice;         // [B]
};

hipError_t launch_vocab_reduce(const UnmaskArgs& a, const Launch& l);

// Most rows (B * S) whose masked positions the reduction compacts: every work-group scans that
// many mask bytes, 16 per thread.
constexpr int kCompactRows = 4096;

// Allocation-free unmasking: the slice partials live in a static device array of this many bytes
// (one copy per device, held until the process ends) instead of a caller workspace.
constexpr size_t kUnmaskStaticScratchBytes = (size_t)4 << 20;
// Device address of the calling thread's current device's copy of that array, resolved with
// hipGetSymbolAddress on the first call per device and cached.
hipError_t unmask_static_scratch(void** ptr);
hipError_t launch_commit(const UnmaskArgs& a, const Launch& l);
hipError_t launch_spec_accept(const UnmaskArgs& a, const Launch& l);
hipError_t launch_loop_init(const uint8_t* mask, int B, int S, uint8_t* active, int32_t* steps_used, const Launch& l);

// ---------------------------------------------------------------------------------------------
// prefix cache append
// ---------------------------------------------------------------------------------------------
struct AppendArgs {
  const uint16_t* k_new;   // [B, S, Hkv, D]
  const uint16_t* v_new;
  uint16_t* k_cache;       // [B, Hkv, Lcap, D]
  uint16_t* v_cache;
  int32_t* prefix_len;     // [B]
  const uint8_t* active;   // [B] or nullptr
  int B, S, Hkv, D;
  int64_t lcap;
};

hipError_t launch_kv_append(const AppendArgs& a, const Launch& l);
// blocks of at most kSeqUnits 16-byte units of K per sequence: copy and length advance in one
// launch (one workgroup per sequence)
constexpr int kSeqUnits = 2048;
bool kv_append_one_launch(const AppendArgs& a);
hipError_t launch_kv_append_seq(const AppendArgs& a, const Launch& l);

// ---------------------------------------------------------------------------------------------
// adaptive loop halting
// ---------------------------------------------------------------------------------------------
struct HaltArgs {
  const void* h_prev;      // [B, n]
  const void* h_cur;
  int is_bf16;
  int B;
  int64_t n;               // values per sequence
  int nslice;              // slices per sequence
  int64_t slice;           // values per slice (multiple of 8)
  float* part;             // [B][nslice][2]: sum (cur - prev)^2, sum prev^2
  float eps;
  int iteration, max_iter;
  float* rel;              // [B] or nullptr
  uint8_t* halt;           // [B]
};

hipError_t launch_halt_reduce(const HaltArgs& a, const Launch& l);

// ---------------------------------------------------------------------------------------------
// block-local bidirectional Mamba scan
// ---------------------------------------------------------------------------------------------
struct MambaArgs {
  const float* h0;          // [B, H, N, P] cached forward boundary state
  const uint16_t* x;        // [B, S, H, P] bf16, forward direction
  const float* dt;          // [B, S, H]
  const uint16_t* Bm;       // [B, S, G, N] bf16
  const uint16_t* Cm;
  const float* A;           // [H]
  const uint16_t* x_r;      // reverse direction, same shapes
  const float* dt_r;
  const uint16_t* Bm_r;
  const uint16_t* Cm_r;
  const float* A_r;
  const float* D;           // [H] skip
  const uint8_t* active;    // [B] or nullptr
  uint16_t* y;              // [B, S, H, P] bf16
  float* h_out;             // [B, H, N, P] or nullptr
  int B, S, H, G, N;        // head_dim P = 64
};

hipError_t launch_mamba_block(const MambaArgs& a, const Launch& l);
hipError_t launch_halt_final(const HaltArgs& a, const Launch& l);
hipError_t launch_len_advance(const AppendArgs& a, const Launch& l);

}  // namespace bd
