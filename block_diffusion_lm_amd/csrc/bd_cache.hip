// Append of a committed block to the prefix cache on gfx950.
//
// Source: Nemotron-TwoTower technical summary, §Architecture and §Generation -- the frozen
// context tower is a causal AR model over the committed tokens and its KV cache grows by each
// committed block before the next one is denoised.
//
// A block of at most kSeqUnits 16-byte units of K (and as many of V) per sequence takes one
// launch: kv_append_seq, one workgroup per sequence, every thread reads the sequence's length,
// issues all its loads, then its stores into the cache rows prefix_len[b] .. prefix_len[b] + S - 1;
// after a workgroup barrier (every thread has read the length, and no other workgroup reads it)
// thread 0 advances prefix_len[b] by S. Larger blocks take two: kv_append, one thread per 16 bytes
// of a (sequence, block position, KV head) row of K and of V over the whole grid, then
// len_advance (a second launch, so no thread reads a length another has already advanced).
// A sequence whose length breaks the precondition (negative, or prefix_len[b] + S above the
// capacity) is skipped by all three kernels: nothing written, its length not advanced, so a stale
// host bound cannot write into another sequence's rows or past the cache.
#include "bd_internal.h"

namespace bd {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void kv_append_kernel(AppendArgs a) {
  const int D8 = a.D / 8;
  const int64_t total = (int64_t)a.B * a.S * a.Hkv * D8;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= total) return;
  const int d8 = (int)(gid % D8);
  const int64_t row = gid / D8;                 // (b, s, g) in the block tensors' order
  const int g = (int)(row % a.Hkv);
  const int s = (int)((row / a.Hkv) % a.S);
  const int b = (int)(row / ((int64_t)a.Hkv * a.S));
  if (a.active && !a.active[b]) return;
  const int64_t len = a.prefix_len[b];
  if (len < 0 || len + a.S > a.lcap) return;
  const int64_t pos = len + s;
  const int64_t src = row * a.D + d8 * 8;
  const int64_t dst = (((int64_t)b * a.Hkv + g) * a.lcap + pos) * a.D + d8 * 8;
  *reinterpret_cast<u32x4*>(a.k_cache + dst) = *reinterpret_cast<const u32x4*>(a.k_new + src);
  *reinterpret_cast<u32x4*>(a.v_cache + dst) = *reinterpret_cast<const u32x4*>(a.v_new + src);
}

template <int U>
__global__ __launch_bounds__(256) void kv_append_seq_kernel(AppendArgs a) {
  const int b = blockIdx.x;
  if (a.active && !a.active[b]) return;   // uniform per workgroup
  const int tid = threadIdx.x;
  const int D8 = a.D / 8;
  const int units = a.S * a.Hkv * D8;     // <= 256 * U
  const int64_t len = a.prefix_len[b];
  if (len < 0 || len + a.S > a.lcap) return;   // uniform per workgroup
  u32x4 k[U], v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int i = tid + u * 256;
    if (i < units) {
      const int64_t src = (int64_t)b * units * 8 + (int64_t)i * 8;   // (s, g, d8) in the block tensors' order
      k[u] = *reinterpret_cast<const u32x4*>(a.k_new + src);
      v[u] = *reinterpret_cast<const u32x4*>(a.v_new + src);
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int i = tid + u * 256;
    if (i < units) {
      const int d8 = i % D8;
      const int g = (i / D8) % a.Hkv;
      const int s = i / (D8 * a.Hkv);
      const int64_t dst = (((int64_t)b * a.Hkv + g) * a.lcap + len + s) * a.D + d8 * 8;
      *reinterpret_cast<u32x4*>(a.k_cache + dst) = k[u];
      *reinterpret_cast<u32x4*>(a.v_cache + dst) = v[u];
    }
  }
  __syncthreads();
  if (tid == 0) a.prefix_len[b] = (int32_t)(len + a.S);
}

__global__ __launch_bounds__(64) void len_advance_kernel(AppendArgs a) {
  const int b = blockIdx.x * 64 + threadIdx.x;
  if (b >= a.B || (a.active && !a.active[b])) return;
  const int64_t len = a.prefix_len[b];
  if (len >= 0 && len + a.S <= a.lcap) a.prefix_len[b] = (int32_t)(len + a.S);
}

}  // namespace

hipError_t launch_kv_append(const AppendArgs& a, const Launch& l) {
  const int64_t total = (int64_t)a.B * a.S * a.Hkv * (a.D / 8);
  return launch_kernel(kv_append_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), l, a);
}

bool kv_append_one_launch(const AppendArgs& a) {
  return (int64_t)a.S * a.Hkv * (a.D / 8) <= kSeqUnits;
}

hipError_t launch_kv_append_seq(const AppendArgs& a, const Launch& l) {
  const int units = a.S * a.Hkv * (a.D / 8);
  const dim3 grid((unsigned)a.B), block(256);
  if (units <= 256) return launch_kernel(kv_append_seq_kernel<1>, grid, block, l, a);
  if (units <= 512) return launch_kernel(kv_append_seq_kernel<2>, grid, block, l, a);
  if (units <= 1024) return launch_kernel(kv_append_seq_kernel<4>, grid, block, l, a);
  return launch_kernel(kv_append_seq_kernel<8>, grid, block, l, a);
}

hipError_t launch_len_advance(const AppendArgs& a, const Launch& l) {
  return launch_kernel(len_advance_kernel, dim3((unsigned)((a.B + 63) / 64)), dim3(64), l, a);
}

}  // namespace bd
