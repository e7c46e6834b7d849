// Append of a committed block to the prefix cache on gfx950.
//
// Source: Nemotron-TwoTower technical summary, §Architecture and §Generation -- the frozen
// context tower is a causal AR model over the committed tokens and its KV cache grows by each
// committed block before the next one is denoised.
//
// kv_append: one thread per 16 bytes of a (sequence, block position, KV head) row of K and of V
// -- coalesced 16-byte loads from the block tensors and stores into the cache rows
// prefix_len[b] .. prefix_len[b] + S - 1. len_advance (a second launch, so no thread reads a
// length another has already advanced): prefix_len[b] += S for every active sequence.
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
  const int64_t pos = (int64_t)a.prefix_len[b] + s;
  const int64_t src = row * a.D + d8 * 8;
  const int64_t dst = (((int64_t)b * a.Hkv + g) * a.lcap + pos) * a.D + d8 * 8;
  *reinterpret_cast<u32x4*>(a.k_cache + dst) = *reinterpret_cast<const u32x4*>(a.k_new + src);
  *reinterpret_cast<u32x4*>(a.v_cache + dst) = *reinterpret_cast<const u32x4*>(a.v_new + src);
}

__global__ __launch_bounds__(64) void len_advance_kernel(AppendArgs a) {
  const int b = blockIdx.x * 64 + threadIdx.x;
  if (b < a.B && (!a.active || a.active[b])) a.prefix_len[b] += a.S;
}

}  // namespace

hipError_t launch_kv_append(const AppendArgs& a, const Launch& l) {
  const int64_t total = (int64_t)a.B * a.S * a.Hkv * (a.D / 8);
  return launch_kernel(kv_append_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), l, a);
}

hipError_t launch_len_advance(const AppendArgs& a, const Launch& l) {
  return launch_kernel(len_advance_kernel, dim3((unsigned)((a.B + 63) / 64)), dim3(64), l, a);
}

}  // namespace bd
