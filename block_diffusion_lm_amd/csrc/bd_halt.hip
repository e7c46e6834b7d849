// Adaptive loop halting on gfx950: relative change of each sequence's hidden state between two
// loop iterations.
//
// Source: Technical summary: LoopMDM, §Adaptive inference -- the looped mid-block stops when the
// relative hidden-state change between consecutive iterations falls below epsilon, or at the
// iteration budget.
//
// halt_reduce: one workgroup per (sequence, slice) streams its slice of both states once with
// 16-byte loads (HBM-bound: 2 x n x element bytes per sequence) and keeps per-thread float32 sums
// of (cur - prev)^2 and prev^2, combined in a fixed order (wave butterflies, then the four waves
// in order). halt_final: one wave per sequence adds its slices in a fixed order and decides.
#include "bd_internal.h"

namespace bd {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float value_at(const void* base, int is_bf16, int64_t j) {
  if (is_bf16) return __uint_as_float((uint32_t)(reinterpret_cast<const uint16_t*>(base)[j]) << 16);
  return reinterpret_cast<const float*>(base)[j];
}

__global__ __launch_bounds__(256) void halt_reduce_kernel(HaltArgs a) {
  const int b = blockIdx.x / a.nslice;
  const int part = blockIdx.x % a.nslice;
  const int tid = threadIdx.x;
  const int64_t v0 = (int64_t)part * a.slice;
  const int64_t v1 = min(v0 + a.slice, a.n);
  const int elt = a.is_bf16 ? 2 : 4;
  const char* pp = reinterpret_cast<const char*>(a.h_prev) + (int64_t)b * a.n * elt;
  const char* pc = reinterpret_cast<const char*>(a.h_cur) + (int64_t)b * a.n * elt;
  float d2 = 0.f, p2 = 0.f;
  if (v0 < v1) {
    const int per = 16 / elt;
    const int64_t nvec = (v1 - v0) / per;
    const u32x4* vp = reinterpret_cast<const u32x4*>(pp + v0 * elt);
    const u32x4* vc = reinterpret_cast<const u32x4*>(pc + v0 * elt);
    auto add = [&](const u32x4 up, const u32x4 uc) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        if (a.is_bf16) {
          const float p_lo = __uint_as_float(up[w] << 16), p_hi = __uint_as_float(up[w] & 0xffff0000u);
          const float c_lo = __uint_as_float(uc[w] << 16), c_hi = __uint_as_float(uc[w] & 0xffff0000u);
          d2 = fmaf(c_lo - p_lo, c_lo - p_lo, d2);
          d2 = fmaf(c_hi - p_hi, c_hi - p_hi, d2);
          p2 = fmaf(p_lo, p_lo, p2);
          p2 = fmaf(p_hi, p_hi, p2);
        } else {
          const float p = __uint_as_float(up[w]), c = __uint_as_float(uc[w]);
          d2 = fmaf(c - p, c - p, d2);
          p2 = fmaf(p, p, p2);
        }
      }
    };
    int64_t i = tid;
    for (; i + 3 * 256 < nvec; i += 4 * 256) {   // four 16-byte loads of each state in flight
      u32x4 up[4], uc[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        up[u] = __builtin_nontemporal_load(vp + i + u * 256);
        uc[u] = __builtin_nontemporal_load(vc + i + u * 256);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) add(up[u], uc[u]);
    }
    for (; i < nvec; i += 256) add(__builtin_nontemporal_load(vp + i), __builtin_nontemporal_load(vc + i));
    for (int64_t j = v0 + nvec * per + tid; j < v1; j += 256) {   // ragged tail of the slice
      const float p = value_at(pp, a.is_bf16, j), c = value_at(pc, a.is_bf16, j);
      d2 = fmaf(c - p, c - p, d2);
      p2 = fmaf(p, p, p2);
    }
  }
#pragma unroll
  for (int msk = 32; msk > 0; msk >>= 1) {
    d2 += __shfl_xor(d2, msk, 64);
    p2 += __shfl_xor(p2, msk, 64);
  }
  __shared__ float red[4][2];
  if ((tid & 63) == 0) {
    red[tid >> 6][0] = d2;
    red[tid >> 6][1] = p2;
  }
  __syncthreads();
  if (tid == 0) {
    float* out = a.part + ((int64_t)b * a.nslice + part) * 2;
    out[0] = ((red[0][0] + red[1][0]) + red[2][0]) + red[3][0];
    out[1] = ((red[0][1] + red[1][1]) + red[2][1]) + red[3][1];
  }
}

// One wave per sequence: lane j adds slices j, j + 64, ... in order, then a fixed butterfly.
__global__ __launch_bounds__(64) void halt_final_kernel(HaltArgs a) {
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const float* pp = a.part + (int64_t)b * a.nslice * 2;
  float d2 = 0.f, p2 = 0.f;
  for (int c = lane; c < a.nslice; c += 64) {
    d2 += pp[2 * c];
    p2 += pp[2 * c + 1];
  }
#pragma unroll
  for (int msk = 32; msk > 0; msk >>= 1) {
    d2 += __shfl_xor(d2, msk, 64);
    p2 += __shfl_xor(p2, msk, 64);
  }
  if (lane == 0) {
    const float r = d2 == 0.f ? 0.f : sqrtf(d2) / sqrtf(p2);   // p2 == 0 < d2: +inf
    if (a.rel) a.rel[b] = r;
    a.halt[b] = (r < a.eps || a.iteration >= a.max_iter) ? 1 : 0;
  }
}

}  // namespace

hipError_t launch_halt_reduce(const HaltArgs& a, const Launch& l) {
  return launch_kernel(halt_reduce_kernel, dim3((unsigned)((int64_t)a.B * a.nslice)), dim3(256), l, a);
}

hipError_t launch_halt_final(const HaltArgs& a, const Launch& l) {
  return launch_kernel(halt_final_kernel, dim3((unsigned)a.B), dim3(64), l, a);
}

}  // namespace bd
