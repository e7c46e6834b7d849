// Confidence unmasking on gfx950.
//
// Source: Nemotron-TwoTower technical summary, §Training and conditioning, sampling bullet
// (Algorithm 2): each step predicts every masked position in parallel; a position whose
// confidence is above the threshold gamma is committed, the others stay masked; the number
// committed per step therefore adapts. Confidence is the largest softmax probability of the
// position's logits, p = 1 / sum_j exp(l_j - max_j l_j); the committed token is the lowest index
// holding the maximum.
//
// vocab_reduce: one workgroup per (masked row, vocabulary slice) streams its slice once with
// 16-byte loads and keeps, per thread, the running (max, first index of the max, sum of
// exp(l - max)). The per-thread states are combined in a fixed order (wave butterflies, then the
// four waves in index order), so a row always gives the same bits -- identical rows give
// identical confidences. HBM-bound: every logit of a masked row is read exactly once.
//
// commit: one wave per sequence merges the slices of each of its S rows in slice order, then
// applies the commit rule with ballots: threshold (strict >), or every masked position on the
// last step, or -- when nothing passes -- the single most confident masked position (lowest
// position on ties).
#include <mutex>

#include "bd_internal.h"

namespace bd {
namespace {

// Scratch of the allocation-free entry point (bd_confidence_unmask_noalloc): the slice partials
// [B*S][vsplit][3] go here instead of into a caller workspace. Every device that runs the library
// holds its own copy until the process ends; calls that overlap on one device share it and race.
// Nothing in it needs clearing: the reduction writes every partial that the commit reads.
// In host code `scratch` only names the array; its device address comes from
// unmask_static_scratch() below.
static __device__ __align__(256) char scratch[kUnmaskStaticScratchBytes];

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

struct Red {
  float m;     // running max
  int idx;     // first index holding m
  float z;     // sum of exp(l - m)
};

// Combine two states; `a` covers lower indices than `b` whenever they hold equal maxima.
__device__ __forceinline__ Red combine(Red a, Red b) {
  Red r;
  r.m = fmaxf(a.m, b.m);
  if (r.m == -INFINITY) {
    r.z = 0.f;
    r.idx = min(a.idx, b.idx);
    return r;
  }
  const float za = a.m == -INFINITY ? 0.f : a.z * __builtin_amdgcn_exp2f((a.m - r.m) * kLog2e);
  const float zb = b.m == -INFINITY ? 0.f : b.z * __builtin_amdgcn_exp2f((b.m - r.m) * kLog2e);
  r.z = za + zb;
  r.idx = (a.m > b.m) ? a.idx : (b.m > a.m) ? b.idx : min(a.idx, b.idx);
  return r;
}

__device__ __forceinline__ Red shfl_xor(Red a, int mask) {
  Red r;
  r.m = __shfl_xor(a.m, mask, 64);
  r.idx = __shfl_xor(a.idx, mask, 64);
  r.z = __shfl_xor(a.z, mask, 64);
  return r;
}

// Fold n values (in index order, first index `base`) into the running state.
template <int N>
__device__ __forceinline__ void fold(Red& st, const float (&x)[N], int base) {
  float lm = x[0];
#pragma unroll
  for (int i = 1; i < N; ++i) lm = fmaxf(lm, x[i]);
  if (lm > st.m) {
    int li = N - 1;
#pragma unroll
    for (int i = N - 1; i >= 0; --i)
      if (x[i] == lm) li = i;
    // rescale the old sum to the new max (old max -inf: nothing to keep)
    st.z = (st.m == -INFINITY) ? 0.f : st.z * __builtin_amdgcn_exp2f((st.m - lm) * kLog2e);
    st.m = lm;
    st.idx = base + li;
  }
  // all values so far -inf (then every x is -inf): exp2(-inf) adds nothing, without a branch
  const float mneg = st.m == -INFINITY ? 0.f : -st.m * kLog2e;
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < N; ++i) acc += __builtin_amdgcn_exp2f(fmaf(x[i], kLog2e, mneg));
  st.z += acc;
}

__device__ __forceinline__ float load_logit(const void* row, int is_bf16, int64_t j) {
  if (is_bf16) return __uint_as_float((uint32_t)(reinterpret_cast<const uint16_t*>(row)[j]) << 16);
  return reinterpret_cast<const float*>(row)[j];
}

// The slice partials of row r combined in slice order; sixteen slices' loads are issued together.
__device__ __forceinline__ Red row_partials(const UnmaskArgs& a, int64_t r) {
  constexpr int U = 16;
  const float* pp = a.part + r * a.vsplit * 3;
  Red st{-INFINITY, 0x7fffffff, 0.f};
  for (int c0 = 0; c0 < a.vsplit; c0 += U) {
    float m[U], x[U], z[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int c = min(c0 + j, a.vsplit - 1);   // past the last slice: reloaded, then skipped
      m[j] = pp[3 * c];
      x[j] = pp[3 * c + 1];
      z[j] = pp[3 * c + 2];
    }
#pragma unroll
    for (int j = 0; j < U; ++j)
      if (c0 + j < a.vsplit) st = combine(st, Red{m[j], __float_as_int(x[j]), z[j]});
  }
  return st;
}

template <bool BF16>
__device__ void reduce_slice(const UnmaskArgs& a, int64_t row, int part);
__device__ void commit_sequence(const UnmaskArgs& a, int b);

// Position of the j-th masked row (rows in order) among the first `rows` <= kCompactRows mask
// bytes, or -1 when fewer are masked. Thread t looks at rows 16 t .. 16 t + 15 (loads issued
// unconditionally, past the end clamped and ignored); counts are scanned over the work-group.
// All threads take part (LDS, barriers); the result is uniform.
__device__ int nth_masked_row(const uint8_t* mask, int rows, int j) {
  __shared__ int wsum[4];
  __shared__ int found;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint8_t mb[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) mb[k] = mask[min(16 * tid + k, rows - 1)];
  uint32_t bits = 0;
#pragma unroll
  for (int k = 0; k < 16; ++k) bits |= (16 * tid + k < rows && mb[k] != 0) ? 1u << k : 0u;
  const int cnt = __popc(bits);
  int inc = cnt;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(inc, d, 64);
    if (lane >= d) inc += o;
  }
  if (lane == 63) wsum[wave] = inc;
  if (tid == 0) found = -1;
  __syncthreads();
  int excl = inc - cnt;
  for (int w = 0; w < wave; ++w) excl += wsum[w];
  if (j >= excl && j < excl + cnt) {
    uint32_t b = bits;
    for (int q = j - excl; q > 0; --q) b &= b - 1;   // drop the lower set bits
    found = 16 * tid + __builtin_ctz(b);
  }
  __syncthreads();
  return found;
}

// Work-group w reduces slice w % vsplit of row w / vsplit -- with `compact`, of the (w / vsplit)-th
// masked row instead, so that the busy work-groups are the first ones of the grid and spread evenly
// over the CUs whatever the mask (with scattered masked rows the direct mapping leaves some CUs with
// several busy work-groups and others with none).
template <bool BF16>
__global__ __launch_bounds__(256) void vocab_reduce_kernel(UnmaskArgs a) {
  const int part = (int)(blockIdx.x % a.vsplit);
  int64_t row = blockIdx.x / a.vsplit;
  if (a.compact && a.mask && a.B * a.S <= 64) {
    // one ballot per wave (lane = row), no LDS or barrier
    const int lane = threadIdx.x & 63;
    const int rows = a.B * a.S;
    uint64_t bits = __builtin_amdgcn_ballot_w64(lane < rows && a.mask[min(lane, rows - 1)] != 0);
    if ((int64_t)__popcll(bits) <= row) return;   // uniform
    for (int q = (int)row; q > 0; --q) bits &= bits - 1;   // drop the lower set bits
    row = __builtin_ctzll(bits);
  } else if (a.compact && a.mask) {
    row = nth_masked_row(a.mask, a.B * a.S, (int)row);
    if (row < 0) return;   // uniform
  } else if (a.mask && !a.mask[row]) {
    return;   // uniform per workgroup
  }
  reduce_slice<BF16>(a, row, part);
}

template <bool BF16>
__device__ void reduce_slice(const UnmaskArgs& a, int64_t row, int part) {
  const int tid = threadIdx.x;
  const int64_t v0 = (int64_t)part * a.slice;
  const int64_t v1 = min(v0 + a.slice, (int64_t)a.vocab);
  Red st{-INFINITY, 0x7fffffff, 0.f};
  if (v0 < v1) {
    constexpr int elt = BF16 ? 2 : 4;
    const char* rowp = reinterpret_cast<const char*>(a.logits) + row * a.row_stride * elt;
    constexpr int per = 16 / elt;                   // elements per 16-byte vector
    const int64_t nvec = (v1 - v0) / per;           // full vectors of the slice
    const u32x4* vp = reinterpret_cast<const u32x4*>(rowp + v0 * elt);
    // vectors t, t + 256, ... in order; four loads in flight at a time
    auto fold_vec = [&](const u32x4 u, int64_t i) {
      if constexpr (BF16) {
        float x[8];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          x[2 * w] = __uint_as_float(u[w] << 16);
          x[2 * w + 1] = __uint_as_float(u[w] & 0xffff0000u);
        }
        fold<8>(st, x, (int)(v0 + i * 8));
      } else {
        float x[4] = {__uint_as_float(u[0]), __uint_as_float(u[1]), __uint_as_float(u[2]), __uint_as_float(u[3])};
        fold<4>(st, x, (int)(v0 + i * 4));
      }
    };
    int64_t i = tid;
    // software-pipelined: the next group's four loads are issued before this group is folded
    if (i + 3 * 256 < nvec) {
      u32x4 u[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) u[k] = __builtin_nontemporal_load(vp + i + k * 256);
      for (; i + 7 * 256 < nvec; i += 4 * 256) {
        u32x4 nx[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) nx[k] = __builtin_nontemporal_load(vp + i + (4 + k) * 256);
#pragma unroll
        for (int k = 0; k < 4; ++k) fold_vec(u[k], i + k * 256);
#pragma unroll
        for (int k = 0; k < 4; ++k) u[k] = nx[k];
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) fold_vec(u[k], i + k * 256);
      i += 4 * 256;
    }
    for (; i < nvec; i += 256) fold_vec(__builtin_nontemporal_load(vp + i), i);
    // ragged tail of the slice (vocab not a multiple of the vector width)
    for (int64_t j = v0 + nvec * per + tid; j < v1; j += 256) {
      float x[1] = {load_logit(rowp, BF16, j)};
      Red t{-INFINITY, 0x7fffffff, 0.f};
      fold<1>(t, x, (int)j);
      st = combine(st, t);
    }
  }
  // Thread t saw vectors t, t+256, ...: for equal maxima the lower thread (or the tail, which
  // comes after every full vector) holds the lower index, and combine() takes the minimum.
#pragma unroll
  for (int msk = 1; msk < 64; msk <<= 1) {
    Red o = shfl_xor(st, msk);
    // keep the operand order fixed for determinism: lower lane first
    st = ((threadIdx.x & msk) == 0) ? combine(st, o) : combine(o, st);
  }
  __shared__ Red wred[4];
  if ((tid & 63) == 0) wred[tid >> 6] = st;
  __syncthreads();
  if (tid == 0) {
    Red r = wred[0];
    for (int w = 1; w < 4; ++w) r = combine(r, wred[w]);
    float* out = a.part + ((int64_t)row * a.vsplit + part) * 3;
    out[0] = r.m;
    out[1] = __int_as_float(r.idx);
    out[2] = r.z;
  }
}

// Commit rule of sequence b, executed by one full wave (lane = block position).
__device__ void commit_sequence(const UnmaskArgs& a, int b) {
  const int s = threadIdx.x & 63;
  const bool in = s < a.S;
  const int64_t r = (int64_t)b * a.S + s;
  // the row's slice partials are loaded together with its mask byte (in bounds for every row of
  // the block; an unmasked row's are stale and dropped), so the commit waits for one round trip
  Red st{-INFINITY, 0x7fffffff, 0.f};
  if (in) st = row_partials(a, r);
  const bool masked = in && a.mask[r] != 0;
  float p = 0.f;
  int tok = -1;
  if (masked) {
    p = 1.0f / st.z;
    tok = st.idx;
  }
  if (in) {
    if (a.conf) a.conf[r] = p;
    if (a.argmax) a.argmax[r] = tok;
  }
  const uint64_t any_masked = __ballot(masked);
  bool pass = masked && (a.commit_all || p > a.gamma);
  uint64_t passed = __ballot(pass);
  if (passed == 0 && a.min_commit && any_masked) {
    // most confident masked position; lowest position on ties
    float bp = masked ? p : -1.f;
    int bs = masked ? s : 0x7fffffff;
#pragma unroll
    for (int msk = 1; msk < 64; msk <<= 1) {
      const float op = __shfl_xor(bp, msk, 64);
      const int os = __shfl_xor(bs, msk, 64);
      if (op > bp || (op == bp && os < bs)) {
        bp = op;
        bs = os;
      }
    }
    pass = masked && s == bs;
    passed = __ballot(pass);
  }
  if (pass) {
    a.tokens[r] = tok;
    a.mask[r] = 0;
  }
  if (s == 0) {
    if (a.n_commit) a.n_commit[b] = (int32_t)__popcll(passed);
    if (a.steps_used && any_masked) a.steps_used[b] = a.step + 1;
    if (a.active_next) a.active_next[b] = (any_masked & ~passed) != 0 ? 1 : 0;
  }
}

__global__ __launch_bounds__(64) void commit_kernel(UnmaskArgs a) { commit_sequence(a, blockIdx.x); }

// Self-speculation check of sequence b by one wave (lane = block position): AR's choice for
// position s is first_choice[b] (s = 0) or the argmax of row b*S + s - 1; the committed run is the
// longest prefix of the draft equal to those choices, then AR's choice at the first mismatch.
__global__ __launch_bounds__(64) void spec_accept_kernel(UnmaskArgs a) {
  const int b = blockIdx.x;
  const int s = threadIdx.x & 63;
  const bool in = s < a.S;
  const int64_t r = (int64_t)b * a.S + s;
  // argmax of row r (the choice for position s + 1)
  int choice_next = -1;
  if (in) {
    choice_next = row_partials(a, r).idx;
  }
  // AR's choice for position s: lane s - 1's row argmax, lane 0 takes first_choice[b]
  const int up = __shfl_up(choice_next, 1, 64);
  const int ar = s == 0 ? a.first_choice[b] : up;
  const bool match = in && a.draft[r] == ar;
  const uint64_t miss = __ballot(in && !match);
  const int k = miss ? __builtin_ctzll(miss) : a.S;   // accepted run length
  if (in) a.tokens[r] = s < k ? a.draft[r] : (s == k ? ar : -1);
  if (s == 0) a.n_commit[b] = k < a.S ? k + 1 : a.S;
  if (in && s == a.S - 1) a.next_choice[b] = k == a.S ? choice_next : -1;
}

__global__ __launch_bounds__(64) void loop_init_kernel(const uint8_t* mask, int S, uint8_t* active,
                                                       int32_t* steps_used) {
  const int b = blockIdx.x;
  const int s = threadIdx.x;
  const bool m = s < S && mask[(int64_t)b * S + s] != 0;
  const uint64_t any = __ballot(m);
  if (s == 0) {
    active[b] = any != 0 ? 1 : 0;
    steps_used[b] = 0;
  }
}

}  // namespace

hipError_t unmask_static_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_vocab_reduce(const UnmaskArgs& a, const Launch& l) {
  const int64_t blocks = (int64_t)a.B * a.S * a.vsplit;
  if (a.is_bf16) return launch_kernel(vocab_reduce_kernel<true>, dim3((unsigned)blocks), dim3(256), l, a);
  return launch_kernel(vocab_reduce_kernel<false>, dim3((unsigned)blocks), dim3(256), l, a);
}

hipError_t launch_commit(const UnmaskArgs& a, const Launch& l) {
  return launch_kernel(commit_kernel, dim3((unsigned)a.B), dim3(64), l, a);
}

hipError_t launch_spec_accept(const UnmaskArgs& a, const Launch& l) {
  return launch_kernel(spec_accept_kernel, dim3((unsigned)a.B), dim3(64), l, a);
}

hipError_t launch_loop_init(const uint8_t* mask, int B, int S, uint8_t* active, int32_t* steps_used, const Launch& l) {
  return launch_kernel(loop_init_kernel, dim3((unsigned)B), dim3(64), l, mask, S, active, steps_used);
}

}  // namespace bd
