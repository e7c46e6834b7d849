// Block-local bidirectional Mamba scan (BDLM Mamba-H) on gfx950.
//
// Source: Hybrid Block Diffusion with Partial Bidirectionality summary, technical §Method --
// completed prefix blocks keep only the forward scan's boundary (recurrent) state and the reverse
// scan is confined to the active block, so the cached prefix state depends on the clean prefix
// alone. The recurrence is the Mamba-2 selective scan (the pages print none; see include/bd.h):
// per head h and block position s, with the forward state starting at the cached boundary state,
//   F_s = exp(dt_s A) F_{s-1} + dt_s B_s x_s^T,  R_s = exp(dtr_s A_r) R_{s+1} + dtr_s Br_s xr_s^T,
//   y_s = C_s^T F_s + Cr_s^T R_s + D x_s,  h_out = F_{S-1}.
//
// The kernel evaluates the closed form of these linear recurrences (cum_s = sum_{k<=s} dt_k,
// cr_s = sum_{k<s} dtr_k):
//   y_s   = exp(A cum_s) (C h0)_s + sum_{j<=s} M_sj x_j + sum_{j>=s} Mr_sj xr_j + D x_s,
//   M_sj  = exp(A (cum_s - cum_j)) dt_j (C_s . B_j),   Mr_sj = exp(A_r (cr_j - cr_s)) dtr_j (Cr_s . Br_j),
//   h_out = exp(A cum_{S-1}) h0 + B^T diag(w) X,       w_j = exp(A (cum_{S-1} - cum_j)) dt_j.
// The products with the state run on float32 MFMA (v_mfma_f32_16x16x4_f32) so the cached state is
// never rounded; C . B of two bf16 rows is exact in float32 and runs on bf16 MFMA
// (v_mfma_f32_16x16x32_bf16).
//
// Per head the state is N x 64 float32 (32 KB at N = 128): read once (and written once when the
// block commits), so the pass is HBM-bound on h0 and h_out. One work-group of four waves per
// (sequence, head). Wave w owns the state rows RW w .. RW w + RW - 1 (RW = N / 4) and all 64
// channels: lane (i = l % 16, k = l / 16) loads channels 4 i .. 4 i + 3 of rows RW w + 16 t + 4 k + r
// as float4 (each load instruction covers four whole 256-byte rows), every load issued before the
// first wait. Channel 4 j + c of an MFMA output tile is column j of the c-th of four tiles, so that
// h0, h_out and y keep that float4 layout. C h0 is contracted over the wave's rows and the four
// waves' partial sums meet in LDS.
//
// 16x16x4 float32 MFMA operand layout (lane l, i = l % 16, k = l / 16): A supplies A[i][k], B
// supplies B[k][i], the accumulator holds D[4 k + r][i] in register r. 16x16x32 bf16: A supplies
// A[i][8 k .. 8 k + 7], B supplies B[8 k .. 8 k + 7][i], same accumulator layout.
#include "bd_internal.h"

namespace bd {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4 mfma16(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float bf_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }
// element c (0..3) of four bf16 packed in two dwords
__device__ __forceinline__ float bf4(uint2 v, int c) {
  const uint32_t w = c < 2 ? v.x : v.y;
  return (c & 1) ? bf_hi(w) : bf_lo(w);
}

template <int N, int SP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(SP == 16 ? 4 : 2))) void mamba_block_kernel(MambaArgs a) {
  constexpr int P = 64;
  constexpr int RW = N / 4;     // state rows per wave
  constexpr int TW = RW / 16;   // 16-row tiles per wave
  constexpr int ST = SP / 16;   // 16-row tiles of the block
  constexpr int K4 = SP / 4;    // 4-position steps of the block
  constexpr int LB = N + 8;     // LDS row pitch of B and C (bf16; 16-byte rows, banks spread)
  constexpr int LT = P + 4;     // LDS row pitch of the partial outputs (floats)
  constexpr int BC_BYTES = 4 * SP * LB * 2;
  constexpr int T_BYTES = 4 * SP * LT * 4;
  // B and C (forward B, forward C, reverse B, reverse C; rows >= S zero) until the last reader is
  // done, then the four waves' partial outputs
  __shared__ __align__(16) char sbuf[BC_BYTES > T_BYTES ? BC_BYTES : T_BYTES];
  __shared__ float sM[2][SP][SP + 1];   // forward M, reverse Mr
  __shared__ float sw[SP], sdec[SP], sdt[2][SP], scum[2][SP];
  __shared__ float sdec_last;
  uint16_t(*sBC)[SP][LB] = reinterpret_cast<uint16_t(*)[SP][LB]>(sbuf);
  float(*sT)[SP][LT] = reinterpret_cast<float(*)[SP][LT]>(sbuf);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int li = lane & 15, lk = lane >> 4;
  const int bh = (int)xcd_local_item(blockIdx.x, gridDim.x);   // the heads of a B/C group share an L2
  const int h = bh % a.H;
  int b = bh / a.H;
  if (a.active && a.B <= 64) {
    // the (bh / H)-th active sequence (one ballot per wave), so that the busy work-groups are the
    // first ones of the grid and spread over every XCD whichever sequences have retired
    const int ln = tid & 63;
    uint64_t bits = __builtin_amdgcn_ballot_w64(ln < a.B && a.active[min(ln, a.B - 1)] != 0);
    if (__popcll(bits) <= b) return;   // uniform
    for (int q = b; q > 0; --q) bits &= bits - 1;   // drop the lower set bits
    b = __builtin_ctzll(bits);
  } else if (a.active && !a.active[b]) {
    return;   // uniform per work-group
  }
  const int g = (int)(((int64_t)h * a.G) / a.H);
  const int S = a.S;
  const int64_t row0 = (int64_t)b * S;   // (b, s = 0) row of the [B, S, ...] inputs

  // ---- every global load first, unconditionally (positions >= S read row S - 1 and are zeroed
  // afterwards, so that no load sits in a branch): B and C, step sizes, x of both directions, the
  // state
  constexpr int NBC = 4 * SP * N / 8;   // 16-byte chunks of B and C, a multiple of 256
  static_assert(NBC % 256 == 0, "B and C chunks must split evenly over the work-group");
  uint4 bc[NBC / 256];
#pragma unroll
  for (int i = 0; i < NBC / 256; ++i) {
    const int e = tid + 256 * i;
    const int t = e / (SP * N / 8), s = (e / (N / 8)) % SP, c8 = e % (N / 8);
    const uint16_t* src = t == 0 ? a.Bm : t == 1 ? a.Cm : t == 2 ? a.Bm_r : a.Cm_r;
    bc[i] = *reinterpret_cast<const uint4*>(src + ((row0 + min(s, S - 1)) * a.G + g) * N + 8 * c8);
  }
  const float dtv_raw = (lane < 32 ? a.dt : a.dt_r)[(row0 + min(lane & 31, S - 1)) * a.H + h];
  uint2 xv[2][K4];   // xv[d][k4] = x_d[4 k4 + k][4 i .. 4 i + 3] (bf16)
#pragma unroll
  for (int d = 0; d < 2; ++d)
#pragma unroll
    for (int k4 = 0; k4 < K4; ++k4)
      xv[d][k4] = *reinterpret_cast<const uint2*>((d ? a.x_r : a.x) + ((row0 + min(4 * k4 + lk, S - 1)) * a.H + h) * P +
                                                  4 * li);
  const float* h0 = a.h0 + ((int64_t)b * a.H + h) * N * P;
  f32x4 hv[TW][4];   // hv[t][r] = h0[RW w + 16 t + 4 k + r][4 i .. 4 i + 3]
#pragma unroll
  for (int t = 0; t < TW; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      hv[t][r] = *reinterpret_cast<const f32x4*>(h0 + (RW * wave + 16 * t + 4 * lk + r) * P + 4 * li);

  // ---- B and C into LDS; prefix sums of the step sizes (wave 0: lanes 0..31 forward, 32..63 reverse)
#pragma unroll
  for (int i = 0; i < NBC / 256; ++i) {
    const int e = tid + 256 * i;
    const int t = e / (SP * N / 8), s = (e / (N / 8)) % SP, c8 = e % (N / 8);
    *reinterpret_cast<uint4*>(&sBC[t][s][8 * c8]) = s < S ? bc[i] : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int d = 0; d < 2; ++d)
#pragma unroll
    for (int k4 = 0; k4 < K4; ++k4)
      if (4 * k4 + lk >= S) xv[d][k4] = make_uint2(0, 0);
  const float A = a.A[h], Ar = a.A_r[h];
  if (wave == 0) {
    const int s = lane & 31;
    const float dtv = s < S ? dtv_raw : 0.f;
    float inc = dtv;
#pragma unroll
    for (int d = 1; d < 32; d <<= 1) {
      const float o = __shfl_up(inc, d, 32);
      if (s >= d) inc += o;
    }
    const float last = __shfl(inc, S - 1, 32);   // forward: cum_{S-1}
    if (s < SP) {
      if (lane < 32) {
        sdt[0][s] = dtv;
        scum[0][s] = inc;
        sw[s] = s < S ? expf(A * (last - inc)) * dtv : 0.f;
        sdec[s] = expf(A * inc);
        if (s == 0) sdec_last = expf(A * last);
      } else {
        sdt[1][s] = dtv;
        scum[1][s] = inc - dtv;   // exclusive
      }
    }
  }
  __syncthreads();

  // ---- G = C B^T (forward) and Gr = Cr Br^T (reverse), masked and scaled into M and Mr
  for (int job = wave; job < 2 * ST * ST; job += 4) {
    const int dir = job / (ST * ST), ti = (job / ST) % ST, tj = job % ST;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k0 = 0; k0 < N; k0 += 32)
      acc = mfma16_bf16(*reinterpret_cast<const bf16x8*>(&sBC[2 * dir + 1][16 * ti + li][k0 + 8 * lk]),
                        *reinterpret_cast<const bf16x8*>(&sBC[2 * dir][16 * tj + li][k0 + 8 * lk]), acc);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int s = 16 * ti + 4 * lk + r, j = 16 * tj + li;
      float m = 0.f;
      if (s < S && j < S) {
        if (dir == 0 && j <= s) m = expf(A * (scum[0][s] - scum[0][j])) * sdt[0][j] * acc[r];
        if (dir == 1 && j >= s) m = expf(Ar * (scum[1][j] - scum[1][s])) * sdt[1][j] * acc[r];
      }
      sM[dir][s][j] = m;
    }
  }

  // ---- this wave's share of exp(A cum_s) (C h0)_s: channel tiles c = 0..3, rows RW w .. RW w + RW - 1
  f32x4 acc[ST][4];
#pragma unroll
  for (int st = 0; st < ST; ++st) {
    const float dec = sdec[16 * st + li];
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[st][c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < TW; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float cv = dec * __uint_as_float((uint32_t)sBC[1][16 * st + li][RW * wave + 16 * t + 4 * lk + r] << 16);
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[st][c] = mfma16(cv, hv[t][r][c], acc[st][c]);
      }
  }

  // ---- the new boundary state: exp(A cum_{S-1}) h0 + B^T diag(w) X, rows of this wave
  if (a.h_out) {
    float* ho = a.h_out + ((int64_t)b * a.H + h) * N * P;
    const float dl = sdec_last;
#pragma unroll
    for (int t = 0; t < TW; ++t) {
      f32x4 hn[4];
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) hn[c][r] = hv[t][r][c] * dl;
#pragma unroll
      for (int k4 = 0; k4 < K4; ++k4) {
        const int k = 4 * k4 + lk;
        const float bw = sw[k] * __uint_as_float((uint32_t)sBC[0][k][RW * wave + 16 * t + li] << 16);
#pragma unroll
        for (int c = 0; c < 4; ++c) hn[c] = mfma16(bw, bf4(xv[0][k4], c), hn[c]);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r)
        *reinterpret_cast<f32x4*>(ho + (RW * wave + 16 * t + 4 * lk + r) * P + 4 * li) =
            f32x4{hn[0][r], hn[1][r], hn[2][r], hn[3][r]};
    }
  }
  __syncthreads();   // M and Mr complete; B and C no longer read

  // ---- intra-block terms of channel tile c = wave, added to this wave's partial sums
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    if (c != wave) continue;
#pragma unroll
    for (int st = 0; st < ST; ++st)
#pragma unroll
      for (int d = 0; d < 2; ++d)
#pragma unroll
        for (int k4 = 0; k4 < K4; ++k4)
          acc[st][c] = mfma16(sM[d][16 * st + li][4 * k4 + lk], bf4(xv[d][k4], c), acc[st][c]);
  }
#pragma unroll
  for (int st = 0; st < ST; ++st)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      *reinterpret_cast<f32x4*>(&sT[wave][16 * st + 4 * lk + r][4 * li]) =
          f32x4{acc[st][0][r], acc[st][1][r], acc[st][2][r], acc[st][3][r]};
  __syncthreads();

  // ---- y = the four partial sums + D x; wave w writes positions 4 k4 + k for k4 = w mod 4
  const float Dh = a.D[h];
#pragma unroll
  for (int k4 = 0; k4 < K4; ++k4) {
    if ((k4 & 3) != wave) continue;
    const int s = 4 * k4 + lk;
    if (s >= S) continue;
    f32x4 v = *reinterpret_cast<const f32x4*>(&sT[0][s][4 * li]);
#pragma unroll
    for (int w = 1; w < 4; ++w) v += *reinterpret_cast<const f32x4*>(&sT[w][s][4 * li]);
    uint32_t o[2];
#pragma unroll
    for (int c = 0; c < 4; c += 2) {
      const float v0 = v[c] + Dh * bf4(xv[0][k4], c), v1 = v[c + 1] + Dh * bf4(xv[0][k4], c + 1);
      o[c / 2] = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v0) |
                 ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v1) << 16);
    }
    *reinterpret_cast<uint2*>(a.y + ((row0 + s) * a.H + h) * P + 4 * li) = make_uint2(o[0], o[1]);
  }
}

}  // namespace

hipError_t launch_mamba_block(const MambaArgs& a, const Launch& l) {
  const dim3 grid((unsigned)((int64_t)a.B * a.H));
  const int key = a.N * 100 + (a.S <= 16 ? 16 : 32);
  switch (key) {
    case 12816: return launch_kernel(mamba_block_kernel<128, 16>, grid, dim3(256), l, a);
    case 12832: return launch_kernel(mamba_block_kernel<128, 32>, grid, dim3(256), l, a);
    case 6416: return launch_kernel(mamba_block_kernel<64, 16>, grid, dim3(256), l, a);
    case 6432: return launch_kernel(mamba_block_kernel<64, 32>, grid, dim3(256), l, a);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace bd
