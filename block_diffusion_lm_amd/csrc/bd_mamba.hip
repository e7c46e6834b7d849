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
//   h_out = exp(A cum_{S-1}) h0 + B^T diag(w) X,       w_j = exp(A (cum_{S-1} - cum_j)) dt_j,
// every product on float32 MFMA (v_mfma_f32_16x16x4_f32) so the cached state is never rounded.
// One work-group of four waves per (sequence, head); wave w owns channels 16 w .. 16 w + 15.
// Per head the state is N x 64 float32 (32 KB at N = 128), read once and written once: the pass
// is HBM-bound on h0 and h_out.
//
// 16x16x4 float32 MFMA operand layout (lane l, i = l % 16, k = l / 16): A supplies A[i][k], B
// supplies B[k][i], the accumulator holds D[4 k + r][i] in register r. The contraction index of
// C h0 is taken in the order the accumulator layout of h0 provides (k = 4 (l / 16) + m at step m),
// so h0 is loaded once, in that layout, for both of its uses.
#include "bd_internal.h"

namespace bd {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float bf(const uint16_t* p, int64_t i) { return __uint_as_float((uint32_t)p[i] << 16); }

template <int N, int SP>
__global__ __launch_bounds__(256) void mamba_block_kernel(MambaArgs a) {
  constexpr int P = 64;
  constexpr int NT = N / 16;   // 16-row tiles of the state
  constexpr int ST = SP / 16;  // 16-row tiles of the block
  constexpr int LDR = N + 1;   // LDS row pitch of B and C (floats)
  __shared__ float sBC[4][SP][LDR];     // forward B, forward C, reverse B, reverse C (rows >= S zero)
  __shared__ float sM[2][SP][SP + 1];   // forward M, reverse Mr
  __shared__ float sdt[2][SP], scum[2][SP];
  __shared__ float sw[SP], sdec[SP];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int li = lane & 15, lk = lane >> 4;
  const int bh = blockIdx.x;
  const int b = bh / a.H, h = bh % a.H;
  if (a.active && !a.active[b]) return;   // uniform per work-group
  const int g = (int)(((int64_t)h * a.G) / a.H);
  const int S = a.S;

  // ---- step sizes and their prefix sums; B and C of group g into LDS as float32
  if (tid < 2 * SP) {
    const int dir = tid / SP, s = tid % SP;
    const float* dtp = dir ? a.dt_r : a.dt;
    sdt[dir][s] = s < S ? dtp[((int64_t)b * S + s) * a.H + h] : 0.f;
  }
  {
    const uint16_t* src[4] = {a.Bm, a.Cm, a.Bm_r, a.Cm_r};
    for (int e = tid; e < 4 * SP * N; e += 256) {
      const int t = e / (SP * N), s = (e / N) % SP, n = e % N;
      sBC[t][s][n] = s < S ? bf(src[t], (((int64_t)b * S + s) * a.G + g) * N + n) : 0.f;
    }
  }
  __syncthreads();
  if (tid < 2) {
    // forward: inclusive sums; reverse: exclusive sums (cr_s = sum_{k<s} dtr_k)
    float c = 0.f;
    for (int s = 0; s < SP; ++s) {
      if (tid == 0) { c += sdt[0][s]; scum[0][s] = c; }
      else { scum[1][s] = c; c += sdt[1][s]; }
    }
  }
  __syncthreads();
  const float A = a.A[h], Ar = a.A_r[h];
  const float cum_last = scum[0][S - 1];
  if (tid < SP) {
    const int s = tid;
    sw[s] = s < S ? expf(A * (cum_last - scum[0][s])) * sdt[0][s] : 0.f;
    sdec[s] = expf(A * scum[0][s]);
  }

  // ---- G = C B^T (forward) and Gr = Cr Br^T (reverse), masked and scaled into M and Mr
  for (int job = wave; job < 2 * ST * ST; job += 4) {
    const int dir = job / (ST * ST), ti = (job / ST) % ST, tj = job % ST;
    const float(*Cq)[LDR] = sBC[2 * dir + 1];
    const float(*Bq)[LDR] = sBC[2 * dir];
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int k0 = 0; k0 < N; k0 += 4)
      acc = mfma16(Cq[16 * ti + li][k0 + lk], Bq[16 * tj + li][k0 + lk], acc);
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
  __syncthreads();

  // ---- per wave: channels p0 .. p0 + 15
  const int p0 = 16 * wave;
  const int p = p0 + li;
  const float* h0 = a.h0 + ((int64_t)b * a.H + h) * N * P;
  f32x4 hs[NT];   // h0 in accumulator layout: hs[nt][r] = h0[16 nt + 4 lk + r][p]
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int r = 0; r < 4; ++r) hs[nt][r] = h0[(16 * nt + 4 * lk + r) * P + p];
  // x and xr at the B-operand positions: xs[d][k4] = x[4 k4 + lk][p]
  float xs[2][SP / 4];
#pragma unroll
  for (int d = 0; d < 2; ++d) {
    const uint16_t* xp = d ? a.x_r : a.x;
#pragma unroll
    for (int k4 = 0; k4 < SP / 4; ++k4) {
      const int s = 4 * k4 + lk;
      xs[d][k4] = s < S ? bf(xp, (((int64_t)b * S + s) * a.H + h) * P + p) : 0.f;
    }
  }
  // y tiles: C h0 (scaled per row afterwards) and the intra-block terms
#pragma unroll
  for (int st = 0; st < ST; ++st) {
    f32x4 t1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int m = 0; m < 4; ++m) t1 = mfma16(sBC[1][16 * st + li][16 * nt + 4 * lk + m], hs[nt][m], t1);
    f32x4 yi = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int d = 0; d < 2; ++d)
#pragma unroll
      for (int k4 = 0; k4 < SP / 4; ++k4) yi = mfma16(sM[d][16 * st + li][4 * k4 + lk], xs[d][k4], yi);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int s = 16 * st + 4 * lk + r;
      if (s < S) {
        const int64_t o = (((int64_t)b * S + s) * a.H + h) * P + p;
        const float v = sdec[s] * t1[r] + yi[r] + a.D[h] * bf(a.x, o);
        a.y[o] = __builtin_bit_cast(uint16_t, (__bf16)v);
      }
    }
  }
  // the new boundary state: exp(A cum_{S-1}) h0 + B^T diag(w) X
  if (a.h_out) {
    const float dec = expf(A * cum_last);
    float* ho = a.h_out + ((int64_t)b * a.H + h) * N * P;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      f32x4 acc = hs[nt] * dec;
#pragma unroll
      for (int k4 = 0; k4 < SP / 4; ++k4) {
        const int k = 4 * k4 + lk;
        acc = mfma16(sw[k] * sBC[0][k][16 * nt + li], xs[0][k4], acc);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) ho[(16 * nt + 4 * lk + r) * P + p] = acc[r];
    }
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
