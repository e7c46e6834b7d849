// Attention of the active block over [prefix cache ; block] on gfx950.
//
// Source: Nemotron-TwoTower technical summary, §Architecture and §Generation -- at every layer
// the denoiser attends to the frozen context tower's KV cache of past blocks (causal
// cross-attention: the whole prefix precedes the block, so all of it is visible) and
// bidirectionally to the current block's own keys and values. One softmax covers both.
//
// Work decomposition. For sequence b and KV head g the R = S * (Hq/Hkv) query rows of the
// group share one key sequence: the prefix_len[b] cached keys followed by the S block keys.
// That sequence is cut into chunks; a workgroup owns one (sequence, KV head, chunk, row tile)
// item. Each wave holds 32*RB query rows in registers (RB 32-row MFMA blocks) and streams the
// chunk's keys through LDS in tiles of 64 keys, double-buffered, the next tile's global loads
// in flight while the current one is consumed.
//
// The host plans chunks for the whole batch; when only some sequences are still active (the
// denoise loop retires sequences as their blocks complete) the kernels re-plan on the device:
// the same grid is spread over the active sequences only, with proportionally shorter chunks,
// so a partly retired batch still occupies every compute unit.
//
// MFMA formulation (v_mfma_f32_32x32x16_bf16). Scores are computed transposed,
// S^T = K Q^T (A = 32 keys x 16 dims from LDS, B = Q^T held in registers), so that every lane
// owns the scores of ONE query row (lane % 32) for 16 of each 32 keys; the other 16 keys of
// that row sit in lane ^ 32. Row max needs one cross-half swap, row sums none until the end.
// The output is also accumulated transposed, O^T += V^T P^T (A = V^T from LDS, B = P^T), whose
// B operand is exactly 8 consecutive accumulator registers of S^T converted to bf16: the key
// order inside each 16-key step is permuted to match, and V is stored transposed in LDS in the
// same permuted order, with an XOR swizzle of its 16-byte chunks that keeps both the
// transposing writes and the operand reads free of bank conflicts.
//
// Softmax: online (running max m, running sum l) in log2 units, exp2 in float32, P rounded to
// bf16 for the P V product; l sums the same bf16-rounded P (v_dot2), so numerator and
// denominator use identical weights. The running max is only raised when a tile's maximum
// exceeds it by more than 8 (log2 units); probabilities relative to a stale max stay below
// 2^8, which fp32 and bf16 hold exactly as well, so the result is unchanged while rescaling of
// the output accumulators becomes rare.
#include "bd_internal.h"

namespace bd {
namespace {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((__vector_size__(4 * sizeof(__bf16))));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazyRescale = 8.0f;
constexpr int kPrioMode = 0;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float other_half(float x) {
  // value of the same register in lane ^ 32
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

__device__ __forceinline__ u32x4 ldg16(const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); }

// Device-side plan of one launch: which (sequence, KV head, chunk, row tile) a workgroup owns.
// With every sequence active this is the host plan. With n_act < B active sequences the same
// number of workgroups is spread over the active ones: splits per (sequence, KV head) grow to
// floor(nsplit * B / n_act) (chunks shrink accordingly, never below one key tile).
struct ItemMap {
  int nsplit;       // splits per (sequence, KV head) in this launch
  int64_t chunk;    // keys per split
};

__device__ __forceinline__ ItemMap device_plan(const AttnArgs& a, int n_act) {
  ItemMap m;
  if (n_act == a.B || n_act == 0 || a.direct) {   // a direct plan has no workspace for partials
    m.nsplit = a.nsplit;
    m.chunk = a.chunk;
    return m;
  }
  const int64_t nkeys = a.max_keys;
  const int64_t ns = ((int64_t)a.nsplit * a.B) / n_act;
  int64_t chunk = (nkeys + ns - 1) / ns;
  chunk = (chunk + 63) / 64 * 64;
  m.chunk = chunk;
  m.nsplit = (int)((nkeys + chunk - 1) / chunk);
  return m;
}

// Number of active sequences, the sequence index of the i-th active one, and the rank of an
// active sequence among them.
__device__ __forceinline__ int count_active(const uint8_t* active, int B) {
  if (!active) return B;
  int n = 0;
  for (int i = 0; i < B; ++i) n += active[i] != 0;
  return n;
}
__device__ __forceinline__ int nth_active(const uint8_t* active, int B, int i) {
  if (!active) return i;
  for (int b = 0; b < B; ++b)
    if (active[b] && i-- == 0) return b;
  return 0;
}
__device__ __forceinline__ int rank_active(const uint8_t* active, int b) {
  if (!active) return b;
  int r = 0;
  for (int i = 0; i < b; ++i) r += active[i] != 0;
  return r;
}

template <int D, int KT_>
struct Geo {
  static constexpr int KT = KT_;                    // keys per LDS tile
  static constexpr int KB = KT / 32;                // 32-key blocks per tile
  static constexpr int KROW = D * 2 + 16;          // bytes per key row of the K tile (padded)
  static constexpr int VROW = KT * 2;               // bytes per dim row of the transposed V tile
  static constexpr int KBYTES = KT * KROW;
  static constexpr int VBYTES = D * VROW;
  static constexpr int BUF = KBYTES + VBYTES;
  static constexpr int KS = D / 16;                 // k-steps of Q K^T
  static constexpr int DB = D / 32;                 // 32-dim blocks of the output
};

// Swizzle of the 16-byte chunks of the transposed V tile: chunk c of dim row d is stored at
// c ^ vt_swz(d). Inside each 16-key step, key 8a+4b+c sits at position 8b+4a+c, so lane half b
// of the P^T operand reads positions 8b..8b+7 as one 16-byte chunk.
__device__ __forceinline__ int vt_swz(int d) { return (d & 7) ^ ((d >> 3) & 7); }

// RB == 1 variants hold half the registers and are meant to run two waves per SIMD.
template <int D, int NW, int RB, int KT>
__global__ __launch_bounds__(NW * 64, (RB == 1 && NW < 8) ? 8 / NW : 1) void attn_split_kernel(AttnArgs a) {
  using G = Geo<D, KT>;
  constexpr int NT = NW * 64;
  constexpr int D8 = D / 8;
  constexpr int ROWS_W = 32 * RB;                    // query rows per wave
  // keys per loading unit: each thread moves UK rows x 8 dims of K and of V per tile
  constexpr int UK = ((G::KT / 4) * D8 >= NT) ? 4 : ((G::KT / 2) * D8 >= NT) ? 2 : 1;
  constexpr int UNITS = (G::KT / UK) * D8;
  constexpr int UPT = UNITS / NT;
  static_assert(UPT >= 1 && UNITS % NT == 0, "tile loading does not divide evenly");

  __shared__ __attribute__((aligned(16))) char smem[2 * G::BUF];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lrow = lane & 31;
  const int half = lane >> 5;

  // ---- work item (XCD-aware: consecutive items land on the same XCD when possible) ----
  const int64_t nitems = (int64_t)gridDim.x;
  int64_t item = blockIdx.x;
  if ((nitems & 7) == 0) item = (item & 7) * (nitems >> 3) + (item >> 3);
  const int n_act = count_active(a.active, a.B);
  const ItemMap im = device_plan(a, n_act);
  const int rt = (int)(item % a.row_tiles);
  const int64_t ps = item / a.row_tiles;
  const int split = (int)(ps % im.nsplit);
  const int64_t pair_a = ps / im.nsplit;              // pair among the active sequences
  if (pair_a >= (int64_t)n_act * a.Hkv) return;
  const int b = nth_active(a.active, a.B, (int)(pair_a / a.Hkv));
  const int g = (int)(pair_a % a.Hkv);
  const int64_t len = a.prefix_len[b];
  const int64_t nkeys = len + a.S;
  const int64_t k_begin = (int64_t)split * im.chunk;
  if (k_begin >= nkeys) return;
  const int64_t k_end = min(k_begin + im.chunk, nkeys);
  const int ntiles = (int)((k_end - k_begin + G::KT - 1) / G::KT);

  const int tile_rows = NW * ROWS_W;
  const int row0 = rt * tile_rows + wave * ROWS_W;    // first query row of this wave
  const bool wave_rows = row0 < a.rows;

  // ---- Q fragments: B operand of S^T = K Q^T (lane: row lrow, dims 8*half .. +7 of a k-step)
  bf16x8 qf[RB][G::KS];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int r = row0 + rb * 32 + lrow;
    if (r < a.rows) {
      const int s = r / a.group;
      const int hq = g * a.group + (r - s * a.group);
      const uint16_t* qp = a.q + (((int64_t)b * a.S + s) * a.Hq + hq) * D + 8 * half;
#pragma unroll
      for (int ks = 0; ks < G::KS; ++ks) qf[rb][ks] = __builtin_bit_cast(bf16x8, ldg16(qp + ks * 16));
    } else {
#pragma unroll
      for (int ks = 0; ks < G::KS; ++ks) qf[rb][ks] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
    }
  }

  const uint16_t* kc = a.k_cache + ((int64_t)b * a.Hkv + g) * a.lcap * D;
  const uint16_t* vc = a.v_cache + ((int64_t)b * a.Hkv + g) * a.lcap * D;
  const int64_t blk_stride = (int64_t)a.Hkv * D;                  // between block positions
  const uint16_t* kb0 = a.k_blk + ((int64_t)b * a.S * a.Hkv + g) * D;
  const uint16_t* vb0 = a.v_blk + ((int64_t)b * a.S * a.Hkv + g) * D;

  // ---- tile loading: registers hold the next tile while the current one is consumed.
  // A tile that lies wholly inside the prefix and the chunk (all but at most two per chunk)
  // is one uniform base pointer plus per-thread constant offsets.
  u32x4 kreg[UK], vreg[UK];
  auto load_unit = [&](int64_t kt0, int i) {
    const int u = tid + NT * i;
    const int d8 = (u % D8) * 8;
    const int kk = (u / D8) * UK;
    if (kt0 + G::KT <= len && kt0 + G::KT <= k_end) {
      const uint16_t* kp = kc + kt0 * D + kk * D + d8;
      const uint16_t* vp = vc + kt0 * D + kk * D + d8;
#pragma unroll
      for (int j = 0; j < UK; ++j) {
        kreg[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kp + j * D));
        vreg[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vp + j * D));
      }
    } else {
#pragma unroll
      for (int j = 0; j < UK; ++j) {
        const int64_t key = kt0 + kk + j;
        if (key < k_end) {
          const uint16_t* kp = key < len ? kc + key * D : kb0 + (key - len) * blk_stride;
          const uint16_t* vp = key < len ? vc + key * D : vb0 + (key - len) * blk_stride;
          kreg[j] = ldg16(kp + d8);
          vreg[j] = ldg16(vp + d8);
        } else {
          kreg[j] = u32x4{0, 0, 0, 0};
          vreg[j] = u32x4{0, 0, 0, 0};
        }
      }
    }
  };
  auto store_unit = [&](char* buf, int i) {
    char* ks = buf;
    char* vt = buf + G::KBYTES;
    const int u = tid + NT * i;
    const int d8 = (u % D8) * 8;
    const int kk = (u / D8) * UK;
#pragma unroll
    for (int j = 0; j < UK; ++j) *reinterpret_cast<u32x4*>(ks + (kk + j) * G::KROW + d8 * 2) = kreg[j];
    // transposed V: dim rows d8 .. d8+7, keys kk .. kk+UK-1 (consecutive positions)
    const int k16 = kk & 15;
    const int a8 = k16 >> 3, b4 = (k16 >> 2) & 1, c = k16 & 3;
    const int chunk = ((kk >> 4) << 1) + b4;              // 16-byte chunk of the position
    const int inchunk = (a8 * 4 + c) * 2;                 // byte offset inside that chunk
#pragma unroll
    for (int w = 0; w < 4; ++w) {
#pragma unroll
      for (int hi = 0; hi < 2; ++hi) {
        const int d = d8 + 2 * w + hi;
        char* dst = vt + d * G::VROW + ((chunk ^ vt_swz(d)) << 4) + inchunk;
        if constexpr (UK == 4) {
          const uint32_t x0 = vreg[0][w], x1 = vreg[1][w], x2 = vreg[2][w], x3 = vreg[3][w];
          u32x2 v;
          if (hi == 0) {
            v[0] = (x0 & 0xffffu) | (x1 << 16);
            v[1] = (x2 & 0xffffu) | (x3 << 16);
          } else {
            v[0] = (x0 >> 16) | (x1 & 0xffff0000u);
            v[1] = (x2 >> 16) | (x3 & 0xffff0000u);
          }
          *reinterpret_cast<u32x2*>(dst) = v;
        } else if constexpr (UK == 2) {
          const uint32_t x0 = vreg[0][w], x1 = vreg[1][w];
          *reinterpret_cast<uint32_t*>(dst) = hi == 0 ? ((x0 & 0xffffu) | (x1 << 16)) : ((x0 >> 16) | (x1 & 0xffff0000u));
        } else {
          const uint32_t x0 = vreg[0][w];
          *reinterpret_cast<uint16_t*>(dst) = (uint16_t)(hi == 0 ? (x0 & 0xffffu) : (x0 >> 16));
        }
      }
    }
  };

  float m_run[RB], l_run[RB];        // running max (log2 units) and this lane's share of the sum
  f32x16 o[G::DB][RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m_run[rb] = -INFINITY;
    l_run[rb] = 0.f;
#pragma unroll
    for (int db = 0; db < G::DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][rb][r] = 0.f;
  }
  const float sc = a.scale_log2;
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  if constexpr (kPrioMode == 1) {
    if (wave >= NW / 2) __builtin_amdgcn_s_setprio(1);
  }

  // With few threads per workgroup a tile is too many registers to hold in flight: those
  // variants load and store a tile right before consuming it.
  constexpr bool kPrefetch = UPT <= 1;
  if (kPrefetch) load_unit(k_begin, 0);
  for (int t = 0; t < ntiles; ++t) {
    char* buf = smem + (t & 1) * G::BUF;
    const int64_t kt0 = k_begin + (int64_t)t * G::KT;
    if (kPrefetch) {
      store_unit(buf, 0);
    } else {
      for (int i = 0; i < UPT; ++i) {
        load_unit(kt0, i);
        store_unit(buf, i);
      }
    }
    __syncthreads();
    if (kPrefetch && t + 1 < ntiles) load_unit(kt0 + G::KT, 0);
    if (!wave_rows) continue;

    const char* ks = buf;
    const char* vt = buf + G::KBYTES;
    const int valid = (int)min((int64_t)G::KT, k_end - kt0);   // keys of this tile inside the chunk

#pragma unroll
    for (int kb = 0; kb < G::KB; ++kb) {
      if (kb * 32 >= valid) break;
      // ---- S^T = K Q^T for 32 keys: sacc[rb], 32 keys x 32 rows each
      if constexpr (kPrioMode == 2) __builtin_amdgcn_s_setprio(1);
      f32x16 sacc[RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[rb][r] = 0.f;
#pragma unroll
      for (int kstep = 0; kstep < G::KS; ++kstep) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(ks + (kb * 32 + lrow) * G::KROW + (kstep * 16 + 8 * half) * 2);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) sacc[rb] = mfma32(kf, qf[rb][kstep], sacc[rb]);
      }
      if (kb * 32 + 32 > valid) {   // keys past the chunk end do not exist for this item
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          if (key >= valid)
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) sacc[rb][r] = -INFINITY;
        }
      }
      if constexpr (kPrioMode == 2) __builtin_amdgcn_s_setprio(0);
      // ---- running max: one (rarely taken) rescale branch per 32 keys
      float mx[RB];
      bool raise_any = false;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        float v = sacc[rb][0];
#pragma unroll
        for (int r = 1; r < 16; ++r) v = fmaxf(v, sacc[rb][r]);
        mx[rb] = fmaxf(v, other_half(v)) * sc;
        raise_any |= mx[rb] > m_run[rb] + kLazyRescale;
      }
      if (__builtin_amdgcn_ballot_w64(raise_any)) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const float mnew = mx[rb] > m_run[rb] + kLazyRescale ? mx[rb] : m_run[rb];
          const float alpha = __builtin_amdgcn_exp2f(m_run[rb] - mnew);   // exp2(-inf) = 0
          l_run[rb] *= alpha;
#pragma unroll
          for (int db = 0; db < G::DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[db][rb][r] *= alpha;
          m_run[rb] = mnew;
        }
      }
      // ---- P = exp2(s*sc - m) in bf16, row sums of the rounded P, O^T += V^T P^T
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        bf16x8 pf[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const float mneg = -m_run[rb];
#pragma unroll
          for (int i = 0; i < 8; ++i) pf[rb][i] = (__bf16)__builtin_amdgcn_exp2f(fmaf(sacc[rb][8 * e + i], sc, mneg));
          float ls = l_run[rb];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const bf16x2 p2 = {pf[rb][2 * i], pf[rb][2 * i + 1]};
            ls = __builtin_amdgcn_fdot2_f32_bf16(p2, ones, ls, false);
          }
          l_run[rb] = ls;
        }
        const int chunk = (kb * 2 + e) * 2 + half;
#pragma unroll
        for (int db = 0; db < G::DB; ++db) {
          const int d = db * 32 + lrow;
          const bf16x8 vf = *reinterpret_cast<const bf16x8*>(vt + d * G::VROW + ((chunk ^ vt_swz(d)) << 4));
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) o[db][rb] = mfma32(vf, pf[rb], o[db][rb]);
        }
      }
    }
  }
  if (!wave_rows) return;

  // ---- epilogue: lane owns row lrow of each row block; dims db*32 + 8*(r/4) + 4*half + r%4
  const int64_t item_act = (pair_a * im.nsplit + split) * a.row_tiles + rt;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const float l_tot = l_run[rb] + other_half(l_run[rb]);
    const int r = row0 + rb * 32 + lrow;
    if (r >= a.rows) continue;
    const int s = r / a.group;
    const int hq = g * a.group + (r - s * a.group);
    if (im.nsplit == 1) {
      const float inv = 1.0f / l_tot;
      uint16_t* op = a.out + (((int64_t)b * a.S + s) * a.Hq + hq) * D;
#pragma unroll
      for (int db = 0; db < G::DB; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int d = db * 32 + 8 * q4 + 4 * half;
          bf16x4 v;
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = (__bf16)(o[db][rb][4 * q4 + i] * inv);
          *reinterpret_cast<bf16x4*>(op + d) = v;
        }
      if (a.lse && half == 0) a.lse[((int64_t)b * a.Hq + hq) * a.S + s] = (m_run[rb] + log2f(l_tot)) * kLn2;
    } else {
      // partial (m, l, acc) of this chunk; merged by the merge kernels
      const int64_t prow = item_act * tile_rows + (r - rt * tile_rows);
      float* ap = a.part_acc + prow * D;
#pragma unroll
      for (int db = 0; db < G::DB; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int d = db * 32 + 8 * q4 + 4 * half;
          const f32x4 v = {o[db][rb][4 * q4], o[db][rb][4 * q4 + 1], o[db][rb][4 * q4 + 2], o[db][rb][4 * q4 + 3]};
          *reinterpret_cast<f32x4*>(ap + d) = v;
        }
      if (half == 0) {
        a.part_ml[prow * 2] = m_run[rb];
        a.part_ml[prow * 2 + 1] = l_tot;
      }
    }
  }
}

// Merge of the chunk partials of every (sequence, KV head, query row): with M = max_c m_c,
//   O = sum_c acc_c 2^(m_c - M) / sum_c l_c 2^(m_c - M),  LSE = (M + log2 sum_c l_c 2^(m_c - M)) ln 2,
// chunks combined in index order.
//
// Narrow form (few chunks): one thread per (row, 4 dims), the chunk loop unrolled so several
// partial loads are in flight per thread.
template <int D>
__global__ __launch_bounds__(256) void attn_merge_narrow_kernel(AttnArgs a, int tile_rows) {
  constexpr int DG = D / 4;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)a.B * a.Hkv * a.rows * DG;
  if (gid >= total) return;
  const int dg = (int)(gid % DG);
  const int64_t rowg = gid / DG;
  const int r = (int)(rowg % a.rows);
  const int pair = (int)(rowg / a.rows);
  const int b = pair / a.Hkv;
  const int g = pair % a.Hkv;
  if (a.active && !a.active[b]) return;
  const int n_act = count_active(a.active, a.B);
  const ItemMap im = device_plan(a, n_act);
  if (im.nsplit == 1) return;   // the split kernel wrote the output itself
  const int64_t pair_a = (int64_t)rank_active(a.active, b) * a.Hkv + g;
  const int64_t nkeys = (int64_t)a.prefix_len[b] + a.S;
  const int ns = (int)min((int64_t)im.nsplit, (nkeys + im.chunk - 1) / im.chunk);
  const int rt = r / tile_rows;
  const int rr = r - rt * tile_rows;
  const int64_t pstride = (int64_t)a.row_tiles * tile_rows;     // partial rows between chunks
  const int64_t p0 = ((pair_a * im.nsplit) * a.row_tiles + rt) * tile_rows + rr;
  float M = -INFINITY;
  for (int c = 0; c < ns; ++c) M = fmaxf(M, a.part_ml[(p0 + c * pstride) * 2]);
  f32x4 num = {0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  int c = 0;
  for (; c + 4 <= ns; c += 4) {
    f32x4 v[4];
    float mm[4], ll[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t pr = p0 + (c + j) * pstride;
      mm[j] = a.part_ml[pr * 2];
      ll[j] = a.part_ml[pr * 2 + 1];
      v[j] = *reinterpret_cast<const f32x4*>(a.part_acc + pr * D + dg * 4);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float w = __builtin_amdgcn_exp2f(mm[j] - M);
      den += ll[j] * w;
      num += v[j] * w;
    }
  }
  for (; c < ns; ++c) {
    const int64_t pr = p0 + c * pstride;
    const float w = __builtin_amdgcn_exp2f(a.part_ml[pr * 2] - M);
    den += a.part_ml[pr * 2 + 1] * w;
    num += *reinterpret_cast<const f32x4*>(a.part_acc + pr * D + dg * 4) * w;
  }
  const float inv = 1.0f / den;
  const int s = r / a.group;
  const int hq = g * a.group + (r - s * a.group);
  bf16x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = (__bf16)(num[i] * inv);
  *reinterpret_cast<bf16x4*>(a.out + (((int64_t)b * a.S + s) * a.Hq + hq) * D + dg * 4) = o;
  if (a.lse && dg == 0) a.lse[((int64_t)b * a.Hq + hq) * a.S + s] = (M + log2f(den)) * kLn2;
}

// Wide form (many chunks): one workgroup per query row: 256 threads = (D/4 groups of 4 dims) x (256/(D/4) split groups);
// split group j sums chunks j, j + SG, ... in order, then the groups are added in index order
// through LDS, so the result does not depend on scheduling.
template <int D>
__global__ __launch_bounds__(256) void attn_merge_wide_kernel(AttnArgs a, int tile_rows) {
  constexpr int DG = D / 4;
  constexpr int SG = 256 / DG;
  __shared__ float red_m[256];
  __shared__ f32x4 red_num[256];
  __shared__ float red_den[256];
  const int tid = threadIdx.x;
  const int64_t rowg = blockIdx.x;
  const int r = (int)(rowg % a.rows);
  const int pair = (int)(rowg / a.rows);
  const int b = pair / a.Hkv;
  const int g = pair % a.Hkv;
  if (a.active && !a.active[b]) return;
  const int n_act = count_active(a.active, a.B);
  const ItemMap im = device_plan(a, n_act);
  if (im.nsplit == 1) return;   // the split kernel wrote the output itself
  const int64_t pair_a = (int64_t)rank_active(a.active, b) * a.Hkv + g;
  const int64_t nkeys = (int64_t)a.prefix_len[b] + a.S;
  const int ns = (int)min((int64_t)im.nsplit, (nkeys + im.chunk - 1) / im.chunk);
  const int rt = r / tile_rows;
  const int rr = r - rt * tile_rows;
  const int64_t pstride = (int64_t)a.row_tiles * tile_rows;     // partial rows between chunks
  const int64_t p0 = ((pair_a * im.nsplit) * a.row_tiles + rt) * tile_rows + rr;
  // M = max over chunks
  float mloc = -INFINITY;
  for (int c = tid; c < ns; c += 256) mloc = fmaxf(mloc, a.part_ml[(p0 + c * pstride) * 2]);
  red_m[tid] = mloc;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) red_m[tid] = fmaxf(red_m[tid], red_m[tid + w]);
    __syncthreads();
  }
  const float M = red_m[0];
  const int dg = tid % DG;
  const int sg = tid / DG;
  f32x4 num = {0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  for (int c = sg; c < ns; c += SG) {
    const int64_t pr = p0 + c * pstride;
    const float w = __builtin_amdgcn_exp2f(a.part_ml[pr * 2] - M);
    den += a.part_ml[pr * 2 + 1] * w;
    num += *reinterpret_cast<const f32x4*>(a.part_acc + pr * D + dg * 4) * w;
  }
  red_num[tid] = num;
  red_den[tid] = den;
  __syncthreads();
  if (sg != 0) return;
  for (int j = 1; j < SG; ++j) {
    num += red_num[j * DG + dg];
    den += red_den[j * DG + dg];
  }
  const float inv = 1.0f / den;
  const int s = r / a.group;
  const int hq = g * a.group + (r - s * a.group);
  bf16x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = (__bf16)(num[i] * inv);
  *reinterpret_cast<bf16x4*>(a.out + (((int64_t)b * a.S + s) * a.Hq + hq) * D + dg * 4) = o;
  if (a.lse && dg == 0) a.lse[((int64_t)b * a.Hq + hq) * a.S + s] = (M + log2f(den)) * kLn2;
}

template <int D, int NW, int RB>
hipError_t launch_split_t(const AttnPlan& plan, const AttnArgs& a, hipStream_t stream) {
  if (plan.key_tile == 128)
    hipLaunchKernelGGL((attn_split_kernel<D, NW, RB, 128>), dim3((unsigned)plan.n_items), dim3(NW * 64), 0, stream, a);
  else
    hipLaunchKernelGGL((attn_split_kernel<D, NW, RB, 64>), dim3((unsigned)plan.n_items), dim3(NW * 64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_split(const AttnPlan& plan, const AttnArgs& a, hipStream_t stream) {
  const int key = plan.waves * 100 + plan.rows_per_wave;
  if (plan.head_dim == 128) {
    switch (key) {
      case 464: return launch_split_t<128, 4, 2>(plan, a, stream);
      case 432: return launch_split_t<128, 4, 1>(plan, a, stream);
      case 832: return launch_split_t<128, 8, 1>(plan, a, stream);
    }
  } else if (plan.head_dim == 64) {
    switch (key) {
      case 464: return launch_split_t<64, 4, 2>(plan, a, stream);
      case 432: return launch_split_t<64, 4, 1>(plan, a, stream);
      case 832: return launch_split_t<64, 8, 1>(plan, a, stream);
    }
  }
  return hipErrorInvalidValue;
}

hipError_t launch_attn_merge(const AttnPlan& plan, const AttnArgs& a, hipStream_t stream) {
  const int64_t rows = (int64_t)a.B * a.Hkv * a.rows;
  const int tile_rows = plan.waves * plan.rows_per_wave;
  if (plan.head_dim != 128 && plan.head_dim != 64) return hipErrorInvalidValue;
  if (plan.wide_merge) {
    if (plan.head_dim == 128)
      hipLaunchKernelGGL((attn_merge_wide_kernel<128>), dim3((unsigned)rows), dim3(256), 0, stream, a, tile_rows);
    else
      hipLaunchKernelGGL((attn_merge_wide_kernel<64>), dim3((unsigned)rows), dim3(256), 0, stream, a, tile_rows);
  } else {
    const unsigned blocks = (unsigned)((rows * (plan.head_dim / 4) + 255) / 256);
    if (plan.head_dim == 128)
      hipLaunchKernelGGL((attn_merge_narrow_kernel<128>), dim3(blocks), dim3(256), 0, stream, a, tile_rows);
    else
      hipLaunchKernelGGL((attn_merge_narrow_kernel<64>), dim3(blocks), dim3(256), 0, stream, a, tile_rows);
  }
  return hipGetLastError();
}

}  // namespace bd
