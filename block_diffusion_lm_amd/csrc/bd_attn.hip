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
// item. Each wave holds 32 query rows in registers and streams the chunk's keys through LDS in
// tiles of 64 keys. Tiles are copied HBM -> LDS by LDS DMA (buffer/global loads with the lds
// modifier, 16 bytes a lane), so the copy takes no registers and, for tiles inside the cached
// prefix, no vector ALU work, into a ring of stages several tiles deep; one barrier per tile
// publishes a landed tile and frees a consumed stage. In eight-wave workgroups four waves issue
// the copies. Within a wave the 32-key blocks are software-pipelined: the QK product of the next
// block is in flight while the current block's exponentials run.
//
// The host sizes the grid (B * nsplit chunk slots per KV head and row tile) from its bound on
// the prefix lengths; the kernels then size the chunks on the device from the actual lengths and
// active flags (balanced_plan, up to kMaxBalancedBatch sequences): a ragged batch gets chunks of
// the size its total work calls for rather than its longest sequence's, and sequences the denoise
// loop has retired give their slots to the active ones, so the grid keeps every compute unit
// busy. Larger batches keep the host's uniform chunks, spread over the active sequences.
// A chunk's partial result is (m, l) in float32 and its normalized output acc / l in bf16, staged
// through the idle tile ring so that it leaves as whole rows; the merge kernel combines the chunks
// of every query row, its work-groups numbered over the active sequences' rows.
//
// MFMA formulation (v_mfma_f32_32x32x16_bf16). Scores are computed transposed,
// S^T = K Q^T (A = 32 keys x 16 dims from LDS, B = Q^T held in registers), so that every lane
// owns the scores of ONE query row (lane % 32) for 16 of each 32 keys; the other 16 keys of
// that row sit in lane ^ 32. Row max needs one cross-half swap, row sums none until the end.
// The output is also accumulated transposed, O^T += V^T P^T (A = V^T, B = P^T), whose B operand
// is exactly 8 consecutive accumulator registers of S^T converted to bf16. V stays row-major in
// LDS; its A operand is gathered with transposing LDS reads (ds_read_b64_tr_b16) whose per-lane
// key addresses follow the key order of those accumulator registers. The 64-byte blocks of V rows
// are swizzled by row (conflict-free transposing reads); the 16-byte chunks of K rows by the low
// three row bits, which leaves two-way bank conflicts between rows r and r + 8 in a 16-lane phase
// (measured: removing the K reads altogether saves under 2 %).
//
// Softmax: online (running max m, running sum l) in log2 units, exp2 in float32, P rounded to
// bf16 for the P V product; l sums the same bf16-rounded P (v_dot2), so numerator and
// denominator use identical weights. The running max is raised lazily: in the general loop only
// when a block's maximum exceeds it by more than 8 (log2 units), in the full-tile loop (which
// computes no row maxima) only when a lane's sum of a block's P values exceeds 256 -- then to the
// block's maximum. Probabilities relative to a stale max stay below 2^8, which fp32 and bf16 hold
// as well as any others, so the result is unchanged while rescaling the output accumulators
// becomes rare.
#include "bd_internal.h"

namespace bd {
namespace {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((__vector_size__(4 * sizeof(__bf16))));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazyRescale = 8.0f;
// Full-tile loop: a lane's sum of one block's 16 P values above this (or not finite) sends the
// block through the slow path, which raises the running max to the block's and recomputes P.
constexpr float kBlockSumLimit = 256.0f;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float other_half(float x) {
  // value of the same register in lane ^ 32
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

__device__ __forceinline__ u32x4 ldg16(const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); }

// a wave-uniform 64-bit value into scalar registers
__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Position of the k-th set bit of m (k < popcount(m)): a binary search on the halves' counts.
__device__ __forceinline__ int select_bit(uint64_t m, int k) {
  int pos = 0;
#pragma unroll
  for (int w = 32; w >= 1; w >>= 1) {
    const uint64_t lo = m & ((1ull << w) - 1);
    const int c = __popcll(lo);
    if (k >= c) {
      k -= c;
      m >>= w;
      pos += w;
    } else {
      m = lo;
    }
  }
  return pos;
}

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

// Active-sequence bookkeeping, shared by a work-group of NT threads: the active flags are scanned
// NT at a time (ceil(B / NT) rounds); every round turns each wave's 64 flags into a ballot mask in
// LDS, from which counts and ranks follow by population counts. All threads take part (the rounds
// hold barriers); the results are uniform across the work-group.
template <int NT>
struct ActiveScan {
  static constexpr int NWV = NT / 64;
  uint64_t* masks;   // NWV masks in LDS
  __device__ void load(const uint8_t* active, int B, int base) {
    const int idx = base + (int)threadIdx.x;
    const uint64_t m = __builtin_amdgcn_ballot_w64(idx < B && active[idx] != 0);
    if ((threadIdx.x & 63) == 0) masks[threadIdx.x >> 6] = m;
    __syncthreads();
  }
  __device__ int chunk_count() const {
    int c = 0;
#pragma unroll
    for (int w = 0; w < NWV; ++w) c += __popcll(masks[w]);
    return c;
  }
  // active flags before offset `off` of the loaded chunk
  __device__ int rank_in_chunk(int off) const {
    int r = 0;
    for (int w = 0; w < off / 64; ++w) r += __popcll(masks[w]);
    const int l = off % 64;
    return r + (l ? __popcll(masks[off / 64] & ((~0ull) >> (64 - l))) : 0);
  }
  // offset in the loaded chunk of its k-th active flag (0 <= k < chunk_count())
  __device__ int select_in_chunk(int k) const {
    for (int w = 0; w < NWV; ++w) {
      uint64_t m = masks[w];
      const int c = __popcll(m);
      if (k < c) {
        for (int j = 0; j < k; ++j) m &= m - 1;   // drop the k lowest set bits
        return w * 64 + __builtin_ctzll(m);
      }
      k -= c;
    }
    return 0;
  }
  // number of active sequences (B without a mask)
  __device__ int count(const uint8_t* active, int B) {
    if (!active) return B;
    int n = 0;
    for (int base = 0; base < B; base += NT) {
      load(active, B, base);
      n += chunk_count();
      __syncthreads();
    }
    return n;
  }
  // the sequence of active rank i
  __device__ int nth(const uint8_t* active, int B, int i) {
    if (!active) return i;
    int before = 0, found = 0;
    for (int base = 0; base < B; base += NT) {
      load(active, B, base);
      const int c = chunk_count();
      if (i >= before && i < before + c) found = base + select_in_chunk(i - before);
      before += c;
      __syncthreads();
    }
    return found;
  }
  // the number of active sequences and the ranks of sequences b[0..R-1] among them (their flags
  // need not be set), in one pass over the flags
  template <int R>
  __device__ void count_ranks(const uint8_t* active, int B, const int (&b)[R], int& n, int (&r)[R]) {
    if (!active) {
      n = B;
#pragma unroll
      for (int k = 0; k < R; ++k) r[k] = b[k];
      return;
    }
    n = 0;
#pragma unroll
    for (int k = 0; k < R; ++k) r[k] = 0;
    for (int base = 0; base < B; base += NT) {
      load(active, B, base);
      const int c = chunk_count();
#pragma unroll
      for (int k = 0; k < R; ++k) {
        if (b[k] >= base + NT) r[k] += c;
        else if (b[k] >= base) r[k] += rank_in_chunk(b[k] - base);
      }
      n += c;
      __syncthreads();
    }
  }
};

// Work-group sums and maximum of three values (every thread takes part; results uniform).
template <int NT>
__device__ __forceinline__ void wg_reduce3(int64_t& sum, int& mx, int& cnt, int64_t* red) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    sum += __shfl_xor(sum, m, 64);
    mx = max(mx, __shfl_xor(mx, m, 64));
    cnt += __shfl_xor(cnt, m, 64);
  }
  if ((threadIdx.x & 63) == 0) {
    red[3 * (threadIdx.x >> 6)] = sum;
    red[3 * (threadIdx.x >> 6) + 1] = mx;
    red[3 * (threadIdx.x >> 6) + 2] = cnt;
  }
  __syncthreads();
  sum = 0;
  mx = 0;
  cnt = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    sum += red[3 * w];
    mx = max(mx, (int)red[3 * w + 1]);
    cnt += (int)red[3 * w + 2];
  }
  __syncthreads();
}

// Length-balanced plan of a split launch (B <= kMaxBalancedBatch, no direct plan). With
// x_b = prefix_len[b] + S keys for an active sequence b (0 otherwise), every active sequence gets
// ns_b = ceil(x_b / C) chunks of C keys, C the smallest multiple of 64 for which all of them fit
// the launch's K = B * nsplit chunk slots per (KV head, row tile); sequence b's chunks take slots
// pfx[b] .. pfx[b + 1] - 1 (pfx: exclusive prefix sums of ns_b in sequence order, pfx[B] the total).
// Ragged lengths then get chunks of the size the total work calls for instead of the longest
// sequence's, and a length above the host's bound still gets all its keys. C is found by bisection
// between lower bound ceil(total / K) (feasible at once when the lengths are equal) and
// min(total / (K - n_act), max_b x_b), both feasible; every work-group of the split and of the
// merge launch computes the same plan from the same inputs.
struct BalancedPlan {
  int64_t chunk;   // C
  int total;       // sum of ns_b
};

template <int NT>
__device__ BalancedPlan balanced_plan(const AttnArgs& a, int* pfx, int64_t* red) {
  constexpr int NR = (kMaxBalancedBatch + NT - 1) / NT;
  const int tid = threadIdx.x;
  uint32_t x[NR];
  int64_t tot = 0;
  int mx = 0, nact = 0;
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    const int b = tid + NT * i;
    const bool on = b < a.B && (!a.active || a.active[b]);
    x[i] = on ? (uint32_t)a.prefix_len[b] + (uint32_t)a.S : 0u;   // (no load past B)
    tot += x[i];
    mx = max(mx, (int)x[i]);
    nact += on ? 1 : 0;
  }
  wg_reduce3<NT>(tot, mx, nact, red);
  BalancedPlan p{64, 0};
  if (nact == 0) return p;
  const int64_t K = (int64_t)a.B * a.nsplit;
  auto fits = [&](uint32_t c) {
    int64_t n = 0;
    int unused_m = 0, unused_c = 0;
#pragma unroll
    for (int i = 0; i < NR; ++i)
      if (x[i]) n += (x[i] + c - 1) / c;
    wg_reduce3<NT>(n, unused_m, unused_c, red);
    return n <= K;
  };
  int64_t lo = max((int64_t)1, (tot + 64 * K - 1) / (64 * K));                 // in 64-key units
  const int64_t hi_a = (tot + 64 * (K - nact) - 1) / (64 * (K - nact));       // K > nact: nsplit >= 2
  int64_t hi = max(lo, min(hi_a, ((int64_t)mx + 63) / 64));
  if (!fits((uint32_t)(lo * 64))) {
    while (hi - lo > 1) {   // lo infeasible, hi feasible
      const int64_t mid = (lo + hi) / 2;
      if (fits((uint32_t)(mid * 64))) hi = mid;
      else lo = mid;
    }
    lo = hi;
  }
  const uint32_t c = (uint32_t)(lo * 64);
  p.chunk = c;
  // exclusive prefix sums of ns_b in sequence order, NT sequences a round
  int base = 0;
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    if (NT * i >= a.B) break;   // uniform
    const int v = (int)((x[i] + c - 1) / c);
    int inc = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(inc, d, 64);
      if ((tid & 63) >= d) inc += o;
    }
    if ((tid & 63) == 63) red[tid >> 6] = inc;
    __syncthreads();
    int before = base, round = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
      const int t = (int)red[w];
      if (w < (tid >> 6)) before += t;
      round += t;
    }
    const int b = tid + NT * i;
    if (b < a.B) pfx[b] = before + inc - v;
    base += round;
    __syncthreads();
  }
  if (tid == 0) pfx[a.B] = base;
  __syncthreads();
  p.total = base;
  return p;
}

// The same plan for B <= 64, computed by one wave on its own (lane = sequence): wave-wide sums by
// shuffles, no LDS and no barrier, so every wave of a work-group derives it independently. The sums
// fit 32 bits (64 sequences of at most 2^23 + 64 keys: prefix capacity check). Lane b receives its
// first chunk slot (pfx) and its chunk count (ns).
__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

__device__ BalancedPlan balanced_plan_wave(const AttnArgs& a, int& pfx, int& ns) {
  const int lane = threadIdx.x & 63;
  const bool on = lane < a.B && (!a.active || a.active[lane]);
  const uint32_t x = on ? (uint32_t)a.prefix_len[lane] + (uint32_t)a.S : 0u;
  const uint32_t tot = wave_sum(x);
  uint32_t mx = x;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, m, 64));
  const int nact = __popcll(__builtin_amdgcn_ballot_w64(on));
  BalancedPlan p{64, 0};
  pfx = 0;
  ns = 0;
  if (nact == 0) return p;
  const uint32_t K = (uint32_t)a.B * (uint32_t)a.nsplit;   // <= 64 * nsplit
  auto fits = [&](uint32_t c) { return wave_sum(x ? (x + c - 1) / c : 0u) <= K; };
  uint32_t lo = max(1u, (tot + 64 * K - 1) / (64 * K));
  const uint32_t hi_a = (tot + 64 * (K - nact) - 1) / (64 * (K - nact));
  uint32_t hi = max(lo, min(hi_a, (mx + 63) / 64));
  if (!fits(lo * 64)) {
    while (hi - lo > 1) {
      const uint32_t mid = (lo + hi) / 2;
      if (fits(mid * 64)) hi = mid;
      else lo = mid;
    }
    lo = hi;
  }
  const uint32_t c = lo * 64;
  p.chunk = c;
  ns = (int)(x ? (x + c - 1) / c : 0u);
  int inc = ns;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(inc, d, 64);
    if (lane >= d) inc += o;
  }
  pfx = inc - ns;
  p.total = __shfl(inc, 63, 64);
  return p;
}

template <int D>
struct Geo {
  static constexpr int KT = kAttnKeyTile;           // keys per LDS tile
  static constexpr int KB = KT / 32;                // 32-key MFMA blocks per tile
  static constexpr int KROW = D * 2;                // bytes per key row of the K tile (16-byte chunks swizzled)
  static constexpr int VROW = D * 2;                // bytes per key row of the V tile (64-byte blocks swizzled)
  static constexpr int KBYTES = KT * KROW;
  static constexpr int VBYTES = KT * VROW;
  static constexpr int STAGE = KBYTES + VBYTES;
  static constexpr int JK = KBYTES / 1024;          // LDS-DMA wave instructions (64 lanes x 16 B) filling K
  static constexpr int J = JK + VBYTES / 1024;      // ... filling a whole stage
  static constexpr int KS = D / 16;                 // k-steps of S^T = K Q^T
  static constexpr int DB = D / 32;                 // 32-dim blocks of the output
  static_assert(KBYTES % 1024 == 0 && VBYTES % 1024 == 0, "stage regions must be whole DMA instructions");
  static_assert(STAGE == attn_stage_bytes(D), "host and device disagree on the stage size");
};

// 64-byte block swizzle of the V tile: block c of key row k is stored at c ^ vswz(k), so that the
// four consecutive key rows one transposing read touches lie in four different bank groups.
template <int D>
__device__ __forceinline__ int vswz(int k) {
  return D == 128 ? (k & 3) : ((k >> 1) & 1);
}

// Transposing LDS read (ds_read_b64_tr_b16). Within each group of 16 lanes, lane r supplies the
// address of 4 consecutive 16-bit values M[r][0..3]; lane j receives M[(j >> 2) + 4 i][j & 3] for
// i = 0..3. With lane r pointing at key (r >> 2) and dims 4 (r & 3) .. +3 of a row-major tile, lane
// j of the group receives dim j of four consecutive keys -- a column of V, i.e. a row of V^T.
//
// read_vt gathers the V^T operands of a 32-key block -- two 16-key steps e, every 32-dim block
// db, two reads each (keys +0..3 and +8..11 of each lane half) -- all issued together and waited
// for inside the same asm block. (Issued through the compiler, every such read would first wait
// for all LDS DMA in flight, i.e. for the tiles being prefetched.) addr[db]: LDS byte address of
// the lane's first key row in block db; OFF: byte offset of the block's first key row.
template <int D, int OFF>
__device__ __forceinline__ void read_vt(const uint32_t (&addr)[D / 32], bf16x8 (&vf)[2][D / 32]) {
  constexpr int R = D * 2;   // bytes per key row
  static_assert(OFF + 24 * R < 65536, "ds offset range");
  uint64_t r[2][D / 16];      // [e][2 db + half]
  if constexpr (D == 128) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %16 offset:%20\n\t"
        "ds_read_b64_tr_b16 %1, %16 offset:%21\n\t"
        "ds_read_b64_tr_b16 %2, %17 offset:%20\n\t"
        "ds_read_b64_tr_b16 %3, %17 offset:%21\n\t"
        "ds_read_b64_tr_b16 %4, %18 offset:%20\n\t"
        "ds_read_b64_tr_b16 %5, %18 offset:%21\n\t"
        "ds_read_b64_tr_b16 %6, %19 offset:%20\n\t"
        "ds_read_b64_tr_b16 %7, %19 offset:%21\n\t"
        "ds_read_b64_tr_b16 %8, %16 offset:%22\n\t"
        "ds_read_b64_tr_b16 %9, %16 offset:%23\n\t"
        "ds_read_b64_tr_b16 %10, %17 offset:%22\n\t"
        "ds_read_b64_tr_b16 %11, %17 offset:%23\n\t"
        "ds_read_b64_tr_b16 %12, %18 offset:%22\n\t"
        "ds_read_b64_tr_b16 %13, %18 offset:%23\n\t"
        "ds_read_b64_tr_b16 %14, %19 offset:%22\n\t"
        "ds_read_b64_tr_b16 %15, %19 offset:%23\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0][0]), "=&v"(r[0][1]), "=&v"(r[0][2]), "=&v"(r[0][3]), "=&v"(r[0][4]), "=&v"(r[0][5]),
          "=&v"(r[0][6]), "=&v"(r[0][7]), "=&v"(r[1][0]), "=&v"(r[1][1]), "=&v"(r[1][2]), "=&v"(r[1][3]),
          "=&v"(r[1][4]), "=&v"(r[1][5]), "=&v"(r[1][6]), "=&v"(r[1][7])
        : "v"(addr[0]), "v"(addr[1]), "v"(addr[2]), "v"(addr[3]), "i"(OFF), "i"(OFF + 8 * R), "i"(OFF + 16 * R),
          "i"(OFF + 24 * R));
  } else {
    static_assert(D == 64, "head_dim 64 or 128");
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8 offset:%10\n\t"
        "ds_read_b64_tr_b16 %1, %8 offset:%11\n\t"
        "ds_read_b64_tr_b16 %2, %9 offset:%10\n\t"
        "ds_read_b64_tr_b16 %3, %9 offset:%11\n\t"
        "ds_read_b64_tr_b16 %4, %8 offset:%12\n\t"
        "ds_read_b64_tr_b16 %5, %8 offset:%13\n\t"
        "ds_read_b64_tr_b16 %6, %9 offset:%12\n\t"
        "ds_read_b64_tr_b16 %7, %9 offset:%13\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0][0]), "=&v"(r[0][1]), "=&v"(r[0][2]), "=&v"(r[0][3]), "=&v"(r[1][0]), "=&v"(r[1][1]),
          "=&v"(r[1][2]), "=&v"(r[1][3])
        : "v"(addr[0]), "v"(addr[1]), "i"(OFF), "i"(OFF + 8 * R), "i"(OFF + 16 * R), "i"(OFF + 24 * R));
  }
#pragma unroll
  for (int e = 0; e < 2; ++e)
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const uint64_t lo = r[e][2 * db], hi = r[e][2 * db + 1];
      vf[e][db] = __builtin_bit_cast(bf16x8, u32x4{(uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi, (uint32_t)(hi >> 32)});
    }
}

// LDS DMA of 16 bytes per lane: lane l's 16 bytes at src land at LDS byte dst + 16 l (dst uniform).
__device__ __forceinline__ void dma16(const char* src, char* dst) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
}

// The same through a buffer resource: lane l's 16 bytes at base(rsrc) + soff + voff. The scalar
// offset carries the tile position, so a tile costs no vector ALU work at all. POLICY is the
// cache policy of the load: kStreamPolicy (bit 1 on gfx950: non-temporal) for a cached K/V stream
// too large to stay in the caches between launches, so that it leaves them to the partials and
// the block rows; 0 (normal) for one small enough to be read again from the last-level cache by
// the next launch (a decode step's 4 MB). The host picks (AttnArgs::stream_kv).
constexpr int kStreamPolicy = 2;
template <int POLICY = 0>
__device__ __forceinline__ void dma16_buf(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t soff, char* dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)dst, 16, voff, soff, 0,
                                           POLICY);
}

// Raw buffer resource over `bytes` bytes at `base` (dword 3: the gfx9 raw-buffer format word).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const void* base, uint64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)min(bytes, (uint64_t)0x7fffffff), 0x00020000);
}

// s_waitcnt vmcnt(N) lgkmcnt(0) (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
template <int N>
__device__ __forceinline__ void wait_vm_lds() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

// NW waves of RB 32-row blocks each. NW * RB == 8 (256 rows): one workgroup per CU; NW * RB == 4:
// two per CU. RB == 2 waves reuse every K and V^T operand read for two MFMAs.
template <int D, int NW, int RB>
__global__ __launch_bounds__(NW * 64, NW * RB == 8 ? 1 : 2) void attn_split_kernel(AttnArgs a) {
  using G = Geo<D>;
  constexpr int NT = NW * 64;
  constexpr int NSTAGE = attn_stages(D, NW * RB);
  constexpr int JV = G::J - G::JK;
  constexpr int NWD = NW >= 8 ? NW / 2 : NW;      // waves that issue the tile copies
  constexpr int NK = G::JK / NWD;                  // K / V DMA instructions such a wave issues per tile
  constexpr int NV = JV / NWD;
  constexpr int NMIN = NK + NV;                    // the waits count on this many per tile
  static_assert(NK * NWD == G::JK && NV * NWD == JV && NWD % 2 == 0, "copies split evenly over the copying waves");
  static_assert(NMIN * 3 < 64 && NSTAGE <= 5, "vmcnt range");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar branches and bases
  const int lrow = lane & 31;
  const int half = lane >> 5;

  // ---- work item (XCD-aware: consecutive items land on the same XCD when possible) ----
  const int64_t nitems = (int64_t)gridDim.x;
  int64_t item = blockIdx.x;
  if ((nitems & 7) == 0) item = (item & 7) * (nitems >> 3) + (item >> 3);
  // (values loaded from memory are made explicitly wave-uniform, so that the tile bookkeeping
  // and the DMA bases below live in scalar registers)
  __shared__ __attribute__((aligned(16))) char smem[NSTAGE * G::STAGE];
  __shared__ uint64_t act_masks[NW];
  __shared__ int64_t red[3 * NW];
  __shared__ int found_b;
  const int rt = (int)(item % a.row_tiles);
  int b, g, nsplit_out;
  int64_t k_begin, k_end, item_out;   // item_out: where the partials go (merge layout)
  if (a.balanced) {
    // slot j of KV head g and the sequence whose chunks hold it; the first work-group also stores
    // the plan's prefix sums for the merge
    const int64_t q = item / a.row_tiles;
    g = (int)(q % a.Hkv);
    const int j = (int)(q / a.Hkv);
    BalancedPlan bp;
    int c;
    if (a.B <= 64) {
      int pfx_l, ns_l;
      bp = balanced_plan_wave(a, pfx_l, ns_l);
      if (blockIdx.x == 0 && wave == 0) {
        if (lane < a.B) a.plan_pfx[lane] = pfx_l;
        if (lane == 0) a.plan_pfx[a.B] = bp.total;
      }
      if (j >= bp.total) return;   // uniform
      const uint64_t hit = __builtin_amdgcn_ballot_w64(ns_l > 0 && pfx_l <= j && j < pfx_l + ns_l);
      b = __builtin_amdgcn_readfirstlane((int)__builtin_ctzll(hit));
      c = j - __builtin_amdgcn_readfirstlane(__shfl(pfx_l, b, 64));
    } else {
      // pfx lives in the tile ring until the first copy; every wave has read it before the barrier
      int* pfx = reinterpret_cast<int*>(smem);
      bp = balanced_plan<NT>(a, pfx, red);
      if (blockIdx.x == 0)
        for (int bb = tid; bb <= a.B; bb += NT) a.plan_pfx[bb] = pfx[bb];
      if (j >= bp.total) return;   // uniform
      for (int bb = tid; bb < a.B; bb += NT)
        if (pfx[bb] <= j && j < pfx[bb + 1]) found_b = bb;
      __syncthreads();
      b = __builtin_amdgcn_readfirstlane(found_b);
      c = j - pfx[b];
      __syncthreads();
    }
    const int64_t nkeys = (int64_t)__builtin_amdgcn_readfirstlane(a.prefix_len[b]) + a.S;
    k_begin = (int64_t)c * bp.chunk;
    k_end = min(k_begin + bp.chunk, nkeys);
    item_out = ((int64_t)j * a.Hkv + g) * a.row_tiles + rt;
    nsplit_out = 2;   // partials always (no direct plan here)
  } else {
    ActiveScan<NT> scan{act_masks};
    const int n_act = __builtin_amdgcn_readfirstlane(scan.count(a.active, a.B));
    const ItemMap im = device_plan(a, n_act);
    const int64_t ps = item / a.row_tiles;
    const int split = (int)(ps % im.nsplit);
    const int64_t pair_a = ps / im.nsplit;              // pair among the active sequences
    if (pair_a >= (int64_t)n_act * a.Hkv) return;
    b = __builtin_amdgcn_readfirstlane(scan.nth(a.active, a.B, (int)(pair_a / a.Hkv)));
    g = (int)(pair_a % a.Hkv);
    const int64_t nkeys = (int64_t)__builtin_amdgcn_readfirstlane(a.prefix_len[b]) + a.S;
    k_begin = (int64_t)split * im.chunk;
    // the last chunk (and a direct plan's only one) runs to the sequence's end, so a length past
    // the host's bound still has all its keys
    k_end = a.direct || split == im.nsplit - 1 ? nkeys : min(k_begin + im.chunk, nkeys);
    item_out = (pair_a * im.nsplit + split) * a.row_tiles + rt;
    nsplit_out = im.nsplit;
  }
  // the plan's values are wave-uniform (the balanced plan derives them with shuffles, in vector
  // registers): keep them in scalar registers for the rest of the kernel
  k_begin = uniform64(k_begin);
  k_end = uniform64(k_end);
  item_out = uniform64(item_out);
  nsplit_out = __builtin_amdgcn_readfirstlane(nsplit_out);
  if (k_begin >= k_end) return;
  const int64_t len = __builtin_amdgcn_readfirstlane(a.prefix_len[b]);
  const int ntiles = (int)((k_end - k_begin + G::KT - 1) / G::KT);

  const int tile_rows = NW * RB * 32;
  const int row0 = rt * tile_rows + wave * RB * 32;   // first query row of this wave
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

  // ---- tile filling by LDS DMA. A stage is JK + JV wave instructions of 1 KB (64 lanes x 16 B):
  // K instruction j writes stage bytes [1024 j, 1024 j + 1024), V instruction j the same range of
  // the V region; copying wave w issues instructions w, w + NWD, ... of each.
  // buffer resources over this (sequence, KV head)'s cached rows (buffer offsets are 32-bit)
  const __amdgpu_buffer_rsrc_t rsrc_k = raw_rsrc(kc, (uint64_t)a.lcap * D * 2);
  const __amdgpu_buffer_rsrc_t rsrc_v = raw_rsrc(vc, (uint64_t)a.lcap * D * 2);
  const uint32_t blk_pitch = (uint32_t)(blk_stride * 2);   // bytes between block positions
  // Per-lane source offsets. K instruction j fills K rows r = 4j + lane / 16 (D = 128; 8j + lane / 8
  // for D = 64) with their 16-byte chunks at swizzled positions: chunk c of row r sits at position
  // c ^ (r & 7), so the K fragment reads below hit eight different bank groups. A lane's position
  // is fixed by the DMA (lane order), so it fetches the chunk that belongs there; r & 7 depends on
  // j only through j's parity, which is the copying wave's parity. V rows keep their 64-byte block
  // swizzle, which does not depend on j at all. Instruction j adds 1024 j to both.
  uint32_t kl, vl;
  {
    constexpr int LPR = D * 2 / 16;   // lanes per row (16-byte chunks per row)
    const int r = (wave & 1) * (1024 / (D * 2)) + lane / LPR;   // row within the pair of instructions
    const int pos = lane % LPR;
    kl = (uint32_t)((lane / LPR) * D * 2 + 16 * (pos ^ (r & 7)));
    const int vr = lane / LPR;
    const int vp = lane * 16;
    vl = (uint32_t)(vr * G::VROW + ((((vp % G::VROW) / 64) ^ vswz<D>(vr)) * 64) + (vp % 64));
  }
  // The tile at kt0 into stage `stage`. A tile that lies wholly inside the cached prefix and the
  // chunk (all but at most two per chunk) is one uniform base per tensor; otherwise sources are
  // per lane: cache rows, block rows past the prefix end, and rows past the chunk end repeating
  // its last key (finite data whose scores are masked).
  auto issue_tile = [&](int stage, int64_t kt0) {
    if (wave >= NWD) return;
    char* dst = smem + stage * G::STAGE;
    if (kt0 + G::KT <= len && kt0 + G::KT <= k_end) {
      const uint32_t soff = (uint32_t)(kt0 * D * 2);
      if (a.stream_kv) {   // uniform
#pragma unroll
        for (int i = 0; i < NK; ++i) {
          const int j = wave + NWD * i;
          dma16_buf<kStreamPolicy>(rsrc_k, kl, soff + 1024 * j, dst + 1024 * j);
        }
#pragma unroll
        for (int i = 0; i < NV; ++i) {
          const int j = wave + NWD * i;
          dma16_buf<kStreamPolicy>(rsrc_v, vl, soff + 1024 * j, dst + G::KBYTES + 1024 * j);
        }
      } else {
#pragma unroll
        for (int i = 0; i < NK; ++i) {
          const int j = wave + NWD * i;
          dma16_buf(rsrc_k, kl, soff + 1024 * j, dst + 1024 * j);
        }
#pragma unroll
        for (int i = 0; i < NV; ++i) {
          const int j = wave + NWD * i;
          dma16_buf(rsrc_v, vl, soff + 1024 * j, dst + G::KBYTES + 1024 * j);
        }
      }
    } else {
      // per lane: cached rows through the cache resources, rows past the prefix end by a global
      // address (the two are exec-masked: each lane issues one), rows past the chunk end repeating
      // its last key. Keys and cache byte offsets fit 32 bits (prefix capacity check).
      const int kt = (int)kt0, kend = (int)k_end, ln = (int)len;
      auto copy = [&](__amdgpu_buffer_rsrc_t rc, const uint16_t* blk, uint32_t off, char* d) {
        const int key = min(kt + (int)(off / (D * 2)), kend - 1);
        const uint32_t col = off % (D * 2);
        if (key < ln) dma16_buf(rc, (uint32_t)key * (D * 2) + col, 0, d);
        else dma16(reinterpret_cast<const char*>(blk) + (size_t)(key - ln) * blk_pitch + col, d);
      };
#pragma unroll
      for (int i = 0; i < NK; ++i) {
        const int j = wave + NWD * i;
        copy(rsrc_k, kb0, kl + 1024 * j, dst + 1024 * j);
      }
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int j = wave + NWD * i;
        copy(rsrc_v, vb0, vl + 1024 * j, dst + G::KBYTES + 1024 * j);
      }
    }
  };

  // ---- operand addresses inside a stage
  // K fragment (A of S^T = K Q^T): key kb*32 + lrow, dims 16 kstep + 8 half .. +7
  // K fragment kstep k reads chunk 2k + half of key lrow, stored at position (2k + half) ^ s with
  // s = lrow & 7: byte 128 (k >> 2) + 32 ((k & 3) ^ (s >> 1)) + 16 (half ^ (s & 1)) of the row.
  uint32_t k_lane[4];
  {
    const int sw = lrow & 7;
#pragma unroll
    for (int q = 0; q < 4; ++q) k_lane[q] = (uint32_t)(lrow * G::KROW + 32 * (q ^ (sw >> 1)) + 16 * (half ^ (sw & 1)));
  }
  // V^T fragment (A of O^T = V^T P^T) for 32-dim block db: two transposing reads, keys
  // 16e + 4 half + 0..3 and 16e + 8 + 4 half + 0..3 -- the key order of the P^T operand below.
  uint32_t v_lane[G::DB];
  {
    const int r = lane & 15;
    const int key = 4 * half + (r >> 2);
    const int dpart = 32 * ((lane >> 4) & 1) + 8 * (r & 3);   // bytes inside the 64-byte block
#pragma unroll
    for (int db = 0; db < G::DB; ++db) v_lane[db] = (uint32_t)(key * G::VROW + ((db ^ vswz<D>(key)) * 64) + dpart);
  }
  const uint32_t smem_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)smem;

  float m_run[RB], l_run[RB];   // running max (log2 units) and this lane's share of the sum
  f32x16 o[RB][G::DB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m_run[rb] = -INFINITY;
    l_run[rb] = 0.f;
#pragma unroll
    for (int db = 0; db < G::DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[rb][db][r] = 0.f;
  }
  const float sc = a.scale_log2;
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

  // this wave's DMA of a tile has landed once at most NMIN * (tiles issued after it) remain;
  // after the barrier every wave's has
  auto wait_tile = [&](int pending) {
    asm volatile("" ::: "memory");
    if (pending >= 3) wait_vm_lds<NMIN * 3>();
    else if (pending == 2) wait_vm_lds<NMIN * 2>();
    else if (pending == 1) wait_vm_lds<NMIN>();
    else wait_vm_lds<0>();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  // K fragments of block kb of the tile in stage st, and S^T = K Q^T from them
  auto load_k = [&](int st, int kb, bf16x8 (&kf)[G::KS]) {
    const char* ks = smem + st * G::STAGE + kb * 32 * G::KROW;
#pragma unroll
    for (int kstep = 0; kstep < G::KS; ++kstep)
      kf[kstep] = *reinterpret_cast<const bf16x8*>(ks + k_lane[kstep & 3] + 128 * (kstep >> 2));
  };
  auto qk = [&](const bf16x8 (&kf)[G::KS], f32x16 (&sacc)[RB]) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[rb][r] = 0.f;
#pragma unroll
    for (int kstep = 0; kstep < G::KS; ++kstep)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) sacc[rb] = mfma32(kf[kstep], qf[rb][kstep], sacc[rb]);
  };
  // Keys past the chunk end do not exist for this item (the block starting at absolute key key0
  // has `keys` < 32 existing keys); in the causal pass, block key j (absolute key len + j) is
  // invisible to block position s when j > s. Only tiles at a chunk end or holding block keys
  // take the branch.
  auto mask_keys = [&](f32x16 (&sacc)[RB], int64_t key0, int keys) {
    const bool causal_here = a.causal && key0 + 32 > len;
    if (keys < 32 || causal_here) {
      const int lim = keys - 4 * half;   // register r holds key key0 + 8 (r / 4) + 4 half + r % 4
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        // last visible register offset of this lane's row in the causal pass
        const int64_t vis = causal_here ? len + (row0 + rb * 32 + lrow) / a.group - key0 - 4 * half : (int64_t)64;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int off = 8 * (r >> 2) + (r & 3);
          if (off >= lim || off > vis) sacc[rb][r] = -INFINITY;
        }
      }
    }
  };
  // block row maxima in log2 units
  auto row_max = [&](const f32x16 (&sacc)[RB], float (&mx)[RB]) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float v = sacc[rb][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) v = fmaxf(v, sacc[rb][r]);
      mx[rb] = fmaxf(v, other_half(v)) * sc;
    }
  };
  // lazy rescale: raise the running max only when the block's exceeds it by more than
  // kLazyRescale (rare after the first block)
  auto rescale = [&](const float (&mx)[RB], bool live) {
    bool raise_any = false;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) raise_any |= live && mx[rb] > m_run[rb] + kLazyRescale;
    if (__builtin_amdgcn_ballot_w64(raise_any)) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const float mnew = live && mx[rb] > m_run[rb] + kLazyRescale ? mx[rb] : m_run[rb];
        // exp2(-inf) = 0 when the first visible keys arrive; a row whose max did not move (possibly
        // still -inf: no visible key yet in the causal pass) keeps its accumulators as they are
        const float alpha = mnew == m_run[rb] ? 1.f : __builtin_amdgcn_exp2f(m_run[rb] - mnew);
        l_run[rb] *= alpha;
#pragma unroll
        for (int db = 0; db < G::DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[rb][db][r] *= alpha;
        m_run[rb] = mnew;
      }
    }
  };
  // P = exp2(s*sc - m) in bf16 for the two 16-key steps e, and the row sums of the rounded P
  auto exp_p = [&](const f32x16 (&sacc)[RB], bf16x8 (&pf)[2][RB]) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      // no visible key yet for this row (causal pass): every P is 0, not exp2(nan)
      const float mneg = m_run[rb] == -INFINITY ? 0.f : -m_run[rb];
      float ls = l_run[rb];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
#pragma unroll
        for (int i = 0; i < 8; ++i) pf[e][rb][i] = (__bf16)__builtin_amdgcn_exp2f(fmaf(sacc[rb][8 * e + i], sc, mneg));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bf16x2 p2 = {pf[e][rb][2 * i], pf[e][rb][2 * i + 1]};
          ls = __builtin_amdgcn_fdot2_f32_bf16(p2, ones, ls, false);
        }
      }
      l_run[rb] = ls;
    }
  };
  // Full-tile variant of exp_p: the running max is finite (set by the first block), and the
  // block's row sums are returned instead of added, so the caller can check them first.
  auto exp_full = [&](const f32x16 (&sacc)[RB], bf16x8 (&pf)[2][RB], float (&bs)[RB]) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const float mneg = -m_run[rb];
      float ls = 0.f;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
#pragma unroll
        for (int i = 0; i < 8; ++i) pf[e][rb][i] = (__bf16)__builtin_amdgcn_exp2f(fmaf(sacc[rb][8 * e + i], sc, mneg));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bf16x2 p2 = {pf[e][rb][2 * i], pf[e][rb][2 * i + 1]};
          ls = __builtin_amdgcn_fdot2_f32_bf16(p2, ones, ls, false);
        }
      }
      bs[rb] = ls;
    }
  };
  // O^T += V^T P^T
  auto pv = [&](const bf16x8 (&vf)[2][G::DB], const bf16x8 (&pf)[2][RB]) {
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int db = 0; db < G::DB; ++db)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) o[rb][db] = mfma32(vf[e][db], pf[e][rb], o[rb][db]);
  };
  // LDS addresses of the V^T reads of block kb of the tile in stage st
  auto v_addr = [&](int st, int kb, uint32_t (&va)[G::DB]) {
#pragma unroll
    for (int db = 0; db < G::DB; ++db) va[db] = smem_lds + st * G::STAGE + G::KBYTES + kb * 32 * G::VROW + v_lane[db];
  };

  static_assert(G::KB == 2, "two 32-key blocks per tile");
  constexpr int AHEAD = NSTAGE >= 3 ? NSTAGE - 1 : NSTAGE;   // tiles issued before the loop
#pragma unroll
  for (int s = 0; s < AHEAD; ++s)
    if (s < ntiles) issue_tile(s, k_begin + (int64_t)s * G::KT);
  wait_tile(min(AHEAD - 1, ntiles - 1));
  f32x16 s_even[RB], s_odd[RB];   // S^T of the even and the odd block of a tile

  // ---- full tiles (ring of NSTAGE >= 3 stages). A tile wholly inside the cached prefix and the
  // chunk needs no key mask. Block j runs as two straight-line regions:
  //   A: V^T reads of block j, the QK product of block j + 1 (K read in the previous B) and the
  //      exponentials of block j -- MFMA and VALU work without dependences between them;
  //   B: the P V product of block j and the K reads of block j + 2.
  // The rare rescale (a branch, see p_of) ends A. Between A and B of the even block of tile t a
  // barrier publishes tile t + 1 and frees tile t - 1's stage for tile t + NSTAGE - 1.
  int t0 = 0;   // first tile of the general loop below
  if constexpr (NSTAGE >= 3) {
    const int64_t fe = min(len, k_end);
    const int nfull = fe > k_begin ? (int)((fe - k_begin) / G::KT) : 0;
    if (nfull > 0) {
      f32x16 s_cur[RB];
      bf16x8 kf[G::KS];
      float mx[RB];
      if (wave_rows) {
        load_k(0, 0, kf);
        qk(kf, s_cur);
        row_max(s_cur, mx);
        rescale(mx, true);
        load_k(0, 1, kf);
      }
      // P of block j with the running max. The row maxima are not computed on this path: a block
      // whose P sum on some lane exceeds kBlockSumLimit (a key above the running max by more than
      // log2(kBlockSumLimit / 16) in log2 units; an overflow shows as inf) takes the rare branch,
      // which raises the running max to the block's (rescaling O and l) and recomputes P, so every
      // P stays <= kBlockSumLimit.
      auto p_of = [&](bf16x8 (&pf)[2][RB]) {
        float bs[RB];
        exp_full(s_cur, pf, bs);
        bool big = false;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) big |= !(bs[rb] <= kBlockSumLimit);
        if (__builtin_amdgcn_ballot_w64(big)) {
          row_max(s_cur, mx);
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) {
            const float mnew = fmaxf(m_run[rb], mx[rb]);
            const float alpha = __builtin_amdgcn_exp2f(m_run[rb] - mnew);
            l_run[rb] *= alpha;
#pragma unroll
            for (int db = 0; db < G::DB; ++db)
#pragma unroll
              for (int r = 0; r < 16; ++r) o[rb][db][r] *= alpha;
            m_run[rb] = mnew;
          }
          exp_full(s_cur, pf, bs);
        }
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) l_run[rb] += bs[rb];
      };
      // block j = 2t + kb of tile t; `last`: the odd block of the last full tile (no block j + 2)
      auto block = [&](int t, int kb, bool last) {
        const int st = t % NSTAGE;
        bf16x8 vf[2][G::DB];
        bf16x8 pf[2][RB];
        f32x16 s_nxt[RB];
        if (wave_rows) {
          uint32_t va[G::DB];
          v_addr(st, kb, va);
          read_vt<D, 0>(va, vf);
          qk(kf, s_nxt);
          p_of(pf);
        }
        if (kb == 0) {
          wait_tile(min(NSTAGE - 3, ntiles - 2 - t));
          if (t + NSTAGE - 1 < ntiles) issue_tile((t + NSTAGE - 1) % NSTAGE, k_begin + (int64_t)(t + NSTAGE - 1) * G::KT);
        }
        if (wave_rows) {
          pv(vf, pf);
          if (!last) load_k((t + 1) % NSTAGE, kb, kf);
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) s_cur[rb] = s_nxt[rb];
        }
      };
      for (int t = 0; t < nfull - 1; ++t) {
        block(t, 0, false);
        block(t, 1, false);
      }
      block(nfull - 1, 0, false);
      block(nfull - 1, 1, true);
      // s_cur holds the QK product of the first block after the full tiles (if any)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) s_even[rb] = s_cur[rb];
      t0 = nfull;
    }
  }
  if (t0 == 0 && wave_rows) {
    bf16x8 kf[G::KS];
    load_k(0, 0, kf);
    qk(kf, s_even);
  }

  // ---- general loop (tiles at a chunk end or holding block keys; every tile when the ring has two
  // stages). Each block reads the K fragments of the next block first, then its own V^T operands,
  // and issues the next block's QK product in the same straight-line region as its own row maxima.
  // A QK product of a block that does not exist (past the last tile, or the odd half of a short
  // last tile) reads stale but in-bounds LDS and is never used. With 2 stages, tile t + 1 is
  // published after tile t's odd block has read its V^T operands, freeing tile t's stage for tile
  // t + 2.
  for (int t = t0; t < ntiles; ++t) {
    const int st = t % NSTAGE;
    const int valid = (int)min((int64_t)G::KT, k_end - (k_begin + (int64_t)t * G::KT));   // keys of tile t
    const bool odd = valid > 32;                  // tile t has a second block
    bf16x8 vf[2][G::DB];
    bf16x8 pf[2][RB];
    float mx[RB];
    // ---- even block
    if (wave_rows) {
      bf16x8 kf[G::KS];
      load_k(st, 1, kf);
      uint32_t va[G::DB];
      v_addr(st, 0, va);
      read_vt<D, 0>(va, vf);
      mask_keys(s_even, k_begin + (int64_t)t * G::KT, min(valid, 32));
      qk(kf, s_odd);
      row_max(s_even, mx);
      rescale(mx, true);
      exp_p(s_even, pf);
      pv(vf, pf);
    }
    if constexpr (NSTAGE >= 3) {
      // publish tile t + 1; tile t - 1's stage is free (waves without rows take part too)
      wait_tile(min(NSTAGE - 3, ntiles - 2 - t));
      if (t + NSTAGE - 1 < ntiles) issue_tile((t + NSTAGE - 1) % NSTAGE, k_begin + (int64_t)(t + NSTAGE - 1) * G::KT);
    }
    // ---- odd block
    if (wave_rows) {
      bf16x8 kf[G::KS];
      if constexpr (NSTAGE >= 3) load_k((t + 1) % NSTAGE, 0, kf);
      uint32_t va[G::DB];
      v_addr(st, 1, va);
      read_vt<D, 0>(va, vf);
      mask_keys(s_odd, k_begin + (int64_t)t * G::KT + 32, max(valid - 32, 0));
      if constexpr (NSTAGE < 3) {
        wait_tile(min(NSTAGE - 2, ntiles - 2 - t));
        if (t + NSTAGE < ntiles) issue_tile(st, k_begin + (int64_t)(t + NSTAGE) * G::KT);
        load_k((t + 1) % NSTAGE, 0, kf);
      }
      qk(kf, s_even);
      row_max(s_odd, mx);
      rescale(mx, odd);
      if (odd) {
        exp_p(s_odd, pf);
        pv(vf, pf);
      }
    } else if constexpr (NSTAGE < 3) {
      wait_tile(min(NSTAGE - 2, ntiles - 2 - t));
      if (t + NSTAGE < ntiles) issue_tile(st, k_begin + (int64_t)(t + NSTAGE) * G::KT);
    }
  }
  // ---- epilogue: lane owns row lrow of each row block; dims db*32 + 8*(r/4) + 4*half + r%4
  // The chunk partials go out through LDS: each wave stages its rows in the (now idle) tile ring and
  // writes them back as whole 256-byte rows, 16 bytes a lane, instead of each lane's 8-byte pieces
  // scattered over 32 rows (the write-back of the partials took ~5 us of a long step).
  constexpr int PITCH = D * 2 + 16;   // staged row (bytes), padded so the rows' writes spread over the banks
  static_assert(NW * RB * 32 * PITCH <= NSTAGE * G::STAGE, "the staged partials fit in the tile ring");
  if (nsplit_out != 1) __syncthreads();   // uniform: every wave is done with the ring
  if (!wave_rows) return;
  if (nsplit_out != 1) {
    char* stage = smem + wave * (RB * 32 * PITCH);
    const int64_t prow0 = item_out * tile_rows + (row0 - rt * tile_rows);   // the wave's first partial row
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const float l_tot = l_run[rb] + other_half(l_run[rb]);
      // the normalized output acc / l in bf16 (zero for a chunk without a visible key) and (m, l)
      const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
      const int rr = rb * 32 + lrow;
#pragma unroll
      for (int db = 0; db < G::DB; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int d = db * 32 + 8 * q4 + 4 * half;
          bf16x4 v;
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = (__bf16)(o[rb][db][4 * q4 + i] * inv);
          *reinterpret_cast<bf16x4*>(stage + rr * PITCH + d * 2) = v;
        }
      if (half == 0 && row0 + rr < a.rows)
        *reinterpret_cast<float2*>(a.part_ml + (prow0 + rr) * 2) = make_float2(m_run[rb], l_tot);
    }
    // rows past a.rows in the last row tile are padding rows of the partial buffer (never read)
    constexpr int CPR = D * 2 / 16;                 // 16-byte pieces of a row
    constexpr int NIT = RB * 32 * CPR / 64;
    char* ap = reinterpret_cast<char*>(a.part_o + prow0 * D);
#pragma unroll
    for (int j = 0; j < NIT; ++j) {
      const int e = j * 64 + lane;
      const int row = e / CPR, c = e % CPR;
      *reinterpret_cast<u32x4*>(ap + row * (D * 2) + c * 16) =
          *reinterpret_cast<const u32x4*>(stage + row * PITCH + c * 16);
    }
    (void)NT;
    return;
  }
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const float l_tot = l_run[rb] + other_half(l_run[rb]);
    const int r = row0 + rb * 32 + lrow;
    if (r >= a.rows) continue;
    const int s = r / a.group;
    const int hq = g * a.group + (r - s * a.group);
    {
      const float inv = 1.0f / l_tot;
      uint16_t* op = a.out + (((int64_t)b * a.S + s) * a.Hq + hq) * D;
#pragma unroll
      for (int db = 0; db < G::DB; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int d = db * 32 + 8 * q4 + 4 * half;
          bf16x4 v;
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = (__bf16)(o[rb][db][4 * q4 + i] * inv);
          *reinterpret_cast<bf16x4*>(op + d) = v;
        }
      if (a.lse && half == 0) a.lse[((int64_t)b * a.Hq + hq) * a.S + s] = (m_run[rb] + log2f(l_tot)) * kLn2;
    }
  }
  (void)NT;
}

// Merge of the chunk partials of every (sequence, KV head, query row): with M = max_c m_c and the
// chunk's normalized output o_c = acc_c / l_c (stored in bf16),
//   O = sum_c l_c 2^(m_c - M) o_c / sum_c l_c 2^(m_c - M),  LSE = (M + log2 sum_c l_c 2^(m_c - M)) ln 2.
// O is a convex combination of the o_c, so their bf16 rounding (2^-9 relative) bounds its error by
// 2^-9 max_c |o_c|, the order of the final bf16 rounding of O; the partials cost half the bytes
// of float32 ones.
//
// 256 threads = RW row slots x CG chunk groups x (D/4 groups of 4 dims); a thread of a row slot
// merges RPT rows (RW x RPT rows per work-group). Chunk group j takes chunks j, j + CG, ... in
// index order, U at a time for each of its rows (all U x RPT loads in flight together), keeping a
// running maximum per row: when a group of U raises it, the sums so far are scaled down first.
// The chunk groups are then combined in index order through LDS, so the result does not depend
// on scheduling. A chunk without a visible key (m = -inf, causal pass) contributes nothing.
template <int D, int CG, int U, int RPT>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs a, int tile_rows) {
  constexpr int DG = D / 4;
  constexpr int RW = 256 / (DG * CG);
  static_assert(RW * DG * CG == 256, "thread layout");
  static_assert(CG == 1 || RPT == 1, "the chunk groups' LDS combine holds one row per thread");
  __shared__ float red_m[CG > 1 ? 256 : 1];
  __shared__ float red_den[CG > 1 ? 256 : 1];
  __shared__ f32x4 red_num[CG > 1 ? 256 : 1];
  const int tid = threadIdx.x;
  const int dg = tid % DG;
  const int cg = (tid / DG) % CG;
  const int rw = tid / (DG * CG);
  // the host keeps B * Hkv * rows below 2^31: 32-bit row arithmetic (no 64-bit division ahead of
  // the first load)
  uint32_t nrows = (uint32_t)a.B * a.Hkv * a.rows;
  uint32_t nitems = gridDim.x;
  // With an active mask over at most 64 sequences the rows are numbered over the active sequences
  // only and the first work-groups of the grid take them, so they spread over every XCD whichever
  // sequences have retired (numbered over all sequences, a lone active sequence's rows would sit on
  // the two XCDs that its quarter of the grid maps to).
  const bool compact = a.active && a.B <= 64;
  // (balanced plan over at most 64 sequences) the plan's prefix sums, one per lane, loaded together
  // with the flags so that both cost one round trip: row k then takes its sequence's by shuffle
  const bool lane_plan = a.balanced && a.B <= 64;
  int pfx_l = 0, pfx_tot = 0;
  if (lane_plan) {
    const int ln = tid & 63;
    pfx_l = a.plan_pfx[min(ln, a.B - 1)];
    pfx_tot = a.plan_pfx[a.B];
  }
  uint64_t act_bits = 0;
  if (compact) {
    const int ln = tid & 63;
    act_bits = __builtin_amdgcn_ballot_w64(ln < a.B && a.active[min(ln, a.B - 1)] != 0);
    nrows = (uint32_t)__popcll(act_bits) * (uint32_t)a.Hkv * a.rows;
    nitems = (nrows + RW * RPT - 1) / (RW * RPT);
    if (blockIdx.x >= nitems) return;   // uniform
  }
  int r[RPT], b[RPT], g[RPT];
  bool act[RPT];
  uint32_t plen[RPT];
#pragma unroll
  for (int k = 0; k < RPT; ++k) {
    // consecutive rows on one XCD: their (m, l) pairs share cache sectors
    const uint32_t rowg = (xcd_local_item(blockIdx.x, nitems) * RPT + k) * RW + rw;
    const bool live = rowg < nrows;
    const uint32_t pair = live ? rowg / (uint32_t)a.rows : 0;
    r[k] = live ? (int)(rowg - pair * (uint32_t)a.rows) : 0;
    const int bn = (int)(pair / (uint32_t)a.Hkv);   // among the active sequences when compact
    g[k] = (int)(pair - (uint32_t)bn * a.Hkv);
    b[k] = compact && live ? select_bit(act_bits, bn) : bn;
    // (uniform plan) the sequence's length first: it is needed last (to drop the chunks past its
    // keys), and its load then overlaps the scan of the active flags and the partial loads
    plen[k] = live && !a.balanced ? a.prefix_len[b[k]] : 0;
    act[k] = live && (compact || !(a.active && !a.active[b[k]]));
  }
  // where row k's chunk partials are (p0[k] + c * pstride, c < nclamp[k]) under either plan; an
  // inactive row reads the workspace's first rows (in bounds, shared by all such rows) and drops
  // them: no branch around the loads
  ItemMap im{a.nsplit, a.chunk};
  int64_t pstride;
  int64_t p0[RPT];
  int nclamp[RPT];
  int nl = 0;   // chunk slots this thread walks
  if (a.balanced) {
    // the split launch's plan (its first work-group stored the prefix sums)
    pstride = (int64_t)a.Hkv * a.row_tiles * tile_rows;   // partial rows between chunks
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
      p0[k] = 0;
      nclamp[k] = 0;
      // (all lanes take part in the shuffles)
      const int Pl = __shfl(pfx_l, b[k], 64);
      const int Pnl = b[k] + 1 < a.B ? __shfl(pfx_l, b[k] + 1, 64) : pfx_tot;
      if (act[k]) {
        const int P = lane_plan ? Pl : a.plan_pfx[b[k]];
        nclamp[k] = (lane_plan ? Pnl : a.plan_pfx[b[k] + 1]) - P;   // every chunk of the sequence holds keys
        const int rt = r[k] / tile_rows;
        p0[k] = (((int64_t)P * a.Hkv + g[k]) * a.row_tiles + rt) * tile_rows + (r[k] - rt * tile_rows);
      }
      nl = max(nl, nclamp[k]);
    }
  } else {
    __shared__ uint64_t act_masks[4];
    ActiveScan<256> scan{act_masks};
    int n_act, rank_b[RPT];   // every thread takes part in the scan's barriers
    scan.count_ranks<RPT>(a.active, a.B, b, n_act, rank_b);
    im = device_plan(a, n_act);
    if (im.nsplit == 1) return;   // the split kernel wrote the output itself
    pstride = (int64_t)a.row_tiles * tile_rows;
    nl = im.nsplit;
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
      p0[k] = 0;
      nclamp[k] = im.nsplit;
      if (act[k]) {
        const int64_t pair_a = (int64_t)rank_b[k] * a.Hkv + g[k];
        const int rt = r[k] / tile_rows;
        p0[k] = ((pair_a * im.nsplit) * a.row_tiles + rt) * tile_rows + (r[k] - rt * tile_rows);
      }
    }
  }
  int ns[RPT];
  float M[RPT], den[RPT];
  f32x4 num[RPT];
#pragma unroll
  for (int k = 0; k < RPT; ++k) {
    M[k] = -INFINITY;
    den[k] = 0.f;
    num[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  for (int c0 = cg; c0 < nl; c0 += U * CG) {
    float mm[RPT][U], ll[RPT][U];
    f32x4 v[RPT][U];
    // every slot loads a chunk of the plan (past the row's last: the last again), so that all the
    // loads of the round are issued before the first is used and before the lengths are known;
    // chunks past a sequence's keys (uniform plan) were not written by this call and are dropped
#pragma unroll
    for (int k = 0; k < RPT; ++k)
#pragma unroll
      for (int j = 0; j < U; ++j) {
        const int c = min(c0 + j * CG, max(nclamp[k] - 1, 0));
        const int64_t pr = p0[k] + c * pstride;
        const float2 ml = *reinterpret_cast<const float2*>(a.part_ml + pr * 2);
        mm[k][j] = ml.x;
        ll[k][j] = ml.y;
        const uint2 raw = *reinterpret_cast<const uint2*>(a.part_o + pr * D + dg * 4);
        v[k][j] = f32x4{__uint_as_float(raw.x << 16), __uint_as_float(raw.x & 0xffff0000u),
                        __uint_as_float(raw.y << 16), __uint_as_float(raw.y & 0xffff0000u)};
      }
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
      const uint32_t chunk = (uint32_t)im.chunk;   // <= max_prefix_len + S < 2^31
      ns[k] = !act[k] ? 0 : a.balanced ? nclamp[k] : (int)min((uint32_t)im.nsplit, (plen[k] + a.S + chunk - 1) / chunk);
#pragma unroll
      for (int j = 0; j < U; ++j)
        if (c0 + j * CG >= ns[k]) {
          mm[k][j] = -INFINITY;
          ll[k][j] = 0.f;
          v[k][j] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      float gm = mm[k][0];
#pragma unroll
      for (int j = 1; j < U; ++j) gm = fmaxf(gm, mm[k][j]);
      if (gm > M[k]) {
        const float sc = M[k] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M[k] - gm);
        den[k] *= sc;
        num[k] *= sc;
        M[k] = gm;
      }
#pragma unroll
      for (int j = 0; j < U; ++j) {
        const float w = mm[k][j] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mm[k][j] - M[k]) * ll[k][j];
        den[k] += w;
        num[k] += v[k][j] * w;
      }
    }
  }
  if constexpr (CG > 1) {
    red_m[tid] = M[0];
    red_den[tid] = den[0];
    red_num[tid] = num[0];
    __syncthreads();
    if (cg != 0) return;
    const int base = rw * DG * CG + dg;
    float Mc = M[0];
#pragma unroll
    for (int j = 1; j < CG; ++j) Mc = fmaxf(Mc, red_m[base + j * DG]);
    den[0] = 0.f;
    num[0] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < CG; ++j) {
      const float mj = red_m[base + j * DG];
      const float w = mj == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mj - Mc);
      den[0] += red_den[base + j * DG] * w;
      num[0] += red_num[base + j * DG] * w;
    }
    M[0] = Mc;
  }
#pragma unroll
  for (int k = 0; k < RPT; ++k) {
    if (!act[k]) continue;
    const float inv = 1.0f / den[k];
    const int s = r[k] / a.group;
    const int hq = g[k] * a.group + (r[k] - s * a.group);
    bf16x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = (__bf16)(num[k][i] * inv);
    *reinterpret_cast<bf16x4*>(a.out + (((int64_t)b[k] * a.S + s) * a.Hq + hq) * D + dg * 4) = o;
    if (a.lse && dg == 0) a.lse[((int64_t)b[k] * a.Hq + hq) * a.S + s] = (M[k] + log2f(den[k])) * kLn2;
  }
}

}  // namespace

hipError_t launch_attn_split(const AttnPlan& plan, const AttnArgs& a, const Launch& l) {
  if (plan.key_tile != kAttnKeyTile) return hipErrorInvalidValue;
  const dim3 grid((unsigned)plan.n_items);
  const dim3 block((unsigned)plan.waves * 64);
  const int key = plan.head_dim * 1000 + plan.waves * 100 + plan.rows_per_wave;
  switch (key) {
    case 128832: return launch_kernel(attn_split_kernel<128, 8, 1>, grid, block, l, a);
    case 128432: return launch_kernel(attn_split_kernel<128, 4, 1>, grid, block, l, a);
    case 64832: return launch_kernel(attn_split_kernel<64, 8, 1>, grid, block, l, a);
    case 64432: return launch_kernel(attn_split_kernel<64, 4, 1>, grid, block, l, a);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_attn_merge(const AttnPlan& plan, const AttnArgs& a, const Launch& l) {
  const int64_t rows = (int64_t)a.B * a.Hkv * a.rows;
  const int tile_rows = plan.waves * plan.rows_per_wave;
  // many chunks per row: eight chunk groups per row; U: chunks per group and round (2, 4 or 8);
  // with one chunk group a thread merges 8 / U rows, so that it keeps eight loads in flight
  const int cg = plan.wide_merge ? 8 : 1;
  const int per = (plan.nsplit + cg - 1) / cg;
  const int u = per <= 2 ? 2 : per <= 4 ? 4 : 8;
  const int rpt = cg == 1 ? 8 / u : 1;
  const int rw = 256 / ((plan.head_dim / 4) * cg);
  const dim3 grid((unsigned)((rows + (int64_t)rw * rpt - 1) / ((int64_t)rw * rpt)));
  switch (plan.head_dim * 1000 + cg * 10 + u) {
#define BD_MERGE(d, c, uu, rr) \
  case d * 1000 + c * 10 + uu: return launch_kernel(attn_merge_kernel<d, c, uu, rr>, grid, dim3(256), l, a, tile_rows);
    BD_MERGE(128, 8, 2, 1) BD_MERGE(128, 8, 4, 1) BD_MERGE(128, 8, 8, 1)
    BD_MERGE(128, 1, 2, 4) BD_MERGE(128, 1, 4, 2) BD_MERGE(128, 1, 8, 1)
    BD_MERGE(64, 8, 2, 1) BD_MERGE(64, 8, 4, 1) BD_MERGE(64, 8, 8, 1)
    BD_MERGE(64, 1, 2, 4) BD_MERGE(64, 1, 4, 2) BD_MERGE(64, 1, 8, 1)
#undef BD_MERGE
    default: return hipErrorInvalidValue;
  }
}

}  // namespace bd
