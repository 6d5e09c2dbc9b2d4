// Block selection for block-sparse prefill on gfx950, float64 throughout.
//
// Steps, in the order of the patty.io review of RBS-Attention (sections on the centroid
// score, mean dilution, the max-key-radius signal, the two independently thresholded
// branches and their union):
//   1-2. stats_kernel  in one grid: the mean of the query rows of every (b, h, query block),
//                      and the centroid of every (b, kv, key block) with its squared radius,
//                      the largest |k_j - c|^2 over the block's keys
//   3. score_kernel    s1 = <qmean, c> for admissible (query block, key block) pairs
//                      (admissible = holds at least one (row, key) pair the position / window
//                      rule allows) on the fp64 MFMA; pairs of 64 x 64 tiles with none are
//                      not computed
//   4. the per-head order statistic of s1 and the per-(b, kv) one of rad2 at the keep
//      fractions: with N values and n = floor(keep*N + 1/2), tau = the (n+1)-th largest
//      (-inf if n >= N), found exactly, and
//   5. mask = admissible and (s1 > tau_mean or rad2 > tau_radius), plus the ascending list of
//      kept key blocks per (b, h, query block) when asked for.
//   Heads of at most CAND_LDS pairs (a chunk's few query blocks):
//        score_kernel   stores s1
//        threshold_direct_kernel  ranks the head's admissible s1 in LDS (and rad2 per (b, kv))
//        mask_kernel    the mask (and lists) from the stored s1
//   Larger heads, in two MFMA passes that store no s1:
//        score_kernel   (histogram pass) counts the admissible s1 of each work item into a
//                       value histogram (a monotone bucket map over [-M, M], M = max|qmean| *
//                       max|c|, the Cauchy-Schwarz bound; values outside clamp to the end
//                       buckets)
//        pick_kernel    sums a head's item histograms and locates the bucket holding
//                       descending rank n and the rank inside it (and ranks rad2 per (b, kv))
//        score_kernel   (mask pass) recomputes s1 and writes the mask: the buckets above the
//                       picked one are kept by mean, those below are not; the picked bucket's
//                       values (a few dozen on typical data) are copied out as candidates
//        threshold_kernel  ranks the candidates (rank n - the count above the bucket) and
//                       marks those above tau_mean in the mask
//      A monotone map puts every value of a higher bucket strictly above every value of a
//      lower one, so rank n overall is rank n - (count above the bucket) inside it.  The two
//      passes compute s1 with the same instructions in the same order, so they agree bit for
//      bit.
// bf16 and f32 inputs widen exactly to f64.  Every reduction that feeds a value has a fixed
// order, so the output is identical from run to run; means are sums of at most a few hundred
// short mantissas and come out exact, so they agree bit for bit with any correct f64
// evaluation.  Only the order of the copied candidates depends on the run, which an order
// statistic does not see.  Steps 1 and 2 read q and k once; the rest is HBM-light.

#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace soc {
namespace {

constexpr int NTHR = 256;
typedef double f64x4 __attribute__((ext_vector_type(4)));
typedef double f64x2 __attribute__((ext_vector_type(2)));

// 8 consecutive elements of a row, loaded raw and widened to double on use.
template <typename T>
struct Row8;
template <>
struct Row8<bf16_t> {
  u32x4 w;
  __device__ __forceinline__ void load(const bf16_t* p) { w = *(const u32x4*)p; }
  __device__ __forceinline__ void widen(double* o) const {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      o[2 * e] = (double)bf16_lo(w[e]);
      o[2 * e + 1] = (double)bf16_hi(w[e]);
    }
  }
};
template <>
struct Row8<float> {
  f32x4 x, y;
  __device__ __forceinline__ void load(const float* p) {
    x = *(const f32x4*)p;
    y = *(const f32x4*)(p + 4);
  }
  __device__ __forceinline__ void widen(double* o) const {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      o[e] = (double)x[e];
      o[4 + e] = (double)y[e];
    }
  }
};

__device__ __forceinline__ int seq_off(const SelectArgs& a, int b) { return a.cache_off ? a.cache_off[b] : a.tk - a.tq; }

__device__ __forceinline__ bool admissible(const SelectArgs& a, int off, int tkb, int qb, int kb) {
  const int p0 = off + qb * a.bs;
  const int p1 = off + min((qb + 1) * a.bs, a.tq) - 1;
  const int j0 = kb * a.bs;
  const int j1 = min((kb + 1) * a.bs, tkb) - 1;
  if (j0 >= tkb) return false;
  bool ok = j0 <= p1;
  if (a.window > 0) ok = ok && (j1 > p0 - a.window);
  return ok;
}

// The admissible key blocks of query block qb in closed form: kb is admissible iff lo <= kb <= hi
// (causal: the block's first key is at most the block's last position and holds a key of the
// sequence; window: the block's last key lies after the first position minus the window, which
// the sequence's last key block always satisfies).  Never empty, and lo and hi do not decrease
// with qb.
__device__ __forceinline__ void adm_range(const SelectArgs& a, int off, int tkb, int qb, int& lo, int& hi) {
  const int nkb_b = (tkb + a.bs - 1) / a.bs;
  const int p0 = off + qb * a.bs, p1 = off + min((qb + 1) * a.bs, a.tq) - 1;
  hi = min(nkb_b - 1, p1 / a.bs);
  lo = 0;
  if (a.window > 0) {
    const int x = p0 - a.window + 1;
    lo = min(x > 0 ? x / a.bs : 0, nkb_b - 1);
  }
}

// Rows per thread loaded in one batch by block_mean (all loads of a batch are in flight
// together).
constexpr int RB = 8;

// Cross-lane moves of a double, as two 32-bit halves.
__device__ __forceinline__ uint32_t lo32(double x) { return (uint32_t)__builtin_bit_cast(uint64_t, x); }
__device__ __forceinline__ uint32_t hi32(double x) { return (uint32_t)(__builtin_bit_cast(uint64_t, x) >> 32); }
__device__ __forceinline__ double from32(uint32_t lo, uint32_t hi) {
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
// x(l) + x(l ^ 32) and x(l) + x(l ^ 16) with gfx950's lane-swap VALU instructions: both lanes of
// a pair get the same sum (the lower lane's value first).
__device__ __forceinline__ double sum_xor32(double x) {
  const auto l = __builtin_amdgcn_permlane32_swap(lo32(x), lo32(x), false, false);
  const auto h = __builtin_amdgcn_permlane32_swap(hi32(x), hi32(x), false, false);
  return from32(l[0], h[0]) + from32(l[1], h[1]);
}
__device__ __forceinline__ double sum_xor16(double x) {
  const auto l = __builtin_amdgcn_permlane16_swap(lo32(x), lo32(x), false, false);
  const auto h = __builtin_amdgcn_permlane16_swap(hi32(x), hi32(x), false, false);
  return from32(l[0], h[0]) + from32(l[1], h[1]);
}
// A DPP lane permutation of a double (CTRL: quad_perm, row_ror or row_half_mirror code).
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double x) {
  const uint32_t l = (uint32_t)__builtin_amdgcn_mov_dpp((int)lo32(x), CTRL, 0xf, 0xf, false);
  const uint32_t h = (uint32_t)__builtin_amdgcn_mov_dpp((int)hi32(x), CTRL, 0xf, 0xf, false);
  return from32(l, h);
}
constexpr int DPP_XOR1 = 0xB1;         // quad_perm [1, 0, 3, 2]
constexpr int DPP_XOR2 = 0x4E;         // quad_perm [2, 3, 0, 1]
constexpr int DPP_HALF_MIRROR = 0x141;  // lane i <-> 7 - i within each 8 lanes
constexpr int DPP_ROR8 = 0x128;         // lane i <-> i ^ 8 within each 16 lanes

// Block mean of rows [r0, r1) of a [rows, D] matrix (row stride st), written to out_lds[D].
// Thread layout: C = D/8 threads per row (8 columns each), NTHR/C row groups; a thread adds
// its rows in ascending order, then the row groups are added in ascending order.  When the
// block fits in one batch (r1 - r0 <= RB * NTHR/C) the loaded rows stay in `rows` and the
// function returns true.
template <typename T, int D>
__device__ bool block_mean(const T* base, int64_t st, int r0, int r1, double* red, double* out_lds, Row8<T>* rows) {
  constexpr int C = D / 8, RG = NTHR / C;
  const int c = threadIdx.x % C, rg = threadIdx.x / C;
  double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int rb = r0 + rg; rb < r1; rb += RB * RG) {
#pragma unroll
    for (int u = 0; u < RB; ++u) {
      const int r = rb + u * RG;
      if (r < r1) rows[u].load(base + (int64_t)r * st + 8 * c);
    }
#pragma unroll
    for (int u = 0; u < RB; ++u) {
      if (rb + u * RG < r1) {
        double x[8];
        rows[u].widen(x);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += x[e];
      }
    }
  }
  if (C == 16) {
    // The wave's 4 row groups (lanes c, c + 16, c + 32, c + 48) are summed with lane swaps;
    // lane (j, c) then writes columns 8c + 2j, 8c + 2j + 1, so each wave stores one
    // contiguous, conflict-free 1 KB row of partial column sums; the 4 waves are added in
    // order.
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = sum_xor16(sum_xor32(acc[e]));
    const int lane = threadIdx.x & 63, j = lane >> 4;
    f64x2 w2;
    w2[0] = j == 0 ? acc[0] : j == 1 ? acc[2] : j == 2 ? acc[4] : acc[6];
    w2[1] = j == 0 ? acc[1] : j == 1 ? acc[3] : j == 2 ? acc[5] : acc[7];
    *(f64x2*)(red + (threadIdx.x >> 6) * D + 8 * c + 2 * j) = w2;
    __syncthreads();
    if (threadIdx.x < D) {
      const double sum = ((red[threadIdx.x] + red[D + threadIdx.x]) + red[2 * D + threadIdx.x]) + red[3 * D + threadIdx.x];
      out_lds[threadIdx.x] = sum / (double)(r1 - r0);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) red[rg * D + 8 * c + e] = acc[e];
    __syncthreads();
    if (threadIdx.x < D) {
      double sum = 0.0;
      for (int g = 0; g < RG; ++g) sum += red[g * D + threadIdx.x];
      out_lds[threadIdx.x] = sum / (double)(r1 - r0);
    }
  }
  __syncthreads();
  return r1 - r0 <= RB * RG;
}

// block_mean for a full block of bf16 rows with D = 128 (RB * RG = 128 rows, the usual block
// size): no row guards, and the loads are buffer loads with the row offset u * RG in the
// scalar operand (no per-row address arithmetic).  The wave's 4 row groups are combined by a
// reduce-scatter of lane swaps (columns 0..3 and 4..7 of a thread split between the lane
// halves, then pairs between the rows of 16), each lane ending with the wave's sums of 2
// columns, stored as one conflict-free 1 KB LDS row per wave; the 4 waves are added in order.
// Rows stay in `rows` (a full block fits one batch).
__device__ void block_mean_full128(const bf16_t* base, int64_t st, double* red, double* out_lds, Row8<bf16_t>* rows) {
  constexpr int D = 128, C = D / 8, RG = NTHR / C;
  const int c = threadIdx.x % C, rg = threadIdx.x / C, lane = threadIdx.x & 63, j = lane >> 4;
  const uint64_t bp = (uint64_t)base;
  const uint64_t bpu = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(bp >> 32)) << 32) |
                       (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)bp);
  const uint32_t row_bytes = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(st * 2));
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)bpu, (short)0, (int)(row_bytes * (RB * RG - 1) + D * 2), 0x00020000);
  const uint32_t voff = (uint32_t)rg * row_bytes + 16u * (uint32_t)c;
#pragma unroll
  for (int u = 0; u < RB; ++u) rows[u].w = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, u * RG * row_bytes, kLoadReadOnce);
  double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int u = 0; u < RB; ++u) {
    double x[8];
    rows[u].widen(x);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += x[e];
  }
  // x(l) + x(l ^ 32) of a in the lower lane half and of b in the upper (v_permlane32_swap);
  // the same between even and odd rows of 16 (v_permlane16_swap)
  auto pair32 = [](double a, double b) __attribute__((always_inline)) {
    const auto l = __builtin_amdgcn_permlane32_swap(lo32(a), lo32(b), false, false);
    const auto h = __builtin_amdgcn_permlane32_swap(hi32(a), hi32(b), false, false);
    return from32(l[0], h[0]) + from32(l[1], h[1]);
  };
  auto pair16 = [](double a, double b) __attribute__((always_inline)) {
    const auto l = __builtin_amdgcn_permlane16_swap(lo32(a), lo32(b), false, false);
    const auto h = __builtin_amdgcn_permlane16_swap(hi32(a), hi32(b), false, false);
    return from32(l[0], h[0]) + from32(l[1], h[1]);
  };
  double k4[4], k2[2];
#pragma unroll
  for (int t = 0; t < 4; ++t) k4[t] = pair32(acc[t], acc[4 + t]);  // columns 4 (j >> 1) + t
#pragma unroll
  for (int t = 0; t < 2; ++t) k2[t] = pair16(k4[t], k4[2 + t]);  // columns 4 (j >> 1) + 2 (j & 1) + t
  f64x2 w2;
  w2[0] = k2[0];
  w2[1] = k2[1];
  *(f64x2*)(red + (threadIdx.x >> 6) * D + 8 * c + 4 * (j >> 1) + 2 * (j & 1)) = w2;
  __syncthreads();
  if (threadIdx.x < D) {
    const double sum = ((red[threadIdx.x] + red[D + threadIdx.x]) + red[2 * D + threadIdx.x]) + red[3 * D + threadIdx.x];
    out_lds[threadIdx.x] = sum / (double)(RB * RG);
  }
  __syncthreads();
}

// Squared norm of an LDS vector (wave 0 computes it; lane 0 writes it).
template <int D>
__device__ __forceinline__ void write_norm2(const double* v, double* dst) {
  if (threadIdx.x < 64) {
    double n2 = 0.0;
#pragma unroll
    for (int t = threadIdx.x; t < D; t += 64) n2 = fma(v[t], v[t], n2);
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) n2 += __shfl_xor(n2, m, 64);
    if (threadIdx.x == 0) *dst = n2;
  }
}

template <typename T, int D>
__device__ __forceinline__ void qmean_block(const SelectArgs& a, int id, double* red, double* mean) {
  const int qb = id % a.nqb;
  const int h = (id / a.nqb) % a.Hq;
  const int b = id / (a.nqb * a.Hq);
  const int64_t bh = (int64_t)b * a.Hq + h;
  const T* base = (const T*)a.q + b * a.q_sb + h * a.q_sh;
  Row8<T> rows[RB];
  const int r0 = qb * a.bs, r1 = min((qb + 1) * a.bs, a.tq);
  if constexpr (std::is_same<T, bf16_t>::value && D == 128) {
    if (r1 - r0 == RB * (NTHR / (D / 8))) {
      block_mean_full128(base + r0 * a.q_st, a.q_st, red, mean, rows);
    } else {
      block_mean<T, D>(base, a.q_st, r0, r1, red, mean, rows);
    }
  } else {
    block_mean<T, D>(base, a.q_st, r0, r1, red, mean, rows);
  }
  if (threadIdx.x < D) a.qmean[(bh * a.nqb + qb) * D + threadIdx.x] = mean[threadIdx.x];
  if (a.keep_mean >= 0.0) write_norm2<D>(mean, a.norm2 + bh * a.nqb + qb);
}

template <typename T, int D>
__device__ __forceinline__ void kstats_block(const SelectArgs& a, int id, double* red, double* cent, double* rmax) {
  const int kb = id % a.nkb;
  const int kvh = (id / a.nkb) % a.Hkv;
  const int b = id / (a.nkb * a.Hkv);
  const int tkb = seq_off(a, b) + a.tq;
  double* crow = a.cent + (((int64_t)b * a.Hkv + kvh) * a.nkb + kb) * D;  // centroids row-major
  if (kb * a.bs >= tkb) {  // block beyond this sequence's keys
    if (threadIdx.x < D) crow[threadIdx.x] = 0.0;
    if (threadIdx.x == 0) {
      a.rad2[((int64_t)b * a.Hkv + kvh) * a.nkb + kb] = SOC_NEG_INF;
      if (a.keep_mean >= 0.0) a.norm2[(int64_t)a.B * a.Hq * a.nqb + ((int64_t)b * a.Hkv + kvh) * a.nkb + kb] = 0.0;
    }
    return;
  }
  const T* base = (const T*)a.k + b * a.k_sb + kvh * a.k_sh;
  const int r0 = kb * a.bs, r1 = min((kb + 1) * a.bs, tkb);
  Row8<T> rows[RB];
  bool kept;
  if constexpr (std::is_same<T, bf16_t>::value && D == 128) {
    if (r1 - r0 == RB * (NTHR / (D / 8))) {
      block_mean_full128(base + r0 * a.k_st, a.k_st, red, cent, rows);
      kept = true;
    } else {
      kept = block_mean<T, D>(base, a.k_st, r0, r1, red, cent, rows);
    }
  } else {
    kept = block_mean<T, D>(base, a.k_st, r0, r1, red, cent, rows);
  }
  if (threadIdx.x < D) crow[threadIdx.x] = cent[threadIdx.x];
  if (a.keep_mean >= 0.0)
    write_norm2<D>(cent, a.norm2 + (int64_t)a.B * a.Hq * a.nqb + ((int64_t)b * a.Hkv + kvh) * a.nkb + kb);

  constexpr int C = D / 8, RG = NTHR / C;
  const int c = threadIdx.x % C, rg = threadIdx.x / C;
  double cv[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) cv[e] = cent[8 * c + e];
  double best = SOC_NEG_INF;
  for (int rb = r0 + rg; rb < r0 + rg + ((r1 - r0 + RB * RG - 1) / (RB * RG)) * RB * RG; rb += RB * RG) {
    // same trip count in every lane (the row-group reduction below shuffles)
    if (!kept) {
#pragma unroll
      for (int u = 0; u < RB; ++u) {
        const int r = rb + u * RG;
        if (r < r1) rows[u].load(base + (int64_t)r * a.k_st + 8 * c);
      }
    }
    double part[RB];
#pragma unroll
    for (int u = 0; u < RB; ++u) {
      const int r = rb + u * RG;
      part[u] = 0.0;
      if (r < r1) {
        double x[8];
        rows[u].widen(x);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const double dlt = x[e] - cv[e];
          part[u] = fma(dlt, dlt, part[u]);
        }
      }
    }
    if (C == 16) {
      // Reduce-scatter of the 8 rows' partial sums over the 16 lanes of the row group in four
      // DPP exchanges: each round a lane keeps half of its rows (by one bit of its index) and
      // adds the partner's values for them; afterwards lanes 2m and 2m + 1 both hold row
      // slot m's full sum (m = bits 3..1 of the lane index).
      const int i = threadIdx.x & 15;
      double k4[4], k2[2], k1;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const bool up = i & 8;
        const double keep = up ? part[4 + t] : part[t], send = up ? part[t] : part[4 + t];
        k4[t] = keep + dpp_f64<DPP_ROR8>(send);
      }
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const bool up = i & 4;
        const double keep = up ? k4[2 + t] : k4[t], send = up ? k4[t] : k4[2 + t];
        k2[t] = keep + dpp_f64<DPP_HALF_MIRROR>(send);
      }
      {
        const bool up = i & 2;
        const double keep = up ? k2[1] : k2[0], send = up ? k2[0] : k2[1];
        k1 = keep + dpp_f64<DPP_XOR2>(send);
      }
      // (addition commutes exactly, so both lanes of the pair get the same sum; the exchange
      // runs in every lane: a DPP move under a partial exec mask would read disabled lanes)
      const double total = k1 + dpp_f64<DPP_XOR1>(k1);
      if (rb + ((i >> 1) & 7) * RG < r1) best = fmax(best, total);
    } else {
#pragma unroll
      for (int u = 0; u < RB; ++u) {
        double pu = part[u];
#pragma unroll
        for (int m = 1; m < C; m <<= 1) pu += __shfl_xor(pu, m, 64);
        if (rb + u * RG < r1) best = fmax(best, pu);
      }
    }
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) best = fmax(best, __shfl_xor(best, m, 64));
  if ((threadIdx.x & 63) == 0) rmax[threadIdx.x >> 6] = best;
  __syncthreads();
  if (threadIdx.x == 0)
    a.rad2[((int64_t)b * a.Hkv + kvh) * a.nkb + kb] = fmax(fmax(rmax[0], rmax[1]), fmax(rmax[2], rmax[3]));
}

// Steps 1 and 2 in one grid: the first B*Hq*nqb workgroups take query blocks, the rest key
// blocks, so the key blocks' second (radius) pass hides inside the query stream.
template <typename T, int D>
__global__ void __launch_bounds__(NTHR) stats_kernel(SelectArgs a) {
  __shared__ double red[NTHR * 8];
  __shared__ double vec[D];
  __shared__ double rmax[NTHR / 64];
  const int nq = a.B * a.Hq * a.nqb;
  if ((int)blockIdx.x < nq)
    qmean_block<T, D>(a, blockIdx.x, red, vec);
  else
    kstats_block<T, D>(a, blockIdx.x - nq, red, vec, rmax);
}

// The monotone map from an admissible s1 to its histogram bucket.  |s1| <= M by
// Cauchy-Schwarz; the map need not be exact at the ends because it clamps, and a degenerate
// M (zero or huge) sends everything to bucket 0, which stays correct (just not narrowing).
struct BucketMap {
  double lo, scale;
  __device__ BucketMap(const SelectArgs& a, int64_t bh, int64_t bkv)
      : BucketMap(a.nmax[bh], a.nmax[(int64_t)a.B * a.Hq + bkv]) {}
  // from the largest |qmean|^2 of the head and the largest |c|^2 of its KV head
  __device__ BucketMap(double m2q, double m2c) {
    const double m = sqrt(m2q) * sqrt(m2c);
    const bool ok = m > 0.0 && m < 1e300;
    lo = ok ? -m : 0.0;
    scale = ok ? (double)kSelBuckets / (2.0 * m) : 0.0;
  }
  __device__ __forceinline__ int operator()(double v) const {
    const double x = (v - lo) * scale;  // non-decreasing in v; NaN only when scale == 0
    return x >= 1.0 ? (x < (double)kSelBuckets ? (int)x : kSelBuckets - 1) : 0;
  }
};

// Workgroup i runs on XCD i % 8.  Renumbers the n workgroups of a grid so that each XCD takes
// one contiguous range of work items: neighbouring items (the tiles of one head, the heads of
// one KV head) share their inputs, which then stay in that XCD's L2.
__device__ __forceinline__ int xcd_contiguous(int bid, int n) {
  const int x = bid & 7, j = bid >> 3, q = n >> 3, r = n & 7;
  return x * q + min(x, r) + j;
}

typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef __attribute__((address_space(3))) const f64x2 lds_f64x2;
typedef __attribute__((address_space(3))) const double lds_cdouble;

// Waits go through the s_waitcnt builtin (gfx9 encoding: vmcnt in bits 3:0 and 15:14,
// expcnt 6:4, lgkmcnt 11:8): the compiler treats it as touching all memory and adds no drain
// of its own for what it already waited for.
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N <= 63, "vmcnt counts at most 63 loads");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}


// A workgroup barrier with no memory fence: __syncthreads() also releases at workgroup scope,
// which drains every pending load and store (vmcnt(0)), and would drain the centroid slices
// in flight.  Where this is used, each wave has waited for the LDS data the others will read
// (its own slice loads, by count) and has consumed every LDS read it issued before the barrier
// (their values feed MFMAs issued before it); the memory clobber keeps the compiler from
// moving memory accesses across it.
__device__ __forceinline__ void barrier_nofence() { asm volatile("s_barrier" ::: "memory"); }

// Score work items.  Rows are the query blocks of the heads that share one KV head, stacked
// (row hl * nqb + qb for the hl-th head of the group: qmean and score rows of those heads are
// consecutive in memory, so a stacked row is also a memory row).  With the histogram on, a
// row tile holds at most 64 rows of one head (ntq per head); otherwise any 64 consecutive
// stacked rows (short query ranges, such as a chunk of a few query blocks, then fill the
// MFMA rows with the group's heads).  Key chunks are kct key tiles of 64 blocks.
struct ScoreGrid {
  int ntq, nrt, ntk, nkc;
  __host__ __device__ ScoreGrid(int g, int nqb, int nkb, bool hist, int kct) {
    ntq = (nqb + 63) / 64;
    nrt = hist ? g * ntq : (g * nqb + 63) / 64;
    ntk = (nkb + 63) / 64;
    nkc = (ntk + kct - 1) / kct;
  }
};

// A score work item: the stacked rows [r0, r1) of (b, kv head) (hl: their head within the
// group, with the histogram on), key tiles [kt0, kt1), and amask: the tiles of those that can
// hold an admissible pair.  The admissible blocks of the item's query blocks qb_min .. qb_max lie
// in [lo(qb_min), hi(qb_max)] (lo and hi do not decrease with qb; rows spanning two heads take
// all query blocks), so a tile outside that range has none; a tile inside it that has none is
// computed and gets -inf.
struct ScoreItem {
  int b, kvh, rt, kc, r0, r1, hl, kt0, kt1, off, tkb;
  unsigned amask;
};
__device__ __forceinline__ ScoreItem score_item_at(const SelectArgs& a, const ScoreGrid& sg, bool hist, int kct, int id) {
  ScoreItem it;
  it.kc = id % sg.nkc;
  id /= sg.nkc;
  it.rt = id % sg.nrt;
  id /= sg.nrt;
  it.kvh = id % a.Hkv;
  it.b = id / a.Hkv;
  it.hl = 0;
  if (hist) {
    it.hl = it.rt / sg.ntq;
    it.r0 = it.hl * a.nqb + (it.rt - it.hl * sg.ntq) * 64;
    it.r1 = min(it.r0 + 64, (it.hl + 1) * a.nqb);
  } else {
    it.r0 = it.rt * 64;
    it.r1 = min(it.r0 + 64, a.g * a.nqb);
  }
  it.off = seq_off(a, it.b);
  it.tkb = it.off + a.tq;
  it.kt0 = it.kc * kct;
  it.kt1 = min(it.kt0 + kct, sg.ntk);
  int qb_min = it.r0 % a.nqb, qb_max = (it.r1 - 1) % a.nqb;
  if (it.r1 - it.r0 > a.nqb || qb_min > qb_max) {
    qb_min = 0;
    qb_max = a.nqb - 1;
  }
  int klo, khi, tmp;
  adm_range(a, it.off, it.tkb, qb_min, klo, tmp);
  adm_range(a, it.off, it.tkb, qb_max, tmp, khi);
  it.amask = 0;
  for (int kt = max(it.kt0, klo / 64); kt < min(it.kt1, khi / 64 + 1); ++kt) it.amask |= 1u << (kt - it.kt0);
  return it;
}

// Calls f(std::integral_constant<int, I>) for I = B .. N - 1 in order.
template <int B, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < N) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, N>(f);
  }
}

// s1 = <qmean, c> on the fp64 MFMA (v_mfma_f64_16x16x4f64: A[i][k] in lane i + 16k, B[k][j]
// in lane j + 16k, D[i][j] in lane j + 16 (i % 4), element i / 4), stored for the pairs of
// every key tile that can hold an admissible pair (-inf at pairs that are not admissible);
// tiles with none are skipped (their scores are never read).  One work item at a time per
// workgroup: up to 64 stacked rows (wave w: rows 16w .. 16w + 15, its query means held in
// registers) times KC key tiles of 64 key blocks.  Each key tile's centroids stream through
// LDS by DMA in NCH slices of CD dims, shared by the 4 waves: slice ch of every tile has its
// own LDS array, chosen at compile time (so the compiler sees which DMA a read depends on),
// refilled with the next tile's slice ch as soon as all waves are past it, which keeps up to
// NCH - 2 slices in flight beside the one in use.  A slice's 16-byte pieces are stored
// XOR-swizzled by column so that the 16 lanes reading one piece index of 16 columns hit
// distinct banks.  At MFMA step s of a slice, lane (i, k) feeds dim E*k + s.
// With the histogram on (HIST), an item's rows stay in one head; the item forms the head's
// bucket map bound M from the squared norms (every item of the head finds the same M and
// writes it to nmax) and counts its admissible s1 into a per-item value histogram of u16
// pairs.
// Ordering: register loads and LDS-DMA loads each complete in issue order, but not in order
// with each other.  An item's register loads (norms, query means) go out first and its first
// tile's slices after them; the first wait drains everything, so afterwards the only loads
// are slice refills, one ordered stream, and a slice has landed once no more than the slice
// loads issued after it remain (pending stores only add to the count; where the compiler adds
// a drain of its own after a tile's stores, it only waits longer).
template <int D, int KC, bool HIST>
__global__ void __launch_bounds__(NTHR, 2) score_kernel(SelectArgs a, int nitems) {
  constexpr int CD = D < 32 ? D : 32;  // dims per centroid slice
  constexpr int NCH = D / CD;          // slices per key tile
  constexpr int E = CD / 4;            // MFMA steps per slice; a lane's dims in a slice
  constexpr int PR = CD / 2;           // 16-byte pieces per column of a slice
  constexpr int PQ = E / 2;            // pieces a lane reads per column subtile and slice
  constexpr int NDMA = PR / 4;         // DMA instructions per thread per slice (1 KB each per wave)
  static_assert(NCH <= 4, "at most 4 slices per key tile");
  __shared__ __attribute__((aligned(16))) double st0[64 * CD];
  __shared__ __attribute__((aligned(16))) double st1[NCH > 1 ? 64 * CD : 2];
  __shared__ __attribute__((aligned(16))) double st2[NCH > 2 ? 64 * CD : 2];
  __shared__ __attribute__((aligned(16))) double st3[NCH > 3 ? 64 * CD : 2];
  __shared__ uint32_t h2[HIST ? kSelBuckets / 2 : 1];
  __shared__ double red[2][NTHR / 64];
  typedef __attribute__((address_space(3))) uint32_t lds_u32;

  const int G = a.g, nqb = a.nqb, nkb = a.nkb;
  const ScoreGrid sg(G, nqb, nkb, HIST, KC);
  // (the wave index made visibly uniform: the DMA's LDS address is a scalar operand)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int li = lane & 15, lk = lane >> 4;

  auto score_item = [&](int id) __attribute__((always_inline)) {
    const ScoreItem it = score_item_at(a, sg, HIST, KC, id);
    const int r0 = it.r0, r1 = it.r1, hl = it.hl, kt0 = it.kt0, off = it.off, tkb = it.tkb;
    const int64_t rowbase = ((int64_t)it.b * a.Hq + (int64_t)it.kvh * G) * nqb;  // memory row of stacked row 0
    const int64_t bkv = (int64_t)it.b * a.Hkv + it.kvh;
    const bool wrows = r0 + 16 * wave < r1;  // the wave has rows in the item
    const unsigned amask = __builtin_amdgcn_readfirstlane(it.amask);  // (uniform: keeps what follows scalar)
    int64_t item = 0, bh = 0;
    if (HIST) {
      bh = (int64_t)it.b * a.Hq + (int64_t)it.kvh * G + hl;
      item = bh * ((int64_t)sg.ntq * sg.nkc) + (int64_t)(it.rt - hl * sg.ntq) * sg.nkc + it.kc;
      if (threadIdx.x == 0) a.tflag[item] = amask != 0;
    }
    if (amask == 0) return;

    // Register loads first: the squared norms for the bucket map bound, the wave's query means
    // (lane (i, k) holds dims ch * CD + E k + s of row r0 + 16 wave + i).
    constexpr int NM = 4;  // norms per thread loaded up front
    double nqv[NM], ncv[NM];
    const double* nq = a.norm2 + bh * nqb;
    const double* nc = a.norm2 + (int64_t)a.B * a.Hq * nqb + bkv * nkb;
    if constexpr (HIST) {
#pragma unroll
      for (int u = 0; u < NM; ++u) {
        const int iq = threadIdx.x + u * NTHR;
        nqv[u] = iq < nqb ? nq[iq] : 0.0;
        ncv[u] = iq < nkb ? nc[iq] : 0.0;
      }
    }
    double A[NCH][E];
    if (wrows) {
      const int ra = min(r0 + 16 * wave + li, r1 - 1);
      const double* qr = a.qmean + (rowbase + ra) * D;
#pragma unroll
      for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
        for (int e2 = 0; e2 < E / 2; ++e2) {
          const f64x2 x = *(const f64x2*)(qr + ch * CD + E * lk + 2 * e2);
          A[ch][2 * e2] = x[0];
          A[ch][2 * e2 + 1] = x[1];
        }
    }

    // the centroid rows of this KV head as a buffer (base made visibly uniform: a descriptor the
    // compiler takes for divergent is applied lane group by lane group)
    const uint64_t cbase = (uint64_t)(a.cent + bkv * nkb * D);
    const uint64_t cbu = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(cbase >> 32)) << 32) |
                         (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)cbase);
    const __amdgpu_buffer_rsrc_t crs =
        __builtin_amdgcn_make_buffer_rsrc((void*)cbu, (short)0, __builtin_amdgcn_readfirstlane(nkb * D * 8), 0x00020000);
    auto tile_of = [&](int n) __attribute__((always_inline)) -> int {  // the n-th key tile of amask
      unsigned m = amask;
      for (int s = 0; s < n; ++s) m &= m - 1;
      return kt0 + __builtin_ctz(m);
    };
    auto stage = [&](auto tag) __attribute__((always_inline)) -> double* {
      constexpr int I = decltype(tag)::value;
      if constexpr (I == 0)
        return st0;
      else if constexpr (I == 1)
        return st1;
      else if constexpr (I == 2)
        return st2;
      else
        return st3;
    };
    // Slice c (key tile c / NCH of the item's active tiles, dims tag * CD ..) into its array.
    // Wave instruction m fills columns m * (64 / PR) ..; lane l's piece lands at column
    // m * (64 / PR) + l / PR, physical piece l % PR, and holds logical piece
    // (l % PR) ^ (column % PR).  Columns past the last key block repeat it (never written out).
    auto issue = [&](int c, auto tag) __attribute__((always_inline)) {
      constexpr int ch = decltype(tag)::value;
      const int kt = tile_of(c / NCH);
      double* st = stage(tag);
#pragma unroll
      for (int u = 0; u < NDMA; ++u) {
        const int m = wave * NDMA + u;
        const int col = m * (64 / PR) + lane / PR;
        const int p = (lane % PR) ^ (col % PR);
        const int kb = min(kt * 64 + col, nkb - 1);
        const uint32_t voff = (uint32_t)((kb * D + ch * CD + 2 * p) * 8);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(crs, (lds_void_ptr)(st + m * 128), 16, voff, 0, 0, 0);
      }
    };

    const int nact = __builtin_popcount(amask), nsl = nact * NCH;
    static_for<0, NCH>([&](auto tag) __attribute__((always_inline)) { issue(decltype(tag)::value, tag); });

    // this lane's outputs: rows r0 + 16 wave + 4 v + lk (admissible key blocks lov .. hiv),
    // key blocks kt * 64 + 16 cs + li
    int lov[4], hiv[4];
    bool rv[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int r = r0 + 16 * wave + 4 * v + lk;
      rv[v] = r < r1;
      adm_range(a, off, tkb, rv[v] ? r % nqb : 0, lov[v], hiv[v]);
    }
    if constexpr (HIST)
      for (int i = threadIdx.x; i < kSelBuckets / 2; i += NTHR) h2[i] = 0;

    f64x4 acc[4];
#pragma unroll
    for (int cs = 0; cs < 4; ++cs) acc[cs] = f64x4{0.0, 0.0, 0.0, 0.0};
    BucketMap bucket(0.0, 0.0);
    double* out = a.score + rowbase * nkb;
    static_for<0, KC>([&](auto ttag) __attribute__((always_inline)) {
      constexpr int ti = decltype(ttag)::value;
      if (ti >= nact) return;
      static_for<0, NCH>([&](auto tag) __attribute__((always_inline)) {
        constexpr int ch = decltype(tag)::value;
        const int c = ti * NCH + ch;
        if (c == 0) {
          // everything issued so far has landed (register loads and the first tile)
          vm_wait<0>();
          if constexpr (HIST) {  // the maxima of the squared norms, across the workgroup at the barrier
            double mq = 0.0, mc = 0.0;
#pragma unroll
            for (int u = 0; u < NM; ++u) {
              mq = fmax(mq, nqv[u]);
              mc = fmax(mc, ncv[u]);
            }
            for (int i = threadIdx.x + NM * NTHR; i < nqb; i += NTHR) mq = fmax(mq, nq[i]);
            for (int i = threadIdx.x + NM * NTHR; i < nkb; i += NTHR) mc = fmax(mc, nc[i]);
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) {
              mq = fmax(mq, __shfl_xor(mq, o, 64));
              mc = fmax(mc, __shfl_xor(mc, o, 64));
            }
            if (lane == 0) {
              red[0][wave] = mq;
              red[1][wave] = mc;
            }
          }
          __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));  // lgkmcnt(0): LDS writes done
          barrier_nofence();
          if constexpr (HIST) {
            const double mq = fmax(fmax(red[0][0], red[0][1]), fmax(red[0][2], red[0][3]));
            const double mc = fmax(fmax(red[1][0], red[1][1]), fmax(red[1][2], red[1][3]));
            if (threadIdx.x == 0) {
              a.nmax[bh] = mq;
              a.nmax[(int64_t)a.B * a.Hq + bkv] = mc;
            }
            bucket = BucketMap(mq, mc);
          }
        } else if (NCH == 1) {  // one slice per tile: refill once everyone is done with the last
          barrier_nofence();
          issue(c, tag);
          vm_wait<0>();
          barrier_nofence();
        } else {
          // slice c has landed once no more than the slice loads issued after it remain:
          // min(NCH - 2, nsl - 1 - c) slices
          const int after = min(NCH - 2, nsl - 1 - c);
          if (after >= 2)
            vm_wait<2 * NDMA>();
          else if (after == 1)
            vm_wait<NDMA>();
          else
            vm_wait<0>();
          // then every wave's slice c has landed and every wave is done with slice c - 1, whose
          // array takes slice c + NCH - 1 (the next tile's slice of the same index)
          barrier_nofence();
          if (c + NCH - 1 < nsl) issue(c + NCH - 1, std::integral_constant<int, (ch + NCH - 1) % NCH>{});
        }
        if (wrows) {
          const double* st = stage(tag);
#pragma unroll
          for (int q = 0; q < PQ; ++q) {
            f64x2 bq[4];
#pragma unroll
            for (int cs = 0; cs < 4; ++cs) {
              const int col = 16 * cs + li;
              bq[cs] = *(lds_f64x2*)((lds_cdouble*)st + col * CD + 2 * ((PQ * lk + q) ^ (col % PR)));
            }
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
              for (int cs = 0; cs < 4; ++cs)
                acc[cs] = __builtin_amdgcn_mfma_f64_16x16x4f64(A[ch][2 * q + s2], bq[cs][s2], acc[cs], 0, 0, 0);
          }
        }
      });
      // The tile's histogram counts (an LDS-typed atomic: the compiler sees it is no DMA
      // target), then its scores (an LDS update placed after a store would wait for it).
      if (wrows) {
        const int kt = tile_of(ti);
        if constexpr (HIST) {
#pragma unroll
          for (int v = 0; v < 4; ++v)
#pragma unroll
            for (int cs = 0; cs < 4; ++cs) {
              const int kb = kt * 64 + 16 * cs + li;
              if (rv[v] && kb >= lov[v] && kb <= hiv[v]) {  // (hiv < nkb)
                const int bk = bucket(acc[cs][v]);
                __hip_atomic_fetch_add((lds_u32*)(h2 + (bk >> 1)), (bk & 1) ? 65536u : 1u, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_WORKGROUP);
              }
            }
        }
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
          for (int cs = 0; cs < 4; ++cs) {
            const int kb = kt * 64 + 16 * cs + li;
            if (rv[v] && kb < nkb)
              out[(int64_t)(r0 + 16 * wave + 4 * v + lk) * nkb + kb] =
                  kb >= lov[v] && kb <= hiv[v] ? acc[cs][v] : SOC_NEG_INF;
          }
      }
#pragma unroll
      for (int cs = 0; cs < 4; ++cs) acc[cs] = f64x4{0.0, 0.0, 0.0, 0.0};
    });
    // The item's histogram: its LDS updates complete, then the barrier (the stores stay in
    // flight).  A second barrier ends the item: every wave is done with the slices and LDS
    // before the next item's DMA and clearing reuse them.
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));  // lgkmcnt(0)
    if constexpr (HIST) {
      barrier_nofence();
      u32x4* dst = (u32x4*)(a.hpart + item * (kSelBuckets / 2)) + 2 * threadIdx.x;
      dst[0] = *(const u32x4*)(h2 + 8 * threadIdx.x);
      dst[1] = *(const u32x4*)(h2 + 8 * threadIdx.x + 4);
      __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));
    }
    barrier_nofence();
  };

  // The workgroups are persistent.  Items, in (b, kv head, row tile, key chunk) order, are cut
  // into 8 contiguous ranges; workgroup i takes range i % 8 (the XCD it runs on: neighbouring
  // items share inputs in that XCD's L2), as the (i / 8)-th of the range's n workgroups, which
  // take its items in snake order (j, 2n - 1 - j, 2n + j, ...: neighbouring items have similar
  // work, so a workgroup's heavy and light items pair up).
  const int gx = blockIdx.x & 7, gj = blockIdx.x >> 3, gn = ((int)gridDim.x - gx + 7) >> 3;
  const int rq = nitems >> 3, rr = nitems & 7;
  const int rbeg = gx * rq + min(gx, rr), rlen = rq + (gx < rr ? 1 : 0);
  for (int m = 0;; ++m) {
    const int k = m * gn + ((m & 1) ? gn - 1 - gj : gj);
    if (k >= rlen) break;
    score_item(rbeg + k);
  }
}

// Wave-wide search in descending value order.  Lane l holds the count c of the l-th of 64
// consecutive value ranges (higher lane = higher values).  Returns the lane L whose range
// holds descending rank `target` (< the wave total), with *above = the count in the lanes
// above L and *total = the wave total.
__device__ __forceinline__ int wave_locate_desc(unsigned long long c, unsigned long long target, unsigned long long* above,
                                unsigned long long* total) {
  const int lane = threadIdx.x & 63;
  unsigned long long s = c;  // inclusive suffix sum over lanes >= this one
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const unsigned long long y = __shfl_down(s, o, 64);
    if (lane + o < 64) s += y;
  }
  const unsigned long long ab = s - c;
  *total = __shfl(s, 0, 64);
  const unsigned long long own = __ballot(ab <= target && target < s);
  const int L = own ? __ffsll(own) - 1 : 0;
  *above = __shfl(ab, L, 64);
  return L;
}


// Exact value at descending rank `rank` (0 = largest) among the finite values of nseg
// segments: vals[s * seg_len + i] for i < counts[s] (one segment when counts is null, count
// values).  8 passes of an 8-bit radix select on order-preserving keys, T threads.
template <int T>
__device__ __forceinline__ double select_desc(const double* vals, int64_t count, const unsigned* counts, int nseg, int64_t seg_len,
                              unsigned long long rank, unsigned* hist, unsigned long long* su) {
  unsigned long long prefix = 0, pmask = 0;
  for (int shift = 56; shift >= 0; shift -= 8) {
    for (int i = threadIdx.x; i < 256; i += T) hist[i] = 0;
    __syncthreads();
    for (int sg = 0; sg < (counts ? nseg : 1); ++sg) {
      const int64_t cnt = counts ? (int64_t)counts[sg] : count;
      const double* v = vals + sg * seg_len;
      for (int64_t i = threadIdx.x; i < cnt; i += T) {
        const double x = v[i];
        if (!(x > SOC_NEG_INF)) continue;
        const uint64_t key = f64_order_key(x);
        if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
      }
    }
    __syncthreads();
    if (threadIdx.x < 64) {  // wave 0 picks the digit: lane l covers digits 4l..4l+3
      const int l = threadIdx.x;
      const unsigned long long c =
          (unsigned long long)hist[4 * l] + hist[4 * l + 1] + hist[4 * l + 2] + hist[4 * l + 3];
      unsigned long long above = 0, total = 0;
      const int L = wave_locate_desc(c, rank, &above, &total);
      unsigned long long r = rank - above;
      int e = 3;
      for (; e > 0; --e) {
        const unsigned h = hist[4 * L + e];
        if (r < h) break;
        r -= h;
      }
      if (l == 0) {
        su[0] = r;
        su[1] = prefix | ((unsigned long long)(4 * L + e) << shift);
      }
    }
    __syncthreads();
    rank = su[0];
    prefix = su[1];
    pmask |= 255ull << shift;
    __syncthreads();
  }
  return f64_from_order_key(prefix);
}

constexpr int CAND_LDS = 2048;  // values selected in LDS (more: straight from memory)
constexpr int CAND_COUNT = 128;  // at most this many candidates: selected by counting
constexpr int LB = 1024;         // buckets of the in-LDS narrowing

// Value at descending rank `rank` (0 = largest) among the finite values of v[0 .. n), held in
// LDS (-inf marks an absent value; rank < their count).  A monotone map of [min, max] of the
// values onto LB buckets narrows the search to the bucket holding the rank (every value of a
// higher bucket is strictly larger); that bucket's values, usually a handful, are ranked by
// counting (a value with g values above it and e equal to it, itself included, holds the
// descending ranks g .. g + e - 1); a bucket of more than CAND_COUNT values goes to the radix
// select over all values.  T threads.  LDS scratch: lb[LB], cand[CAND_COUNT], red[2 * T / 64],
// su[2].
template <int T>
__device__ __forceinline__ double select_lds(const double* v, int n, unsigned long long rank, unsigned* lb, double* cand, double* red,
                             unsigned long long* su) {
  constexpr int NW = T / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  double lo = __builtin_inf(), hi = -__builtin_inf();
  for (int i = threadIdx.x; i < n; i += T) {
    const double x = v[i];
    if (x > SOC_NEG_INF) {
      lo = fmin(lo, x);
      hi = fmax(hi, x);
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    lo = fmin(lo, __shfl_xor(lo, o, 64));
    hi = fmax(hi, __shfl_xor(hi, o, 64));
  }
  if (lane == 0) {
    red[wave] = lo;
    red[NW + wave] = hi;
  }
  for (int i = threadIdx.x; i < LB; i += T) lb[i] = 0;
  __syncthreads();
  lo = red[0];
  hi = red[NW];
  for (int w = 1; w < NW; ++w) {
    lo = fmin(lo, red[w]);
    hi = fmax(hi, red[NW + w]);
  }
  // non-decreasing in x; a zero scale (all equal, or a span that overflows) sends every value
  // to bucket 0, which is still correct
  const double span = hi - lo;
  const double scale = span > 0.0 && span < 1e300 ? (double)LB / span : 0.0;
  auto bucket = [&](double x) __attribute__((always_inline)) -> int {
    const double y = (x - lo) * scale;
    return y >= 1.0 ? (y < (double)LB ? (int)y : LB - 1) : 0;
  };
  for (int i = threadIdx.x; i < n; i += T) {
    const double x = v[i];
    if (x > SOC_NEG_INF) atomicAdd(&lb[bucket(x)], 1u);
  }
  __syncthreads();
  if (threadIdx.x < 64) {  // wave 0: lane l covers buckets 16 l .. 16 l + 15
    unsigned long long c = 0;
#pragma unroll
    for (int e = 0; e < 16; ++e) c += lb[16 * lane + e];
    unsigned long long above = 0, total = 0;
    const int L = wave_locate_desc(c, rank, &above, &total);
    unsigned long long r = rank - above;
    int e = 15;
    for (; e > 0; --e) {
      const unsigned h = lb[16 * L + e];
      if (r < h) break;
      r -= h;
    }
    if (lane == 0) {
      su[0] = r;
      su[1] = 16 * L + e;
    }
  }
  __syncthreads();
  const unsigned long long rin = su[0];
  const int beta = (int)su[1];
  const unsigned cnt = lb[beta];
  __syncthreads();
  if (cnt > (unsigned)CAND_COUNT) return select_desc<T>(v, n, nullptr, 1, 0, rank, lb, su);
  if (threadIdx.x == 0) su[0] = 0;
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += T) {
    const double x = v[i];
    if (x > SOC_NEG_INF && bucket(x) == beta) cand[atomicAdd(&su[0], 1ull)] = x;
  }
  __syncthreads();
  if (threadIdx.x < cnt) {
    const double x = cand[threadIdx.x];
    unsigned g = 0, e = 0;
    for (unsigned j = 0; j < cnt; ++j) {
      const double y = cand[j];
      g += y > x;
      e += y == x;
    }
    if (g <= rin && rin < g + e) red[0] = x;  // values equal to it write the same
  }
  __syncthreads();
  return red[0];
}


// Per (b, kv head): tau_radius = the (n+1)-th largest finite rad2 over the key blocks, n =
// floor(keep_radius * N + 1/2) of the N finite ones (-inf when n >= N).  The values go to
// LDS first when they fit (then the search never waits on memory).  T threads.
template <int T>
__device__ void radius_threshold(const SelectArgs& a, int id, double* cv, unsigned* lb, double* cand, double* red,
                                 unsigned long long* su) {
  const double* vals = a.rad2 + (int64_t)id * a.nkb;
  const bool in_lds = a.nkb <= CAND_LDS;
  if (threadIdx.x == 0) su[0] = 0;
  __syncthreads();
  unsigned long long local = 0;
  for (int i = threadIdx.x; i < a.nkb; i += T) {
    const double x = vals[i];
    if (in_lds) cv[i] = x;
    local += x > SOC_NEG_INF;
  }
  atomicAdd(&su[0], local);
  __syncthreads();
  const unsigned long long N = su[0];
  __syncthreads();
  const double nd = floor(a.keep_radius * (double)N + 0.5);
  double tau = SOC_NEG_INF;
  if (nd < (double)N)
    tau = in_lds ? select_lds<T>(cv, a.nkb, (unsigned long long)nd, lb, cand, red, su)
                 : select_desc<T>(vals, a.nkb, nullptr, 1, 0, (unsigned long long)nd, lb, su);
  if (threadIdx.x == 0) a.tau_radius[id] = tau;
}

// Per head: sums the item histograms of its admissible s1 (fixed item order), then finds the
// bucket that holds descending rank n = floor(keep * N + 1/2) and the rank inside it; writes
// (N, n, bucket or -1 when n >= N, rank) to pick.  One workgroup of 1024 threads per head,
// thread t owning buckets 4t .. 4t+3; items without admissible pairs are not read.  When a
// radius fraction is given, B*Hkv more workgroups at the end of the grid compute tau_radius.
constexpr int PICK_THR = 1024;
static_assert(kSelBuckets == 4 * PICK_THR, "four buckets per thread");
__global__ void __launch_bounds__(PICK_THR) pick_kernel(SelectArgs a) {
  __shared__ uint32_t hist[kSelBuckets];
  const int64_t nbh = (int64_t)a.B * a.Hq;
  if ((int64_t)blockIdx.x >= nbh) {  // the radius thresholds (needed by the mask pass)
    __shared__ double cv[CAND_LDS];
    __shared__ double cand[CAND_COUNT];
    __shared__ double red[2 * PICK_THR / 64];
    __shared__ unsigned long long su[2];
    radius_threshold<PICK_THR>(a, (int)(blockIdx.x - nbh), cv, hist, cand, red, su);
    return;
  }
  const int64_t bh = blockIdx.x;
  const int64_t nitems = sel_items_per_head(a.nqb, a.nkb);
  const u32x2* hp = (const u32x2*)(a.hpart + bh * nitems * (kSelBuckets / 2)) + threadIdx.x;
  const uint32_t* fl = a.tflag + bh * nitems;
  uint32_t c4[4] = {0u, 0u, 0u, 0u};
  auto add = [&](u32x2 w) __attribute__((always_inline)) {
    c4[0] += w[0] & 0xffffu;
    c4[1] += w[0] >> 16;
    c4[2] += w[1] & 0xffffu;
    c4[3] += w[1] >> 16;
  };
  constexpr int PF = 16;  // items' loads in flight
  for (int64_t c0 = 0; c0 < nitems; c0 += 64) {
    // the items of this group of 64 that hold data, as a wave-uniform bit set
    const int64_t ti = c0 + (threadIdx.x & 63);
    uint64_t m = __ballot(ti < nitems && fl[ti] != 0);
    while (m) {
      u32x2 w[PF];
#pragma unroll
      for (int u = 0; u < PF; ++u) {
        w[u] = u32x2{0u, 0u};
        if (m) {
          const int t = __builtin_ctzll(m);
          m &= m - 1;
          w[u] = hp[(c0 + t) * (kSelBuckets / 4)];
        }
      }
#pragma unroll
      for (int u = 0; u < PF; ++u) add(w[u]);
    }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) hist[4 * threadIdx.x + e] = c4[e];
  __syncthreads();
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    unsigned long long c = 0;
#pragma unroll
    for (int i = 0; i < 64; i += 4) {
      const u32x4 w = *(const u32x4*)(hist + 64 * lane + i);
      c += (unsigned long long)w[0] + w[1] + w[2] + w[3];
    }
    unsigned long long above1 = 0, N = 0;
    wave_locate_desc(c, 0, &above1, &N);  // N only
    const double nd = floor(a.keep_mean * (double)N + 0.5);
    long long sel[4] = {(long long)N, (long long)nd, -1, 0};
    if (nd < (double)N) {
      const unsigned long long n = (unsigned long long)nd;
      const int L1 = wave_locate_desc(c, n, &above1, &N);
      unsigned long long above2 = 0, n1 = 0;
      const int L2 = wave_locate_desc(hist[64 * L1 + lane], n - above1, &above2, &n1);
      sel[2] = 64 * L1 + L2;
      sel[3] = (long long)(n - above1 - above2);
    }
    if (lane < 4) a.pick[bh * 4 + lane] = sel[lane];
  }
}

// Per (b, h): tau_mean from the candidates mask_cand_kernel copied out of the picked bucket (a
// segment per query block row), at rank (n - the count above the bucket) among them: gathered
// into LDS when they fit (the usual case: a few dozen), else by the radix select straight from
// the segments.  Then the candidates above tau_mean are marked in the mask (written there by
// radius alone).
__global__ void __launch_bounds__(1024) threshold_kernel(SelectArgs a) {
  __shared__ unsigned lb[LB];
  __shared__ unsigned long long su[2];
  __shared__ unsigned wsum[16];
  __shared__ double cv[CAND_LDS];
  __shared__ int32_t cp[CAND_LDS];
  __shared__ double cand[CAND_COUNT];
  __shared__ double red[2 * 1024 / 64];
  const int64_t bh = blockIdx.x;
  const int64_t* pk = a.pick + bh * 4;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  double tau = SOC_NEG_INF;
  if (pk[2] >= 0) {
    const unsigned long long rank = (unsigned long long)pk[3];
    const unsigned* cnt = a.ccount + bh * a.nqb;
    const double* cnd = a.cand + bh * a.nqb * a.nkb;
    const int32_t* cps = a.cpos + bh * a.nqb * a.nkb;
    uint8_t* mask = a.mask + bh * a.nqb * a.nkb;
    // the rows' segments packed into LDS in row order (1024 rows per pass), while they fit
    unsigned total = 0;
    bool fits = true;
    for (int r0 = 0; r0 < a.nqb; r0 += 1024) {
      const int r = r0 + (int)threadIdx.x;
      const unsigned c = r < a.nqb ? cnt[r] : 0u;
      unsigned incl = c;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const unsigned y = __shfl_up(incl, o, 64);
        if (lane >= o) incl += y;
      }
      if (lane == 63) wsum[wave] = incl;
      __syncthreads();
      unsigned before = total, ptot = 0;
      for (int w = 0; w < 16; ++w) {
        before += w < wave ? wsum[w] : 0u;
        ptot += wsum[w];
      }
      const unsigned o = before + incl - c;
      if (o + c <= (unsigned)CAND_LDS)
        for (unsigned i = 0; i < c; ++i) {
          cv[o + i] = cnd[(int64_t)r * a.nkb + i];
          cp[o + i] = r * a.nkb + cps[(int64_t)r * a.nkb + i];
        }
      total += ptot;
      fits = fits && total <= (unsigned)CAND_LDS;
      __syncthreads();
    }
    if (fits) {
      tau = select_lds<1024>(cv, (int)total, rank, lb, cand, red, su);
      for (unsigned i = threadIdx.x; i < total; i += 1024)
        if (cv[i] > tau) mask[cp[i]] = 1;
    } else {
      tau = select_desc<1024>(cnd, 0, cnt, a.nqb, a.nkb, rank, lb, su);
      for (int r = 0; r < a.nqb; ++r)
        for (unsigned i = threadIdx.x; i < cnt[r]; i += 1024)
          if (cnd[(int64_t)r * a.nkb + i] > tau) mask[(int64_t)r * a.nkb + cps[(int64_t)r * a.nkb + i]] = 1;
    }
  }
  if (threadIdx.x == 0) a.tau_mean[bh] = tau;
}

// Per (b, h) when a head has at most CAND_LDS (query block, key block) pairs: tau_mean straight
// from its scores, held in LDS (-inf at pairs that are not admissible); the same n =
// floor(keep_mean * N + 1/2) over the N admissible ones.  When a radius fraction
// is given, the first B*Hkv workgroups compute tau_radius instead.
__global__ void __launch_bounds__(NTHR) threshold_direct_kernel(SelectArgs a) {
  __shared__ unsigned lb[LB];
  __shared__ unsigned long long su[2];
  __shared__ double cv[CAND_LDS];
  __shared__ double cand[CAND_COUNT];
  __shared__ double red[2 * NTHR / 64];
  const int nrad = a.keep_radius >= 0.0 ? a.B * a.Hkv : 0;
  if ((int)blockIdx.x < nrad) {
    radius_threshold<NTHR>(a, blockIdx.x, cv, lb, cand, red, su);
    return;
  }
  const int64_t bh = blockIdx.x - nrad;  // (launched only with a mean fraction)
  const int b = (int)(bh / a.Hq);
  const int off = seq_off(a, b), tkb = off + a.tq;
  const int P = a.nqb * a.nkb;
  const double* sc = a.score + bh * P;
  if (threadIdx.x == 0) su[0] = 0;
  __syncthreads();
  unsigned long long local = 0;
  for (int i = threadIdx.x; i < P; i += NTHR) {
    const int qb = i / a.nkb, kb = i - qb * a.nkb;
    const bool ok = admissible(a, off, tkb, qb, kb);
    cv[i] = ok ? sc[i] : SOC_NEG_INF;
    local += ok;
  }
  atomicAdd(&su[0], local);
  __syncthreads();
  const unsigned long long N = su[0];
  __syncthreads();
  const double nd = floor(a.keep_mean * (double)N + 0.5);
  const double tau = nd >= (double)N ? SOC_NEG_INF : select_lds<NTHR>(cv, P, (unsigned long long)nd, lb, cand, red, su);
  if (threadIdx.x == 0) a.tau_mean[bh] = tau;
}

// Large heads, after the pick: one wave per (b, h, query block) row reads the row's admissible
// s1 (and rad2; other pairs are not read) and writes the mask bytes: kept by mean when s1's
// bucket lies above the picked one (every admissible pair when tau_mean is -inf), not when it
// lies below; the picked bucket's values are undecided, written by radius alone and copied
// with their key block into the row's own candidate segment (count in ccount[row]), which the
// threshold kernel ranks and marks.
__global__ void __launch_bounds__(NTHR) mask_cand_kernel(SelectArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * (NTHR / 64) + (threadIdx.x >> 6);
  const int64_t rows = (int64_t)a.B * a.Hq * a.nqb;
  if (row >= rows) return;
  const int64_t bh = row / a.nqb;
  const int qb = (int)(row % a.nqb);
  const int h = (int)(bh % a.Hq), b = (int)(bh / a.Hq), kvh = h / a.g;
  const int64_t bkv = (int64_t)b * a.Hkv + kvh;
  const int off = seq_off(a, b), tkb = off + a.tq;
  int lo, hi;
  adm_range(a, off, tkb, qb, lo, hi);
  const long long beta = a.pick[bh * 4 + 2];
  const BucketMap bucket(a, bh, bkv);
  const double t2 = a.tau_radius[bkv];
  const double* sc = a.score + row * a.nkb;
  const double* r2 = a.rad2 + bkv * a.nkb;
  uint8_t* mrow = a.mask + row * a.nkb;
  double* cv = a.cand + row * a.nkb;
  int32_t* cp = a.cpos + row * a.nkb;
  unsigned nc = 0;  // the row's candidates so far
  // The mask bytes go out as one 8-byte store per lane (lane l: blocks 8l .. 8l + 7 of the
  // 512-block chunk, from the kept ballots) when the rows are 8-byte aligned.
  const bool vec = (a.nkb & 7) == 0 && ((uintptr_t)a.mask & 7) == 0;  // (uniform)
  constexpr int MB = 8;  // groups of 64 key blocks whose loads are in flight together
  for (int k0 = 0; k0 < a.nkb; k0 += 64 * MB) {
    double sv[MB], rr[MB];
    uint64_t kbal[MB];
#pragma unroll
    for (int u = 0; u < MB; ++u) {
      const int kb = k0 + 64 * u + lane;
      const bool ad = kb >= lo && kb <= hi;  // (hi < nkb)
      sv[u] = ad ? sc[kb] : 0.0;
      rr[u] = ad ? r2[kb] : 0.0;
    }
#pragma unroll
    for (int u = 0; u < MB; ++u) {
      const int kb = k0 + 64 * u + lane;
      const bool ad = kb >= lo && kb <= hi;
      bool kept = false, cand = false;
      if (ad) {
        if (beta < 0) {
          kept = true;
        } else {
          const int bk = bucket(sv[u]);
          kept = bk > (int)beta;
          cand = bk == (int)beta;
        }
        kept = kept || rr[u] > t2;
      }
      kbal[u] = __ballot(kept);
      if (!vec && kb < a.nkb) mrow[kb] = kept ? 1 : 0;
      const uint64_t bal = __ballot(cand);
      if (cand) {
        const unsigned o = nc + (unsigned)__popcll(bal & ((1ull << lane) - 1ull));
        cv[o] = sv[u];
        cp[o] = kb;
      }
      nc += (unsigned)__popcll(bal);
    }
    if (vec && k0 + 8 * lane < a.nkb) {
      uint64_t w = kbal[0];
#pragma unroll
      for (int u = 1; u < MB; ++u) w = (lane >> 3) == u ? kbal[u] : w;
      const unsigned bits = (unsigned)(w >> (8 * (lane & 7))) & 0xffu;
      uint64_t by = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) by |= (uint64_t)((bits >> i) & 1u) << (8 * i);
      *(uint64_t*)(mrow + k0 + 8 * lane) = by;
    }
  }
  if (lane == 0) a.ccount[row] = nc;
}

// One wave per (b, h, query block) row: the mask bytes and the ascending kept list, 64 key
// blocks per step with a ballot (no barriers).
__global__ void __launch_bounds__(NTHR) mask_kernel(SelectArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * (NTHR / 64) + (threadIdx.x >> 6);
  const int64_t rows = (int64_t)a.B * a.Hq * a.nqb;
  if (row >= rows) return;
  const int h = (int)((row / a.nqb) % a.Hq);
  const int b = (int)(row / ((int64_t)a.nqb * a.Hq));
  const int kvh = h / a.g;
  const int qb = (int)(row % a.nqb);
  const int off = seq_off(a, b), tkb = off + a.tq;
  const double* sc = a.score + row * a.nkb;
  const double* r2 = a.rad2 + ((int64_t)b * a.Hkv + kvh) * a.nkb;
  const double t1 = a.tau_mean[b * a.Hq + h];
  const double t2 = a.tau_radius[b * a.Hkv + kvh];
  uint8_t* mrow = a.mask + row * a.nkb;
  int32_t* lrow = a.list ? a.list + row * (1 + a.nkb) : nullptr;
  int base = 0;
  constexpr int MB = 8;  // groups of 64 key blocks whose loads are in flight together
  for (int k0 = 0; k0 < a.nkb; k0 += 64 * MB) {
    double sv[MB], rr[MB];
    bool ad[MB];
#pragma unroll
    for (int u = 0; u < MB; ++u) {  // (scores of pairs that are not admissible are not read)
      const int kb = k0 + 64 * u + lane;
      ad[u] = kb < a.nkb && admissible(a, off, tkb, qb, kb);
      sv[u] = ad[u] ? sc[kb] : 0.0;
      rr[u] = ad[u] ? r2[kb] : 0.0;
    }
#pragma unroll
    for (int u = 0; u < MB; ++u) {
      const int kb = k0 + 64 * u + lane;
      const bool kept = ad[u] && (sv[u] > t1 || rr[u] > t2);
      if (kb < a.nkb) mrow[kb] = kept ? 1 : 0;
      const unsigned long long bal = __ballot(kept);
      if (kept && lrow) lrow[1 + base + __popcll(bal & ((1ull << lane) - 1ull))] = kb;
      base += __popcll(bal);
    }
  }
  if (lane == 0 && lrow) lrow[0] = base;
}

// Kept lists from a byte mask: list[0] = the row's count, list[1..] = its kept key blocks in
// ascending order.  One wave per row; lane l takes the 8 consecutive blocks 8l .. 8l + 7 of
// each 512-block chunk (one 8-byte load when the rows are 8-byte aligned), and a wave prefix
// sum of the lanes' counts places each lane's blocks.
__global__ void __launch_bounds__(NTHR) list_from_mask_kernel(int64_t rows, int32_t n_kb, const uint8_t* mask,
                                                              int32_t* list) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * (NTHR / 64) + (threadIdx.x >> 6);
  if (row >= rows) return;
  const uint8_t* m = mask + row * n_kb;
  int32_t* lrow = list + row * (1 + (int64_t)n_kb);
  const bool vec = (n_kb & 7) == 0 && ((uintptr_t)mask & 7) == 0;  // (uniform)
  int base = 0;
  for (int k0 = 0; k0 < n_kb; k0 += 512) {
    const int kb0 = k0 + 8 * lane;
    unsigned bits = 0;  // bit i: block kb0 + i is kept
    if (vec) {
      const uint64_t by = kb0 < n_kb ? *(const uint64_t*)(m + kb0) : 0ull;
#pragma unroll
      for (int i = 0; i < 8; ++i) bits |= ((by >> (8 * i)) & 0xffu) ? 1u << i : 0u;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) bits |= (kb0 + i < n_kb && m[kb0 + i] != 0) ? 1u << i : 0u;
    }
    const int c = __popc(bits);
    int incl = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o, 64);
      if (lane >= o) incl += y;
    }
    int at = 1 + base + incl - c;
    while (bits) {
      lrow[at++] = kb0 + __builtin_ctz(bits);
      bits &= bits - 1;
    }
    base += __builtin_amdgcn_readlane(incl, 63);
  }
  if (lane == 0) lrow[0] = base;
}

template <typename T, int D>
hipError_t launch_select_d(const SelectArgs& a, hipStream_t s) {
  const unsigned gq = (unsigned)((int64_t)a.B * a.Hq * a.nqb);
  const unsigned gk = (unsigned)((int64_t)a.B * a.Hkv * a.nkb);
  const bool quant = a.keep_mean >= 0.0;
  const int64_t bh = (int64_t)a.B * a.Hq;
  const int64_t P = (int64_t)a.nqb * a.nkb;
  // Small heads (and given mean thresholds): tau_mean straight from the stored s1, then the
  // mask.  Large heads: s1 and its histograms, the pick, the mask with the picked bucket's
  // candidates, their rank.
  const bool hist = quant && P > CAND_LDS;
  const int64_t nrad = a.keep_radius >= 0.0 ? (int64_t)a.B * a.Hkv : 0;
  hipLaunchKernelGGL((stats_kernel<T, D>), dim3(gq + gk), dim3(NTHR), 0, s, a);
  if (!hist) {
    const ScoreGrid sg(a.g, a.nqb, a.nkb, false, 1);
    const int64_t items = (int64_t)a.B * a.Hkv * sg.nrt * sg.nkc;
    const unsigned swg = (unsigned)min(items, (int64_t)a.score_wgs);  // persistent workgroups
    hipLaunchKernelGGL((score_kernel<D, 1, false>), dim3(swg), dim3(NTHR), 0, s, a, (int)items);
    // the radius thresholds ride in the first workgroups of this grid
    const int64_t gt = nrad + (quant ? bh : 0);
    if (gt > 0) hipLaunchKernelGGL(threshold_direct_kernel, dim3((unsigned)gt), dim3(NTHR), 0, s, a);
    hipLaunchKernelGGL(mask_kernel, dim3((gq + NTHR / 64 - 1) / (NTHR / 64)), dim3(NTHR), 0, s, a);
  } else {
    const ScoreGrid sg(a.g, a.nqb, a.nkb, true, kScoreKC);
    const int64_t items = (int64_t)a.B * a.Hkv * sg.nrt * sg.nkc;
    const unsigned swg = (unsigned)min(items, (int64_t)a.score_wgs);
    hipLaunchKernelGGL((score_kernel<D, kScoreKC, true>), dim3(swg), dim3(NTHR), 0, s, a, (int)items);
    // (the radius thresholds ride at the end of the pick's grid)
    hipLaunchKernelGGL(pick_kernel, dim3((unsigned)(bh + nrad)), dim3(PICK_THR), 0, s, a);
    hipLaunchKernelGGL(mask_cand_kernel, dim3((gq + NTHR / 64 - 1) / (NTHR / 64)), dim3(NTHR), 0, s, a);
    hipLaunchKernelGGL(threshold_kernel, dim3((unsigned)bh), dim3(1024), 0, s, a);
    if (a.list)
      hipLaunchKernelGGL(list_from_mask_kernel, dim3((gq + NTHR / 64 - 1) / (NTHR / 64)), dim3(NTHR), 0, s, (int64_t)gq,
                         a.nkb, a.mask, a.list);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_block_select(const SelectArgs& a, bool in_bf16, hipStream_t s) {
  if ((int64_t)a.B * a.Hq * a.nqb == 0) return hipSuccess;
  if (in_bf16) {
    if (a.d == 128) return launch_select_d<bf16_t, 128>(a, s);
    if (a.d == 64) return launch_select_d<bf16_t, 64>(a, s);
    return hipErrorInvalidValue;
  }
  switch (a.d) {
    case 16: return launch_select_d<float, 16>(a, s);
    case 32: return launch_select_d<float, 32>(a, s);
    case 64: return launch_select_d<float, 64>(a, s);
    case 128: return launch_select_d<float, 128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_list_from_mask(int64_t rows, int32_t n_kb, const uint8_t* mask, int32_t* list, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(list_from_mask_kernel, dim3((unsigned)((rows + NTHR / 64 - 1) / (NTHR / 64))), dim3(NTHR), 0, s, rows,
                     n_kb, mask, list);
  return hipGetLastError();
}

}  // namespace soc
