// Block selection for block-sparse prefill on gfx950, float64 throughout.
//
// Steps, in the order of the patty.io review of RBS-Attention (sections on the centroid
// score, mean dilution, the max-key-radius signal, the two independently thresholded
// branches and their union):
//   1-2. stats_kernel  in one grid: the mean of the query rows of every (b, h, query block),
//                      and the centroid of every (b, kv, key block) with its squared radius,
//                      the largest |k_j - c|^2 over the block's keys
//   3. score_kernel    s1 = <qmean, c> for admissible (query block, key block) pairs, -inf
//                      elsewhere (admissible = holds at least one (row, key) pair the position /
//                      window rule allows); 64 x 64 tiles on the fp64 MFMA
//   4. the per-head order statistic of s1 and the per-(b, kv) one of rad2 at the keep
//      fractions: with N values and n = floor(keep*N + 1/2), tau = the (n+1)-th largest
//      (-inf if n >= N), found exactly:
//        score_kernel   also counts the admissible s1 of its tile into a value histogram
//                       (a monotone bucket map over [-M, M], M = max|qmean| * max|c|, the
//                       Cauchy-Schwarz bound; values outside clamp to the end buckets)
//        pick_kernel    sums the tile histograms of each head and locates the bucket holding
//                       descending rank n and the rank inside it
//        gather_kernel  copies that bucket's values out (a few dozen on typical data)
//        threshold_kernel  radix select on order-preserving 64-bit keys among the copied
//                       values (and among the rad2 of each (b, kv))
//      A monotone map puts every value of a higher bucket strictly above every value of a
//      lower one, so rank n overall is rank n - (count above the bucket) inside it.
//   5. mask_kernel    mask = admissible and (s1 > tau_mean or rad2 > tau_radius), plus the
//                     ascending list of kept key blocks per (b, h, query block), one wave per row
// bf16 and f32 inputs widen exactly to f64.  Every reduction that feeds a value has a fixed
// order, so the output is identical from run to run; means are sums of at most a few hundred
// short mantissas and come out exact, so they agree bit for bit with any correct f64
// evaluation.  Only the candidate gather has a run-dependent order, which an order statistic
// does not see.  Steps 1 and 2 read q and k once; the rest is HBM-light.

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
  block_mean<T, D>(base, a.q_st, qb * a.bs, min((qb + 1) * a.bs, a.tq), red, mean, rows);
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
  const bool kept = block_mean<T, D>(base, a.k_st, r0, r1, red, cent, rows);
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

// Per head (first B*Hq blocks) the largest |qmean|^2, per (b, kv) the largest |c|^2.
__global__ void __launch_bounds__(NTHR) norm_max_kernel(SelectArgs a) {
  __shared__ double wm[NTHR / 64];
  const int64_t nbh = (int64_t)a.B * a.Hq;
  const int64_t id = blockIdx.x;
  const bool qside = id < nbh;
  const int n = qside ? a.nqb : a.nkb;
  const double* v = qside ? a.norm2 + id * a.nqb : a.norm2 + nbh * a.nqb + (id - nbh) * a.nkb;
  double m = 0.0;
  for (int i = threadIdx.x; i < n; i += NTHR) m = fmax(m, v[i]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmax(m, __shfl_xor(m, o, 64));
  if ((threadIdx.x & 63) == 0) wm[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    a.nmax[id] = fmax(fmax(wm[0], wm[1]), fmax(wm[2], wm[3]));
  }
}

// The monotone map from an admissible s1 to its histogram bucket.  |s1| <= M by
// Cauchy-Schwarz; the map need not be exact at the ends because it clamps, and a degenerate
// M (zero or huge) sends everything to bucket 0, which stays correct (just not narrowing).
struct BucketMap {
  double lo, scale;
  __device__ BucketMap(const SelectArgs& a, int64_t bh, int64_t bkv) {
    const double m2q = a.nmax[bh];
    const double m2c = a.nmax[(int64_t)a.B * a.Hq + bkv];
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

constexpr int ST = kScoreTile;

// s1 = <qmean, c> on the fp64 MFMA (v_mfma_f64_16x16x4f64: A[i][k] in lane i + 16k, B[k][j]
// in lane j + 16k, D[i][j] in lane j + 16 (i % 4), element i / 4), one 64 x 64 tile of
// (query block, key block) pairs per workgroup, a 32 x 32 quarter (2 x 2 MFMA tiles) per
// wave; the D/4 steps sum all D dims, each lane reading contiguous 16-byte pieces of its row.  The same pass counts every
// admissible s1 of the tile into a value histogram under the monotone bucket map.
template <int D>
__global__ void __launch_bounds__(NTHR) score_kernel(SelectArgs a) {
  __shared__ uint32_t hist[kSelBuckets];
  __shared__ __attribute__((aligned(16))) double qstage[64 * ((D < 32 ? D : 32) + 2)];
  __shared__ __attribute__((aligned(16))) double cstage[64 * ((D < 32 ? D : 32) + 2)];
  const int ntq = (a.nqb + ST - 1) / ST, ntk = (a.nkb + ST - 1) / ST;
  int id = blockIdx.x;
  const int tkt = id % ntk;
  id /= ntk;
  const int tqt = id % ntq;
  id /= ntq;
  const int h = id % a.Hq, b = id / a.Hq;
  const int kvh = h / a.g;
  const int64_t bh = (int64_t)b * a.Hq + h, bkv = (int64_t)b * a.Hkv + kvh;
  const int off = seq_off(a, b), tkb = off + a.tq;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int li = lane & 15, lk = lane >> 4;
  const int WR = tqt * ST + 32 * (wave >> 1), WC = tkt * ST + 32 * (wave & 1);
  const bool hist_on = a.keep_mean >= 0.0;
  double* out = a.score + bh * a.nqb * a.nkb;

  // this lane's outputs (r, c, v): qb = WR + 16 r + 4 v + lk, kb = WC + 16 c + li; bit (2r + c) * 4 + v
  unsigned adm = 0, inr = 0;
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int qb = WR + 16 * r + 4 * v + lk, kb = WC + 16 * c + li;
        const bool in = qb < a.nqb && kb < a.nkb;
        const int bit = (2 * r + c) * 4 + v;
        inr |= (unsigned)in << bit;
        adm |= (unsigned)(in && admissible(a, off, tkb, qb, kb)) << bit;
      }
  const int64_t tile = (int64_t)bh * ntq * ntk + (int64_t)tqt * ntk + tkt;
  const bool active = __syncthreads_or(adm != 0);
  if (hist_on && threadIdx.x == 0) a.tflag[tile] = active;
  auto out_at = [&](int r, int c, int v) __attribute__((always_inline)) -> double& {
    return out[(int64_t)(WR + 16 * r + 4 * v + lk) * a.nkb + WC + 16 * c + li];
  };
  if (!active) {  // nothing admissible in the tile
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (inr >> ((2 * r + c) * 4 + v) & 1) out_at(r, c, v) = SOC_NEG_INF;
    return;
  }
  if (hist_on)
    for (int i = threadIdx.x; i < kSelBuckets; i += NTHR) hist[i] = 0;

  // Operands staged through LDS in 32-dim chunks (CD dims for small D): the workgroup's 64
  // query-mean rows and 64 centroid rows (past the end: the last row; they feed only outputs
  // that are never written), loaded whole-row-coalesced, the next chunk's loads in flight
  // while the current one is used.  At step e of a chunk lane (i, k) feeds dim k*CD/4 + e.
  constexpr int CD = D < 32 ? D : 32, E = CD / 4, RS = CD + 2;  // RS: padded row stride (doubles)
  constexpr int NLD = 64 * CD / 2 / NTHR;  // 16-byte loads per thread per operand and chunk
  const double* qsrc = a.qmean + bh * a.nqb * D;
  const double* csrc = a.cent + bkv * a.nkb * D;
  f64x2 qpre[NLD], cpre[NLD];
  auto load_chunk = [&](int d0) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
      const int idx = threadIdx.x + u * NTHR;  // 16-byte piece of the 64 x CD chunk
      const int row = idx / (CD / 2), pc = idx % (CD / 2);
      qpre[u] = *(const f64x2*)(qsrc + (int64_t)min(tqt * ST + row, a.nqb - 1) * D + d0 + 2 * pc);
      cpre[u] = *(const f64x2*)(csrc + (int64_t)min(tkt * ST + row, a.nkb - 1) * D + d0 + 2 * pc);
    }
  };
  f64x4 acc[2][2];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int c = 0; c < 2; ++c) acc[r][c] = f64x4{0.0, 0.0, 0.0, 0.0};
  load_chunk(0);
  const int ar0 = 32 * (wave >> 1) + li, bc0 = 32 * (wave & 1) + li;  // this lane's rows in the stage
#pragma unroll 1
  for (int d0 = 0; d0 < D; d0 += CD) {
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
      const int idx = threadIdx.x + u * NTHR;
      const int row = idx / (CD / 2), pc = idx % (CD / 2);
      *(f64x2*)(qstage + row * RS + 2 * pc) = qpre[u];
      *(f64x2*)(cstage + row * RS + 2 * pc) = cpre[u];
    }
    __syncthreads();
    if (d0 + CD < D) load_chunk(d0 + CD);
#pragma unroll
    for (int e2 = 0; e2 < E / 2; ++e2) {
      f64x2 av[2], bv[2];
#pragma unroll
      for (int r = 0; r < 2; ++r) av[r] = *(const f64x2*)(qstage + (ar0 + 16 * r) * RS + lk * E + 2 * e2);
#pragma unroll
      for (int c = 0; c < 2; ++c) bv[c] = *(const f64x2*)(cstage + (bc0 + 16 * c) * RS + lk * E + 2 * e2);
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
          for (int c = 0; c < 2; ++c)
            acc[r][c] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[r][h2], bv[c][h2], acc[r][c], 0, 0, 0);
    }
    __syncthreads();  // the stage is read before the next chunk overwrites it
  }

  if (hist_on) __syncthreads();  // the histogram is cleared
  const BucketMap bucket(a, bh, bkv);
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int bit = (2 * r + c) * 4 + v;
        if (!(inr >> bit & 1)) continue;
        const bool ok = adm >> bit & 1;
        const double sv = ok ? acc[r][c][v] : SOC_NEG_INF;
        out_at(r, c, v) = sv;
        if (hist_on && ok) atomicAdd(&hist[bucket(sv)], 1u);
      }
  if (hist_on) {  // the tile's histogram as u16 pairs (a tile has at most 64*64 values)
    __syncthreads();
    constexpr int PER = kSelBuckets / NTHR;  // buckets per thread
    u32x4* dst = (u32x4*)(a.hpart + tile * (kSelBuckets / 2) + threadIdx.x * (PER / 2));
#pragma unroll
    for (int v = 0; v < PER / 8; ++v) {
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int k = threadIdx.x * PER + 8 * v + 2 * e;
        w[e] = hist[k] | (hist[k + 1] << 16);
      }
      dst[v] = w;
    }
  }
}

// Wave-wide search in descending value order.  Lane l holds the count c of the l-th of 64
// consecutive value ranges (higher lane = higher values).  Returns the lane L whose range
// holds descending rank `target` (< the wave total), with *above = the count in the lanes
// above L and *total = the wave total.
__device__ int wave_locate_desc(unsigned long long c, unsigned long long target, unsigned long long* above,
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

// Per head: sums the tile histograms of its admissible s1 (fixed tile order), then finds the
// bucket that holds descending rank n = floor(keep * N + 1/2) and the rank inside it; writes
// (N, n, bucket or -1 when n >= N, rank) to pick.  One workgroup of 1024 threads per head,
// thread t owning buckets 4t .. 4t+3.
constexpr int PICK_THR = 1024;
static_assert(kSelBuckets == 4 * PICK_THR, "four buckets per thread");
__global__ void __launch_bounds__(PICK_THR) pick_kernel(SelectArgs a) {
  __shared__ uint32_t hist[kSelBuckets];
  const int64_t bh = blockIdx.x;
  const int64_t ntiles = (int64_t)((a.nqb + ST - 1) / ST) * ((a.nkb + ST - 1) / ST);
  const u32x2* hp = (const u32x2*)(a.hpart + bh * ntiles * (kSelBuckets / 2)) + threadIdx.x;
  const uint32_t* fl = a.tflag + bh * ntiles;
  uint32_t c4[4] = {0u, 0u, 0u, 0u};
  auto add = [&](u32x2 w) __attribute__((always_inline)) {
    c4[0] += w[0] & 0xffffu;
    c4[1] += w[0] >> 16;
    c4[2] += w[1] & 0xffffu;
    c4[3] += w[1] >> 16;
  };
  int64_t t = 0;
  for (; t + 8 <= ntiles; t += 8) {  // 8 tiles' loads in flight; tiles without data are masked
    u32x2 w[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) w[u] = hp[(t + u) * (kSelBuckets / 4)];
#pragma unroll
    for (int u = 0; u < 8; ++u) add(fl[t + u] ? w[u] : u32x2{0u, 0u});
  }
  for (; t < ntiles; ++t) add(fl[t] ? hp[t * (kSelBuckets / 4)] : u32x2{0u, 0u});
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

constexpr int GCH = kSelGatherChunk;  // score values scanned per gather workgroup
static_assert(GCH % NTHR == 0, "whole values per thread");

// Copies every s1 of the head's picked bucket (typically a few dozen values) into this
// workgroup's own segment of the candidate array (cand[bh][chunk][...], count in
// ccount[bh][chunk]): a streaming filter over the scores with no atomics.
__global__ void __launch_bounds__(NTHR) gather_kernel(SelectArgs a) {
  __shared__ int wcount[NTHR / 64];
  const int64_t P = (int64_t)a.nqb * a.nkb;
  const int nch = (int)((P + GCH - 1) / GCH);
  const int ch = blockIdx.x % nch;
  const int64_t bh = blockIdx.x / nch;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const long long beta = a.pick[bh * 4 + 2];
  if (beta < 0) return;
  const double* sc = a.score + bh * P;
  const int64_t i0 = (int64_t)ch * GCH;
  double sv[GCH / NTHR];
#pragma unroll
  for (int r = 0; r < GCH / NTHR; ++r) {
    const int64_t i = i0 + r * NTHR + threadIdx.x;
    sv[r] = i < P ? sc[i] : SOC_NEG_INF;
  }
  const BucketMap bucket(a, bh, (int64_t)(bh / a.Hq) * a.Hkv + (bh % a.Hq) / a.g);
  unsigned long long bal[GCH / NTHR];
  int n = 0;
#pragma unroll
  for (int r = 0; r < GCH / NTHR; ++r) {
    bal[r] = __ballot(sv[r] > SOC_NEG_INF && bucket(sv[r]) == (int)beta);
    n += __popcll(bal[r]);
  }
  if (lane == 0) wcount[wave] = n;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += wcount[w];
  double* cd = a.cand + bh * P + i0;
#pragma unroll
  for (int r = 0; r < GCH / NTHR; ++r) {
    if (bal[r] >> lane & 1) cd[base + __popcll(bal[r] & ((1ull << lane) - 1ull))] = sv[r];
    base += __popcll(bal[r]);
  }
  if (threadIdx.x == NTHR - 1) a.ccount[bh * nch + ch] = base;  // the last wave's base is the total
}

// Exact value at descending rank `rank` (0 = largest) among the finite values of nseg
// segments: vals[s * seg_len + i] for i < counts[s] (one segment when counts is null, count
// values).  8 passes of an 8-bit radix select on order-preserving keys, 1024 threads.
__device__ double select_desc(const double* vals, int64_t count, const unsigned* counts, int nseg, int64_t seg_len,
                              unsigned long long rank, unsigned* hist, unsigned long long* su) {
  constexpr int T = 1024;
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

constexpr int CAND_LDS = 2048;  // candidates selected in LDS (more: straight from their segments)

__global__ void __launch_bounds__(1024) threshold_kernel(SelectArgs a) {
  __shared__ unsigned hist[256];
  __shared__ unsigned long long su[2];
  __shared__ unsigned seg_end[64];
  __shared__ double cv[CAND_LDS];
  const int nmean = a.keep_mean >= 0.0 ? a.B * a.Hq : 0;
  int id = blockIdx.x;
  if (id < nmean) {
    const int64_t* pk = a.pick + (int64_t)id * 4;
    double tau = SOC_NEG_INF;
    const int64_t P = (int64_t)a.nqb * a.nkb;
    const int nch = (int)((P + GCH - 1) / GCH);
    const double* cand = a.cand + (int64_t)id * P;
    const unsigned* cnt = a.ccount + (int64_t)id * nch;
    if (pk[2] >= 0) {
      // the candidates of all gather chunks, contiguous in LDS when they fit
      unsigned total = 0;
      if (threadIdx.x < 64) {  // inclusive prefix of the chunk counts, 64 chunks per pass
        unsigned run = 0;
        for (int c0 = 0; c0 < nch; c0 += 64) {
          const unsigned x = c0 + (int)threadIdx.x < nch ? cnt[c0 + threadIdx.x] : 0u;
          unsigned incl = x;
#pragma unroll
          for (int o = 1; o < 64; o <<= 1) {
            const unsigned y = __shfl_up(incl, o, 64);
            if ((int)threadIdx.x >= o) incl += y;
          }
          if (nch <= 64) seg_end[threadIdx.x] = run + incl;
          run += __shfl(incl, 63, 64);
        }
        if (threadIdx.x == 0) su[0] = run;
      }
      __syncthreads();
      total = (unsigned)su[0];
      __syncthreads();
      if (nch <= 64 && total <= (unsigned)CAND_LDS) {
        for (unsigned i = threadIdx.x; i < total; i += 1024) {
          int sg = 0;
          while (seg_end[sg] <= i) ++sg;
          cv[i] = cand[(int64_t)sg * GCH + (i - (sg ? seg_end[sg - 1] : 0u))];
        }
        __syncthreads();
        tau = select_desc(cv, total, nullptr, 1, 0, (unsigned long long)pk[3], hist, su);
      } else {
        tau = select_desc(cand, 0, cnt, nch, GCH, (unsigned long long)pk[3], hist, su);
      }
    }
    if (threadIdx.x == 0) a.tau_mean[id] = tau;
  } else {
    id -= nmean;
    const double* vals = a.rad2 + (int64_t)id * a.nkb;
    if (threadIdx.x == 0) su[0] = 0;
    __syncthreads();
    unsigned long long local = 0;
    for (int i = threadIdx.x; i < a.nkb; i += 1024) local += vals[i] > SOC_NEG_INF;
    atomicAdd(&su[0], local);
    __syncthreads();
    const unsigned long long N = su[0];
    __syncthreads();
    const double nd = floor(a.keep_radius * (double)N + 0.5);
    const double tau = nd >= (double)N ? SOC_NEG_INF : select_desc(vals, a.nkb, nullptr, 1, 0, (unsigned long long)nd, hist, su);
    if (threadIdx.x == 0) a.tau_radius[id] = tau;
  }
}

// Compacts one row of keep flags (kb = 0..n_kb-1) into list[0] = count, list[1..] = kb.
// Called by all 256 threads of the block with the same row.
template <typename KeepFn>
__device__ void compact_row(int n_kb, KeepFn keep, uint8_t* mask_row, int32_t* list_row, int* wsum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int base = 0;
  for (int k0 = 0; k0 < n_kb; k0 += NTHR) {
    const int kb = k0 + threadIdx.x;
    const bool kept = kb < n_kb && keep(kb);
    if (mask_row && kb < n_kb) mask_row[kb] = kept ? 1 : 0;
    const unsigned long long bal = __ballot(kept);
    const int before = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) wsum[wave] = __popcll(bal);
    __syncthreads();
    int wbase = base;
    for (int w = 0; w < wave; ++w) wbase += wsum[w];
    if (kept && list_row) list_row[1 + wbase + before] = kb;
    const int total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
    __syncthreads();
    base += total;
  }
  if (threadIdx.x == 0 && list_row) list_row[0] = base;
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
  const double* sc = a.score + row * a.nkb;
  const double* r2 = a.rad2 + ((int64_t)b * a.Hkv + kvh) * a.nkb;
  const double t1 = a.tau_mean[b * a.Hq + h];
  const double t2 = a.tau_radius[b * a.Hkv + kvh];
  uint8_t* mrow = a.mask + row * a.nkb;
  int32_t* lrow = a.list ? a.list + row * (1 + a.nkb) : nullptr;
  int base = 0;
  for (int k0 = 0; k0 < a.nkb; k0 += 64) {
    const int kb = k0 + lane;
    bool kept = false;
    if (kb < a.nkb) {
      const double sv = sc[kb];
      kept = sv > SOC_NEG_INF && (sv > t1 || r2[kb] > t2);
      mrow[kb] = kept ? 1 : 0;
    }
    const unsigned long long bal = __ballot(kept);
    if (kept && lrow) lrow[1 + base + __popcll(bal & ((1ull << lane) - 1ull))] = kb;
    base += __popcll(bal);
  }
  if (lane == 0 && lrow) lrow[0] = base;
}

__global__ void __launch_bounds__(NTHR) list_from_mask_kernel(int32_t n_kb, const uint8_t* mask, int32_t* list) {
  __shared__ int wsum[4];
  const int64_t row = blockIdx.x;
  const uint8_t* m = mask + row * n_kb;
  compact_row(n_kb, [&](int kb) { return m[kb] != 0; }, nullptr, list + row * (1 + n_kb), wsum);
}

template <typename T, int D>
hipError_t launch_select_d(const SelectArgs& a, hipStream_t s) {
  const unsigned gq = (unsigned)((int64_t)a.B * a.Hq * a.nqb);
  const unsigned gk = (unsigned)((int64_t)a.B * a.Hkv * a.nkb);
  const bool mean_on = a.keep_mean >= 0.0;
  const int64_t bh = (int64_t)a.B * a.Hq;
  hipLaunchKernelGGL((stats_kernel<T, D>), dim3(gq + gk), dim3(NTHR), 0, s, a);
  if (mean_on)
    hipLaunchKernelGGL(norm_max_kernel, dim3((unsigned)(bh + (int64_t)a.B * a.Hkv)), dim3(NTHR), 0, s, a);
  const int64_t ntq = (a.nqb + ST - 1) / ST, ntk = (a.nkb + ST - 1) / ST;
  hipLaunchKernelGGL(score_kernel<D>, dim3((unsigned)(bh * ntq * ntk)), dim3(NTHR), 0, s, a);
  if (mean_on) {
    hipLaunchKernelGGL(pick_kernel, dim3((unsigned)bh), dim3(PICK_THR), 0, s, a);
    const int64_t nch = ((int64_t)a.nqb * a.nkb + GCH - 1) / GCH;
    hipLaunchKernelGGL(gather_kernel, dim3((unsigned)(bh * nch)), dim3(NTHR), 0, s, a);
  }
  const unsigned gt = (mean_on ? a.B * a.Hq : 0) + (a.keep_radius >= 0.0 ? a.B * a.Hkv : 0);
  if (gt) hipLaunchKernelGGL(threshold_kernel, dim3(gt), dim3(1024), 0, s, a);
  if (a.mask)  // (the fused block-sparse prefill reads the scores and thresholds instead)
    hipLaunchKernelGGL(mask_kernel, dim3((gq + NTHR / 64 - 1) / (NTHR / 64)), dim3(NTHR), 0, s, a);
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
  hipLaunchKernelGGL(list_from_mask_kernel, dim3((unsigned)rows), dim3(NTHR), 0, s, n_kb, mask, list);
  return hipGetLastError();
}

}  // namespace soc
