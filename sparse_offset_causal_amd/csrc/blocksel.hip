// Block selection for block-sparse prefill on gfx950, float64 throughout.
//
// Steps, in the order of the patty.io review of RBS-Attention (sections on the centroid
// score, mean dilution, the max-key-radius signal, the two independently thresholded
// branches and their union):
//   1. qmean_kernel   mean of the query rows of every (b, h, query block)
//   2. kstats_kernel  centroid of every (b, kv, key block) and its squared radius, the
//                     largest |k_j - c|^2 over the block's keys
//   3. score_kernel   s1 = <qmean, c> for admissible (query block, key block) pairs,
//                     -inf elsewhere (admissible = holds at least one (row, key) pair the
//                     position / window rule allows); 64 x 64 tiles of s1 per workgroup
//   4. the per-head order statistic of s1 and the per-(b, kv) one of rad2 at the keep
//      fractions: with N values and n = floor(keep*N + 1/2), tau = the (n+1)-th largest
//      (-inf if n >= N), found exactly:
//        score_kernel   also counts the admissible s1 of its tile into a value histogram
//                       (a monotone bucket map over [-M, M], M = max|qmean| * max|c|, the
//                       Cauchy-Schwarz bound; values outside clamp to the end buckets)
//        hist_reduce_kernel  sums the tile histograms of each head
//        gather_kernel  locates the bucket holding descending rank n and copies that
//                       bucket's values out (a few dozen on typical data)
//        threshold_kernel  radix select on order-preserving 64-bit keys among the copied
//                       values (and among the rad2 of each (b, kv))
//      A monotone map puts every value of a higher bucket strictly above every value of a
//      lower one, so rank n overall is rank n - (count above the bucket) inside it.
//   5. mask_kernel    mask = admissible and (s1 > tau_mean or rad2 > tau_radius), plus the
//                     ascending list of kept key blocks per (b, h, query block)
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
#pragma unroll
  for (int e = 0; e < 8; ++e) red[rg * D + 8 * c + e] = acc[e];
  __syncthreads();
  if (threadIdx.x < D) {
    double sum = 0.0;
    for (int g = 0; g < RG; ++g) sum += red[g * D + threadIdx.x];
    out_lds[threadIdx.x] = sum / (double)(r1 - r0);
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
__global__ void __launch_bounds__(NTHR) qmean_kernel(SelectArgs a) {
  __shared__ double red[NTHR * 8];
  __shared__ double mean[D];
  const int qb = blockIdx.x % a.nqb;
  const int h = (blockIdx.x / a.nqb) % a.Hq;
  const int b = blockIdx.x / (a.nqb * a.Hq);
  const int64_t bh = (int64_t)b * a.Hq + h;
  const T* base = (const T*)a.q + b * a.q_sb + h * a.q_sh;
  Row8<T> rows[RB];
  block_mean<T, D>(base, a.q_st, qb * a.bs, min((qb + 1) * a.bs, a.tq), red, mean, rows);
  if (threadIdx.x < D) a.qmean[(bh * a.nqb + qb) * D + threadIdx.x] = mean[threadIdx.x];
  if (a.keep_mean >= 0.0) write_norm2<D>(mean, a.norm2 + bh * a.nqb + qb);
}

template <typename T, int D>
__global__ void __launch_bounds__(NTHR) kstats_kernel(SelectArgs a) {
  __shared__ double red[NTHR * 8];
  __shared__ double cent[D];
  __shared__ double rmax[NTHR / 64];
  const int kb = blockIdx.x % a.nkb;
  const int kvh = (blockIdx.x / a.nkb) % a.Hkv;
  const int b = blockIdx.x / (a.nkb * a.Hkv);
  const int tkb = seq_off(a, b) + a.tq;
  double* cT = a.cT + ((int64_t)b * a.Hkv + kvh) * D * a.nkb;
  if (kb * a.bs >= tkb) {  // block beyond this sequence's keys
    if (threadIdx.x < D) cT[(int64_t)threadIdx.x * a.nkb + kb] = 0.0;
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
  if (threadIdx.x < D) cT[(int64_t)threadIdx.x * a.nkb + kb] = cent[threadIdx.x];
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
#pragma unroll
    for (int u = 0; u < RB; ++u) {
      const int r = rb + u * RG;
      double part = 0.0;
      if (r < r1) {
        double x[8];
        rows[u].widen(x);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const double dlt = x[e] - cv[e];
          part = fma(dlt, dlt, part);
        }
      }
#pragma unroll
      for (int m = 1; m < C; m <<= 1) part += __shfl_xor(part, m, 64);
      if (r < r1) best = fmax(best, part);
    }
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) best = fmax(best, __shfl_xor(best, m, 64));
  if ((threadIdx.x & 63) == 0) rmax[threadIdx.x >> 6] = best;
  __syncthreads();
  if (threadIdx.x == 0)
    a.rad2[((int64_t)b * a.Hkv + kvh) * a.nkb + kb] = fmax(fmax(rmax[0], rmax[1]), fmax(rmax[2], rmax[3]));
}

// Per head (first B*Hq blocks) the largest |qmean|^2, per (b, kv) the largest |c|^2; the
// head blocks also clear the head's candidate counter.
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
    if (qside) a.ccount[id] = 0;
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

template <int D>
__global__ void __launch_bounds__(NTHR) score_kernel(SelectArgs a) {
  constexpr int SD = D < 32 ? D : 32;  // head-dim slice staged per step
  __shared__ double qs[ST][SD + 1];    // +1: the four rows a wave reads land in distinct banks
  __shared__ double cs[SD][ST];
  __shared__ uint32_t hist[kSelBuckets];
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
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
  const int QB0 = tqt * ST, KB0 = tkt * ST;
  const bool hist_on = a.keep_mean >= 0.0;
  double* out = a.score + bh * a.nqb * a.nkb;

  // this thread's outputs: (QB0 + ty + 16 i, KB0 + tx + 16 j)
  unsigned adm = 0, inr = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int qb = QB0 + ty + 16 * i, kb = KB0 + tx + 16 * j;
      const bool in = qb < a.nqb && kb < a.nkb;
      inr |= (unsigned)in << (4 * i + j);
      adm |= (unsigned)(in && admissible(a, off, tkb, qb, kb)) << (4 * i + j);
    }
  const int64_t tile = (int64_t)bh * ntq * ntk + (int64_t)tqt * ntk + tkt;
  const bool active = __syncthreads_or(adm != 0);
  if (hist_on && threadIdx.x == 0) a.tflag[tile] = active;
  if (!active) {  // nothing admissible in the tile
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (inr >> (4 * i + j) & 1) out[(int64_t)(QB0 + ty + 16 * i) * a.nkb + KB0 + tx + 16 * j] = SOC_NEG_INF;
    return;
  }
  if (hist_on)
    for (int i = threadIdx.x; i < kSelBuckets; i += NTHR) hist[i] = 0;

  const double* qm = a.qmean + bh * a.nqb * D;
  const double* cT = a.cT + bkv * D * a.nkb;
  double acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0;
  // Staging: every thread loads NL values of each operand per head-dim slice into registers
  // (rows and columns past the end are clamped to the last one; they feed only outputs that
  // are never written), the next slice's loads in flight while the current one is computed.
  constexpr int NL = ST * SD / NTHR;
  double qr[NL], cr[NL];
  auto load_slice = [&](int t0) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < NL; ++k) {
      const int i = threadIdx.x + k * NTHR;
      const int qb = min(QB0 + i / SD, a.nqb - 1), kb = min(KB0 + i % ST, a.nkb - 1);
      qr[k] = qm[(int64_t)qb * D + t0 + i % SD];
      cr[k] = cT[(int64_t)(t0 + i / ST) * a.nkb + kb];
    }
  };
  load_slice(0);
  for (int t0 = 0; t0 < D; t0 += SD) {
#pragma unroll
    for (int k = 0; k < NL; ++k) {
      const int i = threadIdx.x + k * NTHR;
      qs[i / SD][i % SD] = qr[k];
      cs[i / ST][i % ST] = cr[k];
    }
    __syncthreads();
    if (t0 + SD < D) load_slice(t0 + SD);
#pragma unroll 8
    for (int t = 0; t < SD; ++t) {  // s1 accumulates over the head dimension in ascending order
      double qv[4], cv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) qv[i] = qs[ty + 16 * i][t];
#pragma unroll
      for (int j = 0; j < 4; ++j) cv[j] = cs[t][tx + 16 * j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fma(qv[i], cv[j], acc[i][j]);
    }
    __syncthreads();
  }

  const BucketMap bucket(a, bh, bkv);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (!(inr >> (4 * i + j) & 1)) continue;
      const bool ok = adm >> (4 * i + j) & 1;
      const double sv = ok ? acc[i][j] : SOC_NEG_INF;
      out[(int64_t)(QB0 + ty + 16 * i) * a.nkb + KB0 + tx + 16 * j] = sv;
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

// Sums the per-tile histograms of each head into its value histogram (fixed tile order).
// Grid: B * Hq * (kSelBuckets / 512); each thread owns a pair of buckets.
__global__ void __launch_bounds__(NTHR) hist_reduce_kernel(SelectArgs a) {
  constexpr int PARTS = kSelBuckets / (2 * NTHR);
  const int part = blockIdx.x % PARTS;
  const int64_t bh = blockIdx.x / PARTS;
  const int64_t ntiles = (int64_t)((a.nqb + ST - 1) / ST) * ((a.nkb + ST - 1) / ST);
  const int pair = part * NTHR + threadIdx.x;
  const uint32_t* hp = a.hpart + bh * ntiles * (kSelBuckets / 2) + pair;
  const uint32_t* fl = a.tflag + bh * ntiles;
  uint32_t lo = 0, hi = 0;
  int64_t t = 0;
  for (; t + 8 <= ntiles; t += 8) {  // 8 tiles' loads in flight; tiles without data are masked
    uint32_t w[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) w[u] = hp[(t + u) * (kSelBuckets / 2)];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint32_t m = fl[t + u] ? w[u] : 0u;
      lo += m & 0xffffu;
      hi += m >> 16;
    }
  }
  for (; t < ntiles; ++t) {
    const uint32_t m = fl[t] ? hp[t * (kSelBuckets / 2)] : 0u;
    lo += m & 0xffffu;
    hi += m >> 16;
  }
  a.hist[bh * kSelBuckets + 2 * pair] = lo;
  a.hist[bh * kSelBuckets + 2 * pair + 1] = hi;
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

constexpr int GCH = 32 * NTHR;  // score values scanned per gather workgroup

// Finds, per head, the histogram bucket that holds descending rank n of the admissible s1 and
// appends every s1 of that bucket to the head's candidate list.  Every workgroup of a head
// locates the bucket itself (a 16 KB read); the first records it for threshold_kernel.
__global__ void __launch_bounds__(NTHR) gather_kernel(SelectArgs a) {
  __shared__ long long sel[4];  // N, n, bucket (-1: nothing to gather), rank within bucket
  const int64_t P = (int64_t)a.nqb * a.nkb;
  const int nch = (int)((P + GCH - 1) / GCH);
  const int ch = blockIdx.x % nch;
  const int64_t bh = blockIdx.x / nch;
  const int lane = threadIdx.x & 63;
  // this workgroup's slice of the head's s1, loaded before the bucket search so the two overlap
  const double* sc = a.score + bh * P;
  const int64_t i0 = (int64_t)ch * GCH;
  double sv[GCH / NTHR];
#pragma unroll
  for (int r = 0; r < GCH / NTHR; ++r) {
    const int64_t i = i0 + r * NTHR + threadIdx.x;
    sv[r] = i < P ? sc[i] : SOC_NEG_INF;
  }
  if (threadIdx.x < 64) {
    const uint32_t* hh = a.hist + bh * kSelBuckets;
    unsigned long long c = 0;
#pragma unroll
    for (int i = 0; i < 64; i += 4) {
      const u32x4 w = *(const u32x4*)(hh + 64 * lane + i);
      c += (unsigned long long)w[0] + w[1] + w[2] + w[3];
    }
    unsigned long long above1 = 0, N = 0;
    int L1 = wave_locate_desc(c, 0, &above1, &N);  // N only; L1 recomputed below
    const double nd = floor(a.keep_mean * (double)N + 0.5);
    if (nd >= (double)N) {
      if (lane == 0) {
        sel[0] = (long long)N;
        sel[1] = (long long)nd;
        sel[2] = -1;
        sel[3] = 0;
      }
    } else {
      const unsigned long long n = (unsigned long long)nd;
      L1 = wave_locate_desc(c, n, &above1, &N);
      unsigned long long above2 = 0, n1 = 0;
      const int L2 = wave_locate_desc(hh[64 * L1 + lane], n - above1, &above2, &n1);
      if (lane == 0) {
        sel[0] = (long long)N;
        sel[1] = (long long)n;
        sel[2] = 64 * L1 + L2;
        sel[3] = (long long)(n - above1 - above2);
      }
    }
  }
  __syncthreads();
  if (ch == 0 && threadIdx.x < 4) a.pick[bh * 4 + threadIdx.x] = sel[threadIdx.x];
  const long long beta = sel[2];
  if (beta < 0) return;
  const BucketMap bucket(a, bh, (int64_t)(bh / a.Hq) * a.Hkv + (bh % a.Hq) / a.g);
  double* cd = a.cand + bh * P;
#pragma unroll
  for (int r = 0; r < GCH / NTHR; ++r) {  // same trip count in every lane
    const double v = sv[r];
    const bool m = v > SOC_NEG_INF && bucket(v) == (int)beta;
    const unsigned long long bal = __ballot(m);
    if (bal) {
      unsigned slot = 0;
      if (lane == 0) slot = atomicAdd(&a.ccount[bh], (unsigned)__popcll(bal));
      slot = __shfl(slot, 0, 64);
      if (m) cd[slot + __popcll(bal & ((1ull << lane) - 1ull))] = v;
    }
  }
}

// Exact value at descending rank `rank` (0 = largest) among the finite values of vals[0,
// count): 8 passes of an 8-bit radix select on order-preserving keys, 1024 threads.
__device__ double select_desc(const double* vals, int64_t count, unsigned long long rank, unsigned* hist,
                              unsigned long long* su) {
  constexpr int T = 1024;
  unsigned long long prefix = 0, pmask = 0;
  for (int shift = 56; shift >= 0; shift -= 8) {
    for (int i = threadIdx.x; i < 256; i += T) hist[i] = 0;
    __syncthreads();
    for (int64_t i = threadIdx.x; i < count; i += T) {
      const double x = vals[i];
      if (!(x > SOC_NEG_INF)) continue;
      const uint64_t key = f64_order_key(x);
      if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
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

__global__ void __launch_bounds__(1024) threshold_kernel(SelectArgs a) {
  __shared__ unsigned hist[256];
  __shared__ unsigned long long su[2];
  const int nmean = a.keep_mean >= 0.0 ? a.B * a.Hq : 0;
  int id = blockIdx.x;
  if (id < nmean) {
    const int64_t* pk = a.pick + (int64_t)id * 4;
    double tau = SOC_NEG_INF;
    if (pk[2] >= 0)
      tau = select_desc(a.cand + (int64_t)id * a.nqb * a.nkb, a.ccount[id], (unsigned long long)pk[3], hist, su);
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
    const double tau = nd >= (double)N ? SOC_NEG_INF : select_desc(vals, a.nkb, (unsigned long long)nd, hist, su);
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

__global__ void __launch_bounds__(NTHR) mask_kernel(SelectArgs a) {
  __shared__ int wsum[4];
  const int qb = blockIdx.x % a.nqb;
  const int h = (blockIdx.x / a.nqb) % a.Hq;
  const int b = blockIdx.x / (a.nqb * a.Hq);
  const int kvh = h / a.g;
  const int64_t row = ((int64_t)b * a.Hq + h) * a.nqb + qb;
  const double* sc = a.score + row * a.nkb;
  const double* r2 = a.rad2 + ((int64_t)b * a.Hkv + kvh) * a.nkb;
  const double t1 = a.tau_mean[b * a.Hq + h];
  const double t2 = a.tau_radius[b * a.Hkv + kvh];
  compact_row(
      a.nkb, [&](int kb) { const double s = sc[kb]; return s > SOC_NEG_INF && (s > t1 || r2[kb] > t2); },
      a.mask + row * a.nkb, a.list ? a.list + row * (1 + a.nkb) : nullptr, wsum);
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
  hipLaunchKernelGGL((qmean_kernel<T, D>), dim3(gq), dim3(NTHR), 0, s, a);
  hipLaunchKernelGGL((kstats_kernel<T, D>), dim3(gk), dim3(NTHR), 0, s, a);
  if (mean_on)
    hipLaunchKernelGGL(norm_max_kernel, dim3((unsigned)(bh + (int64_t)a.B * a.Hkv)), dim3(NTHR), 0, s, a);
  const int64_t ntq = (a.nqb + ST - 1) / ST, ntk = (a.nkb + ST - 1) / ST;
  hipLaunchKernelGGL(score_kernel<D>, dim3((unsigned)(bh * ntq * ntk)), dim3(NTHR), 0, s, a);
  if (mean_on) {
    hipLaunchKernelGGL(hist_reduce_kernel, dim3((unsigned)(bh * (kSelBuckets / (2 * NTHR)))), dim3(NTHR), 0, s, a);
    const int64_t nch = ((int64_t)a.nqb * a.nkb + GCH - 1) / GCH;
    hipLaunchKernelGGL(gather_kernel, dim3((unsigned)(bh * nch)), dim3(NTHR), 0, s, a);
  }
  const unsigned gt = (mean_on ? a.B * a.Hq : 0) + (a.keep_radius >= 0.0 ? a.B * a.Hkv : 0);
  if (gt) hipLaunchKernelGGL(threshold_kernel, dim3(gt), dim3(1024), 0, s, a);
  hipLaunchKernelGGL(mask_kernel, dim3(gq), dim3(NTHR), 0, s, a);
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
