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
//                     position / window rule allows)
//   4. threshold_kernel  per (b, h) the order statistic of s1 and per (b, kv) the order
//                     statistic of rad2 at the keep fractions: with N values and
//                     n = floor(keep*N + 1/2), tau = the (n+1)-th largest (-inf if n >= N),
//                     found exactly by an 8-pass radix select on order-preserving 64-bit keys
//   5. mask_kernel    mask = admissible and (s1 > tau_mean or rad2 > tau_radius), plus the
//                     ascending list of kept key blocks per (b, h, query block)
// bf16 and f32 inputs widen exactly to f64.  Every reduction has a fixed order, so the
// output is identical from run to run; means are sums of at most a few hundred short
// mantissas and come out exact, so they agree bit for bit with any correct f64 evaluation.
// All passes are HBM-light except 1 and 2, which read q and k once.

#include "device_common.h"
#include "internal.h"

namespace soc {
namespace {

constexpr int NTHR = 256;

// 8 consecutive elements widened to double.
__device__ __forceinline__ void load8(const bf16_t* p, double* o) {
  const u32x4 w = *(const u32x4*)p;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    o[2 * e] = (double)bf16_lo(w[e]);
    o[2 * e + 1] = (double)bf16_hi(w[e]);
  }
}
__device__ __forceinline__ void load8(const float* p, double* o) {
  const f32x4 a = *(const f32x4*)p, b = *(const f32x4*)(p + 4);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    o[e] = (double)a[e];
    o[4 + e] = (double)b[e];
  }
}

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

// Block mean of rows [r0, r1) of a [rows, D] matrix (row stride st), written to out[D].
// Thread layout: C = D/8 threads per row (8 columns each), 256/C row groups.
template <typename T, int D>
__device__ void block_mean(const T* base, int64_t st, int r0, int r1, double* red, double* out_lds) {
  constexpr int C = D / 8, RG = NTHR / C;
  const int c = threadIdx.x % C, rg = threadIdx.x / C;
  double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int r = r0 + rg; r < r1; r += RG) {
    double x[8];
    load8(base + (int64_t)r * st + 8 * c, x);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += x[e];
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[rg * D + 8 * c + e] = acc[e];
  __syncthreads();
  if (threadIdx.x < D) {
    double s = 0.0;
    for (int g = 0; g < RG; ++g) s += red[g * D + threadIdx.x];
    out_lds[threadIdx.x] = s / (double)(r1 - r0);
  }
  __syncthreads();
}

template <typename T, int D>
__global__ void __launch_bounds__(NTHR) qmean_kernel(SelectArgs a) {
  __shared__ double red[NTHR * 8];
  __shared__ double mean[D];
  const int qb = blockIdx.x % a.nqb;
  const int h = (blockIdx.x / a.nqb) % a.Hq;
  const int b = blockIdx.x / (a.nqb * a.Hq);
  const T* base = (const T*)a.q + b * a.q_sb + h * a.q_sh;
  block_mean<T, D>(base, a.q_st, qb * a.bs, min((qb + 1) * a.bs, a.tq), red, mean);
  if (threadIdx.x < D) a.qmean[(((int64_t)b * a.Hq + h) * a.nqb + qb) * D + threadIdx.x] = mean[threadIdx.x];
}

template <typename T, int D>
__global__ void __launch_bounds__(NTHR) kstats_kernel(SelectArgs a) {
  __shared__ double red[NTHR * 8];
  __shared__ double cent[D];
  __shared__ double rmax[NTHR];
  const int kb = blockIdx.x % a.nkb;
  const int kvh = (blockIdx.x / a.nkb) % a.Hkv;
  const int b = blockIdx.x / (a.nkb * a.Hkv);
  const int tkb = seq_off(a, b) + a.tq;
  double* cT = a.cT + ((int64_t)b * a.Hkv + kvh) * D * a.nkb;
  if (kb * a.bs >= tkb) {  // block beyond this sequence's keys
    if (threadIdx.x < D) cT[(int64_t)threadIdx.x * a.nkb + kb] = 0.0;
    if (threadIdx.x == 0) a.rad2[((int64_t)b * a.Hkv + kvh) * a.nkb + kb] = SOC_NEG_INF;
    return;
  }
  const T* base = (const T*)a.k + b * a.k_sb + kvh * a.k_sh;
  const int r0 = kb * a.bs, r1 = min((kb + 1) * a.bs, tkb);
  block_mean<T, D>(base, a.k_st, r0, r1, red, cent);
  if (threadIdx.x < D) cT[(int64_t)threadIdx.x * a.nkb + kb] = cent[threadIdx.x];

  constexpr int C = D / 8, RG = NTHR / C;
  const int c = threadIdx.x % C, rg = threadIdx.x / C;
  double best = SOC_NEG_INF;
  for (int rbase = r0; rbase < r1; rbase += RG) {  // uniform trip count across the wave
    const int r = rbase + rg;
    double part = 0.0;
    if (r < r1) {
      double x[8];
      load8(base + (int64_t)r * a.k_st + 8 * c, x);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const double dlt = x[e] - cent[8 * c + e];
        part = fma(dlt, dlt, part);
      }
    }
#pragma unroll
    for (int m = 1; m < C; m <<= 1) part += __shfl_xor(part, m, 64);
    if (r < r1) best = fmax(best, part);
  }
  rmax[threadIdx.x] = best;
  __syncthreads();
  if (threadIdx.x == 0) {
    double m = SOC_NEG_INF;
    for (int i = 0; i < NTHR; ++i) m = fmax(m, rmax[i]);
    a.rad2[((int64_t)b * a.Hkv + kvh) * a.nkb + kb] = m;
  }
}

template <int D>
__global__ void __launch_bounds__(NTHR) score_kernel(SelectArgs a) {
  __shared__ double qm[D];
  const int qb = blockIdx.x % a.nqb;
  const int h = (blockIdx.x / a.nqb) % a.Hq;
  const int b = blockIdx.x / (a.nqb * a.Hq);
  const int kvh = h / a.g;
  const int off = seq_off(a, b), tkb = off + a.tq;
  if (threadIdx.x < D) qm[threadIdx.x] = a.qmean[(((int64_t)b * a.Hq + h) * a.nqb + qb) * D + threadIdx.x];
  __syncthreads();
  const double* cT = a.cT + ((int64_t)b * a.Hkv + kvh) * D * a.nkb;
  double* out = a.score + (((int64_t)b * a.Hq + h) * a.nqb + qb) * a.nkb;
  for (int kb = threadIdx.x; kb < a.nkb; kb += NTHR) {
    double s = SOC_NEG_INF;
    if (admissible(a, off, tkb, qb, kb)) {
      s = 0.0;
#pragma unroll 8
      for (int t = 0; t < D; ++t) s = fma(qm[t], cT[(int64_t)t * a.nkb + kb], s);
    }
    out[kb] = s;
  }
}

// Exact (n+1)-th largest of the finite values among `count` strided entries.
__device__ double order_statistic(const double* vals, int64_t count, double keep, unsigned* hist,
                                  unsigned long long* shared_u64) {
  constexpr int T = 1024;
  // population size
  unsigned long long local = 0;
  for (int64_t i = threadIdx.x; i < count; i += T) local += vals[i] > SOC_NEG_INF;
  if (threadIdx.x == 0) shared_u64[0] = 0;
  __syncthreads();
  atomicAdd(&shared_u64[0], local);
  __syncthreads();
  const unsigned long long N = shared_u64[0];
  const double nd = floor(keep * (double)N + 0.5);
  if (nd >= (double)N) return SOC_NEG_INF;
  unsigned long long rank = (unsigned long long)nd;  // descending rank of the answer
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
    if (threadIdx.x == 0) {
      unsigned long long cum = 0;
      int dg = 255;
      for (; dg > 0; --dg) {
        if (cum + hist[dg] > rank) break;
        cum += hist[dg];
      }
      rank -= cum;
      shared_u64[1] = prefix | ((unsigned long long)dg << shift);
    }
    __syncthreads();
    prefix = shared_u64[1];
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
    const double* vals = a.score + (int64_t)id * a.nqb * a.nkb;
    const double tau = order_statistic(vals, (int64_t)a.nqb * a.nkb, a.keep_mean, hist, su);
    if (threadIdx.x == 0) a.tau_mean[id] = tau;
  } else {
    id -= nmean;
    const double* vals = a.rad2 + (int64_t)id * a.nkb;
    const double tau = order_statistic(vals, a.nkb, a.keep_radius, hist, su);
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
  hipLaunchKernelGGL((qmean_kernel<T, D>), dim3(gq), dim3(NTHR), 0, s, a);
  hipLaunchKernelGGL((kstats_kernel<T, D>), dim3(gk), dim3(NTHR), 0, s, a);
  hipLaunchKernelGGL(score_kernel<D>, dim3(gq), dim3(NTHR), 0, s, a);
  const unsigned gt = (a.keep_mean >= 0.0 ? a.B * a.Hq : 0) + (a.keep_radius >= 0.0 ? a.B * a.Hkv : 0);
  if (gt) {
    SelectArgs t = a;
    if (a.keep_radius < 0.0) {  // only the mean branch
      hipLaunchKernelGGL(threshold_kernel, dim3(a.B * a.Hq), dim3(1024), 0, s, t);
    } else {
      hipLaunchKernelGGL(threshold_kernel, dim3(gt), dim3(1024), 0, s, t);
    }
  }
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
