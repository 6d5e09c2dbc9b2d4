// Split-KV decode for gfx950 (bf16 cache, head_dim 128) and the merge pass.
//
// Decode cost is the bytes read from the cache per step (sotaaz.com/post/attention-in-code,
// sections 1 and 5: the cache holds n_kv heads per token, and what a step costs is what it
// reads).  So every workgroup owns one (sequence, KV head, split of `split` keys) and
// serves all g = n_heads / n_kv query heads x tq rows of that group (<= 32 rows) from a
// single read of the split's K and V: K/V bytes cross HBM exactly once per call.
//
// Per workgroup: 4 waves; the split is walked in 128-key tiles loaded cooperatively with
// coalesced 16-byte loads (K row-major with an XOR chunk swizzle, V transposed) and
// prefetched into registers one tile ahead; wave w takes keys 32w..32w+31 of each tile and
// computes S^T = K Q^T and O^T += V^T P^T with v_mfma_f32_32x32x16_bf16 (query rows are the
// MFMA's N columns, padded to 32).  The four waves' running (max, sum, O) are merged through
// LDS at the end and the split's unnormalised partial is written in fp32.  The sink is not
// applied here; the merge adds it exactly once per row.
//
// Merge: per (b, h, r) row, M = max(max_s m_s, sink), L = sum_s l_s 2^(m_s - M) + 2^(sink - M),
// o = sum_s o_s 2^(m_s - M) / L (all in the log2 domain), rounded once to the output type.

#include "device_common.h"
#include "internal.h"

namespace soc {
namespace {

constexpr int D = 128;
constexpr int KT = 128;      // keys per tile
constexpr int NTHR = 256;
constexpr int VST = KT + 8;  // V^T row stride (elements)
constexpr int LDS_BYTES = KT * D * 2 + D * VST * 2;  // 32 KB + 34 KB

__device__ __forceinline__ int vt_col(int key) {
  return (key & ~15) | (key & 3) | ((key & 4) << 1) | ((key & 8) >> 1);
}

__global__ void __launch_bounds__(NTHR) decode_split_bf16_d128(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[LDS_BYTES];
  bf16_t* k_lds = (bf16_t*)lds;
  bf16_t* vt_lds = (bf16_t*)(lds + KT * D * 2);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int s = blockIdx.x % a.nsplit;
  const int rem = blockIdx.x / a.nsplit;
  const int kvh = rem % a.Hkv, b = rem / a.Hkv;
  const int off = a.cache_off ? a.cache_off[b] : a.tk - a.tq;
  const int tkb = off + a.tq;
  const int nsb = (tkb + a.split - 1) / a.split;
  if (s >= nsb) return;  // the merge reads only splits below nsb
  const int ks0 = s * a.split, ks1 = min(ks0 + a.split, tkb);
  const int kv_lo = a.window > 0 ? max(0, off - a.window + 1) : 0;
  const int kbeg = max(ks0, kv_lo), kend = ks1;

  // query row of this lane: rho = head-in-group * tq + r
  const int R = a.g * a.tq;
  const int rho = l32;
  const bool row_ok = rho < R;
  const int h = kvh * a.g + (row_ok ? rho / a.tq : 0);
  const int r = row_ok ? rho % a.tq : 0;
  const int pos = row_ok ? off + r : -1;

  const bf16_t* qp = (const bf16_t*)a.q + b * a.q_sb + h * a.q_sh + (int64_t)r * a.q_st;
  const bf16_t* kp = (const bf16_t*)a.k + b * a.kv_sb + kvh * a.kv_sh;
  const bf16_t* vp = (const bf16_t*)a.v + b * a.kv_sb + kvh * a.kv_sh;

  bf16x8 qf[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    u32x4 z = {0u, 0u, 0u, 0u};
    qf[ks] = row_ok ? *(const bf16x8*)(qp + 16 * ks + 8 * hh) : as_bf16x8(z);
  }

  f32x16 oacc[4];
#pragma unroll
  for (int tb = 0; tb < 4; ++tb)
#pragma unroll
    for (int v = 0; v < 16; ++v) oacc[tb][v] = 0.f;
  float m_run = SOC_NEG_INF, l_run = 0.f;

  u32x4 kreg[8], vreg[8];
  auto load_tile = [&](int jb) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int ci = tid + NTHR * i;
      const int kk = ci >> 4, kc = ci & 15;
      const int vk = ci & 127, vc = ci >> 7;
      u32x4 z = {0u, 0u, 0u, 0u};
      kreg[i] = (jb + kk < kend) ? *(const u32x4*)(kp + (int64_t)(jb + kk) * a.kv_st + kc * 8) : z;
      vreg[i] = (jb + vk < kend) ? *(const u32x4*)(vp + (int64_t)(jb + vk) * a.kv_st + vc * 8) : z;
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int ci = tid + NTHR * i;
      const int kk = ci >> 4, kc = ci & 15;
      *(u32x4*)(k_lds + kk * D + ((kc ^ (kk & 15)) << 3)) = kreg[i];
      const int vk = ci & 127, vc = ci >> 7;
      const int col = vt_col(vk);
      const u32x4 w = vreg[i];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vt_lds[(vc * 8 + 2 * e) * VST + col] = __builtin_bit_cast(bf16_t, (uint16_t)(w[e] & 0xffffu));
        vt_lds[(vc * 8 + 2 * e + 1) * VST + col] = __builtin_bit_cast(bf16_t, (uint16_t)(w[e] >> 16));
      }
    }
  };

  if (kbeg < kend) load_tile(kbeg);
  for (int jb = kbeg; jb < kend; jb += KT) {
    store_tile();
    __syncthreads();
    if (jb + KT < kend) load_tile(jb + KT);

    const int js = jb + 32 * wave;  // this wave's 32 keys
    if (js < kend) {
      f32x16 sacc;
#pragma unroll
      for (int v = 0; v < 16; ++v) sacc[v] = 0.f;
      const int krow = 32 * wave + l32;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const bf16x8 ka = *(const bf16x8*)(k_lds + krow * D + (((2 * ks + hh) ^ (krow & 15)) << 3));
        sacc = mfma32x32x16(ka, qf[ks], sacc);
      }
      float x[16];
      float mx = SOC_NEG_INF;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int j = js + 8 * (v >> 2) + 4 * hh + (v & 3);
        const bool ok = j < kend && j <= pos && (a.window <= 0 || j > pos - a.window);
        x[v] = ok ? sacc[v] * a.scale_log2 : SOC_NEG_INF;
        mx = fmaxf(mx, x[v]);
      }
      mx = fmaxf(mx, swap_halves(mx));
      const float m_new = fmaxf(m_run, mx);
      const float m_use = (m_new == SOC_NEG_INF) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      float lsum = 0.f;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        x[v] = fast_exp2(x[v] - m_use);
        lsum += x[v];
      }
      l_run = l_run * alpha + lsum;
      m_run = m_new;
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[tb][v] *= alpha;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        bf16x8 pb;
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[e] = (bf16_t)x[kk * 8 + e];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
          const bf16x8 va = *(const bf16x8*)(vt_lds + (tb * 32 + l32) * VST + 32 * wave + 16 * kk + 8 * hh);
          oacc[tb] = mfma32x32x16(va, pb, oacc[tb]);
        }
      }
    }
    __syncthreads();
  }

  // Merge the four waves' states through LDS (the tile buffers are free now).
  float* lo = (float*)lds;               // [wave][tb][v][lane]
  float* lml = lo + 4 * 4 * 16 * 64;     // [wave][lane][2]
#pragma unroll
  for (int tb = 0; tb < 4; ++tb)
#pragma unroll
    for (int v = 0; v < 16; ++v) lo[((wave * 4 + tb) * 16 + v) * 64 + lane] = oacc[tb][v];
  lml[(wave * 64 + lane) * 2 + 0] = m_run;
  lml[(wave * 64 + lane) * 2 + 1] = l_run;
  __syncthreads();

  float M = SOC_NEG_INF;
#pragma unroll
  for (int w = 0; w < 4; ++w) M = fmaxf(M, lml[(w * 64 + lane) * 2]);
  const float M_use = (M == SOC_NEG_INF) ? 0.f : M;
  float wt[4], L = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    wt[w] = fast_exp2(lml[(w * 64 + lane) * 2] - M_use);
    L += (lml[(w * 64 + lane) * 2 + 1] + lml[(w * 64 + (lane ^ 32)) * 2 + 1]) * wt[w];
  }
  if (row_ok) {
    const int64_t rowid = ((int64_t)b * a.Hq + h) * a.tq + r;
    float* po = a.part + (rowid * a.nsplit + s) * D;
    const int tb = wave;
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      f32x4 out;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int v = 4 * g4 + e;
        float acc = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) acc += lo[((w * 4 + tb) * 16 + v) * 64 + lane] * wt[w];
        out[e] = acc;
      }
      *(f32x4*)(po + tb * 32 + 8 * g4 + 4 * hh) = out;
    }
    if (wave == 0 && hh == 0) {
      float* pml = a.part + decode_o_floats(a) + (rowid * a.nsplit + s) * 2;
      pml[0] = M;
      pml[1] = L;
    }
  }
}

template <typename OutT>
__global__ void __launch_bounds__(64) decode_merge(AttnArgs a) {
  const int64_t rowid = blockIdx.x;
  const int r = (int)(rowid % a.tq);
  const int h = (int)((rowid / a.tq) % a.Hq);
  const int b = (int)(rowid / ((int64_t)a.tq * a.Hq));
  const int off = a.cache_off ? a.cache_off[b] : a.tk - a.tq;
  const int tkb = off + a.tq;
  const int nsb = (tkb + a.split - 1) / a.split;
  const float* pml = a.part + decode_o_floats(a) + rowid * a.nsplit * 2;
  const float* po = a.part + rowid * a.nsplit * a.d;
  float M = SOC_NEG_INF;
  for (int s = 0; s < nsb; ++s) M = fmaxf(M, pml[2 * s]);
  const float sink_l2 = a.sink ? a.sink[h] * kLog2e : SOC_NEG_INF;
  M = fmaxf(M, sink_l2);
  const float M_use = (M == SOC_NEG_INF) ? 0.f : M;
  float L = fast_exp2(sink_l2 - M_use);
  for (int s = 0; s < nsb; ++s) L += pml[2 * s + 1] * fast_exp2(pml[2 * s] - M_use);
  const float inv = L > 0.f ? 1.f / L : 0.f;
  OutT* op = (OutT*)a.o + b * a.o_sb + h * a.o_sh + (int64_t)r * a.o_st;
  for (int t = threadIdx.x; t < a.d; t += 64) {
    float acc = 0.f;
    for (int s = 0; s < nsb; ++s) acc += po[(int64_t)s * a.d + t] * fast_exp2(pml[2 * s] - M_use);
    op[t] = (OutT)(acc * inv);
  }
}

}  // namespace

hipError_t launch_decode_bf16(const AttnArgs& a, hipStream_t s) {
  const int64_t grid = (int64_t)a.B * a.Hkv * a.nsplit;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(decode_split_bf16_d128, dim3((unsigned)grid), dim3(NTHR), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_decode_merge(const AttnArgs& a, bool out_bf16, hipStream_t s) {
  const int64_t grid = (int64_t)a.B * a.Hq * a.tq;
  if (grid == 0) return hipSuccess;
  if (out_bf16)
    hipLaunchKernelGGL(decode_merge<bf16_t>, dim3((unsigned)grid), dim3(64), 0, s, a);
  else
    hipLaunchKernelGGL(decode_merge<float>, dim3((unsigned)grid), dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace soc
