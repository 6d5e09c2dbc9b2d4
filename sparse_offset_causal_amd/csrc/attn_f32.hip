// float32 attention path for gfx950 (head_dim 16, 32, 64 or 128): prefill and split-KV decode.
//
// Same semantics as the bf16 kernels (sotaaz.com/post/attention-in-code, listing
// attend/causal, sections 1 and 3), computed with plain fp32 VALU arithmetic: one thread
// per query row (prefill) or per (query row, split) (decode), walking only the keys its
// row may see -- [pos - W + 1, pos] clipped at 0, and in block-sparse mode only the listed
// key blocks -- with an online softmax in the log2 domain.  This path serves small head
// dims and tests the split/merge scheme at fp32 accuracy; it is not the throughput path.

#include "device_common.h"
#include "internal.h"

namespace soc {
namespace {

template <int D>
__device__ __forceinline__ void load_row(const float* p, float* out) {
#pragma unroll
  for (int c = 0; c < D / 4; ++c) {
    const f32x4 w = *(const f32x4*)(p + 4 * c);
#pragma unroll
    for (int e = 0; e < 4; ++e) out[4 * c + e] = w[e];
  }
}

template <int D>
struct RowState {
  float m, l, acc[D];
  __device__ void init(float m0, float l0) {
    m = m0;
    l = l0;
#pragma unroll
    for (int t = 0; t < D; ++t) acc[t] = 0.f;
  }
  // Online softmax over keys [j0, j1] (inclusive) of one KV head.
  __device__ void run(const float* q, const float* kp, const float* vp, int64_t kst, int j0, int j1,
                      float scale_log2) {
    for (int j = j0; j <= j1; ++j) {
      float kr[D];
      load_row<D>(kp + (int64_t)j * kst, kr);
      float dot = 0.f;
#pragma unroll
      for (int t = 0; t < D; ++t) dot = fmaf(q[t], kr[t], dot);
      const float x = dot * scale_log2;
      const float m_new = fmaxf(m, x);
      const float alpha = fast_exp2(m - m_new);
      const float p = fast_exp2(x - m_new);
      l = l * alpha + p;
      m = m_new;
      float vr[D];
      load_row<D>(vp + (int64_t)j * kst, vr);
#pragma unroll
      for (int t = 0; t < D; ++t) acc[t] = fmaf(p, vr[t], acc[t] * alpha);
    }
  }
};

template <int D, bool SPARSE>
__global__ void __launch_bounds__(64) prefill_f32_kernel(AttnArgs a) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)a.B * a.Hq * a.tq;
  if (gid >= total) return;
  const int r = (int)(gid % a.tq);
  const int h = (int)((gid / a.tq) % a.Hq);
  const int b = (int)(gid / ((int64_t)a.tq * a.Hq));
  const int kvh = h / a.g;
  const int off = a.cache_off ? a.cache_off[b] : a.tk - a.tq;
  const int pos = off + r;
  const int lo = a.window > 0 ? max(0, pos - a.window + 1) : 0;

  float q[D];
  load_row<D>((const float*)a.q + b * a.q_sb + h * a.q_sh + (int64_t)r * a.q_st, q);
  const float* kp = (const float*)a.k + b * a.kv_sb + kvh * a.kv_sh;
  const float* vp = (const float*)a.v + b * a.kv_sb + kvh * a.kv_sh;

  RowState<D> st;
  if (a.sink)
    st.init(a.sink[h] * kLog2e, 1.f);
  else
    st.init(SOC_NEG_INF, 0.f);
  if (SPARSE && a.block_list) {
    const int32_t* lst = a.block_list + ((int64_t)(b * a.Hq + h) * a.n_qb + r / a.block_size) * a.list_stride;
    const int cnt = lst[0];
    for (int e = 0; e < cnt; ++e) {
      const int kb = lst[1 + e];
      const int j0 = max(lo, kb * a.block_size), j1 = min(pos, kb * a.block_size + a.block_size - 1);
      if (j0 <= j1) st.run(q, kp, vp, a.kv_st, j0, j1, a.scale_log2);
    }
  } else if (SPARSE) {  // block mask: the kept key blocks of the row's range
    const uint8_t* mrow = a.block_mask + ((int64_t)(b * a.Hq + h) * a.n_qb + r / a.block_size) * a.mask_stride;
    for (int kb = lo / a.block_size; kb <= pos / a.block_size; ++kb) {
      if (!mrow[kb]) continue;
      const int j0 = max(lo, kb * a.block_size), j1 = min(pos, kb * a.block_size + a.block_size - 1);
      st.run(q, kp, vp, a.kv_st, j0, j1, a.scale_log2);
    }
  } else {
    st.run(q, kp, vp, a.kv_st, lo, pos, a.scale_log2);
  }
  const float inv = st.l > 0.f ? 1.f / st.l : 0.f;
  float* op = (float*)a.o + b * a.o_sb + h * a.o_sh + (int64_t)r * a.o_st;
#pragma unroll
  for (int t = 0; t < D; ++t) op[t] = st.acc[t] * inv;
}

template <int D>
__global__ void __launch_bounds__(64) decode_split_f32_kernel(AttnArgs a) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t rows = (int64_t)a.B * a.Hq * a.tq;
  if (gid >= rows * a.nsplit) return;
  const int s = (int)(gid % a.nsplit);
  const int64_t rowid = gid / a.nsplit;
  const int r = (int)(rowid % a.tq);
  const int h = (int)((rowid / a.tq) % a.Hq);
  const int b = (int)(rowid / ((int64_t)a.tq * a.Hq));
  const int kvh = h / a.g;
  const int off = a.cache_off ? a.cache_off[b] : a.tk - a.tq;
  const int tkb = off + a.tq;
  const int nsb = (tkb + a.split - 1) / a.split;
  if (s >= nsb) return;
  const int pos = off + r;
  const int lo = a.window > 0 ? max(0, pos - a.window + 1) : 0;
  const int j0 = max(lo, s * a.split), j1 = min(pos, s * a.split + a.split - 1);

  float q[D];
  load_row<D>((const float*)a.q + b * a.q_sb + h * a.q_sh + (int64_t)r * a.q_st, q);
  RowState<D> st;
  st.init(SOC_NEG_INF, 0.f);
  if (j0 <= j1)
    st.run(q, (const float*)a.k + b * a.kv_sb + kvh * a.kv_sh, (const float*)a.v + b * a.kv_sb + kvh * a.kv_sh,
           a.kv_st, j0, j1, a.scale_log2);
  float* po = a.part + (rowid * a.nsplit + s) * a.d;
#pragma unroll
  for (int t = 0; t < D; ++t) po[t] = st.acc[t];
  float* pml = a.part + decode_o_floats(a) + (rowid * a.nsplit + s) * 2;
  pml[0] = st.m;
  pml[1] = st.l;
}

template <int D>
hipError_t launch_prefill_f32_d(const AttnArgs& a, hipStream_t s) {
  const int64_t total = (int64_t)a.B * a.Hq * a.tq;
  const unsigned grid = (unsigned)((total + 63) / 64);
  if (a.block_list || a.block_mask)
    hipLaunchKernelGGL((prefill_f32_kernel<D, true>), dim3(grid), dim3(64), 0, s, a);
  else
    hipLaunchKernelGGL((prefill_f32_kernel<D, false>), dim3(grid), dim3(64), 0, s, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_decode_f32_d(const AttnArgs& a, hipStream_t s) {
  const int64_t total = (int64_t)a.B * a.Hq * a.tq * a.nsplit;
  const unsigned grid = (unsigned)((total + 63) / 64);
  hipLaunchKernelGGL(decode_split_f32_kernel<D>, dim3(grid), dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_f32(const AttnArgs& a, hipStream_t s) {
  if ((int64_t)a.B * a.Hq * a.tq == 0) return hipSuccess;
  switch (a.d) {
    case 16: return launch_prefill_f32_d<16>(a, s);
    case 32: return launch_prefill_f32_d<32>(a, s);
    case 64: return launch_prefill_f32_d<64>(a, s);
    case 128: return launch_prefill_f32_d<128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode_f32(const AttnArgs& a, hipStream_t s) {
  if ((int64_t)a.B * a.Hq * a.tq == 0) return hipSuccess;
  switch (a.d) {
    case 16: return launch_decode_f32_d<16>(a, s);
    case 32: return launch_decode_f32_d<32>(a, s);
    case 64: return launch_decode_f32_d<64>(a, s);
    case 128: return launch_decode_f32_d<128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace soc
