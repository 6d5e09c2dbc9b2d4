// bf16 offset-causal attention prefill for gfx950, head_dim 128.
//
// Computes, per query row r of a tq-row block at cache offset off_b, the softmax over the
// keys j <= off_b + r (and j > off_b + r - W with a window; and only listed key blocks in
// block-sparse mode) of scale * q.k, weighted sum of v, with an optional per-head sink
// logit in the normaliser (sotaaz.com/post/attention-in-code, listing attend/causal and
// sections 1 and 3; patty.io RBS-Attention review, section on block-sparse execution).
//
// Work decomposition
//   workgroup = 4 waves = 128 query rows of one (b, h); wave w owns rows 32w..32w+31.
//   The workgroup walks 64-key tiles of the KV interval its rows can see; tiles outside
//   the interval (beyond the last row's position, before the first row's window, or not
//   in the block list) are never loaded.
//   Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16, so each
//   lane owns one query row (lane % 32) and 16 keys per 32-key block: the row max and sum
//   need one exchange between the two wave halves, and the output O^T = V^T P^T again
//   leaves one row per lane, so the softmax rescale is a per-lane scalar.
//   Masks are computed from indices only on tiles that cross a row's causal limit or
//   window edge.  The online softmax runs in the log2 domain in fp32; P is rounded to bf16
//   for the second MFMA; O accumulates in fp32 and is rounded to bf16 once at the end.
//
// LDS (34 KB): the K tile row-major with a 16-byte-chunk XOR swizzle (conflict-free 16-byte
// reads of 16 consecutive keys), and the V tile transposed (V^T, 128 x 64 plus 8 pad) with
// the key order inside each 16-key group permuted so that a lane's 8 contraction values are
// one 16-byte read.  The next tile is prefetched into registers while the current one is
// being consumed.
//
// Grid order: workgroup i runs on XCD i % 8.  When the number of KV groups (batch x n_kv)
// is a multiple of 8, each XCD is given whole KV groups (their K/V stay in that XCD's L2),
// and within an XCD the query tiles with the most keys are dispatched first.

#include "device_common.h"
#include "internal.h"

namespace soc {
namespace {

constexpr int D = 128;
constexpr int QT = 128;       // query rows per workgroup
constexpr int KT = 64;        // keys per tile
constexpr int NTHR = 256;
constexpr int VST = KT + 8;   // V^T row stride (elements): 144 bytes

// Column of key `key` (0..63) inside a V^T row: bits 2 and 3 swapped, so that the keys
// {4h..4h+3, 8+4h..8+4h+3} of each 16-key group are contiguous at 8h.
__device__ __forceinline__ int vt_col(int key) {
  return (key & ~15) | (key & 3) | ((key & 4) << 1) | ((key & 8) >> 1);
}

__device__ __forceinline__ void map_block(int bid, const AttnArgs& a, int n_qt, int& qt, int& h, int& b) {
  const int units = a.B * a.Hkv;
  if ((units & 7) == 0) {
    const int xcd = bid & 7, j = bid >> 3;
    const int upx = units >> 3;
    const int per_row = upx * a.g;
    const int qt_rev = j / per_row;
    const int rem = j - qt_rev * per_row;
    const int ul = rem / a.g, hg = rem - ul * a.g;
    const int unit = ul * 8 + xcd;
    b = unit / a.Hkv;
    const int kvh = unit - b * a.Hkv;
    h = kvh * a.g + hg;
    qt = n_qt - 1 - qt_rev;
  } else {
    const int per_row = a.B * a.Hq;
    const int qt_rev = bid / per_row;
    const int rem = bid - qt_rev * per_row;
    b = rem / a.Hq;
    h = rem - b * a.Hq;
    qt = n_qt - 1 - qt_rev;
  }
}

template <bool SPARSE>
__global__ void __launch_bounds__(NTHR) prefill_bf16_d128(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) bf16_t k_lds[KT * D];
  __shared__ __attribute__((aligned(16))) bf16_t vt_lds[D * VST];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int n_qt = (a.tq + QT - 1) / QT;
  int qt, h, b;
  map_block(blockIdx.x, a, n_qt, qt, h, b);
  const int kvh = h / a.g;
  const int off = a.cache_off ? a.cache_off[b] : a.tk - a.tq;
  const int tkb = off + a.tq;
  const int row0 = qt * QT;
  const int rowl = min(row0 + QT, a.tq) - 1;
  const int kv_hi = min(tkb, off + rowl + 1);
  const int kv_lo = a.window > 0 ? max(0, off + row0 - a.window + 1) : 0;
  const int t_lo = kv_lo / KT, t_hi = (kv_hi + KT - 1) / KT;

  const int wr0 = row0 + wave * 32;
  const int wrl = min(wr0 + 31, rowl);
  const bool wave_active = wr0 <= rowl;
  const int my_row = wr0 + l32;
  const int my_pos = off + my_row;
  const int wpos_lo = off + wr0, wpos_hi = off + wrl;

  const bf16_t* qp = (const bf16_t*)a.q + b * a.q_sb + h * a.q_sh;
  const bf16_t* kp = (const bf16_t*)a.k + b * a.kv_sb + kvh * a.kv_sh;
  const bf16_t* vp = (const bf16_t*)a.v + b * a.kv_sb + kvh * a.kv_sh;

  bf16x8 qf[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    u32x4 z = {0u, 0u, 0u, 0u};
    qf[ks] = (my_row < a.tq) ? *(const bf16x8*)(qp + (int64_t)my_row * a.q_st + 16 * ks + 8 * hh) : as_bf16x8(z);
  }

  f32x16 oacc[4];
#pragma unroll
  for (int tb = 0; tb < 4; ++tb)
#pragma unroll
    for (int v = 0; v < 16; ++v) oacc[tb][v] = 0.f;
  float m_run = SOC_NEG_INF, l_run = 0.f;
  if (a.sink) {
    m_run = a.sink[h] * kLog2e;
    l_run = hh == 0 ? 1.f : 0.f;
  }

  // Tile sequence: dense = t_lo .. t_hi-1; sparse = the two 64-key halves of each listed
  // 128-key block, restricted to [t_lo, t_hi) (a contiguous run, the list is ascending).
  const int32_t* lst = nullptr;
  int n0 = 0, n1 = 0;
  if (SPARSE) {
    lst = a.block_list + ((int64_t)(b * a.Hq + h) * a.n_qb + qt) * a.list_stride;
    const int cnt = lst[0];
    n1 = 2 * cnt;
    while (n0 < n1 && 2 * lst[1 + (n0 >> 1)] + (n0 & 1) < t_lo) ++n0;
    int e = n0;
    while (e < n1 && 2 * lst[1 + (e >> 1)] + (e & 1) < t_hi) ++e;
    n1 = e;
  } else {
    n0 = 0;
    n1 = max(0, t_hi - t_lo);
  }
  auto tile_of = [&](int n) -> int { return SPARSE ? 2 * lst[1 + (n >> 1)] + (n & 1) : t_lo + n; };

  u32x4 kreg[4], vreg[4];
  auto load_tile = [&](int t) {
    const int jb = t * KT;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ci = tid + NTHR * i;
      const int kk = ci >> 4, kc = ci & 15;  // K: 4 keys x 16 chunks per wave (coalesced)
      const int vk = ci & 63, vc = ci >> 6;  // V: 64 keys x 1 chunk per wave
      u32x4 z = {0u, 0u, 0u, 0u};
      kreg[i] = (jb + kk < kv_hi) ? *(const u32x4*)(kp + (int64_t)(jb + kk) * a.kv_st + kc * 8) : z;
      vreg[i] = (jb + vk < kv_hi) ? *(const u32x4*)(vp + (int64_t)(jb + vk) * a.kv_st + vc * 8) : z;
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ci = tid + NTHR * i;
      const int kk = ci >> 4, kc = ci & 15;
      *(u32x4*)(k_lds + kk * D + ((kc ^ (kk & 15)) << 3)) = kreg[i];
      const int vk = ci & 63, vc = ci >> 6;
      const int col = vt_col(vk);
      const u32x4 w = vreg[i];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vt_lds[(vc * 8 + 2 * e) * VST + col] = __builtin_bit_cast(bf16_t, (uint16_t)(w[e] & 0xffffu));
        vt_lds[(vc * 8 + 2 * e + 1) * VST + col] = __builtin_bit_cast(bf16_t, (uint16_t)(w[e] >> 16));
      }
    }
  };

  if (n0 < n1) load_tile(tile_of(n0));
  for (int n = n0; n < n1; ++n) {
    const int t = tile_of(n);
    store_tile();
    __syncthreads();
    if (n + 1 < n1) load_tile(tile_of(n + 1));

    const int j0 = t * KT;
    const bool skip = !wave_active || j0 > wpos_hi || (a.window > 0 && j0 + KT - 1 <= wpos_lo - a.window);
    if (!skip) {
      const bool need_mask = (j0 + KT - 1 > wpos_lo) || (a.window > 0 && j0 <= wpos_hi - a.window);
      f32x16 s0, s1;
#pragma unroll
      for (int v = 0; v < 16; ++v) { s0[v] = 0.f; s1[v] = 0.f; }
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const int sw = ((2 * ks + hh) ^ (l32 & 15)) << 3;
        const bf16x8 ka = *(const bf16x8*)(k_lds + l32 * D + sw);
        const bf16x8 kb = *(const bf16x8*)(k_lds + (32 + l32) * D + sw);
        s0 = mfma32x32x16(ka, qf[ks], s0);
        s1 = mfma32x32x16(kb, qf[ks], s1);
      }
      float x[32];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        x[v] = s0[v] * a.scale_log2;
        x[16 + v] = s1[v] * a.scale_log2;
      }
      if (need_mask) {
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          const int j = j0 + (i >> 4) * 32 + 8 * ((i & 15) >> 2) + 4 * hh + (i & 3);
          const bool ok = j <= my_pos && (a.window <= 0 || j > my_pos - a.window);
          x[i] = ok ? x[i] : SOC_NEG_INF;
        }
      }
      float mx = x[0];
#pragma unroll
      for (int i = 1; i < 32; ++i) mx = fmaxf(mx, x[i]);
      mx = fmaxf(mx, swap_halves(mx));
      const float m_new = fmaxf(m_run, mx);
      const float m_use = (m_new == SOC_NEG_INF) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      float lsum = 0.f;
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        x[i] = fast_exp2(x[i] - m_use);
        lsum += x[i];
      }
      l_run = l_run * alpha + lsum;
      m_run = m_new;
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[tb][v] *= alpha;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        bf16x8 pb;
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[e] = (bf16_t)x[kk * 8 + e];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
          const bf16x8 va = *(const bf16x8*)(vt_lds + (tb * 32 + l32) * VST + 16 * kk + 8 * hh);
          oacc[tb] = mfma32x32x16(va, pb, oacc[tb]);
        }
      }
    }
    __syncthreads();
  }

  const float lt = l_run + swap_halves(l_run);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (my_row < a.tq) {
    bf16_t* op = (bf16_t*)a.o + b * a.o_sb + h * a.o_sh + (int64_t)my_row * a.o_st;
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (bf16_t)(oacc[tb][4 * g4 + e] * inv);
        *(bf16x4*)(op + tb * 32 + 8 * g4 + 4 * hh) = w;
      }
  }
}

}  // namespace

hipError_t launch_prefill_bf16(const AttnArgs& a, hipStream_t s) {
  const int n_qt = (a.tq + QT - 1) / QT;
  const int64_t grid = (int64_t)n_qt * a.B * a.Hq;
  if (grid == 0) return hipSuccess;
  if (a.block_list)
    hipLaunchKernelGGL(prefill_bf16_d128<true>, dim3((unsigned)grid), dim3(NTHR), 0, s, a);
  else
    hipLaunchKernelGGL(prefill_bf16_d128<false>, dim3((unsigned)grid), dim3(NTHR), 0, s, a);
  return hipGetLastError();
}

}  // namespace soc
