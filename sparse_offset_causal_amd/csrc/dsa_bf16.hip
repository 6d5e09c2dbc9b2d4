// Token top-k sparse attention decode for gfx950 (bf16 in, fp32 accumulate, head_dim 128).
//
// A small scorer (the indexer) rates every token a query token may see, and attention runs
// only over the k best-rated ones; the cache stays whole (sotaaz.com/post/attention-in-code,
// section 5).  Indexer score of cached token s for query token t:
//   sum over indexer heads j of w[j, t] * relu(qi[j, t] . ki[s]).
// The kept set of a query token is its top k visible tokens (all of them if fewer are
// visible); equal scores go to the lower token index.  Every head of the query token attends
// over the same kept set.
//
//   dsa_indexer_kernel  a fixed grid of single-wave workgroups (three per SIMD), each scoring
//                       an equal share of all 16-token blocks of all (sequence, query token)
//                       rows, so that every wave ends at about the same time: scores^T =
//                       Ki Qi^T with v_mfma_f32_16x16x32_bf16 (16 tokens x 16 indexer heads per
//                       MFMA), ReLU and the head weights in fp32, the sum over heads in a fixed
//                       order (DPP within each 16-lane row)
//   dsa_topk_kernel     one 1024-thread workgroup per (sequence, query token): radix select of
//                       the k-th largest score on order-preserving 32-bit keys (digits of 12,
//                       12 and 8 bits; the first histogram is built while the keys are staged
//                       in LDS), then an index-ordered compaction (ties at the threshold:
//                       lowest indices) into an ascending list, one contiguous token segment
//                       per wave
//   dsa_split_kernel    split-KV decode over the kept list: one wave per (sequence, KV head,
//                       query token, split of the list); K rows are gathered by index straight
//                       into registers and V rows by index into LDS (buffer loads with the LDS
//                       bit, per-lane offsets from the list), then the same MFMA / online
//                       softmax scheme as the dense decode; partials merge in decode_merge.

#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace soc {
namespace {

constexpr int D = 128;
constexpr int DI = kDsaIndexDim;
constexpr int KB = 32;
constexpr int NST = 3;
constexpr int VSTAGE = KB * D;
constexpr int MAX_SPLIT = 1024;  // kept-list entries per split (staged in LDS)
constexpr float RESCALE_SLACK = 8.0f;

typedef short s16x4 __attribute__((__vector_size__(8)));
typedef short s16x8 __attribute__((__vector_size__(16)));
typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef __attribute__((address_space(3))) s16x4* lds_s16x4_ptr;

__device__ __forceinline__ f32x4 mfma16k32(bf16x8 a, bf16x8 b, f32x4 c) {
  // lane l: A[l%16][8(l/16)+e], B[8(l/16)+e][l%16], D[4(l/16)+v][l%16]
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// Sum over each row of 16 lanes with DPP (xor 1, xor 2, then the mirrors within 8 and 16
// lanes), the same pairing as a butterfly on lane ^ 1, 2, 4, 8.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_f32<0xb1>(x);   // quad_perm [1,0,3,2]
  x += dpp_f32<0x4e>(x);   // quad_perm [2,3,0,1]
  x += dpp_f32<0x141>(x);  // row_half_mirror
  x += dpp_f32<0x140>(x);  // row_mirror
  return x;
}
__device__ __forceinline__ uint32_t f32_order_key(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  return (u >> 31) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ int seq_off(const AttnArgs& a, int b) { return a.cache_off ? a.cache_off[b] : a.tk - a.tq; }

// ---------------------------------------------------------------------------------------
// Sum and inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_sum_i(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}
__device__ __forceinline__ int wave_incl_prefix_i(int x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  return x;
}

__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(3))) dsa_indexer_kernel(DsaArgs A) {
  const AttnArgs& a = A.at;
  const int lane = threadIdx.x, G = lane >> 4, i16 = lane & 15;
  const int rows = a.B * a.tq;
  // Row r = b * tq + t has nb(r) = ceil(n_vis / 16) blocks of 16 tokens; the blocks of all
  // rows, in row order, are split evenly over the waves of the grid.
  auto row_blocks = [&](int r) __attribute__((always_inline)) -> int {
    if (r >= rows) return 0;
    const int b = r / a.tq, t = r - b * a.tq;
    return (min(a.tk, seq_off(a, b) + t + 1) + 15) >> 4;
  };
  int total = 0;
  for (int r0 = 0; r0 < rows; r0 += 64) total += wave_sum_i(row_blocks(r0 + lane));
  total = __builtin_amdgcn_readfirstlane(total);
  const int W = gridDim.x, wid = blockIdx.x;
  const int lo = (int)((int64_t)total * wid / W), hi = (int)((int64_t)total * (wid + 1) / W);
  if (lo >= hi) return;
  int row = 0, rstart = 0;  // the row holding block lo and the global index of its first block
  for (int r0 = 0, base = 0; r0 < rows; r0 += 64) {
    const int nb = row_blocks(r0 + lane);
    const int incl = base + wave_incl_prefix_i(nb);
    const unsigned long long own = __ballot(nb > 0 && incl - nb <= lo && lo < incl);
    if (own) {
      const int L = __ffsll(own) - 1;
      row = r0 + L;
      rstart = __builtin_amdgcn_readlane(incl - nb, L);
      break;
    }
    base = __builtin_amdgcn_readlane(incl, 63);
  }
  row = __builtin_amdgcn_readfirstlane(row);
  rstart = __builtin_amdgcn_readfirstlane(rstart);

  const int nhb = A.Hi / 16;
  const uint32_t row_bytes = (uint32_t)A.ki_st * 2u;
  const u32x4 z = {0u, 0u, 0u, 0u};
  for (int g = lo; g < hi;) {
    const int b = __builtin_amdgcn_readfirstlane(row / a.tq);
    const int t = __builtin_amdgcn_readfirstlane(row - b * a.tq);
    const int n_vis = __builtin_amdgcn_readfirstlane(min(a.tk, seq_off(a, b) + t + 1));
    const int nb_row = (n_vis + 15) >> 4;
    bf16x8 qb[4][4];
    float w[4];
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
      const int head = 16 * hb + i16;
      const bool ok = hb < nhb;
      const bf16_t* qp = (const bf16_t*)A.qi + b * A.qi_sb + head * A.qi_sh + t * A.qi_st;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) qb[hb][ks] = ok ? *(const bf16x8*)(qp + 32 * ks + 8 * G) : as_bf16x8(z);
      w[hb] = ok ? A.wi[((int64_t)b * A.Hi + head) * a.tq + t] : 0.f;
    }
    const bf16_t* kp = (const bf16_t*)A.ki + b * A.ki_sb;
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)kp, (short)0, (int)(n_vis * row_bytes), 0x00020000);
    float* out = A.scores + ((int64_t)b * a.tq + t) * a.tk;
    const __amdgpu_buffer_rsrc_t ors = __builtin_amdgcn_make_buffer_rsrc((void*)out, (short)0, (int)(n_vis * 4), 0x00020000);
    const int j0 = g - rstart, j1 = min(nb_row, hi - rstart);  // this wave's blocks of the row
    auto load = [&](bf16x8* af, int j) __attribute__((always_inline)) {
      const int tok0 = 16 * j;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        af[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                                krs, (uint32_t)(tok0 + i16) * row_bytes + (uint32_t)(64 * ks + 16 * G), 0, 0));
    };
    auto score = [&](const bf16x8* af, int j) __attribute__((always_inline)) {
      const int tok0 = 16 * j;
      float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int hb = 0; hb < 4; ++hb) {
        if (hb >= nhb) break;  // uniform
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) acc = mfma16k32(af[ks], qb[hb][ks], acc);
#pragma unroll
        for (int v = 0; v < 4; ++v) part[v] = fmaf(w[hb], fmaxf(acc[v], 0.f), part[v]);
      }
      // lane (G, i16): tokens 4G + v, indexer head i16 of each block; sum over the 16 heads.
      // Lane i16 == 0 of each group stores through a buffer whose range ends at the row's
      // last visible token; the other lanes' stores fall outside the range and are dropped
      // (no branch, so the compiler can keep counting the key loads still in flight).
#pragma unroll
      for (int v = 0; v < 4; ++v) part[v] = row16_sum(part[v]);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const uint32_t at = i16 == 0 ? (uint32_t)(tok0 + 4 * G + v) * 4u : 0x80000000u;
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, part[v]), ors, at, 0, 0);
      }
    };
    // the keys of blocks j + 1 and j + 2 are in flight while block j is scored (three
    // rotating buffers; with one block ahead the waves held too few bytes in flight to
    // cover the memory latency)
    // Every load is issued unconditionally (past the segment's last block it reloads that
    // block), so the number of loads in flight is the same on every path.
    bf16x8 fa[4], fb[4], fc[4];
    const int jl = j1 - 1;
    load(fa, min(j0, jl));
    load(fb, min(j0 + 1, jl));
    for (int j = j0; j < j1; j += 3) {
      load(fc, min(j + 2, jl));
      score(fa, j);
      if (j + 1 >= j1) break;
      load(fa, min(j + 3, jl));
      score(fb, j + 1);
      if (j + 2 >= j1) break;
      load(fb, min(j + 4, jl));
      score(fc, j + 2);
    }
    g = rstart + j1;
    rstart += nb_row;
    ++row;
  }
}

// ---------------------------------------------------------------------------------------
// Inclusive suffix sum over the lanes of a wave (lane l gets the sum over lanes >= l).
__device__ __forceinline__ unsigned wave_suffix_sum(unsigned x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const unsigned y = __shfl_down(x, o, 64);
    if (lane + o < 64) x += y;
  }
  return x;
}

// One wave finds the bin holding descending rank `rank` of an NB-bin histogram and the rank
// within that bin: lane l first sums bins [G l, G l + G), then the chosen group's G bins are
// searched one per lane (G = 64) or in turn (G = 4).
template <int NB>
__device__ void locate_digit(const unsigned* hist, unsigned rank, unsigned* digit, unsigned* rank_in) {
  constexpr int G = NB / 64;
  const int lane = threadIdx.x & 63;
  unsigned c = 0;
#pragma unroll
  for (int j = 0; j < G; ++j) c += hist[G * lane + j];
  const unsigned s = wave_suffix_sum(c);
  const unsigned ab = s - c;
  const unsigned long long own = __ballot(ab <= rank && rank < s);
  const int L = own ? __ffsll(own) - 1 : 0;
  unsigned r = rank - (unsigned)__builtin_amdgcn_readlane((int)ab, L);
  if constexpr (G == 64) {
    const unsigned h = hist[G * L + lane];
    const unsigned s2 = wave_suffix_sum(h);
    const unsigned ab2 = s2 - h;
    const unsigned long long own2 = __ballot(ab2 <= r && r < s2);
    const int j = own2 ? __ffsll(own2) - 1 : 0;
    *digit = G * L + j;
    *rank_in = r - (unsigned)__builtin_amdgcn_readlane((int)ab2, j);
  } else {
    int e = G - 1;
    for (; e > 0; --e) {
      const unsigned h = hist[G * L + e];
      if (r < h) break;
      r -= h;
    }
    *digit = G * L + e;
    *rank_in = r;
  }
}

constexpr int TOPK_LDS = 32768;  // scores of up to this many visible tokens are staged in LDS
constexpr int TOPK_BINS = 4096;  // digits of 12, 12 and 8 bits

__global__ void __launch_bounds__(1024) dsa_topk_kernel(DsaArgs A) {
  const AttnArgs& a = A.at;
  __shared__ unsigned hist[TOPK_BINS];
  __shared__ unsigned su[2];
  __shared__ unsigned wcnt[2][16];
  __shared__ uint32_t keys[TOPK_LDS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t = blockIdx.x % a.tq, b = blockIdx.x / a.tq;
  const int n_vis = min(a.tk, seq_off(a, b) + t + 1);
  const int K = A.topk;
  int32_t* lst = A.list + ((int64_t)b * a.tq + t) * K;
  if (n_vis <= K) {  // every visible token is kept
    for (int j = tid; j < n_vis; j += 1024) lst[j] = j;
    if (tid == 0) A.count[b * a.tq + t] = n_vis;
    return;
  }
  const float* sc = A.scores + ((int64_t)b * a.tq + t) * a.tk;
  const bool staged = n_vis <= TOPK_LDS;
  auto key_at = [&](int i) __attribute__((always_inline)) { return staged ? keys[i] : f32_order_key(sc[i]); };

  // Radix select of the key at descending rank K - 1: the histogram of the top 12 bits is
  // built while the keys are staged, then bits 19..8 and 7..0 among the keys that share the
  // digits chosen so far.
  for (int i = tid; i < TOPK_BINS; i += 1024) hist[i] = 0;
  __syncthreads();
  for (int i0 = tid; i0 < n_vis; i0 += 4 * 1024) {
    uint32_t kv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + 1024 * u;
      kv[u] = i < n_vis ? f32_order_key(sc[i]) : 0u;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + 1024 * u;
      if (i < n_vis) {
        if (staged) keys[i] = kv[u];
        atomicAdd(&hist[kv[u] >> 20], 1u);
      }
    }
  }
  __syncthreads();
  unsigned prefix = 0, pmask = 0, rank = (unsigned)(K - 1);
  auto choose = [&](auto nb_tag, int shift, unsigned dmask) __attribute__((always_inline)) {
    constexpr int NB = decltype(nb_tag)::value;
    if (wave == 0) {
      unsigned dg, r;
      locate_digit<NB>(hist, rank, &dg, &r);
      if (lane == 0) {
        su[0] = dg;
        su[1] = r;
      }
    }
    __syncthreads();
    prefix |= su[0] << shift;
    pmask |= dmask << shift;
    rank = su[1];
  };
  auto count_digit = [&](int shift, unsigned dmask, int nb) __attribute__((always_inline)) {
    for (int i = tid; i < nb; i += 1024) hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < n_vis; i += 1024) {
      const uint32_t key = key_at(i);
      if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & dmask], 1u);
    }
    __syncthreads();
  };
  choose(std::integral_constant<int, 4096>{}, 20, 0xfffu);
  count_digit(8, 0xfffu, 4096);
  choose(std::integral_constant<int, 4096>{}, 8, 0xfffu);
  count_digit(0, 0xffu, 256);
  choose(std::integral_constant<int, 256>{}, 0, 0xffu);

  // Ordered compaction: keys above the threshold, then the first rank + 1 keys equal to it in
  // token order.  Wave w owns a contiguous segment of tokens; one count pass and one barrier
  // give every wave its output offset, a second pass writes the indices in order.
  const uint32_t tau = prefix;
  const unsigned need_eq = rank + 1;
  const int seg = ((n_vis + 16 * 64 - 1) / (16 * 64)) * 64;
  const int w0 = wave * seg, w1 = min(w0 + seg, n_vis);
  unsigned gt_c = 0, eq_c = 0;
  for (int c0 = w0; c0 < w0 + seg; c0 += 64) {
    const int i = c0 + lane;
    const bool in = i < w1;
    const uint32_t key = in ? key_at(i) : 0u;
    gt_c += (unsigned)__popcll(__ballot(in && key > tau));
    eq_c += (unsigned)__popcll(__ballot(in && key == tau));
  }
  if (lane == 0) {
    wcnt[0][wave] = gt_c;
    wcnt[1][wave] = eq_c;
  }
  __syncthreads();
  unsigned eq_seen = 0, out = 0;
  for (int w = 0; w < wave; ++w) {
    const unsigned g = wcnt[0][w], e = wcnt[1][w];
    const unsigned left = need_eq > eq_seen ? need_eq - eq_seen : 0u;
    out += g + (e < left ? e : left);
    eq_seen += e;
  }
  const unsigned long long lt_mask = (1ull << lane) - 1ull;
  for (int c0 = w0; c0 < w0 + seg; c0 += 64) {
    const int i = c0 + lane;
    const bool in = i < w1;
    const uint32_t key = in ? key_at(i) : 0u;
    const bool gt = in && key > tau, eq = in && key == tau;
    const unsigned long long beq = __ballot(eq);
    const bool keep = gt || (eq && eq_seen + (unsigned)__popcll(beq & lt_mask) < need_eq);
    const unsigned long long bk = __ballot(keep);
    const unsigned pos = out + (unsigned)__popcll(bk & lt_mask);
    if (keep && pos < (unsigned)K) lst[pos] = i;
    eq_seen += (unsigned)__popcll(beq);
    out += (unsigned)__popcll(bk);
  }
  if (tid == 0) A.count[b * a.tq + t] = K;
}

// ---------------------------------------------------------------------------------------
__device__ __forceinline__ int v_off(int row, int chunk) { return row * D + ((chunk ^ ((row & 3) << 2)) << 3); }

__device__ __forceinline__ void wait_blocks(int blocks_after) {
  static_assert(NST - 1 <= 3, "vmcnt holds at most 63 outstanding loads: 3 blocks of 16");
  if (blocks_after >= 2)
    asm volatile("s_waitcnt vmcnt(32)" ::: "memory");
  else if (blocks_after == 1)
    asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
  else
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) dsa_split_kernel(DsaArgs A) {
  const AttnArgs& a = A.at;
  __shared__ __attribute__((aligned(1024))) bf16_t vlds[NST * VSTAGE];
  __shared__ int32_t ent[MAX_SPLIT];

  const int lane = threadIdx.x;
  const int l32 = lane & 31, hh = lane >> 5;
  int bid = blockIdx.x;
  const int s = __builtin_amdgcn_readfirstlane(bid % a.nsplit);
  bid /= a.nsplit;
  const int t = __builtin_amdgcn_readfirstlane(bid % a.tq);
  bid /= a.tq;
  const int kvh = __builtin_amdgcn_readfirstlane(bid % a.Hkv);
  const int b = __builtin_amdgcn_readfirstlane(bid / a.Hkv);
  const int cnt = __builtin_amdgcn_readfirstlane(A.count[b * a.tq + t]);
  const int ks0 = s * a.split, ks1 = min(ks0 + a.split, cnt);
  const int nblk = ks0 < ks1 ? (ks1 - ks0 + KB - 1) / KB : 0;
  const int32_t* lst = A.list + ((int64_t)b * a.tq + t) * A.topk;
  for (int i = lane; i < nblk * KB; i += 64) ent[i] = ks0 + i < ks1 ? lst[ks0 + i] : 0;

  // query rows: the g heads of KV head kvh at query token t (lane l32 = head in group)
  const bool row_ok = l32 < a.g;
  const int h = kvh * a.g + (row_ok ? l32 : 0);
  const bf16_t* qp = (const bf16_t*)a.q + b * a.q_sb + h * a.q_sh + (int64_t)t * a.q_st;
  bf16x8 qf[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    u32x4 z = {0u, 0u, 0u, 0u};
    qf[ks] = row_ok ? *(const bf16x8*)(qp + 16 * ks + 8 * hh) : as_bf16x8(z);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the list and q are in; only block loads are counted below
  __syncthreads();

  const uint32_t row_bytes = (uint32_t)a.kv_st * 2u;
  const bf16_t* kp = (const bf16_t*)a.k + b * a.kv_sb + kvh * a.kv_sh;
  const bf16_t* vp = (const bf16_t*)a.v + b * a.kv_sb + kvh * a.kv_sh;
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)kp, (short)0, (int)(a.tk * row_bytes), 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)vp, (short)0, (int)(a.tk * row_bytes), 0x00020000);
  const int vr = lane >> 4;
  const uint32_t v_sw = (uint32_t)(((lane & 15) ^ ((vr & 3) << 2)) << 4);

  bf16x8 kreg[NST][8];
  auto issue = [&](int n, auto stage_tag) __attribute__((always_inline)) {
    constexpr int ST = decltype(stage_tag)::value;
    const uint32_t krow = (uint32_t)ent[n * KB + l32] * row_bytes;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      kreg[ST][ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(krs, krow + hh * 16 + ks * 32, 0, 0));
#pragma unroll
    for (int i = 0; i < 8; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void_ptr)(vlds + ST * VSTAGE + i * 512), 16,
                                               (uint32_t)ent[n * KB + 4 * i + vr] * row_bytes + v_sw, 0, 0, 0);
  };
  if (nblk > 0) issue(0, std::integral_constant<int, 0>{});
  if (nblk > 1) issue(1, std::integral_constant<int, 1>{});

  f32x16 oacc[4];
#pragma unroll
  for (int tb = 0; tb < 4; ++tb)
#pragma unroll
    for (int v = 0; v < 16; ++v) oacc[tb][v] = 0.f;
  float m_run = SOC_NEG_INF, l_run = 0.f;
  const float c = a.scale_log2;
  int voff[4];
  {
    const int trj = lane & 15;
    const int tr_row = 4 * hh + (trj >> 2);
    const int tr_col = ((lane >> 4) & 1) * 16 + 4 * (trj & 3);
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      const int col = tb * 32 + tr_col;
      voff[tb] = v_off(tr_row, col >> 3) + (col & 7);
    }
  }

  auto step = [&](int n, auto stage_tag) __attribute__((always_inline)) {
    constexpr int ST = decltype(stage_tag)::value;
    if (n + NST - 1 < nblk) issue(n + NST - 1, std::integral_constant<int, (ST + NST - 1) % NST>{});
    wait_blocks(min(NST - 1, nblk - 1 - n));
    const bf16_t* vt = vlds + ST * VSTAGE;
    const int js = ks0 + n * KB;  // list position of the block's first entry

    f32x16 sacc;
#pragma unroll
    for (int v = 0; v < 16; ++v) sacc[v] = 0.f;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) sacc = mfma32x32x16(kreg[ST][ks], qf[ks], sacc);
    float mx = SOC_NEG_INF;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int j = js + 8 * (v >> 2) + 4 * hh + (v & 3);
      sacc[v] = j < ks1 ? sacc[v] : SOC_NEG_INF;  // the list holds visible tokens only
      mx = fmaxf(mx, sacc[v]);
    }
    mx = pair_max(mx);
    const float m_cand = mx * c;
    const bool upd = m_cand > m_run + RESCALE_SLACK;
    if (__builtin_amdgcn_ballot_w64(upd) != 0) {
      asm volatile("");  // keeps this a branch: the rescale is rare
      const float m_new = upd ? m_cand : m_run;
      const float alpha = upd ? fast_exp2(m_run - m_new) : 1.f;
      l_run *= alpha;
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[tb][v] *= alpha;
      m_run = m_new;
    }
    const float nm = (m_run == SOC_NEG_INF) ? 0.f : -m_run;
    bf16x8 pb[2];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float p = fast_exp2(fmaf(sacc[v], c, nm));
      l_run += p;
      pb[v >> 3][v & 7] = (bf16_t)p;
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(vt + 16 * kk * D + voff[tb]));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(vt + (16 * kk + 8) * D + voff[tb]));
        const s16x8 va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        oacc[tb] = mfma32x32x16(__builtin_bit_cast(bf16x8, va), pb[kk], oacc[tb]);
      }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this stage's LDS reads finish before its refill
  };

  for (int n = 0; n < nblk; n += NST) {
    step(n, std::integral_constant<int, 0>{});
    if (n + 1 < nblk) step(n + 1, std::integral_constant<int, 1>{});
    if (n + 2 < nblk) step(n + 2, std::integral_constant<int, 2>{});
  }

  // every split writes its partial, an empty one (max -inf, sum 0, O 0) included
  const float L = pair_sum(l_run);
  if (row_ok) {
    const int64_t rowid = ((int64_t)b * a.Hq + h) * a.tq + t;
    float* po = a.part + (rowid * a.nsplit + s) * D;
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        f32x4 out;
#pragma unroll
        for (int e = 0; e < 4; ++e) out[e] = oacc[tb][4 * g4 + e];
        *(f32x4*)(po + tb * 32 + 8 * g4 + 4 * hh) = out;
      }
    if (hh == 0) {
      float* pml = a.part + decode_o_floats(a) + (rowid * a.nsplit + s) * 2;
      pml[0] = m_run;
      pml[1] = L;
    }
  }
}

}  // namespace

hipError_t launch_dsa_decode(const DsaArgs& A, hipStream_t s) {
  const AttnArgs& a = A.at;
  const int64_t rows = (int64_t)a.B * a.tq;
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(dsa_indexer_kernel, dim3((unsigned)A.idx_waves), dim3(64), 0, s, A);
  hipLaunchKernelGGL(dsa_topk_kernel, dim3((unsigned)rows), dim3(1024), 0, s, A);
  hipLaunchKernelGGL(dsa_split_kernel, dim3((unsigned)(rows * a.Hkv * a.nsplit)), dim3(64), 0, s, A);
  // every split has a partial: the merge reads all nsplit of them (no offsets, tk = nsplit * split)
  AttnArgs m = a;
  m.cache_off = nullptr;
  m.tk = a.nsplit * a.split;
  return launch_decode_merge(m, true, s);
}

}  // namespace soc
