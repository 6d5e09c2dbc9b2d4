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
//   dsa_indexer_kernel  one 12-wave workgroup per CU, each scoring an equal share of all
//                       16-token blocks of all (sequence, query token) rows, in phases of up
//                       to 4 rows whose queries sit in LDS; the waves take blocks from a
//                       counter in LDS (4 at a time), keep 4 blocks of keys in flight each,
//                       and leave scores in LDS until the phase ends: scores^T = Ki Qi^T with
//                       v_mfma_f32_16x16x32_bf16 (16 tokens x 16 indexer heads per MFMA),
//                       ReLU and the head weights in fp32, the sum over heads in a fixed
//                       order (DPP within each 16-lane row); with each score, a bound on its
//                       fp32 rounding error (one more MFMA per 32 dims)
//   dsa_topk_kernel     one 1024-thread workgroup per (sequence, query token): radix select of
//                       the k-th largest fp32 score on order-preserving 32-bit keys (digits of
//                       12, 12 and 8 bits; the first histogram is built while the keys are
//                       staged in LDS); the tokens within twice the largest error bound of
//                       that threshold are scored again in fp64 (fp64 MFMA) and ranked there,
//                       so the kept set is exactly the top k of the fp64 scores (ties: lower
//                       index); then an index-ordered compaction into an ascending list, one
//                       contiguous token segment per wave
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
typedef double f64x4 __attribute__((ext_vector_type(4)));
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
// The smallest bf16 value >= x (x >= 0, finite).
__device__ __forceinline__ bf16_t bf16_round_up(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  if (u & 0xffffu) u += 0x10000u;
  return __builtin_bit_cast(bf16_t, (uint16_t)(u >> 16));
}
// Covers the fp32 rounding of the sum that forms u before it is rounded up (64 terms).
constexpr float kBoundSumSlack = 1.0f + 0x1p-16f;
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

// Waits go through the s_waitcnt builtin: the compiler treats it as touching all memory (no
// LDS access moves across it) and knows what it waited for, so it adds no drain of its own.
// gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8.
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N <= 63, "vmcnt counts at most 63 loads");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void lds_wait() { __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4)); }

typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;

constexpr int IDX_WAVES = 12;  // waves of the indexer workgroup (one workgroup per CU)
constexpr int IDX_NB = 5;      // key blocks per wave in registers: IDX_NB - 1 in flight while one is scored
constexpr int IDX_RMAX = 4;    // rows whose queries a phase stages in LDS
constexpr int IDX_GRAB = 4;    // blocks a wave takes from the phase's counter at a time
constexpr int IDX_PB = 600;    // blocks of a phase (their scores and bounds wait in LDS)

// One row segment of a phase: row b * tq + t, its blocks j0 .. j0 + len - 1, staged from
// block u0 of the phase.
struct IdxSeg {
  int b, t, nvis, j0, len, u0;
};
// x_s of four values for an index s (by value: selecting whole segments, or through
// references, turns into indexed private memory)
__device__ __forceinline__ int sel4(int s, int x0, int x1, int x2, int x3) {
  return s >= 2 ? (s == 3 ? x3 : x2) : (s == 1 ? x1 : x0);
}

// One workgroup per CU scores a contiguous share of the 16-token blocks of all rows (row
// r = b * tq + t has ceil(n_vis / 16) blocks; rows in order).  The share is cut into phases
// of at most IDX_RMAX row segments and IDX_PB blocks.  In a phase the waves take blocks one
// at a time from a counter in LDS, so the CU's waves finish together however unevenly the
// memory system serves them (a static split leaves the last waves streaming alone); every
// score and bound goes to LDS, and the phase's outputs are written once all its blocks are
// scored, so no store is in flight beside the key loads and the compiler counts those loads
// exactly.
__global__ void __launch_bounds__(64 * IDX_WAVES) __attribute__((amdgpu_waves_per_eu(3))) dsa_indexer_kernel(DsaArgs A) {
  const AttnArgs& a = A.at;
  // query tiles: head h's 16-byte piece c at piece c ^ (h & 15) of its 256-byte row (the
  // B-operand reads of 16 heads then hit 16 different bank groups)
  __shared__ __attribute__((aligned(16))) bf16_t qlds[IDX_RMAX][kDsaMaxIndexHeads * DI];
  __shared__ __attribute__((aligned(16))) bf16_t ulds[IDX_RMAX][DI];
  __shared__ float wlds[IDX_RMAX][kDsaMaxIndexHeads];
  __shared__ __attribute__((aligned(16))) float sst[2][IDX_PB * 16];  // scores, bounds
  __shared__ unsigned ucnt[2];                                         // block counters, by phase parity
  const int tid = threadIdx.x, lane = tid & 63;
  const int G = lane >> 4, i16 = lane & 15;
  const int rows = a.B * a.tq;
  auto row_nvis = [&](int r) __attribute__((always_inline)) -> int {  // visible tokens of row r (0 past the end)
    if (r >= rows) return 0;
    const int b = r / a.tq, t = r - b * a.tq;
    return min(a.tk, seq_off(a, b) + t + 1);
  };
  // Lane l holds n_vis of row rwin + l.  The first window also gives the total when there
  // are at most 64 rows, so the offsets are read once.
  int rwin = 0, nvw = row_nvis(lane);
  int total = wave_sum_i((nvw + 15) >> 4);
  for (int r0 = 64; r0 < rows; r0 += 64) total += wave_sum_i((row_nvis(r0 + lane) + 15) >> 4);
  total = __builtin_amdgcn_readfirstlane(total);
  const int W = gridDim.x, wid = blockIdx.x;
  const int lo = __builtin_amdgcn_readfirstlane((int)((int64_t)total * wid / W));
  const int hi = __builtin_amdgcn_readfirstlane((int)((int64_t)total * (wid + 1) / W));
  if (lo >= hi) return;  // (uniform over the workgroup)
  int row = 0, rstart = 0;  // the row holding block lo and the global index of its first block
  for (int r0 = 0, base = 0; r0 < rows; r0 += 64) {
    if (r0 != rwin) rwin = r0, nvw = row_nvis(r0 + lane);
    const int nb = (nvw + 15) >> 4;
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
  rwin = __builtin_amdgcn_readfirstlane(rwin);
  if (tid < 2) ucnt[tid] = 0;
  __syncthreads();

  const int nhb = A.Hi / 16;
  const uint32_t row_bytes = (uint32_t)A.ki_st * 2u;
  for (int g = lo, phase = 0; g < hi; ++phase) {
    // The phase's row segments (unused ones empty, with u0 past every block).
    auto next_seg = [&](int used) __attribute__((always_inline)) -> IdxSeg {
      IdxSeg sg{0, 0, 1, 0, 0, used};
      if (g < hi && used < IDX_PB) {  // uniform
        if (row >= rwin + 64) rwin = row, nvw = row_nvis(row + lane);
        const int nvis = __builtin_amdgcn_readlane(nvw, row - rwin);
        const int nb = (nvis + 15) >> 4, j0 = g - rstart;
        const int len = min(min(nb - j0, hi - g), IDX_PB - used);
        sg.b = __builtin_amdgcn_readfirstlane(row / a.tq);
        sg.t = __builtin_amdgcn_readfirstlane(row - sg.b * a.tq);
        sg.nvis = nvis, sg.j0 = __builtin_amdgcn_readfirstlane(j0), sg.len = __builtin_amdgcn_readfirstlane(len);
        g += len;
        if (j0 + len == nb) rstart += nb, ++row;
      }
      return sg;
    };
    static_assert(IDX_RMAX == 4, "four segments below");
    const IdxSeg S0 = next_seg(0);
    const IdxSeg S1 = next_seg(S0.u0 + S0.len);
    const IdxSeg S2 = next_seg(S1.u0 + S1.len);
    const IdxSeg S3 = next_seg(S2.u0 + S2.len);
    const int nunits = S3.u0 + S3.len;
    const int ns = 1 + (S1.len > 0) + (S2.len > 0) + (S3.len > 0);
    auto seg_of = [&](int u) __attribute__((always_inline)) -> int { return (u >= S1.u0) + (u >= S2.u0) + (u >= S3.u0); };

    // Block u of the phase, clamped to the last one (the loads past a wave's last block).
    auto load = [&](bf16x8* af, int u) __attribute__((always_inline)) {
      u = min(u, nunits - 1);
      const int s = seg_of(u);
      const int tok0 = 16 * (u + sel4(s, S0.j0 - S0.u0, S1.j0 - S1.u0, S2.j0 - S2.u0, S3.j0 - S3.u0));
      const bf16_t* kp = (const bf16_t*)A.ki + sel4(s, S0.b, S1.b, S2.b, S3.b) * A.ki_sb;
      const int nvis = sel4(s, S0.nvis, S1.nvis, S2.nvis, S3.nvis);
      const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)kp, (short)0, (int)(nvis * row_bytes), 0x00020000);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        af[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                                krs, (uint32_t)(tok0 + i16) * row_bytes + (uint32_t)(64 * ks + 16 * G), 0, 0));
    };
    auto score = [&](const bf16x8* af, int u) __attribute__((always_inline)) {
      const int s = seg_of(u);
      const bf16_t* qs = qlds[0] + s * (kDsaMaxIndexHeads * DI);
      float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int hb = 0; hb < 4; ++hb) {
        if (hb >= nhb) break;  // uniform
        const bf16_t* qrow = qs + (16 * hb + i16) * DI;  // head 16 hb + i16
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) acc = mfma16k32(af[ks], *(const bf16x8*)(qrow + 8 * ((4 * ks + G) ^ i16)), acc);
        const float wv = wlds[0][s * kDsaMaxIndexHeads + 16 * hb + i16];
#pragma unroll
        for (int v = 0; v < 4; ++v) part[v] = fmaf(wv, fmaxf(acc[v], 0.f), part[v]);
      }
      // lane (G, i16): tokens 4G + v, indexer head i16 of each tile; sum over the 16 heads
#pragma unroll
      for (int v = 0; v < 4; ++v) part[v] = row16_sum(part[v]);
      // E = u . |k| for tokens 4G + v (every column; lanes i16 == 0 keep it).  The empty asm
      // makes the LDS address opaque, so the reads stay here instead of holding u in registers;
      // the cast back to the LDS address space keeps them LDS reads (a generic pointer would
      // make them flat loads, which the compiler must also count against the key loads).
      const bf16_t* ua = ulds[0] + s * DI + 8 * G;
      asm volatile("" : "+v"(ua));
      const lds_bf16x8* ul = (const lds_bf16x8*)ua;
      f32x4 eacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) eacc = mfma16k32(as_bf16x8(as_u32x4(af[ks]) & 0x7fff7fffu), ul[4 * ks], eacc);
      if (i16 == 0) {
        *(f32x4*)&sst[0][u * 16 + 4 * G] = f32x4{part[0], part[1], part[2], part[3]};
        *(f32x4*)&sst[1][u * 16 + 4 * G] = f32x4{eacc[0], eacc[1], eacc[2], eacc[3]};
      }
    };
    // A wave takes IDX_GRAB consecutive blocks per counter access (one access per block cost
    // 4 us over the workgroup's waves); the next batch is requested when the current one
    // starts and read when it is needed, so the access's latency stays out of the way.
    unsigned* cnt = &ucnt[phase & 1];
    unsigned nxt = 0;  // (lane 0) first block of the wave's next batch
    int cur = 0, left = 0;
    auto fetch = [&]() __attribute__((always_inline)) {
      if (lane == 0) nxt = __hip_atomic_fetch_add(cnt, (unsigned)IDX_GRAB, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    };
    auto grab = [&]() __attribute__((always_inline)) -> int {  // the wave's next block of the phase
      if (left == 0) {  // uniform
        cur = __builtin_amdgcn_readfirstlane((int)nxt), left = IDX_GRAB;
        fetch();
      }
      --left;
      return cur++;
    };

    // The phase's queries go straight into LDS (1 KB = 4 heads per wave instruction), with the
    // head weights into registers.  Whatever is still counted first retires (after the first
    // phase: the previous phase's stores and its last, unused key loads).
    vm_wait<0>();
    // Each block id is taken one step before its load is issued.  The first ids are taken
    // before the query copies start: the compiler cannot tell the counter from their
    // destination and would make every later counter access wait for them.
    fetch();
    int uid[IDX_NB];
#pragma unroll
    for (int k = 0; k < IDX_NB - 1; ++k) uid[k] = grab();
    int pend = grab();
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    for (int n = wave; n < ns * (A.Hi / 4); n += IDX_WAVES) {  // 4 heads of one row per instruction
      const int s = n / (A.Hi / 4), h = 4 * (n - s * (A.Hi / 4)) + (lane >> 4);
      const bf16_t* qb = (const bf16_t*)A.qi + sel4(s, S0.b, S1.b, S2.b, S3.b) * A.qi_sb + sel4(s, S0.t, S1.t, S2.t, S3.t) * A.qi_st;
      const __amdgpu_buffer_rsrc_t qrs =
          __builtin_amdgcn_make_buffer_rsrc((void*)qb, (short)0, (int)(A.Hi * A.qi_sh * 2), 0x00020000);
      const uint32_t voff = (uint32_t)(h * A.qi_sh + 8 * ((lane & 15) ^ (h & 15))) * 2u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(qrs, (lds_void_ptr)(qlds[0] + s * (kDsaMaxIndexHeads * DI) + (h - (lane >> 4)) * DI), 16, voff, 0, 0, 0);
    }
    float wv = 0.f;
    if (tid < ns * A.Hi) {
      const int s = tid / A.Hi, j = tid - s * A.Hi;
      wv = A.wi[((int64_t)sel4(s, S0.b, S1.b, S2.b, S3.b) * A.Hi + j) * a.tq + sel4(s, S0.t, S1.t, S2.t, S3.t)];
    }
    // The first key blocks go out once every wave's query copies are in, so the copies do not
    // queue behind them, and they are in flight while the error-bound weights are formed.
    vm_wait<0>();
    if (tid < ns * A.Hi) wlds[0][(tid / A.Hi) * kDsaMaxIndexHeads + tid % A.Hi] = wv;
    __syncthreads();
    bf16x8 fbuf[IDX_NB][4];
#pragma unroll
    for (int k = 0; k < IDX_NB - 1; ++k) load(fbuf[k], uid[k]);
    // u[d] = sum_j |w_j| |qi_j[d]| (fp32, rounded up to bf16 with a slack covering the sum's
    // rounding in any order) is read as a B operand broadcast to all 16 columns, so the MFMA
    // of |k| against it gives E = u . |k|, which bounds the fp32 rounding of the score.  Item
    // (s, quarter of the heads, pair of dims) sums its 16 heads; the quarters are added in
    // order after a barrier (the score stage is free until the blocks are scored).
    {
      float* part = sst[0];  // [s][quarter][d]
      const int hq = A.Hi / 4;
      for (int i = tid; i < ns * 4 * (DI / 2); i += 64 * IDX_WAVES) {
        const int s = i / (4 * (DI / 2)), r = i % (4 * (DI / 2)), q4 = r / (DI / 2), d = 2 * (r % (DI / 2));
        float p0 = 0.f, p1 = 0.f;
#pragma unroll 8
        for (int j = q4 * hq; j < (q4 + 1) * hq; ++j) {
          const float w = fabsf(wlds[s][j]);
          const uint32_t qq = *(const uint32_t*)&qlds[s][j * DI + 8 * ((d >> 3) ^ (j & 15)) + (d & 7)];
          p0 = fmaf(w, fabsf(__builtin_bit_cast(float, qq << 16)), p0);
          p1 = fmaf(w, fabsf(__builtin_bit_cast(float, qq & 0xffff0000u)), p1);
        }
        part[(s * 4 + q4) * DI + d] = p0;
        part[(s * 4 + q4) * DI + d + 1] = p1;
      }
      __syncthreads();
      for (int i = tid; i < ns * DI; i += 64 * IDX_WAVES) {
        const int s = i / DI, d = i % DI;
        const float p = ((part[(s * 4) * DI + d] + part[(s * 4 + 1) * DI + d]) + part[(s * 4 + 2) * DI + d]) + part[(s * 4 + 3) * DI + d];
        ulds[s][d] = bf16_round_up(p * kBoundSumSlack);
      }
    }
    __syncthreads();

    // IDX_NB rotating register buffers: a block is scored while the wave's next IDX_NB - 1
    // are in flight.  A wave's ids rise in the order of its buffers, so once a buffer holds an
    // id past the phase, so do all after it.  Every step issues its load (past the phase it
    // reloads the phase's last block) and only the scoring is skipped, and the loop is left
    // only at the top of a round: the same loads are in flight on every path, so the compiler
    // counts them exactly (an exit in mid-round would be merged into the loop's latch).
    for (;;) {
      if (uid[0] >= nunits) break;  // uniform
#pragma unroll
      for (int u = 0; u < IDX_NB; ++u) {
        const int nx = (u + IDX_NB - 1) % IDX_NB;
        const int cur = uid[u];
        uid[nx] = pend;
        pend = grab();
        load(fbuf[nx], uid[nx]);
        if (cur < nunits) score(fbuf[u], cur);  // uniform
      }
    }
    __syncthreads();  // every block of the phase is scored
    // The phase's scores and bounds go out, two tokens per thread and round, through buffers
    // whose range ends at the row's last visible token.
    auto flush = [&](const IdxSeg sg) __attribute__((always_inline)) {
      const int64_t r = (int64_t)sg.b * a.tq + sg.t;
      const uint32_t nbytes = (uint32_t)sg.nvis * 4u;
      const __amdgpu_buffer_rsrc_t ors = __builtin_amdgcn_make_buffer_rsrc((void*)(A.scores + r * a.tk), (short)0, (int)nbytes, 0x00020000);
      const __amdgpu_buffer_rsrc_t ers = __builtin_amdgcn_make_buffer_rsrc((void*)(A.ebound + r * a.tk), (short)0, (int)nbytes, 0x00020000);
      for (int i = 2 * tid; i < 16 * sg.len; i += 2 * 64 * IDX_WAVES) {
        const uint32_t at = (uint32_t)(16 * sg.j0 + i) * 4u;
        const int e = 16 * sg.u0 + i;
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, sst[0][e]), ors, at, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, sst[0][e + 1]), ors, at + 4u, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, sst[1][e]), ers, at, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, sst[1][e + 1]), ers, at + 4u, 0, 0);
      }
    };
    flush(S0), flush(S1), flush(S2), flush(S3);
    if (tid == 0) ucnt[phase & 1] = 0;  // used again two phases on, after several barriers
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

constexpr int TOPK_LDS = 32768;  // scores of up to this many visible tokens are staged in LDS
constexpr int TOPK_BINS = 4096;  // digits of 12, 12 and 8 bits (32-bit keys); 12 x 4, 8 x 2 (64-bit)

// |fp32 score - exact score| <= kScoreErrBound * E for every token (E = u . |k| from the
// indexer).  Each head's 128-term dot product is accumulated in fp32 (relative error at most
// 128 * 2^-24 of sum |q_d k_d|), and the weighted ReLU terms are summed over at most 64 heads
// with at most 8 roundings (2^-21 of sum |w_j relu(dot_j)|, itself <= E); together below
// 2^-16 * E.  The bound used is 4x that, which also covers E's own fp32 rounding and an MFMA
// that accumulated with twice the rounding error of round-to-nearest.
constexpr double kScoreErrBound = 0x1p-14;

__device__ __forceinline__ uint64_t f64_key(double x) { return f64_order_key(x); }

// Block-wide sums and maxima over the 16 waves of the top-k workgroup (through `red`, 16 slots).
__device__ __forceinline__ unsigned block_sum_u(unsigned x, unsigned* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  __syncthreads();
  if (lane == 0) red[wave] = x;
  __syncthreads();
  unsigned t = 0;
#pragma unroll
  for (int w = 0; w < 16; ++w) t += red[w];
  return t;
}
__device__ __forceinline__ float block_max_f(float x, unsigned* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  __syncthreads();
  if (lane == 0) red[wave] = __builtin_bit_cast(unsigned, x);
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int w = 0; w < 16; ++w) t = fmaxf(t, __builtin_bit_cast(float, red[w]));
  return t;
}

constexpr int BAND_LDS = 1024;  // band sizes decided in LDS; larger bands by fp64 radix select

__global__ void __launch_bounds__(1024) dsa_topk_kernel(DsaArgs A) {
  const AttnArgs& a = A.at;
  __shared__ __attribute__((aligned(16))) unsigned hist[TOPK_BINS];
  __shared__ unsigned su[2];
  __shared__ unsigned wcnt[2][16];
  __shared__ unsigned red[16];
  __shared__ unsigned nband_s;
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
  const int64_t row_off = ((int64_t)b * a.tq + t) * a.tk;
  const float* sc = A.scores + row_off;
  const float* eb = A.ebound + row_off;
  double* s64 = A.s64 + row_off;
  int32_t* band = A.band + row_off;
  const bool staged = n_vis <= TOPK_LDS;
  auto key_at = [&](int i) __attribute__((always_inline)) { return staged ? keys[i] : f32_order_key(sc[i]); };
  auto f32_of_key = [](uint32_t k) __attribute__((always_inline)) {
    return __builtin_bit_cast(float, (k >> 31) ? (k & 0x7fffffffu) : ~k);
  };

  // 1. The fp32 threshold tau32 (the key at descending rank K - 1) by radix select: the
  // histogram of the top 12 bits is built while the keys are staged (and the largest error
  // bound taken), then bits 19..8 and 7..0 among the keys that share the digits chosen so far.
  for (int i = tid; i < TOPK_BINS; i += 1024) hist[i] = 0;
  if (tid == 0) nband_s = 0;
  __syncthreads();
  float emax = 0.f;
  for (int i0 = tid; i0 < n_vis; i0 += 16 * 1024) {
    // 16 scores and 16 bounds per thread in flight (one round for 16384 tokens)
    float sv[16], ev[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int i = i0 + 1024 * u;
      sv[u] = i < n_vis ? sc[i] : 0.f;
      ev[u] = i < n_vis ? eb[i] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int i = i0 + 1024 * u;
      emax = fmaxf(emax, ev[u]);
      if (i < n_vis) {
        const uint32_t kv = f32_order_key(sv[u]);
        if (staged) keys[i] = kv;
        atomicAdd(&hist[kv >> 20], 1u);
      }
    }
  }
  __syncthreads();
  unsigned rank = (unsigned)(K - 1);
  // The bin holding descending rank `rank` of an NB-bin histogram, and the rank inside it:
  // thread t owns bins 4t .. 4t+3 (one conflict-free 16-byte read), each wave sums its 256
  // bins, the wave holding the rank is found from the 16 wave totals, then its lane, then the
  // bin (higher bins = higher keys = lower descending ranks).
  __shared__ unsigned wtot[16];
  auto pick = [&](auto nb_tag) __attribute__((always_inline)) -> unsigned {  // digit; updates rank
    constexpr int NB = decltype(nb_tag)::value;
    u32x4 h4 = {0u, 0u, 0u, 0u};
    if (4 * tid < NB) h4 = *(const u32x4*)(hist + 4 * tid);
    const unsigned c = h4[0] + h4[1] + h4[2] + h4[3];
    const unsigned sfx = wave_suffix_sum(c);  // this lane's and the higher lanes' bins
    if (lane == 0) wtot[wave] = sfx;
    __syncthreads();
    unsigned above = 0;  // count in the waves above this one
    for (int w = 15; w > wave; --w) above += wtot[w];
    const unsigned wt = wtot[wave];
    if (above <= rank && rank < above + wt) {  // (wave-uniform) the rank lies in this wave
      const unsigned r = rank - above;
      const unsigned ab = sfx - c;
      if (ab <= r && r < sfx) {  // exactly one lane
        unsigned rr = r - ab;
        int e = 3;
        for (; e > 0; --e) {
          if (rr < h4[e]) break;
          rr -= h4[e];
        }
        su[0] = 4 * tid + e;
        su[1] = rr;
      }
    }
    __syncthreads();
    const unsigned dg = su[0];
    rank = su[1];
    return dg;
  };
  uint32_t prefix = 0, pmask = 0;
  auto count32 = [&](int shift, unsigned dmask, int nb) __attribute__((always_inline)) {
    for (int i = tid; i < nb; i += 1024) hist[i] = 0;
    __syncthreads();
    for (int i0 = tid; i0 < n_vis; i0 += 8 * 1024) {  // 8 key reads in flight
      uint32_t kk[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) kk[u] = i0 + 1024 * u < n_vis ? key_at(i0 + 1024 * u) : ~prefix;
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (i0 + 1024 * u < n_vis && (kk[u] & pmask) == prefix) atomicAdd(&hist[(kk[u] >> shift) & dmask], 1u);
    }
    __syncthreads();
  };
  prefix |= pick(std::integral_constant<int, 4096>{}) << 20;
  pmask |= 0xfffu << 20;
  count32(8, 0xfffu, 4096);
  prefix |= pick(std::integral_constant<int, 4096>{}) << 8;
  pmask |= 0xfffu << 8;
  count32(0, 0xffu, 256);
  prefix |= pick(std::integral_constant<int, 256>{});
  const double tau32 = (double)f32_of_key(prefix);

  // 2. The exact decision.  Every token's fp32 score is within D = max_i kScoreErrBound * E_i
  // of its exact score, so the exact K-th largest score lies within D of tau32: a token with
  // s32 > tau32 + 2D is kept for certain, one with s32 < tau32 - 2D dropped for certain, and
  // the tokens in between (the band, never empty) are scored again in fp64 and decided by
  // that score.  The kept set is then the top K of the fp64 scores, equal scores to the lower
  // token index.
  const double bw = 2.0 * kScoreErrBound * (double)block_max_f(emax, red);
  // The two comparisons as key comparisons: s32 > x iff s32 > (the largest float <= x), and
  // s32 < y iff s32 < (the smallest float >= y); consecutive keys are consecutive floats.
  uint32_t key_hi, key_lo;
  {
    const double x = tau32 + bw, y = tau32 - bw;
    key_hi = f32_order_key((float)x);
    if ((double)f32_of_key(key_hi) > x) key_hi -= 1u;
    key_lo = f32_order_key((float)y);
    if ((double)f32_of_key(key_lo) < y) key_lo += 1u;
  }
  auto certain = [&](uint32_t key) __attribute__((always_inline)) -> int {  // 2 kept, 0 dropped, 1 band
    return key > key_hi ? 2 : key < key_lo ? 0 : 1;
  };
  // Wave w owns the contiguous token segment [w * seg, (w + 1) * seg): the classification
  // counts each segment's certain keeps, the decision adds each segment's band keeps, and the
  // compaction writes every segment's kept tokens at the offset those counts give.
  const int seg = ((n_vis + 16 * 64 - 1) / (16 * 64)) * 64;
  const int w0 = wave * seg, w1 = min(w0 + seg, n_vis);
  __shared__ unsigned wkeep[16];
  // the band in small rows lives in LDS, in the histogram's space (free from here on)
  uint64_t* bkey = reinterpret_cast<uint64_t*>(hist);
  int32_t* bidx = reinterpret_cast<int32_t*>(hist + 2 * BAND_LDS);
  static_assert(3 * BAND_LDS <= TOPK_BINS, "band arrays fit in the histogram's LDS");
  unsigned gt_w = 0;  // this wave's certain keeps
  for (int c0 = w0; c0 < w0 + seg; c0 += 4 * 64) {  // (seg is a multiple of 64) 4 key reads in flight
    int cls[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = c0 + 64 * u + lane;
      cls[u] = c0 + 64 * u < w0 + seg && i < w1 ? certain(key_at(i)) : 0;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = c0 + 64 * u + lane;
      const int c = cls[u];
      gt_w += (unsigned)__popcll(__ballot(c == 2));
      const unsigned long long bb = __ballot(c == 1);
      if (bb) {  // (wave-uniform) band tokens in this chunk: rare
        unsigned base = 0;
        if (lane == 0) base = atomicAdd(&nband_s, (unsigned)__popcll(bb));
        base = __builtin_amdgcn_readfirstlane(base);
        if (c == 1) {
          const unsigned e = base + (unsigned)__popcll(bb & ((1ull << lane) - 1ull));
          band[e] = i;
          if (e < BAND_LDS) bidx[e] = i;
        }
      }
    }
  }
  if (lane == 0) {
    wcnt[0][wave] = gt_w;
    wkeep[wave] = 0u;
  }
  __syncthreads();  // (also publishes nband_s and the band lists)
  unsigned n_in = 0;
#pragma unroll
  for (int w = 0; w < 16; ++w) n_in += wcnt[0][w];
  const int n_band = (int)nband_s;
  const bool in_lds = n_band <= BAND_LDS;
  const int R = K - (int)n_in;  // band tokens to keep (>= 1)

  // fp64 scores of the band on the fp64 MFMA (v_mfma_f64_16x16x4f64: A[i][k] in lane i + 16k,
  // B[k][j] in lane j + 16k, D[i][j] in lane j + 16 (i % 4), element i / 4).  A wave takes 16
  // band tokens (rows i) and the indexer heads 16 at a time (columns j); lane (slot, G) feeds
  // dims 32G + m of its token's key and of its head's query at step m = 0..31, so the 32 steps
  // sum all 128 dims.  ReLU and the head weight apply to each full dot product, the heads of a
  // tile are summed across their 16 lanes and the tiles in order: a fixed order throughout, so
  // equal key rows get equal scores.
  {
    const int Hi = A.Hi;
    const int slot = lane & 15, G = lane >> 4;
    const bf16_t* kbase = (const bf16_t*)A.ki + b * A.ki_sb;
    const int ngroups = (n_band + 15) / 16;
    const int ntiles = (Hi + 15) / 16;  // head tiles of 16 (at most 16)
    const int gpr = 16 / ntiles;        // groups per round: one (group, head tile) item per wave
    // the items' partial sums over their 16 heads: 16 tokens each, in the histogram's last
    // quarter (free: the band keys and indices use the first three)
    double* part = reinterpret_cast<double*>(hist + 3 * BAND_LDS);
    static_assert(16 * 16 * sizeof(double) <= BAND_LDS * sizeof(unsigned), "partials fit");
    for (int g0 = 0; g0 < ngroups; g0 += gpr) {
      const int grp = g0 + wave / ntiles, tile = wave % ntiles;
      if (wave < gpr * ntiles && grp < ngroups) {
        const int e = min(grp * 16 + slot, n_band - 1);  // slots past the band repeat its last token
        const int tok = in_lds ? bidx[e] : band[e];
        const u32x4* kp = (const u32x4*)(kbase + (int64_t)tok * A.ki_st + 32 * G);
        const int head = tile * 16 + slot;
        const bool hok = head < Hi;
        const u32x4* qp = (const u32x4*)((const bf16_t*)A.qi + b * A.qi_sb + (hok ? head : 0) * A.qi_sh + t * A.qi_st + 32 * G);
        u32x4 kc[4], qc[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          kc[c] = kp[c];
          qc[c] = hok ? qp[c] : u32x4{0u, 0u, 0u, 0u};
        }
        const double wj = hok ? (double)A.wi[((int64_t)b * Hi + head) * a.tq + t] : 0.0;
        f64x4 acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
        for (int c = 0; c < 4; ++c) {  // 8 steps per 16 bytes of key and query
#pragma unroll
          for (int m = 0; m < 8; ++m) {
            const uint32_t kw = kc[c][m >> 1], qw2 = qc[c][m >> 1];
            const double av = (double)((m & 1) ? bf16_hi(kw) : bf16_lo(kw));
            const double bv = (double)((m & 1) ? bf16_hi(qw2) : bf16_lo(qw2));
            acc = __builtin_amdgcn_mfma_f64_16x16x4f64(av, bv, acc, 0, 0, 0);
          }
          __builtin_amdgcn_sched_barrier(0);  // converts one chunk at a time (registers)
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          double term = wj * (acc[v] > 0.0 ? acc[v] : 0.0);
#pragma unroll
          for (int o = 1; o < 16; o <<= 1) term += __shfl_xor(term, o, 64);  // the tile's 16 heads
          if (slot == 0) part[wave * 16 + 4 * v + G] = term;  // token 4v + G of the group
        }
      }
      __syncthreads();
      // each group's score: its tiles' partials added in head order (a fixed order: equal key
      // rows get equal scores)
      if (tid < gpr * 16) {
        const int gi = tid >> 4, sl = tid & 15;
        const int ei = (g0 + gi) * 16 + sl;
        if (g0 + gi < ngroups && ei < n_band) {
          double sc64 = 0.0;
          for (int ti = 0; ti < ntiles; ++ti) sc64 += part[(gi * ntiles + ti) * 16 + sl];
          if (in_lds)
            bkey[ei] = f64_key(sc64);
          else
            s64[band[ei]] = sc64;
        }
      }
      __syncthreads();
    }
  }

  uint64_t tau64 = 0;
  unsigned need_eq = 0;
  if (in_lds) {
    // Each band token's rank in (fp64 score descending, token index ascending); the first R
    // are kept.  The decision is written over the token's fp32 key (+inf kept, -inf dropped),
    // so the compaction below classifies every token from its key alone.
    constexpr uint32_t KEY_POS_INF = 0xff800000u, KEY_NEG_INF = 0x007fffffu;  // f32_order_key(+-inf)
    uint32_t dec = 0;
    int itok = -1;
    if (tid < n_band) {
      const uint64_t ke = bkey[tid];
      itok = bidx[tid];
      int rk = 0;
      for (int f = 0; f < n_band; ++f) {
        const uint64_t kf = bkey[f];
        rk += (kf > ke) | ((kf == ke) & (bidx[f] < itok));
      }
      dec = rk < R ? KEY_POS_INF : KEY_NEG_INF;
    }
    __syncthreads();  // every rank is taken before any key changes
    if (itok >= 0) {
      if (staged)
        keys[itok] = dec;
      else
        const_cast<float*>(sc)[itok] = f32_of_key(dec);
      if (dec == KEY_POS_INF) atomicAdd(&wkeep[itok / seg], 1u);
    }
  } else {
    // fp64 radix select over the band: descending rank R - 1 (digits of 12 x 4, 8 x 2)
    rank = (unsigned)max(0, min(R - 1, n_band - 1));
    uint64_t p64 = 0, m64 = 0;
    auto count64 = [&](int shift, unsigned dmask, int nb) __attribute__((always_inline)) {
      for (int i = tid; i < nb; i += 1024) hist[i] = 0;
      __syncthreads();
      for (int e = tid; e < n_band; e += 1024) {
        const uint64_t key = f64_key(s64[band[e]]);
        if ((key & m64) == p64) atomicAdd(&hist[(unsigned)(key >> shift) & dmask], 1u);
      }
      __syncthreads();
    };
#pragma unroll 1
    for (int shift = 52; shift >= 16; shift -= 12) {
      count64(shift, 0xfffu, 4096);
      p64 |= (uint64_t)pick(std::integral_constant<int, 4096>{}) << shift;
      m64 |= (uint64_t)0xfff << shift;
    }
#pragma unroll 1
    for (int shift = 8; shift >= 0; shift -= 8) {
      count64(shift, 0xffu, 256);
      p64 |= (uint64_t)pick(std::integral_constant<int, 256>{}) << shift;
      m64 |= (uint64_t)0xff << shift;
    }
    tau64 = p64;
    need_eq = rank + 1;
  }
  __syncthreads();

  // 3. Ordered compaction: every token kept for certain or by its fp64 score, then (large
  // bands) the first need_eq band tokens equal to tau64 in token order.  Wave w owns a
  // contiguous segment of tokens; one count pass and one barrier give every wave its output
  // offset, a second pass writes the indices in order.
  auto cls_at = [&](int i) __attribute__((always_inline)) -> int {  // 2 keep, 1 tie at tau64, 0 drop
    const int c = certain(key_at(i));
    if (c != 1 || in_lds) return c;  // (small bands: already decided in the keys)
    const uint64_t k64 = f64_key(s64[i]);
    return k64 > tau64 ? 2 : k64 == tau64 ? 1 : 0;
  };
  const unsigned long long lt_mask = (1ull << lane) - 1ull;
  if (in_lds) {
    // every key is now decided (band keys were set to +-inf): each segment's keeps are its
    // certain keeps plus its band keeps, so one pass writes them at their offsets
    unsigned out = 0;
    for (int w = 0; w < wave; ++w) out += wcnt[0][w] + wkeep[w];
    for (int c0 = w0; c0 < w0 + seg; c0 += 64) {
      const int i = c0 + lane;
      const bool keep = i < w1 && key_at(i) > key_hi;
      const unsigned long long bk = __ballot(keep);
      const unsigned pos = out + (unsigned)__popcll(bk & lt_mask);
      if (keep && pos < (unsigned)K) lst[pos] = i;
      out += (unsigned)__popcll(bk);
    }
    if (tid == 0) A.count[b * a.tq + t] = K;
    return;
  }
  unsigned gt_c = 0, eq_c = 0;
  for (int c0 = w0; c0 < w0 + seg; c0 += 64) {
    const int i = c0 + lane;
    const int c = i < w1 ? cls_at(i) : 0;
    gt_c += (unsigned)__popcll(__ballot(c == 2));
    eq_c += (unsigned)__popcll(__ballot(c == 1));
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
  for (int c0 = w0; c0 < w0 + seg; c0 += 64) {
    const int i = c0 + lane;
    const int c = i < w1 ? cls_at(i) : 0;
    const unsigned long long beq = __ballot(c == 1);
    const bool keep = c == 2 || (c == 1 && eq_seen + (unsigned)__popcll(beq & lt_mask) < need_eq);
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

static_assert(16 * (NST - 1) <= 63, "vmcnt holds at most 63 outstanding loads");

__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) dsa_split_kernel(DsaArgs A) {
  const AttnArgs& a = A.at;
  // one LDS variable per V stage, so that the compiler can tell which stage a pending DMA
  // writes (with one array it drains every load before each block's V reads)
  static_assert(NST == 3, "one LDS variable per stage");
  __shared__ __attribute__((aligned(1024))) bf16_t vst0[VSTAGE];
  __shared__ __attribute__((aligned(1024))) bf16_t vst1[VSTAGE];
  __shared__ __attribute__((aligned(1024))) bf16_t vst2[VSTAGE];
  auto vstage = [&](auto stage_tag) __attribute__((always_inline)) -> bf16_t* {
    constexpr int ST = decltype(stage_tag)::value;
    return ST == 0 ? vst0 : ST == 1 ? vst1 : vst2;
  };
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
  vm_wait<0>();  // the list and q are in; only block loads are counted below
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
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void_ptr)(vstage(stage_tag) + i * 512), 16,
                                               (uint32_t)ent[n * KB + 4 * i + vr] * row_bytes + v_sw, 0, 0,
                                               kLoadReadOnce);
  };
  // Every step issues one block (past the last block it issues the last block again, into a
  // stage already consumed), so exactly NST - 1 blocks are younger than the one a step
  // consumes and one constant wait covers every step.
  if (nblk > 0) {
    issue(0, std::integral_constant<int, 0>{});
    issue(min(1, nblk - 1), std::integral_constant<int, 1>{});
  }

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
    issue(min(n + NST - 1, nblk - 1), std::integral_constant<int, (ST + NST - 1) % NST>{});
    // Block n's K registers and V stage have landed.  Loads into registers and LDS-DMA loads
    // each retire in issue order but not in order with each other, so the wait allows only
    // the 8 * (NST - 1) loads of one kind that were issued after block n's.
    vm_wait<8 * (NST - 1)>();
    // The wait orders memory accesses only: an MFMA reading the K registers could still be
    // scheduled above it, guarded just by the compiler's own count, which takes all loads as
    // one ordered stream.  Passing the registers through an empty asm after the wait ties
    // their use to it.
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) asm volatile("" : "+v"(kreg[ST][ks]));
    const bf16_t* vt = vstage(stage_tag);
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
    lds_wait();  // this stage's LDS reads finish before its refill
  };

  int n = 0;
  for (; n + NST <= nblk; n += NST) {
    step(n, std::integral_constant<int, 0>{});
    step(n + 1, std::integral_constant<int, 1>{});
    step(n + 2, std::integral_constant<int, 2>{});
  }
  if (n < nblk) step(n, std::integral_constant<int, 0>{});
  if (n + 1 < nblk) step(n + 1, std::integral_constant<int, 1>{});
  vm_wait<0>();  // the repeated last blocks land before the LDS is released

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
  hipLaunchKernelGGL(dsa_indexer_kernel, dim3((unsigned)A.idx_waves), dim3(64 * IDX_WAVES), 0, s, A);
  hipLaunchKernelGGL(dsa_topk_kernel, dim3((unsigned)rows), dim3(1024), 0, s, A);
  hipLaunchKernelGGL(dsa_split_kernel, dim3((unsigned)(rows * a.Hkv * a.nsplit)), dim3(64), 0, s, A);
  // every split has a partial: the merge reads all nsplit of them (no offsets, tk = nsplit * split)
  AttnArgs m = a;
  m.cache_off = nullptr;
  m.tk = a.nsplit * a.split;
  return launch_decode_merge(m, true, s);
}

}  // namespace soc
