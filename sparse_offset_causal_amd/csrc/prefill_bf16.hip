// bf16 offset-causal attention prefill for gfx950, head_dim 128.
//
// Computes, per query row r of a tq-row block at cache offset off_b, the softmax over the
// keys j <= off_b + r (and j > off_b + r - W with a window; and only listed key blocks in
// block-sparse mode) of scale * q.k, weighted sum of v, with an optional per-head sink
// logit in the normaliser (sotaaz.com/post/attention-in-code, listing attend/causal and
// sections 1 and 3; patty.io RBS-Attention review, section on block-sparse execution).
//
// Work decomposition
//   workgroup = 4 waves of 32 query rows each.  With a window and GQA they are gs = 4 (or 2)
//   query heads of one KV group over the same rows (32 rows x 4 heads, or 64 rows x 2
//   heads): every wave then needs the same key tiles, so none idles through a tile at a
//   window edge.  Otherwise (no window, no GQA, or block-sparse mode with its per-head lists
//   of 128-row blocks) they are 128 rows of one head, wave w owning rows 32w..32w+31.
//   The workgroup walks 64-key tiles of the KV interval its rows can see; tiles outside
//   the interval (beyond the last row's position, before the first row's window, or not
//   in the block list) are never loaded.
//   Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16, so each
//   lane owns one query row (lane % 32) and 16 keys per 32-key block: the row max and sum
//   need one exchange between the two wave halves, and the output O^T = V^T P^T again
//   leaves one row per lane, so the softmax rescale is a per-lane scalar.
//   Masks are computed from indices only on tiles that cross a row's causal limit, and
//   separately only on tiles that cross a row's window edge.  The online softmax runs in
//   the log2 domain in fp32 with the scale folded into the exponent's FMA; the running max
//   is only raised (and O, l rescaled) when a row's max grows by more than 2^8, so most
//   tiles skip the rescale; P is rounded to bf16 for the second MFMA; O accumulates in fp32
//   and is rounded to bf16 once at the end.
//
// Memory path
//   K and V tiles go HBM -> LDS directly (global_load_lds_dwordx4, 1 KB per wave
//   instruction, no register staging) into a double buffer: the loads of tile n+1 are in
//   flight while tile n is consumed, with one barrier per tile.  Both tiles are row-major
//   with a 16-byte-chunk XOR swizzle applied on the load side.  K is read as the MFMA A
//   operand with ds_read_b128 (chunk' = chunk ^ (row & 15): 16 consecutive keys hit 16
//   distinct bank groups), four MFMA steps ahead of use.  V is read already transposed with
//   ds_read_b64_tr_b16 (each 16-lane group reads a 4-key x 16-column block; chunk' = chunk ^
//   4*(row & 3) makes the two groups of a half-wave cover all 64 banks once).  The loads are buffer loads whose
//   range ends at the last row any query of the workgroup may see: later rows read as zero
//   and are masked.  All LDS and DMA addressing is per-lane offsets fixed at kernel start
//   plus immediates or one scalar per tile.
//
// Grid order: workgroup i runs on XCD i % 8.  When the number of KV groups (batch x n_kv)
// is a multiple of 8, each XCD is given whole KV groups (their K/V stay in that XCD's L2);
// within an XCD the workgroups of one KV group are dispatched together (all its query
// tiles and heads, the query tiles with the most keys first), so they stream the group's
// K/V tiles at about the same time.  With per-sequence cache offsets (up to 64 sequences)
// the KV groups are taken in descending order of their sequence's cached length.

#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace soc {
namespace {

constexpr int D = 128;
constexpr int QT = 128;  // query rows per workgroup
constexpr int KT = 64;   // keys per tile
constexpr int NTHR = 256;
constexpr int TILE_ELEMS = KT * D;              // one K or V tile, 16 KB
constexpr int BUF_ELEMS = 2 * TILE_ELEMS;       // K then V
constexpr float RESCALE_SLACK = 8.0f;           // log2 units the running max may lag
constexpr int KAHEAD = 4;                       // K fragment reads in flight ahead of the S MFMAs

typedef short s16x4 __attribute__((__vector_size__(8)));
typedef short s16x8 __attribute__((__vector_size__(16)));
typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef __attribute__((address_space(3))) s16x4* lds_s16x4_ptr;

// The sequence of descending-length rank r (0 = the most cached keys; equal offsets in
// sequence order) among the batch's B <= 64 sequences, from the cache offsets: lane i counts
// the sequences ranked before sequence i, and the lane whose count is r names it.  One wave.
__device__ __forceinline__ int seq_of_rank(const AttnArgs& a, int r) {
  const int lane = threadIdx.x & 63;
  const int my = lane < a.B ? a.cache_off[lane] : 0;  // lanes past B are never read or chosen
  int before = 0;
  for (int j = 0; j < a.B; ++j) {
    const int oj = __builtin_amdgcn_readlane(my, j);
    before += (oj > my) | ((oj == my) & (j < lane));
  }
  const unsigned long long hit = __builtin_amdgcn_ballot_w64(lane < a.B && before == r);
  return __ffsll(hit) - 1;
}

// Workgroup -> (row group rg, first query head hq of its head group, sequence b).  A
// workgroup takes gs query heads of one KV group (gs divides g) over rwg = 128 / gs rows.
__device__ __forceinline__ void map_block(int bid, const AttnArgs& a, int n_rg, int gs, int& rg, int& hq, int& b) {
  const int hgn = a.g / gs;  // head groups per KV head
  const int units = a.B * a.Hkv;
  if ((units & 7) == 0) {
    // unit-major within the XCD: all row groups and heads of one KV group run together, so
    // the group's K/V stream is fetched from HBM about once and re-read from L2.  With
    // per-sequence cache offsets (a batch of chunks at different cache lengths) the units are
    // taken longest sequence first, so the grid does not end on a long sequence's tiles.
    const int xcd = bid & 7, j = bid >> 3;
    const int per_unit = n_rg * hgn;
    const int ul = j / per_unit;
    const int rem = j - ul * per_unit;
    const int rg_rev = rem / hgn, hgi = rem - rg_rev * hgn;
    const int unit = ul * 8 + xcd;
    const int br = unit / a.Hkv;
    const int kvh = unit - br * a.Hkv;
    b = (a.cache_off && a.B > 1 && a.B <= 64) ? seq_of_rank(a, br) : br;
    hq = kvh * a.g + hgi * gs;
    rg = n_rg - 1 - rg_rev;
  } else {
    const int hgs = a.Hq / gs;
    const int per_row = a.B * hgs;
    const int rg_rev = bid / per_row;
    const int rem = bid - rg_rev * per_row;
    b = rem / hgs;
    hq = (rem - b * hgs) * gs;
    rg = n_rg - 1 - rg_rev;
  }
}

// Query heads a workgroup stacks.  With a window and GQA the waves take gs heads of one KV
// group over the same 32-row block, so every wave needs the same key tiles (a 128-row
// workgroup's waves each skip one tile of the range at a window edge); the remaining 4 / gs
// factor of waves take further 32-row blocks.  Causal prefill without a window keeps 128
// rows of one head (measured 1 % faster that way, the window 2 % slower); block-sparse mode
// stacks rows only (its lists differ by head and are per 128-row block).
__host__ __device__ inline int heads_per_workgroup(const AttnArgs& a) {
  if (a.block_list || a.block_mask || a.window <= 0) return 1;
  return (a.g & 3) == 0 ? 4 : (a.g & 1) == 0 ? 2 : 1;
}

// Element offset of (row, 16-byte chunk) inside a K / V tile.
__device__ __forceinline__ int k_off(int row, int chunk) { return row * D + ((chunk ^ (row & 15)) << 3); }
__device__ __forceinline__ int v_off(int row, int chunk) { return row * D + ((chunk ^ ((row & 3) << 2)) << 3); }

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Which key blocks a workgroup walks: all in its range, those of a kept-block list, or those a
// block mask marks.
enum SparseMode { kDense = 0, kList = 1, kMask = 2 };

constexpr int KBITS = 64;  // chunks of 64 key blocks whose kept sets a workgroup caches in LDS

template <int MODE, bool HSTACK>
__global__ void __launch_bounds__(NTHR) __attribute__((amdgpu_waves_per_eu(2)))
prefill_bf16_d128(AttnArgs a) {
  __shared__ uint64_t kbits[MODE == kMask ? KBITS : 1];
  __shared__ __attribute__((aligned(1024))) bf16_t lds[2 * BUF_ELEMS];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  const int gs = HSTACK ? heads_per_workgroup(a) : 1;
  const int rwg = QT / gs;  // query rows per workgroup
  const int n_rg = (a.tq + rwg - 1) / rwg;
  int rg, hq, b;
  map_block(blockIdx.x, a, n_rg, gs, rg, hq, b);
  rg = __builtin_amdgcn_readfirstlane(rg);  // integer division leaves these in VGPRs
  hq = __builtin_amdgcn_readfirstlane(hq);
  b = __builtin_amdgcn_readfirstlane(b);
  const int h = HSTACK ? __builtin_amdgcn_readfirstlane(hq + wave % gs) : hq;  // this wave's query head
  const int rb = HSTACK ? wave / gs : wave;                                      // this wave's 32-row block
  const int kvh = __builtin_amdgcn_readfirstlane(hq / a.g);
  // Per-workgroup scalars are made provably wave-uniform so tile-level branches stay scalar.
  const int off = __builtin_amdgcn_readfirstlane(a.cache_off ? a.cache_off[b] : a.tk - a.tq);
  const int tkb = off + a.tq;
  const int row0 = rg * rwg;
  const int rowl = min(row0 + rwg, a.tq) - 1;
  const int kv_hi = min(tkb, off + rowl + 1);
  const int kv_lo = a.window > 0 ? max(0, off + row0 - a.window + 1) : 0;
  const int t_lo = kv_lo / KT, t_hi = (kv_hi + KT - 1) / KT;

  const int wr0 = row0 + rb * 32;
  const int wrl = min(wr0 + 31, rowl);
  const bool wave_active = wr0 <= rowl;
  const int my_row = wr0 + l32;
  const int my_pos = off + my_row;
  const int wpos_lo = off + wr0, wpos_hi = off + wrl;

  const bf16_t* qp = (const bf16_t*)a.q + b * a.q_sb + h * a.q_sh;
  const bf16_t* kp = (const bf16_t*)a.k + b * a.kv_sb + kvh * a.kv_sh;
  const bf16_t* vp = (const bf16_t*)a.v + b * a.kv_sb + kvh * a.kv_sh;

  // Tile sequence: dense = t_lo .. t_hi-1; sparse = the two 64-key halves of each listed (or
  // marked) 128-key block, restricted to [t_lo, t_hi) (a contiguous run, in ascending order).
  const int32_t* lst = nullptr;
  const uint8_t* mrow = nullptr;
  auto kept_block = [&](int kb) __attribute__((always_inline)) -> bool { return mrow[kb] != 0; };
  int n0 = 0, n1 = 0;
  const int kb_lo = t_lo >> 1, kb_hi = (t_hi - 1) >> 1;  // key blocks holding tiles of the range
  // Mask rows are read 64 key blocks at a time: lane j reads block c + j (blocks
  // outside [kb_lo, kb_hi] count as not kept) and a ballot gives the wave-uniform set.
  auto mask_bits = [&](int c) __attribute__((always_inline)) -> uint64_t {
    const int kb = c + lane;
    const bool kept = kb >= kb_lo && kb <= kb_hi && kept_block(kb);
    return __builtin_amdgcn_ballot_w64(kept);
  };
  if (MODE == kList) {
    lst = a.block_list + ((int64_t)(b * a.Hq + h) * a.n_qb + rg) * a.list_stride;  // rows of block rg
    const int cnt = lst[0];
    n1 = 2 * cnt;
    while (n0 < n1 && 2 * lst[1 + (n0 >> 1)] + (n0 & 1) < t_lo) ++n0;
    int e = n0;
    while (e < n1 && 2 * lst[1 + (e >> 1)] + (e & 1) < t_hi) ++e;
    n1 = e;
  } else if (MODE == kMask) {
    mrow = a.block_mask + ((int64_t)(b * a.Hq + h) * a.n_qb + rg) * a.mask_stride;
    if (t_lo < t_hi) {
      // The kept sets of the first KBITS chunks of 64 blocks go to LDS once per workgroup (its
      // waves share one (b, h, query block) row here), each wave taking every fourth chunk.
      const int nch = (kb_hi - kb_lo) / 64 + 1;
      for (int ci = wave; ci < min(nch, KBITS); ci += 4) {
        const uint64_t bits = mask_bits(kb_lo + 64 * ci);
        if (lane == 0) kbits[ci] = bits;
      }
      __syncthreads();
      int kept = 0;
      for (int ci = 0; ci < nch; ++ci)
        kept += __builtin_popcountll(ci < KBITS ? kbits[ci] : mask_bits(kb_lo + 64 * ci));
      // each kept block holds two tiles, less a half below t_lo or at t_hi
      n1 = 2 * kept;
      if ((t_lo & 1) && kept_block(kb_lo)) --n1;
      if ((t_hi & 1) && kept_block(kb_hi)) --n1;
      n1 = __builtin_amdgcn_readfirstlane(n1);
    }
  } else {
    n1 = max(0, t_hi - t_lo);
  }
  // Sparse mode keeps the list in registers, 64 entries per load (lane j holds entry
  // lchunk + j), so a tile's index is a lane read rather than a memory round trip that would
  // sit between a tile's start and its successor's DMA.
  int lchunk = -64, lreg = 0;
  // Mask mode walks its row in order: mc is the chunk of 64 blocks being read, mbits its kept
  // blocks not yet taken, mkb the block whose upper half comes next when modd is set.
  int mc = kb_lo - 64, mkb = 0;
  uint64_t mbits = 0;
  bool modd = false;
  auto tile_of = [&](int n) __attribute__((always_inline)) -> int {
    if (MODE == kDense) return t_lo + n;
    if (MODE == kMask) {  // the next tile of the sequence (tiles are asked for in order)
      for (;;) {
        if (modd) {
          modd = false;
          if (2 * mkb + 1 < t_hi) return 2 * mkb + 1;
          continue;
        }
        while (mbits == 0) {  // ends: the count says a kept block is left
          mc += 64;
          const int ci = (mc - kb_lo) >> 6;
          mbits = ci < KBITS ? kbits[ci] : mask_bits(mc);
        }
        mkb = mc + __builtin_ctzll(mbits);
        mbits &= mbits - 1;
        modd = true;
        if (2 * mkb >= t_lo) return 2 * mkb;
      }
    }
    const int e = n >> 1;
    if ((e & ~63) != lchunk) {  // uniform; once per 64 list entries
      lchunk = e & ~63;
      lreg = lchunk + lane < ((n1 + 1) >> 1) ? lst[1 + lchunk + lane] : 0;
    }
    return 2 * __builtin_amdgcn_readlane(lreg, e & 63) + (n & 1);
  };

  // HBM -> LDS for one tile: wave w fills 1 KB blocks 4w..4w+3 (rows 16w..16w+15) of K and V.
  // Buffer loads with a per-lane byte offset fixed for the kernel (row in tile, swizzled
  // chunk) and the tile's first row in the scalar offset; rows at or beyond kv_hi fall
  // outside the buffer's range and read as zero.
  const uint32_t row_bytes = (uint32_t)a.kv_st * 2u;
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)kp, (short)0, (int)(kv_hi * row_bytes), 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)vp, (short)0, (int)(kv_hi * row_bytes), 0x00020000);
  uint32_t kdma[4], vdma[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (wave * 4 + i) * 4 + (lane >> 4);
    const int sl = lane & 15;
    kdma[i] = r * row_bytes + (uint32_t)((sl ^ (r & 15)) << 4);
    vdma[i] = r * row_bytes + (uint32_t)((sl ^ ((r & 3) << 2)) << 4);
  }
  auto issue_tile = [&](int t, int buf) __attribute__((always_inline)) {
    const uint32_t tile_off = (uint32_t)(t * KT) * row_bytes;
    bf16_t* kdst = lds + buf * BUF_ELEMS;
    bf16_t* vdst = kdst + TILE_ELEMS;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int blk = wave * 4 + i;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void_ptr)(kdst + blk * 512), 16, kdma[i], tile_off, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void_ptr)(vdst + blk * 512), 16, vdma[i], tile_off, 0, 0);
    }
  };

  // the tile of step n + 1, found (and its loads issued) at the start of step n
  int t_next = n0 < n1 ? tile_of(n0) : 0;
  if (n0 < n1) issue_tile(t_next, 0);

  // Dense mode: the wave's 32 query rows go HBM -> LDS by DMA too, into its own 8 KB of the
  // second buffer (free until the first tile step fills it): whole rows, four per instruction,
  // 16-byte chunk c of row r at chunk c ^ (r & 15); rows at or beyond tq fall outside the buffer
  // range and read as zero.  They are read into registers in the MFMA operand layout before the
  // loop.  The sparse modes, whose workgroups walk few tiles, load them into registers directly
  // (the LDS route's extra barrier cost them more than its whole-row loads saved).
  const uint32_t q_row_bytes = (uint32_t)a.q_st * 2u;
  bf16_t* qlds = lds + BUF_ELEMS + wave * (32 * D);
  if constexpr (MODE == kDense) {
    // (base and range made visibly uniform: a descriptor the compiler takes for divergent is
    // applied lane group by lane group)
    const int nq = __builtin_amdgcn_readfirstlane(max(0, min(32, a.tq - wr0)));
    const uint64_t qb = (uint64_t)(qp + (int64_t)wr0 * a.q_st);
    const uint64_t qbu = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(qb >> 32)) << 32) |
                         (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)qb);
    const __amdgpu_buffer_rsrc_t qrs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)qbu, (short)0, __builtin_amdgcn_readfirstlane((int)(nq * q_row_bytes)), 0x00020000);
    const int qr = lane >> 4;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(qrs, (lds_void_ptr)(qlds + i * 512), 16,
                                               qr * q_row_bytes + (uint32_t)(((lane & 15) ^ ((4 * i + qr) & 15)) << 4),
                                               (uint32_t)(4 * i) * q_row_bytes, 0, 0);
  }
  bf16x8 qf[8];
  if constexpr (MODE != kDense) {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      u32x4 z = {0u, 0u, 0u, 0u};
      qf[ks] = (my_row < a.tq) ? *(const bf16x8*)(qp + (int64_t)my_row * a.q_st + 16 * ks + 8 * hh) : as_bf16x8(z);
    }
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
  const float c = a.scale_log2;

  // Per-lane LDS element offsets, fixed for the whole kernel, so that every LDS read in the
  // loop is one of these plus an immediate (second key block, kk, hi/lo, buffer).
  //   K (A operand of S^T): key l32 (+32), chunk 2*ks + hh.
  //   V (ds_read_b64_tr_b16): lane j of each 16-lane group points at key 4*hh + j/4 (+16kk, +8)
  //   and columns tb*32 + 16*((lane>>4)&1) + 4*(j%4) .. +3; the row's swizzle term 4*(row&3)
  //   depends only on the lane, so only the chunk part varies with tb.
  int koff[8], voff[4];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) koff[ks] = k_off(l32, 2 * ks + hh);
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

  auto compute_tile = [&](const bf16_t* kt, const bf16_t* vt, int j0, bool mask_hi, bool mask_lo)
                          __attribute__((always_inline)) {
    f32x16 s0, s1;
#pragma unroll
    for (int v = 0; v < 16; ++v) { s0[v] = 0.f; s1[v] = 0.f; }
    // K fragments are read KAHEAD steps ahead of the MFMAs that use them; the scheduling
    // barriers keep the compiler from sinking the reads back next to their uses.
    bf16x8 kf0[8], kf1[8];
#pragma unroll
    for (int ks = 0; ks < KAHEAD; ++ks) {
      kf0[ks] = *(const bf16x8*)(kt + koff[ks]);
      kf1[ks] = *(const bf16x8*)(kt + 32 * D + koff[ks]);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      if (ks + KAHEAD < 8) {
        kf0[ks + KAHEAD] = *(const bf16x8*)(kt + koff[ks + KAHEAD]);
        kf1[ks + KAHEAD] = *(const bf16x8*)(kt + 32 * D + koff[ks + KAHEAD]);
      }
      s0 = mfma32x32x16(kf0[ks], qf[ks], s0);
      s1 = mfma32x32x16(kf1[ks], qf[ks], s1);
      __builtin_amdgcn_sched_barrier(0);
    }
    // Index masks, each only on the tiles that need it: the causal limit (keys after a row's
    // position) and the window edge (keys at or before position - W).
    if (mask_hi) {
      asm volatile("");  // keeps this a branch: only tiles on the diagonal pay for it
      const int hi_lim = my_pos - j0;  // key offset e (from j0) is visible iff e <= hi_lim
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int e = 8 * (i >> 2) + 4 * hh + (i & 3);
        s0[i] = e <= hi_lim ? s0[i] : SOC_NEG_INF;
        s1[i] = e + 32 <= hi_lim ? s1[i] : SOC_NEG_INF;
      }
    }
    if (mask_lo) {
      asm volatile("");  // keeps this a branch: only tiles on a window edge pay for it
      const int lo_lim = my_pos - a.window - j0;  // visible iff e > lo_lim
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int e = 8 * (i >> 2) + 4 * hh + (i & 3);
        s0[i] = e > lo_lim ? s0[i] : SOC_NEG_INF;
        s1[i] = e + 32 > lo_lim ? s1[i] : SOC_NEG_INF;
      }
    }
    float mx = fmaxf(s0[0], s1[0]);
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, fmaxf(s0[i], s1[i]));
    mx = pair_max(mx);
    const float m_cand = mx * c;
    const bool upd = m_cand > m_run + RESCALE_SLACK;
    if (__builtin_amdgcn_ballot_w64(upd) != 0) {
      asm volatile("");  // keeps this a branch: the rescale is rare, never speculate it
      // lanes that do not raise their max keep alpha = 1 (their m_run may still be -inf)
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
    float lsum = 0.f;
    bf16x8 pb[4];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p0 = fast_exp2(fmaf(s0[i], c, nm));
      const float p1 = fast_exp2(fmaf(s1[i], c, nm));
      lsum += p0 + p1;
      pb[i >> 3][i & 7] = (bf16_t)p0;
      pb[2 + (i >> 3)][i & 7] = (bf16_t)p1;
    }
    l_run += lsum;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(vt + 16 * kk * D + voff[tb]));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(vt + (16 * kk + 8) * D + voff[tb]));
        const s16x8 va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        oacc[tb] = mfma32x32x16(__builtin_bit_cast(bf16x8, va), pb[kk], oacc[tb]);
      }
    }
  };

  auto tile_step = [&](int n, auto buf_tag) __attribute__((always_inline)) {
    constexpr int BUF = decltype(buf_tag)::value;
    const int t = t_next;
    if (n + 1 < n1) {
      t_next = tile_of(n + 1);
      issue_tile(t_next, BUF ^ 1);
    }
    const bf16_t* kt = lds + BUF * BUF_ELEMS;
    const bf16_t* vt = kt + TILE_ELEMS;

    const int j0 = t * KT;
    const bool skip = !wave_active || j0 > wpos_hi || (a.window > 0 && j0 + KT - 1 <= wpos_lo - a.window);
    if (!skip) {
      // Only tiles that cross a row's causal limit (or window edge) apply that index mask.
      const bool mask_hi = j0 + KT - 1 > wpos_lo;
      const bool mask_lo = a.window > 0 && j0 <= wpos_hi - a.window;
      compute_tile(kt, vt, j0, mask_hi, mask_lo);
    }
    wait_vmem();
    __syncthreads();
  };

  wait_vmem();
  __syncthreads();
  if constexpr (MODE == kDense) {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = *(const bf16x8*)(qlds + l32 * D + (((2 * ks + hh) ^ (l32 & 15)) << 3));
    // every wave has its query fragments before the first tile step's DMA refills the buffer
    __syncthreads();
  }
  for (int n = n0; n < n1; n += 2) {
    tile_step(n, std::integral_constant<int, 0>{});
    if (n + 1 < n1) tile_step(n + 1, std::integral_constant<int, 1>{});
  }

  const float lt = pair_sum(l_run);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  // The output tile goes out through LDS (free once the loop's last barrier has passed): each
  // wave writes its 32 rows x 128 columns into its own 8 KB, 16-byte chunk c of row r at chunk
  // c ^ (r & 15), then stores whole rows, four per instruction (lane j: row 4i + j / 16, chunk
  // j % 16), instead of 8 bytes of 32 different rows per instruction.
  bf16_t* ot = lds + wave * (32 * D);
#pragma unroll
  for (int tb = 0; tb < 4; ++tb)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      bf16x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = (bf16_t)(oacc[tb][4 * g4 + e] * inv);
      *(bf16x4*)(ot + l32 * D + (((4 * tb + g4) ^ (l32 & 15)) << 3) + 4 * hh) = w;
    }
  bf16_t* ob = (bf16_t*)a.o + b * a.o_sb + h * a.o_sh;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int rr = 4 * i + (lane >> 4), ch = lane & 15;
    const u32x4 x = *(const u32x4*)(ot + rr * D + ((ch ^ (rr & 15)) << 3));
    if (wr0 + rr < a.tq) *(u32x4*)(ob + (int64_t)(wr0 + rr) * a.o_st + 8 * ch) = x;
  }
}

}  // namespace

hipError_t launch_prefill_bf16(const AttnArgs& a, hipStream_t s) {
  const int gs = heads_per_workgroup(a);
  const int n_rg = (a.tq + QT / gs - 1) / (QT / gs);
  const int64_t grid = (int64_t)n_rg * a.B * (a.Hq / gs);
  if (grid == 0) return hipSuccess;
  if (a.block_list)
    hipLaunchKernelGGL((prefill_bf16_d128<kList, false>), dim3((unsigned)grid), dim3(NTHR), 0, s, a);
  else if (a.block_mask)
    hipLaunchKernelGGL((prefill_bf16_d128<kMask, false>), dim3((unsigned)grid), dim3(NTHR), 0, s, a);
  else if (gs > 1)
    hipLaunchKernelGGL((prefill_bf16_d128<kDense, true>), dim3((unsigned)grid), dim3(NTHR), 0, s, a);
  else
    hipLaunchKernelGGL((prefill_bf16_d128<kDense, false>), dim3((unsigned)grid), dim3(NTHR), 0, s, a);
  return hipGetLastError();
}

}  // namespace soc
