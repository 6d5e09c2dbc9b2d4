// Split-KV decode for gfx950 (bf16 cache, head_dim 128) and the merge pass.
//
// Decode cost is the bytes read from the cache per step (sotaaz.com/post/attention-in-code,
// sections 1 and 5: the cache holds n_kv heads per token, and what a step costs is what it
// reads).  So every workgroup owns one (sequence, KV head, split of `split` keys) and
// serves all g = n_heads / n_kv query heads x tq rows of that group (<= 32 rows) from a
// single read of the split's K and V: K/V bytes cross HBM exactly once per call.
//
// A workgroup is one wave.  It streams its split in 32-key blocks, keeping NST-1 blocks in
// flight while it consumes one: K goes HBM -> registers directly, already in the MFMA
// A-operand layout (lane = key, 16-byte chunks of its row), and V goes HBM -> LDS by DMA
// (buffer_load ... lds, row-major with a 16-byte-chunk XOR swizzle) for the transposed
// read.  With only V in LDS (8 KB per stage) several such waves fit on a CU, which is what
// keeps enough bytes in flight to stream the cache at HBM rate.  Being alone in its
// workgroup, a wave only waits on its own vector-memory counter, never on a barrier.  Per
// block it computes S^T = K Q^T (query rows are the MFMA's N columns, padded to 32) and
// O^T += V^T P^T with v_mfma_f32_32x32x16_bf16, V read transposed by ds_read_b64_tr_b16,
// with an online softmax in the log2 domain (running max raised only when it grows by more
// than 2^8).  The split's unnormalised partial (max, sum, O) is written in fp32.  The sink is
// not applied here; the merge adds it exactly once per row.
//
// Ordering.  Every wait is in the source, through the s_waitcnt builtin, which the compiler
// treats as touching all memory, so no LDS access moves across it:
//   * a block's K registers and V stage are complete before the step that consumes them
//     reads them or (ring mode) writes its stage.  Loads into registers and LDS-DMA loads
//     each retire in issue order, but not in order with each other: a wait that counted
//     them as one ordered stream (at most the younger blocks' 32 loads outstanding) let a
//     stage's own DMA land after the step had written the ring's new V row into it.  So a
//     step waits until at most 16 loads are outstanding: if any of block n's 8 K or 8 V
//     loads were still pending, the 16 loads of the same kind issued after it (blocks n+1
//     and n+2) would be pending too.  One younger block stays in flight.
//     The wait orders memory accesses only, so the K registers pass through an empty asm
//     after it: otherwise the compiler may schedule the QK MFMAs above it, guarded by its own
//     counts, which assume one in-order stream of loads.
//   * a stage's transposed reads have completed before the DMA that refills it is issued:
//     each step ends with lgkmcnt(0).
// Each stage is a separate LDS variable, so the compiler can tell which stage a pending DMA
// writes and adds no wait of its own (with the three stages in one array it drained every
// load before each block's V reads).
//
// Work order: when the grid takes several rounds of the chip, workgroup i does not take the
// i-th (sequence, KV head, split) in grid order but the i-th in longest-first order: every
// full split, then the partial splits by block count (largest first), then the empty splits
// below a window; sequence, split and KV head break ties.  Each workgroup finds its item from
// the sequence lengths with wave prefix sums and a 64-bucket histogram of the partial sizes.
// Without it the splits of the last sequences in grid order start last and the chip idles
// while they finish.
//
// Ring mode (a W-slot ring per (sequence, KV head), n tokens written before the step): the
// filled slots are 0 .. min(n, W - 1), and the split holding slot n % W stages the step's
// new K/V row in LDS, puts it in place of the slot's old row (in the K registers and in the
// V stage) when that block arrives, and writes it into the slot after its last read.
//
// Merge: per (b, h, r) row, M = max(max_s m_s, sink), L = sum_s l_s 2^(m_s - M) + 2^(sink - M),
// o = sum_s o_s 2^(m_s - M) / L (all in the log2 domain), rounded once to the output type.

#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace soc {
namespace {

constexpr int D = 128;
constexpr int KB = 32;                  // keys per block
constexpr int NST = 3;                  // blocks resident per wave: one consumed, NST-1 in flight
constexpr int VSTAGE = KB * D;          // V elements of one LDS stage (8 KB)
constexpr float RESCALE_SLACK = 8.0f;

typedef short s16x4 __attribute__((__vector_size__(8)));
typedef short s16x8 __attribute__((__vector_size__(16)));
typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef __attribute__((address_space(3))) s16x4* lds_s16x4_ptr;

__device__ __forceinline__ int v_off(int row, int chunk) { return row * D + ((chunk ^ ((row & 3) << 2)) << 3); }

// s_waitcnt vmcnt(N) through the builtin rather than inline assembly: the compiler's own wait
// insertion then knows these loads have landed (it cannot read an asm statement) and adds no
// waits of its own for them.  gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4 and
// lgkmcnt 11:8 left at their maxima (no wait).
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N <= 63, "vmcnt counts at most 63 loads");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Block n's loads have all retired, `BLOCKS_AFTER` younger blocks (8 K and 8 V loads each)
// having been issued since: at most 8 * BLOCKS_AFTER loads may then be outstanding (each kind
// retires in order within itself only).
template <int BLOCKS_AFTER>
__device__ __forceinline__ void wait_blocks() {
  static_assert(16 * BLOCKS_AFTER <= 63, "vmcnt holds at most 63 outstanding loads");
  vm_wait<8 * BLOCKS_AFTER>();
}

// s_waitcnt lgkmcnt(0): every LDS access of this wave has completed.
__device__ __forceinline__ void lds_wait() { __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4)); }

__device__ __forceinline__ int wave_incl_prefix(int x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  return x;
}

// The (sequence, KV head, split) of workgroup `item` in longest-first order (see the header);
// false when the item is past the last split of the call.  hist: 64 ints of LDS.  One wave.
__device__ bool lpt_item(const AttnArgs& a, int item, int* hist, int& b_out, int& kvh_out, int& s_out) {
  const int lane = threadIdx.x & 63;
  const int fb = (a.split + KB - 1) / KB;  // blocks of a full split
  const int unit = item / a.Hkv;
  kvh_out = item - unit * a.Hkv;
  // Splits of sequence bb: s < s_lo are empty (below the window), s_lo is the first with keys,
  // nsb - 1 the last; the full ones are sf0 .. sf0 + nfull - 1; p1 / p2 are the block counts of
  // the first / last split when it is partial (else 0).
  auto info = [&](int bb, int& s_lo, int& nsb, int& sf0, int& nfull, int& p1, int& p2) __attribute__((always_inline)) {
    s_lo = nsb = sf0 = nfull = p1 = p2 = 0;
    if (bb >= a.B) return;
    const int off = seq_cache_off(a, bb);
    // never a split index past the workspace's nsplit, whatever the offsets hold (a valid
    // offset has off + tq <= tk <= nsplit * split, so this changes nothing for those)
    const int tkb = min(off + a.tq, a.nsplit * a.split);
    const int kv_lo = a.window > 0 ? max(0, min(off - a.window + 1, tkb - 1)) : 0;
    nsb = (tkb + a.split - 1) / a.split;
    s_lo = kv_lo / a.split;
    const int bf = (min((s_lo + 1) * a.split, tkb) - kv_lo + KB - 1) / KB;
    const bool has_last = nsb - 1 > s_lo;
    const int bl = has_last ? (tkb - (nsb - 1) * a.split + KB - 1) / KB : 0;
    sf0 = bf == fb ? s_lo : s_lo + 1;
    const int sf1 = has_last ? (bl == fb ? nsb - 1 : nsb - 2) : (bf == fb ? s_lo : s_lo - 1);
    nfull = max(0, sf1 - sf0 + 1);
    p1 = bf < fb ? bf : 0;
    p2 = has_last && bl < fb ? bl : 0;
  };
  auto cls = [&](int blocks) __attribute__((always_inline)) { return (blocks * 64 - 1) / fb; };  // 0..63
  int s_lo, nsb, sf0, nfull, p1, p2;
  // full splits, in (sequence, split) order
  int base = 0;
  for (int c0 = 0; c0 < a.B; c0 += 64) {
    info(c0 + lane, s_lo, nsb, sf0, nfull, p1, p2);
    const int incl = base + wave_incl_prefix(nfull);
    const unsigned long long own = __ballot(nfull > 0 && unit < incl && unit >= incl - nfull);
    if (own) {
      const int L = __ffsll(own) - 1;
      b_out = c0 + L;
      s_out = __builtin_amdgcn_readlane(sf0 + unit - (incl - nfull), L);
      return true;
    }
    base = __builtin_amdgcn_readlane(incl, 63);
  }
  int u = unit - base;
  // partial splits, largest block count first: histogram of their size classes
  hist[lane] = 0;
  __syncthreads();
  for (int c0 = 0; c0 < a.B; c0 += 64) {
    info(c0 + lane, s_lo, nsb, sf0, nfull, p1, p2);
    if (p1) atomicAdd(&hist[cls(p1)], 1);
    if (p2) atomicAdd(&hist[cls(p2)], 1);
  }
  __syncthreads();
  const int hc = hist[63 - lane];  // lane r: class 63 - r, so the prefix runs largest first
  const int hincl = wave_incl_prefix(hc);
  const int ptotal = __builtin_amdgcn_readlane(hincl, 63);
  if (u < ptotal) {
    const unsigned long long ownc = __ballot(hc > 0 && u < hincl && u >= hincl - hc);
    const int r = __ffsll(ownc) - 1;
    const int csel = 63 - r;
    const int m = u - __builtin_amdgcn_readlane(hincl - hc, r);  // rank within the class
    base = 0;
    for (int c0 = 0; c0 < a.B; c0 += 64) {
      info(c0 + lane, s_lo, nsb, sf0, nfull, p1, p2);
      const int c1 = p1 && cls(p1) == csel, c2 = p2 && cls(p2) == csel;
      const int cnt = c1 + c2;
      const int incl = base + wave_incl_prefix(cnt);
      const unsigned long long own = __ballot(cnt > 0 && m < incl && m >= incl - cnt);
      if (own) {
        const int L = __ffsll(own) - 1;
        const int k = m - (incl - cnt);  // 0: this sequence's first such split, 1: its second
        b_out = c0 + L;
        s_out = __builtin_amdgcn_readlane(c1 && k == 0 ? s_lo : nsb - 1, L);
        return true;
      }
      base = __builtin_amdgcn_readlane(incl, 63);
    }
    return false;  // not reached: the histogram counted this split
  }
  u -= ptotal;
  // empty splits below a window, in (sequence, split) order
  base = 0;
  for (int c0 = 0; c0 < a.B; c0 += 64) {
    info(c0 + lane, s_lo, nsb, sf0, nfull, p1, p2);
    const int incl = base + wave_incl_prefix(s_lo);
    const unsigned long long own = __ballot(s_lo > 0 && u < incl && u >= incl - s_lo);
    if (own) {
      const int L = __ffsll(own) - 1;
      b_out = c0 + L;
      s_out = __builtin_amdgcn_readlane(u - (incl - s_lo), L);
      return true;
    }
    base = __builtin_amdgcn_readlane(incl, 63);
  }
  return false;
}

template <bool RING, bool FUSED>
__global__ void __launch_bounds__(FUSED ? 128 : 64) __attribute__((amdgpu_waves_per_eu(2)))
decode_split_bf16_d128(AttnArgs a) {
  constexpr int NW = FUSED ? 2 : 1;  // waves (splits) per workgroup
  static_assert(NST == 3, "one LDS variable per stage");
  __shared__ __attribute__((aligned(1024))) bf16_t vst0[NW * VSTAGE];
  __shared__ __attribute__((aligned(1024))) bf16_t vst1[NW * VSTAGE];
  __shared__ __attribute__((aligned(1024))) bf16_t vst2[NW * VSTAGE];

  const int lane = threadIdx.x & 63;
  const int wave = FUSED ? __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) : 0;
  const int l32 = lane & 31, hh = lane >> 5;
  // V stage ST; this wave's part of it starts wofs elements in (folded into the per-lane
  // read offsets, so that each stage's base stays a constant of the instruction)
  auto vstage = [&](auto stage_tag) __attribute__((always_inline)) -> bf16_t* {
    constexpr int ST = decltype(stage_tag)::value;
    return ST == 0 ? vst0 : ST == 1 ? vst1 : vst2;
  };
  const int wofs = wave * VSTAGE;
  int s_i, kvh_i, b_i;
  if constexpr (FUSED) {
    s_i = wave;
    kvh_i = blockIdx.x % a.Hkv;
    b_i = blockIdx.x / a.Hkv;
  } else if constexpr (!RING) {
    __shared__ int lpt_hist[64];
    if (a.lpt) {
      if (!lpt_item(a, blockIdx.x, lpt_hist, b_i, kvh_i, s_i)) return;
    } else {
      s_i = blockIdx.x % a.nsplit;
      const int rem = blockIdx.x / a.nsplit;
      kvh_i = rem % a.Hkv;
      b_i = rem / a.Hkv;
    }
  } else {
    s_i = blockIdx.x % a.nsplit;
    const int rem = blockIdx.x / a.nsplit;
    kvh_i = rem % a.Hkv;
    b_i = rem / a.Hkv;
  }
  const int s = __builtin_amdgcn_readfirstlane(s_i);
  const int kvh = __builtin_amdgcn_readfirstlane(kvh_i);
  const int b = __builtin_amdgcn_readfirstlane(b_i);
  const int off = __builtin_amdgcn_readfirstlane(seq_cache_off(a, b));
  const int tkb = off + a.tq;
  const int nsb = (tkb + a.split - 1) / a.split;
  if (!FUSED && s >= nsb) return;  // the merge reads only splits below nsb
  const int ks0 = s * a.split, ks1 = min(ks0 + a.split, tkb);
  // Ring mode: the split that holds slot ring_n[b] % tk attends over the step's new K/V row
  // in place of the slot's old contents (staged in LDS) and writes the new row into the slot
  // at its end.
  __shared__ __attribute__((aligned(16))) bf16_t newrow_w[NW][2][D];  // K then V of the step
  bf16_t (&newrow)[2][D] = newrow_w[wave];
  const int slot = RING ? __builtin_amdgcn_readfirstlane(a.ring_n[b] % a.tk) : -1;
  const bool own_slot = RING && slot >= ks0 && slot < ks1;
  if (own_slot) {
    const int64_t nrow = b * a.new_sb + kvh * a.new_sh;
    if (lane < 16)
      *(u32x4*)(&newrow[0][8 * lane]) = *(const u32x4*)((const bf16_t*)a.k_new + nrow + 8 * lane);
    else if (lane < 32)
      *(u32x4*)(&newrow[1][8 * (lane - 16)]) = *(const u32x4*)((const bf16_t*)a.v_new + nrow + 8 * (lane - 16));
  }
  const int kv_lo = a.window > 0 ? max(0, off - a.window + 1) : 0;
  const int kbeg = max(ks0, kv_lo), kend = ks1;
  const int nblk = kbeg < kend ? (kend - kbeg + KB - 1) / KB : 0;

  // K and V through buffer resources whose range ends at the split's last key: later rows
  // read as zero (and are masked).  K goes straight to registers in the MFMA A-operand
  // layout (lane: key l32, chunks 2ks+hh), V goes HBM -> LDS by DMA for the transposed read.
  const uint32_t row_bytes = (uint32_t)a.kv_st * 2u;
  const bf16_t* kp = (const bf16_t*)a.k + b * a.kv_sb + kvh * a.kv_sh;
  const bf16_t* vp = (const bf16_t*)a.v + b * a.kv_sb + kvh * a.kv_sh;
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)kp, (short)0, (int)(kend * row_bytes), 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)vp, (short)0, (int)(kend * row_bytes), 0x00020000);
  const uint32_t k_lane = l32 * row_bytes + hh * 16;
  const int vr = lane >> 4;  // row within each 4-row DMA block
  const uint32_t v_lane = vr * row_bytes + (uint32_t)(((lane & 15) ^ ((vr & 3) << 2)) << 4);

  bf16x8 kreg[NST][8];
  auto issue = [&](int n, auto stage_tag) __attribute__((always_inline)) {
    constexpr int ST = decltype(stage_tag)::value;
    const uint32_t blk_off = (uint32_t)(kbeg + n * KB) * row_bytes;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      kreg[ST][ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(krs, k_lane + ks * 32, blk_off, 0));
#pragma unroll
    for (int i = 0; i < 8; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void_ptr)(vstage(stage_tag) + wofs + i * 512), 16, v_lane,
                                               blk_off + 4 * i * row_bytes, 0, kLoadReadOnce);
  };

  // query row of this lane: rho = head-in-group * tq + r
  const int R = a.g * a.tq;
  const bool row_ok = l32 < R;
  const int h = kvh * a.g + (row_ok ? l32 / a.tq : 0);
  const int r = row_ok ? l32 % a.tq : 0;
  const int pos = row_ok ? off + r : -1;
  const bf16_t* qp = (const bf16_t*)a.q + b * a.q_sb + h * a.q_sh + (int64_t)r * a.q_st;
  bf16x8 qf[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    u32x4 z = {0u, 0u, 0u, 0u};
    qf[ks] = row_ok ? *(const bf16x8*)(qp + 16 * ks + 8 * hh) : as_bf16x8(z);
  }
  vm_wait<0>();  // only block loads are counted below

  // Every step issues one block (past the last block it issues the last block again, into a
  // stage already consumed), so exactly NST - 1 blocks are younger than the one a step
  // consumes on every path; with the issue behind a condition the compiler could not count
  // the loads in flight at the loop head and drained them all there, once per NST blocks.
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
      voff[tb] = wofs + v_off(tr_row, col >> 3) + (col & 7);
    }
  }

  auto step = [&](int n, auto stage_tag) __attribute__((always_inline)) {
    constexpr int ST = decltype(stage_tag)::value;
    issue(min(n + NST - 1, nblk - 1), std::integral_constant<int, (ST + NST - 1) % NST>{});
    wait_blocks<NST - 1>();  // block n's K registers and V stage have landed
    // The wait orders memory accesses only: an MFMA reading the K registers could still be
    // scheduled above it, guarded just by the compiler's own count, which takes all loads as
    // one ordered stream.  Passing the registers through an empty asm after the wait ties
    // their use to it.
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) asm volatile("" : "+v"(kreg[ST][ks]));
    const bf16_t* vt = vstage(stage_tag);
    const int js = kbeg + n * KB;
    if (RING && own_slot && slot >= js && slot < js + KB) {  // uniform: the ring slot being overwritten
      const int rr = slot - js;
      if (l32 == rr) {
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) kreg[ST][ks] = *(const bf16x8*)(&newrow[0][16 * ks + 8 * hh]);
      }
      if (lane < 16) *(u32x4*)(const_cast<bf16_t*>(vt) + wofs + v_off(rr, lane)) = *(const u32x4*)(&newrow[1][8 * lane]);
    }

    f32x16 sacc;
#pragma unroll
    for (int v = 0; v < 16; ++v) sacc[v] = 0.f;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) sacc = mfma32x32x16(kreg[ST][ks], qf[ks], sacc);
    float mx = SOC_NEG_INF;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int j = js + 8 * (v >> 2) + 4 * hh + (v & 3);
      const bool ok = (j < kend) & (j <= pos) & ((a.window <= 0) | (j > pos - a.window));
      sacc[v] = ok ? sacc[v] : SOC_NEG_INF;
      mx = fmaxf(mx, sacc[v]);
    }
    mx = pair_max(mx);
    const float m_cand = mx * c;
    const bool upd = m_cand > m_run + RESCALE_SLACK;
    if (__builtin_amdgcn_ballot_w64(upd) != 0) {
      asm volatile("");  // keeps this a branch: the rescale is rare, never speculate it
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
    lds_wait();  // this stage's LDS reads finish before the next step's DMA refills it
  };

  int n = 0;
  for (; n + NST <= nblk; n += NST) {
    step(n, std::integral_constant<int, 0>{});
    step(n + 1, std::integral_constant<int, 1>{});
    step(n + 2, std::integral_constant<int, 2>{});
  }
  if (n < nblk) step(n, std::integral_constant<int, 0>{});
  if (n + 1 < nblk) step(n + 1, std::integral_constant<int, 1>{});
  vm_wait<0>();  // the repeated last blocks land before LDS reuse or exit

  const float L = pair_sum(l_run);
  if constexpr (FUSED) {
    // Merge of the workgroup's two splits: the (max, sum) pairs through LDS, each wave scales
    // its O by 2^(m - M) / L_total (the sink counted once), wave 1 hands its share to wave 0
    // through its own V stages (idle once its loop is done), and wave 0 writes the output.
    __shared__ float mlx[2][32][2];
    if (hh == 0) {
      mlx[wave][l32][0] = m_run;
      mlx[wave][l32][1] = L;
    }
    __syncthreads();
    const float m0 = mlx[0][l32][0], m1 = mlx[1][l32][0];
    const float sink_l2 = a.sink && row_ok ? a.sink[h] * kLog2e : SOC_NEG_INF;
    const float M = fmaxf(fmaxf(m0, m1), sink_l2);
    const float Mu = M == SOC_NEG_INF ? 0.f : M;
    const float Lt = mlx[0][l32][1] * fast_exp2(m0 - Mu) + mlx[1][l32][1] * fast_exp2(m1 - Mu) + fast_exp2(sink_l2 - Mu);
    const float wgt = Lt > 0.f ? fast_exp2(m_run - Mu) / Lt : 0.f;
    // wave 1's stages 0 and 1: 32 floats per lane each (O columns tb = 0, 1 and tb = 2, 3)
    float* xo0 = reinterpret_cast<float*>(vst0 + VSTAGE);
    float* xo1 = reinterpret_cast<float*>(vst1 + VSTAGE);
    auto xo = [&](int idx) __attribute__((always_inline)) -> float& {
      return idx < 32 ? xo0[idx * 64 + lane] : xo1[(idx - 32) * 64 + lane];
    };
    if (wave == 1) {
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int v = 0; v < 16; ++v) xo(tb * 16 + v) = oacc[tb][v] * wgt;
    }
    __syncthreads();
    if (wave == 0 && row_ok) {
      bf16_t* orow = (bf16_t*)a.o + b * a.o_sb + h * a.o_sh + (int64_t)r * a.o_st;
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          bf16x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            w[e] = (bf16_t)fmaf(oacc[tb][4 * g4 + e], wgt, xo(tb * 16 + 4 * g4 + e));
          *(bf16x4*)(orow + tb * 32 + 8 * g4 + 4 * hh) = w;
        }
    }
  } else if (row_ok) {
    const int64_t rowid = ((int64_t)b * a.Hq + h) * a.tq + r;
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
  if (RING && own_slot) {  // the append: every load of the old slot has completed
    const int64_t rrow = b * a.kv_sb + kvh * a.kv_sh + (int64_t)slot * a.kv_st;
    if (lane < 16)
      *(u32x4*)((bf16_t*)a.k + rrow + 8 * lane) = *(const u32x4*)(&newrow[0][8 * lane]);
    else if (lane < 32)
      *(u32x4*)((bf16_t*)a.v + rrow + 8 * (lane - 16)) = *(const u32x4*)(&newrow[1][8 * (lane - 16)]);
  }
}

__device__ __forceinline__ float wave_max_f(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ float wave_sum_f(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// One wave per output row.  The splits' (max, sum) pairs are spread over the lanes (64 splits
// per pass) and reduced across the wave; each split's weight 2^(m_s - M) / L is then taken
// from its lane, and the partial outputs are summed with several loads in flight.
template <typename OutT>
__global__ void __launch_bounds__(64) decode_merge(AttnArgs a) {
  const int64_t rowid = blockIdx.x;
  const int lane = threadIdx.x;
  const int r = (int)(rowid % a.tq);
  const int h = (int)((rowid / a.tq) % a.Hq);
  const int b = (int)(rowid / ((int64_t)a.tq * a.Hq));
  const int off = seq_cache_off(a, b);
  const int tkb = off + a.tq;
  // splits written for this row (never more than the workspace holds, whatever the offset)
  const int nsb = __builtin_amdgcn_readfirstlane(min((tkb + a.split - 1) / a.split, a.nsplit));
  const float* pml = a.part + decode_o_floats(a) + rowid * a.nsplit * 2;
  const float* po = a.part + rowid * a.nsplit * a.d;
  float M = SOC_NEG_INF;
  for (int s0 = 0; s0 < nsb; s0 += 64)
    if (s0 + lane < nsb) M = fmaxf(M, pml[2 * (s0 + lane)]);
  const float sink_l2 = a.sink ? a.sink[h] * kLog2e : SOC_NEG_INF;
  M = fmaxf(wave_max_f(M), sink_l2);
  const float M_use = (M == SOC_NEG_INF) ? 0.f : M;
  float Lp = 0.f;
  for (int s0 = 0; s0 < nsb; s0 += 64)
    if (s0 + lane < nsb) Lp += pml[2 * (s0 + lane) + 1] * fast_exp2(pml[2 * (s0 + lane)] - M_use);
  const float L = wave_sum_f(Lp) + fast_exp2(sink_l2 - M_use);
  const float inv = L > 0.f ? 1.f / L : 0.f;
  auto weight = [&](int wl_bits, int s) __attribute__((always_inline)) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(wl_bits, s));
  };
  // columns lane and lane + 64 (head_dim <= 128); every lane stays active through the split
  // loop, so each split's weight can be read from its lane
  const bool c0 = lane < a.d, c1 = lane + 64 < a.d;
  float acc0 = 0.f, acc1 = 0.f;
  for (int s0 = 0; s0 < nsb; s0 += 64) {
    // lane j holds the weight 2^(m_s - M) of split s0 + j
    const int wl = __builtin_bit_cast(int, s0 + lane < nsb ? fast_exp2(pml[2 * (s0 + lane)] - M_use) : 0.f);
    const int n = min(64, nsb - s0);
    const float* pp = po + (int64_t)s0 * a.d + lane;
    int s = 0;
    for (; s + 4 <= n; s += 4) {
      float v0[4], v1[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        v0[u] = c0 ? pp[(int64_t)(s + u) * a.d] : 0.f;
        v1[u] = c1 ? pp[(int64_t)(s + u) * a.d + 64] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float w = weight(wl, s + u);
        acc0 += v0[u] * w;
        acc1 += v1[u] * w;
      }
    }
    for (; s < n; ++s) {
      const float w = weight(wl, s);
      if (c0) acc0 += pp[(int64_t)s * a.d] * w;
      if (c1) acc1 += pp[(int64_t)s * a.d + 64] * w;
    }
  }
  OutT* op = (OutT*)a.o + b * a.o_sb + h * a.o_sh + (int64_t)r * a.o_st;
  if (c0) op[lane] = (OutT)(acc0 * inv);
  if (c1) op[lane + 64] = (OutT)(acc1 * inv);
}

}  // namespace

hipError_t launch_decode_bf16(const AttnArgs& a, hipStream_t s) {
  if (a.fused) {  // ring decode, at most two splits: both in one workgroup, merged in place
    const int64_t grid = (int64_t)a.B * a.Hkv;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL((decode_split_bf16_d128<true, true>), dim3((unsigned)grid), dim3(128), 0, s, a);
    return hipGetLastError();
  }
  const int64_t grid = (int64_t)a.B * a.Hkv * a.nsplit;
  if (grid == 0) return hipSuccess;
  if (a.ring_n)
    hipLaunchKernelGGL((decode_split_bf16_d128<true, false>), dim3((unsigned)grid), dim3(64), 0, s, a);
  else
    hipLaunchKernelGGL((decode_split_bf16_d128<false, false>), dim3((unsigned)grid), dim3(64), 0, s, a);
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
