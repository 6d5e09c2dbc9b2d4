// Multi-head latent attention decode for gfx950 (bf16 in, fp32 accumulate).
//
// The cache holds, per token, a latent c_kv (512 wide) and one rope key k_rope (64 wide)
// shared by every head; head h's key is [c_kv @ w_uk[h], k_rope] and its value
// c_kv @ w_uv[h] (sotaaz.com/post/attention-in-code, section 4).  Decode never builds those:
// the query is folded into latent space once (q_lat = w_uk[h] q_nope), scores are
// q_lat . c_kv + q_rope . k_rope, the softmax average is taken over the latents, and w_uv
// is applied once per row to the averaged latent.  So a step reads 576 numbers per cached
// token, shared by all heads.
//
//   mla_absorb_q_kernel     q_lat^T = w_uk[h] q_nope^T for 16 query rows of one head per wave
//                           (v_mfma_f32_16x16x32_bf16, rounded to bf16); also clears the work
//                           queue of the split pass
//   mla_split_kernel        persistent 4-wave workgroups (two per CU: the LDS ring allows two)
//                           that take (sequence, group of 16 query rows, split of keys) items
//                           from an atomic queue; the 16 rows (heads x query tokens) are the N
//                           columns of the MFMAs.  The four waves share the ring: each loads a
//                           quarter of every block, computes a quarter of the 576-dim score
//                           contraction (the partial score blocks are summed through LDS, in a
//                           fixed order, so every wave holds the same scores) and a quarter of
//                           the 512-dim latent output.  Latent rows go HBM ->
//                           registers (two 16-key blocks ahead) -> LDS (a 2-stage ring,
//                           16-byte chunks XOR-swizzled by key); S^T = [C, R] [q_lat, q_rope]^T with
//                           v_mfma_f32_16x16x32_bf16 over 576 dims; online softmax in the log2
//                           domain; O^T += C^T P^T with v_mfma_f32_16x16x16bf16_1k, C read
//                           transposed by ds_read_b64_tr_b16.  Each item's unnormalised
//                           (max, sum, latent O) goes to the workspace.
//   mla_merge_kernel        log-sum-exp merge of a row's splits into its latent output (fp32)
//   mla_expand_kernel       o = w_uv[h]^T o_lat for 16 rows and 32 output dims of one head per
//                           workgroup, rounded to bf16

#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace soc {
namespace {

constexpr int MR = kMlaRank, MDR = kMlaRope, MDN = kMlaNope, MDV = kMlaV;
constexpr int MKB = 16;                      // keys per block
constexpr int MNST = 2;                      // LDS stages = register buffers; 2 blocks in flight
constexpr int LAT_STAGE = MKB * MR;          // latent elements of one stage (16 KB)
constexpr int ROPE_STAGE = MKB * MDR;        // rope elements of one stage (2 KB)
constexpr int MSTAGE = LAT_STAGE + ROPE_STAGE;

typedef short s16x4 __attribute__((__vector_size__(8)));
typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef __attribute__((address_space(3))) s16x4* lds_s16x4_ptr;

__device__ __forceinline__ f32x4 mfma16k32(bf16x8 a, bf16x8 b, f32x4 c) {
  // lane l: A[l%16][8(l/16)+e], B[8(l/16)+e][l%16], D[4(l/16)+v][l%16]
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16k16(bf16x4 a, bf16x4 b, f32x4 c) {
  // lane l: A[l%16][4(l/16)+e], B[4(l/16)+e][l%16], D[4(l/16)+v][l%16]
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------------------
// q_lat^T [512 x 16 rows] = w_uk[h] [512 x 128] q_nope^T [128 x 16 rows], one wave per
// (head, 16 rows (b, t), 64 of the 512 latent dims); lane l: A = w_uk rows 16mb + l%16, B = row l%16 of q_nope,
// D = q_lat dims 16mb + 4(l/16) + v of row l%16.
__global__ void __launch_bounds__(64) mla_absorb_q_kernel(MlaArgs a) {
  const int lane = threadIdx.x, G = lane >> 4, i16 = lane & 15;
  if (blockIdx.x == 0 && lane == 0) *a.queue = 0u;  // work queue of the split pass
  const int part = blockIdx.x & 7;  // 64 latent dims per wave
  const int h = (blockIdx.x >> 3) % a.H;
  const int grp = (blockIdx.x >> 3) / a.H;
  const int nrow = a.B * a.tq;
  const int idx = grp * 16 + i16;
  const bool ok = idx < nrow;
  const int b = ok ? idx / a.tq : 0, t = ok ? idx % a.tq : 0;
  const bf16_t* qn = (const bf16_t*)a.q_nope + b * a.qn_sb + h * a.qn_sh + t * a.qn_st;
  bf16x8 qb[4];
  const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) qb[ks] = ok ? *(const bf16x8*)(qn + 32 * ks + 8 * G) : as_bf16x8(z);
  const bf16_t* wk = (const bf16_t*)a.w_uk + (int64_t)h * MR * MDN;
  const int R = a.H * a.tq;
  bf16_t* out = (bf16_t*)a.q_lat + ((int64_t)b * R + h * a.tq + t) * MR;
#pragma unroll
  for (int mb = 4 * part; mb < 4 * part + 4; ++mb) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      acc = mfma16k32(*(const bf16x8*)(wk + (int64_t)(16 * mb + i16) * MDN + 32 * ks + 8 * G), qb[ks], acc);
    if (ok) {
      bf16x4 w;
#pragma unroll
      for (int v = 0; v < 4; ++v) w[v] = (bf16_t)acc[v];
      *(bf16x4*)(out + 16 * mb + 4 * G) = w;
    }
  }
}

// ---------------------------------------------------------------------------------------
// Loads per wave per block: 4 latent rows (1 KB each) and a quarter (512 B) of the rope tile.
constexpr int WAVE_LOADS = 5;
// s_waitcnt vmcnt(N) through the builtin rather than inline assembly: the compiler's own wait
// insertion then knows these loads have landed and adds no waits of its own for them (it
// cannot read an asm statement, and without that it drained every load before the first
// use of the query fragments in each block).  gfx9 encoding: vmcnt in bits 3:0 and 15:14,
// expcnt 6:4 and lgkmcnt 11:8 left at their maxima (no wait).
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N <= 63, "vmcnt counts at most 63 loads");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
template <int AFTER>
__device__ __forceinline__ void wait_wave_blocks() {
  static_assert(AFTER * WAVE_LOADS <= 63, "vmcnt counts at most 63 loads");
  vm_wait<AFTER * WAVE_LOADS>();
}

__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) mla_split_kernel(MlaArgs a) {
  __shared__ __attribute__((aligned(1024))) bf16_t lds[MNST * MSTAGE];
  __shared__ __attribute__((aligned(16))) float xs[4][64][4];  // each wave's partial score block
  __shared__ uint32_t item_sh;

  const int tid = threadIdx.x, lane = tid & 63, G = lane >> 4, i16 = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int R = a.H * a.tq;
  const int nrg = (R + 15) / 16;
  const uint32_t n_items = (uint32_t)a.B * nrg * a.nsplit;

  // fixed per-lane LDS element offsets
  //   S A operand (key i16 of the block, chunk 4ks + G): i16*512 + ((4ks + G) ^ i16) * 8.
  //     Wave w takes the latent dim chunks ks = w + 4j (j < 4): the swizzle touches only the
  //     low four chunk bits, so chunk ks sits at lat_b + 128 j
  //   rope A operand (key i16, chunk 4kr + G):          i16*64 + ((4kr + G) ^ (i16 & 7)) * 8,
  //     rope chunk kr = w for waves 0 and 1
  //   PV A operand, ds_read_b64_tr_b16 (lane j of group G: key 4G + j/4, dims 16db + 4(j%4)..+3):
  //   with db = 8u + w this wave's dim blocks are u = wave, offset trb[w] + wave*128
  int trb[8];
  const int lat_b = i16 * 512 + (((4 * wave + G) ^ i16) << 3);
  const int rope_b = i16 * 64 + (((4 * (wave & 1) + G) ^ (i16 & 7)) << 3);
  {
    const int kk = 4 * G + (i16 >> 2);
    const int x = (i16 & 3) >> 1;
#pragma unroll
    for (int w = 0; w < 8; ++w) trb[w] = kk * 512 + ((((2 * w + x) ^ kk)) << 3) + 4 * (i16 & 1) + wave * 128;
  }
  // DMA lane offsets: latent row of key i goes to LDS row i (1 KB), LDS chunk j holding the
  // row's chunk j ^ i; the rope tile holds key k's chunk j ^ (k & 7) at chunk j.  Wave w loads
  // latent rows 4w..4w+3 and rope keys 4w..4w+3 (lanes 0..31).
  const uint32_t rope_key = 4u * wave + (uint32_t)((lane & 31) >> 3);  // lanes 32..63 repeat lanes 0..31
  const float c = a.scale_log2;

  for (;;) {
    __syncthreads();  // every wave is done with the previous item's LDS and item_sh
    if (tid == 0) item_sh = atomicAdd(a.queue, 1u);
    __syncthreads();
    const uint32_t item = __builtin_amdgcn_readfirstlane(item_sh);
    if (item >= n_items) break;
    const int s = (int)(item % (uint32_t)a.nsplit);
    const int rg = (int)((item / (uint32_t)a.nsplit) % (uint32_t)nrg);
    const int b = (int)(item / ((uint32_t)a.nsplit * nrg));
    const int off = __builtin_amdgcn_readfirstlane(a.cache_off ? a.cache_off[b] : a.tk - a.tq);
    const int tkb = off + a.tq;
    const int nsb = (tkb + a.split - 1) / a.split;
    if (s >= nsb) continue;  // the merge reads only splits below nsb
    const int ks0 = s * a.split, ks1 = min(ks0 + a.split, tkb);
    const int nblk = (ks1 - ks0 + MKB - 1) / MKB;

    // this lane's query row (MFMA column)
    const int rho = rg * 16 + i16;
    const bool row_ok = rho < R;
    const int h = row_ok ? rho / a.tq : 0, t = row_ok ? rho % a.tq : 0;
    const int pos = row_ok ? off + t : -1;

    // latent and rope rows of this sequence; rows at or beyond the split's end read as zero
    const uint32_t crow = (uint32_t)a.c_st * 2u, rrow = (uint32_t)a.r_st * 2u;
    const bf16_t* cb = (const bf16_t*)a.c_kv + b * a.c_sb;
    const bf16_t* rb = (const bf16_t*)a.k_rope + b * a.r_sb;
    const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc((void*)cb, (short)0, (int)(ks1 * crow), 0x00020000);
    const __amdgpu_buffer_rsrc_t rrs = __builtin_amdgcn_make_buffer_rsrc((void*)rb, (short)0, (int)(ks1 * rrow), 0x00020000);
    const uint32_t rope_v = rope_key * rrow + (uint32_t)(16 * (lane & 7));
    // register staging of one block: latent rows 4 wave + i (lane: 16-byte chunk `lane`),
    // rope keys 4 wave + lane/8 (lanes < 32: chunk lane & 7)
    u32x4 stg[MNST][5];
    auto issue = [&](int n, auto buf_tag) __attribute__((always_inline)) {
      constexpr int BUF = decltype(buf_tag)::value;
      const uint32_t k0 = (uint32_t)(ks0 + n * MKB);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        stg[BUF][i] = __builtin_amdgcn_raw_buffer_load_b128(crs, (uint32_t)(4 * wave + i) * crow + (uint32_t)(16 * lane),
                                                            k0 * crow, kLoadReadOnce);
      // every lane loads (lanes 32..63 the same bytes as lanes 0..31, one request per line), so
      // a block is always WAVE_LOADS loads and the compiler can count them
      stg[BUF][4] = __builtin_amdgcn_raw_buffer_load_b128(rrs, rope_v, k0 * rrow, 0);
    };
    // registers -> LDS stage, XOR-swizzled in 16-byte chunks by key
    auto store = [&](auto buf_tag) __attribute__((always_inline)) {
      constexpr int BUF = decltype(buf_tag)::value;
      bf16_t* lat = lds + BUF * MSTAGE;
      bf16_t* rop = lat + LAT_STAGE;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = 4 * wave + i;
        *(u32x4*)(lat + key * 512 + ((lane ^ key) << 3)) = stg[BUF][i];
      }
      if (lane < 32) *(u32x4*)(rop + rope_key * 64 + (((lane & 7) ^ (rope_key & 7)) << 3)) = stg[BUF][4];
    };

    // query fragments (B operand of S^T): dims 32ks + 8G .. +7 of row rho for this wave's
    // latent chunks ks = wave + 4j, then its rope chunk (used by waves 0 and 1)
    bf16x8 qf[5];
    {
      const bf16_t* ql = (const bf16_t*)a.q_lat + ((int64_t)b * R + rho) * MR;
      const bf16_t* qr = (const bf16_t*)a.q_rope + b * a.qr_sb + h * a.qr_sh + t * a.qr_st;
      const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int j = 0; j < 4; ++j) qf[j] = row_ok ? *(const bf16x8*)(ql + 32 * (wave + 4 * j) + 8 * G) : as_bf16x8(z);
      qf[4] = row_ok ? *(const bf16x8*)(qr + 32 * (wave & 1) + 8 * G) : as_bf16x8(z);
    }
    vm_wait<0>();  // only block loads are counted below

    // Every step issues one block (past the last block it issues the last block again into
    // the registers it just stored), so exactly one block is younger than the one a step
    // stores on every path.  With the issues and waits behind conditions the compiler could
    // not count the loads in flight and drained them all once every two blocks.
    if (nblk > 0) {
      issue(0, std::integral_constant<int, 0>{});
      __builtin_amdgcn_sched_barrier(0);  // block 0's loads stay ahead of block 1's (the waits count on it)
      issue(min(1, nblk - 1), std::integral_constant<int, 1>{});
    }

    f32x4 oacc[8];
#pragma unroll
    for (int d = 0; d < 8; ++d) oacc[d] = (f32x4){0.f, 0.f, 0.f, 0.f};
    float m_run = SOC_NEG_INF, l_run = 0.f;

    auto step = [&](int n, auto stage_tag) __attribute__((always_inline)) {
      constexpr int ST = decltype(stage_tag)::value;
      wait_wave_blocks<1>();  // block n+1 (issued earlier) may stay in flight; block n's registers have landed
      store(std::integral_constant<int, ST>{});  // stage ST held block n-2: every wave finished it before barrier n-1
      issue(min(n + 2, nblk - 1), std::integral_constant<int, ST>{});  // the registers just stored
      __syncthreads();  // every wave's part of block n is in LDS
      const bf16_t* lat = lds + ST * MSTAGE;
      const bf16_t* rop = lat + LAT_STAGE;

      // this wave's share of the score contraction: latent chunks wave + 4j, rope chunk wave
      f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
      s0 = mfma16k32(*(const bf16x8*)(lat + lat_b), qf[0], s0);
      s1 = mfma16k32(*(const bf16x8*)(lat + lat_b + 128), qf[1], s1);
      s0 = mfma16k32(*(const bf16x8*)(lat + lat_b + 256), qf[2], s0);
      s1 = mfma16k32(*(const bf16x8*)(lat + lat_b + 384), qf[3], s1);
      if (wave < 2) s0 = mfma16k32(*(const bf16x8*)(rop + rope_b), qf[4], s0);
      // partial blocks summed through LDS in wave order, so every wave gets the same scores;
      // xs is rewritten only after the next block's barrier, which every wave reaches after
      // its reads below
      *(f32x4*)&xs[wave][lane][0] = s0 + s1;
      __syncthreads();
      const f32x4 sc = ((*(const f32x4*)&xs[0][lane][0] + *(const f32x4*)&xs[1][lane][0]) +
                        *(const f32x4*)&xs[2][lane][0]) + *(const f32x4*)&xs[3][lane][0];
      // lane: keys 4G + v of the block for row i16 (every wave holds the whole score block)
      const int j0 = ks0 + n * MKB + 4 * G;
      float sv[4];
      float mx = SOC_NEG_INF;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int j = j0 + v;
        sv[v] = (j < ks1 && j <= pos) ? sc[v] : SOC_NEG_INF;
        mx = fmaxf(mx, sv[v]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_cand = mx * c;
      const bool upd = m_cand > m_run + 8.0f;
      if (__builtin_amdgcn_ballot_w64(upd) != 0) {
        asm volatile("");  // keeps this a branch: the rescale is rare
        const float m_new = upd ? m_cand : m_run;
        const float alpha = upd ? fast_exp2(m_run - m_new) : 1.f;
        l_run *= alpha;
#pragma unroll
        for (int d = 0; d < 8; ++d)
#pragma unroll
          for (int v = 0; v < 4; ++v) oacc[d][v] *= alpha;
        m_run = m_new;
      }
      const float nm = (m_run == SOC_NEG_INF) ? 0.f : -m_run;
      bf16x4 pb;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float p = fast_exp2(fmaf(sv[v], c, nm));
        l_run += p;
        pb[v] = (bf16_t)p;
      }
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const s16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(lat + trb[w]));
        oacc[w] = mfma16k16(__builtin_bit_cast(bf16x4, va), pb, oacc[w]);
      }
    };

    static_assert(MNST == 2, "the buffer rotation below is written for two stages");
    int n = 0;
    for (; n + MNST <= nblk; n += MNST) {
      step(n, std::integral_constant<int, 0>{});
      step(n + 1, std::integral_constant<int, 1>{});
    }
    if (n < nblk) step(n, std::integral_constant<int, 0>{});
    vm_wait<0>();  // the repeated last block lands before the registers are reused

    // the row's sum over the 4 lanes that share it
    l_run += __shfl_xor(l_run, 16, 64);
    l_run += __shfl_xor(l_run, 32, 64);
    if (row_ok && wave == 0 && G == 0) {
      const int64_t prow = ((int64_t)b * R + rho) * a.nsplit + s;
      a.part_ml[2 * prow] = m_run;
      a.part_ml[2 * prow + 1] = l_run;
    }
    // The partial latent output goes out through LDS: each wave's 16 rows x 128 dims (dims
    // 128 wave + 16 w + 4 G + v in lane (i16, G)) into its own 8 KB, 16-byte chunk c of row r
    // at chunk c ^ r, then stored as whole 512-byte row slices, two rows per instruction,
    // instead of 64 bytes of each of 16 rows per instruction.  The barrier: every wave is done
    // with the last block's stage.
    __syncthreads();
    float* ost = reinterpret_cast<float*>(lds) + wave * (16 * 128);
#pragma unroll
    for (int w = 0; w < 8; ++w) *(f32x4*)(ost + i16 * 128 + (((4 * w + G) ^ i16) << 2)) = oacc[w];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = 2 * i + (lane >> 5), cc = lane & 31;
      const f32x4 x = *(const f32x4*)(ost + r * 128 + ((cc ^ r) << 2));
      if (rg * 16 + r < R) {
        const int64_t prow = ((int64_t)b * R + rg * 16 + r) * a.nsplit + s;
        *(f32x4*)(a.part_o + prow * MR + 128 * wave + 4 * cc) = x;
      }
    }
  }  // work loop
}

// Merge of one row's splits for 256 latent dims per workgroup (grid: rows x 2):
// o_lat[d] = sum_s 2^(m_s - M) o_s[d] / sum_s 2^(m_s - M) l_s, M = max_s m_s (0 if no token).
__global__ void __launch_bounds__(256) mla_merge_kernel(MlaArgs a) {
  __shared__ float wgt[kMlaMaxSplits];
  __shared__ float inv_l;
  const int row = blockIdx.x >> 1, half = blockIdx.x & 1;  // row = b * R + rho
  const int R = a.H * a.tq;
  const int b = row / R, t = (row % R) % a.tq;
  const int off = a.cache_off ? a.cache_off[b] : a.tk - a.tq;
  const int nsb = min((off + a.tq + a.split - 1) / a.split, a.nsplit);  // never past the workspace
  const int64_t p0 = (int64_t)row * a.nsplit;
  (void)t;
  if (threadIdx.x < 64) {  // wave 0: max over splits, then the weights and their sum
    float M = SOC_NEG_INF;
    for (int k = threadIdx.x; k < nsb; k += 64) M = fmaxf(M, a.part_ml[2 * (p0 + k)]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
    const float Ms = M == SOC_NEG_INF ? 0.f : M;
    float L = 0.f;
    for (int k = threadIdx.x; k < nsb; k += 64) {
      const float m = a.part_ml[2 * (p0 + k)];
      const float w = m == SOC_NEG_INF ? 0.f : fast_exp2(m - Ms);
      wgt[k] = w;
      L = fmaf(w, a.part_ml[2 * (p0 + k) + 1], L);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) L += __shfl_xor(L, o, 64);
    if (threadIdx.x == 0) inv_l = L > 0.f ? 1.f / L : 0.f;  // a row with no visible token outputs 0
  }
  __syncthreads();
  const int d = half * 256 + threadIdx.x;
  // eight splits per step with independent accumulators, so eight loads are in flight
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  int k = 0;
  for (; k + 8 <= nsb; k += 8) {
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = a.part_o[(p0 + k + e) * MR + d];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = fmaf(wgt[k + e], x[e], acc[e]);
  }
  for (; k < nsb; ++k) acc[k & 7] = fmaf(wgt[k], a.part_o[(p0 + k) * MR + d], acc[k & 7]);
  const float sum = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
  a.o_lat[(int64_t)row * MR + d] = sum * inv_l;
}

// o[row, 32q + j] = sum_r o_lat[row, r] w_uv[h, r, 32q + j] for 16 rows (b, t) of head h
// (grid: H x row groups x 4 quarters of the output width).
__global__ void __launch_bounds__(256) mla_expand_kernel(MlaArgs a) {
  __shared__ __attribute__((aligned(16))) float ol[16][MR + 4];  // rows padded: 16 rows hit 16 bank groups
  __shared__ __attribute__((aligned(16))) float part[16][32];    // upper latent half's partial products
  __shared__ __attribute__((aligned(16))) bf16_t ws[MR][32];  // w_uv[h][:, 32 q4 .. 32 q4 + 31]
  const int q4 = blockIdx.x & 3;
  const int hg = blockIdx.x >> 2;
  const int h = hg % a.H, grp = hg / a.H;
  const int nrow = a.B * a.tq;
  const int R = a.H * a.tq;
  {  // the 16 latent rows in 16-byte pieces, all loads in flight at once: rows past the end
     // load the last row (no branch around the loads) and are stored as 0
    f32x4 v[16 * MR / 4 / 256];
#pragma unroll
    for (int k = 0; k < 16 * MR / 4 / 256; ++k) {
      const int i = threadIdx.x + 256 * k, r = i / (MR / 4), c = i % (MR / 4);
      const int idx = min(grp * 16 + r, nrow - 1);
      const int b = idx / a.tq, t = idx - b * a.tq;
      v[k] = *(const f32x4*)(a.o_lat + ((int64_t)b * R + h * a.tq + t) * MR + 4 * c);
    }
#pragma unroll
    for (int k = 0; k < 16 * MR / 4 / 256; ++k) {
      const int i = threadIdx.x + 256 * k, r = i / (MR / 4), c = i % (MR / 4);
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      *(f32x4*)&ol[r][4 * c] = grp * 16 + r < nrow ? v[k] : z;
    }
  }
  {  // the 512 x 32 weight slice in 16-byte pieces, all loads in flight at once
    const bf16_t* wsrc = (const bf16_t*)a.w_uv + (int64_t)h * MR * MDV + 32 * q4;
#pragma unroll
    for (int k = 0; k < MR * 4 / 256; ++k) {
      const int i = threadIdx.x + 256 * k, r = i >> 2, c = i & 3;
      *(u32x4*)&ws[r][8 * c] = *(const u32x4*)(wsrc + (int64_t)r * MDV + 8 * c);
    }
  }
  __syncthreads();
  // o[16 rows][32 dims] = ol[16][512] ws[512][32] in fp32 with v_mfma_f32_16x16x4f32 (lane l:
  // A[l%16][l/16], B[l/16][l%16], D[4(l/16)+v][l%16]); wave w takes output dims 16 (w & 1) ..
  // over latent half w >> 1, in two accumulator chains; the upper half's products go through LDS
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int jt = wv & 1, kh = wv >> 1;
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
  for (int k0 = 256 * kh; k0 < 256 * kh + 256; k0 += 8) {
    acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(ol[lane & 15][k0 + (lane >> 4)], (float)ws[k0 + (lane >> 4)][16 * jt + (lane & 15)],
                                                acc0, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(ol[lane & 15][k0 + 4 + (lane >> 4)],
                                                (float)ws[k0 + 4 + (lane >> 4)][16 * jt + (lane & 15)], acc1, 0, 0, 0);
  }
  const f32x4 acc = acc0 + acc1;  // rows 4 (lane/16) + v, dim 16 jt + lane % 16
  if (kh == 1) {
#pragma unroll
    for (int v = 0; v < 4; ++v) part[4 * (lane >> 4) + v][16 * jt + (lane & 15)] = acc[v];
  }
  __syncthreads();
  if (kh == 0) {
    const int dout = 32 * q4 + 16 * jt + (lane & 15);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int r = 4 * (lane >> 4) + v, idx = grp * 16 + r;
      if (idx < nrow) {
        const int b = idx / a.tq, t = idx % a.tq;
        ((bf16_t*)a.o)[b * a.o_sb + h * a.o_sh + t * a.o_st + dout] = (bf16_t)(acc[v] + part[r][16 * jt + (lane & 15)]);
      }
    }
  }
}

}  // namespace

hipError_t launch_mla_decode(const MlaArgs& a, hipStream_t s) {
  const int64_t groups = ((int64_t)a.B * a.tq + 15) / 16;
  const int64_t g1 = groups * a.H;
  if (g1 == 0) return hipSuccess;
  hipLaunchKernelGGL(mla_absorb_q_kernel, dim3((unsigned)(8 * g1)), dim3(64), 0, s, a);
  const int64_t nrg = ((int64_t)a.H * a.tq + 15) / 16;
  const int64_t items = (int64_t)a.B * nrg * a.nsplit;
  const int64_t wgs = items < a.n_waves ? items : a.n_waves;
  hipLaunchKernelGGL(mla_split_kernel, dim3((unsigned)wgs), dim3(256), 0, s, a);
  const int64_t rows = (int64_t)a.B * a.H * a.tq;
  hipLaunchKernelGGL(mla_merge_kernel, dim3((unsigned)(2 * rows)), dim3(256), 0, s, a);
  hipLaunchKernelGGL(mla_expand_kernel, dim3((unsigned)(4 * g1)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace soc
