// Internal declarations shared by the HIP kernels and the C-ABI dispatch layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace soc {

constexpr float kLog2e = 1.4426950408889634f;

// Arguments of one attention launch (prefill or decode).  Strides are in elements.
struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  int64_t q_sb, q_sh, q_st;
  int64_t kv_sb, kv_sh, kv_st;
  int64_t o_sb, o_sh, o_st;
  int32_t B, Hq, Hkv, g, tq, tk, d;
  const int32_t* cache_off;  // device [B] or null (offset tk - tq)
  int32_t window;            // <= 0: none
  const float* sink;         // device [Hq] or null
  float scale_log2;          // softmax scale * log2(e)
  // block-sparse prefill: a kept-block list or a block mask (at most one of them)
  const int32_t* block_list;  // device [B, Hq, n_qb, list_stride] or null
  const uint8_t* block_mask;  // device [B, Hq, n_qb, mask_stride] or null
  int32_t block_size, n_qb, list_stride, mask_stride;
  // split-KV decode
  float* part;     // workspace: partial sums, [B*Hq*tq][nsplit][d] floats, then [..][nsplit][2]
  int32_t nsplit;  // splits per sequence (capacity)
  int32_t split;   // keys per split
  int32_t lpt;     // bf16 decode: workgroups take the splits longest first (grids of several rounds)
  int32_t fused;   // bf16 ring decode with nsplit <= 2: one workgroup per (sequence, KV head) merges
                   // its two splits itself and writes the output (no partials, no merge kernel)
  // ring-buffer decode (bf16): the cache is a tk-slot ring per (sequence, KV head), ring_n[b]
  // tokens written before this step; the step's K/V rows (k_new, v_new) go to slot
  // ring_n[b] % tk, and the step attends over the min(ring_n[b] + 1, tk) filled slots.
  const int32_t* ring_n;  // device [B] or null (no ring)
  const void* k_new;
  const void* v_new;
  int64_t new_sb, new_sh;
};

// Cache offset of sequence b: the ring's filled slots minus one, the caller's offset, or
// tk - tq.
__device__ inline int seq_cache_off(const AttnArgs& a, int b) {
  if (a.ring_n) return min(a.ring_n[b], a.tk - 1);
  return a.cache_off ? a.cache_off[b] : a.tk - a.tq;
}

// Decode workspace layout helpers (floats).
__host__ __device__ inline size_t decode_rows(const AttnArgs& a) { return (size_t)a.B * a.Hq * a.tq; }
__host__ __device__ inline size_t decode_o_floats(const AttnArgs& a) { return decode_rows(a) * a.nsplit * a.d; }
__host__ __device__ inline size_t decode_ml_floats(const AttnArgs& a) { return decode_rows(a) * a.nsplit * 2; }

// Buckets of the per-head score histogram that narrows the order statistic; the side of the
// square tile of (query block, key block) scores one MFMA pass covers; the key tiles of one
// work item of the histogram pass (whose rows stay in one head).
constexpr int kSelBuckets = 4096;
constexpr int kScoreTile = 64;
constexpr int kScoreKC = 2;
// Items per head of the histogram pass: 64-row tiles of the head's query blocks times key
// chunks of kScoreKC 64-block tiles.
__host__ __device__ inline int64_t sel_items_per_head(int nqb, int nkb) {
  return (int64_t)((nqb + kScoreTile - 1) / kScoreTile) *
         (((nkb + kScoreTile - 1) / kScoreTile + kScoreKC - 1) / kScoreKC);
}

struct SelectArgs {
  const void* q;
  const void* k;
  int64_t q_sb, q_sh, q_st;
  int64_t k_sb, k_sh, k_st;
  int32_t B, Hq, Hkv, g, tq, tk, d, bs, nqb, nkb;  // nkb = ceil(tk / bs)
  const int32_t* cache_off;
  int32_t window;
  double keep_mean, keep_radius;
  double* tau_mean;    // [B, Hq]
  double* tau_radius;  // [B, Hkv]
  uint8_t* mask;       // [B, Hq, nqb, nkb]
  int32_t* list;       // [B, Hq, nqb, 1 + nkb] or null
  double* qmean;       // workspace [B, Hq, nqb, d]
  double* cent;        // workspace [B, Hkv, nkb, d]  key-block centroids
  double* rad2;        // workspace [B, Hkv, nkb]
  double* score;       // workspace [B, Hq, nqb, nkb]  (heads scored in one pass)
  double* norm2;       // workspace [B, Hq, nqb] |qmean|^2 then [B, Hkv, nkb] |c|^2
  double* nmax;        // workspace [B*Hq] max |qmean|^2 per head, then [B*Hkv] max |c|^2
  uint32_t* hpart;     // workspace [B, Hq, items, kSelBuckets / 2]  per-item histograms (u16 pairs)
  uint32_t* tflag;     // workspace [B, Hq, items]  1 if the item holds an admissible pair
  uint32_t* ccount;    // workspace [B, Hq, nqb]  candidates of the order statistic per row
  int64_t* pick;       // workspace [B, Hq, 4]  (N, n, bucket, rank within bucket)
  double* cand;        // workspace [B, Hq, nqb, nkb]  candidate values, a segment per row
  int32_t* cpos;       // workspace [B, Hq, nqb, nkb]  their key blocks
  int32_t score_wgs;   // persistent workgroups of the score kernel (two per CU)
};

// One decode step's K/V rows into a W-slot ring cache (slot n_seen[b] % W) and the
// per-sequence cache offset min(n_seen[b], W - 1) that the split-KV decode then uses.
struct RingAppendArgs {
  const void* k_new;
  const void* v_new;
  int64_t n_sb, n_sh;  // element strides of k_new / v_new (batch, head)
  void* k_ring;
  void* v_ring;
  int64_t r_sb, r_sh, r_st;  // element strides of the rings (batch, head, slot)
  const int32_t* n_seen;     // [B]
  int32_t* cache_off_out;    // [B]
  int32_t B, Hkv, W, row_bytes, esz;
};

hipError_t launch_ring_append(const RingAppendArgs& r, hipStream_t s);

// Multi-head latent attention decode (bf16; latent width 512, rope width 64, per-head
// query/key width 128 and value width 128).  Rows rho = h * tq + t of sequence b.
constexpr int kMlaRank = 512, kMlaRope = 64, kMlaNope = 128, kMlaV = 128;
struct MlaArgs {
  const void* q_nope;
  int64_t qn_sb, qn_sh, qn_st;
  const void* q_rope;
  int64_t qr_sb, qr_sh, qr_st;
  const void* c_kv;
  int64_t c_sb, c_st;
  const void* k_rope;
  int64_t r_sb, r_st;
  const void* w_uk;  // [H, 512, 128]
  const void* w_uv;  // [H, 512, 128]
  void* o;
  int64_t o_sb, o_sh, o_st;
  const int32_t* cache_off;
  int32_t B, H, tq, tk;
  float scale_log2;
  void* q_lat;      // workspace bf16 [B, H*tq, 512]
  float* part_o;    // workspace f32 [B*H*tq, nsplit, 512]
  float* part_ml;   // workspace f32 [B*H*tq, nsplit, 2]
  float* o_lat;     // workspace f32 [B*H*tq, 512]  merged latent outputs
  uint32_t* queue;  // workspace: next work item of the split kernel (cleared by the absorb kernel)
  int32_t nsplit, split;
  int32_t n_waves;  // persistent split waves
};
// Token top-k sparse attention decode (bf16, head_dim 128, indexer width 128).
constexpr int kDsaIndexDim = 128, kDsaMaxIndexHeads = 64;
struct DsaArgs {
  AttnArgs at;          // q, k, v, o, strides, shape, cache_off, sink, scale, part/nsplit/split
  const void* qi;       // [B, Hi, tq, 128]
  int64_t qi_sb, qi_sh, qi_st;
  const void* ki;       // [B, tk, 128]
  int64_t ki_sb, ki_st;
  const float* wi;      // [B, Hi, tq]
  int32_t Hi, topk;
  float* scores;        // workspace [B, tq, tk]  fp32 indexer scores
  float* ebound;        // workspace [B, tq, tk]  E = u . |k| per token (bounds the fp32 score error)
  double* s64;          // workspace [B, tq, tk]  fp64 scores of the tokens near the threshold
  int32_t* band;        // workspace [B, tq, tk]  those tokens' indices (any order)
  int32_t* list;        // [B, tq, topk] kept token indices, ascending
  int32_t* count;       // [B, tq]
  int32_t idx_waves;    // workgroups of the indexer grid (one per CU; each scores an equal share of all blocks)
};
hipError_t launch_dsa_decode(const DsaArgs& a, hipStream_t s);

constexpr int kMlaMaxSplits = 256;  // splits per sequence the merge accepts
hipError_t launch_mla_decode(const MlaArgs& a, hipStream_t s);
hipError_t launch_prefill_bf16(const AttnArgs& a, hipStream_t s);
hipError_t launch_prefill_f32(const AttnArgs& a, hipStream_t s);
hipError_t launch_decode_bf16(const AttnArgs& a, hipStream_t s);
hipError_t launch_decode_f32(const AttnArgs& a, hipStream_t s);
hipError_t launch_decode_merge(const AttnArgs& a, bool out_bf16, hipStream_t s);
hipError_t launch_block_select(const SelectArgs& a, bool in_bf16, hipStream_t s);
hipError_t launch_list_from_mask(int64_t rows, int32_t n_kb, const uint8_t* mask, int32_t* list,
                                 hipStream_t s);

}  // namespace soc
