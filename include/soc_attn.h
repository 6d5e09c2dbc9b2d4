/*
 * soc_attn.h -- C ABI of the offset-causal attention library for AMD Instinct MI355X (gfx950).
 *
 * What is computed (all entry points)
 * -----------------------------------
 * Masked scaled-dot-product attention whose causal rule uses absolute positions
 * (sotaaz.com/post/attention-in-code, section "the one function every design uses",
 * functions attend and causal; the tilnote.io note on the Express framework, section
 * "causal attention is a position problem"):
 *
 *   off_b  = cache offset of sequence b (tokens already cached before the query block)
 *   Tk_b   = off_b + tq            (the block's own K/V rows are already in the cache)
 *   pos(r) = off_b + r             absolute position of query row r, 0 <= r < tq
 *   key j is visible to row r iff   j <= pos(r)
 *                              and  (window <= 0  or  j > pos(r) - window)
 *                              and  (no block list  or  key block j/bs is kept for
 *                                    query block r/bs of this head)
 *   s_j = scale * <q_r, k_j>;  o_r = sum_j e^{s_j} v_j / (sum_j e^{s_j} + [sink] e^{sink_h})
 *   over visible j; a row with no visible key and no sink is 0.
 *
 * Grouped-query sharing (same page, section 1): query head h reads stored KV head
 * h / (n_heads / n_kv); KV heads are never replicated.  The sink (same page, section 3)
 * is one float32 logit per query head, in the same units as s_j (after the scale),
 * that joins the softmax normaliser and has no value behind it.  The window keeps W
 * keys including the query's own (factory.pai-world.com "Attention Variants", sliding
 * window section, mask figure and build step 2).
 *
 * Layout and ownership
 * --------------------
 *  - Tensors are [batch, heads, tokens, head_dim] with head_dim contiguous; the other
 *    three strides are given in ELEMENTS (attn_strides_t).  K and V share one stride set.
 *  - q, k, v, o, sink, cache_off, block lists, masks, thresholds and workspaces are
 *    DEVICE pointers owned by the caller.  The library never allocates or frees memory.
 *  - bf16 path: head_dim = 128; every row start must be 16-byte aligned (pointers
 *    16-byte aligned, strides multiples of 8 elements).  f32 path: head_dim in
 *    {16, 32, 64, 128}, rows 16-byte aligned.
 *  - Every call is asynchronous on the given stream; it returns once work is queued.
 *  - Calls are re-entrant; the library keeps no mutable global state except a
 *    thread-local error message and lazily read device properties.
 *
 * Errors
 * ------
 *  Non-zero returns are negative ATTN_E_* codes; attn_last_error() then returns a
 *  thread-local message describing the failure.  Argument errors are detected before
 *  any device work is queued.  Device-side preconditions (0 <= off_b, off_b + tq <= tk,
 *  block-list indices in range) are the caller's; with the environment variable
 *  ATTN_DEBUG=1 the library checks cache offsets on the host (one synchronous copy)
 *  and synchronises after each launch to report launch failures.
 */
#ifndef SOC_ATTN_H
#define SOC_ATTN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { ATTN_BF16 = 0, ATTN_F32 = 1 } attn_dtype_t;

enum {
  ATTN_OK = 0,
  ATTN_E_INVAL = -1,       /* bad argument: null pointer, sizes, alignment, n_heads % n_kv != 0, tq > tk */
  ATTN_E_UNSUPPORTED = -2, /* (dtype, head_dim, block_size, rows per KV group) combination not built */
  ATTN_E_WORKSPACE = -3,   /* workspace missing or smaller than the matching *_workspace_bytes() */
  ATTN_E_HIP = -4          /* the HIP runtime reported an error while queueing work */
};

/* Strides in elements of the batch, head and token axes (head_dim is contiguous). */
typedef struct {
  int64_t b, h, t;
} attn_strides_t;

/* tk = K/V rows addressable per sequence: the uniform key count when cache_off is NULL
 * (then off_b = tk - tq for every b), otherwise the cache capacity. */
typedef struct {
  int32_t batch, n_heads, n_kv, head_dim, tq, tk;
  attn_dtype_t dtype;
} attn_shape_t;

/*
 * attn_prefill -- attention for a block of tq query rows per sequence (prefill, chunked
 * prefill or decode) against the cache.
 *
 *  q          [batch, n_heads, tq, head_dim]   (dtype)
 *  k, v       [batch, n_kv, tk, head_dim]      (dtype), strides kv_strides (bf16: the
 *             token stride must be nonzero, else ATTN_E_UNSUPPORTED)
 *  o          [batch, n_heads, tq, head_dim]   output (dtype), written for every row
 *  cache_off  device int32 [batch], or NULL (off_b = tk - tq)
 *  window     <= 0: no window; W > 0 keeps keys pos-W < j <= pos.  Key tiles entirely
 *             outside the window or beyond pos are never read.
 *  sink       device float32 [n_heads] or NULL (a -inf entry behaves as no sink)
 *  scale      <= 0 means 1/sqrt(head_dim)
 *  block_mask NULL, or device uint8 [batch, n_heads, nQB, nKB] with nQB = ceil(tq /
 *             block_size), nKB = ceil(tk / block_size): a nonzero entry keeps key block kb
 *             for query block qb of head h (the attend(q, k, v, mask, sink) mask of
 *             sotaaz.com/post/attention-in-code, "the one function every design uses", at
 *             block granularity).  Query block qb covers rows [qb*bs, (qb+1)*bs) of the tq
 *             block; key block kb covers absolute keys [kb*bs, (kb+1)*bs).  The causal and
 *             window rules still apply inside kept blocks; unkept key blocks are never read
 *             (patty.io RBS-Attention review, section on regular block-sparse execution).
 *             The kernel walks each mask row itself: no workspace is needed.
 *  block_list NULL, or the same selection as kept-block lists: device int32 [batch, n_heads,
 *             nQB, 1 + nKB], entry 0 of each (b, h, qb) row the count n of kept key blocks,
 *             entries 1..n the kept key block indices in ascending order (as written by
 *             attn_block_select).  At most one of block_mask and block_list may be non-NULL
 *             (both: ATTN_E_INVAL); with neither the prefill is dense.
 *  block_size ignored when both are NULL; bf16 path requires 128.
 */
int attn_prefill(const attn_shape_t* shape, const void* q, attn_strides_t q_strides, const void* k,
                 const void* v, attn_strides_t kv_strides, void* o, attn_strides_t o_strides,
                 const int32_t* cache_off, int32_t window, const float* sink, float scale,
                 const uint8_t* block_mask, const int32_t* block_list, int32_t block_size,
                 hipStream_t stream);

/*
 * attn_decode_workspace_bytes -- bytes of device workspace attn_decode needs for this
 * shape and split size (split_tokens <= 0 selects the default split).  Returns 0 for
 * an invalid shape.
 */
size_t attn_decode_workspace_bytes(const attn_shape_t* shape, int32_t split_tokens);

/*
 * attn_decode -- split-KV attention for a few query rows per sequence (decode steps or
 * short speculative blocks).  Same arguments and semantics as attn_prefill without a
 * block list.  The keys of each sequence are cut into splits of split_tokens; one pass
 * computes an unnormalised partial (running max, sum, weighted V sum) per split and
 * query row in float32 into the workspace, a second pass merges the partials with the
 * sink (added exactly once per row) and writes o.  Each K/V element is read once per
 * call: all n_heads / n_kv query heads of a group are served from one read.
 *  bf16 path: (n_heads / n_kv) * tq <= 32.  f32 path: any tq.
 *  workspace  device memory of at least attn_decode_workspace_bytes(shape, split_tokens)
 *             bytes (256-byte aligned); its contents on entry do not matter.
 */
int attn_decode(const attn_shape_t* shape, const void* q, attn_strides_t q_strides, const void* k,
                const void* v, attn_strides_t kv_strides, void* o, attn_strides_t o_strides,
                const int32_t* cache_off, int32_t window, const float* sink, float scale,
                void* workspace, size_t workspace_bytes, int32_t split_tokens, hipStream_t stream);

/*
 * attn_decode_noalloc -- attn_decode for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation, kernels and arguments as attn_decode, without the workspace
 * arguments.  The per-split partials go to a scratch array the library holds in device
 * memory, one per GPU it runs on, of attn_decode_noalloc_max_scratch_bytes() bytes
 * (32 MiB), kept until the process ends.  Nothing is allocated or freed by the call.
 *  - Shapes whose workspace (attn_decode_workspace_bytes) exceeds that size are rejected
 *    with ATTN_E_WORKSPACE; use attn_decode with a caller workspace for those.
 *  - All calls on one GPU share its array, which keeps the last call's contents (no part
 *    of it needs to start at zero).  Calls that overlap on one GPU (concurrent streams or
 *    threads) race on it: serialise them, e.g. on one stream.
 *  - ATTN_DEBUG's host check of cache_off is not made (it copies to host memory).
 */
int attn_decode_noalloc(const attn_shape_t* shape, const void* q, attn_strides_t q_strides, const void* k,
                        const void* v, attn_strides_t kv_strides, void* o, attn_strides_t o_strides,
                        const int32_t* cache_off, int32_t window, const float* sink, float scale,
                        int32_t split_tokens, hipStream_t stream);

/* attn_decode_noalloc_max_scratch_bytes -- size of attn_decode_noalloc's per-GPU scratch. */
size_t attn_decode_noalloc_max_scratch_bytes(void);

/*
 * attn_ring_decode_workspace_bytes -- bytes of device workspace attn_ring_decode needs
 * (split_tokens <= 0 selects the default split).  Returns 0 for an invalid shape.
 */
size_t attn_ring_decode_workspace_bytes(const attn_shape_t* shape, int32_t split_tokens);

/*
 * attn_ring_decode -- one decode step of sliding-window attention over a W-slot ring
 * cache, appending the step's K/V itself (sotaaz.com/post/attention-in-code, section 2,
 * the ring-buffer cache: token n's K/V go to slot n mod W over the oldest entry, and the
 * step attends to the filled slots in any order, which a softmax cannot tell apart).
 *
 *  shape      tq = 1; tk = W, the ring's slots per (sequence, KV head).
 *  q          [batch, n_heads, 1, head_dim]                 (dtype)
 *  k_new, v_new [batch, n_kv, 1, head_dim], strides new_strides: the step's K/V rows.
 *  k_ring, v_ring [batch, n_kv, W, head_dim], strides ring_strides; updated in place:
 *             slot n_seen[b] % W of every KV head of sequence b receives k_new / v_new.
 *  n_seen     device int32 [batch], >= 0: tokens of sequence b written to the ring
 *             before this step.  Read only; the caller advances it after the step.
 *  o          [batch, n_heads, 1, head_dim] output: attention of q over the
 *             min(n_seen[b] + 1, W) filled slots, the new token included.  This equals
 *             attn_prefill with window W at position n_seen[b] over the whole history.
 *  sink, scale as attn_prefill (the sink joins the normaliser once per row).
 *  workspace  at least attn_ring_decode_workspace_bytes(shape, split_tokens) bytes.
 * bf16: the split-KV decode of attn_decode runs over the ring itself; the split that holds
 * slot n_seen[b] % W attends over the new row in place of the slot's old contents and writes
 * the new row into the slot when it has finished reading.  With at most two splits per ring
 * (the default for W up to twice the split size) both splits of a (sequence, KV head) run in
 * one workgroup and merge there: one kernel, the workspace unused.  With more splits the
 * split kernel writes partials to the workspace and the merge kernel follows.  fp32: a small
 * append kernel writes the rows first, then the split-KV decode and merge run.  Same dtype
 * and head_dim rules as attn_decode; bf16 needs n_heads / n_kv <= 32.
 */
int attn_ring_decode(const attn_shape_t* shape, const void* q, attn_strides_t q_strides, const void* k_new,
                     const void* v_new, attn_strides_t new_strides, void* k_ring, void* v_ring,
                     attn_strides_t ring_strides, void* o, attn_strides_t o_strides, const int32_t* n_seen,
                     const float* sink, float scale, void* workspace, size_t workspace_bytes, int32_t split_tokens,
                     hipStream_t stream);

/*
 * Multi-head latent attention (sotaaz.com/post/attention-in-code, section 4).  The cache
 * holds per token a latent c_kv of width kv_rank and one key k_rope of width rope_dim
 * shared by all heads.  Head h's key is [c_kv @ w_uk[h], k_rope] and its value
 * c_kv @ w_uv[h]; the query is [q_nope, q_rope].  Built: bf16, kv_rank 512, rope_dim 64,
 * nope_dim 128, v_dim 128 (the DeepSeek-V2-Lite layout the page describes).
 */
typedef struct {
  int32_t batch, n_heads, tq, tk; /* tk = cache rows addressable per sequence */
  int32_t kv_rank, rope_dim, nope_dim, v_dim;
  attn_dtype_t dtype;
} attn_mla_shape_t;

/*
 * attn_mla_decode_workspace_bytes -- device workspace for attn_mla_decode (split_tokens
 * <= 0 selects the default split).  Returns 0 for an invalid or unsupported shape.
 */
size_t attn_mla_decode_workspace_bytes(const attn_mla_shape_t* shape, int32_t split_tokens);

/*
 * attn_mla_decode -- MLA for a few query tokens per sequence against the latent cache,
 * in absorbed form: no per-head key or value is built; each step reads kv_rank + rope_dim
 * numbers per cached token, shared by all heads.
 *
 *  q_nope     [batch, n_heads, tq, nope_dim], q_rope [batch, n_heads, tq, rope_dim]
 *  c_kv       [batch, tk, kv_rank], k_rope [batch, tk, rope_dim]: strides in elements with
 *             .b (sequence) and .t (token); .h is ignored.  May be views of one
 *             [batch, tk, kv_rank + rope_dim] buffer.
 *  w_uk       [n_heads, kv_rank, nope_dim], w_uv [n_heads, kv_rank, v_dim], contiguous
 *  o          [batch, n_heads, tq, v_dim] output
 *  cache_off  device int32 [batch] or NULL (off_b = tk - tq): query token t of sequence b
 *             sits at position off_b + t and sees cached tokens j <= off_b + t.
 *  scale      <= 0 means 1/sqrt(nope_dim + rope_dim).
 *  workspace  at least attn_mla_decode_workspace_bytes(shape, split_tokens) bytes.
 *  Steps: q_lat = w_uk[h] q_nope (rounded to bf16); split-KV attention of [q_lat, q_rope]
 *  over [c_kv, k_rope] averaging c_kv, in fp32; log-sum-exp merge; o = w_uv[h]^T o_lat.
 *  At most 256 splits per sequence (ceil(tk / split_tokens) <= 256).
 */
int attn_mla_decode(const attn_mla_shape_t* shape, const void* q_nope, attn_strides_t qn_strides,
                    const void* q_rope, attn_strides_t qr_strides, const void* c_kv, attn_strides_t ckv_strides,
                    const void* k_rope, attn_strides_t kr_strides, const void* w_uk, const void* w_uv, void* o,
                    attn_strides_t o_strides, const int32_t* cache_off, float scale, void* workspace,
                    size_t workspace_bytes, int32_t split_tokens, hipStream_t stream);

/*
 * attn_dsa_decode_workspace_bytes -- device workspace for attn_dsa_decode (split_tokens
 * <= 0 selects the default).  Returns 0 for an invalid shape.
 */
size_t attn_dsa_decode_workspace_bytes(const attn_shape_t* shape, int32_t topk, int32_t split_tokens);

/*
 * attn_dsa_decode -- token top-k sparse attention for a few query tokens per sequence
 * (sotaaz.com/post/attention-in-code, section 5): an indexer scores every token a query
 * token may see,
 *     score(t, s) = sum over indexer heads j of wi[j, t] * relu(qi[j, t] . ki[s]),
 * and every head of that query token attends only over its top-k visible tokens (all of
 * them if fewer than k are visible; equal scores go to the lower token index).  The cache
 * stays whole; only the kept rows of K and V are read.
 *
 *  q, k, v, o, cache_off, sink, scale: as attn_decode (bf16, head_dim 128; k/v hold tk rows
 *             per sequence; query token t of sequence b sits at position off_b + t).
 *  qi         [batch, index_heads, tq, 128] bf16;  ki [batch, tk, 128] bf16 (strides .b, .t;
 *             .h ignored);  wi device float32 [batch, index_heads, tq], contiguous.
 *  index_heads a multiple of 16, at most 64;  topk >= 1.
 *  kept_list  device int32 [batch, tq, topk] or NULL: the kept token indices of each query
 *             token in ascending order (entries past kept_count unspecified).
 *  kept_count device int32 [batch, tq] or NULL.
 *  workspace  at least attn_dsa_decode_workspace_bytes(shape, topk, split_tokens) bytes.
 *  split_tokens: kept-list entries per split, at most 1024.  bf16 needs n_heads / n_kv <= 32.
 */
int attn_dsa_decode(const attn_shape_t* shape, const void* q, attn_strides_t q_strides, const void* k, const void* v,
                    attn_strides_t kv_strides, void* o, attn_strides_t o_strides, const int32_t* cache_off,
                    const float* sink, float scale, const void* qi, attn_strides_t qi_strides, const void* ki,
                    attn_strides_t ki_strides, const float* wi, int32_t index_heads, int32_t topk,
                    int32_t* kept_list, int32_t* kept_count, void* workspace, size_t workspace_bytes,
                    int32_t split_tokens, hipStream_t stream);

/*
 * attn_block_select_workspace_bytes -- device workspace for attn_block_select.
 */
size_t attn_block_select_workspace_bytes(const attn_shape_t* shape, int32_t block_size);

/*
 * attn_block_select -- block mask for block-sparse prefill: a mean-centroid score OR'd
 * with a max-key-radius rescue score (patty.io review of RBS-Attention: sections on the
 * centroid score, mean dilution, the radius signal and the two independently thresholded
 * branches).  All arithmetic is float64 from exact bf16/f32 -> f64 conversion.
 *
 *  qmean[b,h,qb]   = mean of q rows [qb*bs, min((qb+1)*bs, tq))
 *  c[b,kv,kb]      = mean of k rows [kb*bs, min((kb+1)*bs, Tk_b))
 *  rad2[b,kv,kb]   = max over those rows of |k_j - c|^2
 *  (qb, kb) admissible iff it holds at least one (row, key) pair the position/window
 *  rule allows;  s1 = <qmean, c> on admissible pairs (unscaled).
 *  Thresholds (order statistics, per prompt and head): with population size N and
 *  n = floor(keep * N + 0.5), tau = the (n+1)-th largest value (-inf when n >= N).
 *    tau_mean[b,h]    over the admissible s1 of (b, h)        (keep = keep_mean)
 *    tau_radius[b,kv] over rad2 of the key blocks of (b, kv)  (keep = keep_radius)
 *  mask[b,h,qb,kb] = admissible and (s1 > tau_mean[b,h] or rad2[b,h/g,kb] > tau_radius[b,h/g])
 *
 *  q [batch, n_heads, tq, d], k [batch, n_kv, tk, d] (dtype); cache_off as attn_prefill.
 *  keep_mean, keep_radius  fractions in [0, 1]; a negative value means the matching
 *             tau array is an INPUT (caller's absolute threshold) instead of an output.
 *  tau_mean   device double [batch, n_heads];  tau_radius device double [batch, n_kv]
 *  block_mask device uint8 [batch, n_heads, ceil(tq/bs), ceil(tk/bs)] output (0/1;
 *             blocks at or beyond Tk_b are 0)
 *  block_list device int32 [batch, n_heads, ceil(tq/bs), 1 + ceil(tk/bs)] output or NULL,
 *             in the format attn_prefill reads.
 *  workspace  at least attn_block_select_workspace_bytes(shape, block_size) bytes.
 *  block_size >= 1 (the bf16 block-sparse prefill consumes block_size = 128).
 */
int attn_block_select(const attn_shape_t* shape, const void* q, attn_strides_t q_strides, const void* k,
                      attn_strides_t k_strides, const int32_t* cache_off, int32_t window, int32_t block_size,
                      double keep_mean, double keep_radius, double* tau_mean, double* tau_radius,
                      uint8_t* block_mask, int32_t* block_list, void* workspace, size_t workspace_bytes,
                      hipStream_t stream);

/*
 * attn_block_sparse_prefill_workspace_bytes -- device workspace attn_block_sparse_prefill needs
 * (the block selection's); 0 for an invalid shape.
 */
size_t attn_block_sparse_prefill_workspace_bytes(const attn_shape_t* shape, int32_t block_size);

/*
 * attn_block_sparse_prefill -- block selection and block-sparse prefill in one call (patty.io
 * RBS-Attention review: the mean-centroid and max-radius sieves chosen per prompt and head, and
 * the regular block-sparse execution they feed, section on how regular sparsity persuades the
 * GPU).  Computes exactly attn_block_select's mask followed by attn_prefill over it: the
 * selection's last pass writes the byte mask (into the workspace, or block_mask_out) and the
 * prefill walks each row's marked key blocks straight from it; no kept list is built.  With a
 * cache offset this is the query-chunked selection of a chunked prefill: query block qb covers rows
 * [qb*bs, (qb+1)*bs) of the tq-row chunk, key blocks are absolute.
 *  q, k, v, o, cache_off, window, sink, scale: as attn_prefill (bf16: head_dim 128).
 *  block_size, keep_mean, keep_radius, tau_mean, tau_radius: as attn_block_select (bf16:
 *             block_size 128); the thresholds are written (or read, with a negative keep
 *             fraction) as there.
 *  block_mask_out  NULL, or device uint8 [batch, n_heads, nQB, nKB] to receive the mask (the
 *             prefill then reads it from there instead of the workspace).
 *  workspace  at least attn_block_sparse_prefill_workspace_bytes(shape, block_size) bytes.
 */
int attn_block_sparse_prefill(const attn_shape_t* shape, const void* q, attn_strides_t q_strides, const void* k,
                              const void* v, attn_strides_t kv_strides, void* o, attn_strides_t o_strides,
                              const int32_t* cache_off, int32_t window, const float* sink, float scale,
                              int32_t block_size, double keep_mean, double keep_radius, double* tau_mean,
                              double* tau_radius, uint8_t* block_mask_out, void* workspace,
                              size_t workspace_bytes, hipStream_t stream);

/*
 * attn_block_list_from_mask -- compact a caller-made block mask
 * (device uint8 [rows, n_kb], nonzero = kept, rows = batch*n_heads*nQB) into the
 * block-list format attn_prefill reads (device int32 [rows, 1 + n_kb]).
 */
int attn_block_list_from_mask(int64_t rows, int32_t n_kb, const uint8_t* block_mask, int32_t* block_list,
                              hipStream_t stream);

/* Thread-local description of the last non-zero return on this thread ("" if none). */
const char* attn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SOC_ATTN_H */
