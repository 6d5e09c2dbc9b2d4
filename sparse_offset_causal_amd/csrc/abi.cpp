// C-ABI entry points: argument validation, variant selection, workspace carving, launches.
// Every argument error is detected here, before any device work is queued.

#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <mutex>
#include <string>
#include <vector>

#include "internal.h"
#include "soc_attn.h"

namespace {

thread_local std::string g_err;

int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

bool debug_mode() {
  static const bool on = [] {
    const char* e = std::getenv("ATTN_DEBUG");
    return e && e[0] == '1';
  }();
  return on;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(ATTN_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t elem_size(attn_dtype_t t) { return t == ATTN_BF16 ? 2 : 4; }

bool strides_ok(const attn_strides_t& s, size_t esz) {
  const int64_t m = (int64_t)(16 / esz);
  return s.b >= 0 && s.h >= 0 && s.t >= 0 && s.b % m == 0 && s.h % m == 0 && s.t % m == 0;
}

// Common shape checks.  Returns ATTN_OK or an error code (message set).
int check_shape(const attn_shape_t* s) {
  if (!s) return fail(ATTN_E_INVAL, "shape is NULL");
  if (s->batch < 0 || s->n_heads < 1 || s->n_kv < 1 || s->head_dim < 1 || s->tq < 0 || s->tk < 0)
    return fail(ATTN_E_INVAL, "shape has a negative or zero size");
  if (s->n_heads % s->n_kv != 0) return fail(ATTN_E_INVAL, "n_heads must be a multiple of n_kv");
  if (s->tq > s->tk) return fail(ATTN_E_INVAL, "tq > tk: the query block's keys must already be in the cache");
  if (s->tk > (1 << 30)) return fail(ATTN_E_INVAL, "tk above 2^30 is not supported");
  if (s->dtype != ATTN_BF16 && s->dtype != ATTN_F32) return fail(ATTN_E_UNSUPPORTED, "unknown dtype");
  return ATTN_OK;
}

int check_attn_dtype(const attn_shape_t* s) {
  if (s->dtype == ATTN_BF16 && s->head_dim != 128)
    return fail(ATTN_E_UNSUPPORTED, "bf16 attention is built for head_dim 128 only");
  if (s->dtype == ATTN_F32 && s->head_dim != 16 && s->head_dim != 32 && s->head_dim != 64 && s->head_dim != 128)
    return fail(ATTN_E_UNSUPPORTED, "f32 attention supports head_dim 16, 32, 64 or 128");
  return ATTN_OK;
}

int check_tensors(const attn_shape_t* s, const void* q, attn_strides_t qs, const void* k, const void* v,
                  attn_strides_t kvs, const void* o, attn_strides_t os) {
  if (!q || !k || !v || !o) return fail(ATTN_E_INVAL, "q, k, v and o must be non-NULL device pointers");
  const size_t esz = elem_size(s->dtype);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(ATTN_E_INVAL, "q, k, v and o must be 16-byte aligned");
  if (!strides_ok(qs, esz) || !strides_ok(kvs, esz) || !strides_ok(os, esz))
    return fail(ATTN_E_INVAL, "strides must be non-negative multiples of 16 bytes (in elements)");
  // the bf16 kernels address K/V through buffer ranges of (rows x token stride) bytes
  if (s->dtype == ATTN_BF16 && kvs.t == 0)
    return fail(ATTN_E_UNSUPPORTED, "bf16 k/v need a nonzero token stride (one row per token)");
  return ATTN_OK;
}

int check_offsets_debug(const attn_shape_t* s, const int32_t* cache_off, hipStream_t stream) {
  if (!debug_mode() || !cache_off || s->batch == 0) return ATTN_OK;
  std::vector<int32_t> h(s->batch);
  hipError_t e = hipMemcpyAsync(h.data(), cache_off, sizeof(int32_t) * s->batch, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "ATTN_DEBUG: reading cache_off");
  for (int b = 0; b < s->batch; ++b)
    if (h[b] < 0 || (int64_t)h[b] + s->tq > s->tk)
      return fail(ATTN_E_INVAL, "ATTN_DEBUG: cache_off[" + std::to_string(b) + "] = " + std::to_string(h[b]) +
                                    " violates 0 <= off and off + tq <= tk");
  return ATTN_OK;
}

int finish(hipError_t e, hipStream_t stream, const char* what) {
  if (e != hipSuccess) return hip_fail(e, what);
  if (debug_mode()) {
    e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_fail(e, what);
  }
  g_err.clear();
  return ATTN_OK;
}

soc::AttnArgs make_args(const attn_shape_t* s, const void* q, attn_strides_t qs, const void* k, const void* v,
                        attn_strides_t kvs, void* o, attn_strides_t os, const int32_t* cache_off, int32_t window,
                        const float* sink, float scale) {
  soc::AttnArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.q_sb = qs.b; a.q_sh = qs.h; a.q_st = qs.t;
  a.kv_sb = kvs.b; a.kv_sh = kvs.h; a.kv_st = kvs.t;
  a.o_sb = os.b; a.o_sh = os.h; a.o_st = os.t;
  a.B = s->batch;
  a.Hq = s->n_heads;
  a.Hkv = s->n_kv;
  a.g = s->n_heads / s->n_kv;
  a.tq = s->tq;
  a.tk = s->tk;
  a.d = s->head_dim;
  a.cache_off = cache_off;
  a.window = window;
  a.sink = sink;
  const double sc = scale > 0.f ? (double)scale : 1.0 / std::sqrt((double)s->head_dim);
  a.scale_log2 = (float)(sc * 1.4426950408889634);
  return a;
}

// Keys per decode split: long splits amortise each wave's pipeline start-up; shorter ones
// keep at least ~1024 workgroups (two per CU slot, four rounds) when the batch is small.
int default_split(const attn_shape_t* s) {
  int split = 2048;
  while (split > 256 && (int64_t)s->batch * s->n_kv * ((s->tk + split - 1) / split) < 1024) split /= 2;
  return split;
}

size_t round_up(size_t x, size_t m) { return (x + m - 1) / m * m; }

struct SelectLayout {
  int nqb, nkb;
  size_t qmean, cT, rad2, score, norm2, nmax, hpart, tflag, ccount, pick, cand, cpos, wmask, total;  // byte offsets
};

SelectLayout select_layout(const attn_shape_t* s, int bs) {
  SelectLayout L{};
  L.nqb = (s->tq + bs - 1) / bs;
  L.nkb = (s->tk + bs - 1) / bs;
  const size_t d8 = sizeof(double);
  size_t off = 0;
  L.qmean = off;
  off = round_up(off + d8 * s->batch * s->n_heads * L.nqb * s->head_dim, 256);
  L.cT = off;
  off = round_up(off + d8 * s->batch * s->n_kv * s->head_dim * L.nkb, 256);
  L.rad2 = off;
  off = round_up(off + d8 * s->batch * s->n_kv * L.nkb, 256);
  L.score = off;
  const size_t bh = (size_t)s->batch * s->n_heads;
  off = round_up(off + d8 * bh * L.nqb * L.nkb, 256);
  L.norm2 = off;
  off = round_up(off + d8 * (bh * L.nqb + (size_t)s->batch * s->n_kv * L.nkb), 256);
  L.nmax = off;
  off = round_up(off + d8 * (bh + (size_t)s->batch * s->n_kv), 256);
  const size_t items = (size_t)soc::sel_items_per_head(L.nqb, L.nkb);
  L.hpart = off;
  off = round_up(off + sizeof(uint16_t) * bh * items * soc::kSelBuckets, 256);
  L.tflag = off;
  off = round_up(off + sizeof(uint32_t) * bh * items, 256);
  L.ccount = off;
  off = round_up(off + sizeof(uint32_t) * bh * L.nqb, 256);
  L.pick = off;
  off = round_up(off + sizeof(int64_t) * bh * 4, 256);
  L.cand = off;
  off = round_up(off + d8 * bh * L.nqb * L.nkb, 256);
  L.cpos = off;
  off = round_up(off + sizeof(int32_t) * bh * L.nqb * L.nkb, 256);
  L.wmask = off;  // the mask, when the caller takes none (the fused call)
  off = round_up(off + bh * L.nqb * L.nkb, 256);
  L.total = off;
  return L;
}

int check_mla_shape(const attn_mla_shape_t* s) {
  if (!s) return fail(ATTN_E_INVAL, "shape is NULL");
  if (s->batch < 0 || s->n_heads < 1 || s->tq < 0 || s->tk < 0)
    return fail(ATTN_E_INVAL, "batch, tq, tk must be >= 0 and n_heads >= 1");
  if (s->tq > s->tk) return fail(ATTN_E_INVAL, "tq > tk: the query tokens must already be in the cache");
  if (s->dtype != ATTN_BF16 || s->kv_rank != soc::kMlaRank || s->rope_dim != soc::kMlaRope ||
      s->nope_dim != soc::kMlaNope || s->v_dim != soc::kMlaV)
    return fail(ATTN_E_UNSUPPORTED, "MLA decode is built for bf16 with kv_rank 512, rope_dim 64, nope_dim 128, v_dim 128");
  return ATTN_OK;
}

int mla_default_split(const attn_mla_shape_t* s) {
  // work items of 1024 tokens: 512 measured 4-5 % slower on the batch-64 workload (more
  // partials for the merge, more item starts), 2048 slower again (about one item per
  // persistent workgroup plus a short second round); longer splits only where 256 per
  // sequence would not cover the cache
  int split = 1024;
  while ((int64_t)(s->tk + split - 1) / split > soc::kMlaMaxSplits) split *= 2;
  return split;
}

int device_cus() {
  static thread_local int cached_dev = -1, cached_cus = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (dev != cached_dev) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached_dev = dev;
    cached_cus = n;
  }
  return cached_cus;
}

struct MlaLayout {
  size_t q_lat, part_o, part_ml, o_lat, queue, total;
  int split, nsplit;
};

MlaLayout mla_layout(const attn_mla_shape_t* s, int32_t split_tokens) {
  MlaLayout L{};
  L.split = split_tokens > 0 ? split_tokens : mla_default_split(s);
  L.nsplit = s->tk > 0 ? (s->tk + L.split - 1) / L.split : 1;
  const size_t rows = (size_t)s->batch * s->n_heads * s->tq;
  size_t off = 0;
  L.q_lat = off;
  off = round_up(off + rows * soc::kMlaRank * 2, 256);
  L.part_o = off;
  off = round_up(off + rows * L.nsplit * soc::kMlaRank * sizeof(float), 256);
  L.part_ml = off;
  off = round_up(off + rows * L.nsplit * 2 * sizeof(float), 256);
  L.o_lat = off;
  off = round_up(off + rows * soc::kMlaRank * sizeof(float), 256);
  L.queue = off;
  off = round_up(off + sizeof(uint32_t), 256);
  L.total = off;
  return L;
}

struct DsaLayout {
  size_t part, scores, ebound, s64, band, list, count, total;
  int split, nsplit;
};

DsaLayout dsa_layout(const attn_shape_t* s, int topk, int32_t split_tokens) {
  DsaLayout L{};
  // default: splits of 1024 kept entries when that still gives every CU four split waves
  // (batch 64, top 2048: 0.209 against 0.214 ms per step for 256), else 256
  if (split_tokens > 0) {
    L.split = split_tokens;
  } else {
    const int64_t kv_rows = (int64_t)s->batch * s->n_kv * s->tq;
    L.split = kv_rows * ((topk + 1023) / 1024) >= 4 * (int64_t)device_cus() ? 1024 : 256;
  }
  L.nsplit = topk > 0 ? (topk + L.split - 1) / L.split : 1;
  const size_t rows = (size_t)s->batch * s->n_heads * s->tq;
  const size_t qrows = (size_t)s->batch * s->tq;
  size_t off = 0;
  L.part = off;
  off = round_up(off + rows * L.nsplit * (s->head_dim + 2) * sizeof(float), 256);
  L.scores = off;
  off = round_up(off + qrows * (size_t)s->tk * sizeof(float), 256);
  L.ebound = off;
  off = round_up(off + qrows * (size_t)s->tk * sizeof(float), 256);
  L.s64 = off;
  off = round_up(off + qrows * (size_t)s->tk * sizeof(double), 256);
  L.band = off;
  off = round_up(off + qrows * (size_t)s->tk * sizeof(int32_t), 256);
  L.list = off;
  off = round_up(off + qrows * (size_t)(topk > 0 ? topk : 1) * sizeof(int32_t), 256);
  L.count = off;
  off = round_up(off + qrows * sizeof(int32_t), 256);
  L.total = off;
  return L;
}

}  // namespace

extern "C" {

const char* attn_last_error(void) { return g_err.c_str(); }

int attn_prefill(const attn_shape_t* shape, const void* q, attn_strides_t q_strides, const void* k, const void* v,
                 attn_strides_t kv_strides, void* o, attn_strides_t o_strides, const int32_t* cache_off,
                 int32_t window, const float* sink, float scale, const uint8_t* block_mask,
                 const int32_t* block_list, int32_t block_size, hipStream_t stream) {
  int rc = check_shape(shape);
  if (rc) return rc;
  if ((rc = check_attn_dtype(shape))) return rc;
  if (shape->tq == 0 || shape->batch == 0) {
    g_err.clear();
    return ATTN_OK;
  }
  if ((rc = check_tensors(shape, q, q_strides, k, v, kv_strides, o, o_strides))) return rc;
  if (block_mask && block_list) return fail(ATTN_E_INVAL, "pass a block mask or a block list, not both");
  if (block_list || block_mask) {
    if (block_size < 1) return fail(ATTN_E_INVAL, "block_size must be >= 1 with a block mask or list");
    if (shape->dtype == ATTN_BF16 && block_size != 128)
      return fail(ATTN_E_UNSUPPORTED, "the bf16 block-sparse prefill needs block_size 128");
  }
  const int64_t nqt = (shape->tq + 127) / 128;
  if (nqt * shape->batch * shape->n_heads >= (int64_t)1 << 31) return fail(ATTN_E_INVAL, "problem too large for one grid");
  if (shape->dtype == ATTN_BF16 && (int64_t)shape->tk * kv_strides.t * 2 > (int64_t)0xffffffff)
    return fail(ATTN_E_UNSUPPORTED, "one (sequence, KV head) cache slice spans more than 4 GiB (tk * token stride)");
  if ((rc = check_offsets_debug(shape, cache_off, stream))) return rc;

  soc::AttnArgs a = make_args(shape, q, q_strides, k, v, kv_strides, o, o_strides, cache_off, window, sink, scale);
  if (block_list || block_mask) {
    a.block_list = block_list;
    a.block_mask = block_mask;
    a.block_size = block_size;
    a.n_qb = (shape->tq + block_size - 1) / block_size;
    a.mask_stride = (shape->tk + block_size - 1) / block_size;
    a.list_stride = 1 + a.mask_stride;
  }
  const hipError_t e = shape->dtype == ATTN_BF16 ? soc::launch_prefill_bf16(a, stream) : soc::launch_prefill_f32(a, stream);
  return finish(e, stream, "attn_prefill launch");
}

size_t attn_decode_workspace_bytes(const attn_shape_t* shape, int32_t split_tokens) {
  if (check_shape(shape) != ATTN_OK) return 0;
  const int split = split_tokens > 0 ? split_tokens : default_split(shape);
  const size_t nsplit = shape->tk > 0 ? (size_t)((shape->tk + split - 1) / split) : 1;
  const size_t rows = (size_t)shape->batch * shape->n_heads * shape->tq;
  return round_up(rows * nsplit * (shape->head_dim + 2) * sizeof(float), 256);
}

}  // extern "C"

namespace {

// Scratch of attn_decode_noalloc: the decode workspace (per-split partials) for callers that
// cannot allocate.  Each device the library runs on holds its own copy of the array until
// the process ends; host code reaches it only through the address hipGetSymbolAddress
// returns for the current device (the array's name is a host-side stand-in).
constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Address of the current device's scratch array, looked up once per device.
int noalloc_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "attn_decode_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(ATTN_E_UNSUPPORTED, "attn_decode_noalloc: device index above 63");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return hip_fail(e, "attn_decode_noalloc: hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return ATTN_OK;
}

int decode_impl(const attn_shape_t* shape, const void* q, attn_strides_t q_strides, const void* k, const void* v,
                attn_strides_t kv_strides, void* o, attn_strides_t o_strides, const int32_t* cache_off,
                int32_t window, const float* sink, float scale, void* workspace, size_t workspace_bytes,
                int32_t split_tokens, hipStream_t stream, bool noalloc) {
  int rc = check_shape(shape);
  if (rc) return rc;
  if ((rc = check_attn_dtype(shape))) return rc;
  if (shape->tq == 0 || shape->batch == 0) {
    g_err.clear();
    return ATTN_OK;
  }
  if ((rc = check_tensors(shape, q, q_strides, k, v, kv_strides, o, o_strides))) return rc;
  if (shape->dtype == ATTN_BF16 && (int64_t)shape->tk * kv_strides.t * 2 > (int64_t)0xffffffff)
    return fail(ATTN_E_UNSUPPORTED, "one (sequence, KV head) cache slice spans more than 4 GiB (tk * token stride)");
  if (shape->dtype == ATTN_BF16 && (shape->n_heads / shape->n_kv) * shape->tq > 32)
    return fail(ATTN_E_UNSUPPORTED, "bf16 decode serves at most 32 query rows per KV head ((n_heads/n_kv)*tq <= 32)");
  const int split = split_tokens > 0 ? split_tokens : default_split(shape);
  const int64_t nsplit = (shape->tk + split - 1) / split;
  const size_t need = attn_decode_workspace_bytes(shape, split);
  if (noalloc) {
    if (need > kNoAllocScratchBytes)
      return fail(ATTN_E_WORKSPACE, "attn_decode_noalloc: this shape needs " + std::to_string(need) +
                                        " bytes of scratch, above the library's fixed " +
                                        std::to_string(kNoAllocScratchBytes) + " (use attn_decode with a workspace)");
    if ((rc = noalloc_scratch(&workspace))) return rc;
    workspace_bytes = kNoAllocScratchBytes;
  }
  if (!workspace) return fail(ATTN_E_WORKSPACE, "workspace is NULL");
  if (!aligned16(workspace)) return fail(ATTN_E_WORKSPACE, "workspace must be 16-byte aligned");
  if (workspace_bytes < need)
    return fail(ATTN_E_WORKSPACE, "workspace too small: need " + std::to_string(need) + " bytes");
  if ((int64_t)shape->batch * shape->n_heads * shape->tq * nsplit >= (int64_t)1 << 31)
    return fail(ATTN_E_INVAL, "problem too large for one grid");
  // (the ATTN_DEBUG offset check copies the offsets into host memory: not done without allocation)
  if (!noalloc && (rc = check_offsets_debug(shape, cache_off, stream))) return rc;

  soc::AttnArgs a = make_args(shape, q, q_strides, k, v, kv_strides, o, o_strides, cache_off, window, sink, scale);
  a.part = static_cast<float*>(workspace);
  a.nsplit = (int32_t)nsplit;
  a.split = split;
  // longest-first order once the splits take more than one round of the chip (about six
  // single-wave split workgroups fit on a CU)
  a.lpt = (int64_t)shape->batch * shape->n_kv * nsplit > 6 * (int64_t)device_cus();
  hipError_t e = shape->dtype == ATTN_BF16 ? soc::launch_decode_bf16(a, stream) : soc::launch_decode_f32(a, stream);
  if (e != hipSuccess) return hip_fail(e, "attn_decode split launch");
  e = soc::launch_decode_merge(a, shape->dtype == ATTN_BF16, stream);
  return finish(e, stream, "attn_decode merge launch");
}

}  // namespace

extern "C" {

int attn_decode(const attn_shape_t* shape, const void* q, attn_strides_t q_strides, const void* k, const void* v,
                attn_strides_t kv_strides, void* o, attn_strides_t o_strides, const int32_t* cache_off,
                int32_t window, const float* sink, float scale, void* workspace, size_t workspace_bytes,
                int32_t split_tokens, hipStream_t stream) {
  return decode_impl(shape, q, q_strides, k, v, kv_strides, o, o_strides, cache_off, window, sink, scale, workspace,
                     workspace_bytes, split_tokens, stream, false);
}

size_t attn_decode_noalloc_max_scratch_bytes(void) { return kNoAllocScratchBytes; }

int attn_decode_noalloc(const attn_shape_t* shape, const void* q, attn_strides_t q_strides, const void* k,
                        const void* v, attn_strides_t kv_strides, void* o, attn_strides_t o_strides,
                        const int32_t* cache_off, int32_t window, const float* sink, float scale,
                        int32_t split_tokens, hipStream_t stream) {
  return decode_impl(shape, q, q_strides, k, v, kv_strides, o, o_strides, cache_off, window, sink, scale, nullptr, 0,
                     split_tokens, stream, true);
}

size_t attn_ring_decode_workspace_bytes(const attn_shape_t* shape, int32_t split_tokens) {
  if (check_shape(shape) != ATTN_OK) return 0;
  return attn_decode_workspace_bytes(shape, split_tokens) + round_up(sizeof(int32_t) * shape->batch, 256);
}

int attn_ring_decode(const attn_shape_t* shape, const void* q, attn_strides_t q_strides, const void* k_new,
                     const void* v_new, attn_strides_t new_strides, void* k_ring, void* v_ring,
                     attn_strides_t ring_strides, void* o, attn_strides_t o_strides, const int32_t* n_seen,
                     const float* sink, float scale, void* workspace, size_t workspace_bytes, int32_t split_tokens,
                     hipStream_t stream) {
  int rc = check_shape(shape);
  if (rc) return rc;
  if ((rc = check_attn_dtype(shape))) return rc;
  if (shape->batch == 0) {
    g_err.clear();
    return ATTN_OK;
  }
  if (shape->tq != 1) return fail(ATTN_E_INVAL, "ring decode takes one query row per sequence (tq = 1)");
  if ((rc = check_tensors(shape, q, q_strides, k_ring, v_ring, ring_strides, o, o_strides))) return rc;
  if (!k_new || !v_new || !n_seen) return fail(ATTN_E_INVAL, "k_new, v_new and n_seen must be non-NULL device pointers");
  const size_t esz = elem_size(shape->dtype);
  if (!aligned16(k_new) || !aligned16(v_new)) return fail(ATTN_E_INVAL, "k_new and v_new must be 16-byte aligned");
  if (!strides_ok(new_strides, esz)) return fail(ATTN_E_INVAL, "strides must be non-negative multiples of 16 bytes (in elements)");
  if (shape->dtype == ATTN_BF16 && (int64_t)shape->tk * ring_strides.t * 2 > (int64_t)0xffffffff)
    return fail(ATTN_E_UNSUPPORTED, "one (sequence, KV head) ring slice spans more than 4 GiB (W * slot stride)");
  if (shape->dtype == ATTN_BF16 && shape->n_heads / shape->n_kv > 32)
    return fail(ATTN_E_UNSUPPORTED, "bf16 decode serves at most 32 query rows per KV head (n_heads/n_kv <= 32)");
  const int split = split_tokens > 0 ? split_tokens : default_split(shape);
  const int64_t nsplit = (shape->tk + split - 1) / split;
  const size_t part_bytes = attn_decode_workspace_bytes(shape, split);
  const size_t need = attn_ring_decode_workspace_bytes(shape, split);
  if (!workspace) return fail(ATTN_E_WORKSPACE, "workspace is NULL");
  if (!aligned16(workspace)) return fail(ATTN_E_WORKSPACE, "workspace must be 16-byte aligned");
  if (workspace_bytes < need)
    return fail(ATTN_E_WORKSPACE, "workspace too small: need " + std::to_string(need) + " bytes");
  if ((int64_t)shape->batch * shape->n_heads * nsplit >= (int64_t)1 << 31)
    return fail(ATTN_E_INVAL, "problem too large for one grid");
  if (debug_mode()) {
    std::vector<int32_t> h(shape->batch);
    hipError_t e = hipMemcpyAsync(h.data(), n_seen, sizeof(int32_t) * shape->batch, hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_fail(e, "ATTN_DEBUG: reading n_seen");
    for (int b = 0; b < shape->batch; ++b)
      if (h[b] < 0) return fail(ATTN_E_INVAL, "ATTN_DEBUG: n_seen[" + std::to_string(b) + "] is negative");
  }

  if (shape->dtype == ATTN_BF16) {
    // one kernel pass: the split holding each ring's slot substitutes and appends the new row
    soc::AttnArgs a = make_args(shape, q, q_strides, k_ring, v_ring, ring_strides, o, o_strides, nullptr, 0, sink, scale);
    a.part = static_cast<float*>(workspace);
    a.nsplit = (int32_t)nsplit;
    a.split = split;
    a.ring_n = n_seen;
    a.k_new = k_new;
    a.v_new = v_new;
    a.new_sb = new_strides.b;
    a.new_sh = new_strides.h;
    a.fused = nsplit <= 2;  // both splits of a ring in one workgroup, merged there
    hipError_t e = soc::launch_decode_bf16(a, stream);
    if (a.fused) return finish(e, stream, "attn_ring_decode launch");
    if (e != hipSuccess) return hip_fail(e, "attn_ring_decode split launch");
    e = soc::launch_decode_merge(a, true, stream);
    return finish(e, stream, "attn_ring_decode merge launch");
  }
  int32_t* offs = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + part_bytes);
  soc::RingAppendArgs r{};
  r.k_new = k_new;
  r.v_new = v_new;
  r.n_sb = new_strides.b;
  r.n_sh = new_strides.h;
  r.k_ring = k_ring;
  r.v_ring = v_ring;
  r.r_sb = ring_strides.b;
  r.r_sh = ring_strides.h;
  r.r_st = ring_strides.t;
  r.n_seen = n_seen;
  r.cache_off_out = offs;
  r.B = shape->batch;
  r.Hkv = shape->n_kv;
  r.W = shape->tk;
  r.esz = (int32_t)esz;
  r.row_bytes = (int32_t)(shape->head_dim * esz);
  hipError_t e = soc::launch_ring_append(r, stream);
  if (e != hipSuccess) return hip_fail(e, "attn_ring_decode append launch");

  soc::AttnArgs a = make_args(shape, q, q_strides, k_ring, v_ring, ring_strides, o, o_strides, offs, 0, sink, scale);
  a.part = static_cast<float*>(workspace);
  a.nsplit = (int32_t)nsplit;
  a.split = split;
  e = soc::launch_decode_f32(a, stream);
  if (e != hipSuccess) return hip_fail(e, "attn_ring_decode split launch");
  e = soc::launch_decode_merge(a, false, stream);
  return finish(e, stream, "attn_ring_decode merge launch");
}

size_t attn_mla_decode_workspace_bytes(const attn_mla_shape_t* shape, int32_t split_tokens) {
  if (check_mla_shape(shape) != ATTN_OK) return 0;
  return mla_layout(shape, split_tokens).total;
}

int attn_mla_decode(const attn_mla_shape_t* shape, const void* q_nope, attn_strides_t qn_strides,
                    const void* q_rope, attn_strides_t qr_strides, const void* c_kv, attn_strides_t ckv_strides,
                    const void* k_rope, attn_strides_t kr_strides, const void* w_uk, const void* w_uv, void* o,
                    attn_strides_t o_strides, const int32_t* cache_off, float scale, void* workspace,
                    size_t workspace_bytes, int32_t split_tokens, hipStream_t stream) {
  int rc = check_mla_shape(shape);
  if (rc) return rc;
  if (shape->tq == 0 || shape->batch == 0) {
    g_err.clear();
    return ATTN_OK;
  }
  if (!q_nope || !q_rope || !c_kv || !k_rope || !w_uk || !w_uv || !o)
    return fail(ATTN_E_INVAL, "q_nope, q_rope, c_kv, k_rope, w_uk, w_uv and o must be non-NULL device pointers");
  if (!aligned16(q_nope) || !aligned16(q_rope) || !aligned16(c_kv) || !aligned16(k_rope) || !aligned16(w_uk) ||
      !aligned16(w_uv) || !aligned16(o))
    return fail(ATTN_E_INVAL, "all tensors must be 16-byte aligned");
  const attn_strides_t ckv_bt{ckv_strides.b, 0, ckv_strides.t}, kr_bt{kr_strides.b, 0, kr_strides.t};
  if (!strides_ok(qn_strides, 2) || !strides_ok(qr_strides, 2) || !strides_ok(ckv_bt, 2) || !strides_ok(kr_bt, 2) ||
      !strides_ok(o_strides, 2))
    return fail(ATTN_E_INVAL, "strides must be non-negative multiples of 16 bytes (in elements)");
  if (ckv_strides.t < soc::kMlaRank || kr_strides.t < soc::kMlaRope)
    return fail(ATTN_E_INVAL, "c_kv / k_rope token strides must be at least kv_rank / rope_dim");
  if ((int64_t)shape->tk * ckv_strides.t * 2 > (int64_t)0x7fffffff || (int64_t)shape->tk * kr_strides.t * 2 > (int64_t)0x7fffffff)
    return fail(ATTN_E_UNSUPPORTED, "one sequence's latent cache spans more than 2 GiB");
  const MlaLayout L = mla_layout(shape, split_tokens);
  if (L.nsplit > soc::kMlaMaxSplits)
    return fail(ATTN_E_INVAL, "more than 256 splits per sequence: raise split_tokens");
  if (!workspace) return fail(ATTN_E_WORKSPACE, "workspace is NULL");
  if (!aligned16(workspace)) return fail(ATTN_E_WORKSPACE, "workspace must be 16-byte aligned");
  if (workspace_bytes < L.total)
    return fail(ATTN_E_WORKSPACE, "workspace too small: need " + std::to_string(L.total) + " bytes");
  const int64_t nrg = ((int64_t)shape->n_heads * shape->tq + 15) / 16;
  if ((int64_t)shape->batch * nrg * L.nsplit >= (int64_t)1 << 31) return fail(ATTN_E_INVAL, "problem too large for one grid");
  {
    attn_shape_t s2{shape->batch, 1, 1, 128, shape->tq, shape->tk, ATTN_BF16};
    if ((rc = check_offsets_debug(&s2, cache_off, stream))) return rc;
  }
  soc::MlaArgs a{};
  a.q_nope = q_nope;
  a.qn_sb = qn_strides.b; a.qn_sh = qn_strides.h; a.qn_st = qn_strides.t;
  a.q_rope = q_rope;
  a.qr_sb = qr_strides.b; a.qr_sh = qr_strides.h; a.qr_st = qr_strides.t;
  a.c_kv = c_kv;
  a.c_sb = ckv_strides.b; a.c_st = ckv_strides.t;
  a.k_rope = k_rope;
  a.r_sb = kr_strides.b; a.r_st = kr_strides.t;
  a.w_uk = w_uk;
  a.w_uv = w_uv;
  a.o = o;
  a.o_sb = o_strides.b; a.o_sh = o_strides.h; a.o_st = o_strides.t;
  a.cache_off = cache_off;
  a.B = shape->batch;
  a.H = shape->n_heads;
  a.tq = shape->tq;
  a.tk = shape->tk;
  const float sc = scale > 0.f ? scale : 1.f / std::sqrt((float)(shape->nope_dim + shape->rope_dim));
  a.scale_log2 = sc * soc::kLog2e;
  char* ws = static_cast<char*>(workspace);
  a.q_lat = ws + L.q_lat;
  a.part_o = reinterpret_cast<float*>(ws + L.part_o);
  a.part_ml = reinterpret_cast<float*>(ws + L.part_ml);
  a.o_lat = reinterpret_cast<float*>(ws + L.o_lat);
  a.queue = reinterpret_cast<uint32_t*>(ws + L.queue);
  a.nsplit = L.nsplit;
  a.split = L.split;
  a.n_waves = 2 * device_cus();  // the split kernel's LDS use allows two waves per CU
  return finish(soc::launch_mla_decode(a, stream), stream, "attn_mla_decode launch");
}

size_t attn_dsa_decode_workspace_bytes(const attn_shape_t* shape, int32_t topk, int32_t split_tokens) {
  if (check_shape(shape) != ATTN_OK || topk < 1) return 0;
  return dsa_layout(shape, topk, split_tokens).total;
}

int attn_dsa_decode(const attn_shape_t* shape, const void* q, attn_strides_t q_strides, const void* k, const void* v,
                    attn_strides_t kv_strides, void* o, attn_strides_t o_strides, const int32_t* cache_off,
                    const float* sink, float scale, const void* qi, attn_strides_t qi_strides, const void* ki,
                    attn_strides_t ki_strides, const float* wi, int32_t index_heads, int32_t topk,
                    int32_t* kept_list, int32_t* kept_count, void* workspace, size_t workspace_bytes,
                    int32_t split_tokens, hipStream_t stream) {
  int rc = check_shape(shape);
  if (rc) return rc;
  if (shape->dtype != ATTN_BF16 || shape->head_dim != 128)
    return fail(ATTN_E_UNSUPPORTED, "sparse top-k decode is built for bf16 with head_dim 128");
  if (topk < 1) return fail(ATTN_E_INVAL, "topk must be >= 1");
  if (index_heads < 16 || index_heads > soc::kDsaMaxIndexHeads || index_heads % 16 != 0)
    return fail(ATTN_E_UNSUPPORTED, "index_heads must be 16, 32, 48 or 64");
  if (shape->tq == 0 || shape->batch == 0) {
    g_err.clear();
    return ATTN_OK;
  }
  if ((rc = check_tensors(shape, q, q_strides, k, v, kv_strides, o, o_strides))) return rc;
  if (!qi || !ki || !wi) return fail(ATTN_E_INVAL, "qi, ki and wi must be non-NULL device pointers");
  if (!aligned16(qi) || !aligned16(ki)) return fail(ATTN_E_INVAL, "qi and ki must be 16-byte aligned");
  const attn_strides_t ki_bt{ki_strides.b, 0, ki_strides.t};
  if (!strides_ok(qi_strides, 2) || !strides_ok(ki_bt, 2))
    return fail(ATTN_E_INVAL, "strides must be non-negative multiples of 16 bytes (in elements)");
  if (ki_strides.t < soc::kDsaIndexDim) return fail(ATTN_E_INVAL, "ki token stride must be at least 128");
  if ((shape->n_heads / shape->n_kv) > 32)
    return fail(ATTN_E_UNSUPPORTED, "bf16 decode serves at most 32 query rows per KV head (n_heads/n_kv <= 32)");
  if ((int64_t)shape->tk * kv_strides.t * 2 > (int64_t)0x7fffffff || (int64_t)shape->tk * ki_strides.t * 2 > (int64_t)0x7fffffff)
    return fail(ATTN_E_UNSUPPORTED, "one (sequence, KV head) cache slice spans more than 2 GiB");
  const DsaLayout L = dsa_layout(shape, topk, split_tokens);
  if (L.split > 1024) return fail(ATTN_E_INVAL, "split_tokens must be at most 1024");
  if (!workspace) return fail(ATTN_E_WORKSPACE, "workspace is NULL");
  if (!aligned16(workspace)) return fail(ATTN_E_WORKSPACE, "workspace must be 16-byte aligned");
  if (workspace_bytes < L.total)
    return fail(ATTN_E_WORKSPACE, "workspace too small: need " + std::to_string(L.total) + " bytes");
  if ((int64_t)shape->batch * shape->tq * shape->n_kv * L.nsplit >= (int64_t)1 << 31 ||
      (int64_t)shape->batch * shape->tq * ((shape->tk + 255) / 256) >= (int64_t)1 << 31)
    return fail(ATTN_E_INVAL, "problem too large for one grid");
  if ((rc = check_offsets_debug(shape, cache_off, stream))) return rc;

  soc::DsaArgs A{};
  A.at = make_args(shape, q, q_strides, k, v, kv_strides, o, o_strides, cache_off, 0, sink, scale);
  char* ws = static_cast<char*>(workspace);
  A.at.part = reinterpret_cast<float*>(ws + L.part);
  A.at.nsplit = L.nsplit;
  A.at.split = L.split;
  A.qi = qi;
  A.qi_sb = qi_strides.b; A.qi_sh = qi_strides.h; A.qi_st = qi_strides.t;
  A.ki = ki;
  A.ki_sb = ki_strides.b; A.ki_st = ki_strides.t;
  A.wi = wi;
  A.Hi = index_heads;
  A.topk = topk;
  A.scores = reinterpret_cast<float*>(ws + L.scores);
  A.ebound = reinterpret_cast<float*>(ws + L.ebound);
  A.s64 = reinterpret_cast<double*>(ws + L.s64);
  A.band = reinterpret_cast<int32_t*>(ws + L.band);
  A.list = kept_list ? kept_list : reinterpret_cast<int32_t*>(ws + L.list);
  A.count = kept_count ? kept_count : reinterpret_cast<int32_t*>(ws + L.count);
  A.idx_waves = device_cus();  // one 12-wave indexer workgroup per CU
  return finish(soc::launch_dsa_decode(A, stream), stream, "attn_dsa_decode launch");
}

size_t attn_block_select_workspace_bytes(const attn_shape_t* shape, int32_t block_size) {
  if (check_shape(shape) != ATTN_OK || block_size < 1) return 0;
  return select_layout(shape, block_size).total;
}

}  // extern "C"

namespace {

// Validation and workspace carving shared by attn_block_select and attn_block_sparse_prefill.
// Returns ATTN_OK with *out filled, kNoWork for an empty call, or an error code.
constexpr int kNoWork = 1;
int select_setup(const attn_shape_t* shape, const void* q, attn_strides_t q_strides, const void* k,
                 attn_strides_t k_strides, const int32_t* cache_off, int32_t window, int32_t block_size,
                 double keep_mean, double keep_radius, double* tau_mean, double* tau_radius, uint8_t* block_mask,
                 int32_t* block_list, void* workspace, size_t workspace_bytes, hipStream_t stream, bool need_mask,
                 soc::SelectArgs* out) {
  int rc = check_shape(shape);
  if (rc) return rc;
  if (block_size < 1) return fail(ATTN_E_INVAL, "block_size must be >= 1");
  const int d = shape->head_dim;
  if (shape->dtype == ATTN_BF16 && d != 128 && d != 64)
    return fail(ATTN_E_UNSUPPORTED, "bf16 block selection supports head_dim 64 or 128");
  if (shape->dtype == ATTN_F32 && d != 16 && d != 32 && d != 64 && d != 128)
    return fail(ATTN_E_UNSUPPORTED, "f32 block selection supports head_dim 16, 32, 64 or 128");
  if (shape->tq == 0 || shape->batch == 0) return kNoWork;
  if (!q || !k) return fail(ATTN_E_INVAL, "q and k must be non-NULL device pointers");
  if (!tau_mean || !tau_radius || (need_mask && !block_mask))
    return fail(ATTN_E_INVAL, need_mask ? "tau_mean, tau_radius and block_mask must be non-NULL device pointers"
                                        : "tau_mean and tau_radius must be non-NULL device pointers");
  const size_t esz = elem_size(shape->dtype);
  if (!aligned16(q) || !aligned16(k)) return fail(ATTN_E_INVAL, "q and k must be 16-byte aligned");
  if (!strides_ok(q_strides, esz) || !strides_ok(k_strides, esz))
    return fail(ATTN_E_INVAL, "strides must be non-negative multiples of 16 bytes (in elements)");
  if (std::isnan(keep_mean) || std::isnan(keep_radius)) return fail(ATTN_E_INVAL, "keep fractions must not be NaN");
  const SelectLayout L = select_layout(shape, block_size);
  if (!workspace) return fail(ATTN_E_WORKSPACE, "workspace is NULL");
  if (!aligned16(workspace)) return fail(ATTN_E_WORKSPACE, "workspace must be 16-byte aligned");
  if (workspace_bytes < L.total)
    return fail(ATTN_E_WORKSPACE, "workspace too small: need " + std::to_string(L.total) + " bytes");
  if ((int64_t)shape->batch * shape->n_heads * L.nqb >= (int64_t)1 << 31 ||
      (int64_t)shape->batch * shape->n_kv * L.nkb >= (int64_t)1 << 31)
    return fail(ATTN_E_INVAL, "problem too large for one grid");
  if ((int64_t)L.nqb * L.nkb >= (int64_t)1 << 31)
    return fail(ATTN_E_INVAL, "too many (query block, key block) pairs per head");
  if ((rc = check_offsets_debug(shape, cache_off, stream))) return rc;

  soc::SelectArgs a{};
  a.q = q;
  a.k = k;
  a.q_sb = q_strides.b; a.q_sh = q_strides.h; a.q_st = q_strides.t;
  a.k_sb = k_strides.b; a.k_sh = k_strides.h; a.k_st = k_strides.t;
  a.B = shape->batch;
  a.Hq = shape->n_heads;
  a.Hkv = shape->n_kv;
  a.g = shape->n_heads / shape->n_kv;
  a.tq = shape->tq;
  a.tk = shape->tk;
  a.d = d;
  a.bs = block_size;
  a.nqb = L.nqb;
  a.nkb = L.nkb;
  a.cache_off = cache_off;
  a.window = window;
  a.keep_mean = keep_mean;
  a.keep_radius = keep_radius;
  a.tau_mean = tau_mean;
  a.tau_radius = tau_radius;
  char* ws = static_cast<char*>(workspace);
  a.mask = block_mask ? block_mask : reinterpret_cast<uint8_t*>(ws + L.wmask);
  a.list = block_list;
  a.qmean = reinterpret_cast<double*>(ws + L.qmean);
  a.cent = reinterpret_cast<double*>(ws + L.cT);
  a.rad2 = reinterpret_cast<double*>(ws + L.rad2);
  a.score = reinterpret_cast<double*>(ws + L.score);
  a.norm2 = reinterpret_cast<double*>(ws + L.norm2);
  a.nmax = reinterpret_cast<double*>(ws + L.nmax);
  a.hpart = reinterpret_cast<uint32_t*>(ws + L.hpart);
  a.tflag = reinterpret_cast<uint32_t*>(ws + L.tflag);
  a.ccount = reinterpret_cast<uint32_t*>(ws + L.ccount);
  a.pick = reinterpret_cast<int64_t*>(ws + L.pick);
  a.cand = reinterpret_cast<double*>(ws + L.cand);
  a.cpos = reinterpret_cast<int32_t*>(ws + L.cpos);
  a.score_wgs = 2 * device_cus();  // the score kernel's LDS and registers allow two per CU
  *out = a;
  return ATTN_OK;
}

}  // namespace

extern "C" {

int attn_block_select(const attn_shape_t* shape, const void* q, attn_strides_t q_strides, const void* k,
                      attn_strides_t k_strides, const int32_t* cache_off, int32_t window, int32_t block_size,
                      double keep_mean, double keep_radius, double* tau_mean, double* tau_radius,
                      uint8_t* block_mask, int32_t* block_list, void* workspace, size_t workspace_bytes,
                      hipStream_t stream) {
  soc::SelectArgs a;
  const int rc = select_setup(shape, q, q_strides, k, k_strides, cache_off, window, block_size, keep_mean, keep_radius,
                              tau_mean, tau_radius, block_mask, block_list, workspace, workspace_bytes, stream, true, &a);
  if (rc == kNoWork) {
    g_err.clear();
    return ATTN_OK;
  }
  if (rc) return rc;
  const hipError_t e = soc::launch_block_select(a, shape->dtype == ATTN_BF16, stream);
  return finish(e, stream, "attn_block_select launch");
}

size_t attn_block_sparse_prefill_workspace_bytes(const attn_shape_t* shape, int32_t block_size) {
  return attn_block_select_workspace_bytes(shape, block_size);
}

int attn_block_sparse_prefill(const attn_shape_t* shape, const void* q, attn_strides_t q_strides, const void* k,
                              const void* v, attn_strides_t kv_strides, void* o, attn_strides_t o_strides,
                              const int32_t* cache_off, int32_t window, const float* sink, float scale,
                              int32_t block_size, double keep_mean, double keep_radius, double* tau_mean,
                              double* tau_radius, uint8_t* block_mask_out, void* workspace, size_t workspace_bytes,
                              hipStream_t stream) {
  int rc = check_shape(shape);
  if (rc) return rc;
  if ((rc = check_attn_dtype(shape))) return rc;
  if (shape->tq == 0 || shape->batch == 0) {
    g_err.clear();
    return ATTN_OK;
  }
  if ((rc = check_tensors(shape, q, q_strides, k, v, kv_strides, o, o_strides))) return rc;
  if (shape->dtype == ATTN_BF16 && block_size != 128)
    return fail(ATTN_E_UNSUPPORTED, "the bf16 block-sparse prefill needs block_size 128");
  if (shape->dtype == ATTN_BF16 && (int64_t)shape->tk * kv_strides.t * 2 > (int64_t)0xffffffff)
    return fail(ATTN_E_UNSUPPORTED, "one (sequence, KV head) cache slice spans more than 4 GiB (tk * token stride)");
  const int64_t nqt = (shape->tq + 127) / 128;
  if (nqt * shape->batch * shape->n_heads >= (int64_t)1 << 31) return fail(ATTN_E_INVAL, "problem too large for one grid");
  soc::SelectArgs sa;
  rc = select_setup(shape, q, q_strides, k, kv_strides, cache_off, window, block_size, keep_mean, keep_radius, tau_mean,
                    tau_radius, block_mask_out, nullptr, workspace, workspace_bytes, stream, false, &sa);
  if (rc) return rc;  // (kNoWork is excluded above)
  hipError_t e = soc::launch_block_select(sa, shape->dtype == ATTN_BF16, stream);
  if (e != hipSuccess) return hip_fail(e, "attn_block_sparse_prefill selection launch");
  soc::AttnArgs a = make_args(shape, q, q_strides, k, v, kv_strides, o, o_strides, cache_off, window, sink, scale);
  a.block_size = block_size;
  a.n_qb = sa.nqb;
  a.mask_stride = sa.nkb;
  a.list_stride = 1 + sa.nkb;
  a.block_mask = sa.mask;  // the selection's mask (the caller's, or the workspace's)
  e = shape->dtype == ATTN_BF16 ? soc::launch_prefill_bf16(a, stream) : soc::launch_prefill_f32(a, stream);
  return finish(e, stream, "attn_block_sparse_prefill prefill launch");
}

int attn_block_list_from_mask(int64_t rows, int32_t n_kb, const uint8_t* block_mask, int32_t* block_list,
                              hipStream_t stream) {
  if (rows < 0 || n_kb < 1) return fail(ATTN_E_INVAL, "rows must be >= 0 and n_kb >= 1");
  if (rows == 0) {
    g_err.clear();
    return ATTN_OK;
  }
  if (!block_mask || !block_list) return fail(ATTN_E_INVAL, "block_mask and block_list must be non-NULL");
  if (rows >= (int64_t)1 << 31) return fail(ATTN_E_INVAL, "too many rows for one grid");
  return finish(soc::launch_list_from_mask(rows, n_kb, block_mask, block_list, stream), stream,
                "attn_block_list_from_mask launch");
}

}  // extern "C"
