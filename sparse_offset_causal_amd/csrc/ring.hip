// Ring-buffer cache append for sliding-window decode on gfx950.
//
// A layer that attends only to the last W tokens keeps W slots per KV head; token number n
// goes into slot n mod W, overwriting the oldest entry, and attention runs over the filled
// slots in any order (sotaaz.com/post/attention-in-code, section 2, the ring-buffer cache).
// This kernel (the fp32 path; the bf16 split-KV decode substitutes and appends the new row
// itself) writes one step's K and V rows into their slot and, per sequence, the offset that
// makes the split-KV decode read exactly the filled slots: with min(n + 1, W) slots filled,
// a one-row query at cache offset min(n, W - 1) sees slots 0 .. min(n, W - 1).
//
// One workgroup of 64 threads per (sequence, KV head); each thread copies one 16-byte
// chunk of the K row or of the V row (a row is at most 512 bytes: 32 chunks).

#include "device_common.h"
#include "internal.h"

namespace soc {
namespace {

__global__ void __launch_bounds__(64) ring_append_kernel(RingAppendArgs r) {
  const int kvh = blockIdx.x % r.Hkv;
  const int b = blockIdx.x / r.Hkv;
  const int n = r.n_seen[b];
  const int slot = n % r.W;
  const int chunks = r.row_bytes / 16;
  const int t = threadIdx.x;
  const bool is_v = t >= chunks;
  const int c = is_v ? t - chunks : t;
  if (c < chunks) {
    const char* src = (const char*)(is_v ? r.v_new : r.k_new) + (b * r.n_sb + kvh * r.n_sh) * r.esz;
    char* dst = (char*)(is_v ? r.v_ring : r.k_ring) + (b * r.r_sb + kvh * r.r_sh + (int64_t)slot * r.r_st) * r.esz;
    *(u32x4*)(dst + 16 * c) = *(const u32x4*)(src + 16 * c);
  }
  if (kvh == 0 && t == 0) r.cache_off_out[b] = min(n, r.W - 1);
}

}  // namespace

hipError_t launch_ring_append(const RingAppendArgs& r, hipStream_t s) {
  const int64_t grid = (int64_t)r.B * r.Hkv;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(ring_append_kernel, dim3((unsigned)grid), dim3(64), 0, s, r);
  return hipGetLastError();
}

}  // namespace soc
