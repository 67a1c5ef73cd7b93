// Paged KV append: the step's K/V are written into their cache pages before
// attention reads the cache ("05. Chunked Prefill" section 8; tbr8.org deep
// dive 4.2, 16-token pages).  Pure bit copy.
//
// One workgroup per packed token.  K rows are copied as 16-byte pieces into
// the token-major K page; V is scattered into the transposed V page
// (slot-minor), 2 bytes per head dimension.  Tokens of one page write the
// same 32-byte V rows, which the L2 merges before they reach HBM.

#include "device.h"
#include "internal.h"
#include "tiles.h"

namespace cpa {

template <int D>
__global__ __launch_bounds__(128) void append_kernel(
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    const int32_t* __restrict__ qsl, const int32_t* __restrict__ ctx,
    const int32_t* __restrict__ bt, int bt_stride, int num_seqs, int num_kv_heads,
    uint16_t* __restrict__ k_cache, uint16_t* __restrict__ v_cache) {
  const int t = blockIdx.x;
  // row of token t: the last s with qsl[s] <= t
  int lo = 0, hi = num_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (qsl[mid] <= t) lo = mid; else hi = mid - 1;
  }
  const int s = lo;
  const int p = ctx[s] + (t - qsl[s]);
  const int64_t blk = bt[(int64_t)s * bt_stride + p / kBlock];
  const int slot = p % kBlock;

  constexpr int kParts = D / 8;  // 16-byte pieces per head row
  const int pieces = num_kv_heads * kParts;
  const uint4* ksrc = reinterpret_cast<const uint4*>(k_new + (int64_t)t * num_kv_heads * D);
  const uint4* vsrc = reinterpret_cast<const uint4*>(v_new + (int64_t)t * num_kv_heads * D);
  for (int c = threadIdx.x; c < pieces; c += blockDim.x) {
    const int g = c / kParts, part = c % kParts;
    const int64_t page = (blk * num_kv_heads + g) * (int64_t)(kBlock * D);
    const uint4 kv = ksrc[c];
    *reinterpret_cast<uint4*>(k_cache + page + slot * D + part * 8) = kv;
    const uint4 vv = vsrc[c];
    uint16_t* vdst = v_cache + page + (int64_t)(part * 8) * kBlock + slot;
    const uint32_t w[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      vdst[(2 * i) * kBlock] = (uint16_t)(w[i] & 0xFFFFu);
      vdst[(2 * i + 1) * kBlock] = (uint16_t)(w[i] >> 16);
    }
  }
}

hipError_t launch_append(const void* k_new, const void* v_new, const int32_t* qsl,
                         const int32_t* ctx, const int32_t* bt, int bt_stride, int num_seqs,
                         int num_tokens, int num_kv_heads, int head_dim, void* k_cache,
                         void* v_cache, hipStream_t stream) {
  dim3 grid(num_tokens), block(128);
  const auto* kn = static_cast<const uint16_t*>(k_new);
  const auto* vn = static_cast<const uint16_t*>(v_new);
  auto* kc = static_cast<uint16_t*>(k_cache);
  auto* vc = static_cast<uint16_t*>(v_cache);
  if (head_dim == 128)
    hipLaunchKernelGGL(append_kernel<128>, grid, block, 0, stream, kn, vn, qsl, ctx, bt, bt_stride,
                       num_seqs, num_kv_heads, kc, vc);
  else
    hipLaunchKernelGGL(append_kernel<64>, grid, block, 0, stream, kn, vn, qsl, ctx, bt, bt_stride,
                       num_seqs, num_kv_heads, kc, vc);
  return hipGetLastError();
}

}  // namespace cpa
