// Paged KV append: the step's K/V are written into their cache pages before
// attention reads the cache ("05. Chunked Prefill" section 8; tbr8.org deep
// dive 4.2, 16-token pages).  Pure bit copy.
//
// One workgroup per packed token.  A token t with query_start_loc[t] == t and
// query_start_loc[t+1] == t+1 is row t's only token (every decode row, which
// come first); other tokens find their row by a binary search.  K rows are
// copied as 16-byte pieces into the token-major K page; V is scattered into
// the transposed V page (slot-minor), 2 bytes per head dimension, lanes
// walking consecutive d so one store instruction covers 2 KiB of one page.
// Tokens of one page write the same 32-byte V rows, which the L2 merges
// before they reach HBM.

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
  int s;
  if (t < num_seqs && qsl[t] == t && qsl[t + 1] == t + 1) {
    s = t;
  } else {  // the last s with qsl[s] <= t
    int lo = 0, hi = num_seqs - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (qsl[mid] <= t) lo = mid; else hi = mid - 1;
    }
    s = lo;
  }
  const int p = ctx[s] + (t - qsl[s]);
  const int64_t blk = bt[(int64_t)s * bt_stride + p / kBlock];
  const int slot = p % kBlock;
  const int64_t page0 = blk * num_kv_heads * (int64_t)(kBlock * D);

  constexpr int kParts = D / 8;  // 16-byte pieces per head row
  const uint4* ksrc = reinterpret_cast<const uint4*>(k_new + (int64_t)t * num_kv_heads * D);
  for (int c = threadIdx.x; c < num_kv_heads * kParts; c += blockDim.x) {
    const int g = c / kParts, part = c % kParts;
    *reinterpret_cast<uint4*>(k_cache + page0 + (int64_t)g * (kBlock * D) + slot * D + part * 8) =
        ksrc[c];
  }
  const uint16_t* vsrc = v_new + (int64_t)t * num_kv_heads * D;
  for (int c = threadIdx.x; c < num_kv_heads * D; c += blockDim.x) {
    const int g = c / D, d = c % D;
    v_cache[page0 + (int64_t)g * (kBlock * D) + d * kBlock + slot] = vsrc[c];
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
