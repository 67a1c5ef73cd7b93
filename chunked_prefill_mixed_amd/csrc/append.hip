// Paged KV append: the step's K/V are written into their cache pages before
// attention reads the cache ("05. Chunked Prefill" section 8; tbr8.org deep
// dive 4.2, 16-token pages).  Pure bit copy.
//
// One wave per packed token, 4 tokens per workgroup.  A token's row is found
// in one step: the wave's lanes read query_start_loc in parallel (64 entries
// per load, all loads in flight together) and the row is the number of rows
// that start at or before the token, minus one (rows that schedule no token
// share their start with the next row and are skipped by the count).  Then
// context_len and the page id: three dependent loads in all, where a binary
// search would chain about log2(rows) of them.  K rows are copied as 16-byte
// pieces into the token-major K page; V is scattered into the transposed V
// page (slot-minor), 2 bytes per head dimension, lanes walking consecutive d
// so one store instruction covers 2 KiB of one page.  Tokens of one page
// write the same 32-byte V rows, which the L2 merges before they reach HBM.

#include "device.h"
#include "internal.h"
#include "tiles.h"

namespace cpa {

constexpr int kAppendWaves = 4;  // tokens per workgroup

template <int D>
__global__ __launch_bounds__(64 * kAppendWaves) void append_kernel(
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    const int32_t* __restrict__ qsl, const int32_t* __restrict__ ctx,
    const int32_t* __restrict__ bt, int bt_stride, int num_seqs, int num_tokens,
    int num_kv_heads, uint16_t* __restrict__ k_cache, uint16_t* __restrict__ v_cache) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * kAppendWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (t >= num_tokens) return;  // whole wave; no barrier below

  // row s = #{i < num_seqs : qsl[i] <= t} - 1; qsl is non-decreasing and
  // qsl[num_seqs] = num_tokens > t
  int count = 0;
  for (int base = 0; base < num_seqs; base += 64) {
    const int i = base + lane;
    const bool le = i < num_seqs && qsl[i] <= t;
    count += __builtin_popcountll(__ballot(le));
  }
  const int s = count - 1;
  const int p = ctx[s] + (t - qsl[s]);
  const int64_t blk = bt[(int64_t)s * bt_stride + p / kBlock];
  const int slot = p % kBlock;
  const int64_t page0 = blk * num_kv_heads * (int64_t)(kBlock * D);

  constexpr int kParts = D / 8;  // 16-byte pieces per head row
  const uint4* ksrc = reinterpret_cast<const uint4*>(k_new + (int64_t)t * num_kv_heads * D);
  for (int c = lane; c < num_kv_heads * kParts; c += 64) {
    const int g = c / kParts, part = c % kParts;
    *reinterpret_cast<uint4*>(k_cache + page0 + (int64_t)g * (kBlock * D) + slot * D + part * 8) =
        ksrc[c];
  }
  const uint16_t* vsrc = v_new + (int64_t)t * num_kv_heads * D;
  for (int c = lane; c < num_kv_heads * D; c += 64) {
    const int g = c / D, d = c % D;
    v_cache[page0 + (int64_t)g * (kBlock * D) + d * kBlock + slot] = vsrc[c];
  }
}

hipError_t launch_append(const void* k_new, const void* v_new, const int32_t* qsl,
                         const int32_t* ctx, const int32_t* bt, int bt_stride, int num_seqs,
                         int num_tokens, int num_kv_heads, int head_dim, void* k_cache,
                         void* v_cache, hipStream_t stream) {
  dim3 grid((num_tokens + kAppendWaves - 1) / kAppendWaves), block(64 * kAppendWaves);
  const auto* kn = static_cast<const uint16_t*>(k_new);
  const auto* vn = static_cast<const uint16_t*>(v_new);
  auto* kc = static_cast<uint16_t*>(k_cache);
  auto* vc = static_cast<uint16_t*>(v_cache);
  if (head_dim == 128)
    hipLaunchKernelGGL(append_kernel<128>, grid, block, 0, stream, kn, vn, qsl, ctx, bt, bt_stride,
                       num_seqs, num_tokens, num_kv_heads, kc, vc);
  else
    hipLaunchKernelGGL(append_kernel<64>, grid, block, 0, stream, kn, vn, qsl, ctx, bt, bt_stride,
                       num_seqs, num_tokens, num_kv_heads, kc, vc);
  return hipGetLastError();
}

}  // namespace cpa
