// Prefill-chunk flash attention kernel: one workgroup of chunk_waves(D) waves
// per work item (32 query rows per wave, all of one KV head, one piece of its
// keys).  The body and its design are in chunk_body.h.

#include "chunk_body.h"

namespace cpa {

// launch bounds: at least two waves per SIMD (one 8-wave or two 4-wave
// workgroups per CU), so at most 256 registers per lane
template <int D, int G>
__global__ __launch_bounds__(64 * chunk_waves(D), 8 / chunk_waves(D)) void chunk_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_cache,
    const uint16_t* __restrict__ v_cache, const int32_t* __restrict__ bt, int bt_stride,
    const int32_t* __restrict__ qsl, const int32_t* __restrict__ ctx,
    const int32_t* __restrict__ tiles, int num_tiles, int num_q_heads, int num_kv_heads,
    float scale_log2, uint16_t* __restrict__ out, float* __restrict__ lse, ChunkPartials part) {
  chunk_body<D, G>(q, k_cache, v_cache, bt, bt_stride, qsl, ctx, tiles, num_tiles, num_q_heads,
                   num_kv_heads, scale_log2, out, lse, part, blockIdx.x);
}

template <int D, int G>
static void launch_chunk_t(const void* q, const void* kc, const void* vc, const int32_t* bt,
                           int bt_stride, const int32_t* qsl, const int32_t* ctx,
                           const int32_t* tiles, int num_tiles, int hq, int hkv, float sl2,
                           void* out, float* lse, ChunkPartials part, hipStream_t stream) {
  hipLaunchKernelGGL((chunk_kernel<D, G>), dim3(num_tiles * hkv), dim3(64 * chunk_waves(D)), 0,
                     stream, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(kc),
                     static_cast<const uint16_t*>(vc), bt, bt_stride, qsl, ctx, tiles, num_tiles,
                     hq, hkv, sl2, static_cast<uint16_t*>(out), lse, part);
}

hipError_t launch_chunk(const void* q, const void* k_cache, const void* v_cache, const int32_t* bt,
                        int bt_stride, const int32_t* qsl, const int32_t* ctx,
                        const int32_t* tiles, int num_tiles, int num_q_heads, int num_kv_heads,
                        int head_dim, float scale_log2, void* out, float* lse, ChunkPartials part,
                        hipStream_t stream) {
  const int G = num_q_heads / num_kv_heads;
  // G = 0 instances: any other group, read at run time
#define CPA_CHK(DD, GG)                                                                        \
  if (head_dim == DD && (G == GG || GG == 0)) {                                               \
    launch_chunk_t<DD, GG>(q, k_cache, v_cache, bt, bt_stride, qsl, ctx, tiles, num_tiles,      \
                           num_q_heads, num_kv_heads, scale_log2, out, lse, part, stream);      \
    return hipGetLastError();                                                                   \
  }
  CPA_CHK(128, 1) CPA_CHK(128, 2) CPA_CHK(128, 4) CPA_CHK(128, 8) CPA_CHK(128, 0)
  CPA_CHK(64, 1) CPA_CHK(64, 2) CPA_CHK(64, 4) CPA_CHK(64, 8) CPA_CHK(64, 0)
#undef CPA_CHK
  return hipErrorInvalidValue;
}

}  // namespace cpa
