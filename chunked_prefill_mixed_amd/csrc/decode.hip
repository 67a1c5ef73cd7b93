// Split-KV decode kernel: one wave per (key piece, KV head, 32 query heads of
// the group), 4 per workgroup.
// The body and its design are in decode_body.h.

#include "decode_body.h"

namespace cpa {

template <int D, int G>
__global__ __launch_bounds__(64 * kDecodeWaves) void decode_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_cache,
    const uint16_t* __restrict__ v_cache, const int32_t* __restrict__ bt, int bt_stride,
    const int32_t* __restrict__ splits, int num_q_heads, int num_kv_heads, int num_items,
    float scale_log2, uint16_t* __restrict__ out, float* __restrict__ lse, Partials ws) {
  decode_body<D, G>(q, k_cache, v_cache, bt, bt_stride, splits, num_q_heads, num_kv_heads,
                    num_items, scale_log2, out, lse, ws, blockIdx.x * kDecodeWaves);
}

template <int D, int G>
static void launch_decode_t(const void* q, const void* kc, const void* vc, const int32_t* bt,
                            int bt_stride, const int32_t* splits, int num_splits, int hq, int hkv,
                            float sl2, void* out, float* lse, Partials ws, hipStream_t stream) {
  // a run-time group (G = 0) of more than 32 heads takes a wave per 32 heads
  const int items = num_splits * hkv * (G > 0 ? 1 : decode_group_waves(hq / hkv));
  hipLaunchKernelGGL((decode_kernel<D, G>), dim3((items + kDecodeWaves - 1) / kDecodeWaves),
                     dim3(64 * kDecodeWaves), 0, stream, static_cast<const uint16_t*>(q),
                     static_cast<const uint16_t*>(kc), static_cast<const uint16_t*>(vc), bt,
                     bt_stride, splits, hq, hkv, items, sl2, static_cast<uint16_t*>(out), lse, ws);
}

hipError_t launch_decode(const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* bt, int bt_stride, const int32_t* qsl,
                         const int32_t* splits, int num_splits, int num_q_heads, int num_kv_heads,
                         int head_dim, float scale_log2, void* out, float* lse, Partials ws,
                         hipStream_t stream) {
  const int G = num_q_heads / num_kv_heads;
  // G = 0 instances: any other group, read at run time
#define CPA_DEC(DD, GG)                                                                        \
  if (head_dim == DD && (G == GG || GG == 0)) {                                               \
    launch_decode_t<DD, GG>(q, k_cache, v_cache, bt, bt_stride, splits, num_splits,             \
                            num_q_heads, num_kv_heads, scale_log2, out, lse, ws, stream);       \
    return hipGetLastError();                                                                   \
  }
  CPA_DEC(128, 1) CPA_DEC(128, 2) CPA_DEC(128, 4) CPA_DEC(128, 8) CPA_DEC(128, 0)
  CPA_DEC(64, 1) CPA_DEC(64, 2) CPA_DEC(64, 4) CPA_DEC(64, 8) CPA_DEC(64, 0)
#undef CPA_DEC
  return hipErrorInvalidValue;
}

}  // namespace cpa
