// A step's decode pieces and chunk tiles in one launch.
//
// The decode pieces are bound by HBM bandwidth and the chunk tiles by the
// matrix cores ("How Chunked Prefill Stops Decode Starvation", "The stall"
// and "The payoff"; tbr8.org deep dive section 1), and the two touch
// different output rows and partial slots, so nothing orders them inside the
// step.  Launched as one grid, the kernel boundary between them goes away.
// Every workgroup has the chunk workgroup's chunk_waves(D) waves; a decode
// workgroup runs one (piece, KV head) item per wave, as the decode kernel's
// do.  The caller uses it only when the chunk tiles alone fill a resident
// round (mixed_slots).
//
// Which part comes first in the grid (workgroups are dispatched in order):
// when the decode workgroups fit one resident round of this kernel (one
// workgroup per CU at head_dim 128, three at 64), they go first and start
// together while the chunk tiles take the other slots and then the slots the
// decode frees; otherwise the chunk tiles go first and the decode pieces fill
// the slots that the chunk's last round leaves idle.  The decode count is
// rounded up to a multiple of 8 when it leads, so chunk workgroup w still
// lands on XCD w % 8 (the chunk's XCD-aware work order relies on it).

#include "chunk_body.h"
#include "decode_body.h"

namespace cpa {

template <int D, int G>
__global__ __launch_bounds__(64 * chunk_waves(D), 8 / chunk_waves(D)) void mixed_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_cache,
    const uint16_t* __restrict__ v_cache, const int32_t* __restrict__ bt, int bt_stride,
    const int32_t* __restrict__ qsl, const int32_t* __restrict__ ctx,
    const int32_t* __restrict__ tiles, int num_tiles, const int32_t* __restrict__ splits,
    int num_items, int num_q_heads, int num_kv_heads, float scale_log2,
    uint16_t* __restrict__ out, float* __restrict__ lse, ChunkPartials cpart, Partials dpart,
    int decode_lead) {
  const int w = blockIdx.x;
  const int chunk_wgs = num_tiles * num_kv_heads;
  // decode_lead: workgroups [0, decode_lead) are decode (0: chunk first)
  const bool is_decode = decode_lead ? w < decode_lead : w >= chunk_wgs;
  if (is_decode)
    decode_body<D, G>(q, k_cache, v_cache, bt, bt_stride, splits, num_q_heads, num_kv_heads,
                      num_items, scale_log2, out, lse, dpart,
                      (decode_lead ? w : w - chunk_wgs) * chunk_waves(D));
  else
    chunk_body<D, G>(q, k_cache, v_cache, bt, bt_stride, qsl, ctx, tiles, num_tiles, num_q_heads,
                     num_kv_heads, scale_log2, out, lse, cpart, w - decode_lead);
}

template <int D, int G>
static void launch_mixed_t(const void* q, const void* kc, const void* vc, const int32_t* bt,
                           int bt_stride, const int32_t* qsl, const int32_t* ctx,
                           const int32_t* tiles, int num_tiles, const int32_t* splits,
                           int num_splits, int hq, int hkv, float sl2, void* out, float* lse,
                           ChunkPartials cpart, Partials dpart, hipStream_t stream) {
  // a run-time group (G = 0) of more than 32 heads takes a wave per 32 heads
  const int items = num_splits * hkv * (G > 0 ? 1 : decode_group_waves(hq / hkv));
  constexpr int W = chunk_waves(D);  // decode items per workgroup
  const int decode_wgs = (items + W - 1) / W;
  const int decode_lead = decode_wgs <= mixed_slots(D) ? (decode_wgs + 7) / 8 * 8 : 0;
  const int wgs = num_tiles * hkv + (decode_lead ? decode_lead : decode_wgs);
  hipLaunchKernelGGL((mixed_kernel<D, G>), dim3(wgs), dim3(64 * W), 0, stream,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(kc),
                     static_cast<const uint16_t*>(vc), bt, bt_stride, qsl, ctx, tiles, num_tiles,
                     splits, items, hq, hkv, sl2, static_cast<uint16_t*>(out), lse, cpart, dpart,
                     decode_lead);
}

hipError_t launch_mixed(const void* q, const void* k_cache, const void* v_cache, const int32_t* bt,
                        int bt_stride, const int32_t* qsl, const int32_t* ctx,
                        const int32_t* tiles, int num_tiles, const int32_t* splits, int num_splits,
                        int num_q_heads, int num_kv_heads, int head_dim, float scale_log2,
                        void* out, float* lse, ChunkPartials cpart, Partials dpart,
                        hipStream_t stream) {
  const int G = num_q_heads / num_kv_heads;
  // G = 0 instances: any other group, read at run time
#define CPA_MIX(DD, GG)                                                                        \
  if (head_dim == DD && (G == GG || GG == 0)) {                                               \
    launch_mixed_t<DD, GG>(q, k_cache, v_cache, bt, bt_stride, qsl, ctx, tiles, num_tiles,      \
                           splits, num_splits, num_q_heads, num_kv_heads, scale_log2, out, lse, \
                           cpart, dpart, stream);                                               \
    return hipGetLastError();                                                                   \
  }
  CPA_MIX(128, 1) CPA_MIX(128, 2) CPA_MIX(128, 4) CPA_MIX(128, 8) CPA_MIX(128, 0)
  CPA_MIX(64, 1) CPA_MIX(64, 2) CPA_MIX(64, 4) CPA_MIX(64, 8) CPA_MIX(64, 0)
#undef CPA_MIX
  return hipErrorInvalidValue;
}

}  // namespace cpa
