// Split-KV decode attention and the log-sum-exp merge of its pieces.
//
// A decode row's single query reads its whole cached context from HBM each
// step ("How Chunked Prefill Stops Decode Starvation", "The stall"; tbr8.org
// deep dive section 1), so this kernel is bound by HBM bandwidth: about 4
// flops per byte of K/V at 4 query heads per KV head.  It uses VALU dot
// products and lane exchanges, not matrix cores.
//
// One wave per (key split, KV head).  All G query heads that share the KV
// head are served by the one read of each 16-token page.
//   K page [16][D]: lane l owns key l/4 and the 8-wide d pieces
//     (l%4)*8 + 32j; the wave's four 16-byte loads per lane read 64-byte
//     runs of each key row.  Scores: v_dot2_f32_bf16 over the lane's d
//     pieces, then a 2-step DPP sum inside each quad.
//   V page [D][16] (transposed): lane l owns d = 32j + l/2 and keys
//     8*(l%2)..+8, one contiguous 16-byte load per j; the whole wave reads
//     the 4 KiB page in 1 KiB contiguous sweeps.  P*V: v_dot2 over the
//     lane's 8 keys with the bf16 probabilities (moved from key-owner lanes
//     through 64 bytes of LDS per head).
// Online softmax in fp32 with a wave-uniform running max per head.  A row
// covered by one split writes its bf16 output directly; otherwise each split
// writes unnormalised fp32 (acc, max, sum) and merge_kernel combines them:
//   M = max m_i,  L = sum l_i 2^(m_i - M),  out = sum acc_i 2^(m_i - M) / L.

#include "device.h"
#include "internal.h"
#include "tiles.h"

namespace cpa {

template <int D, int G>
__global__ __launch_bounds__(64) void decode_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_cache,
    const uint16_t* __restrict__ v_cache, const int32_t* __restrict__ bt, int bt_stride,
    const int32_t* __restrict__ qsl, const int32_t* __restrict__ splits, int num_q_heads,
    int num_kv_heads, float scale_log2, uint16_t* __restrict__ out, float* __restrict__ lse,
    Partials ws) {
  constexpr int J = D / 32;  // 16-byte pieces per lane per page, for K and for V
  __shared__ __align__(16) uint16_t pbuf[2][G][kBlock];

  const int lane = threadIdx.x;
  const int g = blockIdx.x % num_kv_heads;
  const int sp = blockIdx.x / num_kv_heads;
  const int4 e = reinterpret_cast<const int4*>(splits)[sp];
  const int row = e.x, kv_begin = e.y, kv_end = e.z, slot = e.w;
  const int t = qsl[row];
  const int kk = lane >> 2, qd = lane & 3, par = lane & 1;

  uint4 qf[G][J];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int j = 0; j < J; ++j)
      qf[h][j] = *reinterpret_cast<const uint4*>(
          q + ((int64_t)t * num_q_heads + g * G + h) * D + qd * 8 + 32 * j);

  float m[G], lsum[G], acc[G][J];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = neg_inf();
    lsum[h] = 0.f;
#pragma unroll
    for (int j = 0; j < J; ++j) acc[h][j] = 0.f;
  }

  const int32_t* btrow = bt + (int64_t)row * bt_stride;
  const int pg0 = kv_begin / kBlock, pg1 = (kv_end + kBlock - 1) / kBlock;
  for (int pg = pg0; pg < pg1; ++pg) {
    const int buf = (pg - pg0) & 1;
    const int64_t page = ((int64_t)btrow[pg] * num_kv_heads + g) * (kBlock * D);
    uint4 kf[J], vf[J];
#pragma unroll
    for (int j = 0; j < J; ++j)
      kf[j] = *reinterpret_cast<const uint4*>(k_cache + page + kk * D + qd * 8 + 32 * j);
#pragma unroll
    for (int j = 0; j < J; ++j)
      vf[j] = *reinterpret_cast<const uint4*>(v_cache + page + j * 512 + lane * 8);

    const bool valid = pg * kBlock + kk < kv_end;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float a = 0.f;
#pragma unroll
      for (int j = 0; j < J; ++j) a = dot8_bf16(qf[h][j], kf[j], a);
      a += dpp<kQuadXor1>(a);
      a += dpp<kQuadXor2>(a);
      const float s = valid ? a : neg_inf();
      float mx = fmaxf(s, dpp<kRowHalfMirror>(s));
      mx = fmaxf(mx, dpp<kRowMirror>(mx));
      mx = fmaxf(mx, xor_lane(mx, 16));
      mx = fmaxf(mx, xor_lane(mx, 32));
      const float mn = fmaxf(m[h], mx);
      const float alpha = fast_exp2((m[h] - mn) * scale_log2);
      m[h] = mn;
      const float p = fast_exp2((s - mn) * scale_log2);
      lsum[h] = lsum[h] * alpha + (qd == 0 ? p : 0.f);
#pragma unroll
      for (int j = 0; j < J; ++j) acc[h][j] *= alpha;
      if (qd == (h & 3)) pbuf[buf][h][kk] = to_bf16(p);
    }
    // keys past the split's end in its last page: their V slots may hold
    // anything (even NaN); zero them so 0 * V stays 0
    const int nvalid = kv_end - pg * kBlock - 8 * par;
    if (nvalid < 8) {
#pragma unroll
      for (int j = 0; j < J; ++j) {
        uint32_t w[4] = {vf[j].x, vf[j].y, vf[j].z, vf[j].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t keep_lo = (2 * i < nvalid) ? 0xFFFFu : 0u;
          const uint32_t keep_hi = (2 * i + 1 < nvalid) ? 0xFFFF0000u : 0u;
          w[i] &= (keep_lo | keep_hi);
        }
        vf[j] = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const uint4 pp = *reinterpret_cast<const uint4*>(&pbuf[buf][h][8 * par]);
#pragma unroll
      for (int j = 0; j < J; ++j) acc[h][j] = dot8_bf16(pp, vf[j], acc[h][j]);
    }
  }

#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float l = wave_sum(lsum[h]);
    const int hq = g * G + h;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const float a = acc[h][j] + dpp<kQuadXor1>(acc[h][j]);
      const int d = 32 * j + (lane >> 1);
      if (par == 0) {
        if (slot < 0)
          out[((int64_t)t * num_q_heads + hq) * D + d] = to_bf16(a / l);
        else
          ws.acc[((int64_t)slot * num_q_heads + hq) * D + d] = a;
      }
    }
    if (lane == 0) {
      const float m2 = m[h] * scale_log2;
      if (slot < 0) {
        if (lse) lse[(int64_t)t * num_q_heads + hq] = (m2 + __log2f(l)) * kLn2;
      } else {
        ws.m[(int64_t)slot * num_q_heads + hq] = m2;
        ws.l[(int64_t)slot * num_q_heads + hq] = l;
      }
    }
  }
}

template <int D>
__global__ __launch_bounds__(D) void merge_kernel(const int32_t* __restrict__ merges,
                                                  const int32_t* __restrict__ qsl, int num_q_heads,
                                                  Partials ws, uint16_t* __restrict__ out,
                                                  float* __restrict__ lse) {
  const int4 e = reinterpret_cast<const int4*>(merges)[blockIdx.x];
  const int row = e.x, first = e.y, n = e.z;
  const int h = blockIdx.y, d = threadIdx.x;
  float M = neg_inf();
  for (int i = 0; i < n; ++i) M = fmaxf(M, ws.m[(int64_t)(first + i) * num_q_heads + h]);
  float L = 0.f, o = 0.f;
  for (int i = 0; i < n; ++i) {
    const int64_t ph = (int64_t)(first + i) * num_q_heads + h;
    const float w = fast_exp2(ws.m[ph] - M);
    L += ws.l[ph] * w;
    o += ws.acc[ph * D + d] * w;
  }
  const int t = qsl[row];
  out[((int64_t)t * num_q_heads + h) * D + d] = to_bf16(o / L);
  if (lse && d == 0) lse[(int64_t)t * num_q_heads + h] = (M + __log2f(L)) * kLn2;
}

template <int D, int G>
static void launch_decode_t(const void* q, const void* kc, const void* vc, const int32_t* bt,
                            int bt_stride, const int32_t* qsl, const int32_t* splits,
                            int num_splits, int hq, int hkv, float sl2, void* out, float* lse,
                            Partials ws, hipStream_t stream) {
  hipLaunchKernelGGL((decode_kernel<D, G>), dim3(num_splits * hkv), dim3(64), 0, stream,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(kc),
                     static_cast<const uint16_t*>(vc), bt, bt_stride, qsl, splits, hq, hkv, sl2,
                     static_cast<uint16_t*>(out), lse, ws);
}

hipError_t launch_decode(const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* bt, int bt_stride, const int32_t* qsl,
                         const int32_t* splits, int num_splits, int num_q_heads, int num_kv_heads,
                         int head_dim, float scale_log2, void* out, float* lse, Partials ws,
                         hipStream_t stream) {
  const int G = num_q_heads / num_kv_heads;
#define CPA_DEC(DD, GG)                                                                        \
  if (head_dim == DD && G == GG) {                                                              \
    launch_decode_t<DD, GG>(q, k_cache, v_cache, bt, bt_stride, qsl, splits, num_splits,        \
                            num_q_heads, num_kv_heads, scale_log2, out, lse, ws, stream);       \
    return hipGetLastError();                                                                   \
  }
  CPA_DEC(128, 1) CPA_DEC(128, 2) CPA_DEC(128, 4) CPA_DEC(128, 8)
  CPA_DEC(64, 1) CPA_DEC(64, 2) CPA_DEC(64, 4) CPA_DEC(64, 8)
#undef CPA_DEC
  return hipErrorInvalidValue;
}

hipError_t launch_merge(const int32_t* merges, int num_merges, const int32_t* qsl, int num_q_heads,
                        int head_dim, Partials ws, void* out, float* lse, hipStream_t stream) {
  dim3 grid(num_merges, num_q_heads);
  if (head_dim == 128)
    hipLaunchKernelGGL(merge_kernel<128>, grid, dim3(128), 0, stream, merges, qsl, num_q_heads, ws,
                       static_cast<uint16_t*>(out), lse);
  else
    hipLaunchKernelGGL(merge_kernel<64>, grid, dim3(64), 0, stream, merges, qsl, num_q_heads, ws,
                       static_cast<uint16_t*>(out), lse);
  return hipGetLastError();
}

}  // namespace cpa
