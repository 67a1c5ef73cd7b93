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
//   K page [16][D]: lane l owns keys l/8 and l/8 + 8 and the 8-wide d
//     pieces (l%8)*8 + 64j; each 16-byte load instruction of the wave reads
//     8 whole 128-byte lines (8 lanes per key row).  Scores: v_dot2_f32_bf16
//     over the lane's d pieces, then a 3-step DPP sum over the row's 8 lanes.
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

#ifndef CPA_DECODE_WAVES_PER_WG
#define CPA_DECODE_WAVES_PER_WG 4   // independent (split, KV head) items per workgroup
#endif

namespace cpa {

constexpr int kDecodeWaves = CPA_DECODE_WAVES_PER_WG;

// Orders one wave's LDS writes before its own later LDS reads by other lanes
// (LDS executes a wave's operations in order; this stops the compiler from
// moving them and makes the writes visible at wavefront scope).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

template <int D, int G>
__global__ __launch_bounds__(64 * kDecodeWaves) void decode_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_cache,
    const uint16_t* __restrict__ v_cache, const int32_t* __restrict__ bt, int bt_stride,
    const int32_t* __restrict__ qsl, const int32_t* __restrict__ splits, int num_q_heads,
    int num_kv_heads, int num_items, float scale_log2, uint16_t* __restrict__ out,
    float* __restrict__ lse, Partials ws) {
  constexpr int J = D / 32;   // 16-byte V pieces per lane per page
  constexpr int JK = D / 64;  // 16-byte K pieces per lane per key (2 keys per lane)
  __shared__ __align__(16) uint16_t pbuf_all[kDecodeWaves][2][G][kBlock];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int item = blockIdx.x * kDecodeWaves + wave;
  if (item >= num_items) return;  // whole wave; no workgroup barrier below
  auto& pbuf = pbuf_all[wave];
  const int g = item % num_kv_heads;
  const int sp = item / num_kv_heads;
  const int4 e = reinterpret_cast<const int4*>(splits)[sp];
  const int row = e.x, kv_begin = e.y, kv_end = e.z, slot = e.w;
  // decode rows come first and hold one token each, so row s is packed token s
  const int t = row;
  (void)qsl;
  const int kg = lane >> 3, dp = lane & 7, par = lane & 1;

  uint4 qf[G][JK];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int j = 0; j < JK; ++j)
      qf[h][j] = *reinterpret_cast<const uint4*>(
          q + ((int64_t)t * num_q_heads + g * G + h) * D + dp * 8 + 64 * j);

  float m[G], lsum[G], acc[G][J];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = neg_inf();
    lsum[h] = 0.f;
#pragma unroll
    for (int j = 0; j < J; ++j) acc[h][j] = 0.f;
  }

  const int32_t* btrow = bt + (int64_t)row * bt_stride;
  // a split spans at most 64 pages (the planner guarantees it): one coalesced
  // load of its page ids, then v_readlane per page
  const int pg0 = kv_begin / kBlock, npages = (kv_end + kBlock - 1) / kBlock - pg0;
  const int my_blk = lane < npages ? btrow[pg0 + lane] : 0;
  auto page_base = [&](int i) -> int64_t {
    const int blk = __builtin_amdgcn_readlane(my_blk, i);
    return ((int64_t)blk * num_kv_heads + g) * (kBlock * D);
  };
  // per-lane offsets inside a (page, KV head) piece, in 16-byte units; the
  // page base is wave-uniform, so every load is scalar base + fixed 32-bit
  // lane offset and no address register is rewritten per page
  const uint32_t koff = (uint32_t)(kg * D + dp * 8) / 8;
  const uint32_t voff = (uint32_t)lane;
  // two register sets, used in turn: while one page is computed the other's
  // loads are in flight, and each compute waits only for its own page
  uint4 ka[2 * JK], va[J], kb[2 * JK], vb[J];
  auto load_page = [&](int64_t page, uint4 (&kd)[2 * JK], uint4 (&vd)[J]) {
    const uint4* kp = reinterpret_cast<const uint4*>(k_cache + page);
    const uint4* vp = reinterpret_cast<const uint4*>(v_cache + page);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int j = 0; j < JK; ++j) kd[ks * JK + j] = kp[koff + (8 * ks * D + 64 * j) / 8];
#pragma unroll
    for (int j = 0; j < J; ++j) vd[j] = vp[voff + j * 64];
  };
  auto compute_page = [&](int i, uint4 (&kc)[2 * JK], uint4 (&vc)[J]) {
    const int pg = pg0 + i;
    const int buf = i & 1;
    const bool valid0 = pg * kBlock + kg < kv_end;
    const bool valid1 = pg * kBlock + kg + 8 < kv_end;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float a0 = 0.f, a1 = 0.f;
#pragma unroll
      for (int j = 0; j < JK; ++j) {
        a0 = dot8_bf16(qf[h][j], kc[j], a0);
        a1 = dot8_bf16(qf[h][j], kc[JK + j], a1);
      }
      a0 += dpp<kQuadXor1>(a0);
      a1 += dpp<kQuadXor1>(a1);
      a0 += dpp<kQuadXor2>(a0);
      a1 += dpp<kQuadXor2>(a1);
      a0 += dpp<kRowHalfMirror>(a0);
      a1 += dpp<kRowHalfMirror>(a1);
      const float s0 = valid0 ? a0 : neg_inf();
      const float s1 = valid1 ? a1 : neg_inf();
      float mx = fmaxf(s0, s1);
      mx = fmaxf(mx, dpp<kRowMirror>(mx));
      mx = fmaxf(mx, xor_lane(mx, 16));
      mx = fmaxf(mx, xor_lane(mx, 32));
      const float mn = fmaxf(m[h], mx);
      const float alpha = fast_exp2((m[h] - mn) * scale_log2);
      m[h] = mn;
      const float p0 = fast_exp2((s0 - mn) * scale_log2);
      const float p1 = fast_exp2((s1 - mn) * scale_log2);
      lsum[h] = lsum[h] * alpha + (dp == 0 ? p0 + p1 : 0.f);
#pragma unroll
      for (int j = 0; j < J; ++j) acc[h][j] *= alpha;
      // the row's 8 lanes hold the same two scores; lane dp publishes value
      // dp, dp+8, ... of the (key slot, head) pairs
#pragma unroll
      for (int v = 0; v < 2 * G; v += 8)
        if (v + dp < 2 * G && (v + dp) % G == h)
          pbuf[buf][h][kg + 8 * ((v + dp) / G)] = to_bf16((v + dp) / G ? p1 : p0);
    }
    // keys past the split's end in its last page: their V slots may hold
    // anything (even NaN); zero them so 0 * V stays 0
    const int nvalid = kv_end - pg * kBlock - 8 * par;
    if (nvalid < 8) {
#pragma unroll
      for (int j = 0; j < J; ++j) {
        uint32_t w[4] = {vc[j].x, vc[j].y, vc[j].z, vc[j].w};
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          const uint32_t keep_lo = (2 * e2 < nvalid) ? 0xFFFFu : 0u;
          const uint32_t keep_hi = (2 * e2 + 1 < nvalid) ? 0xFFFF0000u : 0u;
          w[e2] &= (keep_lo | keep_hi);
        }
        vc[j] = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
    wave_lds_sync();
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const uint4 pp = *reinterpret_cast<const uint4*>(&pbuf[buf][h][8 * par]);
#pragma unroll
      for (int j = 0; j < J; ++j) acc[h][j] = dot8_bf16(pp, vc[j], acc[h][j]);
    }
  };

  // pages in pairs with no early exit: for an odd count the pair's second
  // page is past the split end, every key of it is masked (p = 0, the
  // running max and sums are unchanged) and its loads re-read the last page
  // (an L2 hit), which keeps the loop free of branches around the loads
  load_page(page_base(0), ka, va);
  const int npairs = (npages + 1) / 2;
  for (int ip = 0; ip < npairs; ++ip) {
    const int i = 2 * ip;
    load_page(page_base(min(i + 1, npages - 1)), kb, vb);
    compute_page(i, ka, va);
    load_page(page_base(min(i + 2, npages - 1)), ka, va);
    compute_page(i + 1, kb, vb);
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

// Combine the splits of a decode row: one wave per (row, query head).  The
// lanes read the splits' max and sum in parallel; each lane then owns D/64
// output dimensions and sums the splits' fp32 partials for them.
template <int D>
__global__ __launch_bounds__(64) void merge_kernel(const int32_t* __restrict__ merges,
                                                   const int32_t* __restrict__ qsl, int num_q_heads,
                                                   Partials ws, uint16_t* __restrict__ out,
                                                   float* __restrict__ lse) {
  constexpr int PER = D / 64;
  const int4 e = reinterpret_cast<const int4*>(merges)[blockIdx.x];
  const int row = e.x, first = e.y, n = e.z;
  const int h = blockIdx.y, lane = threadIdx.x;
  float M = neg_inf();
  for (int i = lane; i < n; i += 64) M = fmaxf(M, ws.m[(int64_t)(first + i) * num_q_heads + h]);
  M = wave_max(M);
  float L = 0.f;
  for (int i = lane; i < n; i += 64) {
    const int64_t ph = (int64_t)(first + i) * num_q_heads + h;
    L += ws.l[ph] * fast_exp2(ws.m[ph] - M);
  }
  L = wave_sum(L);
  float o[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) o[k] = 0.f;
#pragma unroll 4
  for (int i = 0; i < n; ++i) {
    const int64_t ph = (int64_t)(first + i) * num_q_heads + h;
    const float w = fast_exp2(ws.m[ph] - M);
#pragma unroll
    for (int k = 0; k < PER; ++k) o[k] += w * ws.acc[ph * D + lane + 64 * k];
  }
  const int t = qsl[row];
  const float inv = 1.f / L;
#pragma unroll
  for (int k = 0; k < PER; ++k)
    out[((int64_t)t * num_q_heads + h) * D + lane + 64 * k] = to_bf16(o[k] * inv);
  if (lse && lane == 0) lse[(int64_t)t * num_q_heads + h] = (M + __log2f(L)) * kLn2;
}

template <int D, int G>
static void launch_decode_t(const void* q, const void* kc, const void* vc, const int32_t* bt,
                            int bt_stride, const int32_t* qsl, const int32_t* splits,
                            int num_splits, int hq, int hkv, float sl2, void* out, float* lse,
                            Partials ws, hipStream_t stream) {
  const int items = num_splits * hkv;
  hipLaunchKernelGGL((decode_kernel<D, G>), dim3((items + kDecodeWaves - 1) / kDecodeWaves),
                     dim3(64 * kDecodeWaves), 0, stream, static_cast<const uint16_t*>(q),
                     static_cast<const uint16_t*>(kc), static_cast<const uint16_t*>(vc), bt,
                     bt_stride, qsl, splits, hq, hkv, items, sl2, static_cast<uint16_t*>(out), lse,
                     ws);
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
    hipLaunchKernelGGL(merge_kernel<128>, grid, dim3(64), 0, stream, merges, qsl, num_q_heads, ws,
                       static_cast<uint16_t*>(out), lse);
  else
    hipLaunchKernelGGL(merge_kernel<64>, grid, dim3(64), 0, stream, merges, qsl, num_q_heads, ws,
                       static_cast<uint16_t*>(out), lse);
  return hipGetLastError();
}

}  // namespace cpa
