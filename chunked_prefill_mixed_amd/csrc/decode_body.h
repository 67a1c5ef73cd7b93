// Split-KV decode attention, the body of one decode workgroup: the decode
// kernel (decode.hip) and the mixed launch (mixed.hip) run it.  Its pieces
// are merged by merge_kernel (merge.hip).
//
// A decode row's single query reads its whole cached context from HBM each
// step ("How Chunked Prefill Stops Decode Starvation", "The stall"; tbr8.org
// deep dive section 1), so this kernel is bound by HBM bandwidth: about 4
// flops per byte of K/V at 4 query heads per KV head.
//
// One wave per (key piece, KV head).  All G query heads that share the KV
// head are served by the one read of each 16-token page, and both products
// run on the matrix cores so the wave's vector work per page stays small
// next to the time its 8 KiB take to arrive:
//   S^T[16 keys][16 cols] = K Q^T      v_mfma_f32_16x16x32_bf16, D/32 steps;
//                                      K pages hold their keys in 8-value
//                                      pieces ([D/8][16][8]), so the A operand
//                                      of step kk (pieces 4kk..4kk+3 of all 16
//                                      keys) is one contiguous 1 KB load;
//                                      column n of Q^T holds query head n of
//                                      the group (16 per block; a run-time
//                                      group holds two blocks per wave against
//                                      the same K/V, one wave per 32 heads;
//                                      columns past the group repeat a head
//                                      and are never stored)
//   O^T[D][16 cols] += V^T P^T         v_mfma_f32_16x16x16_bf16, D/16 blocks;
//                                      V pages are stored transposed ([D][16])
//                                      so each lane loads its A operand as 8
//                                      contiguous bytes, and P^T is the S^T
//                                      accumulator itself (lane (g4, n) holds
//                                      keys 4*g4..+4 of column n in both)
// Online softmax per column in fp32: the 4 keys of a lane, then across the 4
// lane groups with two exchanges.  The reference max only moves when a page
// exceeds it by more than 2^8 (always on the first page), so the accumulator
// rescale is rare; numerator and denominator share the reference.  A row
// covered by one piece writes its bf16 output directly; otherwise each piece
// writes unnormalised fp32 (acc, max, sum) and merge_kernel (merge.hip) combines
// them:
//   M = max m_i,  L = sum l_i 2^(m_i - M),  out = sum acc_i 2^(m_i - M) / L.

#pragma once

#include "device.h"
#include "internal.h"
#include "tiles.h"

#ifndef CPA_DECODE_STAGES
#define CPA_DECODE_STAGES 2   // pages each wave holds in registers: one computed, the rest loading
#endif

namespace cpa {

constexpr int kDecodeWaves = 4;  // independent (piece, KV head) waves per workgroup
constexpr int kStages = CPA_DECODE_STAGES;

typedef short short4_t __attribute__((ext_vector_type(4)));

// The work of one decode wave: wave w of the workgroup takes item
// first_item + w (kDecodeWaves waves per decode-kernel workgroup; the mixed
// launch's decode workgroups have the chunk workgroup's waves).
template <int D, int G>
__device__ __forceinline__ void decode_body(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_cache,
    const uint16_t* __restrict__ v_cache, const int32_t* __restrict__ bt, int bt_stride,
    const int32_t* __restrict__ splits, int num_q_heads, int num_kv_heads, int num_items,
    float scale_log2, uint16_t* __restrict__ out, float* __restrict__ lse, Partials ws,
    int first_item) {
  constexpr int KK = D / 32;  // S^T steps over d
  constexpr int MB = D / 16;  // O^T blocks of 16 d rows
  constexpr int PAGE_BYTES = kBlock * D * 2;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int item = first_item + wave;  // wave w of the workgroup takes item first_item + w
  if (item >= num_items) return;  // whole wave; no workgroup barrier below
  // query heads per KV head: compiled in (at most 8, one block of 16
  // columns), or (G = 0) read at run time, in ceil(G / 16) blocks of 16
  // columns, up to NB of them per wave against the same K/V registers:
  // item = (piece x KV head) x waves + wave of the group
  static_assert(G >= 0 && G <= kDecodeCols, "compiled groups fit one block of columns");
  constexpr int NB = G > 0 ? 1 : kDecodeWaveBlocks;
  const int grp = G > 0 ? G : num_q_heads / num_kv_heads;
  const int nwv = G > 0 ? 1 : decode_group_waves(grp);
  const int wv = G > 0 ? 0 : item % nwv;
  const int pk = G > 0 ? item : item / nwv;
  const int g = pk % num_kv_heads;
  const int4 e = reinterpret_cast<const int4*>(splits)[pk / num_kv_heads];
  const int row = e.x, kv_begin = e.y, kv_end = e.z, slot = e.w;
  // decode rows come first and hold one token each, so row s is packed token s
  const int t = row;
  const int n = lane & 15;   // column of S^T and O^T
  const int g4 = lane >> 4;  // lane group: d pieces of S^T, keys 4*g4..+4 of P^T and O^T
  // blocks of this wave that hold heads of the group (wave-uniform: the last
  // wave of an odd block count holds one)
  const bool two = NB > 1 && decode_column_blocks(grp) - NB * wv > 1;
  // block b's column n holds query head col[b] of the group; columns past the
  // group repeat a head of it and are never stored
  constexpr int kGroup = G > 0 ? G : 1;  // the compiled group (a divisor in the G > 0 path)
  int col[NB], hq[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    col[b] = kDecodeCols * (NB * wv + b) + n;
    hq[b] = g * grp + (G > 0 ? n % kGroup : min(col[b], grp - 1));
  }

  // B operand of S^T: Q[hq][32 kk + 8 g4 .. +8]
  uint4 qf[NB][KK];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const uint16_t* qrow = q + ((int64_t)t * num_q_heads + hq[b]) * D + 8 * g4;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) qf[b][kk] = *reinterpret_cast<const uint4*>(qrow + 32 * kk);
  }

  const int32_t* btrow = bt + (int64_t)row * bt_stride;
  // a piece spans at most 64 pages (the planner guarantees it): one
  // coalesced load of its page ids, then v_readlane per page
  const int pg0 = kv_begin / kBlock, npages = (kv_end + kBlock - 1) / kBlock - pg0;
  const int my_blk = btrow[pg0 + min(lane, npages - 1)];
  // Loads go through a buffer resource built per page from the wave-uniform
  // page address: scalar base, fixed per-lane byte offsets, and the hardware
  // range check keeps every access inside the one (page, KV head) piece.
  // K[n][32 kk + 8 g4 ..] is piece 4 kk + g4 of key n: byte 1024 kk + 16 (16 g4 + n)
  const uint32_t kbyte = (uint32_t)lane * 16;              // + 1024 kk
  const uint32_t vbyte = (uint32_t)(n * kBlock + 4 * g4) * 2;  // + 512 mb: V^T[16 mb + n][4 g4 ..]
  uint4 kset[kStages][KK];
  uint2 vset[kStages][MB];
  auto load_page = [&](int i, uint4 (&kd)[KK], uint2 (&vd)[MB]) {
    const int blk = __builtin_amdgcn_readlane(my_blk, i);
    const int64_t page = ((int64_t)blk * num_kv_heads + g) * (kBlock * D);
    const auto kr = make_page_rsrc(k_cache + page, PAGE_BYTES);
    const auto vr = make_page_rsrc(v_cache + page, PAGE_BYTES);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) kd[kk] = buffer_load16<kNonTemporal>(kr, kbyte + 1024 * kk);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) vd[mb] = buffer_load8<kNonTemporal>(vr, vbyte + 512 * mb);
  };

  float m[NB], lsum[NB];
  f32x4_t acc[NB][MB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    m[b] = neg_inf();
    lsum[b] = 0.f;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[b][mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  // one block's softmax and O^T update for the page, from its S^T
  auto softmax_pv = [&](int b, f32x4_t s, const uint2 (&vc)[MB]) {
    float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    mx = fmaxf(mx, xor_lane(mx, 16));
    mx = fmaxf(mx, xor_lane(mx, 32));
    // move the reference max only when this page exceeds it by more than 2^8
    // (always on the first page, where m is -inf)
    const bool grow = (mx - m[b]) * scale_log2 > 8.f;
    if (__any(grow)) {
      // rare: rescale the running sums; the empty asm keeps the compiler from
      // hoisting this out of the branch and running it on every page
      asm volatile("" ::: "memory");
      const float mn = grow ? mx : m[b];
      const float alpha = fast_exp2((m[b] - mn) * scale_log2);
      m[b] = mn;
      lsum[b] *= alpha;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) acc[b][mb] *= alpha;
    }
    const float msc = m[b] * scale_log2;
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) p[r] = fast_exp2(__builtin_fmaf(s[r], scale_log2, -msc));
    lsum[b] += (p[0] + p[1]) + (p[2] + p[3]);
    const uint2 pb = make_uint2(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]));
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
      acc[b][mb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
          __builtin_bit_cast(short4_t, vc[mb]), __builtin_bit_cast(short4_t, pb), acc[b][mb], 0,
          0, 0);
  };
  auto compute_page = [&](int i, const uint4 (&kc)[KK], uint2 (&vc)[MB]) {
    const int key0 = (pg0 + i) * kBlock;
    f32x4_t s[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      s[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      if (b > 0 && !two) continue;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        s[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kc[kk]),
                                                       __builtin_bit_cast(bf16x8_t, qf[b][kk]),
                                                       s[b], 0, 0, 0);
    }
    // the piece's last page (or one past it): mask keys at or past kv_end,
    // and zero their V entries (unwritten or sentinel data must not reach
    // P*V, where 0 * NaN would not vanish).  The test is wave-uniform.
    if (key0 + kBlock > kv_end) {
      const int nvalid = kv_end - key0 - 4 * g4;
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (r >= nvalid) s[b][r] = neg_inf();
      const uint32_t keep0 = (nvalid > 0 ? 0xFFFFu : 0u) | (nvalid > 1 ? 0xFFFF0000u : 0u);
      const uint32_t keep1 = (nvalid > 2 ? 0xFFFFu : 0u) | (nvalid > 3 ? 0xFFFF0000u : 0u);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) vc[mb] = make_uint2(vc[mb].x & keep0, vc[mb].y & keep1);
    }
    softmax_pv(0, s[0], vc);
#pragma unroll
    for (int b = 1; b < NB; ++b)
      if (two) softmax_pv(b, s[b], vc);
  };

  // pages in groups of kStages with no early exit: pages past the piece end
  // are masked in full (p = 0; the running max and sums are unchanged) and
  // their loads re-read the last page (an L2 hit), which keeps the loop free
  // of branches around the loads
#pragma unroll
  for (int u = 0; u + 1 < kStages; ++u) load_page(min(u, npages - 1), kset[u], vset[u]);
  for (int i0 = 0; i0 < npages; i0 += kStages) {
#pragma unroll
    for (int u = 0; u < kStages; ++u) {
      constexpr int kLast = kStages - 1;
      load_page(min(i0 + u + kLast, npages - 1), kset[(u + kLast) % kStages],
                vset[(u + kLast) % kStages]);
      compute_page(i0 + u, kset[u], vset[u]);
    }
  }

  // column sums over the 4 lane groups (each summed its own keys), with every
  // lane active
  float ls[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    ls[b] = lsum[b] + xor_lane(lsum[b], 16);
    ls[b] += xor_lane(ls[b], 32);
  }
  const int d0 = 4 * g4;  // this lane's O^T rows inside each 16-row block
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    if (b > 0 && !two) break;
    if (col[b] >= grp) continue;
    if (slot < 0) {
      const float inv = 1.f / ls[b];
      uint16_t* orow = out + ((int64_t)t * num_q_heads + hq[b]) * D + d0;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        *reinterpret_cast<uint2*>(orow + 16 * mb) =
            make_uint2(pack_bf16x2(acc[b][mb][0] * inv, acc[b][mb][1] * inv),
                       pack_bf16x2(acc[b][mb][2] * inv, acc[b][mb][3] * inv));
      if (lse && g4 == 0)
        lse[(int64_t)t * num_q_heads + hq[b]] = (m[b] * scale_log2 + __log2f(ls[b])) * kLn2;
    } else {
      const int64_t ph = (int64_t)slot * num_q_heads + hq[b];
      float* arow = ws.acc + ph * D + d0;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        *reinterpret_cast<float4*>(arow + 16 * mb) =
            make_float4(acc[b][mb][0], acc[b][mb][1], acc[b][mb][2], acc[b][mb][3]);
      if (g4 == 0) {
        ws.m[ph] = m[b] * scale_log2;
        ws.l[ph] = ls[b];
      }
    }
  }
}

}  // namespace cpa
