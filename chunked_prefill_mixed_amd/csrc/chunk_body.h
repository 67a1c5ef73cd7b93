// Prefill-chunk flash attention on bf16 matrix cores (gfx950 MFMA), the body
// of one chunk workgroup: the chunk kernel (chunk.hip) and the mixed launch
// (mixed.hip) run it.
//
// A chunk's queries attend to the whole cached prefix of their row (every
// earlier chunk) and causally inside the chunk ("05. Chunked Prefill"
// section 3; tbr8.org deep dive 4.1; "How Chunked Prefill Stops Decode
// Starvation", "The fix"): key k is visible to chunk query j iff
// k <= context_len + j.  Attention cost stays quadratic in the prompt
// ("How Chunked Prefill Stops Decode Starvation", "The payoff"), so with a
// long prefix this kernel is bound by matrix-core throughput.
//
// Workgroup = 4 waves = 128 query rows of one KV head: 128/G tokens times the
// G query heads that share the KV head (their rows share every K/V tile).
// Each wave owns 32 rows, one per lane column n = lane % 32.
//   S^T[64 keys][32 rows] = K Q^T    v_mfma_f32_32x32x16_bf16, K from LDS (A),
//                                    Q^T kept in registers (B)
//   online softmax per row (column) in fp32, P^T rounded to bf16
//   O^T[D][32 rows] += V^T P^T       V^T pages from LDS (A), P^T straight from
//                                    the S^T accumulators (B)
// K rows are fed to the S^T MFMA in a permuted order so that each lane's
// accumulator registers 0-7 / 8-15 hold 8 consecutive keys of one page: that
// is exactly the B-operand layout of the PV MFMA, so P never goes through
// LDS.  V is stored transposed inside each cache page ([D][16]), so the PV
// A operand is one 16-byte read per lane, with no transpose.
// K/V tiles of 64 keys (4 pages) are staged in LDS by all 256 threads with
// global_load_lds_dwordx4 (straight from memory into LDS, no register
// staging); the next tile's loads are in flight while the current one is
// computed.  The lane-to-LDS-slot order of those loads is fixed, so the LDS
// layout is chosen by which 16 bytes each lane fetches.  K pages hold their
// keys in 8-value pieces ([D/8][16][8]) and are copied as they are: the 16
// keys a 16-lane group reads at one piece are 256 contiguous bytes, which
// covers all 64 banks.  V^T rows keep their two 8-key halves swapped when
// bit 3 of d is set (conflict-free fragment reads).  A tile that reaches past
// the piece's last key goes through registers instead, so the V slots past
// the end can be zeroed.
// Only tiles that reach past the first query's last visible key apply the
// causal mask.
//
// A work item may cover only a piece [kv_begin, kv_end) of its tile's keys
// (a long, fully visible prefix is cut into pieces so small chunks still fill
// the GPU); such a piece writes its unnormalised fp32 output, running max and
// sum, and merge_kernel (merge.hip) combines the pieces:
//   M = max m_i,  L = sum l_i 2^(m_i - M),  out = sum acc_i 2^(m_i - M) / L.
// The running max used as the exponent reference is only moved when a tile's
// max exceeds it by more than 2^8, so the 16-64 accumulator rescale almost
// never runs; the sums stay exact because numerator and denominator share the
// reference, and each probability stays below 2^8.

#pragma once

#include <type_traits>

#include "device.h"
#include "internal.h"
#include "tiles.h"

namespace cpa {

// The work of chunk workgroup wg (one work item of the XCD-remapped order).
template <int D, int G>
__device__ __forceinline__ void chunk_body(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_cache,
    const uint16_t* __restrict__ v_cache, const int32_t* __restrict__ bt, int bt_stride,
    const int32_t* __restrict__ qsl, const int32_t* __restrict__ ctx,
    const int32_t* __restrict__ tiles, int num_tiles, int num_q_heads, int num_kv_heads,
    float scale_log2, uint16_t* __restrict__ out, float* __restrict__ lse, Partials part, int wg) {
  constexpr int KS = D / 16;               // 16-wide d steps of S^T = K Q^T
  constexpr int DB = D / 32;               // 32-row d blocks of O^T
  constexpr int PAGE = kBlock * D;         // elements of one (page, KV head)
  constexpr int CHUNKS = 4 * PAGE / 8;     // 16-byte pieces per 64-key tile (K or V)
  constexpr int PER_THREAD = CHUNKS / 256;
  static_assert(CHUNKS % 256 == 0, "tile must split evenly over 256 threads");

  // two stages: one tile is read while the next is written
  __shared__ __align__(16) uint16_t k_lds_buf[2][kKvTile * D];
  __shared__ __align__(16) uint16_t v_lds_buf[2][4 * PAGE];

  const int item = xcd_remap(wg, num_tiles * num_kv_heads);
  const int g = item / num_tiles;
  const int4* tp = reinterpret_cast<const int4*>(tiles) + 2 * (item % num_tiles);
  const int4 te0 = tp[0], te1 = tp[1];
  const int row = te0.x, qb = te0.y, qe = te0.z, kv_begin = te0.w;
  const int kv_end = te1.x, slot = te1.y;  // kv_end <= context + qe
  const int c = ctx[row];
  const int t0 = qsl[row];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int ncol = lane & 31, half = lane >> 5;
  const int r = wave * 32 + ncol;
  int j = qb + r / G;
  const bool row_ok = j < qe;
  if (!row_ok) j = qe - 1;  // ragged tail: recompute the last query, store nothing
  const int hq = g * G + (r % G);
  const int qlimit = c + j;

  // B operand of S^T: Q[j][hq][16ks + 8half .. +8]
  uint4 qf[KS];
  {
    const uint16_t* qrow = q + ((int64_t)(t0 + j) * num_q_heads + hq) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[ks] = *reinterpret_cast<const uint4*>(qrow + 16 * ks + 8 * half);
  }

  // A-operand row this lane supplies to S^T, mapped to a physical key so
  // that accumulator register rr holds key 16*(rr/8) + 8*half + rr%8.
  const int mb = ncol >> 3, mh = (ncol >> 2) & 1, mi = ncol & 3;
  const int krow = 16 * (mb >> 1) + 8 * mh + 4 * (mb & 1) + mi;

  float m = neg_inf(), lsum = 0.f;
  f32x16_t o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[db][i] = 0.f;

  const int32_t* btrow = bt + (int64_t)row * bt_stride;
  const int kt0 = kv_begin / kKvTile;
  const int n_kv = (kv_end + kKvTile - 1) / kKvTile;

  uint4 kreg[PER_THREAD], vreg[PER_THREAD];
  // Page ids come in windows of 64 pages (16 tiles), one id per lane, read a
  // window ahead of their use; a tile's ids are taken with v_readlane.  The
  // pages slot i of a wave stages is the same for all its lanes.
  auto load_window = [&](int w) {
    const int pg = 64 * w + lane;
    return pg * kBlock < kv_end ? btrow[pg] : 0;
  };
  int win = kt0 / 16;  // window held in id_cur
  int id_cur = load_window(win), id_next = load_window(win + 1);
  auto tile_ids = [&](int kt, int (&ids)[PER_THREAD]) {
    if (kt / 16 != win) {  // first tile of the next window
      id_cur = id_next;
      ++win;
      id_next = load_window(win + 1);
    }
#pragma unroll
    for (int i = 0; i < PER_THREAD; ++i) {
      const int pg = kt * 4 + (wave_u * 64 + 256 * i) / (PAGE / 8);
      ids[i] = __builtin_amdgcn_readlane(id_cur, pg - 64 * win);
    }
  };
  // the ragged last tile of a piece, through registers: pages at or past
  // kv_end are not read, V slots past it are zeroed
  auto load_tile = [&](int kt, const int (&ids)[PER_THREAD]) {
#pragma unroll
    for (int i = 0; i < PER_THREAD; ++i) {
      const int cidx = tid + 256 * i;
      const int kp = cidx / (PAGE / 8);
      const int w = cidx % (PAGE / 8);
      const int pg = kt * 4 + kp;
      const int key0 = pg * kBlock;
      if (key0 < kv_end) {
        const int64_t base = ((int64_t)ids[i] * num_kv_heads + g) * PAGE;
        kreg[i] = *reinterpret_cast<const uint4*>(k_cache + base + w * 8);
        uint4 v = *reinterpret_cast<const uint4*>(v_cache + base + w * 8);
        // V piece w covers d = w/2 and page slots 8*(w%2)..+8; zero slots
        // at or past kv_end (unwritten or sentinel data must not reach P*V)
        const int nvalid = kv_end - key0 - 8 * (w & 1);
        if (nvalid < 8) {
          uint32_t x[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t keep = ((2 * e < nvalid) ? 0xFFFFu : 0u) |
                                  ((2 * e + 1 < nvalid) ? 0xFFFF0000u : 0u);
            x[e] &= keep;
          }
          v = make_uint4(x[0], x[1], x[2], x[3]);
        }
        vreg[i] = v;
      } else {
        kreg[i] = make_uint4(0, 0, 0, 0);
        vreg[i] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  // a whole tile below kv_end: thread tid fills 16-byte LDS slot p = tid +
  // 256 i of the K and of the V stage.  Slot p lies in page p / (PAGE / 8) of
  // the tile (the same page for the whole wave) and at the same place inside
  // it for every i: K slot s = p % (PAGE / 8) is the page's own slot s (piece
  // s / 16 of key s % 16); V slot s holds row d = s / 2, half (s & 1) ^ bit 3
  // of d.
  const uint32_t k_lane_bytes = 16u * (tid % (PAGE / 8));
  const int v_s = tid % (PAGE / 8), v_d = v_s >> 1;
  const uint32_t v_lane_bytes = 2u * (v_d * kBlock + 8 * ((v_s & 1) ^ ((v_d >> 3) & 1)));
  auto issue_direct = [&](int stage, const int (&ids)[PER_THREAD]) {
#pragma unroll
    for (int i = 0; i < PER_THREAD; ++i) {
      const int64_t base = ((int64_t)ids[i] * num_kv_heads + g) * PAGE * 2;  // bytes
      const int lds_off = (wave_u * 64 + 256 * i) * 8;
      load_lds16(reinterpret_cast<const char*>(k_cache) + base + k_lane_bytes,
                 &k_lds_buf[stage][lds_off]);
      load_lds16(reinterpret_cast<const char*>(v_cache) + base + v_lane_bytes,
                 &v_lds_buf[stage][lds_off]);
    }
  };
  auto store_tile = [&](int stage) {
    uint16_t* k_lds = k_lds_buf[stage];
    uint16_t* v_lds = v_lds_buf[stage];
#pragma unroll
    for (int i = 0; i < PER_THREAD; ++i) {
      const int cidx = tid + 256 * i;
      const int kp = cidx / (PAGE / 8);
      const int w = cidx % (PAGE / 8);
      *reinterpret_cast<uint4*>(&k_lds[kp * PAGE + w * 8]) = kreg[i];
      // V^T row d = w/2 keeps its two 8-key halves swapped when bit 3 of d is
      // set, so 16 lanes reading half 0 of rows d..d+15 hit distinct banks
      const int d = w >> 1, hh = (w & 1) ^ ((d >> 3) & 1);
      *reinterpret_cast<uint4*>(&v_lds[kp * PAGE + d * kBlock + 8 * hh]) = vreg[i];
    }
  };

  // tile kt is whole (all 64 keys below kv_end) or the ragged last one
  auto whole = [&](int kt) { return (kt + 1) * kKvTile <= kv_end; };
  {
    int ids[PER_THREAD];
    tile_ids(kt0, ids);
    if (whole(kt0)) {
      issue_direct(0, ids);
    } else {
      load_tile(kt0, ids);
      store_tile(0);
    }
  }
  wait_vmem();
  __syncthreads();

  // one 64-key tile; MASK is a compile-time switch so tiles wholly visible to
  // every row of the tile carry no masking code at all.  On entry the tile is
  // in LDS stage (kt - kt0) & 1.
  auto tile = [&](auto mask_tag, int kt) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int stage = (kt - kt0) & 1;
    const uint16_t* k_lds = k_lds_buf[stage];
    const uint16_t* v_lds = v_lds_buf[stage];
    // start the next tile into the other stage (last read in tile kt - 1,
    // before the barrier that ended it)
    const bool more = kt + 1 < n_kv;
    const bool next_whole = whole(kt + 1);
    if (more) {
      int ids[PER_THREAD];
      tile_ids(kt + 1, ids);
      if (next_whole)
        issue_direct(stage ^ 1, ids);
      else
        load_tile(kt + 1, ids);
    }

    // S^T = K Q^T for two 32-key blocks, the two accumulator chains interleaved
    f32x16_t s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
    // K fragments are read kAhead MFMAs before their use, so LDS latency
    // hides behind the MFMAs in flight
    constexpr int kAhead = 4;
    uint4 ka[2 * KS];
#pragma unroll
    for (int i = 0; i < 2 * KS; ++i) {
      // key kr = 32 (i & 1) + krow of the tile, piece 2 (i >> 1) + half
      const int kr = 32 * (i & 1) + krow;
      ka[i] = *reinterpret_cast<const uint4*>(
          &k_lds[(kr / kBlock) * PAGE + ((2 * (i >> 1) + half) * kBlock + kr % kBlock) * 8]);
    }
#pragma unroll
    for (int i = 0; i < 2 * KS; ++i)
      s[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, ka[i]),
                                                         __builtin_bit_cast(bf16x8_t, qf[i >> 1]),
                                                         s[i & 1], 0, 0, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);
#pragma unroll
    for (int i = 0; i < 2 * KS - kAhead; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kAhead, 0);

    if constexpr (MASK) {
      const int key_base = kt * kKvTile;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          const int key = key_base + 32 * kb + 16 * (rr >> 3) + 8 * half + (rr & 7);
          if (key > qlimit) s[kb][rr] = neg_inf();
        }
    }

    // the first PV A operands (V^T fragments, independent of P) are read
    // now, so their LDS latency hides behind the softmax below
    const int vh = half ^ ((ncol >> 3) & 1);  // the swizzled half holding keys 8*half..
    auto vfrag = [&](int i) {  // i = kp * DB + db
      return *reinterpret_cast<const uint4*>(
          &v_lds[(i / DB) * PAGE + (32 * (i % DB) + ncol) * kBlock + 8 * vh]);
    };
    constexpr int kVAhead = 4;
    uint4 va[kVAhead];
#pragma unroll
    for (int i = 0; i < kVAhead; ++i) va[i] = vfrag(i);
    __builtin_amdgcn_sched_barrier(0);

    // tile max per row (four independent chains, then across the half-waves)
    float pm[4] = {neg_inf(), neg_inf(), neg_inf(), neg_inf()};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) pm[rr & 3] = fmaxf(pm[rr & 3], s[kb][rr]);
    const float mx = half_max(fmaxf(fmaxf(pm[0], pm[1]), fmaxf(pm[2], pm[3])));

    // probabilities against the current reference max, bf16-rounded as the
    // PV product uses them, and their row sum (two per v_dot2, four partial
    // sums).  They are computed before the tile max is known, and computed
    // again in the rare case the reference has to move.
    uint4 pb[4];
    float ps[4];
    auto probs = [&](float msc) {
#pragma unroll
      for (int kp = 0; kp < 4; ++kp) {
        float pv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
          pv[i] = fast_exp2(__builtin_fmaf(s[kp >> 1][8 * (kp & 1) + i], scale_log2, -msc));
        pb[kp] = make_uint4(pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]),
                            pack_bf16x2(pv[4], pv[5]), pack_bf16x2(pv[6], pv[7]));
        ps[kp] = sum2_bf16(pb[kp].w,
                           sum2_bf16(pb[kp].z, sum2_bf16(pb[kp].y, sum2_bf16(pb[kp].x, 0.f))));
      }
    };
    probs(m * scale_log2);
    // move the reference max only when this tile exceeds it by more than 2^8
    // (always on a row's first tile, where m is -inf)
    const bool grow = (mx - m) * scale_log2 > 8.f;
    if (__builtin_expect(__any(grow), 0)) {
      // rare: rescale the running sums; the empty asm keeps the compiler from
      // hoisting this out of the branch and running it on every tile
      asm volatile("" ::: "memory");
      const float mn = grow ? mx : m;
      const float alpha = fast_exp2((m - mn) * scale_log2);
      m = mn;
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
      probs(m * scale_log2);
    }
    lsum += (ps[0] + ps[1]) + (ps[2] + ps[3]);

    // O^T += V^T P^T, one page (16 keys) per MFMA, the DB accumulator chains
    // interleaved; V fragments read kVAhead MFMAs before their use
#pragma unroll
    for (int i = 0; i < 4 * DB; ++i) {
      const uint4 a = va[i % kVAhead];
      if (i + kVAhead < 4 * DB) va[i % kVAhead] = vfrag(i + kVAhead);
      o[i % DB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                          __builtin_bit_cast(bf16x8_t, pb[i / DB]),
                                                          o[i % DB], 0, 0, 0);
    }

    // the next tile must be in LDS before any wave reads it
    if (more) {
      if (!next_whole) store_tile(stage ^ 1);
      wait_vmem();
      __syncthreads();
    }
  };

  // tile kt needs the causal mask iff its last key is past the tile's first
  // query's limit: kt*64 + 63 > context + q_begin
  const int kt_mask = max(kt0, min(n_kv, (c + qb + 1) / kKvTile));
  for (int kt = kt0; kt < kt_mask; ++kt) tile(std::integral_constant<bool, false>(), kt);
  for (int kt = kt_mask; kt < n_kv; ++kt) tile(std::integral_constant<bool, true>(), kt);

  lsum = half_sum(lsum);
  if (row_ok && slot >= 0) {
    // one piece of a split tile: unnormalised partial for merge_kernel
    const int64_t pr = ((int64_t)slot * num_kv_heads + g) * kChunkRows + r;
    float* acc = part.acc + pr * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = 32 * db + 8 * g4 + 4 * half;
        *reinterpret_cast<float4*>(acc + d) =
            make_float4(o[db][4 * g4 + 0], o[db][4 * g4 + 1], o[db][4 * g4 + 2], o[db][4 * g4 + 3]);
      }
    if (half == 0) {
      part.m[pr] = m * scale_log2;
      part.l[pr] = lsum;
    }
  } else if (row_ok) {
    const float inv = 1.f / lsum;
    uint16_t* orow = out + ((int64_t)(t0 + j) * num_q_heads + hq) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = 32 * db + 8 * g4 + 4 * half;
        uint2 v;
        v.x = pack_bf16x2(o[db][4 * g4 + 0] * inv, o[db][4 * g4 + 1] * inv);
        v.y = pack_bf16x2(o[db][4 * g4 + 2] * inv, o[db][4 * g4 + 3] * inv);
        *reinterpret_cast<uint2*>(orow + d) = v;
      }
    if (lse && half == 0)
      lse[(int64_t)(t0 + j) * num_q_heads + hq] = (m * scale_log2 + __log2f(lsum)) * kLn2;
  }
}

}  // namespace cpa
