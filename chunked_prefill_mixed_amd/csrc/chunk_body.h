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
// Workgroup = W = chunk_waves(D) waves = 32 W query rows of one KV head (256
// at head_dim 128, 128 at 64): floor(32 W / G) tokens times the G query heads
// that share the KV head; all its rows share every K/V tile it loads.  Each wave
// owns 32 rows, one per lane column n = lane % 32.
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
//
// Software pipeline, one 64-key tile t per iteration: the matrix cores
// compute S(t+1) = K(t+1) Q^T while the vector units turn S(t) into
// probabilities, then O += V(t) P(t).  So each wave always has matrix work
// to overlap with its own exponentials, whatever the other wave on its SIMD
// is doing.  K runs two tiles ahead of its use and V one, in two LDS stages
// each: iteration t loads K(t+2) into the stage K(t) used and V(t+1) into
// the stage V(t-1) used, with one barrier per tile.  The loads go straight
// from memory into LDS (global_load_lds_dwordx4, by all the threads, issued
// as inline assembly so the compiler does not make the current tile's LDS
// reads wait for them).  The lane-to-LDS-slot order of those loads is fixed,
// so the LDS layout is chosen by which 16 bytes each lane fetches.  K pages
// hold their keys in 8-value pieces ([D/8][16][8]) and are copied as they
// are: the 16 keys a 16-lane group reads at one piece are 256 contiguous
// bytes, which covers all 64 banks.  V^T rows keep their two 8-key halves
// swapped when bit 3 of d is set (conflict-free fragment reads).
//
// The last tile of a piece may reach past the piece's last key: its pages at
// or past the end load page 0 (any valid page) instead.  Its keys past the
// end lie past every row's causal limit, so the mask removes their scores;
// their V values (unwritten or stale slots, possibly NaN) are zeroed in the
// fragment registers before the PV product, where 0 * NaN would not vanish.
// Only tiles that reach past the first query's last visible key apply the
// causal mask.
//
// A work item may cover only a piece [kv_begin, kv_end) of its tile's keys
// (a long, fully visible prefix is cut into pieces so small chunks still fill
// the GPU); such a piece writes its output over its own keys o_i (normalised
// by its own sum, in bf16), its running max m_i and sum l_i, and merge_kernel
// (merge.hip) combines the pieces:
//   M = max m_i,  L = sum l_i 2^(m_i - M),  out = sum l_i 2^(m_i - M) o_i / L.
// The running max used as the exponent reference is the first tile's row max
// and moves only when a later tile's max exceeds it by more than 8 (log2
// units of the scaled score), so the 16-64 accumulator rescale almost never
// runs; the sums stay exact because numerator and denominator share the
// reference, and each probability stays below 2^8.

#pragma once

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
    float scale_log2, uint16_t* __restrict__ out, float* __restrict__ lse, ChunkPartials part, int wg) {
  constexpr int KS = D / 16;               // 16-wide d steps of S^T = K Q^T
  constexpr int DB = D / 32;               // 32-row d blocks of O^T
  constexpr int PAGE = kBlock * D;         // elements of one (page, KV head)
  constexpr int CHUNKS = 4 * PAGE / 8;     // 16-byte pieces per 64-key tile (K or V)
  constexpr int NT = 64 * chunk_waves(D);  // threads of the workgroup
  constexpr int ROWS = chunk_rows(D);      // query rows of the workgroup
  constexpr int PER_THREAD = CHUNKS / NT;
  static_assert(CHUNKS % NT == 0, "tile must split evenly over the threads");
  static_assert(NT % (PAGE / 8) == 0, "a thread's load slots sit at one place in every page");

  // two stages each: K(t+1) is read while K(t+2) is written, V(t) while V(t+1)
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
  // query heads per KV head: compiled in, or (G = 0) read at run time
  const int grp = G > 0 ? G : num_q_heads / num_kv_heads;
  int r = wave * 32 + ncol;  // the wave's row, one per lane column
  int j = qb + r / grp;
  const bool row_ok = j < qe;
  if (!row_ok) j = qe - 1;  // ragged tail: recompute the last query, store nothing
  const int hq = g * grp + (r % grp);
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

  f32x16_t o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[db][i] = 0.f;

  const int32_t* btrow = bt + (int64_t)row * bt_stride;
  const int kt0 = kv_begin / kKvTile;
  const int n_kv = (kv_end + kKvTile - 1) / kKvTile;

  // Page ids come in windows of 64 pages (16 tiles), one id per lane, read a
  // window ahead of their use.  Pages at or past kv_end read as page 0, so the
  // last tile's loads stay inside the pool.  id_cur holds window win and
  // id_next window win + 1; the K loads, the leading ones, move them on.
  auto load_window = [&](int w) {
    const int pg = 64 * w + lane;
    return pg * kBlock < kv_end ? btrow[pg] : 0;
  };
  int win = kt0 / 16;
  int id_cur = load_window(win), id_next = load_window(win + 1);
  // Load slot i of this wave covers 16-byte slot p = tid + NT i of a stage:
  // page p / (PAGE / 8) of the tile (the same page for the whole wave) at the
  // same place inside it for every i.  K slot s = p % (PAGE / 8) is the
  // page's own slot s (piece s / 16 of key s % 16); V slot s holds row
  // d = s / 2, half (s & 1) ^ bit 3 of d.
  const uint32_t k_lane_bytes = 16u * (tid % (PAGE / 8));
  const int v_s = tid % (PAGE / 8), v_d = v_s >> 1;
  const uint32_t v_lane_bytes = 2u * (v_d * kBlock + 8 * ((v_s & 1) ^ ((v_d >> 3) & 1)));
  // byte offset, in either cache, of this KV head's part of the page under
  // load slot i of tile kt (wave-uniform); computed once per tile, when its
  // K is loaded, and used again for its V one iteration later
  const char* k_head = reinterpret_cast<const char*>(k_cache) + (int64_t)g * PAGE * 2;
  const char* v_head = reinterpret_cast<const char*>(v_cache) + (int64_t)g * PAGE * 2;
  const uint32_t page_bytes = (uint32_t)num_kv_heads * PAGE * 2;  // below 2^21 (kMaxKvHeads)
  auto page_offsets = [&](int kt, int64_t (&off)[PER_THREAD]) {
    if ((kt >> 4) != win) {  // tiles advance one at a time: at most one window
      id_cur = id_next;
      ++win;
      id_next = load_window(win + 1);
    }
#pragma unroll
    for (int i = 0; i < PER_THREAD; ++i) {
      const int pg = kt * 4 + (wave_u * 64 + NT * i) / (PAGE / 8);
      // page ids are non-negative: an unsigned 32 x 32 -> 64-bit product
      off[i] = (int64_t)((uint64_t)(uint32_t)__builtin_amdgcn_readlane(id_cur, pg & 63) *
                         page_bytes);
    }
  };
  auto issue_k = [&](const int64_t (&off)[PER_THREAD], int stage) {
#pragma unroll
    for (int i = 0; i < PER_THREAD; ++i)
      load_lds16(k_head + off[i], k_lane_bytes,
                 lds_address(&k_lds_buf[stage][(wave_u * 64 + NT * i) * 8]));
  };
  auto issue_v = [&](const int64_t (&off)[PER_THREAD], int stage) {
#pragma unroll
    for (int i = 0; i < PER_THREAD; ++i)
      load_lds16(v_head + off[i], v_lane_bytes,
                 lds_address(&v_lds_buf[stage][(wave_u * 64 + NT * i) * 8]));
  };

  // S^T = K Q^T of the tile in K stage `stage`: two 32-key blocks, their
  // accumulator chains interleaved, K fragments read kAhead MFMAs before use
  constexpr int kAhead = 4;
  auto kfrag = [&](int stage, int i) {
    // key kr = 32 (i & 1) + krow of the tile, piece 2 (i >> 1) + half
    const int kr = 32 * (i & 1) + krow;
    return *reinterpret_cast<const uint4*>(
        &k_lds_buf[stage][(kr / kBlock) * PAGE + ((2 * (i >> 1) + half) * kBlock + kr % kBlock) * 8]);
  };
  auto mask = [&](f32x16_t (&s)[2], int kt) {
    const int key_base = kt * kKvTile;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int key = key_base + 32 * kb + 16 * (rr >> 3) + 8 * half + (rr & 7);
        if (key > qlimit) s[kb][rr] = neg_inf();
      }
  };
  auto row_max = [&](const f32x16_t (&s)[2]) {
    float pm[4] = {neg_inf(), neg_inf(), neg_inf(), neg_inf()};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) pm[rr & 3] = fmaxf(pm[rr & 3], s[kb][rr]);
    return half_max(fmaxf(fmaxf(pm[0], pm[1]), fmaxf(pm[2], pm[3])));
  };

  // probabilities of S(t) against the reference max, bf16-rounded as the PV
  // product uses them, and their sums (two per v_dot2, four partial sums)
  uint4 pb[4];
  float ps[4];
  auto probs = [&](const f32x16_t (&s)[2], float msc) {
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
  // S(t+1) into sn while the probabilities of S(t) are computed.  The work
  // is laid out in 2 KS slots, one MFMA each: slot i issues the K fragment
  // read for slot i + kAhead, MFMA i, then its share of the 16 probability
  // units (unit u: elements 2u and 2u+1 of the lane's 32: two fma, two
  // exponentials, one bf16 pack, one v_dot2 into the page's sum; one unit
  // per slot at head_dim 128, two at 64).  The vector work runs while the
  // MFMA does; a scheduling barrier after each slot keeps the compiler from
  // regrouping all MFMAs ahead of all vector work.
  constexpr int kUnitsPerSlot = 16 / (2 * KS);
  static_assert(kUnitsPerSlot * 2 * KS == 16, "16 probability units over the MFMA slots");
  static_assert(2 * PER_THREAD <= 2 * KS, "a tile's K and V loads fit in the slots");
  // at head_dim 64 the loads stay ahead of the slots: issued from the slots
  // they cost 2 more VGPRs (170), one workgroup per CU fewer
  constexpr bool kLoadsInSlots = D > 64;
  auto qk_and_probs = [&](f32x16_t (&sn)[2], int kstage, const f32x16_t (&s)[2], float msc,
                          auto&& dma) {
    uint4 ka[kAhead];
#pragma unroll
    for (int i = 0; i < kAhead; ++i) ka[i] = kfrag(kstage, i);
    uint32_t pw[4][4];
#pragma unroll
    for (int kp = 0; kp < 4; ++kp) ps[kp] = 0.f;
    const f32x16_t zero = {};
#pragma unroll
    for (int i = 0; i < 2 * KS; ++i) {
      const uint4 a = ka[i % kAhead];
      if (i + kAhead < 2 * KS) ka[i % kAhead] = kfrag(kstage, i + kAhead);
      sn[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                          __builtin_bit_cast(bf16x8_t, qf[i >> 1]),
                                                          i < 2 ? zero : sn[i & 1], 0, 0, 0);
      dma(i);
#pragma unroll
      for (int uu = 0; uu < kUnitsPerSlot; ++uu) {
        const int u = i * kUnitsPerSlot + uu;
        const int kp = u >> 2, e2 = u & 3;  // page kp, pair e2 of its 8 keys
        const int x = 8 * (kp & 1) + 2 * e2;
        const float p0 = fast_exp2(__builtin_fmaf(s[kp >> 1][x], scale_log2, -msc));
        const float p1 = fast_exp2(__builtin_fmaf(s[kp >> 1][x + 1], scale_log2, -msc));
        pw[kp][e2] = pack_bf16x2(p0, p1);
        ps[kp] = sum2_bf16(pw[kp][e2], ps[kp]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int kp = 0; kp < 4; ++kp) pb[kp] = make_uint4(pw[kp][0], pw[kp][1], pw[kp][2], pw[kp][3]);
  };
  auto qk = [&](f32x16_t (&sn)[2], int kstage) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) sn[kb][i] = 0.f;
    uint4 ka[2 * KS];
#pragma unroll
    for (int i = 0; i < 2 * KS; ++i) ka[i] = kfrag(kstage, i);
#pragma unroll
    for (int i = 0; i < 2 * KS; ++i)
      sn[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, ka[i]),
                                                          __builtin_bit_cast(bf16x8_t, qf[i >> 1]),
                                                          sn[i & 1], 0, 0, 0);
  };
  // O^T += V^T P^T over the tile in V stage `stage`, one page (16 keys) per
  // MFMA, the DB accumulator chains interleaved.  With `ragged`, V values of
  // keys at or past kv_end (key base kt * 64) are zeroed first.
  constexpr int kVAhead = 4;
  const int vh = half ^ ((ncol >> 3) & 1);  // the swizzled half holding keys 8*half..
  auto vfrag = [&](int stage, int i) {  // i = kp * DB + db
    return *reinterpret_cast<const uint4*>(
        &v_lds_buf[stage][(i / DB) * PAGE + (32 * (i % DB) + ncol) * kBlock + 8 * vh]);
  };
  auto pv = [&](int stage, bool ragged, int kt) {
    uint4 va[4 * DB];
#pragma unroll
    for (int i = 0; i < 4 * DB; ++i) va[i] = vfrag(stage, i);
#pragma unroll
    for (int i = 0; i < 4 * DB; ++i) {
      uint4 a = va[i];
      if (ragged) {
        // keys kt*64 + 16 kp + 8 half + e, e < 8, of this lane's fragment
        const int nvalid = kv_end - (kt * kKvTile + 16 * (i / DB) + 8 * half);
        uint32_t x[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t keep = ((2 * e < nvalid) ? 0xFFFFu : 0u) |
                                ((2 * e + 1 < nvalid) ? 0xFFFF0000u : 0u);
          x[e] &= keep;
        }
        a = make_uint4(x[0], x[1], x[2], x[3]);
      }
      o[i % DB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                          __builtin_bit_cast(bf16x8_t, pb[i / DB]),
                                                          o[i % DB], 0, 0, 0);
    }
    if (!ragged) {
      // V fragments read kVAhead MFMAs before their use
      __builtin_amdgcn_sched_group_barrier(0x100, kVAhead, 0);
#pragma unroll
      for (int i = 0; i < 4 * DB; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i + kVAhead < 4 * DB) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }
  };

  // tile kt needs the causal mask iff its last key is past the tile's first
  // query's limit: kt*64 + 63 > context + q_begin
  const int kt_mask = max(kt0, min(n_kv, (c + qb + 1) / kKvTile));

  // prologue: K(kt0) in K stage 0; then K(kt0+1) and V(kt0) load while
  // S(kt0) is computed; its row max is the first reference max
  int64_t off_a[PER_THREAD], off_b[PER_THREAD];  // page offsets of tiles kt0, kt0 + 1
  page_offsets(kt0, off_a);
  issue_k(off_a, 0);
  wait_vmem();
  __syncthreads();
  issue_v(off_a, 0);
  if (kt0 + 1 < n_kv) {
    page_offsets(kt0 + 1, off_b);
    issue_k(off_b, 1);
  }
  f32x16_t sa[2], sb[2];
  qk(sa, 0);
  if (kt0 >= kt_mask) mask(sa, kt0);
  float m = row_max(sa);  // finite: every row sees the piece's first key
  float lsum = 0.f;
  wait_vmem();
  __syncthreads();

  // the rare move of the reference max: the tile's row max beats it by more
  // than 8, which a probability above 2^8, and then the sum, shows
  auto rescale_if_needed = [&](const f32x16_t (&s)[2]) {
    float tsum = (ps[0] + ps[1]) + (ps[2] + ps[3]);
    if (__builtin_expect(__any(!(tsum <= 256.f)), 0)) {
      // the empty asm keeps the compiler from hoisting this out of the
      // branch and running it on every tile
      asm volatile("" ::: "memory");
      const float mx = row_max(s);
      const bool grow = (mx - m) * scale_log2 > 8.f;  // the same in both halves of a row
      const float mn = grow ? mx : m;
      const float alpha = fast_exp2((m - mn) * scale_log2);
      m = mn;
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
      probs(s, m * scale_log2);
      tsum = (ps[0] + ps[1]) + (ps[2] + ps[3]);
    }
    lsum += tsum;
  };
  // Tile kt with a next tile: s holds S(kt), sn receives S(kt+1).  LDS holds
  // V(kt) in V stage st and K(kt+1) in K stage st ^ 1; off_next holds the page
  // offsets of tile kt+1 and receives those of tile kt+2.
  auto step = [&](const f32x16_t (&s)[2], f32x16_t (&sn)[2], int64_t (&off_next)[PER_THREAD],
                  int64_t (&off_after)[PER_THREAD], int kt) {
    const int st = (kt - kt0) & 1;
    // K(kt+2) into the stage K(kt) used and V(kt+1) into the stage V(kt-1)
    // used.  At head_dim 128 one 16-byte load per lane goes out in each of
    // the first 2 PER_THREAD slots, K first: issued together right after the
    // barrier, a tile's loads held the wave for about a fifth of its tile
    // (measured at 8 loads per lane, with 4-wave workgroups), and from the
    // slots that time overlaps other waves' matrix work.  Past the piece's
    // last tile the K offsets are those of page 0, so the spare loads stay
    // inside the pool.
    if constexpr (kLoadsInSlots) {
      page_offsets(kt + 2, off_after);
    } else {
      if (kt + 2 < n_kv) {
        page_offsets(kt + 2, off_after);
        issue_k(off_after, st);
      }
      issue_v(off_next, st ^ 1);
    }
    auto dma = [&](int i) {
      if (!kLoadsInSlots) return;
      if (i < PER_THREAD)
        load_lds16(k_head + off_after[i], k_lane_bytes,
                   lds_address(&k_lds_buf[st][(wave_u * 64 + NT * i) * 8]));
      else if (i < 2 * PER_THREAD)
        load_lds16(v_head + off_next[i - PER_THREAD], v_lane_bytes,
                   lds_address(&v_lds_buf[st ^ 1][(wave_u * 64 + NT * (i - PER_THREAD)) * 8]));
    };
    qk_and_probs(sn, st ^ 1, s, m * scale_log2, dma);
    rescale_if_needed(s);
    pv(st, false, kt);
    if (kt + 1 >= kt_mask) mask(sn, kt + 1);
    // the next tiles must be in LDS, and every wave done with this one,
    // before any wave goes on
    wait_vmem();
    __syncthreads();
  };
  // every tile but the last, two per trip so that S(kt) and S(kt+1) swap
  // registers without copies; the last tile, the only one that can reach
  // past kv_end, on its own
  const int last = n_kv - 1;
  int kt = kt0;
  for (; kt + 2 <= last; kt += 2) {
    step(sa, sb, off_b, off_a, kt);
    step(sb, sa, off_a, off_b, kt + 1);
  }
  if (kt < last) {
    step(sa, sb, off_b, off_a, kt);
    ++kt;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) sa[kb] = sb[kb];
  }
  probs(sa, m * scale_log2);
  rescale_if_needed(sa);
  if ((last + 1) * kKvTile > kv_end)
    pv((last - kt0) & 1, true, last);
  else
    pv((last - kt0) & 1, false, last);

  lsum = half_sum(lsum);
  // the output addresses are derived again here rather than kept in
  // registers through the loop
  asm volatile("" : "+v"(j), "+v"(r));
  const int hq_out = g * grp + (r % grp);
  if (row_ok && slot >= 0) {
    // one piece of a split tile, for merge_kernel: its output over its own
    // keys (normalised by its own sum) in bf16, the sum and max in fp32
    const int64_t pr = ((int64_t)slot * num_kv_heads + g) * ROWS + r;
    const float inv = 1.f / lsum;
    uint16_t* prow = part.out + pr * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = 32 * db + 8 * g4 + 4 * half;
        uint2 v;
        v.x = pack_bf16x2(o[db][4 * g4 + 0] * inv, o[db][4 * g4 + 1] * inv);
        v.y = pack_bf16x2(o[db][4 * g4 + 2] * inv, o[db][4 * g4 + 3] * inv);
        *reinterpret_cast<uint2*>(prow + d) = v;
      }
    if (half == 0) {
      part.m[pr] = m * scale_log2;
      part.l[pr] = lsum;
    }
  } else if (row_ok) {
    const float inv = 1.f / lsum;
    uint16_t* orow = out + ((int64_t)(t0 + j) * num_q_heads + hq_out) * D;
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
      lse[(int64_t)(t0 + j) * num_q_heads + hq_out] = (m * scale_log2 + __log2f(lsum)) * kLn2;
  }
}

}  // namespace cpa
