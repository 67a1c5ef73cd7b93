// Prefill-chunk flash attention on bf16 matrix cores (gfx950 MFMA).
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
// K/V tiles of 64 keys (4 pages) are staged in LDS by all 256 threads; the
// next tile's global loads are in flight while the current one is computed.
// Only tiles that reach past the first query's last visible key apply the
// causal mask.

#include "device.h"
#include "internal.h"
#include "tiles.h"

namespace cpa {

template <int D, int G>
__global__ __launch_bounds__(256, 2) void chunk_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_cache,
    const uint16_t* __restrict__ v_cache, const int32_t* __restrict__ bt, int bt_stride,
    const int32_t* __restrict__ qsl, const int32_t* __restrict__ ctx,
    const int32_t* __restrict__ tiles, int num_tiles, int num_q_heads, int num_kv_heads,
    float scale_log2, uint16_t* __restrict__ out, float* __restrict__ lse) {
  constexpr int KS = D / 16;               // 16-wide d steps of S^T = K Q^T
  constexpr int DB = D / 32;               // 32-row d blocks of O^T
  constexpr int KSTR = D + 8;              // padded K row in LDS (elements)
  constexpr int PAGE = kBlock * D;         // elements of one (page, KV head)
  constexpr int CHUNKS = 4 * PAGE / 8;     // 16-byte pieces per 64-key tile (K or V)
  constexpr int PER_THREAD = CHUNKS / 256;
  static_assert(CHUNKS % 256 == 0, "tile must split evenly over 256 threads");

  __shared__ __align__(16) uint16_t k_lds[kKvTile * KSTR];
  __shared__ __align__(16) uint16_t v_lds[4 * PAGE];

  const int item = xcd_remap(blockIdx.x, num_tiles * num_kv_heads);
  const int g = item / num_tiles;
  const int4 te = reinterpret_cast<const int4*>(tiles)[item % num_tiles];
  const int row = te.x, qb = te.y, qe = te.z;
  const int c = ctx[row];
  const int t0 = qsl[row];
  const int kv_end = c + qe;  // keys visible to the tile's last query

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
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
  const int n_kv = (kv_end + kKvTile - 1) / kKvTile;

  uint4 kreg[PER_THREAD], vreg[PER_THREAD];
  auto load_tile = [&](int kt) {
#pragma unroll
    for (int i = 0; i < PER_THREAD; ++i) {
      const int cidx = tid + 256 * i;
      const int kp = cidx / (PAGE / 8);
      const int w = cidx % (PAGE / 8);
      const int pg = kt * 4 + kp;
      const int key0 = pg * kBlock;
      if (key0 < kv_end) {
        const int64_t base = ((int64_t)btrow[pg] * num_kv_heads + g) * PAGE;
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
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < PER_THREAD; ++i) {
      const int cidx = tid + 256 * i;
      const int kp = cidx / (PAGE / 8);
      const int w = cidx % (PAGE / 8);
      const int key = kp * kBlock + w / (D / 8);
      const int part = w % (D / 8);
      *reinterpret_cast<uint4*>(&k_lds[key * KSTR + part * 8]) = kreg[i];
      *reinterpret_cast<uint4*>(&v_lds[kp * PAGE + w * 8]) = vreg[i];
    }
  };

  load_tile(0);
  for (int kt = 0; kt < n_kv; ++kt) {
    __syncthreads();  // every wave is done with the previous tile
    store_tile();
    __syncthreads();
    if (kt + 1 < n_kv) load_tile(kt + 1);

    // S^T = K Q^T for two 32-key blocks
    f32x16_t s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
      const uint16_t* krow_p = &k_lds[(32 * kb + krow) * KSTR + 8 * half];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint4 a = *reinterpret_cast<const uint4*>(krow_p + 16 * ks);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                        __builtin_bit_cast(bf16x8_t, qf[ks]),
                                                        s[kb], 0, 0, 0);
      }
    }

    const int key_base = kt * kKvTile;
    if (key_base + kKvTile - 1 > c + qb) {  // tile reaches past some query's last key
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          const int key = key_base + 32 * kb + 16 * (rr >> 3) + 8 * half + (rr & 7);
          if (key > qlimit) s[kb][rr] = neg_inf();
        }
    }

    float mx = neg_inf();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) mx = fmaxf(mx, s[kb][rr]);
    mx = fmaxf(mx, xor_lane(mx, 32));
    const float mn = fmaxf(m, mx);
    const float alpha = fast_exp2((m - mn) * scale_log2);
    m = mn;
    const float msc = mn * scale_log2;

    float psum = 0.f;
    uint4 pb[4];
#pragma unroll
    for (int kp = 0; kp < 4; ++kp) {
      float pv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        pv[i] = fast_exp2(__builtin_fmaf(s[kp >> 1][8 * (kp & 1) + i], scale_log2, -msc));
        psum += pv[i];
      }
      pb[kp] = make_uint4(pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]),
                          pack_bf16x2(pv[4], pv[5]), pack_bf16x2(pv[6], pv[7]));
    }
    lsum = lsum * alpha + psum;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[db][i] *= alpha;

    // O^T += V^T P^T, one page (16 keys) per MFMA
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int kp = 0; kp < 4; ++kp) {
        const uint4 a =
            *reinterpret_cast<const uint4*>(&v_lds[kp * PAGE + (32 * db + ncol) * kBlock + 8 * half]);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                        __builtin_bit_cast(bf16x8_t, pb[kp]),
                                                        o[db], 0, 0, 0);
      }
  }

  lsum += xor_lane(lsum, 32);
  if (row_ok) {
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

template <int D, int G>
static void launch_chunk_t(const void* q, const void* kc, const void* vc, const int32_t* bt,
                           int bt_stride, const int32_t* qsl, const int32_t* ctx,
                           const int32_t* tiles, int num_tiles, int hq, int hkv, float sl2,
                           void* out, float* lse, hipStream_t stream) {
  hipLaunchKernelGGL((chunk_kernel<D, G>), dim3(num_tiles * hkv), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(kc),
                     static_cast<const uint16_t*>(vc), bt, bt_stride, qsl, ctx, tiles, num_tiles,
                     hq, hkv, sl2, static_cast<uint16_t*>(out), lse);
}

hipError_t launch_chunk(const void* q, const void* k_cache, const void* v_cache, const int32_t* bt,
                        int bt_stride, const int32_t* qsl, const int32_t* ctx,
                        const int32_t* tiles, int num_tiles, int num_q_heads, int num_kv_heads,
                        int head_dim, float scale_log2, void* out, float* lse, hipStream_t stream) {
  const int G = num_q_heads / num_kv_heads;
#define CPA_CHK(DD, GG)                                                                        \
  if (head_dim == DD && G == GG) {                                                              \
    launch_chunk_t<DD, GG>(q, k_cache, v_cache, bt, bt_stride, qsl, ctx, tiles, num_tiles,      \
                           num_q_heads, num_kv_heads, scale_log2, out, lse, stream);            \
    return hipGetLastError();                                                                   \
  }
  CPA_CHK(128, 1) CPA_CHK(128, 2) CPA_CHK(128, 4) CPA_CHK(128, 8)
  CPA_CHK(64, 1) CPA_CHK(64, 2) CPA_CHK(64, 4) CPA_CHK(64, 8)
#undef CPA_CHK
  return hipErrorInvalidValue;
}

}  // namespace cpa
