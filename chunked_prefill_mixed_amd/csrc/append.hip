// Paged KV append: the step's K/V are written into their cache pages before
// attention reads the cache ("05. Chunked Prefill" section 8; tbr8.org deep
// dive 4.2, 16-token pages).  Pure bit copy.
//
// One wave per packed token, 4 tokens per workgroup.  A token's row is found
// in one step: the wave's lanes read query_start_loc and context_lens in
// parallel (64 entries per load, all loads in flight together) and the row is
// the number of rows that start at or before the token, minus one (rows that
// schedule no token share their start with the next row and are skipped by
// the count).  The row's start, end and context are then read out of those
// registers, so the page id is the second and last dependent load, where a
// binary search would chain about log2(rows) of them (steps of 512 rows or
// more reload the three values: one more dependent load).
//
// Both page layouts keep neighbouring slots side by side, so both are written
// per aligned group of 8 slots.  K pages hold their keys in 8-value pieces
// ([D/8][16][8] per KV head): piece c of the group's 8 slots is 128
// contiguous bytes.  When all 8 slots are new (inside a chunk) the group's 8
// waves share its K, wave r copying the blocks of 8 pieces r, r + 8, ... of
// all 8 slots, so every store fills whole lines; otherwise (a decode row's token, the ends of
// a chunk) each token's wave copies its own 16-byte pieces.  V pages are
// stored transposed ([D][16]), so one token's V is a column of 2-byte values:
// the wave of the group's first new token loads the V rows of the group's new
// tokens (coalesced, Hkv*D*2 bytes each), and every lane turns the 8 values
// of each of its (head, d) pairs into one 16-byte store.  A group that is
// only partly new keeps its other slots: only the new ones are written; a
// group with one new slot (a decode token) stores the values of the token's
// own V row, which load before the row lookup, so its chain after the lookup
// is the stores alone.  When
// a whole page is new, its 16 waves share its V instead and write whole
// 32-byte rows (whole lines): two 8-slot halves written by different waves
// would meet in one line as partial writes.

#include "device.h"
#include "internal.h"
#include "tiles.h"

namespace cpa {

constexpr int kAppendWaves = 4;  // tokens per workgroup
constexpr int kVGroup = 8;       // slots written together (16 bytes of a V row, 128 of a K piece)
constexpr int kLookupChunks = 8;  // rows the lookup holds in registers: fewer than 512

template <int D>
__global__ __launch_bounds__(64 * kAppendWaves) void append_kernel(
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    const int32_t* __restrict__ qsl, const int32_t* __restrict__ ctx,
    const int32_t* __restrict__ bt, int bt_stride, int num_seqs, int num_tokens,
    int num_kv_heads, uint16_t* __restrict__ k_cache, uint16_t* __restrict__ v_cache) {
  constexpr int PAGE = kBlock * D;
  constexpr int kParts = D / 8;  // 16-byte pieces per head row
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * kAppendWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (t >= num_tokens) return;  // whole wave; no barrier below
  const int hd = num_kv_heads * D;  // values of one token's K (or V) row

  // the token's own V values (8 per lane, two passes) do not depend on its
  // row: they load while the row is looked up, for the one-new-slot case
  uint4 vown[2];
#pragma unroll
  for (int u = 0; u < 2; ++u)
    vown[u] = *reinterpret_cast<const uint4*>(v_new + (int64_t)t * hd + min(lane * 8 + 512 * u, hd - 8));

  // row s = #{i < num_seqs : qsl[i] <= t} - 1; qsl is non-decreasing and
  // qsl[num_seqs] = num_tokens > t
  int s, q0, q1, c;
  if (num_seqs < 64 * kLookupChunks) {
    // lane i of chunk k holds qsl[64 k + i] and context_lens[64 k + i], all
    // loaded at once; the row's start, end and context are then read out of
    // those registers, so the page id is the second dependent load
    const int nchunks = num_seqs / 64 + 1;  // chunks holding qsl[0 .. num_seqs]
    int qv[kLookupChunks] = {}, cv[kLookupChunks] = {};
#pragma unroll
    for (int k = 0; k < kLookupChunks; ++k) {
      if (k < nchunks) {  // wave-uniform
        const int i = 64 * k + lane;
        qv[k] = i <= num_seqs ? qsl[i] : 0x7fffffff;
        cv[k] = i < num_seqs ? ctx[i] : 0;
      }
    }
    int count = 0;
#pragma unroll
    for (int k = 0; k < kLookupChunks; ++k)
      if (k < nchunks) count += __builtin_popcountll(__ballot(64 * k + lane < num_seqs && qv[k] <= t));
    s = count - 1;
    auto pick = [&](const int (&v)[kLookupChunks], int i) {  // v[i / 64] of lane i % 64
      int x = 0;
#pragma unroll
      for (int k = 0; k < kLookupChunks; ++k)
        if (k == i / 64) x = __builtin_amdgcn_readlane(v[k], i % 64);
      return x;
    };
    q0 = pick(qv, s);
    q1 = pick(qv, s + 1);
    c = pick(cv, s);
  } else {
    int count = 0;
    for (int base = 0; base < num_seqs; base += 64) {
      const int i = base + lane;
      const bool le = i < num_seqs && qsl[i] <= t;
      count += __builtin_popcountll(__ballot(le));
    }
    s = count - 1;
    q0 = qsl[s];
    q1 = qsl[s + 1];
    c = ctx[s];
  }
  const int p = c + (t - q0);
  const int64_t blk = bt[(int64_t)s * bt_stride + p / kBlock];
  const int64_t page0 = blk * num_kv_heads * (int64_t)PAGE;
  const int gbeg = p & ~(kVGroup - 1);
  const int row_end = c + (q1 - q0);  // one past the row's last new position
  const int kpieces = hd / 8;  // 16-byte pieces of a K row: e = head * D/8 + c

  // K piece e of page slot o lands in piece row c of the head's page
  auto kdst = [&](int e, int o) {
    return reinterpret_cast<uint4*>(k_cache + page0 + (int64_t)(e / kParts) * PAGE +
                                    ((e % kParts) * kBlock + o) * 8);
  };
  if (gbeg >= c && gbeg + kVGroup <= row_end) {
    // all 8 slots new: the pieces come in blocks of 8 and the wave in slot r
    // of the group takes blocks b = r, r + 8, ...; lane (j = lane / 8,
    // i = lane % 8) copies piece 8 b + i of slot j, so one instruction reads
    // 8 whole 128-byte lines of k_new and writes 8 whole lines of the page
    const int r = p - gbeg, j = lane / kVGroup, i = lane % kVGroup;
    const uint16_t* src = k_new + (int64_t)(t - r + j) * hd;  // token of slot j
    for (int b0 = r; b0 < kpieces / 8; b0 += 4 * 8) {
      uint4 x[4];  // loads clamped into the token's row; stores only in range
#pragma unroll
      for (int u = 0; u < 4; ++u)
        x[u] = *reinterpret_cast<const uint4*>(src + min(8 * (b0 + 8 * u) + i, kpieces - 1) * 8);
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (b0 + 8 * u < kpieces / 8) *kdst(8 * (b0 + 8 * u) + i, gbeg % kBlock + j) = x[u];
    }
  } else {
    // the token's own pieces
    const uint16_t* src = k_new + (int64_t)t * hd;
    for (int e0 = lane; e0 < kpieces; e0 += 4 * 64) {
      uint4 x[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        x[u] = *reinterpret_cast<const uint4*>(src + min(e0 + 64 * u, kpieces - 1) * 8);
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (e0 + 64 * u < kpieces) *kdst(e0 + 64 * u, p % kBlock) = x[u];
    }
  }

  // V, whole page new (inside a chunk): the page's 16 waves share its V.  The
  // wave in slot r takes the rows f = (head, d) in [r R, r R + R), R = Hkv D /
  // 16, one per lane: it gathers the row's 16 values (one 2-byte load from
  // each token; a lane group reads 128 contiguous bytes) and stores the whole
  // 32-byte row, so 4 neighbouring lanes fill a 128-byte line.
  const int pbeg = p & ~(kBlock - 1);
  if (pbeg >= c && pbeg + kBlock <= row_end) {
    const int r = p - pbeg, R = hd / kBlock;
    const uint16_t* src = v_new + (int64_t)(t - r) * hd;  // token of page slot 0
    for (int f = r * R + lane; f < (r + 1) * R; f += 64) {
      uint32_t w[kBlock / 2];
#pragma unroll
      for (int j = 0; j < kBlock / 2; ++j)
        w[j] = (uint32_t)src[(int64_t)(2 * j) * hd + f] |
               ((uint32_t)src[(int64_t)(2 * j + 1) * hd + f] << 16);
      uint4* dst = reinterpret_cast<uint4*>(v_cache + page0 + (int64_t)(f / D) * PAGE +
                                            (f % D) * kBlock);
      dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
      dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
    }
    return;
  }

  // V otherwise: only the wave of a group's first new token
  if (p != gbeg && t != q0) return;
  const int nnew = min(gbeg + kVGroup, row_end) - p;  // new slots p .. p + nnew - 1
  const int lo = p - gbeg;                            // first new slot inside the group
  const bool whole = lo == 0 && nnew == kVGroup;
  uint16_t* vpage = v_cache + page0 + (gbeg % kBlock);  // + g * PAGE + d * 16: the group's 8 slots
  if (nnew == 1) {
    // one new slot (a decode token): the token's 8 values per lane and pass
    // (the first two passes already loaded), one 2-byte store per (head, d)
    uint16_t* vslot = vpage + lo;
    for (int f0 = lane * 8; f0 < hd; f0 += 2 * 64 * 8) {
      uint4 x[2] = {vown[0], vown[1]};
      if (f0 != lane * 8) {
#pragma unroll
        for (int u = 0; u < 2; ++u)
          x[u] = *reinterpret_cast<const uint4*>(v_new + (int64_t)t * hd + min(f0 + 512 * u, hd - 8));
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        if (f0 + 512 * u >= hd) continue;
        const uint32_t wd[4] = {x[u].x, x[u].y, x[u].z, x[u].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int f = f0 + 512 * u + e;
          vslot[(int64_t)(f / D) * PAGE + (f % D) * kBlock] = (uint16_t)(wd[e / 2] >> (16 * (e & 1)));
        }
      }
    }
    return;
  }
  // each lane takes 8 consecutive (head, d) values per pass: one 16-byte load
  // of each new token, one 16-byte store per (head, d)
  for (int f0 = lane * 8; f0 < hd; f0 += 64 * 8) {
    uint4 x[kVGroup];  // x[j]: the values of slot j (token t + j - lo) when new
#pragma unroll
    for (int j = 0; j < kVGroup; ++j) {
      const bool in = j >= lo && j < lo + nnew;
      // slots that are not new read token t's row (always in range) and are
      // then replaced by the cached values
      x[j] = *reinterpret_cast<const uint4*>(v_new + (int64_t)(t + (in ? j - lo : 0)) * hd + f0);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int f = f0 + e;  // (head, d) = (f / D, f % D)
      uint16_t* dst = vpage + (int64_t)(f / D) * PAGE + (f % D) * kBlock;
      uint32_t w[kVGroup];
#pragma unroll
      for (int j = 0; j < kVGroup; ++j) {
        const uint32_t word = e < 2 ? x[j].x : e < 4 ? x[j].y : e < 6 ? x[j].z : x[j].w;
        w[j] = (word >> (16 * (e & 1))) & 0xFFFFu;
      }
      if (whole) {
        *reinterpret_cast<uint4*>(dst) = make_uint4(w[0] | (w[1] << 16), w[2] | (w[3] << 16),
                                                    w[4] | (w[5] << 16), w[6] | (w[7] << 16));
      } else {
#pragma unroll
        for (int j = 0; j < kVGroup; ++j)
          if (j >= lo && j < lo + nnew) dst[j] = (uint16_t)w[j];
      }
    }
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
