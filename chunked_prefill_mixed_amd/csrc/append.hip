// Paged KV append: the step's K/V are written into their cache pages before
// attention reads the cache ("05. Chunked Prefill" section 8; tbr8.org deep
// dive 4.2, 16-token pages).  Pure bit copy.
//
// One wave per packed token, 4 tokens per workgroup.  A token's row is found
// in one step: the wave's lanes read query_start_loc in parallel (64 entries
// per load, all loads in flight together) and the row is the number of rows
// that start at or before the token, minus one (rows that schedule no token
// share their start with the next row and are skipped by the count).  Then
// context_len and the page id: three dependent loads in all, where a binary
// search would chain about log2(rows) of them.
//
// K rows are copied as 16-byte pieces into the token-major K page.  V pages
// are stored transposed ([D][16] per page and KV head), so one token's V is a
// column of 2-byte values.  V is therefore written per aligned group of 8
// slots: the wave of the group's first new token loads the V rows of the
// group's new tokens (coalesced, Hkv*D*2 bytes each), and every lane turns the
// 8 values of each of its (head, d) pairs into one 16-byte store.  A group
// that is only partly new (a decode row's token, the ends of a chunk) keeps
// its other slots: only the new ones are written, 2 bytes each.

#include "device.h"
#include "internal.h"
#include "tiles.h"

namespace cpa {

constexpr int kAppendWaves = 4;  // tokens per workgroup
constexpr int kVGroup = 8;       // V slots written together (16 bytes)

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

  // the token's K row does not depend on its row: its first two 16-byte
  // pieces per lane load while the row is looked up
  const uint4* ksrc = reinterpret_cast<const uint4*>(k_new + (int64_t)t * num_kv_heads * D);
  const int kpieces = num_kv_heads * kParts;
  uint4 k0 = make_uint4(0, 0, 0, 0), k1 = make_uint4(0, 0, 0, 0);
  if (lane < kpieces) k0 = ksrc[lane];
  if (lane + 64 < kpieces) k1 = ksrc[lane + 64];

  // row s = #{i < num_seqs : qsl[i] <= t} - 1; qsl is non-decreasing and
  // qsl[num_seqs] = num_tokens > t
  int count = 0;
  for (int base = 0; base < num_seqs; base += 64) {
    const int i = base + lane;
    const bool le = i < num_seqs && qsl[i] <= t;
    count += __builtin_popcountll(__ballot(le));
  }
  const int s = count - 1;
  const int q0 = qsl[s], c = ctx[s];
  const int p = c + (t - q0);
  const int64_t blk = bt[(int64_t)s * bt_stride + p / kBlock];
  const int slot = p % kBlock;
  const int64_t page0 = blk * num_kv_heads * (int64_t)PAGE;

  auto kdst = [&](int e) {
    return reinterpret_cast<uint4*>(k_cache + page0 + (int64_t)(e / kParts) * PAGE + slot * D +
                                    (e % kParts) * 8);
  };
  if (lane < kpieces) *kdst(lane) = k0;
  if (lane + 64 < kpieces) *kdst(lane + 64) = k1;
  for (int e = lane + 128; e < kpieces; e += 64) *kdst(e) = ksrc[e];

  // V: only the wave of a group's first new token
  const int gbeg = p & ~(kVGroup - 1);
  if (p != gbeg && t != q0) return;
  const int row_end = c + (qsl[s + 1] - q0);        // one past the row's last new position
  const int nnew = min(gbeg + kVGroup, row_end) - p;  // new slots p .. p + nnew - 1
  const int lo = p - gbeg;                            // first new slot inside the group
  const bool whole = lo == 0 && nnew == kVGroup;
  uint16_t* vpage = v_cache + page0 + (gbeg % kBlock);  // + g * PAGE + d * 16: the group's 8 slots
  // each lane takes 8 consecutive (head, d) values per pass: one 16-byte load
  // of each new token, one 16-byte store per (head, d)
  const int hd = num_kv_heads * D;
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
