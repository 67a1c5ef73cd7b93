// Log-sum-exp merge of split decode rows and split chunk tiles, one launch.
//
// A row whose keys were cut into pieces has, per piece i and query head, an
// unnormalised fp32 output acc_i, the max m_i (log2 units of the scaled score)
// and the sum l_i of the piece's weights relative to m_i.  The exact softmax
// output over all the row's keys is
//   M = max m_i,  L = sum l_i 2^(m_i - M),  out = sum acc_i 2^(m_i - M) / L,
// the incremental-softmax identity the split relies on (tbr8.org deep dive
// 7.2 names the incremental computation; the pieces never need correcting
// because each covers a fixed key range).  lse = (M + log2 L) ln 2.
//
// Workgroups [0, chunk_blocks) merge chunk tiles, the rest decode rows, so
// both merges of a step cost one launch.  Neither part uses a barrier.

#include <type_traits>

#include "device.h"
#include "internal.h"
#include "tiles.h"

namespace cpa {

// One wave per (decode row, query head), each lane owning D/64 output
// dimensions.  Splits are taken B at a time, every load of a batch (the
// splits' max and sum, broadcast to all lanes, and this lane's partial
// values) issued before any is used, so a batch costs one memory round trip;
// batches fold into a running max, sum and output.  B (4, 8 or 16) is the
// smallest that takes the row's splits in one batch, so few loads go to the
// padding entries of a batch.
template <int D, int B>
__device__ __forceinline__ void merge_decode_batches(int first, int n, int h, int num_q_heads,
                                                     const Partials& ws, float& M, float& L,
                                                     float (&o)[D / 64]) {
  constexpr int PER = D / 64;
  const int lane = threadIdx.x & 63;
  for (int i0 = 0; i0 < n; i0 += B) {
    float mi[B], lv[B], a[B][PER];
#pragma unroll
    for (int i = 0; i < B; ++i) {
      const bool in = i0 + i < n;
      const int64_t ph = (int64_t)(first + (in ? i0 + i : i0)) * num_q_heads + h;
      mi[i] = in ? ws.m[ph] : neg_inf();
      lv[i] = ws.l[ph];
#pragma unroll
      for (int k = 0; k < PER; ++k) a[i][k] = ws.acc[ph * D + lane + 64 * k];
    }
    float Mb = M;
#pragma unroll
    for (int i = 0; i < B; ++i) Mb = fmaxf(Mb, mi[i]);
    const float alpha = fast_exp2(M - Mb);  // 0 on the first batch (M = -inf)
    L *= alpha;
#pragma unroll
    for (int k = 0; k < PER; ++k) o[k] *= alpha;
#pragma unroll
    for (int i = 0; i < B; ++i) {
      const float w = fast_exp2(mi[i] - Mb);  // 0 for the padding entries
      L += w * lv[i];
#pragma unroll
      for (int k = 0; k < PER; ++k) o[k] += w * a[i][k];
    }
    M = Mb;
  }
}

template <int D>
__device__ __forceinline__ void merge_decode_head(const int32_t* __restrict__ merges, int entry,
                                                  int h, const int32_t* __restrict__ qsl,
                                                  int num_q_heads, const Partials& ws,
                                                  uint16_t* __restrict__ out,
                                                  float* __restrict__ lse) {
  constexpr int PER = D / 64;
  const int4 e = reinterpret_cast<const int4*>(merges)[entry];
  const int row = e.x, first = e.y, n = e.z;
  const int lane = threadIdx.x & 63;
  float M = neg_inf(), L = 0.f;
  float o[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) o[k] = 0.f;
  if (n <= 4)
    merge_decode_batches<D, 4>(first, n, h, num_q_heads, ws, M, L, o);
  else if (n <= 8)
    merge_decode_batches<D, 8>(first, n, h, num_q_heads, ws, M, L, o);
  else
    merge_decode_batches<D, 16>(first, n, h, num_q_heads, ws, M, L, o);
  const int t = qsl[row];
  const float inv = 1.f / L;
#pragma unroll
  for (int k = 0; k < PER; ++k)
    out[((int64_t)t * num_q_heads + h) * D + lane + 64 * k] = to_bf16(o[k] * inv);
  if (lse && lane == 0) lse[(int64_t)t * num_q_heads + h] = (M + __log2f(L)) * kLn2;
}

// RPW rows of one (chunk merge entry, KV head) per workgroup; each row is
// handled by LPR = D/4 lanes, each owning 4 consecutive d values, so a partial
// row is one contiguous sweep.  A chunk piece's partial is its output over its
// own keys, already divided by its sum l_i, in bf16: it enters with weight
// l_i 2^(m_i - M).  Pieces are taken B at a time (2, 4 or 8, the smallest
// that takes the tile's pieces in one batch, up to 8): every lane issues all
// loads of a batch (each piece's max and sum, the same address for the row's
// lanes, and its 8 bytes of the piece's output) before using any, so a batch
// costs one memory round trip; batches fold into a running max, sum and
// output as in the decode merge.
constexpr int kChunkMergeBatch = 8;  // the largest chunk-merge batch

template <int D, int G>
__device__ __forceinline__ void merge_chunk_rows(const int32_t* __restrict__ merges, int block,
                                                 const int32_t* __restrict__ qsl, int num_q_heads,
                                                 int num_kv_heads, const ChunkPartials& part,
                                                 uint16_t* __restrict__ out,
                                                 float* __restrict__ lse) {
  constexpr int LPR = D / 4;             // lanes per row
  constexpr int RPW = 256 / LPR;         // rows per workgroup
  constexpr int ROWS = chunk_rows(D);    // rows of a chunk tile and partial slot
  constexpr int RG = ROWS / RPW;         // workgroups per (merge entry, KV head)
  const int rg = block % RG;
  const int g = (block / RG) % num_kv_heads;
  const int4* ep = reinterpret_cast<const int4*>(merges) + 2 * (block / (RG * num_kv_heads));
  const int4 e0 = ep[0], e1 = ep[1];
  const int row = e0.x, qb = e0.y, qe = e0.z, first = e0.w, n = e1.x;
  const int li = threadIdx.x % LPR;
  const int r = rg * RPW + threadIdx.x / LPR;
  const int grp = G > 0 ? G : num_q_heads / num_kv_heads;  // G = 0: read at run time
  const int j = qb + r / grp;
  if (j >= qe) return;  // past the chunk end
  const int64_t stride = (int64_t)num_kv_heads * ROWS;  // rows between consecutive slots
  const int64_t base = ((int64_t)first * num_kv_heads + g) * ROWS + r;
  const int d = 4 * li;

  float M = neg_inf(), L = 0.f;
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  auto batches = [&](auto bsz) {
    constexpr int B = decltype(bsz)::value;
    for (int i0 = 0; i0 < n; i0 += B) {
      float mi[B], lv[B];
      uint2 a[B];
#pragma unroll
      for (int i = 0; i < B; ++i) {
        const bool in = i0 + i < n;
        const int64_t pr = base + (int64_t)(in ? i0 + i : i0) * stride;
        mi[i] = in ? part.m[pr] : neg_inf();
        lv[i] = part.l[pr];
        a[i] = *reinterpret_cast<const uint2*>(part.out + pr * D + d);
      }
      float Mb = M;
#pragma unroll
      for (int i = 0; i < B; ++i) Mb = fmaxf(Mb, mi[i]);
      const float alpha = fast_exp2(M - Mb);  // 0 on the first batch (M = -inf)
      L *= alpha;
      o.x *= alpha; o.y *= alpha; o.z *= alpha; o.w *= alpha;
#pragma unroll
      for (int i = 0; i < B; ++i) {
        const float w = fast_exp2(mi[i] - Mb) * lv[i];  // 0 for the padding entries
        L += w;
        o.x += w * bf16_lo(a[i].x); o.y += w * bf16_hi(a[i].x);
        o.z += w * bf16_lo(a[i].y); o.w += w * bf16_hi(a[i].y);
      }
      M = Mb;
    }
  };
  // batch size from the piece count, uniform over the workgroup
  if (n <= 2)
    batches(std::integral_constant<int, 2>{});
  else if (n <= 4)
    batches(std::integral_constant<int, 4>{});
  else
    batches(std::integral_constant<int, kChunkMergeBatch>{});
  const float inv = 1.f / L;
  const int hq = g * grp + (r % grp);
  const int t0 = qsl[row];
  uint2 v;
  v.x = pack_bf16x2(o.x * inv, o.y * inv);
  v.y = pack_bf16x2(o.z * inv, o.w * inv);
  *reinterpret_cast<uint2*>(out + ((int64_t)(t0 + j) * num_q_heads + hq) * D + d) = v;
  if (lse && li == 0) lse[(int64_t)(t0 + j) * num_q_heads + hq] = (M + __log2f(L)) * kLn2;
}

template <int D, int G>
__global__ __launch_bounds__(256) void merge_kernel(
    const int32_t* __restrict__ dmerges, int num_decode_pairs, const int32_t* __restrict__ cmerges,
    int chunk_blocks, const int32_t* __restrict__ qsl, int num_q_heads, int num_kv_heads,
    Partials dws, ChunkPartials cws, uint16_t* __restrict__ out, float* __restrict__ lse) {
  if ((int)blockIdx.x < chunk_blocks) {
    merge_chunk_rows<D, G>(cmerges, blockIdx.x, qsl, num_q_heads, num_kv_heads, cws, out, lse);
    return;
  }
  // four (decode row, query head) pairs per workgroup, one per wave
  const int pair = ((int)blockIdx.x - chunk_blocks) * 4 + (threadIdx.x >> 6);
  if (pair >= num_decode_pairs) return;
  merge_decode_head<D>(dmerges, pair / num_q_heads, pair % num_q_heads, qsl, num_q_heads, dws,
                       out, lse);
}

hipError_t launch_merges(const int32_t* dmerges, int num_decode_merges, const int32_t* cmerges,
                         int num_chunk_merges, const int32_t* qsl, int num_q_heads,
                         int num_kv_heads, int head_dim, Partials dws, ChunkPartials cws, void* out,
                         float* lse, hipStream_t stream) {
  const int G = num_q_heads / num_kv_heads;
  const int chunk_blocks =
      num_chunk_merges * num_kv_heads * (chunk_rows(head_dim) / (256 / (head_dim / 4)));
  const int pairs = num_decode_merges * num_q_heads;
  const dim3 grid(chunk_blocks + (pairs + 3) / 4), block(256);
  auto* o = static_cast<uint16_t*>(out);
  // G = 0 instances: any other group, read at run time
#define CPA_MRG(DD, GG)                                                                        \
  if (head_dim == DD && (G == GG || GG == 0)) {                                               \
    hipLaunchKernelGGL((merge_kernel<DD, GG>), grid, block, 0, stream, dmerges, pairs, cmerges, \
                       chunk_blocks, qsl, num_q_heads, num_kv_heads, dws, cws, o, lse);         \
    return hipGetLastError();                                                                   \
  }
  CPA_MRG(128, 1) CPA_MRG(128, 2) CPA_MRG(128, 4) CPA_MRG(128, 8) CPA_MRG(128, 0)
  CPA_MRG(64, 1) CPA_MRG(64, 2) CPA_MRG(64, 4) CPA_MRG(64, 8) CPA_MRG(64, 0)
#undef CPA_MRG
  return hipErrorInvalidValue;
}

}  // namespace cpa
