// Paged KV append: the step's K/V are written into their cache pages before
// attention reads the cache ("05. Chunked Prefill" section 8; tbr8.org deep
// dive 4.2, 16-token pages).  Pure bit copy.
//
// One workgroup per page task: a (row, page) pair the step writes into, with
// its new slots [o0, o1) (a whole page inside a chunk; a partial page at a
// chunk's ends; one slot for a decode row).  The grid covers an upper bound
// on the number of tasks (a row of n tokens touches at most n/16 + 2 pages);
// the first wave of each workgroup finds its task by a prefix count of the
// rows' page counts (the counts of 512 rows loaded in one round), and
// workgroups past the last task exit.  After that one dependent round, every
// thread issues all of its loads (up to 8 K pieces and one V unit per round;
// one round at 8 KV heads of 128) before its first store, and the page id
// arrives by a scalar load in the meantime, so a task costs about two memory
// latencies.  Loads and stores go through buffer resources limited to the
// task's source rows and to its page: an index past the task reads zero or
// has its store dropped by the hardware, so the copy has no branches around
// its memory operations and its waits count exactly the loads it needs.
//
// K pages hold their keys in 8-value pieces ([Hkv][D/8][16][8]), so piece c
// of slot o of head h is 16 bytes at ((h * D/8 + c) * 16 + o) * 16: with the
// new slots innermost, consecutive threads write consecutive 16-byte pieces
// (a whole page is 32 KB written front to back at head_dim 128, Hkv 8) and
// read 16 bytes of consecutive tokens' rows.
//
// V pages are stored transposed ([Hkv][D][16]): row (h, d) holds the 16
// slots' values, 32 bytes.  A thread takes a unit (h, 8 d values, one half of
// the page's slots): it loads the 8 d values of each of the half's 8 tokens
// (16 bytes each), transposes the 8 x 8 block of 2-byte values in registers
// (one byte-permute per output dword) and stores 8 half-rows of 16 bytes.  A
// half that is only partly new stores its new slots' 2-byte values alone,
// leaving the others as they are.

#include "device.h"
#include "internal.h"
#include "tiles.h"

namespace cpa {

constexpr int kAppendThreads = 256;

// Inclusive prefix sum over the wave (64 lanes).
__device__ __forceinline__ int wave_inclusive_scan(int x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int k = 1; k < 64; k <<= 1) {
    const int y = __shfl_up(x, k, 64);
    if (lane >= k) x += y;
  }
  return x;
}

// dword i (0..3) and 16-bit element e (0..7) of the 16 bytes in v
__device__ __forceinline__ uint32_t dword(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}
__device__ __forceinline__ uint32_t elem16(const uint4& v, int e) {
  return (dword(v, e >> 1) >> (16 * (e & 1))) & 0xFFFFu;
}

constexpr int kRowsPerLane = 8;  // rows each lookup lane holds: 512 per round

template <int D>
__global__ __launch_bounds__(kAppendThreads) void append_kernel(
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    const int32_t* __restrict__ qsl, const int32_t* __restrict__ ctx,
    const int32_t* __restrict__ bt, int bt_stride, int num_seqs, int num_kv_heads,
    uint16_t* __restrict__ k_cache, uint16_t* __restrict__ v_cache) {
  constexpr int PAGE = kBlock * D;  // elements of one (page, KV head)
  constexpr int PIECES = D / 8;     // 16-byte pieces per head row
  constexpr int T = kAppendThreads;
  __shared__ int task[5];  // row, page index in the row, o0, o1, packed token of slot o0

  const int tid = threadIdx.x;
  if (tid < 64) {
    // the task's row: the first row whose running page count passes the
    // workgroup id; rows that schedule no token touch no page.  Lane i holds
    // rows 8i .. 8i+7 of a round of 512 (clamped, unconditional loads, all in
    // flight together), sums their page counts, and one wave scan over the
    // lanes' sums finds the lane whose rows hold the task.
    const int lane = tid;
    const int want = blockIdx.x;
    int base = 0;
    bool found = false;
    for (int r0 = 0; r0 < num_seqs && !found; r0 += 64 * kRowsPerLane) {
      const int first = r0 + kRowsPerLane * lane;
      int q[kRowsPerLane + 1], c[kRowsPerLane], pages[kRowsPerLane];
#pragma unroll
      for (int j = 0; j <= kRowsPerLane; ++j) q[j] = qsl[min(first + j, num_seqs)];
#pragma unroll
      for (int j = 0; j < kRowsPerLane; ++j) c[j] = ctx[min(first + j, num_seqs - 1)];
      int total = 0;
#pragma unroll
      for (int j = 0; j < kRowsPerLane; ++j) {
        // rows past the last one clamp both starts to query_start_loc[num_seqs]: no tokens
        const int n = q[j + 1] - q[j];
        pages[j] = n > 0 ? (c[j] + n + kBlock - 1) / kBlock - c[j] / kBlock : 0;
        total += pages[j];
      }
      const int incl = base + wave_inclusive_scan(total);
      const bool mine = want >= incl - total && want < incl;
      found = __ballot(mine) != 0;
      if (mine) {
        // the lane's row that holds the task: the first whose pages pass want
        int run = incl - total, sel = -1, before = 0;
#pragma unroll
        for (int j = 0; j < kRowsPerLane; ++j) {
          if (sel < 0 && want < run + pages[j]) {
            sel = j;
            before = run;
          }
          run += pages[j];
        }
        int q0 = 0, n = 0, cc = 0;
#pragma unroll
        for (int j = 0; j < kRowsPerLane; ++j)
          if (j == sel) {
            q0 = q[j];
            n = q[j + 1] - q[j];
            cc = c[j];
          }
        const int pg = cc / kBlock + (want - before);
        const int o0 = max(cc, pg * kBlock) - pg * kBlock;
        task[0] = first + sel;
        task[1] = pg;
        task[2] = o0;
        task[3] = min(cc + n, pg * kBlock + kBlock) - pg * kBlock;  // o1
        task[4] = q0 + (pg * kBlock + o0 - cc);
      }
      base = __builtin_amdgcn_readlane(incl, 63);
    }
    if (lane == 0 && !found) task[0] = -1;
  }
  __syncthreads();
  const int row = __builtin_amdgcn_readfirstlane(task[0]);
  if (row < 0) return;  // past the last task (uniform over the workgroup)
  const int pg = __builtin_amdgcn_readfirstlane(task[1]);
  const int o0 = __builtin_amdgcn_readfirstlane(task[2]);
  const int o1 = __builtin_amdgcn_readfirstlane(task[3]);
  const int t0 = __builtin_amdgcn_readfirstlane(task[4]);
  // the page id is a scalar load; it overlaps the data loads issued below
  const int blk = bt[(int64_t)row * bt_stride + pg];
  const int nnew = o1 - o0;
  const int hd = num_kv_heads * D;            // values of one token's K (or V) row
  const int ngroups = num_kv_heads * PIECES;  // (head, 8-value group) pairs
  const int page_bytes = num_kv_heads * PAGE * 2;
  // byte ranges: the new tokens' rows, and the page (all KV heads)
  const auto kin = make_page_rsrc(k_new + (int64_t)t0 * hd, nnew * hd * 2);
  const auto vin = make_page_rsrc(v_new + (int64_t)t0 * hd, nnew * hd * 2);
  const bool whole = nnew == kBlock;

  // K: pieces e = (group, new slot), slots innermost; V: units u = (half of
  // the slots that holds a new one, group), groups innermost.  A round loads a
  // thread's 8 K pieces and its V unit's 8 token rows before any store; an
  // index past the task loads from / stores to an offset outside its range,
  // which the hardware turns into a zero load / a dropped store.
  const int h_lo = o0 / 8, nhalves = (o1 - 1) / 8 - h_lo + 1;
  const int kn = ngroups * nnew, vn = ngroups * nhalves;
  for (int k0 = 0, v0 = 0; k0 < kn || v0 < vn; k0 += 8 * T, v0 += T) {
    uint4 kx[8];
    uint32_t kdst[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int e = k0 + j * T + tid;
      const int i = whole ? (e & (kBlock - 1)) : e % nnew;  // new slot o0 + i
      const int g = whole ? (e >> 4) : e / nnew;
      const bool in = e < kn;
      kx[j] = buffer_load16(kin, in ? (uint32_t)(i * hd + g * 8) * 2 : kOffNone);
      kdst[j] = in ? (uint32_t)((g * kBlock + o0 + i) * 8) * 2 : kOffNone;
    }
    const int u = v0 + tid;
    const bool vin_range = u < vn;
    const int hg = u % ngroups, half = h_lo + u / ngroups;  // hg = head * PIECES + group
    const int s0 = max(o0, 8 * half), s1 = min(o1, 8 * half + 8);  // the half's new slots
    uint4 vx[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int o = 8 * half + j;
      const bool in = vin_range && o >= s0 && o < s1;
      vx[j] = buffer_load16(vin, in ? (uint32_t)((o - o0) * hd + hg * 8) * 2 : kOffNone);
    }
    // the page id is first used here, after the loads: the empty asm keeps
    // the compiler from moving that use (and its wait) ahead of them
    int page = blk;
    asm volatile("" : "+s"(page));
    const auto kout = make_page_rsrc(k_cache + (int64_t)page * (num_kv_heads * PAGE), page_bytes);
    const auto vout = make_page_rsrc(v_cache + (int64_t)page * (num_kv_heads * PAGE), page_bytes);
#pragma unroll
    for (int j = 0; j < 8; ++j) buffer_store16(kx[j], kout, kdst[j]);
    // row (head, 8 group + k) of the page, slots 8 half .. 8 half + 7
    const uint32_t vrow = (uint32_t)(hg * 8 * kBlock + 8 * half) * 2;
    if (s1 - s0 == 8) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        // output dword m holds slots 2m, 2m+1 of value k
        const uint32_t sel = (k & 1) ? 0x07060302u : 0x05040100u;
        uint32_t w[4];
#pragma unroll
        for (int m = 0; m < 4; ++m)
          w[m] = __builtin_amdgcn_perm(dword(vx[2 * m + 1], k >> 1), dword(vx[2 * m], k >> 1), sel);
        buffer_store16(make_uint4(w[0], w[1], w[2], w[3]), vout,
                       vin_range ? vrow + k * kBlock * 2 : kOffNone);
      }
    } else if (vin_range) {
      // a partly new half: the new slots' 2-byte values alone
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int o = 8 * half + j;
        if (o >= s0 && o < s1) {
#pragma unroll
          for (int k = 0; k < 8; ++k) buffer_store2((uint16_t)elem16(vx[j], k), vout, vrow + (k * kBlock + j) * 2);
        }
      }
    }
  }
}

hipError_t launch_append(const void* k_new, const void* v_new, const int32_t* qsl,
                         const int32_t* ctx, const int32_t* bt, int bt_stride, int num_seqs,
                         int num_tokens, int num_kv_heads, int head_dim, void* k_cache,
                         void* v_cache, hipStream_t stream) {
  // a row of n new tokens touches at most ceil(n / 16) + 1 pages
  const int64_t tasks = (int64_t)num_tokens / kBlock + 2LL * num_seqs;
  if (tasks > INT32_MAX) return hipErrorInvalidValue;
  const dim3 grid((unsigned)tasks), block(kAppendThreads);
  const auto* kn = static_cast<const uint16_t*>(k_new);
  const auto* vn = static_cast<const uint16_t*>(v_new);
  auto* kc = static_cast<uint16_t*>(k_cache);
  auto* vc = static_cast<uint16_t*>(v_cache);
  if (head_dim == 128)
    hipLaunchKernelGGL(append_kernel<128>, grid, block, 0, stream, kn, vn, qsl, ctx, bt, bt_stride,
                       num_seqs, num_kv_heads, kc, vc);
  else
    hipLaunchKernelGGL(append_kernel<64>, grid, block, 0, stream, kn, vn, qsl, ctx, bt, bt_stride,
                       num_seqs, num_kv_heads, kc, vc);
  return hipGetLastError();
}

}  // namespace cpa
