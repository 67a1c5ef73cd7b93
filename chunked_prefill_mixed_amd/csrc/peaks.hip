// Measured ceilings for the bench's roofline report (libcpa_peaks.so; not part
// of the attention path): a streaming device read and a streaming copy for
// HBM bandwidth and an MFMA-only loop on random operands for dense bf16
// matrix throughput.  The published MI355X
// figures (8 TB/s, 2.5 PFLOP/s dense bf16) are the roofline peaks; these are
// what the GPU sustains under the same clocks and power limits.

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Both streams give each workgroup one contiguous range of the buffer and use
// non-temporal accesses with 8 16-byte words in flight per lane: the fastest
// of the access patterns tried on this GPU (grid-stride and cached loads reach
// 10-20% less).
constexpr int kThreads = 256;
constexpr int kUnroll = 8;

// dst[i] = src[i] over n 16-byte words; n is a multiple of gridDim.x * 2048
__global__ __launch_bounds__(kThreads) void copy_kernel(u32x4_t* __restrict__ dst,
                                                        const u32x4_t* __restrict__ src,
                                                        int64_t n) {
  const int64_t per = n / gridDim.x;
  const u32x4_t* s = src + (int64_t)blockIdx.x * per;
  u32x4_t* d = dst + (int64_t)blockIdx.x * per;
  for (int64_t i = threadIdx.x; i + (kUnroll - 1) * kThreads < per; i += kUnroll * kThreads) {
    u32x4_t v[kUnroll];
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) v[k] = __builtin_nontemporal_load(s + i + k * kThreads);
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) __builtin_nontemporal_store(v[k], d + i + k * kThreads);
  }
}

// reads n 16-byte words (a multiple of gridDim.x * 2048); one word per thread
// (the xor of what it read) is written so the loads are not dead code
__global__ __launch_bounds__(kThreads) void read_kernel(const u32x4_t* __restrict__ src,
                                                        int64_t n, uint32_t* __restrict__ out) {
  const int64_t per = n / gridDim.x;
  const u32x4_t* s = src + (int64_t)blockIdx.x * per;
  uint32_t x = 0;
  for (int64_t i = threadIdx.x; i + (kUnroll - 1) * kThreads < per; i += kUnroll * kThreads) {
    u32x4_t v[kUnroll];
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) v[k] = __builtin_nontemporal_load(s + i + k * kThreads);
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) x ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = x;
}

// MFMA-only loop: kChains independent v_mfma_f32_32x32x16_bf16 accumulation
// chains per wave, kSets register operand sets with random bf16 values in
// (-2, 2) rotated so consecutive MFMAs see different bits.  Matrix-core
// throughput on this chip depends on the operand bits (power): constant
// operands run ~40% faster than random ones, and the attention kernels
// multiply random data, so the ceiling is taken with random operands.  One
// float per thread is written so nothing is dead code.
constexpr int kChains = 4;
constexpr int kSets = 8;

__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}
// two bf16 values uniform in (-2, 2) from the hash of i
__device__ __forceinline__ uint32_t random_bf16x2(uint32_t i) {
  const uint32_t h = mix32(i);
  const __bf16 lo = (__bf16)(((int)(h & 0xFFFF) - 32768) * (2.f / 32768.f));
  const __bf16 hi = (__bf16)(((int)(h >> 16) - 32768) * (2.f / 32768.f));
  return (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
}

__global__ __launch_bounds__(256) void mfma_kernel(float* __restrict__ out, int iters) {
  u32x4_t a[kSets], b[kSets];
  const uint32_t t = (uint32_t)(blockIdx.x * blockDim.x + threadIdx.x) * (8 * kSets);
  for (int s = 0; s < kSets; ++s)
    for (int e = 0; e < 4; ++e) {
      a[s][e] = random_bf16x2(t + 8 * s + e);
      b[s][e] = random_bf16x2(t + 8 * s + e + 4);
    }
  f32x16_t acc[kChains];
  for (int c = 0; c < kChains; ++c) acc[c] = f32x16_t{};
  for (int it = 0; it < iters; ++it)
#pragma unroll
    for (int s = 0; s < kSets; ++s)
      acc[s % kChains] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          __builtin_bit_cast(bf16x8_t, a[s]), __builtin_bit_cast(bf16x8_t, b[(s + it) % kSets]),
          acc[s % kChains], 0, 0, 0);
  float s = 0.f;
  for (int c = 0; c < kChains; ++c)
    for (int i = 0; i < 16; ++i) s += acc[c][i];
  out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

extern "C" {

constexpr int kStreamBlocks = 2048;  // 8 workgroups per CU

// Copies bytes (a multiple of 16 * 2048 * 2048) from src to dst on stream.  0, -1 or -5.
int cpa_peak_copy(void* dst, const void* src, int64_t bytes, void* stream) {
  const int64_t unit = 16LL * kStreamBlocks * kUnroll * kThreads;
  if (!dst || !src || bytes <= 0 || bytes % unit) return -1;
  hipLaunchKernelGGL(copy_kernel, dim3(kStreamBlocks), dim3(kThreads), 0, (hipStream_t)stream,
                     static_cast<u32x4_t*>(dst), static_cast<const u32x4_t*>(src), bytes / 16);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

// Reads bytes (a multiple of 16 * 2048 * 2048) from src; out must hold
// 2048 * 256 uint32.  0, -1 or -5.
int cpa_peak_read(const void* src, int64_t bytes, uint32_t* out, void* stream) {
  const int64_t unit = 16LL * kStreamBlocks * kUnroll * kThreads;
  if (!src || !out || bytes <= 0 || bytes % unit) return -1;
  hipLaunchKernelGGL(read_kernel, dim3(kStreamBlocks), dim3(kThreads), 0, (hipStream_t)stream,
                     static_cast<const u32x4_t*>(src), bytes / 16, out);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

// Runs workgroups x 256 threads of the MFMA loop for iters iterations; out must
// hold workgroups * 256 floats.  Flops = workgroups * 4 waves * iters * 8 MFMAs
// * 32768.  0 or -5.
int cpa_peak_mfma(float* out, int workgroups, int iters, void* stream) {
  if (!out || workgroups <= 0 || iters <= 0) return -1;
  hipLaunchKernelGGL(mfma_kernel, dim3(workgroups), dim3(256), 0, (hipStream_t)stream, out,
                     iters);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

}  // extern "C"
