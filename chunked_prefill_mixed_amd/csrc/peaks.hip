// Measured ceilings for the bench's roofline report (libcpa_peaks.so; not part
// of the attention path): a streaming device read and a streaming copy for
// HBM bandwidth and an MFMA-only loop for dense bf16 matrix throughput.  The published MI355X
// figures (8 TB/s, 2.5 PFLOP/s dense bf16) are the roofline peaks; these are
// what the box sustains under the same clocks and power limits.

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// dst[i] = src[i] over n 16-byte words, grid-stride, 4 words in flight per lane
__global__ __launch_bounds__(256) void copy_kernel(uint4* __restrict__ dst,
                                                   const uint4* __restrict__ src, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const uint4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    dst[i] = a;
    dst[i + stride] = b;
    dst[i + 2 * stride] = c;
    dst[i + 3 * stride] = d;
  }
  for (; i < n; i += stride) dst[i] = src[i];
}

// reads n 16-byte words, grid-stride, 8 words in flight per lane; one word per
// thread (the xor of what it read) is written so the loads are not dead code
__global__ __launch_bounds__(256) void read_kernel(const uint4* __restrict__ src, int64_t n,
                                                   uint32_t* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t x = 0;
  for (; i + 7 * stride < n; i += 8 * stride) {
    uint4 v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = src[i + k * stride];
#pragma unroll
    for (int k = 0; k < 8; ++k) x ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  for (; i < n; i += stride) x ^= src[i].x ^ src[i].y ^ src[i].z ^ src[i].w;
  out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = x;
}

// kChains independent v_mfma_f32_32x32x16_bf16 accumulation chains per wave on
// register operands; one float per thread is written so nothing is dead code
constexpr int kChains = 4;
__global__ __launch_bounds__(256) void mfma_kernel(float* __restrict__ out, int iters) {
  bf16x8_t a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(1e-3f * (threadIdx.x + i));
    b[i] = (__bf16)(1e-3f * (i - (int)threadIdx.x));
  }
  f32x16_t acc[kChains];
  for (int c = 0; c < kChains; ++c) acc[c] = f32x16_t{};
  for (int it = 0; it < iters; ++it)
#pragma unroll
    for (int c = 0; c < kChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  float s = 0.f;
  for (int c = 0; c < kChains; ++c)
    for (int i = 0; i < 16; ++i) s += acc[c][i];
  out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

extern "C" {

// Copies bytes (a multiple of 16) from src to dst on stream.  0 or -5 (launch failure).
int cpa_peak_copy(void* dst, const void* src, int64_t bytes, void* stream) {
  if (!dst || !src || bytes <= 0 || bytes % 16) return -1;
  hipLaunchKernelGGL(copy_kernel, dim3(256 * 8), dim3(256), 0, (hipStream_t)stream,
                     static_cast<uint4*>(dst), static_cast<const uint4*>(src), bytes / 16);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

// Reads bytes (a multiple of 16) from src; out must hold 2048 * 256 uint32.  0 or -5.
int cpa_peak_read(const void* src, int64_t bytes, uint32_t* out, void* stream) {
  if (!src || !out || bytes <= 0 || bytes % 16) return -1;
  hipLaunchKernelGGL(read_kernel, dim3(256 * 8), dim3(256), 0, (hipStream_t)stream,
                     static_cast<const uint4*>(src), bytes / 16, out);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

// Runs workgroups x 256 threads of the MFMA loop for iters iterations; out must
// hold workgroups * 256 floats.  Flops = workgroups * 4 waves * iters * 4 chains
// * 32768.  0 or -5.
int cpa_peak_mfma(float* out, int workgroups, int iters, void* stream) {
  if (!out || workgroups <= 0 || iters <= 0) return -1;
  hipLaunchKernelGGL(mfma_kernel, dim3(workgroups), dim3(256), 0, (hipStream_t)stream, out,
                     iters);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

}  // extern "C"
