// Device helpers for the gfx950 kernels: bf16 packing, dot products, DPP
// lane exchanges and the XCD-aware workgroup order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cpa {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int v4u32_t __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

// 2^x on the transcendental unit (v_exp_f32).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// fp32 -> bf16 bits, round to nearest even (lowers to v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint16_t to_bf16(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}
// The two bf16 values of a dword (low half first) as fp32, exactly.
__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xFFFF0000u); }

// acc + sum_i a_i * b_i over 8 bf16 pairs held in 4 dwords, fp32 accumulate
// (v_dot2_f32_bf16: two products per instruction).
__device__ __forceinline__ float dot8_bf16(uint4 a, uint4 b, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.x),
                                        __builtin_bit_cast(bf16x2_t, b.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.y),
                                        __builtin_bit_cast(bf16x2_t, b.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.z),
                                        __builtin_bit_cast(bf16x2_t, b.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.w),
                                        __builtin_bit_cast(bf16x2_t, b.w), acc, false);
  return acc;
}

// Buffer resource (V#) over [base, base + bytes): raw (unstructured) access,
// stride 0; loads past the range return 0.  The last word holds the
// gfx9-family default data format for untyped dword access.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_page_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}
// Cache policy of a load: 0 = default, kNonTemporal = streamed once (the nt
// bit), which spares the caches data that no other wave will read again.
constexpr int kNonTemporal = 2;
// 16 bytes at byte offset off of the resource (buffer_load_dwordx4).
template <int POLICY = 0>
__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, POLICY));
}
// 8 bytes at byte offset off of the resource (buffer_load_dwordx2).
template <int POLICY = 0>
__device__ __forceinline__ uint2 buffer_load8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, POLICY));
}
// Stores of 16 and 2 bytes at byte offset off; a store past the range is
// dropped by the hardware, so an offset of kOffNone skips it without a branch.
constexpr uint32_t kOffNone = 0x80000000u;
__device__ __forceinline__ void buffer_store16(uint4 v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u32_t, v), r, off, 0, 0);
}
__device__ __forceinline__ void buffer_store2(uint16_t v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b16(v, r, off, 0, 0);
}

// 16 bytes per lane from global memory straight into LDS
// (global_load_lds_dwordx4): lane l's bytes land at lds_wave_base + 16 * l,
// and lds_wave_base (a byte address in LDS) must be the same for every lane of
// the wave.  Completion is counted by vmcnt, so the data may be read after
// s_waitcnt vmcnt(0) and a barrier.  The load is written as inline assembly:
// the compiler then does not see it write LDS and does not make later LDS
// reads wait for it (with the builtin it adds that wait wherever it cannot
// tell two double-buffered stages apart).  The caller orders it: wait_vmem()
// and a barrier before any wave reads the bytes.
__device__ __forceinline__ void load_lds16(const void* src, uint32_t lds_wave_base) {
  asm volatile("global_load_lds_dwordx4 %0, off" : : "v"(src), "{m0}"(lds_wave_base) : "memory");
}
// The same with a wave-uniform 64-bit base (SGPRs) and a 32-bit per-lane byte
// offset: the lane's 16 bytes come from base + lane_offset.
__device__ __forceinline__ void load_lds16(const void* base, uint32_t lane_offset,
                                           uint32_t lds_wave_base) {
  asm volatile("global_load_lds_dwordx4 %0, %1"
               :
               : "v"(lane_offset), "s"(base), "{m0}"(lds_wave_base)
               : "memory");
}
// LDS byte address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }


// DPP lane exchanges inside a 16-lane row.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
constexpr int kQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kRowMirror = 0x140;     // lane i <-> 15-i inside a row
constexpr int kRowHalfMirror = 0x141; // lane i <-> 7-i inside each half row

__device__ __forceinline__ float xor_lane(float x, int mask) {
  return __shfl_xor(x, mask, 64);
}

// Combine lane i with lane i ^ 32 in every lane.  v_permlane32_swap
// exchanges lanes 32-63 of one register with lanes 0-31 of another, so after
// swapping two copies of x each lane holds its own value and its partner's;
// the leading s_nop covers the VALU-write-to-permlane-read wait states.
__device__ __forceinline__ float half_max(float x) {
  float y = x;
  asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(x), "+v"(y));
  return fmaxf(x, y);
}
__device__ __forceinline__ float half_sum(float x) {
  float y = x;
  asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(x), "+v"(y));
  return x + y;
}

// acc + the two bf16 values packed in p (v_dot2_f32_bf16 against 1.0, 1.0)
__device__ __forceinline__ float sum2_bf16(uint32_t p, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, p),
                                         __builtin_bit_cast(bf16x2_t, 0x3F803F80u), acc, false);
}

__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp<kQuadXor1>(x));
  x = fmaxf(x, dpp<kQuadXor2>(x));
  x = fmaxf(x, dpp<kRowHalfMirror>(x));
  x = fmaxf(x, dpp<kRowMirror>(x));
  x = fmaxf(x, xor_lane(x, 16));
  x = fmaxf(x, xor_lane(x, 32));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
  x += dpp<kQuadXor1>(x);
  x += dpp<kQuadXor2>(x);
  x += dpp<kRowHalfMirror>(x);
  x += dpp<kRowMirror>(x);
  x += xor_lane(x, 16);
  x += xor_lane(x, 32);
  return x;
}

// Workgroups are handed to the 8 XCDs round-robin by linear id.  Remap so
// each XCD runs one contiguous range of work items: items that share K/V
// (same KV head of one row) then share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int b, int n) {
  const int x = b & 7, i = b >> 3;
  const int base = n >> 3, rem = n & 7;
  return x * base + (x < rem ? x : rem) + i;
}

}  // namespace cpa
