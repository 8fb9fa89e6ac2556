// Device-side helpers shared by the MSA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));
typedef int32_t i32x16_t __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;
constexpr int kHeadDim = 128;
constexpr int kIdxDim = 64;
constexpr float kLog2e = 1.4426950408889634f;

// Two floats -> two bf16 (round to nearest even) packed low-first.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ uint16_t to_bf16(float f) {
  return (uint16_t)(pack_bf16x2(f, 0.f) & 0xffffu);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// D = A * B + C on a 32x32x16 bf16 MFMA.  Per lane l (wave64):
//   A: 8 values of row m = l % 32, k = 8 * (l / 32) + 0..7
//   B: 8 values of col n = l % 32, k = 8 * (l / 32) + 0..7
//   C/D: 16 values of col n = l % 32, rows 8 * (i / 4) + 4 * (l / 32) + i % 4
__device__ __forceinline__ f32x16_t mfma32x32x16(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Row index (within a 32x32 C tile) of accumulator element i held by a lane
// in half hf = lane / 32.
__device__ __forceinline__ constexpr int c_row(int i, int hf) { return 8 * (i >> 2) + 4 * hf + (i & 3); }

__device__ __forceinline__ float wave_max_pair(float x) {  // max with lane ^ 32
  return fmaxf(x, __shfl_xor(x, 32));
}
__device__ __forceinline__ float wave_sum_pair(float x) { return x + __shfl_xor(x, 32); }

// Orders a wave's LDS writes before other lanes' later reads of them (and
// those reads before later writes): lanes exchanging data through LDS.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Sign-extend the four int8 lanes of a dword.
__device__ __forceinline__ int sx8(uint32_t w, int byte) { return ((int)(w << (24 - 8 * byte))) >> 24; }

__device__ __forceinline__ int sdot4(int a, int b, int c) { return __builtin_amdgcn_sdot4(a, b, c, false); }

// Floor division of a (possibly negative) sum by a positive count.
__device__ __forceinline__ int floor_div(int s, int n) {
  int q = s / n;
  return (q * n != s && s < 0) ? q - 1 : q;
}

}  // namespace msa
