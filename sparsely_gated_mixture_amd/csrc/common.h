// Device helpers shared by the gfx950 kernels of the MoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;   // CDNA wavefront width
constexpr int kXcds = 8;    // MI355X: 8 accelerator complex dies, one L2 each

// fp32 -> bf16 bit pattern, round to nearest, ties to even; NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float((uint32_t)h << 16);
}

// Monotone map float -> uint32 (larger float -> larger key); -0.0 and +0.0
// share one key so they compare equal.
__device__ __forceinline__ uint32_t ordered_key(float v) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_to_float(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}

// Butterfly reductions over the 64 lanes.  Every lane ends with the same
// bits (each step adds / compares the same two operands in both partners).
__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    unsigned long long o = __shfl_xor(v, m, kWave);
    v = o > v ? o : v;
  }
  return v;
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

// Block index -> linear tile index such that each XCD gets one contiguous
// range of tiles (workgroups are dealt to the XCDs round robin), so tiles
// that share operands land on the same L2.  Returns -1 for an idle block.
__device__ __forceinline__ int xcd_tile(int total) {
  const int per = (total + kXcds - 1) / kXcds;
  const int xcd = (int)(blockIdx.x % kXcds);
  const int j = (int)(blockIdx.x / kXcds);
  if (j >= per) return -1;
  const int t = xcd * per + j;
  return t < total ? t : -1;
}

}  // namespace moe
