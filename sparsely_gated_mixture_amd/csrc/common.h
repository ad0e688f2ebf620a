// Device helpers shared by the gfx950 kernels of the MoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;   // CDNA wavefront width

// Token of merged rows base .. base + 7 for the lane's group of 8 (lane / 8),
// base wave-uniform: eight scalar loads (through the constant address space,
// so they count on lgkmcnt and leave the vector-memory count of the copies
// alone), each index clamped to [0, n - 1], then the lane's pick.
__device__ __forceinline__ int row_token8(const int32_t* perm, int base, int n, int lane) {
  typedef __attribute__((address_space(4))) const int32_t cint;
  cint* q = (cint*)perm;
  int v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = base + i;
    v[i] = q[r < n ? r : n - 1];
  }
  const int g = lane >> 3;
  int t = v[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) t = g == i ? v[i] : t;
  return t;
}

// Workgroups a persistent grouped GEMM puts to work on `total` items: the
// whole grid, or its share of a side-by-side run (cu_split), raised until no
// workgroup holds more than kMaxTilesPerWG items (one holds at most
// ceil(total / used) + 1 of them), never above the grid.  A multiple of kXcds.
__device__ inline int gemm_used_grid(const GemmBf16Args& p, int total) {
  const int grid = (int)gridDim.x;
  if (!p.cu_split) return grid;
  const int big = *p.cu_split;
  int want = (p.cu_big ? big : p.num_cus - big) / kXcds * kXcds;
  const int need =
      ((total + kMaxTilesPerWG - 2) / (kMaxTilesPerWG - 1) + kXcds - 1) / kXcds * kXcds;
  want = want > need ? want : need;
  return want < grid ? want : grid;
}

// fp32 -> bf16 bit pattern, round to nearest, ties to even; NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Two fp32 values as packed bf16 bits (a in the low half) with the gfx950
// conversion instruction (v_cvt_pk_bf16_f32): round to nearest, ties to
// even, NaN stays NaN -- the same bits as f32_to_bf16 for every non-NaN
// input.
__device__ __forceinline__ uint32_t bf16x2_bits(float a, float b) {
  typedef __bf16 bf2_t __attribute__((ext_vector_type(2)));
  typedef float f2_t __attribute__((ext_vector_type(2)));
  const bf2_t v = __builtin_convertvector((f2_t){a, b}, bf2_t);
  return __builtin_bit_cast(uint32_t, v);
}

// Eight E4M3 codes (bytes of `raw`, lowest first) as eight bf16 values, with
// the gfx950 conversion instruction (v_cvt_scalef32_pk_bf16_fp8, scale 1).
// Every E4M3 value is exact in bf16, so the widening loses nothing.
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(uint2 raw) {
  typedef __bf16 bf2_t __attribute__((ext_vector_type(2)));
  const bf2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)raw.x, 1.0f, false);
  const bf2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)raw.x, 1.0f, true);
  const bf2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)raw.y, 1.0f, false);
  const bf2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)raw.y, 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
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

// Wave-wide reductions with DPP: pairwise and quad swaps, then rotations by
// 4 and 8 inside each 16-lane row, then the four row results (lanes 0, 16,
// 32, 48) combined in a fixed order in scalar registers.  The result is
// wave-uniform and the summation order is the same on every call.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL,
                                                    0xF, 0xF, false));
}
constexpr int kDppSwap1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kDppSwap2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kDppRor4 = 0x124;  // row_ror:4
constexpr int kDppRor8 = 0x128;  // row_ror:8

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<kDppSwap1>(v));
  v = max(v, dpp_u32<kDppSwap2>(v));
  v = max(v, dpp_u32<kDppRor4>(v));
  v = max(v, dpp_u32<kDppRor8>(v));
  const uint32_t r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
  const uint32_t r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
  return max(max(r0, r1), max(r2, r3));
}

__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += dpp_f32<kDppSwap1>(v);
  v += dpp_f32<kDppSwap2>(v);
  v += dpp_f32<kDppRor4>(v);
  v += dpp_f32<kDppRor8>(v);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (r0 + r1) + (r2 + r3);
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

// Sum over the NT threads of a block: a butterfly inside each wavefront (all
// lanes end with the same bits), then the NT/64 wave sums added in wave
// order.  Same order on every call.  `sh` holds at least NT/64 doubles; every
// thread gets the total.
template <int NT>
__device__ __forceinline__ double block_sum(double v, double* sh) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  double r = 0.0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) r += sh[i];
  __syncthreads();
  return r;
}

// Exclusive prefix sum of one int per thread over a block of NT threads
// (shuffle scan inside each wavefront, wave totals in LDS); also returns the
// block total.  `sh` holds at least NT/64 ints.
template <int NT>
__device__ __forceinline__ int2 block_exscan(int v, int* sh) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += u;
  }
  if (lane == 63) sh[w] = incl;
  __syncthreads();
  int base = 0, total = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    base += i < w ? sh[i] : 0;
    total += sh[i];
  }
  __syncthreads();
  return make_int2(base + incl - v, total);
}

// Squared coefficient of variation of v[0..n) with the population variance,
// two passes, 0 when the mean is 0 (arXiv 1701.06538 summary, xyznot.com,
// load-balancing losses: L = w * CV(.)^2).
template <int NT>
__device__ double block_cv2(const float* v, int n, double* sh) {
  double s = 0.0;
  for (int i = threadIdx.x; i < n; i += NT) s += (double)v[i];
  const double mean = block_sum<NT>(s, sh) / n;
  if (mean == 0.0) return 0.0;
  double q = 0.0;
  for (int i = threadIdx.x; i < n; i += NT) {
    const double dv = (double)v[i] - mean;
    q += dv * dv;
  }
  return (block_sum<NT>(q, sh) / n) / (mean * mean);
}

// losses[0] = w_imp * CV(importance)^2, losses[1] = w_load * CV(load)^2 (0
// without load), losses[2] = alpha * n * sum_i f_i P_i with f_i =
// counts_pre[i]/(T*k) and P_i = importance[i]/T (MoE survey, tufusi.com 3.2);
// losses[3] = w_z * stats[0] / T (router z-loss: mean squared norm of the
// pre-softmax logits) and losses[4] = -w_ent * stats[1] / T (minus the mean
// gate entropy), both 0 without stats or tokens (wkbse.com, part 2).
template <int NT>
__device__ void block_aux_losses(const float* importance, const float* load,
                                 const int32_t* counts_pre, const float* stats, int T, int k,
                                 int n, float w_imp, float w_load, float alpha, float w_z,
                                 float w_ent, float* losses, double* sh) {
  const double li = (double)w_imp * block_cv2<NT>(importance, n, sh);
  const double ll = load ? (double)w_load * block_cv2<NT>(load, n, sh) : 0.0;
  double fp = 0.0;
  if (T > 0) {
    for (int i = threadIdx.x; i < n; i += NT)
      fp += ((double)counts_pre[i] / ((double)T * k)) * ((double)importance[i] / T);
  }
  const double sw = (double)alpha * n * block_sum<NT>(fp, sh);
  if (threadIdx.x == 0) {
    losses[0] = (float)li;
    losses[1] = (float)ll;
    losses[2] = (float)sw;
    const bool st = stats && T > 0;
    losses[3] = st ? (float)((double)w_z * (double)stats[0] / T) : 0.f;
    losses[4] = st ? (float)(-(double)w_ent * (double)stats[1] / T) : 0.f;
  }
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
