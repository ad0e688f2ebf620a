// Packing of expert weights into FP8 E4M3 with a per-row scale, on gfx950.
//
// The DeepSeek-V3 summary of the MoE survey (tufusi.com, section 9) runs its
// main computation in FP8; here the expert weights are stored as E4M3 codes
// (1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits, largest finite
// value 448, no infinities) with one fp32 scale per output row:
//   scale = amax(row) / 448 (1 for a zero row),  code = E4M3(w / scale),
// both divisions in IEEE single precision, rounding to the nearest code with
// ties to an even mantissa, magnitudes past 448 saturating to 448.
//
// Packed layout of one [N, K] matrix (K % 64 == 0, N even): the codes of row
// pair p (rows 2p, 2p+1) and K block b (columns 64b .. 64b+63) are 128
// consecutive bytes, row 2p's 64 codes then row 2p+1's, at byte offset
// (p * K/64 + b) * 128; the N fp32 scales follow the N*K code bytes.  A
// grouped GEMM step (64 columns of 2 rows) then copies whole 128-byte lines.
#include <math.h>

#include "common.h"
#include "launch.h"

namespace moe {
namespace {

// E4M3 code of a finite or NaN fp32 value, from the format's definition.
__device__ __forceinline__ uint32_t e4m3_code(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fabsf(v);
  if (!(a == a)) return 0x7fu;
  if (a >= 464.f) return sign | 0x7eu;  // 464 is the tie between 448 and 480: even code 448
  if (a < 0.015625f) {                  // below 2^-6: subnormal steps of 2^-9
    return sign | (uint32_t)rintf(a * 512.f);  // 8 -> 0x08, the smallest normal
  }
  int e = (int)((__float_as_uint(a) >> 23) & 0xffu) - 127;  // a is a normal fp32 here
  const float mant = a * __uint_as_float((uint32_t)(127 - e) << 23);  // in [1, 2)
  int m = (int)rintf((mant - 1.f) * 8.f);
  if (m == 8) {
    m = 0;
    ++e;
  }
  return sign | (uint32_t)((e + 7) << 3) | (uint32_t)m;
}

// One block per (expert, row): the row's largest magnitude (an order-free
// max), its scale, then the codes.
template <typename T>
__global__ __launch_bounds__(256) void pack_fp8_kernel(const T* __restrict__ src, int N, int K,
                                                       uint8_t* __restrict__ dst) {
  __shared__ float red[4];
  const int e = blockIdx.y, n = blockIdx.x;
  const T* row = src + ((long long)e * N + n) * K;
  auto val = [&](int k) -> float {
    if constexpr (sizeof(T) == 2) return bf16_to_f32(row[k]);
    else return row[k];
  };
  float amax = 0.f;
  for (int k = threadIdx.x; k < K; k += 256) amax = fmaxf(amax, fabsf(val(k)));
  amax = __uint_as_float(wave_max_u32(__float_as_uint(amax)));  // non-negative floats order as uints
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float scale = amax > 0.f ? __fdiv_rn(amax, 448.f) : 1.f;
  uint8_t* base = dst + (long long)e * ((long long)N * K + 4LL * N);
  uint8_t* codes = base + ((long long)(n >> 1) * (K / 64)) * 128 + (n & 1) * 64;
  for (int k = threadIdx.x; k < K; k += 256)
    codes[(k >> 6) * 128 + (k & 63)] = (uint8_t)e4m3_code(__fdiv_rn(val(k), scale));
  if (threadIdx.x == 0) ((float*)(base + (long long)N * K))[n] = scale;
}

}  // namespace

hipError_t launch_pack_fp8(int n_experts, int N, int K, int src_bf16, const void* src, void* dst,
                           hipStream_t s) {
  if (n_experts <= 0 || N <= 0) return hipSuccess;
  ProfScope ps("pack_fp8", s);
  const dim3 grid((unsigned)N, (unsigned)n_experts);
  if (src_bf16)
    pack_fp8_kernel<uint16_t><<<grid, dim3(256), 0, s>>>((const uint16_t*)src, N, K,
                                                         (uint8_t*)dst);
  else
    pack_fp8_kernel<float><<<grid, dim3(256), 0, s>>>((const float*)src, N, K, (uint8_t*)dst);
  return hipGetLastError();
}

}  // namespace moe
