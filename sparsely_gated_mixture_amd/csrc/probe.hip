// Peak probes: a loop of MFMA instructions on register operands and nothing
// else, and a plain HBM read stream, so that the attainable bf16 / fp32
// matrix rates and read bandwidth of the device can be measured next to the
// datasheet figures the layer's kernels are graded against.
//
// Each 64-lane wave keeps four independent accumulators and issues four
// MFMAs per iteration (v_mfma_f32_32x32x16_bf16: 32768 flops each;
// v_mfma_f32_32x32x2f32: 4096 flops each).  The operands depend on the lane
// and the loop counter, and every lane stores one value of the result, so
// the compiler can neither fold nor drop the loop.
#include "common.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kProbeThreads = 256;  // 4 waves per block

__global__ __launch_bounds__(kProbeThreads) void mfma_bf16_loop(int iters, float* sink) {
  const int t = threadIdx.x;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (float)((t + i) & 7));
    b[i] = (__bf16)(0.002f * (float)((t * 3 + i) & 7));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, b, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int v = 0; v < 16; ++v) s += c0[v] + c1[v] + c2[v] + c3[v];
  sink[(long long)blockIdx.x * kProbeThreads + t] = s;
}

__global__ __launch_bounds__(kProbeThreads) void mfma_f32_loop(int iters, float* sink) {
  const int t = threadIdx.x;
  const float a = 0.001f * (float)(t & 7), b = 0.002f * (float)((t * 3) & 7);
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x2f32(b, a, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x2f32(a, a, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x2f32(b, b, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int v = 0; v < 16; ++v) s += c0[v] + c1[v] + c2[v] + c3[v];
  sink[(long long)blockIdx.x * kProbeThreads + t] = s;
}

// HBM read stream: block b reads its own contiguous segment of the buffer
// (about n16 / gridDim chunks of 16 bytes), 32 KB per iteration with eight
// independent 16-byte loads per thread in flight, and folds them into a
// per-thread checksum, so the loads cannot be dropped.  Thread t of a block
// reads the chunks whose offset within the segment is t modulo 256.
__global__ __launch_bounds__(kProbeThreads) void hbm_read_stream(const uint4* __restrict__ buf,
                                                                 long long n16, float* sink) {
  const long long per = (n16 + gridDim.x - 1) / gridDim.x;
  const long long beg = (long long)blockIdx.x * per;
  const long long end = min(n16, beg + per);
  uint32_t acc = 0;
  for (long long base = beg + threadIdx.x; base < end; base += 8 * kProbeThreads) {
    uint4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const long long i = base + u * kProbeThreads;
      v[u] = i < end ? buf[i] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  sink[(long long)blockIdx.x * kProbeThreads + threadIdx.x] = (float)(acc & 0xffffu);
}

}  // namespace

hipError_t launch_hbm_read_probe(const void* buf, long long bytes, int blocks, float* sink,
                                 hipStream_t s) {
  hbm_read_stream<<<dim3((unsigned)blocks), dim3(kProbeThreads), 0, s>>>(
      (const uint4*)buf, bytes / 16, sink);
  return hipGetLastError();
}

hipError_t launch_mfma_probe(bool bf16, int blocks, int iters, float* sink, hipStream_t s) {
  if (bf16)
    mfma_bf16_loop<<<dim3((unsigned)blocks), dim3(kProbeThreads), 0, s>>>(iters, sink);
  else
    mfma_f32_loop<<<dim3((unsigned)blocks), dim3(kProbeThreads), 0, s>>>(iters, sink);
  return hipGetLastError();
}

}  // namespace moe
