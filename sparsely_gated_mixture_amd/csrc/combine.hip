// Combine and auxiliary losses on gfx950.
//
// Combine (arXiv 1701.06538 summary, xyznot.com, "Method and key formulas":
// y = sum_i G(x)_i E_i(x)): a gather -- one wavefront per token reads the
// expert rows of its kept slots in slot order and writes its output row once.
// No atomics, so the sum order is fixed.  An optional base row (the shared
// expert's output, MoE survey, tufusi.com 6.2: y = E_shared(x) + sum g_i
// E_i(x)) starts the sum.
//
// Aux losses (same page, load-balancing losses; MoE survey, tufusi.com 3.2;
// wkbse.com MoE introduction, part 2): one block computes, in double
// precision with fixed-order tree reductions, w_imp*CV(Importance)^2,
// w_load*CV(Load)^2 (population variance, two passes), alpha*n*sum_i f_i P_i,
// the mean router z statistic and minus the mean gate entropy.
#include "common.h"
#include "launch.h"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y_perm,
                                                      const int32_t* __restrict__ slot_pos,
                                                      const float* __restrict__ topk_w,
                                                      const float* __restrict__ y_base, int T,
                                                      int k, int d, float* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int32_t* sp = slot_pos + (long long)t * k;
  const float* w = topk_w + (long long)t * k;
  for (int c = lane * 4; c < d; c += 64 * 4) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (y_base) acc = *(const f32x4*)(y_base + (long long)t * d + c);
    for (int s = 0; s < k; ++s) {
      const int pos = sp[s];
      if (pos < 0) continue;
      const float ws = w[s];
      const f32x4 v = *(const f32x4*)(y_perm + (long long)pos * d + c);
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] = fmaf(ws, v[q], acc[q]);
    }
    *(f32x4*)(y + (long long)t * d + c) = acc;
  }
}

__global__ __launch_bounds__(256) void aux_kernel(const float* __restrict__ importance,
                                                  const float* __restrict__ load,
                                                  const int32_t* __restrict__ counts_pre,
                                                  const float* __restrict__ gate_stats, int T,
                                                  int k, int n, float w_imp, float w_load,
                                                  float alpha, float w_z, float w_ent,
                                                  float* __restrict__ losses) {
  __shared__ double sh[256];
  block_aux_losses<256>(importance, load, counts_pre, gate_stats, T, k, n, w_imp, w_load, alpha,
                        w_z, w_ent, losses, sh);
}

}  // namespace

hipError_t launch_combine(const float* y_perm, const int32_t* slot_pos, const float* topk_w,
                          const float* y_base, int T, int k, int d, float* y, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  ProfScope ps("combine", s);
  combine_kernel<<<dim3((T + 3) / 4), dim3(256), 0, s>>>(y_perm, slot_pos, topk_w, y_base, T, k,
                                                         d, y);
  return hipGetLastError();
}

hipError_t launch_aux(const float* importance, const float* load, const int32_t* counts_pre,
                      const float* gate_stats, int T, int k, int n, float w_imp, float w_load,
                      float alpha, float w_z, float w_ent, float* losses, hipStream_t s) {
  ProfScope ps("aux_loss", s);
  aux_kernel<<<dim3(1), dim3(256), 0, s>>>(importance, load, counts_pre, gate_stats, T, k, n,
                                           w_imp, w_load, alpha, w_z, w_ent, losses);
  return hipGetLastError();
}

}  // namespace moe
