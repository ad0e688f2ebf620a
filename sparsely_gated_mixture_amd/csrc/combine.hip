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

// One wavefront per token.  Lane s holds the token's slot s (position and
// weight, k <= 64), broadcast with readlane; each pass covers 512 columns
// with two 16-byte vectors per lane, so the loads of every kept row of the
// pass are independent.  Per element: acc = base, then acc = fma(w_s, row_s,
// acc) in slot order.
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y_perm,
                                                      const int32_t* __restrict__ slot_pos,
                                                      const float* __restrict__ topk_w,
                                                      const float* __restrict__ y_base, int T,
                                                      int k, int d, float* __restrict__ y) {
  constexpr int V = 2;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int my_pos = lane < k ? slot_pos[(long long)t * k + lane] : -1;
  const float my_w = lane < k ? topk_w[(long long)t * k + lane] : 0.f;
  for (int c0 = 0; c0 < d; c0 += 64 * 4 * V) {
    bool ok[V];
    int cc[V];
    f32x4 acc[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
      cc[v] = c0 + (v * 64 + lane) * 4;
      ok[v] = cc[v] < d;
      acc[v] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (y_base && ok[v]) acc[v] = *(const f32x4*)(y_base + (long long)t * d + cc[v]);
    }
    for (int s = 0; s < k; ++s) {
      const int pos = __builtin_amdgcn_readlane(my_pos, s);
      if (pos < 0) continue;
      const float ws = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_w), s));
#pragma unroll
      for (int v = 0; v < V; ++v)
        if (ok[v]) {
          const f32x4 x = *(const f32x4*)(y_perm + (long long)pos * d + cc[v]);
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[v][q] = fmaf(ws, x[q], acc[v][q]);
        }
    }
#pragma unroll
    for (int v = 0; v < V; ++v)
      if (ok[v]) *(f32x4*)(y + (long long)t * d + cc[v]) = acc[v];
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
