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
// wkbse.com MoE introduction, part 2), as an extra block of the layer
// forward's combine launch or a launch of their own: one block computes, in double
// precision with fixed-order tree reductions, w_imp*CV(Importance)^2,
// w_load*CV(Load)^2 (population variance, two passes), alpha*n*sum_i f_i P_i,
// the mean router z statistic and minus the mean gate entropy.
#include "common.h"
#include "launch.h"

namespace moe {
namespace {

typedef unsigned int v2u32 __attribute__((ext_vector_type(2)));

// wpt wavefronts per token (1 while the batch fills the chip, else up to 8,
// each taking every wpt-th pass of the row).  Lane s holds the token's slot s
// (position and weight, k <= 64), broadcast with readlane; each pass covers
// 512 columns with two 16-byte vectors per lane.  The slots go in groups of eight: the
// loads of a group's rows are all issued before its multiply-adds, so a wave
// keeps 16 KB of y_perm in flight.  Each slot's row is read through a
// buffer descriptor over that row (scalar registers: the row is the same for
// the whole wave); a dropped slot's descriptor spans nothing, so its loads
// return zeros without a memory access and no branch breaks the group.
// Per element: acc = base, then acc = fma(w_s, row_s, acc) in slot order (a
// dropped slot adds w_s * 0).  TY: the element type of y_perm (float, or
// uint16_t for bf16 rows, widened exactly to fp32 before the multiply-add).
template <typename TY>
__global__ __launch_bounds__(256) void combine_kernel(const TY* __restrict__ y_perm,
                                                      const int32_t* __restrict__ slot_pos,
                                                      const float* __restrict__ topk_w,
                                                      const float* __restrict__ y_base, int T,
                                                      int k, int d, int wpt,
                                                      float* __restrict__ y, const AuxArgs aux) {
  // Block 0 of a launch with losses computes them, beside the token blocks
  // (dispatched first, it does not extend the launch's tail).
  if (aux.losses && blockIdx.x == 0) {
    __shared__ double sh[256];
    block_aux_losses<256>(aux.importance, aux.load, aux.counts_pre, aux.gate_stats, aux.T, aux.k,
                          aux.n, aux.w_imp, aux.w_load, aux.alpha, aux.w_z, aux.w_ent,
                          aux.losses, sh);
    return;
  }
  constexpr int V = 2;
  constexpr int G = 8;  // slots per group of loads
  const int lane = threadIdx.x & 63;
  const int gw = ((int)blockIdx.x - (aux.losses ? 1 : 0)) * 4 + (threadIdx.x >> 6);
  const int t = gw / wpt, part = gw % wpt;
  if (t >= T) return;
  const int my_pos = lane < k ? slot_pos[(long long)t * k + lane] : -1;
  const float my_w = lane < k ? topk_w[(long long)t * k + lane] : 0.f;
  constexpr int kOutOfRange = 0x40000000;  // past every row's descriptor
  for (int c0 = part * 64 * 4 * V; c0 < d; c0 += 64 * 4 * V * wpt) {
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
    for (int s0 = 0; s0 < k; s0 += G) {
      f32x4 x[G][V];
      float ws[G];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const int s = s0 + g;  // s < 64 always; lanes past k hold pos -1 and weight 0
        const int pos = __builtin_amdgcn_readlane(my_pos, s & 63);
        ws[g] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_w), s & 63));
        const bool live = pos >= 0 && s < k;
        constexpr int ES = (int)sizeof(TY);
        const __amdgpu_buffer_rsrc_t yr = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<TY*>(y_perm) + (long long)(live ? pos : 0) * d, (short)0,
            live ? d * ES : 0, 0x00020000);
#pragma unroll
        for (int v = 0; v < V; ++v) {
          if constexpr (ES == 4) {
            x[g][v] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                    yr, ok[v] ? cc[v] * 4 : kOutOfRange, 0, 0));
          } else {
            // 4 bf16 values; each widens to fp32 by a 16-bit shift
            const v2u32 r = __builtin_amdgcn_raw_buffer_load_b64(
                yr, ok[v] ? cc[v] * 2 : kOutOfRange, 0, 0);
            x[g][v] = f32x4{__uint_as_float(r[0] << 16), __uint_as_float(r[0] & 0xffff0000u),
                            __uint_as_float(r[1] << 16), __uint_as_float(r[1] & 0xffff0000u)};
          }
        }
      }
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int v = 0; v < V; ++v)
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[v][q] = fmaf(ws[g], x[g][v][q], acc[v][q]);
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

hipError_t launch_combine(const void* y_perm, const int32_t* slot_pos, const float* topk_w,
                          const float* y_base, int T, int k, int d, float* y, hipStream_t s,
                          const AuxArgs* aux, bool y_bf16) {
  if (T <= 0) {
    if (aux && aux->losses)
      return launch_aux(aux->importance, aux->load, aux->counts_pre, aux->gate_stats, aux->T,
                        aux->k, aux->n, aux->w_imp, aux->w_load, aux->alpha, aux->w_z,
                        aux->w_ent, aux->losses, s);
    return hipSuccess;
  }
  // Waves per token: enough for about 8192 waves (32 per CU), at most one
  // per 512-column pass and at most 8.
  const int passes = (d + 511) / 512;
  int wpt = (8192 + T - 1) / T;
  wpt = wpt < 1 ? 1 : wpt > 8 ? 8 : wpt;
  if (wpt > passes) wpt = passes;
  const long long waves = (long long)T * wpt;
  const AuxArgs ax = aux ? *aux : AuxArgs{};
  const long long blocks = (waves + 3) / 4 + (ax.losses ? 1 : 0);
  ProfScope ps("combine", s);
  if (y_bf16)
    combine_kernel<uint16_t><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(
        (const uint16_t*)y_perm, slot_pos, topk_w, y_base, T, k, d, wpt, y, ax);
  else
    combine_kernel<float><<<dim3((unsigned)blocks), dim3(256), 0, s>>>((const float*)y_perm, slot_pos, topk_w,
                                                                       y_base, T, k, d, wpt, y, ax);
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
