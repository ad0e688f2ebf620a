// Gating network epilogue on gfx950: one wavefront per token row.
//
// Reads the fp32 logits written by the gate GEMM and computes, per row,
//   H_j = clean_j (+ bias_j) + z_j * Softplus(raw_j)      (noisy gate)
// then KeepTopK by k+1 rounds of a wave-wide arg-max over 64-bit keys
// (ordered float bits << 32 | ~index: larger H first, lower index first on
// equal H), the softmax over the kept values (or the Switch full softmax),
// and the per-expert sums behind the auxiliary losses:
//   Importance_j += G_j,  Load_j += Phi((clean_j - thr_j) / Softplus(raw_j)),
// thr_j = H_(k+1) if j is kept, H_(k) otherwise.
// Definitions: arXiv 1701.06538 summary (xyznot.com), "Method and key
// formulas": Noisy Top-K gating and the load-balancing losses; Switch router:
// MoE survey (tufusi.com) section 3.1.
//
// Sums are deterministic: each lane owns fixed experts (j = lane + 64q) and
// accumulates its rows in order; waves are combined in LDS in a fixed order;
// blocks write partial vectors that a second kernel adds in block order.
#include <math.h>

#include "common.h"
#include "launch.h"

namespace moe {
namespace {

__device__ __forceinline__ float softplus_f(float z) {
  return fmaxf(z, 0.f) + log1pf(expf(-fabsf(z)));
}

__device__ __forceinline__ int readlane_i(int v, int l) { return __builtin_amdgcn_readlane(v, l); }
__device__ __forceinline__ float readlane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

template <int NPL>
__global__ __launch_bounds__(256) void topk_kernel(const TopkArgs p) {
  extern __shared__ float red[];  // [2][4][n]
  const int n = p.n, k = p.k;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

  int row_begin, row_end, part, g = 0;
  const bool grouped = p.tile_expert != nullptr;
  if (grouped) {
    if ((int)blockIdx.x >= *p.tile_count) return;
    part = blockIdx.x;
    g = p.tile_expert[part];
    row_begin = p.tile_row0[part];
    row_end = min(row_begin + p.tile_rows, p.offsets[g + 1]);
  } else {
    part = blockIdx.x;
    row_begin = part * p.rows_per_block;
    row_end = min(row_begin + p.rows_per_block, p.rows);
  }

  float imp[NPL], ld[NPL];
#pragma unroll
  for (int q = 0; q < NPL; ++q) imp[q] = ld[q] = 0.f;

  const int R = min(k + 1, n);
  for (int r = row_begin + wave; r < row_end; r += 4) {
    // Token / slot of this row, and where its noise and outputs live.
    long long noise_row, out_base;
    float wprim = 1.f;
    int id_base = 0;
    if (grouped) {
      const int t = p.row_token[r];
      int s = 0;
      for (int q = 0; q < p.k1; ++q)
        if (p.prim_idx[(long long)t * p.k1 + q] == g) s = q;
      noise_row = ((long long)t * p.k1 + s) * n;
      out_base = (long long)t * p.k1 * k + (long long)s * k;
      wprim = p.prim_w[(long long)t * p.k1 + s];
      id_base = g * n;
    } else {
      noise_row = (long long)r * n;
      out_base = (long long)r * k;
    }
    const float* lg = p.logits + (long long)r * p.ldl;

    float cl[NPL], sp[NPL], hv[NPL];
    unsigned long long key[NPL];
#pragma unroll
    for (int q = 0; q < NPL; ++q) {
      const int j = lane + 64 * q;
      const bool ok = j < n;
      float c = 0.f, s = 1.f, h = 0.f;
      if (ok) {
        c = lg[j];
        if (p.bias) c += p.bias[j];
        h = c;
        if (p.noisy) {
          s = softplus_f(lg[n + j]);
          h = c + p.noise[noise_row + j] * s;
        }
      }
      cl[q] = c;
      sp[q] = s;
      hv[q] = h;
      key[q] = ok ? (((unsigned long long)ordered_key(h) << 32) | (unsigned)(~j)) : 0ull;
    }

    unsigned selmask = 0;
    int my_j = 0;
    float my_v = 0.f, v0 = 0.f, v_km1 = 0.f, v_k = -INFINITY;
    for (int rd = 0; rd < R; ++rd) {
      unsigned long long best = 0;
#pragma unroll
      for (int q = 0; q < NPL; ++q) best = key[q] > best ? key[q] : best;
      best = wave_max_u64(best);
      const int j = (int)(~(unsigned)(best & 0xffffffffull));
      const float v = key_to_float((unsigned)(best >> 32));
      if (lane == (j & 63)) {
#pragma unroll
        for (int q = 0; q < NPL; ++q)
          if (q == (j >> 6)) {
            key[q] = 0ull;
            if (rd < k) selmask |= 1u << q;
          }
      }
      if (rd == lane) {
        my_j = j;
        my_v = v;
      }
      if (rd == 0) v0 = v;
      if (rd == k - 1) v_km1 = v;
      if (rd == k) v_k = v;
    }

    // Gate weights of the kept slots (lane s holds slot s).
    float w;
    float zsum = 0.f;
    if (p.switch_mode) {
      float ls = 0.f;
#pragma unroll
      for (int q = 0; q < NPL; ++q)
        if (lane + 64 * q < n) ls += expf(hv[q] - v0);
      zsum = wave_sum_f32(ls);
      w = (lane < k) ? expf(my_v - v0) / zsum : 0.f;
    } else {
      const float e = (lane < k) ? expf(my_v - v0) : 0.f;
      zsum = wave_sum_f32(e);
      w = e / zsum;
    }
    if (lane < k) {
      p.topk_idx[out_base + lane] = id_base + my_j;
      p.topk_w[out_base + lane] = wprim * w;
    }

    // Importance: the dense gate vector (Switch: the full softmax).
    if (p.switch_mode) {
#pragma unroll
      for (int q = 0; q < NPL; ++q)
        if (lane + 64 * q < n) imp[q] += expf(hv[q] - v0) / zsum;
    } else {
      for (int s = 0; s < k; ++s) {
        const int js = readlane_i(my_j, s);
        const float ws = readlane_f(w, s) * wprim;
        if (lane == (js & 63)) {
#pragma unroll
          for (int q = 0; q < NPL; ++q)
            if (q == (js >> 6)) imp[q] += ws;
        }
      }
    }
    // Load: smooth count P(x, j).
    if (p.noisy) {
#pragma unroll
      for (int q = 0; q < NPL; ++q) {
        if (lane + 64 * q < n) {
          const float thr = ((selmask >> q) & 1u) ? v_k : v_km1;
          const float z = (cl[q] - thr) / sp[q];
          ld[q] += 0.5f * erfcf(-z * 0.70710678118654752f);
        }
      }
    }
  }

  // Combine the 4 waves in a fixed order, then write this block's partials.
  float* ri = red;
  float* rl = red + 4 * n;
#pragma unroll
  for (int q = 0; q < NPL; ++q) {
    const int j = lane + 64 * q;
    if (j < n) {
      ri[wave * n + j] = imp[q];
      rl[wave * n + j] = ld[q];
    }
  }
  __syncthreads();
  for (int j = threadIdx.x; j < n; j += 256) {
    const float si = ((ri[j] + ri[n + j]) + ri[2 * n + j]) + ri[3 * n + j];
    p.part_imp[(long long)part * n + j] = si;
    if (p.part_load) {
      const float sl = ((rl[j] + rl[n + j]) + rl[2 * n + j]) + rl[3 * n + j];
      p.part_load[(long long)part * n + j] = sl;
    }
  }
}

// out[j] = sum of part[p][j] over p.  64 columns per block; 16 part-lanes per
// column each add every 16th partial in ascending order (coalesced rows,
// many loads in flight), then lane sums are added in lane order: the same
// order on every call.
constexpr int kColLanes = 16;
__global__ __launch_bounds__(1024) void colsum_kernel(const float* __restrict__ part, int nparts,
                                                      int n, float* __restrict__ out) {
  __shared__ double sh[kColLanes][64];
  const int c = threadIdx.x & 63, q = threadIdx.x >> 6;
  const int j = blockIdx.x * 64 + c;
  double s = 0.0;
  if (j < n) {
#pragma unroll 8
    for (int p = q; p < nparts; p += kColLanes) s += (double)part[(long long)p * n + j];
  }
  sh[q][c] = s;
  __syncthreads();
  if (q == 0 && j < n) {
    double t = 0.0;
    for (int r = 0; r < kColLanes; ++r) t += sh[r][c];
    out[j] = (float)t;
  }
}

// One thread per (group g, expert e): sum the tiles of group g in order.
__global__ void hier_finalize_kernel(const float* __restrict__ part_imp,
                                     const float* __restrict__ part_load,
                                     const int32_t* __restrict__ tile_expert,
                                     const int32_t* __restrict__ tile_count,
                                     const int32_t* __restrict__ group_counts,
                                     const float* __restrict__ load_primary, int a, int b,
                                     float* __restrict__ importance, float* __restrict__ load) {
  const int id = blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= a * b) return;
  const int g = id / b, e = id % b;
  const int nt = *tile_count;
  // Tiles are in group order: find the first tile of g by binary search.
  int lo = 0, hi = nt;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (tile_expert[mid] < g) lo = mid + 1; else hi = mid;
  }
  double si = 0.0, sl = 0.0;
  for (int t = lo; t < nt && tile_expert[t] == g; ++t) {
    si += (double)part_imp[(long long)t * b + e];
    if (part_load) sl += (double)part_load[(long long)t * b + e];
  }
  importance[id] = (float)si;
  if (load) {
    const int cnt = group_counts[g];
    load[id] = cnt > 0 ? (float)((double)load_primary[g] * sl / (double)cnt) : 0.f;
  }
}

template <int NPL>
hipError_t launch_topk_t(const TopkArgs& a, int grid, hipStream_t s) {
  const size_t shm = (size_t)2 * 4 * a.n * sizeof(float);
  ProfScope ps(a.tile_expert ? "gate_topk_grouped" : "gate_topk", s);
  topk_kernel<NPL><<<dim3(grid), dim3(256), shm, s>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_topk(const TopkArgs& a, hipStream_t s) {
  const int grid = a.tile_expert ? a.max_tiles
                                 : (a.rows + a.rows_per_block - 1) / a.rows_per_block;
  if (grid <= 0) return hipSuccess;
  const int npl = (a.n + 63) / 64;
  if (npl <= 1) return launch_topk_t<1>(a, grid, s);
  if (npl <= 2) return launch_topk_t<2>(a, grid, s);
  if (npl <= 4) return launch_topk_t<4>(a, grid, s);
  if (npl <= 8) return launch_topk_t<8>(a, grid, s);
  if (npl <= 16) return launch_topk_t<16>(a, grid, s);
  return launch_topk_t<32>(a, grid, s);
}

hipError_t launch_colsum(const float* part, int nparts, int n, float* out, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  ProfScope ps("gate_colsum", s);
  colsum_kernel<<<dim3((n + 63) / 64), dim3(64 * kColLanes), 0, s>>>(part, nparts, n, out);
  return hipGetLastError();
}

hipError_t launch_hier_finalize(const float* part_imp, const float* part_load,
                                const int32_t* tile_expert, const int32_t* tile_count,
                                const int32_t* group_counts, const float* load_primary, int a,
                                int b, float* importance, float* load, hipStream_t s) {
  const int total = a * b;
  if (total <= 0) return hipSuccess;
  ProfScope ps("hier_finalize", s);
  hier_finalize_kernel<<<dim3((total + 255) / 256), dim3(256), 0, s>>>(
      part_imp, part_load, tile_expert, tile_count, group_counts, load_primary, a, b,
      importance, load);
  return hipGetLastError();
}

}  // namespace moe
