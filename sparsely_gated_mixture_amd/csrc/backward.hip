// Backward pass of the flat MoE layer on gfx950: the kernels around the
// expert GEMMs (those are in ggemm_bwd.hip) and the gate epilogue (gate.hip).
//
// The gradients follow the chain rule through the forward with the routing
// held fixed (arXiv 1701.06538 summary, xyznot.com, FAQ: the selection comes
// before the softmax, so the kept gate values stay differentiable).
// Objective: L = sum_t <dy_t, y_t> + sum_j dl_j * losses_j.
//
// Kernels:
//  * combine_bwd: per token, dG[t,s] = <dy_t, y_perm[row]> and the expert's
//    output gradient row = bf16(topk_w[t,s] * dy_t), for each kept slot;
//  * loss_grad: dImportance, dLoad and the z / entropy coefficients from the
//    upstream loss gradients (one block, double precision);
//  * gate_wgrad (fp32 MFMA, split over tokens) + wgrad_reduce: the gate's
//    weight gradients dlogits^T x, partial products summed in a fixed order;
//  * transpose_gate: [W_g; W_noise]^T for the input gradient through the
//    gate (then the forward's split-bf16 gate GEMM, gemm_gate.hip);
//  * seg_colsum: per-expert column sums of bf16 rows (expert bias gradients);
//  * dx_gather: per token, the gate's input gradient plus its kept rows'
//    input gradients in slot order (plus the shared expert's);
//  * swiglu_hidden: silu(a) * b rounded to bf16, from the saved
//    pre-activations, with the forward epilogue's arithmetic.
// Every sum has a fixed order: the results are bitwise reproducible.
#include <math.h>

#include "common.h"
#include "launch.h"
#include "lds_dma.h"

namespace moe {
namespace {

template <bool F32OUT>
__global__ __launch_bounds__(256) void combine_bwd_kernel(
    const float* __restrict__ dy, const float* __restrict__ y_perm,
    const int32_t* __restrict__ slot_pos, const float* __restrict__ topk_w, int T, int k, int d,
    float* __restrict__ dG, void* __restrict__ dout) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* dyr = dy + (long long)t * d;
  for (int s = 0; s < k; ++s) {
    const int pos = slot_pos[(long long)t * k + s];
    if (pos < 0) {
      if (lane == 0) dG[(long long)t * k + s] = 0.f;
      continue;
    }
    const float w = topk_w[(long long)t * k + s];
    const float* yr = y_perm + (long long)pos * d;
    float acc = 0.f;
    for (int c = lane * 4; c < d; c += 256) {
      const f32x4 g = *(const f32x4*)(dyr + c);
      const f32x4 v = *(const f32x4*)(yr + c);
#pragma unroll
      for (int q = 0; q < 4; ++q) acc = fmaf(g[q], v[q], acc);
      if constexpr (F32OUT) {
        *(f32x4*)((float*)dout + (long long)pos * d + c) =
            f32x4{w * g[0], w * g[1], w * g[2], w * g[3]};
      } else {
        *(uint2*)((uint16_t*)dout + (long long)pos * d + c) =
            make_uint2(bf16x2_bits(w * g[0], w * g[1]), bf16x2_bits(w * g[2], w * g[3]));
      }
    }
    const float tot = wave_sum_dpp(acc);
    if (lane == 0) dG[(long long)t * k + s] = tot;
  }
}

// d CV(v)^2 / d v_i = (2 / (n m^2)) ((v_i - m) - var / m) with the mean m and
// the population variance var; 0 when m = 0 (CV^2 is 0 there).
__global__ __launch_bounds__(256) void loss_grad_kernel(
    const float* __restrict__ importance, const float* __restrict__ load,
    const int32_t* __restrict__ counts_pre, const float* __restrict__ dl, int T, int k, int n,
    float w_imp, float w_load, float alpha, float w_z, float w_ent, float* __restrict__ dimp,
    float* __restrict__ dload, float* __restrict__ coef) {
  __shared__ double sh[4];
  const double d0 = dl[0], d1 = dl[1], d2 = dl[2], d3 = dl[3], d4 = dl[4];
  for (int pass = 0; pass < 2; ++pass) {
    const float* v = pass == 0 ? importance : load;
    float* out = pass == 0 ? dimp : dload;
    if (!v) break;
    const double scale = pass == 0 ? d0 * w_imp : d1 * w_load;
    double s = 0.0;
    for (int i = threadIdx.x; i < n; i += 256) s += (double)v[i];
    const double m = block_sum<256>(s, sh) / n;
    double q = 0.0;
    for (int i = threadIdx.x; i < n; i += 256) {
      const double dv = (double)v[i] - m;
      q += dv * dv;
    }
    const double var = block_sum<256>(q, sh) / n;
    for (int i = threadIdx.x; i < n; i += 256) {
      double g = m != 0.0 ? scale * (2.0 / (n * m * m)) * (((double)v[i] - m) - var / m) : 0.0;
      if (pass == 0 && T > 0)
        g += d2 * alpha * n * ((double)counts_pre[i] / ((double)T * k)) / T;
      out[i] = (float)g;
    }
  }
  if (threadIdx.x == 0) {
    coef[0] = T > 0 ? (float)(d3 * w_z / T) : 0.f;
    coef[1] = T > 0 ? (float)(d4 * w_ent / T) : 0.f;
    coef[2] = coef[0];  // the same z coefficient without an entropy term
    coef[3] = 0.f;
  }
}

// ---------------------------------------------------------------------------
// Gate weight gradients: P[split][m][c] = sum over tokens t of the split's
// range of dlogits[t][m] * x[t][c] (v_mfma_f32_32x32x2f32), then
// out[m][c] = sum of P over the splits in order.  Both operands are token
// rows, so their tiles are copied to LDS as stored.  128 x 128 output tiles
// of D[c][m] (c: model dim, m: logit column) on 4 waves; K-steps of 32
// tokens, double-buffered.
// ---------------------------------------------------------------------------
constexpr int kGwTile = 128, kGwBK = 32, kGwHalf = kGwBK * kGwTile * 4;  // 16 KB

// Byte offset of (token row r, column c) in a 32 x 128 fp32 tile; 16-byte
// chunks of odd rows are moved by 8 chunks, so the two rows a read touches
// use different banks.
__device__ __forceinline__ uint32_t gw_off(int r, int c) {
  return (uint32_t)(r * 512 + ((((c >> 2) ^ ((r & 1) << 3))) << 4) + (c & 3) * 4);
}

__global__ __launch_bounds__(256, 2) void gate_wgrad_kernel(GateWgradArgs p) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[4 * kGwHalf];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wc = wave >> 1, wm = wave & 1;
  const int CT = (p.d + kGwTile - 1) / kGwTile, MT = (p.M + kGwTile - 1) / kGwTile;
  const int t = xcd_tile(p.splits * CT * MT);
  if (t < 0) return;
  const int split = t / (CT * MT);
  const int rem = t % (CT * MT);
  const int c0 = (rem / MT) * kGwTile, m0 = (rem % MT) * kGwTile;
  const int t_lo = split * p.tokens_per_split;
  const int t_hi = min(p.T, t_lo + p.tokens_per_split);
  const int nsteps = t_hi > t_lo ? (t_hi - t_lo + kGwBK - 1) / kGwBK : 0;
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;

  auto issue = [&](int step, int st) {
    const int tb = t_lo + step * kGwBK;
    const uint32_t sx = lds0 + st * 2 * kGwHalf, sg = sx + kGwHalf;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int pos = (wave * 4 + q) * 64 + lane;  // 16-byte chunk of the tile
      const int r = pos >> 5;
      const int cc = ((pos & 31) ^ ((r & 1) << 3)) << 2;
      const int tok = tb + r;
      const void* sxp = kZeroChunk;
      const void* sgp = kZeroChunk;
      if (tok < t_hi) {
        if (c0 + cc < p.d) sxp = p.x + (long long)tok * p.d + c0 + cc;
        if (m0 + cc < p.M) sgp = p.dlogits + (long long)tok * p.ldd + m0 + cc;
      }
      dma16(sxp, sx + (wave * 4 + q) * 1024);
      dma16(sgp, sg + (wave * 4 + q) * 1024);
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  if (nsteps > 0) issue(0, 0);
  for (int g = 0; g < nsteps; ++g) {
    if (g + 1 < nsteps) {
      issue(g + 1, (g + 1) & 1);
      wait_vm<8>();
    } else {
      wait_vm<0>();
    }
    __syncthreads();
    const uint8_t* sx = smem + (g & 1) * 2 * kGwHalf;
    const uint8_t* sg = sx + kGwHalf;
#pragma unroll
    for (int kk = 0; kk < kGwBK / 2; ++kk) {
      const int r = 2 * kk + (lane >> 5);
      float a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = *(const float*)(sx + gw_off(r, wc * 64 + i * 32 + (lane & 31)));
#pragma unroll
      for (int j = 0; j < 2; ++j)
        b[j] = *(const float*)(sg + gw_off(r, wm * 64 + j * 32 + (lane & 31)));
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }

  // lane holds D[c .. c+3][m]: P[split][m][c .. c+3]
  float* P = p.partial + (long long)split * p.M * p.d;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int m = m0 + wm * 64 + j * 32 + (lane & 31);
    if (m >= p.M) continue;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = c0 + wc * 64 + i * 32 + 8 * q + 4 * (lane >> 5);
        if (c >= p.d) continue;
        *(f32x4*)(P + (long long)m * p.d + c) =
            f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                  acc[i][j][4 * q + 3]};
      }
  }
}

// out row m (< n: dw_gate, else dw_noise row m - n) = sum of the splits' rows.
__global__ __launch_bounds__(256) void wgrad_reduce_kernel(const float* __restrict__ partial,
                                                           int splits, int M, int n, int d,
                                                           float* __restrict__ dw_gate,
                                                           float* __restrict__ dw_noise) {
  const long long i4 = ((long long)blockIdx.x * 256 + threadIdx.x) * 4;
  const long long total = (long long)M * d;
  if (i4 >= total) return;
  // The splits are added in order; their loads go out four at a time.
  f32x4 s = *(const f32x4*)(partial + i4);
  int sp = 1;
  for (; sp + 4 <= splits; sp += 4) {
    f32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = *(const f32x4*)(partial + (long long)(sp + u) * total + i4);
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int q = 0; q < 4; ++q) s[q] += v[u][q];
  }
  for (; sp < splits; ++sp) {
    const f32x4 v = *(const f32x4*)(partial + (long long)sp * total + i4);
#pragma unroll
    for (int q = 0; q < 4; ++q) s[q] += v[q];
  }
  const long long m = i4 / d, c = i4 % d;
  float* out = m < n ? dw_gate + m * d + c : dw_noise + (m - n) * d + c;
  *(f32x4*)out = s;
}

// wt[c][j] = j < n ? w_gate[j][c] : (j < 2n and w_noise ? w_noise[j-n][c] : 0),
// for c < d, j < ldk.
__global__ __launch_bounds__(256) void transpose_gate_kernel(const float* __restrict__ w_gate,
                                                             const float* __restrict__ w_noise,
                                                             int n, int d, int ldk,
                                                             float* __restrict__ wt) {
  __shared__ float tile[32][33];
  const int j0 = blockIdx.x * 32, c0 = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 8 rows per pass
  for (int r = ty; r < 32; r += 8) {
    const int j = j0 + r, c = c0 + tx;
    float v = 0.f;
    if (c < d) {
      if (j < n) v = w_gate[(long long)j * d + c];
      else if (w_noise && j < 2 * n) v = w_noise[(long long)(j - n) * d + c];
    }
    tile[r][tx] = v;
  }
  __syncthreads();
  for (int r = ty; r < 32; r += 8) {
    const int c = c0 + r, j = j0 + tx;
    if (c < d && j < ldk) wt[(long long)c * ldk + j] = tile[tx][r];
  }
}

// out[e][c] = sum over the rows of segment e (in row order) of src[row][c].
template <bool F32>
__global__ __launch_bounds__(256) void seg_colsum_kernel(const void* __restrict__ src,
                                                         long long ld,
                                                         const int32_t* __restrict__ offsets,
                                                         int N, float* __restrict__ out) {
  const int e = blockIdx.y;
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= N) return;
  double s = 0.0;
  for (int r = offsets[e]; r < offsets[e + 1]; ++r) {
    const long long i = (long long)r * ld + c;
    s += F32 ? (double)((const float*)src)[i] : (double)bf16_to_f32(((const uint16_t*)src)[i]);
  }
  out[(long long)e * N + c] = (float)s;
}

// dx[t] = the gate's dx + the shared expert's + the two-level secondary
// gates' rows of the token + its kept slots' rows of dinput, added in that
// order (slot order within each), one wavefront per token.  Lane s holds the
// token's slot s; each pass covers 512 columns with two 16-byte vectors per
// lane, so every source row's loads of the pass are independent.
__global__ __launch_bounds__(256) void dx_gather_kernel(const float* __restrict__ dx_gate,
                                                        const float* __restrict__ dx_shared,
                                                        const float* __restrict__ du_perm,
                                                        const int32_t* __restrict__ slot_pos,
                                                        int T, int k, int d,
                                                        const float* __restrict__ du2,
                                                        const int32_t* __restrict__ slot2, int k2,
                                                        float* __restrict__ dx) {
  constexpr int V = 2;  // 16-byte vectors per lane per pass: a 512-wide row in one pass
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  // Lane s holds the token's slot s (k, k2 <= 64), broadcast with readlane.
  const int my = lane < k ? slot_pos[(long long)t * k + lane] : -1;
  const int my2 = lane < k2 ? slot2[(long long)t * k2 + lane] : -1;
  for (int c0 = 0; c0 < d; c0 += 64 * 4 * V) {
    bool ok[V];
    long long off[V];
    f32x4 acc[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int c = c0 + (v * 64 + lane) * 4;
      ok[v] = c < d;
      off[v] = c;
      acc[v] = ok[v] ? *(const f32x4*)(dx_gate + (long long)t * d + c) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    if (dx_shared) {
#pragma unroll
      for (int v = 0; v < V; ++v)
        if (ok[v]) {
          const f32x4 x = *(const f32x4*)(dx_shared + (long long)t * d + off[v]);
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[v][q] += x[q];
        }
    }
    for (int s = 0; s < k2; ++s) {  // the two-level secondary gates' rows
      const long long pos = __builtin_amdgcn_readlane(my2, s);
#pragma unroll
      for (int v = 0; v < V; ++v)
        if (ok[v]) {
          const f32x4 x = *(const f32x4*)(du2 + pos * d + off[v]);
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[v][q] += x[q];
        }
    }
    for (int s = 0; s < k; ++s) {
      const int pos = __builtin_amdgcn_readlane(my, s);
      if (pos < 0) continue;
#pragma unroll
      for (int v = 0; v < V; ++v)
        if (ok[v]) {
          const f32x4 x = *(const f32x4*)(du_perm + (long long)pos * d + off[v]);
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[v][q] += x[q];
        }
    }
#pragma unroll
    for (int v = 0; v < V; ++v)
      if (ok[v]) *(f32x4*)(dx + (long long)t * d + off[v]) = acc[v];
  }
}

// Two-level layer, per token: the gradient of each combined slot's product
// weight w = w1_s * w2_{s,s2}, gw = dG + dImportance[expert] + c_ent (ln w + 1)
// (Importance and the entropy are taken over the products), becomes
// dG1[t,s] = sum over s2 of gw * w2 (in slot order) and dG2[t,s,s2] = gw * w1_s,
// with w2 = w / w1_s.  One thread per (token, primary slot).
__global__ __launch_bounds__(256) void hier_product_bwd_kernel(
    const int32_t* __restrict__ topk_idx, const float* __restrict__ topk_w,
    const float* __restrict__ prim_w, const float* __restrict__ dG,
    const float* __restrict__ dimp, const float* __restrict__ coef, int T, int k1, int k2,
    float* __restrict__ dG1, float* __restrict__ dG2) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long long)T * k1) return;
  const int k = k1 * k2;
  const long long t = i / k1;
  const int s = (int)(i % k1);
  const float c_ent = coef[1];
  const float w1 = prim_w[i];
  float acc = 0.f;
  for (int s2 = 0; s2 < k2; ++s2) {
    const long long j = t * k + (long long)s * k2 + s2;
    const float w = topk_w[j];
    float gw = dG[j] + dimp[topk_idx[j]];
    if (w > 0.f) gw += c_ent * (logf(w) + 1.f);
    acc = fmaf(gw, w / w1, acc);
    dG2[i * k2 + s2] = gw * w1;
  }
  dG1[i] = acc;
}

// Two-level factorised load Load_H[g*b+e] = Load_p[g] Load_g[e] / |X_g|:
// dLoad_p[g] = sum over e of dLoad_H * Load_g[e] / |X_g| (in e order),
// dLoad_g[g][e] = dLoad_H * Load_p[g] / |X_g|; zero for a group no token
// reaches.  One block per group.
__global__ __launch_bounds__(64) void hier_dload_kernel(const float* __restrict__ dload_h,
                                                        const float* __restrict__ load_p,
                                                        const float* __restrict__ load_g,
                                                        const int32_t* __restrict__ counts,
                                                        int b, float* __restrict__ dload_p,
                                                        float* __restrict__ dload_g) {
  const int g = blockIdx.x;
  const int cnt = counts[g];
  const float inv = cnt > 0 ? 1.f / (float)cnt : 0.f;
  float part = 0.f;
  for (int e = threadIdx.x; e < b; e += 64) {
    const float dh = dload_h[(long long)g * b + e];
    dload_g[(long long)g * b + e] = dh * load_p[g] * inv;
    part = fmaf(dh, load_g[(long long)g * b + e], part);
  }
  const float tot = wave_sum_dpp(part);
  if (threadIdx.x == 0) dload_p[g] = tot * inv;
}

// hid = bf16(silu(a) * b) with the forward epilogue's expression.
__global__ __launch_bounds__(256) void swiglu_hidden_kernel(const float* __restrict__ a,
                                                            const float* __restrict__ b,
                                                            long long n4,
                                                            uint16_t* __restrict__ hid) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  const f32x4 av = *(const f32x4*)(a + 4 * i), bv = *(const f32x4*)(b + 4 * i);
  float f[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) f[q] = av[q] / (1.f + expf(-av[q])) * bv[q];
  *(uint2*)(hid + 4 * i) = make_uint2(bf16x2_bits(f[0], f[1]), bf16x2_bits(f[2], f[3]));
}

}  // namespace

hipError_t launch_combine_bwd(const float* dy, const float* y_perm, const int32_t* slot_pos,
                              const float* topk_w, int T, int k, int d, float* dG, void* dout,
                              int dout_f32, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  ProfScope ps("bwd_combine", s);
  const dim3 grid((T + 3) / 4);
  if (dout_f32)
    combine_bwd_kernel<true><<<grid, dim3(256), 0, s>>>(dy, y_perm, slot_pos, topk_w, T, k, d,
                                                        dG, dout);
  else
    combine_bwd_kernel<false><<<grid, dim3(256), 0, s>>>(dy, y_perm, slot_pos, topk_w, T, k, d,
                                                         dG, dout);
  return hipGetLastError();
}

hipError_t launch_loss_grad(const float* importance, const float* load,
                            const int32_t* counts_pre, const float* dlosses, int T, int k, int n,
                            float w_imp, float w_load, float alpha, float w_z, float w_ent,
                            float* dimp, float* dload, float* coef, hipStream_t s) {
  ProfScope ps("bwd_loss_grad", s);
  loss_grad_kernel<<<dim3(1), dim3(256), 0, s>>>(importance, load, counts_pre, dlosses, T, k, n,
                                                 w_imp, w_load, alpha, w_z, w_ent, dimp, dload,
                                                 coef);
  return hipGetLastError();
}

int gate_wgrad_splits(int T, int d, int M) {
  const int tiles = ((d + kGwTile - 1) / kGwTile) * ((M + kGwTile - 1) / kGwTile);
  int splits = (256 + tiles - 1) / tiles;        // about one tile per CU
  const int max_splits = (T + 255) / 256;        // at least 256 tokens per split
  if (splits > max_splits) splits = max_splits;
  return splits < 1 ? 1 : splits;
}

hipError_t launch_gate_wgrad(const GateWgradArgs& a, float* dw_gate, float* dw_noise,
                             hipStream_t s) {
  // No tokens: every tile has no K-steps and stores zeros.
  const int tiles = ((a.d + kGwTile - 1) / kGwTile) * ((a.M + kGwTile - 1) / kGwTile);
  const long long total = (long long)a.splits * tiles;
  {
    ProfScope ps("bwd_gate_wgrad", s);
    gate_wgrad_kernel<<<dim3((unsigned)((total + kXcds - 1) / kXcds * kXcds)), dim3(256), 0, s>>>(
        a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const long long n4 = (long long)a.M * a.d / 4;
  ProfScope ps("bwd_gate_wgrad_reduce", s);
  wgrad_reduce_kernel<<<dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s>>>(
      a.partial, a.splits, a.M, a.n, a.d, dw_gate, dw_noise);
  return hipGetLastError();
}

hipError_t launch_transpose_gate(const float* w_gate, const float* w_noise, int n, int d,
                                 int ldk, float* wt, hipStream_t s) {
  ProfScope ps("bwd_transpose_gate", s);
  transpose_gate_kernel<<<dim3((ldk + 31) / 32, (d + 31) / 32), dim3(256), 0, s>>>(
      w_gate, w_noise, n, d, ldk, wt);
  return hipGetLastError();
}

hipError_t launch_seg_colsum(const void* src, int src_f32, long long ld, const int32_t* offsets,
                             int n_seg, int N, float* out, hipStream_t s) {
  if (n_seg <= 0 || N <= 0) return hipSuccess;
  ProfScope ps("bwd_bias_colsum", s);
  const dim3 grid((N + 255) / 256, n_seg);
  if (src_f32)
    seg_colsum_kernel<true><<<grid, dim3(256), 0, s>>>(src, ld, offsets, N, out);
  else
    seg_colsum_kernel<false><<<grid, dim3(256), 0, s>>>(src, ld, offsets, N, out);
  return hipGetLastError();
}

hipError_t launch_dx_gather(const float* dx_gate, const float* dx_shared, const float* du_perm,
                            const int32_t* slot_pos, int T, int k, int d, const float* du2,
                            const int32_t* slot2, int k2, float* dx, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  ProfScope ps("bwd_dx_gather", s);
  dx_gather_kernel<<<dim3((T + 3) / 4), dim3(256), 0, s>>>(dx_gate, dx_shared, du_perm, slot_pos,
                                                           T, k, d, du2, slot2, du2 ? k2 : 0, dx);
  return hipGetLastError();
}

hipError_t launch_hier_product_bwd(const int32_t* topk_idx, const float* topk_w,
                                   const float* prim_w, const float* dG, const float* dimp,
                                   const float* coef, int T, int k1, int k2, float* dG1,
                                   float* dG2, hipStream_t s) {
  const long long rows = (long long)T * k1;
  if (rows <= 0) return hipSuccess;
  ProfScope ps("bwd_hier_product", s);
  hier_product_bwd_kernel<<<dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, s>>>(
      topk_idx, topk_w, prim_w, dG, dimp, coef, T, k1, k2, dG1, dG2);
  return hipGetLastError();
}

hipError_t launch_hier_dload(const float* dload_h, const float* load_p, const float* load_g,
                             const int32_t* counts, int a, int b, float* dload_p,
                             float* dload_g, hipStream_t s) {
  if (a <= 0) return hipSuccess;
  ProfScope ps("bwd_hier_dload", s);
  hier_dload_kernel<<<dim3(a), dim3(64), 0, s>>>(dload_h, load_p, load_g, counts, b, dload_p,
                                                 dload_g);
  return hipGetLastError();
}

hipError_t launch_swiglu_hidden(const float* a, const float* b, long long elems, uint16_t* hid,
                                hipStream_t s) {
  const long long n4 = elems / 4;
  if (n4 <= 0) return hipSuccess;
  ProfScope ps("bwd_swiglu_hidden", s);
  swiglu_hidden_kernel<<<dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s>>>(a, b, n4, hid);
  return hipGetLastError();
}

}  // namespace moe
