// Gating network epilogue on gfx950: one wavefront per token row, 16 (large
// n: 8) wavefronts per block, each prefetching its next row while it works on
// the current one, so every row of a block is in flight at once for the usual
// row counts.
//
// Reads the fp32 logits written by the gate GEMM (the sum of its K-split
// partials, added in split order and written back for the backward) and
// computes, per row,
//   H_j = clean_j (+ bias_j) + z_j * Softplus(raw_j)      (noisy gate)
// then KeepTopK by k+1 rounds of a wave-wide arg-max (DPP max of the ordered
// float keys, then a ballot for the lowest index holding the maximum: larger
// H first, lower index first on equal H), the softmax over the kept values
// (or the Switch full softmax, or the sigmoid gate's renormalised
// affinities), and the per-expert sums behind the auxiliary losses:
//   Importance_j += G_j,  Load_j += Phi((clean_j - thr_j) / Softplus(raw_j)),
// thr_j = H_(k+1) if j is kept, H_(k) otherwise; per block also the sum of
// the squared pre-softmax logits (router z-loss) and of the gate
// distributions' entropies.
// Definitions: arXiv 1701.06538 summary (xyznot.com), "Method and key
// formulas": Noisy Top-K gating and the load-balancing losses; Switch router:
// MoE survey (tufusi.com) section 3.1; sigmoid gate with a selection-only
// bias: same survey, sections 6.2 and 6.3; z-loss and gate entropy: wkbse.com
// MoE introduction, part 2.
//
// Sums are deterministic: each lane owns fixed experts (j = lane + 64q) and
// accumulates its rows in order; waves are combined in LDS in a fixed order;
// blocks write partial vectors that a second kernel adds in block order.
#include <math.h>

#include "colsum.h"
#include "common.h"
#include "launch.h"

namespace moe {
namespace {

// Softplus(z) = max(z, 0) + log1p(e), e = exp(-|z|) in (0, 1].  e comes
// from the hardware exp2 and log1p(e) from Goldberg's correction: with
// u = 1 + e rounded, log1p(e) = log(u) * e / (u - 1), within a few ulps when
// log is (D. Goldberg, "What every computer scientist should know about
// floating-point arithmetic", 1991, Theorem 4), and e itself when u rounds
// to 1.  About a tenth of the instructions of log1pf(expf(.)).
// v_exp_f32 / v_log_f32 / v_rcp_f32 (base-2 exponential and logarithm and
// the reciprocal, each within about 1 ulp).
__device__ __forceinline__ float hw_exp(float x) {
  return __builtin_amdgcn_exp2f(x * 1.44269504088896341f);
}
__device__ __forceinline__ float hw_log(float x) {
  return __builtin_amdgcn_logf(x) * 0.693147180559945309f;
}
__device__ __forceinline__ float hw_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

__device__ __forceinline__ float softplus_f(float z) {
  const float e = hw_exp(-fabsf(z));
  const float u = 1.f + e;
  const float l = u == 1.f ? e : hw_log(u) * (e * hw_rcp(u - 1.f));
  return fmaxf(z, 0.f) + l;
}

// Phi(z) = erfc(-z / sqrt 2) / 2, branch-free.  erfc(y) for y >= 0 is the
// Chebyshev-fitted form t exp(-y^2 + P(t)), t = 1 / (1 + y/2), of Press,
// Teukolsky, Vetterling and Flannery, "Numerical Recipes" (2nd ed., section
// 6.2, erfcc), fractional error below 1.2e-7; then Phi(z) = erfc(y)/2 for
// z < 0 and 1 - erfc(y)/2 for z >= 0, y = |z| / sqrt 2.  Evaluated in fp32
// with the hardware exp2 and reciprocal: within 2.2e-7 of Phi absolutely
// (checked against a double-precision normal CDF over [-12, 12]).
__device__ __forceinline__ float std_normal_cdf(float z) {
  const float y = fabsf(z) * 0.70710678118654752f;
  const float t = hw_rcp(fmaf(0.5f, y, 1.f));
  float p = 0.17087277f;
  p = fmaf(p, t, -0.82215223f);
  p = fmaf(p, t, 1.48851587f);
  p = fmaf(p, t, -1.13520398f);
  p = fmaf(p, t, 0.27886807f);
  p = fmaf(p, t, -0.18628806f);
  p = fmaf(p, t, 0.09678418f);
  p = fmaf(p, t, 0.37409196f);
  p = fmaf(p, t, 1.00002368f);
  p = fmaf(p, t, -1.26551223f);
  const float e = t * hw_exp(fmaf(-y, y, p));  // erfc(y)
  return z >= 0.f ? fmaf(-0.5f, e, 1.f) : 0.5f * e;
}

__device__ __forceinline__ int readlane_i(int v, int l) { return __builtin_amdgcn_readlane(v, l); }
__device__ __forceinline__ float readlane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// Per-row inputs of one wavefront: lane owns experts j = lane + 64 q.
template <int NPL>
struct RowIn {
  float c[NPL];  // clean logit (+ bias)
  float r[NPL];  // raw noise logit (noisy gate only)
  float z[NPL];  // standard normal draw (noisy gate only)
};

template <int NPL, int NW>
__global__ __launch_bounds__(NW * 64) void topk_kernel(const TopkArgs p) {
  extern __shared__ float red[];  // [NW][n]
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

  // Where row r's noise and outputs live.
  auto locate = [&](int r, long long& noise_row, long long& out_base, float& wprim) {
    if (grouped) {
      const int t = p.row_token[r];
      int s = 0;
      for (int q = 0; q < p.k1; ++q)
        if (p.prim_idx[(long long)t * p.k1 + q] == g) s = q;
      noise_row = ((long long)t * p.k1 + s) * n;
      out_base = (long long)t * p.k1 * k + (long long)s * k;
      wprim = p.prim_w[(long long)t * p.k1 + s];
    } else {
      noise_row = (long long)r * n;
      out_base = (long long)r * k;
      wprim = 1.f;
    }
  };
  auto fetch = [&](int r, RowIn<NPL>& in) {
    long long nrow, ob;
    float wp;
    locate(r, nrow, ob, wp);
    float* lg = p.logits + (long long)r * p.ldl;
    // Lanes past n load entry 0 (every load stays unconditional, so a row's
    // loads are all in flight together) and keep 0.
    int jc[NPL];
#pragma unroll
    for (int q = 0; q < NPL; ++q) jc[q] = lane + 64 * q < n ? lane + 64 * q : 0;
#pragma unroll
    for (int q = 0; q < NPL; ++q) {
      const bool ok = lane + 64 * q < n;
      const float c = lg[jc[q]];
      in.c[q] = ok ? c : 0.f;
      in.r[q] = 0.f;
      in.z[q] = 0.f;
    }
    if (p.noisy) {
#pragma unroll
      for (int q = 0; q < NPL; ++q) {
        const bool ok = lane + 64 * q < n;
        const float rv = lg[n + jc[q]];
        const float zv = p.noise[nrow + jc[q]];
        in.r[q] = ok ? rv : 0.f;
        in.z[q] = ok ? zv : 0.f;
      }
    }
    if (p.nsplit > 1) {  // the gate GEMM's K-split partials, added in split order
      for (int sp = 1; sp < p.nsplit; ++sp) {
        const float* part = lg + sp * p.split_stride;
        float pc[NPL], pr[NPL];
#pragma unroll
        for (int q = 0; q < NPL; ++q) pc[q] = part[jc[q]];
        if (p.noisy) {
#pragma unroll
          for (int q = 0; q < NPL; ++q) pr[q] = part[n + jc[q]];
#pragma unroll
          for (int q = 0; q < NPL; ++q) in.r[q] += pr[q];
        }
#pragma unroll
        for (int q = 0; q < NPL; ++q) in.c[q] += pc[q];
      }
#pragma unroll
      for (int q = 0; q < NPL; ++q) {
        const int j = lane + 64 * q;
        if (j < n) {
          lg[j] = in.c[q];
          if (p.noisy) lg[n + j] = in.r[q];
        }
      }
    }
  };

  float zacc = 0.f, eacc = 0.f;  // this wave's z-loss and entropy sums
  float imp[NPL], ld[NPL], bias[NPL];
#pragma unroll
  for (int q = 0; q < NPL; ++q) {
    imp[q] = ld[q] = 0.f;
    const int j = lane + 64 * q;
    bias[q] = (p.bias && j < n) ? p.bias[j] : 0.f;
  }

  const int R = min(k + 1, n);
  RowIn<NPL> cur, nxt;
  int r = row_begin + wave;
  if (r < row_end) fetch(r, cur);
  for (; r < row_end; r += NW) {
    if (r + NW < row_end) fetch(r + NW, nxt);  // next row in flight
    long long noise_row, out_base;
    float wprim;
    locate(r, noise_row, out_base, wprim);

    float cl[NPL], sp[NPL], hv[NPL];
    uint32_t key[NPL];
#pragma unroll
    for (int q = 0; q < NPL; ++q) {
      const int j = lane + 64 * q;
      const bool ok = j < n;
      cl[q] = cur.c[q] + bias[q];
      sp[q] = 1.f;
      hv[q] = cl[q];
      if (p.noisy) {
        sp[q] = softplus_f(cur.r[q]);
        hv[q] = cl[q] + cur.z[q] * sp[q];
      }
      key[q] = ok ? ordered_key(hv[q]) : 0u;
    }
    // Router z-loss statistic: the logits the softmax sees (the sigmoid
    // gate's are the bias-free network logits).
    {
      float zl = 0.f;
#pragma unroll
      for (int q = 0; q < NPL; ++q) {
        const float v = p.sigmoid_mode ? cur.c[q] : hv[q];
        if (lane + 64 * q < n) zl = fmaf(v, v, zl);
      }
      zacc += wave_sum_dpp(zl);
    }

    // k+1 rounds of arg-max: the largest key wins; among equal keys the
    // lowest index (lowest q, then lowest lane) wins.
    uint32_t selmask = 0;
    int my_j = 0;
    float my_v = 0.f, v0 = 0.f, v_km1 = 0.f, v_k = -INFINITY;
    for (int rd = 0; rd < R; ++rd) {
      uint32_t best = 0;
#pragma unroll
      for (int q = 0; q < NPL; ++q) best = max(best, key[q]);
      const uint32_t m = wave_max_u32(best);
      int j = 0;
#pragma unroll
      for (int q = 0; q < NPL; ++q) {
        const unsigned long long b = __ballot(key[q] == m);
        if (b) {
          j = 64 * q + __builtin_ctzll(b);
          break;
        }
      }
      const float v = key_to_float(m);
      if (lane == (j & 63)) {
#pragma unroll
        for (int q = 0; q < NPL; ++q)
          if (q == (j >> 6)) {
            key[q] = 0u;
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
    float w, zsum;
    if (p.switch_mode) {
      float ls = 0.f;
#pragma unroll
      for (int q = 0; q < NPL; ++q)
        if (lane + 64 * q < n) ls += expf(hv[q] - v0);
      zsum = wave_sum_dpp(ls);
      w = (lane < k) ? expf(my_v - v0) / zsum : 0.f;
    } else if (p.sigmoid_mode) {
      // s = Sigmoid(h) of the kept expert's bias-free logit, fetched from the
      // lane that owns it; weights s / sum of the kept s.
      float hsel = 0.f;
#pragma unroll
      for (int q = 0; q < NPL; ++q) {
        const float t = __shfl(cur.c[q], my_j & 63, kWave);
        if (q == (my_j >> 6)) hsel = t;
      }
      const float sg = (lane < k) ? hw_rcp(1.f + hw_exp(-hsel)) : 0.f;
      zsum = wave_sum_dpp(sg);
      w = sg * hw_rcp(zsum);
    } else {
      const float e = (lane < k) ? expf(my_v - v0) : 0.f;
      zsum = wave_sum_dpp(e);
      w = e / zsum;
    }
    if (lane < k) {
      p.topk_idx[out_base + lane] = (grouped ? g * n : 0) + my_j;
      p.topk_w[out_base + lane] = wprim * w;
    }

    // Importance: the dense gate vector (Switch: the full softmax).  Entropy
    // of the gate distribution: Switch -sum p ln p = ln Z - sum p (H - H_max);
    // otherwise over the kept weights (times the primary weight in the
    // two-level secondary gate, which makes the rows of a token add up to the
    // entropy of the product distribution).
    if (p.switch_mode) {
      float pe = 0.f;
#pragma unroll
      for (int q = 0; q < NPL; ++q)
        if (lane + 64 * q < n) {
          const float dl = hv[q] - v0;
          const float pj = expf(dl) / zsum;
          imp[q] += pj;
          pe = fmaf(pj, dl, pe);
        }
      eacc += hw_log(zsum) - wave_sum_dpp(pe);
    } else {
      const float W = wprim * w;
      eacc += wave_sum_dpp((lane < k && W > 0.f) ? -W * hw_log(W) : 0.f);
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
          const float zz = (cl[q] - thr) * hw_rcp(sp[q]);
          ld[q] += std_normal_cdf(zz);
        }
      }
    }
    cur = nxt;
  }

  // Combine the waves in a fixed order, then write this block's partials.
  if (p.part_stats) {
    __shared__ float st[2][NW];
    if (lane == 0) {
      st[0][wave] = zacc;
      st[1][wave] = eacc;
    }
    __syncthreads();
    if (threadIdx.x < 2) {
      float a = 0.f;
      for (int w2 = 0; w2 < NW; ++w2) a += st[threadIdx.x][w2];
      p.part_stats[(long long)part * 2 + threadIdx.x] = a;
    }
  }
  for (int pass = 0; pass < 2; ++pass) {
    float* out = pass == 0 ? p.part_imp : p.part_load;
    if (!out) break;
#pragma unroll
    for (int q = 0; q < NPL; ++q) {
      const int j = lane + 64 * q;
      if (j < n) red[wave * n + j] = pass == 0 ? imp[q] : ld[q];
    }
    __syncthreads();
    for (int j = threadIdx.x; j < n; j += NW * 64) {
      float sacc = red[j];
      for (int w2 = 1; w2 < NW; ++w2) sacc += red[w2 * n + j];
      out[(long long)part * n + j] = sacc;
    }
    __syncthreads();
  }
}

// Backward of the flat gate for one token row per wavefront, the selection
// (topk_idx) held fixed.  The chain, per row (arXiv 1701.06538 summary,
// xyznot.com, FAQ on back-propagating through the top-k: the kept values
// stay differentiable; reading notes, chenshi221.pages.dev, "Noisy Top-K
// Gating": the noise lets the load loss pass gradients):
//  1. gradient on the gate distribution: dG from the combine on the kept
//     slots, dImportance, and c_ent (ln g + 1) from the entropy statistic;
//  2. through the normalisation: softmax over the kept values, softmax over
//     all n (Switch), or Sigmoid divided by the kept sum;
//  3. + 2 c_z Z_j from the z statistic (Z = H; the sigmoid gate: h);
//  4. the smooth load P_j = Phi((clean_j - thr_j) / sp_j): into clean_j,
//     sp_j and the threshold, which is the H of the rank-k expert (kept j)
//     or of the rank k-1 expert (other j);
//  5. H = clean + z sp: d raw = (d sp + z dH) Sigmoid(raw).
// H, sp and the thresholds are recomputed with the forward's arithmetic.
// Writes dlogits[r][j] = dL/d clean_j (sigmoid gate: dL/d h_j) and, for a
// noisy gate, dlogits[r][n + j] = dL/d raw_j, zeros in the rest of the row;
// per block, the column sums of the clean part in row order (for the logit
// bias).
template <int NPL, int NW>
__global__ __launch_bounds__(NW * 64) void gate_bwd_kernel(const GateBwdArgs p) {
  extern __shared__ float red[];  // [NW][n]
  const int n = p.n, k = p.k;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int part = blockIdx.x;
  const bool grouped = p.tile_expert != nullptr;
  int row_begin, row_end, g = 0;
  if (grouped) {
    if (part >= *p.tile_count) return;
    g = p.tile_expert[part];
    row_begin = p.tile_row0[part];
    row_end = min(row_begin + p.tile_rows, p.offsets[g + 1]);
  } else {
    row_begin = part * p.rows_per_block;
    row_end = min(row_begin + p.rows_per_block, p.T);
  }
  const float c_z = p.coef[0], c_ent = p.coef[1];
  const float* dload_v = (p.noisy && p.dload) ? p.dload + (long long)g * n : nullptr;

  float bias[NPL], dimp[NPL], dload[NPL], dbacc[NPL];
#pragma unroll
  for (int q = 0; q < NPL; ++q) {
    const int j = lane + 64 * q;
    const bool ok = j < n;
    bias[q] = (p.bias && ok) ? p.bias[j] : 0.f;
    dimp[q] = (p.dimp && ok) ? p.dimp[j] : 0.f;
    dload[q] = (dload_v && ok) ? dload_v[j] : 0.f;
    dbacc[q] = 0.f;
  }

  for (int r = row_begin + wave; r < row_end; r += NW) {
    // Where row r's noise, slots and slot gradients live: flat, token r;
    // grouped, the (token, primary slot) pair dispatched to row r, whose
    // secondary slots are the combined slots s*k .. s*k+k-1 of the token.
    long long noise_row, slot_base, dg_base;
    int id_off = 0;
    if (grouped) {
      const int t = p.row_token[r];
      int sl = 0;
      for (int q = 0; q < p.k1; ++q)
        if (p.prim_idx[(long long)t * p.k1 + q] == g) sl = q;
      noise_row = ((long long)t * p.k1 + sl) * n;
      slot_base = (long long)t * p.k1 * k + (long long)sl * k;
      dg_base = ((long long)t * p.k1 + sl) * k;
      id_off = g * n;
    } else {
      noise_row = (long long)r * n;
      slot_base = dg_base = (long long)r * k;
    }
    const float* lg = p.logits + (long long)r * p.ldl;
    float c[NPL], cl[NPL], sp[NPL], hv[NPL], rw[NPL], zn[NPL];
#pragma unroll
    for (int q = 0; q < NPL; ++q) {
      const int j = lane + 64 * q;
      const bool ok = j < n;
      c[q] = ok ? lg[j] : 0.f;
      rw[q] = (ok && p.noisy) ? lg[n + j] : 0.f;
      zn[q] = (ok && p.noisy) ? p.noise[noise_row + j] : 0.f;
      cl[q] = c[q] + bias[q];
      sp[q] = 1.f;
      hv[q] = cl[q];
      if (p.noisy) {
        sp[q] = softplus_f(rw[q]);
        hv[q] = cl[q] + zn[q] * sp[q];
      }
    }
    // Slots: lane s < k holds slot s.
    const int my_j = lane < k ? p.topk_idx[slot_base + lane] - id_off : 0;
    const float my_dg = lane < k ? p.dG[dg_base + lane] : 0.f;
    uint32_t kept = 0;
    for (int s = 0; s < k; ++s) {
      const int js = readlane_i(my_j, s);
      if (lane == (js & 63)) kept |= 1u << (js >> 6);
    }
    // H of the expert in slot s (fetched from the lane that owns it).
    auto h_of = [&](int js) {
      float v = 0.f;
#pragma unroll
      for (int q = 0; q < NPL; ++q) {
        const float t = __shfl(hv[q], js & 63, kWave);
        if (q == (js >> 6)) v = t;
      }
      return v;
    };
    // The slot's gate weight: the forward's (flat), or the secondary
    // softmax over the kept values recomputed with the forward's arithmetic
    // (grouped: the stored weight is the product with the primary weight).
    float my_w;
    if (grouped) {
      const float v0 = h_of(readlane_i(my_j, 0));
      const float hj = h_of(my_j);
      const float e = lane < k ? expf(hj - v0) : 0.f;
      my_w = e / wave_sum_dpp(e);
    } else {
      my_w = lane < k ? p.topk_w[slot_base + lane] : 0.f;
    }

    float dH[NPL];
#pragma unroll
    for (int q = 0; q < NPL; ++q) dH[q] = 0.f;
    if (p.switch_mode) {
      const int j0 = readlane_i(my_j, 0);
      const float v0 = h_of(j0);
      float ls = 0.f;
#pragma unroll
      for (int q = 0; q < NPL; ++q)
        if (lane + 64 * q < n) ls += expf(hv[q] - v0);
      const float Z = wave_sum_dpp(ls);
      const float lnZ = hw_log(Z);
      const float dg0 = readlane_f(my_dg, 0);
      float pr[NPL], gp[NPL], dotl = 0.f;
#pragma unroll
      for (int q = 0; q < NPL; ++q) {
        const int j = lane + 64 * q;
        pr[q] = 0.f;
        gp[q] = 0.f;
        if (j < n) {
          pr[q] = expf(hv[q] - v0) / Z;
          gp[q] = dimp[q] + (pr[q] > 0.f ? c_ent * ((hv[q] - v0) - lnZ + 1.f) : 0.f) +
                  (j == j0 ? dg0 : 0.f);
          dotl = fmaf(pr[q], gp[q], dotl);
        }
      }
      const float dot = wave_sum_dpp(dotl);
#pragma unroll
      for (int q = 0; q < NPL; ++q) dH[q] = pr[q] * (gp[q] - dot);
    } else {
      float gg = 0.f;
      if (lane < k) {
        gg = my_dg + (p.dimp ? p.dimp[my_j] : 0.f);
        if (my_w > 0.f) gg += c_ent * (hw_log(my_w) + 1.f);
      }
      const float dot = wave_sum_dpp(lane < k ? my_w * gg : 0.f);
      float dz;
      if (p.sigmoid_mode) {
        float hsel = 0.f;
#pragma unroll
        for (int q = 0; q < NPL; ++q) {
          const float t = __shfl(c[q], my_j & 63, kWave);
          if (q == (my_j >> 6)) hsel = t;
        }
        const float sg = lane < k ? hw_rcp(1.f + hw_exp(-hsel)) : 0.f;
        const float S = wave_sum_dpp(sg);
        dz = lane < k ? sg * (1.f - sg) / S * (gg - dot) : 0.f;
      } else {
        dz = lane < k ? my_w * (gg - dot) : 0.f;
      }
      for (int s = 0; s < k; ++s) {
        const int js = readlane_i(my_j, s);
        const float v = readlane_f(dz, s);
        if (lane == (js & 63)) {
#pragma unroll
          for (int q = 0; q < NPL; ++q)
            if (q == (js >> 6)) dH[q] += v;
        }
      }
    }
    // z statistic
#pragma unroll
    for (int q = 0; q < NPL; ++q)
      if (lane + 64 * q < n) dH[q] = fmaf(2.f * c_z, p.sigmoid_mode ? c[q] : hv[q], dH[q]);

    float dcl[NPL], dsp[NPL];
#pragma unroll
    for (int q = 0; q < NPL; ++q) dcl[q] = dsp[q] = 0.f;
    if (p.noisy) {
      // The rank-k expert: the largest H outside the kept set, lowest index
      // first on equal H (as in the forward's selection).
      uint32_t key[NPL], best = 0;
#pragma unroll
      for (int q = 0; q < NPL; ++q) {
        const bool ok = lane + 64 * q < n && !((kept >> q) & 1u);
        key[q] = ok ? ordered_key(hv[q]) : 0u;
        best = max(best, key[q]);
      }
      const uint32_t m = wave_max_u32(best);
      int jk = -1;
      if (m != 0u) {
#pragma unroll
        for (int q = 0; q < NPL; ++q) {
          const unsigned long long b = __ballot(key[q] == m);
          if (b) {
            jk = 64 * q + __builtin_ctzll(b);
            break;
          }
        }
      }
      const float v_k = jk >= 0 ? key_to_float(m) : -INFINITY;
      const int jkm1 = readlane_i(my_j, k - 1);
      const float v_km1 = h_of(jkm1);
      float sk = 0.f, sn = 0.f;
#pragma unroll
      for (int q = 0; q < NPL; ++q) {
        if (lane + 64 * q < n) {
          const bool kq = (kept >> q) & 1u;
          const float thr = kq ? v_k : v_km1;
          if (thr != -INFINITY) {
            const float rs = hw_rcp(sp[q]);
            const float zz = (cl[q] - thr) * rs;
            const float g = dload[q] * (expf(-0.5f * zz * zz) * 0.398942280401432678f) * rs;
            dcl[q] = g;
            dsp[q] = -g * zz;
            if (kq) sk += g; else sn += g;
          }
        }
      }
      const float SK = wave_sum_dpp(sk), SN = wave_sum_dpp(sn);
      if (jk >= 0 && lane == (jk & 63)) {
#pragma unroll
        for (int q = 0; q < NPL; ++q)
          if (q == (jk >> 6)) dH[q] -= SK;
      }
      if (lane == (jkm1 & 63)) {
#pragma unroll
        for (int q = 0; q < NPL; ++q)
          if (q == (jkm1 >> 6)) dH[q] -= SN;
      }
    }

    float* out = p.dlogits + (long long)r * p.ldd;
#pragma unroll
    for (int q = 0; q < NPL; ++q) {
      const int j = lane + 64 * q;
      if (j < n) {
        const float dc = dH[q] + dcl[q];
        out[j] = dc;
        dbacc[q] += dc;
        if (p.noisy) out[n + j] = (dsp[q] + zn[q] * dH[q]) * hw_rcp(1.f + hw_exp(-rw[q]));
      }
    }
    // Columns past the written ones are zero: products over the padded row
    // width then add nothing.
    for (int j = (p.noisy ? 2 * n : n) + lane; j < p.ldd; j += 64) out[j] = 0.f;
  }

  if (p.part_db) {
#pragma unroll
    for (int q = 0; q < NPL; ++q) {
      const int j = lane + 64 * q;
      if (j < n) red[wave * n + j] = dbacc[q];
    }
    __syncthreads();
    for (int j = threadIdx.x; j < n; j += NW * 64) {
      float sacc = red[j];
      for (int w2 = 1; w2 < NW; ++w2) sacc += red[w2 * n + j];
      p.part_db[(long long)part * n + j] = sacc;
    }
  }
}

// The gate's column sums in their own launch; blockIdx.y selects the vector.
__global__ __launch_bounds__(kColThreads) void colsum_kernel(const ColsumArgs a, int nparts) {
  colsum_block(a, nparts, (int)blockIdx.x, (int)blockIdx.y);
}

// One block: the secondary tiles' statistics in tile order, plus the
// primary gate's z statistic.
__global__ __launch_bounds__(256) void hier_stats_kernel(const float* __restrict__ prim,
                                                         const float* __restrict__ part,
                                                         const int32_t* __restrict__ tile_count,
                                                         float* __restrict__ out) {
  __shared__ double sh[4];
  const int nt = *tile_count;
  double z = 0.0, e = 0.0;
  for (int t = threadIdx.x; t < nt; t += 256) {
    z += (double)part[2 * t];
    e += (double)part[2 * t + 1];
  }
  z = block_sum<256>(z, sh);
  e = block_sum<256>(e, sh);
  if (threadIdx.x == 0) {
    out[0] = (float)((double)prim[0] + z);
    out[1] = (float)e;
  }
}

// One thread per (group g, expert e): sum the tiles of group g in order.
__global__ void hier_finalize_kernel(const float* __restrict__ part_imp,
                                     const float* __restrict__ part_load,
                                     const int32_t* __restrict__ tile_expert,
                                     const int32_t* __restrict__ tile_count,
                                     const int32_t* __restrict__ group_counts,
                                     const float* __restrict__ load_primary, int a, int b,
                                     float* __restrict__ importance, float* __restrict__ load,
                                     float* __restrict__ load_g) {
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
  if (load_g) load_g[id] = (float)sl;
  if (load) {
    const int cnt = group_counts[g];
    load[id] = cnt > 0 ? (float)((double)load_primary[g] * sl / (double)cnt) : 0.f;
  }
}

template <int NPL>
hipError_t launch_topk_t(const TopkArgs& a, int grid, hipStream_t s) {
  constexpr int NW = NPL <= 8 ? 16 : 8;  // the same rule as topk_waves()
  const size_t shm = (size_t)NW * a.n * sizeof(float);
  ProfScope ps(a.tile_expert ? "gate_topk_grouped" : "gate_topk", s);
  topk_kernel<NPL, NW><<<dim3(grid), dim3(NW * 64), shm, s>>>(a);
  return hipGetLastError();
}

template <int NPL>
hipError_t launch_gate_bwd_t(const GateBwdArgs& a, int grid, hipStream_t s) {
  // Fewer rows in flight than the forward (more live values per row); every
  // choice divides the forward's rows-per-block.
  constexpr int NW = NPL <= 4 ? 16 : NPL <= 16 ? 8 : 4;
  const size_t shm = (size_t)NW * a.n * sizeof(float);
  ProfScope ps("bwd_gate", s);
  gate_bwd_kernel<NPL, NW><<<dim3(grid), dim3(NW * 64), shm, s>>>(a);
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

hipError_t launch_gate_bwd(const GateBwdArgs& a, hipStream_t s) {
  const int grid = a.tile_expert ? a.max_tiles : (a.T + a.rows_per_block - 1) / a.rows_per_block;
  if (grid <= 0) return hipSuccess;
  const int npl = (a.n + 63) / 64;
  if (npl <= 1) return launch_gate_bwd_t<1>(a, grid, s);
  if (npl <= 2) return launch_gate_bwd_t<2>(a, grid, s);
  if (npl <= 4) return launch_gate_bwd_t<4>(a, grid, s);
  if (npl <= 8) return launch_gate_bwd_t<8>(a, grid, s);
  if (npl <= 16) return launch_gate_bwd_t<16>(a, grid, s);
  return launch_gate_bwd_t<32>(a, grid, s);
}

hipError_t launch_colsum(int nparts, ColsumVec v0, ColsumVec v1, ColsumVec v2, hipStream_t s) {
  const ColsumVec v[3] = {v0, v1, v2};
  ColsumArgs a;
  int nmax;
  const int nv = colsum_pack(v, a, nmax);
  if (nv == 0) return hipSuccess;
  ProfScope ps("gate_colsum", s);
  colsum_kernel<<<dim3((nmax + 63) / 64, nv), dim3(kColThreads), 0, s>>>(a, nparts);
  return hipGetLastError();
}

hipError_t launch_hier_stats(const float* prim, const float* part, const int32_t* tile_count,
                             float* out, hipStream_t s) {
  ProfScope ps("hier_stats", s);
  hier_stats_kernel<<<dim3(1), dim3(256), 0, s>>>(prim, part, tile_count, out);
  return hipGetLastError();
}

hipError_t launch_hier_finalize(const float* part_imp, const float* part_load,
                                const int32_t* tile_expert, const int32_t* tile_count,
                                const int32_t* group_counts, const float* load_primary, int a,
                                int b, float* importance, float* load, float* load_g,
                                hipStream_t s) {
  const int total = a * b;
  if (total <= 0) return hipSuccess;
  ProfScope ps("hier_finalize", s);
  hier_finalize_kernel<<<dim3((total + 255) / 256), dim3(256), 0, s>>>(
      part_imp, part_load, tile_expert, tile_count, group_counts, load_primary, a, b,
      importance, load, load_g);
  return hipGetLastError();
}

}  // namespace moe
