// The expert backward's GEMMs for fp32 experts (v_mfma_f32_32x32x2_f32).
//
// The same products and modes as the bf16 kernels (ggemm_bwd.hip), at fp32:
// C[c][m] = sum_k A[k][m] * B(k, c), A K-major, B row-major by merged row
// (ROWS) or K-major (WGRAD).  The fp32 matrix instruction takes one element
// of each operand per lane (lane l: row or column l % 32 at k = l / 32), so a
// K-major tile needs no transposition: lanes 0-31 read 32 consecutive
// columns of one K row.  The row-major B tile of ROWS mode is stored with a
// padded row (BK + 1 floats), so the 32 rows one read touches fall in
// different banks.
// 64 x 64 output tiles on 4 waves (32 x 32 each), K steps of 16 staged
// through registers into a double-buffered LDS tile.  Epilogues: plain fp32,
// or the ReLU mask (the forward's fp32 hidden value > 0).
#include "common.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kT = 64;          // tile rows and columns of D
constexpr int kBK = 16;         // K per step
constexpr int kThreads = 256;   // 4 waves, 2 x 2
constexpr int kNKld = kBK + 1;  // padded row of the row-major B tile

template <int MODE, int EPI>
__global__ __launch_bounds__(kThreads) void ggemm_bwd_f32_kernel(GemmBwdArgs p) {
  __shared__ float sa[2][kBK][kT];
  __shared__ float sb[2][MODE == BWD_ROWS ? kT * kNKld : kBK * kT];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int MT = (p.M + kT - 1) / kT;
  const float* Af = (const float*)p.A;
  const float* A2f = (const float*)p.A2;
  const float* Bf = (const float*)p.B;

  int e, m0, c0, c_end, k_lo, k_hi;
  if constexpr (MODE == BWD_ROWS) {
    // each tile of the dispatch's map (p.tile_rows rows) in kT-row parts
    const int SUB = p.tile_rows / kT;
    const int total = *p.tile_count * SUB * MT;
    const int t = (int)blockIdx.x;
    if (t >= total) return;
    const int rt = t / (SUB * MT), rem = t % (SUB * MT);
    m0 = (rem % MT) * kT;
    e = p.tile_expert[rt];
    c0 = p.tile_row0[rt] + (rem / MT) * kT;
    c_end = p.offsets[e + 1];
    if (c0 >= c_end) return;
    k_lo = 0;
    k_hi = p.K;
  } else {
    const int NT = (p.N + kT - 1) / kT;
    const int t = (int)blockIdx.x;
    if (t >= p.n_experts * MT * NT) return;
    e = t / (MT * NT);
    const int r = t % (MT * NT);
    c0 = (r / MT) * kT;
    m0 = (r % MT) * kT;
    c_end = p.N;
    k_lo = p.offsets[e];
    k_hi = p.offsets[e + 1];
  }
  const float* A = Af + (long long)e * p.strideA;
  const float* A2 = A2f ? A2f + (long long)e * p.strideA : nullptr;
  const int nsteps = (k_hi - k_lo + kBK - 1) / kBK;

  // Thread tid loads element (row kr, column cc..cc+3) of each K-major tile
  // (16 rows x 64), or (row r, k kk..kk+3) of the row-major one (64 x 16).
  const int kr = tid >> 4, cc = (tid & 15) * 4;
  f32x4 ra, rb;
  auto load = [&](int step) {
    const int k = k_lo + step * kBK + kr;
    ra = f32x4{0.f, 0.f, 0.f, 0.f};
    if (k < k_hi && m0 + cc < p.M) {
      const long long ka = p.rowmap_a ? (long long)p.rowmap_a[k] : (long long)k;
      const float* src = (A2 && k >= p.k_split) ? A2 + (long long)(k - p.k_split) * p.lda
                                                : A + ka * p.lda;
      ra = *(const f32x4*)(src + m0 + cc);
    }
    rb = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (MODE == BWD_ROWS) {
      const int r = tid >> 2, kk = (tid & 3) * 4;
      const int row = min(c0 + r, c_end - 1);  // rows past the segment: valid, never stored
      rb = *(const f32x4*)(Bf + (long long)row * p.ldb + k_lo + step * kBK + kk);
    } else {
      if (k < k_hi && c0 + cc < p.N)
        rb = *(const f32x4*)(Bf + (long long)k * p.ldb + c0 + cc);
    }
  };
  auto store = [&](int buf) {
    *(f32x4*)&sa[buf][kr][cc] = ra;
    if constexpr (MODE == BWD_ROWS) {
      const int r = tid >> 2, kk = (tid & 3) * 4;
#pragma unroll
      for (int q = 0; q < 4; ++q) sb[buf][r * kNKld + kk + q] = rb[q];
    } else {
      *(f32x4*)&sb[buf][kr * kT + cc] = rb;
    }
  };

  f32x16 acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.f;
  if (nsteps > 0) {
    load(0);
    store(0);
  }
  __syncthreads();
  for (int g = 0; g < nsteps; ++g) {
    const int cur = g & 1;
    if (g + 1 < nsteps) load(g + 1);
#pragma unroll
    for (int kk = 0; kk < kBK / 2; ++kk) {
      const int k = 2 * kk + (lane >> 5);
      const float a = sa[cur][k][wm * 32 + (lane & 31)];
      const int c = wn * 32 + (lane & 31);
      const float b = MODE == BWD_ROWS ? sb[cur][c * kNKld + k] : sb[cur][k * kT + c];
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc, 0, 0, 0);
    }
    if (g + 1 < nsteps) store(cur ^ 1);
    __syncthreads();
  }

  // lane holds D[m .. m+3][c] for m = base + 8 q + 4 (lane / 32)
  const int c = c0 + wn * 32 + (lane & 31);
  if (c >= c_end) return;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int m = m0 + wm * 32 + 8 * q + 4 * (lane >> 5);
    if (m >= p.M) continue;
    f32x4 v = {acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
    float* out;
    if constexpr (MODE == BWD_WGRAD) {
      out = (c < p.c_split)
                ? p.C + (long long)e * p.strideC + (long long)c * p.ldc + m
                : p.C2 + (long long)e * p.strideC + (long long)(c - p.c_split) * p.ldc + m;
    } else {
      out = p.C + (long long)c * p.ldc + m;
    }
    if constexpr (EPI == BEPI_RELU_MASK) {
      const f32x4 h = *(const f32x4*)(p.aux_a + (long long)c * p.ldaux + m);
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = h[u] > 0.f ? v[u] : 0.f;
    }
    if constexpr (MODE == BWD_WGRAD)
      __builtin_nontemporal_store(v, (f32x4*)out);  // written once, not read again here
    else
      *(f32x4*)out = v;
  }
}

}  // namespace

hipError_t launch_gemm_bwd_f32(const GemmBwdArgs& a, int mode, int epi, const char* name,
                               hipStream_t s) {
  const int MT = (a.M + kT - 1) / kT;
  long long blocks;
  if (mode == BWD_ROWS)
    blocks = (long long)a.max_tiles * (a.tile_rows / kT) * MT;
  else
    blocks = (long long)a.n_experts * MT * ((a.N + kT - 1) / kT);
  if (blocks <= 0) return hipSuccess;
  ProfScope ps(name, s);
  if (mode == BWD_ROWS) {
    const dim3 grid((unsigned)blocks);
    if (epi == BEPI_RELU_MASK)
      ggemm_bwd_f32_kernel<BWD_ROWS, BEPI_RELU_MASK><<<grid, kThreads, 0, s>>>(a);
    else
      ggemm_bwd_f32_kernel<BWD_ROWS, BEPI_F32><<<grid, kThreads, 0, s>>>(a);
  } else {
    ggemm_bwd_f32_kernel<BWD_WGRAD, BEPI_F32><<<dim3((unsigned)blocks), kThreads, 0, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace moe
