// fp32 GEMM on the gfx950 matrix cores (v_mfma_f32_32x32x2_f32).
//
// Used for fp32 experts (grouped rows, ReLU and bias fused).  The gate
// logits (flat, primary and secondary) use gemm_gate.hip, which reaches fp32
// accuracy on the bf16 instruction.  C = A . B^T with both operands
// K-contiguous; tiles 64x64 (4 waves in a 2x2 grid) or 128x128 (8 waves in
// a 2x4 grid: half the operand re-reads of 64x64 tiles, two waves per SIMD),
// BK = 32, double-buffered LDS with register prefetch, one barrier per K
// step, epilogue staged through LDS for full-width stores.
#include "common.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kBK = 32;
constexpr int kLDK = kBK + 4;  // padded LDS row (floats): conflict-free b128 reads

template <int BM, int WGM, int WGN>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_f32_kernel(const GemmF32Args p) {
  constexpr int NT = 64 * WGM * WGN;  // threads
  constexpr int BN = BM;
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int FM = WM / 32, FN = WN / 32;
  constexpr int ACH = BM * kBK / 4 / NT;  // float4 chunks per thread (A)
  constexpr int BCH = BN * kBK / 4 / NT;
  static_assert(ACH >= 1 && BCH >= 1 && FM >= 1 && FN >= 1, "bad tile shape");
  constexpr int STAGE = (BM + BN) * kLDK;
  constexpr int LDC = BN + 4;
  static_assert(BM * LDC <= 2 * STAGE, "epilogue staging must fit");
  __shared__ __attribute__((aligned(16))) float smem[2 * STAGE];

  const int nN = (p.N + BN - 1) / BN;
  const int mtiles = p.tile_count ? *p.tile_count : p.mtiles;
  const int L = xcd_tile(mtiles * nN);
  if (L < 0) return;
  const int mt = L / nN, nt = L % nN;
  int g = 0, row0, row_end;
  if (p.tile_expert) {
    g = p.tile_expert[mt];
    row0 = p.tile_row0[mt];
    row_end = p.offsets[g + 1];
  } else {
    row0 = mt * BM;
    row_end = p.M;
  }
  const int n0 = nt * BN;
  const int tid = threadIdx.x;
  const int K = p.K;

  // Per-thread global sources (advance by kBK per step).
  const float* asrc[ACH];
  bool aok[ACH];
  int akc[ACH], arow[ACH];
#pragma unroll
  for (int i = 0; i < ACH; ++i) {
    const int c = tid + NT * i;
    const int r = c / (kBK / 4);
    akc[i] = (c % (kBK / 4)) * 4;
    arow[i] = r;
    const int gr = row0 + r;
    aok[i] = gr < row_end;
    const long long src_row = aok[i] ? (p.rowmap ? (long long)p.rowmap[gr] : (long long)gr) : 0;
    asrc[i] = p.A + src_row * p.lda + akc[i];
  }
  const float* bsrc[BCH];
  bool bok[BCH];
  int bkc[BCH], brow[BCH];
#pragma unroll
  for (int i = 0; i < BCH; ++i) {
    const int c = tid + NT * i;
    const int r = c / (kBK / 4);
    bkc[i] = (c % (kBK / 4)) * 4;
    brow[i] = r;
    const int gn = n0 + r;
    bok[i] = gn < p.N;
    const float* base = p.B1 + (long long)g * p.strideB1 + (long long)gn * K;
    if (gn >= p.n1) base = p.B2 + (long long)g * p.strideB2 + (long long)(gn - p.n1) * K;
    bsrc[i] = (bok[i] ? base : p.B1) + bkc[i];
  }

  f32x4 ra[ACH], rb[BCH];
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
      const bool ok = aok[i] && (k0 + akc[i] < K);
      ra[i] = ok ? *(const f32x4*)(asrc[i] + k0) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int i = 0; i < BCH; ++i) {
      const bool ok = bok[i] && (k0 + bkc[i] < K);
      rb[i] = ok ? *(const f32x4*)(bsrc[i] + k0) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };
  auto store = [&](int buf) {
    float* As = smem + buf * STAGE;
    float* Bs = As + BM * kLDK;
#pragma unroll
    for (int i = 0; i < ACH; ++i) *(f32x4*)(As + arow[i] * kLDK + akc[i]) = ra[i];
#pragma unroll
    for (int i = 0; i < BCH; ++i) *(f32x4*)(Bs + brow[i] * kLDK + bkc[i]) = rb[i];
  };

  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const int lr = lane & 31, lh = lane >> 5;

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int nk = (K + kBK - 1) / kBK;
  load(0);
  store(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load((kt + 1) * kBK);
    const float* As = smem + cur * STAGE;
    const float* Bs = As + BM * kLDK;
    // Lanes 0-31 feed k-slot 0 of each MFMA with k in [0,16) of the tile,
    // lanes 32-63 feed k-slot 1 with k in [16,32): A and B agree on the
    // k of every slot, so each MFMA adds two distinct k terms.
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      f32x4 av[FM], bv[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        av[i] = *(const f32x4*)(As + (wm * WM + i * 32 + lr) * kLDK + lh * 16 + s4 * 4);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        bv[j] = *(const f32x4*)(Bs + (wn * WN + j * 32 + lr) * kLDK + lh * 16 + s4 * 4);
#pragma unroll
      for (int ss = 0; ss < 4; ++ss)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[i][ss], bv[j][ss], acc[i][j], 0,
                                                             0, 0);
    }
    if (kt + 1 < nk) store(cur ^ 1);
    __syncthreads();
  }

  // Stage the tile in LDS (32x32 accumulator layout: column lane%32, row
  // 8*(v/4) + 4*(lane/32) + v%4), then write full rows.
  float* Cs = smem;
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = wm * WM + i * 32 + (v >> 2) * 8 + lh * 4 + (v & 3);
        const int c = wn * WN + j * 32 + lr;
        Cs[r * LDC + c] = acc[i][j][v];
      }
  __syncthreads();
  const float* bias = p.bias ? p.bias + (long long)g * p.stride_bias : nullptr;
  for (int c = tid; c < BM * BN / 4; c += NT) {
    const int r = c / (BN / 4);
    const int cc = (c % (BN / 4)) * 4;
    const int gr = row0 + r;
    const int gc = n0 + cc;
    if (gr >= row_end || gc >= p.N) continue;
    f32x4 v = *(const f32x4*)(Cs + r * LDC + cc);
    float* out = p.C + (long long)gr * p.ldc + gc;
    if (gc + 4 <= p.N) {
      if (bias) {
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] += bias[gc + q];
      }
      if (p.relu) {
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = fmaxf(v[q], 0.f);
      }
      *(f32x4*)out = v;
    } else {
      for (int q = 0; q < 4 && gc + q < p.N; ++q) {
        float t = v[q] + (bias ? bias[gc + q] : 0.f);
        out[q] = p.relu ? fmaxf(t, 0.f) : t;
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm_f32(const GemmF32Args& a, int bm, hipStream_t s) {
  const int nN = (a.N + bm - 1) / bm;
  const long long max_total = (long long)a.max_mtiles * nN;
  if (max_total <= 0) return hipSuccess;
  const long long grid = (max_total + kXcds - 1) / kXcds * kXcds;
  ProfScope ps(a.prof_name ? a.prof_name : bm == 128 ? "gemm_f32_bm128" : "gemm_f32_bm64", s);
  if (bm == 128)
    gemm_f32_kernel<128, 2, 4><<<dim3((unsigned)grid), dim3(512), 0, s>>>(a);
  else
    gemm_f32_kernel<64, 2, 2><<<dim3((unsigned)grid), dim3(256), 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace moe
