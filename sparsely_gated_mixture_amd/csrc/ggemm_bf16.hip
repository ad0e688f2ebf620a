// Grouped GEMM of the expert FFNs on the gfx950 matrix cores
// (v_mfma_f32_32x32x16_bf16: bf16 operands, fp32 accumulation).
//
// One launch covers every expert: a device-side tile map lists the M-tiles
// (kBf16BM rows of one expert's merged batch) and every workgroup takes one
// (M-tile, N-tile) pair.  The weights of expert e are B[e] = [N, K] (out x in,
// K contiguous) and the activations A = [rows, K], so both operands stream
// along K.  Tile 128 x 128 (SwiGLU: 128 x 64 outputs over the W1 and W3 rows),
// BK = 64, four waves in a 2x2 grid, double-buffered padded LDS (one barrier
// per K step), epilogue staged through LDS for 16-byte coalesced stores.
// Epilogues: ReLU(+bias) -> bf16 hidden, silu(g)*u -> bf16 hidden,
// identity(+bias) -> fp32 expert output.
// Workgroups are mapped so that each XCD owns a contiguous run of tiles: the
// N-tiles of one M-tile (which share the activation tile) and the M-tiles of
// one expert (which share its weight tiles) meet in the same L2.
#include <math.h>

#include "common.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kBK = 64;
constexpr int kLDK = kBK + 8;  // padded LDS row (bf16): 144 B, conflict-free b128 reads

template <int BM, int BN, int EPI>
__global__ __launch_bounds__(256) void ggemm_bf16_kernel(const GemmBf16Args p) {
  constexpr int NB = (EPI == EPI_SWIGLU_BF16) ? 2 : 1;  // weight matrices per tile
  constexpr int BROWS = NB * BN;                         // weight rows per tile
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int FM = WM / 32, FN = WN / 32;
  constexpr int ACH = BM * kBK / 8 / 256;     // 16-byte chunks per thread
  constexpr int BCH = BROWS * kBK / 8 / 256;
  constexpr int STAGE = (BM + BROWS) * kLDK;  // bf16 elements per stage
  constexpr int LDC = BN + 4;
  static_assert(BM * LDC * 4 <= 2 * STAGE * 2, "epilogue staging must fit");
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * STAGE];

  const int nN = (p.N + BN - 1) / BN;
  const int L = xcd_tile(*p.tile_count * nN);
  if (L < 0) return;
  const int mt = L / nN, nt = L % nN;
  const int e = p.tile_expert[mt];
  const int row0 = p.tile_row0[mt];
  const int row_end = p.offsets[e + 1];
  const int n0 = nt * BN;
  const int K = p.K;
  const int tid = threadIdx.x;

  const uint16_t* asrc[ACH];
  bool aok[ACH];
  int aoff[ACH], akc[ACH];
#pragma unroll
  for (int i = 0; i < ACH; ++i) {
    const int c = tid + 256 * i;
    const int r = c / (kBK / 8), kc = (c % (kBK / 8)) * 8;
    aoff[i] = r * kLDK + kc;
    akc[i] = kc;
    aok[i] = row0 + r < row_end;
    asrc[i] = p.A + (long long)(aok[i] ? row0 + r : row0) * p.lda + kc;
  }
  const uint16_t* bsrc[BCH];
  bool bok[BCH];
  int boff[BCH], bkc[BCH];
#pragma unroll
  for (int i = 0; i < BCH; ++i) {
    const int c = tid + 256 * i;
    const int r = c / (kBK / 8), kc = (c % (kBK / 8)) * 8;
    const int which = r / BN, rn = r % BN;
    boff[i] = r * kLDK + kc;
    bkc[i] = kc;
    bok[i] = n0 + rn < p.N;
    const uint16_t* base = (which == 0 ? p.B1 : p.B3) + (long long)e * p.strideB;
    bsrc[i] = base + (long long)(bok[i] ? n0 + rn : 0) * K + kc;
  }

  uint4 ra[ACH], rb[BCH];
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
      const bool ok = aok[i] && (k0 + akc[i] < K);
      ra[i] = ok ? *(const uint4*)(asrc[i] + k0) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int i = 0; i < BCH; ++i) {
      const bool ok = bok[i] && (k0 + bkc[i] < K);
      rb[i] = ok ? *(const uint4*)(bsrc[i] + k0) : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  auto store = [&](int buf) {
    uint16_t* As = smem + buf * STAGE;
    uint16_t* Bs = As + BM * kLDK;
#pragma unroll
    for (int i = 0; i < ACH; ++i) *(uint4*)(As + aoff[i]) = ra[i];
#pragma unroll
    for (int i = 0; i < BCH; ++i) *(uint4*)(Bs + boff[i]) = rb[i];
  };

  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 31, lh = lane >> 5;

  f32x16 acc[NB][FM][FN];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[b][i][j][v] = 0.f;

  const int nk = (K + kBK - 1) / kBK;
  load(0);
  store(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load((kt + 1) * kBK);
    const uint16_t* As = smem + cur * STAGE;
    const uint16_t* Bs = As + BM * kLDK;
    // 32x32x16 operand layout: lane supplies row (lane%32), k = 8*(lane/32)..+7.
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      bf16x8 af[FM], bfr[NB][FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[i] = *(const bf16x8*)(As + (wm * WM + i * 32 + lr) * kLDK + kk * 16 + lh * 8);
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          bfr[b][j] =
              *(const bf16x8*)(Bs + (b * BN + wn * WN + j * 32 + lr) * kLDK + kk * 16 + lh * 8);
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[b][i][j] =
                __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[b][j], acc[b][i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) store(cur ^ 1);
    __syncthreads();
  }

  // Stage the (activated) tile as fp32 in LDS: accumulator element v of a
  // 32x32 block sits at column lane%32, row 8*(v/4) + 4*(lane/32) + v%4.
  float* Cs = (float*)smem;
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = wm * WM + i * 32 + (v >> 2) * 8 + lh * 4 + (v & 3);
        const int c = wn * WN + j * 32 + lr;
        float val;
        if constexpr (EPI == EPI_SWIGLU_BF16) {
          const float gv = acc[0][i][j][v], uv = acc[NB - 1][i][j][v];
          val = gv / (1.f + expf(-gv)) * uv;
        } else {
          val = acc[0][i][j][v];
        }
        Cs[r * LDC + c] = val;
      }
  __syncthreads();

  const float* bias = p.bias ? p.bias + (long long)e * p.N : nullptr;
  if constexpr (EPI == EPI_IDENT_F32) {
    for (int c = tid; c < BM * BN / 4; c += 256) {
      const int r = c / (BN / 4), cc = (c % (BN / 4)) * 4;
      const int gr = row0 + r, gc = n0 + cc;
      if (gr >= row_end || gc >= p.N) continue;
      f32x4 v = *(const f32x4*)(Cs + r * LDC + cc);
      if (bias) {
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] += bias[gc + q];
      }
      *(f32x4*)((float*)p.C + (long long)gr * p.ldc + gc) = v;
    }
  } else {
    for (int c = tid; c < BM * BN / 8; c += 256) {
      const int r = c / (BN / 8), cc = (c % (BN / 8)) * 8;
      const int gr = row0 + r, gc = n0 + cc;
      if (gr >= row_end || gc >= p.N) continue;
      const f32x4 v0 = *(const f32x4*)(Cs + r * LDC + cc);
      const f32x4 v1 = *(const f32x4*)(Cs + r * LDC + cc + 4);
      float f[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
      if constexpr (EPI == EPI_RELU_BF16) {
#pragma unroll
        for (int q = 0; q < 8; ++q) f[q] = fmaxf(f[q] + (bias ? bias[gc + q] : 0.f), 0.f);
      }
      uint4 pk;
      pk.x = (uint32_t)f32_to_bf16(f[0]) | ((uint32_t)f32_to_bf16(f[1]) << 16);
      pk.y = (uint32_t)f32_to_bf16(f[2]) | ((uint32_t)f32_to_bf16(f[3]) << 16);
      pk.z = (uint32_t)f32_to_bf16(f[4]) | ((uint32_t)f32_to_bf16(f[5]) << 16);
      pk.w = (uint32_t)f32_to_bf16(f[6]) | ((uint32_t)f32_to_bf16(f[7]) << 16);
      *(uint4*)((uint16_t*)p.C + (long long)gr * p.ldc + gc) = pk;
    }
  }
}

template <int BM, int BN, int EPI>
hipError_t launch_t(const GemmBf16Args& a, hipStream_t s) {
  const int nN = (a.N + BN - 1) / BN;
  const long long max_total = (long long)a.max_mtiles * nN;
  if (max_total <= 0) return hipSuccess;
  const long long grid = (max_total + kXcds - 1) / kXcds * kXcds;
  ProfScope ps(EPI == EPI_RELU_BF16     ? "ggemm_bf16_relu"
               : EPI == EPI_SWIGLU_BF16 ? "ggemm_bf16_swiglu"
                                        : "ggemm_bf16_out",
               s);
  ggemm_bf16_kernel<BM, BN, EPI><<<dim3((unsigned)grid), dim3(256), 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_bf16(const GemmBf16Args& a, int epi, hipStream_t s) {
  switch (epi) {
    case EPI_RELU_BF16:
      return launch_t<kBf16BM, 128, EPI_RELU_BF16>(a, s);
    case EPI_SWIGLU_BF16:
      return launch_t<kBf16BM, 64, EPI_SWIGLU_BF16>(a, s);
    default:
      return launch_t<kBf16BM, 128, EPI_IDENT_F32>(a, s);
  }
}

}  // namespace moe
