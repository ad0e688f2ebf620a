// Gate logits C = x . [W_g; W_noise]^T (fp32 in, fp32 out) on the bf16 matrix
// cores, at fp32 accuracy.
//
// The fp32 matrix instruction (v_mfma_f32_32x32x2_f32) runs at 1/16 of the
// bf16 one on gfx950.  Each fp32 operand v is split exactly into three bf16
// parts, v = hi + mid + lo (hi = bf16(v), mid = bf16(v - hi), lo = bf16(v -
// hi - mid); the first two differences are exact in fp32, and the parts
// carry 24 significant bits together), and a.b is summed from the six
// products whose size is at least 2^-18 of a.b's: hi.hi, hi.mid, mid.hi,
// hi.lo, lo.hi, mid.mid.  The omitted products (mid.lo, lo.mid, lo.lo) are
// below 2^-25 of it, under the fp32 accumulation's own rounding (the split of
// Dekker and Ogita-Rump-Oishi's error-free transformations, in the form used
// for emulated single-precision GEMM on low-precision matrix units, e.g.
// Henry, Tang and Heinecke, "Leveraging the bfloat16 artificial intelligence
// datatype for higher-precision computations", 2019).
//
// Accumulation: rounding each partial sum into one fp32 accumulator K/16 x 6
// times would leave a random walk of about sqrt(K/16 x 6) half-ulps (~1e-6
// of |logit| at d = 7168, the size of the closest top-k gaps of such
// batches).  So the five small products go to their own accumulator (their
// roundings are 2^-8 smaller), and the hi.hi products are summed in chunks of
// 256 K into a fresh accumulator that is then added to the total: about
// sqrt(K/256) roundings at full magnitude.
//
// The split is made once per element, when a tile is stored to LDS: the fp32
// tile is loaded to registers, split, and written as three bf16 tiles.  MFMA:
// v_mfma_f32_32x32x16_bf16 computing D = W . x^T (gate columns as rows of D),
// so each lane ends with four consecutive logit columns of one token.
// Tiles 128 x 128 on 8 waves (4 across the columns) or 64 x 64 on 4 waves,
// K steps of 32, two LDS stages, fp32 loads two steps ahead in registers.
//
// K-split (flat mode): with few tiles and a long K (T = 4096 tokens, 256
// experts and d = 7168 make 256 tiles of 64 x 64, one per CU, each 7168 deep)
// a CU would hold one workgroup's two steps of loads in flight and wait on
// them; split into ranges of K, the items fill every CU three times over.
// Each range starts on a 256-element chunk boundary and writes its own fp32
// partial; the gate epilogue adds the partials in split order (a fixed
// order, so the logits do not depend on scheduling), one more level of the
// chunked accumulation above.
#include "common.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kBK = 32;         // K per step
constexpr int kRowB = kBK * 2;  // bytes of one bf16 row of a tile component

// 16-byte chunk c (0..3) of row r sits at c ^ (r/4 % 4): the 32 rows one
// fragment read touches spread over every bank.
__device__ __forceinline__ int gswz(int r, int c) {
  return r * kRowB + ((c ^ ((r >> 2) & 3)) << 4);
}

// Split four fp32 values into three packed bf16 parts (2 dwords each).
__device__ __forceinline__ void split3(const f32x4 v, uint2& hi, uint2& mid, uint2& lo) {
  hi = make_uint2(bf16x2_bits(v[0], v[1]), bf16x2_bits(v[2], v[3]));
  float r[4];
  r[0] = v[0] - __uint_as_float(hi.x << 16);
  r[1] = v[1] - __uint_as_float(hi.x & 0xffff0000u);
  r[2] = v[2] - __uint_as_float(hi.y << 16);
  r[3] = v[3] - __uint_as_float(hi.y & 0xffff0000u);
  mid = make_uint2(bf16x2_bits(r[0], r[1]), bf16x2_bits(r[2], r[3]));
  r[0] -= __uint_as_float(mid.x << 16);
  r[1] -= __uint_as_float(mid.x & 0xffff0000u);
  r[2] -= __uint_as_float(mid.y << 16);
  r[3] -= __uint_as_float(mid.y & 0xffff0000u);
  lo = make_uint2(bf16x2_bits(r[0], r[1]), bf16x2_bits(r[2], r[3]));
}

template <int BM, int WGM, int WGN>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_gate_kernel(const GemmF32Args p) {
  constexpr int NT = 64 * WGM * WGN;
  constexpr int BN = BM;                    // tokens per tile (columns of D)
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int FM = WM / 32, FN = WN / 32;
  constexpr int CH = BM * kBK / 4 / NT;     // float4 chunks per thread per operand
  constexpr int COMP = BM * kRowB;          // bytes of one bf16 component tile
  constexpr int STAGE = 6 * COMP;           // W hi/mid/lo, x hi/mid/lo
  static_assert(CH >= 1 && FM >= 1 && FN >= 1, "bad tile shape");
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];

  // D rows: gate columns (W rows); D columns: tokens.  Flat mode: tokens
  // [mt*BN, M).  Grouped mode (a device tile map of BN-row tiles): rows
  // [tile_row0, min(+BN, offsets[g+1])) of group g, whose weights are
  // B1 + g*strideB1 | B2 + g*strideB2, token rows read through rowmap.
  // K-split (flat mode): work item L is (split, M-tile, column tile) with the
  // column tile fastest, so an XCD's neighbouring items share token rows.
  const bool grouped = p.tile_expert != nullptr;
  const int nW = (p.N + BM - 1) / BM;
  const int nsplit = grouped ? 1 : max(1, p.ksplit);
  const int tiles = (grouped ? *p.tile_count : p.mtiles) * nW;
  const int L = xcd_tile(tiles * nsplit);
  if (L < 0) return;
  const int ks = L / tiles, mt = (L % tiles) / nW, wt = L % nW;
  const int col0 = wt * BM;
  int tok0 = mt * BN, tok_end = p.M;
  const float* B1 = p.B1;
  const float* B2 = p.B2;
  if (grouped) {
    const int g = p.tile_expert[mt];
    tok0 = p.tile_row0[mt];
    tok_end = min(tok0 + BN, p.offsets[g + 1]);
    B1 += (long long)g * p.strideB1;
    if (B2) B2 += (long long)g * p.strideB2;
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  // This item's K range [kb, K); the ranges start at multiples of 256, so
  // the accumulation chunks below stay aligned to K = 0.
  const int klen = nsplit > 1 ? gate_split_len(p.K, nsplit) : p.K;
  const int kb = ks * klen;
  const int K = min(p.K, kb + klen);
  float* const C = p.C + (long long)ks * p.split_stride;

  // Global sources of this thread's chunks (row r, k offset kc), and where
  // the x chunks' bf16 copy goes (first column tile of a flat launch with
  // a_bf16).
  const bool xcopy = p.a_bf16 && !grouped && wt == 0;
  const float* wsrc[CH];
  const float* xsrc[CH];
  uint16_t* xdst[CH];
  bool wok[CH], xok[CH];
  int rr[CH], kc[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int c = tid + NT * i;
    rr[i] = c / (kBK / 4);
    kc[i] = (c % (kBK / 4)) * 4;
    const int gc = col0 + rr[i];
    wok[i] = gc < p.N;
    const float* wrow =
        gc < p.n1 ? B1 + (long long)gc * p.K : B2 + (long long)(gc - p.n1) * p.K;
    wsrc[i] = (wok[i] ? wrow : B1) + kb + kc[i];
    const int gt = tok0 + rr[i];
    xok[i] = gt < tok_end;
    const long long arow = !xok[i] ? 0 : p.rowmap ? (long long)p.rowmap[gt] : (long long)gt;
    xsrc[i] = p.A + arow * p.lda + kb + kc[i];
    xdst[i] = xcopy ? p.a_bf16 + (long long)gt * p.K + kb + kc[i] : nullptr;
  }
  // Two register buffers: step s's fp32 chunks live in buffer s % 2, are
  // loaded two steps ahead and split into LDS one step ahead.
  f32x4 rw[2][CH], rx[2][CH];
  auto load = [&](int k0, int rb) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const bool kin = kb + k0 + kc[i] < K;
      rw[rb][i] = (wok[i] && kin) ? *(const f32x4*)(wsrc[i] + k0) : f32x4{0.f, 0.f, 0.f, 0.f};
      rx[rb][i] = (xok[i] && kin) ? *(const f32x4*)(xsrc[i] + k0) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };
  // Split register buffer rb (the step at K offset k0 of this range) into
  // LDS stage buf.
  auto store = [&](int buf, int rb, int k0) {
    uint8_t* st = smem + buf * STAGE;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int off = gswz(rr[i], kc[i] >> 3) + ((kc[i] >> 2) & 1) * 8;
      uint2 h, m, l;
      split3(rw[rb][i], h, m, l);
      *(uint2*)(st + 0 * COMP + off) = h;
      *(uint2*)(st + 1 * COMP + off) = m;
      *(uint2*)(st + 2 * COMP + off) = l;
      split3(rx[rb][i], h, m, l);
      if (xcopy && xok[i] && kb + k0 + kc[i] < K) *(uint2*)(xdst[i] + k0) = h;
      *(uint2*)(st + 3 * COMP + off) = h;
      *(uint2*)(st + 4 * COMP + off) = m;
      *(uint2*)(st + 5 * COMP + off) = l;
    }
  };

  f32x16 acc[FM][FN], chunk[FM][FN], small[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = chunk[i][j][v] = small[i][j][v] = 0.f;
  constexpr int kChunkSteps = 256 / kBK;

  const int nk = (K - kb + kBK - 1) / kBK;
  const int lr = lane & 31, lh = lane >> 5;
  // Step kt (register buffer and LDS stage rb = kt % 2): load step kt+2,
  // compute step kt, split step kt+1 into the other stage.
  auto step = [&](int kt, int rb) {
    if (kt + 2 < nk) load((kt + 2) * kBK, rb);
    const uint8_t* st = smem + rb * STAGE;
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      bf16x8 a[3][FM], b[3][FN];
#pragma unroll
      for (int q = 0; q < 3; ++q) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
          a[q][i] = *(const bf16x8*)(st + q * COMP + gswz(wm * WM + i * 32 + lr, 2 * kk + lh));
#pragma unroll
        for (int j = 0; j < FN; ++j)
          b[q][j] =
              *(const bf16x8*)(st + (3 + q) * COMP + gswz(wn * WN + j * 32 + lr, 2 * kk + lh));
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          f32x16 c = small[i][j];
          c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1][i], b[1][j], c, 0, 0, 0);
          c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[2][i], b[0][j], c, 0, 0, 0);
          c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0][i], b[2][j], c, 0, 0, 0);
          c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1][i], b[0][j], c, 0, 0, 0);
          small[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0][i], b[1][j], c, 0, 0, 0);
          chunk[i][j] =
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0][i], b[0][j], chunk[i][j], 0, 0, 0);
        }
    }
    if ((kt + 1) % kChunkSteps == 0 || kt + 1 == nk) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            acc[i][j][v] += chunk[i][j][v];
            chunk[i][j][v] = 0.f;
          }
    }
    if (kt + 1 < nk) store(rb ^ 1, rb ^ 1, (kt + 1) * kBK);
    __syncthreads();
  };
  load(0, 0);
  if (nk > 1) load(kBK, 1);
  store(0, 0, 0);
  __syncthreads();
  for (int kt = 0; kt < nk; kt += 2) {
    step(kt, 0);
    if (kt + 1 < nk) step(kt + 1, 1);
  }
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] += small[i][j][v];

  // lane holds D[col .. col+3][tok]: four consecutive logit columns of token tok
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int tok = tok0 + wn * WN + j * 32 + lr;
    if (tok >= tok_end) continue;
    float* crow = C + (long long)tok * p.ldc;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = col0 + wm * WM + i * 32 + 8 * q + 4 * lh;
        if (col >= p.N) continue;
        const f32x4 v = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                         acc[i][j][4 * q + 3]};
        if (col + 4 <= p.N) {
          *(f32x4*)(crow + col) = v;
        } else {
          for (int u = 0; u < 4 && col + u < p.N; ++u) crow[col + u] = v[u];
        }
      }
  }
}

}  // namespace

hipError_t launch_gemm_gate(const GemmF32Args& a, int bm, hipStream_t s) {
  if (a.bias || a.relu) return hipErrorInvalidValue;  // not an epilogue of this kernel
  if (a.ksplit > 1 && (a.tile_expert || gate_split_len(a.K, a.ksplit) * (a.ksplit - 1) >= a.K))
    return hipErrorInvalidValue;  // flat mode only, and every split non-empty
  const int nW = (a.N + bm - 1) / bm;
  const long long total = (long long)(a.tile_expert ? a.max_mtiles : a.mtiles) * nW *
                          (a.ksplit > 1 ? a.ksplit : 1);
  if (total <= 0) return hipSuccess;
  const long long grid = (total + kXcds - 1) / kXcds * kXcds;
  ProfScope ps(a.prof_name ? a.prof_name : "gate_gemm_bf16x6", s);
  if (bm == 128)
    gemm_gate_kernel<128, 4, 2><<<dim3((unsigned)grid), dim3(512), 0, s>>>(a);
  else
    gemm_gate_kernel<64, 2, 2><<<dim3((unsigned)grid), dim3(256), 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace moe
