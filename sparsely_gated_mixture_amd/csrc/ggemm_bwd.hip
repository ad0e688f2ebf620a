// Grouped bf16 GEMMs of the expert backward on the gfx950 matrix cores
// (v_mfma_f32_32x32x16_bf16, fp32 accumulation).
//
// Every product of the backward has an operand whose reduction index runs
// down its rows (a weight matrix used transposed, or the merged rows of an
// expert summed over).  Such an operand is staged in LDS as stored, K rows
// of 128 contiguous columns, and its MFMA fragments (8 consecutive K of one
// column per lane) are read with the gfx950 transposing LDS read
// ds_read_b64_tr_b16: within each 16-lane group, lane j addresses row
// k0 + j/4 at columns c0 + 4(j%4) .. +3, and lane i receives column c0 + i at
// rows k0 .. k0+3.  Two such reads make one fragment.
//
// The kernel computes D[m][c] = sum_k A[k][m] * B(k, c) for one 128 x 128
// tile per workgroup (4 waves, 64 x 64 each) and stores C[c][m] = D[m][c],
// so each lane holds four consecutive output columns.  A is always stored
// K-major (row k holds the M columns).  Two modes:
//  * ROWS: c runs over the merged rows of one expert (a 128-row tile of the
//    dispatch's tile map), A is that expert's weight matrix, B is stored
//    row-major by merged row with K contiguous and is read with plain
//    16-byte LDS reads.  Used for the input gradients of the two layers.
//  * WGRAD: one expert per tile, K runs over the expert's merged rows (a
//    ragged count, zero rows included: the tile is then stored as zeros),
//    and B is stored K-major like A.  Used for the weight gradients.
// Epilogues: ReLU mask (dpre = dhid where the forward's hidden value is
// positive) to bf16; SwiGLU (da, db from the saved pre-activations) to
// bf16; plain fp32.  Each one stages the finished tile through LDS, so its
// global reads and writes cover whole row segments.
// Operands go to LDS by direct global->LDS copies: ROWS mode keeps a ring of
// two 32 KB stages (the next K-step's copies are issued before the current
// step's MFMAs); WGRAD mode one stage, with four workgroups per CU.
#include <math.h>

#include "common.h"
#include "launch.h"
#include "lds_dma.h"

namespace moe {
namespace {

constexpr int kTile = 128;     // tile rows and columns of D
constexpr int kBK = 64;        // K per step
constexpr int kThreads = 256;  // 4 waves in a 2 x 2 grid
constexpr int kHalf = 16384;   // bytes of one operand's stage
constexpr int kStage = 2 * kHalf;

typedef short s16x4 __attribute__((ext_vector_type(4)));
#define LDS_AS __attribute__((address_space(3)))

// Byte offset of (row k, column m) in a K-major tile (256-byte rows of 128
// bf16).  16-byte chunk c of row k sits at c ^ 4 (k % 4): the eight rows one
// transposing read touches (k0 .. k0+3 and k0+8 .. k0+11, 64 bytes each)
// then cover every bank twice instead of one 64-byte window eight times.
__device__ __forceinline__ uint32_t km_off(int k, int m) {
  return (uint32_t)(k * 256 + ((((m >> 3) ^ ((k & 3) << 2))) << 4) + (m & 7) * 2);
}

// Byte offset of (row c, K-chunk ch of 8 bf16) in a row-major tile of 128
// rows of 64 K (128-byte rows); chunk ch of row c sits at ch ^ (c/2 % 8).
__device__ __forceinline__ uint32_t nk_off(int c, int ch) {
  return (uint32_t)(c * 128 + ((ch ^ ((c >> 1) & 7)) << 4));
}

// One MFMA fragment (8 consecutive K of column `col0 + lane % 32`, K rows
// kk*16 + 8 (lane / 32) ..) of a K-major tile at LDS byte `base`.
__device__ __forceinline__ bf16x8 frag_km(uint32_t base, int kk, int col0, int lane) {
  const int krow = kk * 16 + 8 * (lane >> 5) + ((lane & 15) >> 2);
  const int col = col0 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (LDS_AS s16x4*)(uintptr_t)(base + km_off(krow, col)));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (LDS_AS s16x4*)(uintptr_t)(base + km_off(krow + 4, col)));
  const short v[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// One fragment of a row-major tile: row row0 + lane % 32, K kk*16 + 8 (lane/32) ..
__device__ __forceinline__ bf16x8 frag_nk(const uint8_t* smem_b, int kk, int row0, int lane) {
  const int r = row0 + (lane & 31);
  return *(const bf16x8*)(smem_b + nk_off(r, 2 * kk + (lane >> 5)));
}

__device__ __forceinline__ float sigmoidf_(float x) { return 1.f / (1.f + expf(-x)); }

template <int MODE, int EPI>
__global__ __launch_bounds__(kThreads, MODE == BWD_WGRAD ? 4 : 2) void ggemm_bwd_kernel(
    GemmBwdArgs p) {
  // ROWS: K = d or h, two stages so that a step's copies overlap the previous
  // step's MFMAs.  WGRAD: K = an expert's rows (often one or two steps) and a
  // 64 KB fp32 tile to store per workgroup; one stage and four workgroups per
  // CU overlap one workgroup's stores with the others' loads better than a
  // deeper ring would (measured: 143 against 168 us for a 512 MB gradient).
  constexpr int NST = MODE == BWD_WGRAD ? 1 : 2;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NST * kStage];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int MT = (p.M + kTile - 1) / kTile;

  // --- the tile --------------------------------------------------------
  int e, m0, c0, c_end, k_lo, k_hi;
  if constexpr (MODE == BWD_ROWS) {
    // tiles (row tile, M tile), M fastest; each XCD takes one contiguous run
    const int total = *p.tile_count * MT;
    const int per = (total + kXcds - 1) / kXcds;
    const int j = (int)(blockIdx.x / kXcds);
    if (j >= per) return;
    const int t = (int)(blockIdx.x % kXcds) * per + j;
    if (t >= total) return;
    const int rt = t / MT;
    m0 = (t % MT) * kTile;
    e = p.tile_expert[rt];
    c0 = p.tile_row0[rt];
    c_end = p.offsets[e + 1];
    k_lo = 0;
    k_hi = p.K;
  } else {
    const int NT = (p.N + kTile - 1) / kTile;
    const int t = xcd_tile(p.n_experts * MT * NT);
    if (t < 0) return;
    e = t / (MT * NT);
    const int r = t % (MT * NT);
    c0 = (r / MT) * kTile;
    m0 = (r % MT) * kTile;
    c_end = p.N;
    k_lo = p.offsets[e];
    k_hi = p.offsets[e + 1];
  }
  const uint16_t* A = p.A + (long long)e * p.strideA;
  const uint16_t* A2 = p.A2 ? p.A2 + (long long)e * p.strideA : nullptr;
  const int nsteps = (k_hi - k_lo + kBK - 1) / kBK;
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;

  // --- copies of one K-step into stage `st` -----------------------------
  // Wave w writes LDS kilobytes 4w .. 4w+3 of each operand's half-stage;
  // position p (16-byte chunk) of a K-major half is row p/16, physical chunk
  // p%16; of a row-major half, row p/8, physical chunk p%8.
  auto issue = [&](int step, int st) {
    const int kb = k_lo + step * kBK;
    const uint32_t sa = lds0 + st * kStage, sb = sa + kHalf;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int pos = (wave * 4 + q) * 64 + lane;
      const int kr = pos >> 4;
      const int m = m0 + (((pos & 15) ^ ((kr & 3) << 2)) << 3);
      const int k = kb + kr;
      const void* src = kZeroChunk;
      if (k < k_hi && m < p.M) {
        src = (A2 && k >= p.k_split) ? (const void*)(A2 + (long long)(k - p.k_split) * p.lda + m)
                                     : (const void*)(A + (long long)k * p.lda + m);
      }
      dma16(src, sa + (wave * 4 + q) * 1024);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int pos = (wave * 4 + q) * 64 + lane;
      const void* src = kZeroChunk;
      if constexpr (MODE == BWD_ROWS) {
        const int r = pos >> 3;
        const int ch = (pos & 7) ^ ((r >> 1) & 7);
        const int row = min(c0 + r, c_end - 1);  // rows past the segment: a valid row, never stored
        src = p.B + (long long)row * p.ldb + kb + ch * 8;
      } else {
        const int kr = pos >> 4;
        const int c = c0 + (((pos & 15) ^ ((kr & 3) << 2)) << 3);
        const int k = kb + kr;
        if (k < k_hi && c < p.N) src = p.B + (long long)k * p.ldb + c;
      }
      dma16(src, sb + (wave * 4 + q) * 1024);
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  if (NST == 2 && nsteps > 0) issue(0, 0);
  for (int g = 0; g < nsteps; ++g) {
    if constexpr (NST == 1) {
      issue(g, 0);
      wait_vm<0>();
    } else if (g + 1 < nsteps) {
      issue(g + 1, (g + 1) & 1);
      wait_vm<8>();
    } else {
      wait_vm<0>();
    }
    __syncthreads();
    const int st = NST == 2 ? (g & 1) : 0;
    const uint32_t sa = lds0 + st * kStage;
    const uint8_t* sb_ptr = smem + st * kStage + kHalf;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) af[i] = frag_km(sa, kk, wm * 64 + i * 32, lane);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if constexpr (MODE == BWD_ROWS)
          bfr[j] = frag_nk(sb_ptr, kk, wn * 64 + j * 32, lane);
        else
          bfr[j] = frag_km(sa + kHalf, kk, wn * 64 + j * 32, lane);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }

  // --- epilogue: lane holds D[m .. m+3][c] for m = base + 8 q + 4 (lane/32)
  {
    // The tile goes through LDS as fp32 in two halves of 64 rows c (the rows
    // of the waves with wn == half; 16-byte chunk j of row c at j ^ (c % 32)).
    // Then 32 lanes take one row c, four consecutive columns m each, so every
    // instruction covers two whole row segments: 512 bytes of fp32 output, or
    // the bf16 output with its mask / pre-activation reads, contiguous.  The
    // ring is free: the K loop ended with a barrier.
    float* st = (float*)smem;
    const int ch = lane & 31;
    const int m = m0 + ch * 4;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      if (wn == half) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int cl = j * 32 + (lane & 31);
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int cw = (wm * 64 + i * 32 + 8 * q + 4 * (lane >> 5)) >> 2;
              *(f32x4*)(st + cl * kTile + ((cw ^ (cl & 31)) << 2)) =
                  f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                        acc[i][j][4 * q + 3]};
            }
        }
      }
      __syncthreads();
#pragma unroll 4
      for (int rr = 0; rr < 8; ++rr) {
        const int cl = rr * 8 + wave * 2 + (lane >> 5);
        const int c = c0 + half * 64 + cl;
        if (c >= c_end || m >= p.M) continue;
        const f32x4 v = *(const f32x4*)(st + cl * kTile + ((ch ^ (cl & 31)) << 2));
        if constexpr (MODE == BWD_WGRAD) {
          // The weight gradients are written once and not read again by the
          // layer: non-temporal stores keep their half-gigabyte stream from
          // leaving the Infinity Cache full of dirty lines that the kernels
          // after it would have to write back.  The kernel itself runs at the
          // same speed (it meets the write-backs of the kernels before it);
          // a whole training step at T=8192, d=512, h=1024, n=256, k=4 gains
          // about 2 % (1008 against 1025 us).
          float* out = (c < p.c_split)
                           ? p.C + (long long)e * p.strideC + (long long)c * p.ldc + m
                           : p.C2 + (long long)e * p.strideC + (long long)(c - p.c_split) * p.ldc + m;
          __builtin_nontemporal_store(v, (f32x4*)out);
        } else if constexpr (EPI == BEPI_F32) {
          *(f32x4*)(p.C + (long long)c * p.ldc + m) = v;
        } else if constexpr (EPI == BEPI_RELU_MASK) {
          const uint2 hv = *(const uint2*)(p.aux_h + (long long)c * p.ldaux + m);
          const uint32_t hw[2] = {hv.x, hv.y};
          float f[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const uint16_t hb = (uint16_t)(hw[u >> 1] >> (16 * (u & 1)));
            f[u] = bf16_to_f32(hb) > 0.f ? v[u] : 0.f;
          }
          *(uint2*)(p.Cb + (long long)c * p.ldc + m) =
              make_uint2(bf16x2_bits(f[0], f[1]), bf16x2_bits(f[2], f[3]));
        } else {  // BEPI_SWIGLU: v = dhid; a, b saved in fp32
          const f32x4 a = *(const f32x4*)(p.aux_a + (long long)c * p.ldaux + m);
          const f32x4 b = *(const f32x4*)(p.aux_b + (long long)c * p.ldaux + m);
          float da[4], db[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const float s = sigmoidf_(a[u]);
            da[u] = v[u] * b[u] * s * (1.f + a[u] * (1.f - s));
            db[u] = v[u] * a[u] * s;
          }
          uint16_t* row = p.Cb + (long long)c * p.ldc;
          *(uint2*)(row + m) = make_uint2(bf16x2_bits(da[0], da[1]), bf16x2_bits(da[2], da[3]));
          *(uint2*)(row + p.c_split + m) =
              make_uint2(bf16x2_bits(db[0], db[1]), bf16x2_bits(db[2], db[3]));
        }
      }
      __syncthreads();
    }
  }
}

template <int MODE, int EPI>
hipError_t launch_t(const GemmBwdArgs& a, const char* name, hipStream_t s) {
  const int MT = (a.M + kTile - 1) / kTile;
  long long blocks;
  if (MODE == BWD_ROWS) {
    const long long total = (long long)a.max_tiles * MT;
    blocks = (total + kXcds - 1) / kXcds * kXcds;
  } else {
    const int NT = (a.N + kTile - 1) / kTile;
    const long long total = (long long)a.n_experts * MT * NT;
    blocks = (total + kXcds - 1) / kXcds * kXcds;
  }
  if (blocks <= 0) return hipSuccess;
  ProfScope ps(name, s);
  ggemm_bwd_kernel<MODE, EPI><<<dim3((unsigned)blocks), dim3(kThreads), 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_bwd(const GemmBwdArgs& a, int mode, int epi, const char* name,
                           hipStream_t s) {
  if (mode == BWD_ROWS) {
    switch (epi) {
      case BEPI_RELU_MASK: return launch_t<BWD_ROWS, BEPI_RELU_MASK>(a, name, s);
      case BEPI_SWIGLU: return launch_t<BWD_ROWS, BEPI_SWIGLU>(a, name, s);
      default: return launch_t<BWD_ROWS, BEPI_F32>(a, name, s);
    }
  }
  return launch_t<BWD_WGRAD, BEPI_F32>(a, name, s);
}

}  // namespace moe
