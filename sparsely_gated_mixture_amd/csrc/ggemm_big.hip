// Grouped GEMM of the expert FFNs with 256 x 256 tiles (gfx950,
// v_mfma_f32_32x32x16_bf16: bf16 operands, fp32 accumulation), for merged
// batches whose experts carry hundreds to thousands of rows.
//
// Same contract as the 128-row kernel (ggemm_bf16.hip): a device tile map
// lists M-tiles -- here 256 rows of one expert's merged batch -- and the work
// items are (M-tile, N-tile) pairs; W[e] = [N, K] (out x in) and X = [rows,
// K], both streaming along K; epilogues ReLU(+bias) -> bf16, SwiGLU -> bf16,
// identity(+bias) -> fp32.
//
// What differs is the shape of the work per compute unit:
//  * one 4-wave workgroup per CU (one wave per SIMD), each wave a 128 x 128
//    block of the 256 x 256 tile with its 256 fp32 accumulators in the
//    accumulation registers: per 16-wide K slice a wave reads 8 LDS
//    fragments for 16 MFMAs (half a fragment per MFMA), and the tile reuses
//    each weight row over 256 token rows;
//  * the operands reach LDS through registers: each K-step of 64 (32 KB per
//    operand) is loaded two steps ahead into one of two register sets (buffer
//    loads, 16 per thread), then written to one of two LDS stages, so two
//    steps' loads (128 KB per CU) are in flight while a step computes;
//  * the load cursor runs across tile boundaries, so the next tile's first
//    steps load while this tile finishes and stores;
//  * loads never leave their operand: each buffer descriptor spans the
//    tile's rows only (the segment's live rows, the weight rows below N), and
//    an out-of-range offset returns zeros without a memory access -- rows
//    past a segment's end, columns past N, chunks past K and the extra step
//    of an odd step count all read as zeros;
//  * LDS rows are 128 bytes (8 chunks of 16 bytes), chunk c of row r at
//    position c ^ ((r >> 1) & 7), so the fragment reads of 16 consecutive
//    rows hit 16 distinct bank groups.
// The MFMA computes D = W . X^T (weights as the A operand), so each lane ends
// with 4 consecutive output columns of each of its rows.
// SwiGLU: a tile's 256 weight rows are 128 columns of W1 and the same 128
// columns of W3, ordered so that each wave holds 64 columns of both and each
// lane the matching pairs: the epilogue forms silu(g) * u in registers.
#include <math.h>

#include "common.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kBM = kBigBM;    // rows per M-tile (the big tile map's granularity)
constexpr int kBK = 64;        // K per step
constexpr int kRowB = 128;     // LDS bytes per row and step (kBK bf16)
constexpr int kTileB = 256 * kRowB;  // one operand's 32 KB per step
constexpr int kStage = 2 * kTileB;   // 64 KB per LDS stage
constexpr int kThreads = 256;
constexpr int kGroupM = 4;           // M-tiles per group of the work order
// A buffer offset this large lies beyond every descriptor's range: the load
// returns zeros.
constexpr int kOutOfRange = 0x40000000;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int swz(int r, int c) { return (c ^ ((r >> 1) & 7)) << 4; }

// A buffer descriptor over `bytes` bytes from `base` (raw, 32-bit data
// format: plain byte addressing with a range check).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, long long bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           (int)min(bytes, (long long)kOutOfRange), 0x00020000);
}

// The loads of one step: thread t moves chunk (t & 7) of tile rows
// (t >> 3) + 32 i, i < 8, of each operand.  Activation row r of the tile is
// row row0 + r of X; weight row r is a column of W1 or W3 (see col_of).
struct Cursor {
  __amdgpu_buffer_rsrc_t xr, wr1, wr3;
  int tile;  // tile the cursor is in (index into this workgroup's list)
  int k;     // K-step within it
};

template <int EPI>
struct Shape {
  static constexpr bool kSwiglu = EPI == EPI_SWIGLU_BF16;
  // Output columns per tile (SwiGLU: 128 columns of W1 and of W3).
  static constexpr int kCols = kSwiglu ? 128 : 256;
  // Tile weight row r = lr + 32 i: its matrix (0: W1, 1: W3) and its column
  // offset from the tile's first column.  SwiGLU: rows [128 w, 128 w + 64)
  // are W1 columns 64 w + (r % 64), the next 64 rows the same W3 columns.
  static __device__ __forceinline__ int matrix(int i) { return kSwiglu ? (i >> 1) & 1 : 0; }
  static __device__ __forceinline__ int col(int i) {
    return kSwiglu ? (i >> 2) * 64 + (i & 1) * 32 : i * 32;
  }
};

template <int EPI, bool HAS_BIAS>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void
ggemm_big_kernel(const GemmBf16Args p) {
  using S = Shape<EPI>;
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  __shared__ int4 meta[kMaxTilesPerWG];  // per tile: expert, first row, end row, first column
  // The kernel keeps its accumulators in the accumulation registers; telling
  // the compiler that it uses them keeps every MFMA in that form.
  asm volatile("" ::: "a0");

  // This workgroup's tiles: XCD x owns tiles [x*per, (x+1)*per); its
  // workgroups take every wpx-th of them.
  const int nN = (p.N + S::kCols - 1) / S::kCols;
  const int total = *p.tile_count * nN;
  const int per = (total + kXcds - 1) / kXcds;
  const int xcd = (int)(blockIdx.x % kXcds), slot = (int)(blockIdx.x / kXcds);
  const int wpx = (int)(gridDim.x / kXcds);
  const int first = xcd * per + slot;
  const int last = min(total, (xcd + 1) * per);
  const int ntiles = first < last ? (last - first + wpx - 1) / wpx : 0;
  if (ntiles == 0) return;
  const int tid = threadIdx.x;
  // Item L -> (M-tile, N-tile) in groups of kGroupM consecutive M-tiles:
  // within a group the M-tile varies fastest, so the 32 workgroups of an XCD
  // work on about 4 M-tiles x 8 N-tiles at a time (their activation and
  // weight slices of a K-step fit the XCD's L2 many steps over).
  const int mtiles = *p.tile_count;
  for (int t = tid; t < ntiles; t += kThreads) {
    const int L = first + t * wpx;
    const int grp = L / (kGroupM * nN), r = L % (kGroupM * nN);
    const int gsz = min(kGroupM, mtiles - grp * kGroupM);
    const int mt = grp * kGroupM + r % gsz, nt = r / gsz;
    const int e = p.tile_expert[mt];
    meta[t] = make_int4(e, p.tile_row0[mt], p.offsets[e + 1], nt * S::kCols);
  }
  __syncthreads();

  const int K = p.K;
  const int nk = (K + kBK - 1) / kBK;
  const int nk2 = (nk + 1) & ~1;  // steps per tile: an odd count runs one on zeros
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int lc = tid & 7, lr = tid >> 3;
  const int lr32 = lane & 31, lh = lane >> 5;
  const long long xrow = p.lda * 2, wrow = (long long)K * 2;  // bytes per row
  const int vx = lr * (int)xrow + lc * 16, vw = lr * (int)wrow + lc * 16;

  // ---- load cursor ------------------------------------------------------
  Cursor cur;
  auto set_tile = [&](int ti) {
    const int4 m = meta[ti];
    const int e = __builtin_amdgcn_readfirstlane(m.x);
    const int row0 = __builtin_amdgcn_readfirstlane(m.y);
    const int end = __builtin_amdgcn_readfirstlane(m.z);
    const int col0 = __builtin_amdgcn_readfirstlane(m.w);
    const int live = min(kBM, end - row0);
    cur.xr = rsrc(p.A + (long long)row0 * p.lda, (long long)live * xrow);
    const uint8_t* w1 = (const uint8_t*)p.B1 + (long long)e * p.strideB;
    const int wlive = min(S::kSwiglu ? 128 : 256, p.N - col0);
    cur.wr1 = rsrc(w1 + (long long)col0 * wrow, (long long)wlive * wrow);
    if constexpr (S::kSwiglu) {
      const uint8_t* w3 = (const uint8_t*)p.B3 + (long long)e * p.strideB;
      cur.wr3 = rsrc(w3 + (long long)col0 * wrow, (long long)wlive * wrow);
    }
  };
  cur.tile = 0;
  cur.k = 0;
  set_tile(0);
  // Quarter q of the loads of step (cur.tile, cur.k) into R: activation rows
  // (q < 2) or weight rows (q >= 2) 32 i + lr for i = 4 (q % 2) .. + 3.  Past
  // the last tile, and at steps past K, the offsets leave the descriptors'
  // ranges and the loads return zeros.  advance() moves the cursor on.
  int oor = 0, so = 0;
  auto gload_q = [&](u32x4 (&R)[16], int q) {
    if (q == 0) {
      const int k = cur.k;
      const bool live = cur.tile < ntiles && k < nk;
      // chunks past K in the last step read as zeros (K is a multiple of 8)
      const bool kin = k * kBK + lc * 8 < K;
      oor = (live && kin) ? 0 : kOutOfRange;
      so = k * 128;
    }
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int i = (q & 1) * 4 + ii;
      if (q < 2) {
        R[i] = __builtin_amdgcn_raw_buffer_load_b128(cur.xr, vx + i * 32 * (int)xrow + oor, so, 0);
      } else {
        const int vo = vw + S::col(i) * (int)wrow + oor;
        R[8 + i] =
            __builtin_amdgcn_raw_buffer_load_b128(S::matrix(i) ? cur.wr3 : cur.wr1, vo, so, 0);
      }
    }
  };
  auto advance = [&]() {
    if (++cur.k == nk2) {
      cur.k = 0;
      if (++cur.tile < ntiles) set_tile(cur.tile);
    }
  };
  auto gload = [&](u32x4 (&R)[16]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) gload_q(R, q);
    advance();
  };
  const int wofs = lr * kRowB + swz(lr, lc);  // rows lr + 32 i share lr's swizzle
  // Rows 32 i + lr, i = 4 h .. 4 h + 3, of both operands into `stage`.
  auto swrite_h = [&](int stage, const u32x4 (&R)[16], int h) {
    uint8_t* base = smem + stage * kStage + wofs;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int i = h * 4 + ii;
      *(u32x4*)(base + i * 32 * kRowB) = R[i];
      *(u32x4*)(base + kTileB + i * 32 * kRowB) = R[8 + i];
    }
  };
  auto swrite = [&](int stage, const u32x4 (&R)[16]) {
    swrite_h(stage, R, 0);
    swrite_h(stage, R, 1);
  };

  // ---- compute ------------------------------------------------------------
  f32x16 acc[4][4];
  // Fragments of one 16-wide K slice: weight rows wn*128 + b*32 + lr32 and
  // activation rows wm*128 + j*32 + lr32 (all sharing lr32's swizzle), chunk
  // 2 kk + lh.
  const int fs = (lr32 >> 1) & 7, fo = lr32 * kRowB;
  auto rdfrag = [&](const uint8_t* st, int kk, bf16x8 (&wf)[4], bf16x8 (&xf)[4]) {
    const int o = fo + (((2 * kk + lh) ^ fs) << 4);
#pragma unroll
    for (int b = 0; b < 4; ++b)
      wf[b] = *(const bf16x8*)(st + kTileB + (wn * 128 + b * 32) * kRowB + o);
#pragma unroll
    for (int j = 0; j < 4; ++j) xf[j] = *(const bf16x8*)(st + (wm * 128 + j * 32) * kRowB + o);
  };
  auto mfmas = [&](const bf16x8 (&wf)[4], const bf16x8 (&xf)[4]) {
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[b][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[b], xf[j], acc[b][j], 0, 0, 0);
  };
  // One K-step from LDS stage `stage`: load the step two ahead into Rl,
  // compute, write Rw (the next step, loaded a step ago) into the other
  // stage, barrier.
  // One K-step from LDS stage `stage`, four 16-wide K slices.  Spread among
  // each slice's 16 MFMAs: a quarter of the loads of the step two ahead
  // (into Rl), the next slice's 8 fragment reads, and in slices 2 and 3 half
  // of the LDS writes of the next step (Rw, loaded a step ago) into the other
  // stage -- every wave finished reading that stage before the previous
  // barrier.  Issued back to back, the loads would hold up the MFMAs behind
  // them (in-order issue); spread out, the copies and the MFMAs overlap.
  auto group = [&](bool writes, bool reads) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);             // a load
      if (writes) __builtin_amdgcn_sched_group_barrier(0x200, 2, 0);  // two LDS writes
      if (reads) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // two LDS reads
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);             // four MFMAs
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  auto step = [&](int stage, u32x4 (&Rl)[16], const u32x4 (&Rw)[16]) {
    const uint8_t* st = smem + stage * kStage;
    bf16x8 wa[4], xa[4], wb[4], xb[4];
    rdfrag(st, 0, wa, xa);
    gload_q(Rl, 0);
    rdfrag(st, 1, wb, xb);
    mfmas(wa, xa);
    group(false, true);
    gload_q(Rl, 1);
    rdfrag(st, 2, wa, xa);
    mfmas(wb, xb);
    group(false, true);
    gload_q(Rl, 2);
    swrite_h(stage ^ 1, Rw, 0);
    rdfrag(st, 3, wb, xb);
    mfmas(wa, xa);
    group(true, true);
    gload_q(Rl, 3);
    advance();
    swrite_h(stage ^ 1, Rw, 1);
    mfmas(wb, xb);
    group(true, false);
    __syncthreads();
  };
  u32x4 R0[16], R1[16];
  gload(R0);
  gload(R1);
  swrite(0, R0);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int4 m = meta[t];
    const int e = __builtin_amdgcn_readfirstlane(m.x);
    const int row0 = __builtin_amdgcn_readfirstlane(m.y);
    const int end = __builtin_amdgcn_readfirstlane(m.z);
    const int col0 = __builtin_amdgcn_readfirstlane(m.w);
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[b][j][v] = 0.f;
    for (int g = 0; g < nk2; g += 2) {
      step(0, R0, R1);
      step(1, R1, R0);
    }

    // Epilogue.  D[n][m]: lane holds token row m = lr32 of each 32 x 32
    // block and weight rows n = 8 (v / 4) + 4 lh + v % 4.
    const float* bias = HAS_BIAS ? p.bias + (long long)e * p.N : nullptr;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int gr = row0 + wm * 128 + j * 32 + lr32;
      if (gr >= end) continue;
      if constexpr (EPI == EPI_SWIGLU_BF16) {
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int gc = col0 + wn * 64 + b * 32 + 8 * q + 4 * lh;
            if (gc >= p.N) continue;
            float f[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const float gv = acc[b][j][4 * q + v], uv = acc[b + 2][j][4 * q + v];
              f[v] = gv / (1.f + expf(-gv)) * uv;
            }
            *(uint2*)((uint16_t*)p.C + (long long)gr * p.ldc + gc) =
                make_uint2(bf16x2_bits(f[0], f[1]), bf16x2_bits(f[2], f[3]));
          }
      } else {
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int gc = col0 + wn * 128 + b * 32 + 8 * q + 4 * lh;
            if (gc >= p.N) continue;
            float f[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              f[v] = acc[b][j][4 * q + v];
              if constexpr (HAS_BIAS) f[v] += bias[gc + v];
              if constexpr (EPI == EPI_RELU_BF16) f[v] = fmaxf(f[v], 0.f);
            }
            if constexpr (EPI == EPI_IDENT_F32)
              *(f32x4*)((float*)p.C + (long long)gr * p.ldc + gc) = f32x4{f[0], f[1], f[2], f[3]};
            else
              *(uint2*)((uint16_t*)p.C + (long long)gr * p.ldc + gc) =
                  make_uint2(bf16x2_bits(f[0], f[1]), bf16x2_bits(f[2], f[3]));
          }
      }
    }
  }
}

template <int EPI, bool HAS_BIAS>
hipError_t launch_t(const GemmBf16Args& a, hipStream_t s) {
  using S = Shape<EPI>;
  const int nN = (a.N + S::kCols - 1) / S::kCols;
  const long long max_total = (long long)a.max_mtiles * nN;
  if (max_total <= 0) return hipSuccess;
  long long grid = (long long)a.num_cus / kXcds * kXcds;
  if (grid < kXcds) grid = kXcds;
  const long long per = (max_total + kXcds - 1) / kXcds;
  while ((per + grid / kXcds - 1) / (grid / kXcds) > kMaxTilesPerWG) grid += kXcds;
  static const char* const kNames[3] = {"ggemm_big_relu", "ggemm_big_swiglu", "ggemm_big_out"};
  ProfScope ps(a.prof_name ? a.prof_name : kNames[EPI], s);
  const void* fn = (const void*)ggemm_big_kernel<EPI, HAS_BIAS>;
  hipError_t err = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, 2 * kStage);
  if (err != hipSuccess) return err;
  ggemm_big_kernel<EPI, HAS_BIAS><<<dim3((unsigned)grid), dim3(kThreads), 2 * kStage, s>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_big(const GemmBf16Args& a, int epi, hipStream_t s) {
  const bool bias = a.bias != nullptr;
  switch (epi) {
    case EPI_RELU_BF16:
      return bias ? launch_t<EPI_RELU_BF16, true>(a, s) : launch_t<EPI_RELU_BF16, false>(a, s);
    case EPI_SWIGLU_BF16:
      return launch_t<EPI_SWIGLU_BF16, false>(a, s);
    default:
      return bias ? launch_t<EPI_IDENT_F32, true>(a, s) : launch_t<EPI_IDENT_F32, false>(a, s);
  }
}

}  // namespace moe
