// Grouped GEMM of the expert FFNs with 256 x 256 tiles (gfx950,
// v_mfma_f32_32x32x16_bf16: bf16 operands, fp32 accumulation), for merged
// batches whose experts carry hundreds to thousands of rows.
//
// Same contract as the 128-row kernel (ggemm_bf16.hip): a device tile map
// lists M-tiles -- here 256 rows of one expert's merged batch -- and the work
// items are (M-tile, N-tile) pairs; W[e] = [N, K] (out x in) and X = [rows,
// K], both streaming along K; epilogues ReLU(+bias) -> bf16, SwiGLU -> bf16,
// identity(+bias) -> fp32 or bf16.
//
// What differs is the shape of the work per compute unit:
//  * one 4-wave workgroup per CU (one wave per SIMD), each wave a 128 x 128
//    block of the 256 x 256 tile with its 256 fp32 accumulators in the
//    accumulation registers: per 16-wide K slice a wave reads 8 LDS
//    fragments for 16 MFMAs (half a fragment per MFMA), and the tile reuses
//    each weight row over 256 token rows;
//  * the operands go from memory straight into LDS (buffer loads with the
//    LDS destination bit, no registers in between, issued by the copy
//    helper of lds_dma.h): two LDS stages of one 64-wide K-step (32 KB per
//    operand); while a step computes from one stage, its 16 copies per wave
//    fill the other with the next step.  The copies are issued an eighth at
//    a time between the step's first 32 MFMAs, so the matrix unit keeps busy
//    while the copy instructions issue; each step ends with the wave's
//    copies landed (an explicit vmcnt wait) and one workgroup barrier;
//  * the copy cursor runs across tile boundaries, so the next tile's first
//    step loads while this tile finishes and stores;
//  * copies never leave their operand: each buffer descriptor spans the
//    tile's rows only (the segment's live rows, the weight rows below N), and
//    an out-of-range offset returns zeros without a memory access -- rows
//    past a segment's end, columns past N and chunks past K all read as
//    zeros; past the last tile the descriptors span nothing;
//  * LDS rows are 128 bytes (8 chunks of 16 bytes), chunk c of row r at
//    position c ^ ((r >> 1) & 7), so the fragment reads of 16 consecutive
//    rows hit 16 distinct bank groups.  A copy moves 8 rows x 128 bytes into
//    1 KB of LDS, lane i to bytes 16 i; lane i therefore reads the logical
//    chunk that belongs at physical chunk i % 8 of its row;
//  * work order: items in groups of kBigGroupM M-tiles (M fastest), cut into
//    chunks of one XCD's workgroup count and dealt to the 8 XCDs in turn, so
//    the XCDs work on neighbouring chunks -- mostly the same expert -- at the
//    same time and its weights are fetched from HBM once for all of them
//    (the repeats hit the Infinity Cache), while within an XCD the chunk's
//    ~4 M-tiles x 8 N-tiles share their K-slices in the XCD's L2.
// The MFMA computes D = W . X^T (weights as the A operand), so each lane ends
// with 4 consecutive output columns of each of its rows.
// SwiGLU: a tile's 256 weight rows are 128 columns of W1 and the same 128
// columns of W3, ordered so that each wave holds 64 columns of both and each
// lane the matching pairs: the epilogue forms silu(g) * u in registers.
// FP8 weights (E4M3 codes in the packed layout of moe_pack_fp8_weights: row
// pairs, 128 bytes per pair and 64-wide K block, then one fp32 scale per
// row): a weight row takes 64 bytes of LDS per step (16 codes = one 16-wide
// K slice per 16-byte chunk, chunk c at c ^ ((row >> 1) & 3)), so a step's
// weights are 16 KB in 4 copies per wave; each lane reads its 8 codes of a
// slice and widens them to bf16 in registers, and the epilogue multiplies
// each output column by its row scale.
#include <math.h>

#include "common.h"
#include "launch.h"
#include "lds_dma.h"

namespace moe {
namespace {

constexpr int kBM = kBigBM;    // rows per M-tile (the big tile map's granularity)
constexpr int kBK = 64;        // K per step
constexpr int kRowB = 128;     // LDS bytes per row and step (kBK bf16)
constexpr int kTileB = 256 * kRowB;  // the activations' 32 KB per step
constexpr int kThreads = 256;
// A buffer offset this large lies beyond every descriptor's range: the load
// returns zeros.
constexpr int kOutOfRange = 0x40000000;


// Weight rows in LDS: bf16 128 bytes per row and step, FP8 64.
template <bool FP8>
struct WRows {
  static constexpr int kRowB = FP8 ? 64 : 128;
  static constexpr int kTileB = 256 * kRowB;      // a step's weights
  static constexpr int kStage = ::moe::kTileB + kTileB;  // activations + weights
  static constexpr int kCopies = FP8 ? 4 : 8;     // weight copies per wave and step
};

template <int EPI>
struct Shape {
  static constexpr bool kSwiglu = EPI == EPI_SWIGLU_BF16;
  // Output columns per tile (SwiGLU: 128 columns of W1 and of W3).
  static constexpr int kCols = kSwiglu ? 128 : 256;
  // Tile weight rows [32 i, 32 i + 32): their matrix (0: W1, 1: W3) and
  // column offset from the tile's first column.  SwiGLU: rows [128 w, 128 w
  // + 64) are W1 columns 64 w + (r % 64), the next 64 rows the same W3
  // columns.
  static __device__ __forceinline__ int matrix(int i) { return kSwiglu ? (i >> 1) & 1 : 0; }
  static __device__ __forceinline__ int col(int i) {
    return kSwiglu ? (i >> 2) * 64 + (i & 1) * 32 : i * 32;
  }
};

template <int EPI, bool HAS_BIAS, bool FP8>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void
ggemm_big_kernel(const GemmBf16Args p) {
  using S = Shape<EPI>;
  using W = WRows<FP8>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * W::kStage];
  __shared__ int4 meta[kMaxTilesPerWG];  // per tile: expert, first row, end row, first column
  // The kernel keeps its accumulators in the accumulation registers; telling
  // the compiler that it uses them keeps every MFMA in that form.
  asm volatile("" ::: "a0");

  // This workgroup's items: chunks of wpx consecutive items (wpx = the
  // workgroups per XCD) go to the XCDs in turn, chunk c to XCD c % 8; slot s
  // of an XCD takes item s of each of its chunks.
  const int nN = (p.N + S::kCols - 1) / S::kCols;
  const int total = *p.tile_count * nN;
  // Side by side with the 128-row GEMM (this kernel on the caller's stream,
  // the other on a side stream): the lowest-numbered workgroups return at
  // once and the top `used` ones work, renumbered from 0 (on the XCD their
  // hardware number gives: grid and used are multiples of kXcds).  Measured
  // on MI355X: with the returning workgroups numbered after the working ones
  // instead, the kernel on the side stream did not start until this one
  // ended; the side kernel's own returning workgroups numbered last are
  // harmless, numbered first they held it back the same way.
  const int used = gemm_used_grid(p, total);
  const int bid = (int)blockIdx.x - ((int)gridDim.x - used);
  if (bid < 0) return;
  const int xcd = bid % kXcds, slot = bid / kXcds;
  const int wpx = used / kXcds;
  const int nchunks = (total + wpx - 1) / wpx;
  int ntiles = xcd < nchunks ? (nchunks - xcd + kXcds - 1) / kXcds : 0;
  if (ntiles > 0 && xcd + kXcds * (ntiles - 1) == nchunks - 1 &&
      (nchunks - 1) * wpx + slot >= total)
    --ntiles;  // this slot is past the end of the last, partial chunk
  if (ntiles == 0) return;
  const int tid = threadIdx.x;
  // Item L -> (M-tile, N-tile) in groups of kBigGroupM consecutive M-tiles,
  // the M-tile varying fastest within a group.
  const int mtiles = *p.tile_count;
  for (int t = tid; t < ntiles; t += kThreads) {
    const int L = (t * kXcds + xcd) * wpx + slot;
    const int grp = L / (kBigGroupM * nN), r = L % (kBigGroupM * nN);
    const int gsz = min(kBigGroupM, mtiles - grp * kBigGroupM);
    const int mt = grp * kBigGroupM + r % gsz, nt = r / gsz;
    const int e = p.tile_expert[mt];
    meta[t] = make_int4(e, p.tile_row0[mt], p.offsets[e + 1], nt * S::kCols);
  }
  __syncthreads();

  const int K = p.K;
  const int nk = (K + kBK - 1) / kBK;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int lr32 = lane & 31, lh = lane >> 5;

  // ---- copy cursor ------------------------------------------------------
  // Activations (and bf16 weights): copy j (0..7) moves tile rows 32 j + 8
  // wave + lane / 8 into LDS bytes [(4 j + wave) * 1024, +1024) of the
  // operand's part of a stage: physical chunk lane % 8 of its row, which
  // holds logical chunk (lane % 8) ^ ((row >> 1) & 7) -- the same for every
  // j, since 32 j leaves bits 1..3 of the row alone.
  // FP8 weights: copy j (0..3) moves tile rows 64 j + 16 wave + lane / 4
  // (64-byte LDS rows): physical chunk lane % 4, logical chunk (lane % 4) ^
  // ((row >> 1) & 3) = (lane % 4) ^ ((lane / 8) % 4); those rows are rows 16
  // (wave % 2) + lane / 4 of the 32-row weight blocks 2 j + wave / 2.
  const int lchunk = (lane & 7) ^ ((4 * wave + (lane >> 4)) & 7);
  const int lrow = 8 * wave + (lane >> 3);  // row within each 32-row block
  const long long xrowb = p.lda * 2;
  const long long wrow = (long long)K * 2;  // bf16 weight row; FP8: bytes per row pair
  const int xoff0 = lrow * (int)xrowb + lchunk * 16;
  int woff0;
  if constexpr (FP8) {
    const int rin = 16 * (wave & 1) + (lane >> 2);
    const int lc8 = (lane & 3) ^ ((lane >> 3) & 3);
    woff0 = (rin >> 1) * (int)wrow + (rin & 1) * 64 + lc8 * 16;
  } else {
    woff0 = lrow * (int)wrow + lchunk * 16;
  }
  rsrc_t xr, wr1, wr3;
  // Byte offset of this lane's row in activation copy q: its row within the
  // tile's descriptor, or (rows through the permutation) its token's row in
  // the whole of A, past the descriptor for rows past the segment.
  int xo[8];
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
  int ct = 0, ck = 0;  // the cursor: tile, K-step
  auto set_tile = [&](int ti) {
    const int4 m = meta[ti];
    const int e = __builtin_amdgcn_readfirstlane(m.x);
    const int row0 = __builtin_amdgcn_readfirstlane(m.y);
    const int end = __builtin_amdgcn_readfirstlane(m.z);
    const int col0 = __builtin_amdgcn_readfirstlane(m.w);
    if (p.row_token) {
      xr = buffer_rsrc(p.A, (long long)p.a_rows * xrowb);
      const int n = min(end, p.row_token_n);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int base = row0 + 32 * q + 8 * wave;
        const int tok = row_token8(p.row_token, base, n, lane);
        xo[q] = base + (lane >> 3) < end ? tok * (int)xrowb + lchunk * 16 : kOutOfRange;
      }
    } else {
      xr = buffer_rsrc(p.A + (long long)row0 * p.lda, (long long)min(kBM, end - row0) * xrowb);
#pragma unroll
      for (int q = 0; q < 8; ++q) xo[q] = xoff0 + q * 32 * (int)xrowb;
    }
    const int wlive = min(S::kCols, p.N - col0);
    // bf16: rows [col0, col0 + wlive); FP8: the row pairs holding them (col0 is even)
    const long long wbase = FP8 ? (long long)(col0 >> 1) * wrow : (long long)col0 * wrow;
    const long long wbytes = FP8 ? (long long)((wlive + 1) >> 1) * wrow : (long long)wlive * wrow;
    const uint8_t* w1 = (const uint8_t*)p.B1 + (long long)e * p.strideB;
    wr1 = buffer_rsrc(w1 + wbase, wbytes);
    if constexpr (S::kSwiglu) {
      const uint8_t* w3 = (const uint8_t*)p.B3 + (long long)e * p.strideB;
      wr3 = buffer_rsrc(w3 + wbase, wbytes);
    } else {
      wr3 = wr1;
    }
  };
  set_tile(0);
  auto advance = [&]() {
    if (++ck == nk) {
      ck = 0;
      if (++ct < ntiles) {
        set_tile(ct);
      } else {  // past the last tile: descriptors that span nothing
        xr = buffer_rsrc(p.A, 0);
        wr1 = buffer_rsrc(p.B1, 0);
        wr3 = wr1;
      }
    }
  };
  // Copy q of the cursor's step into stage st: q < 8 the activation rows of
  // block q, else weight copy q - 8.  FP8 weights need K % 64 == 0 (no tail).
  auto copy = [&](int st, int q) {
    const uint32_t sb = lds0 + st * W::kStage + wave * 1024;
    const int koff = ck * 128;
    const int oor = ck * kBK + lchunk * 8 < K ? 0 : kOutOfRange;
    if (q < 8) {
      bdma16(xr, (int)((uint32_t)xo[q] + (uint32_t)oor), koff, sb + q * 4096);
    } else {
      const int j = q - 8;
      const int blk = FP8 ? 2 * j + (wave >> 1) : j;  // 32-row weight block
      const int wo = FP8 ? woff0 + (S::col(blk) >> 1) * (int)wrow
                         : woff0 + S::col(blk) * (int)wrow + oor;
      bdma16(S::matrix(blk) ? wr3 : wr1, wo, koff, sb + kTileB + j * 4096);
    }
  };
  constexpr int kCopies = 8 + W::kCopies;     // per wave and step

  // ---- compute ------------------------------------------------------------
  f32x16 acc[4][4];
  // Fragments of one 16-wide K slice: weight rows wn*128 + b*32 + lr32 and
  // activation rows wm*128 + j*32 + lr32 (all sharing lr32's swizzle), chunk
  // 2 kk + lh (FP8 weights: the lh half of 16-byte chunk kk).
  const int fs = (lr32 >> 1) & 7, fo = lr32 * kRowB;
  auto frag_off = [&](int kk) { return fo + (((2 * kk + lh) ^ fs) << 4); };
  // FP8: this lane's 8 codes of weight block b in slice kk.
  auto wraw = [&](const uint8_t* st, int kk, int b) -> uint2 {
    const int r = wn * 128 + b * 32 + lr32;
    return *(const uint2*)(st + kTileB + r * W::kRowB + ((kk ^ ((lr32 >> 1) & 3)) << 4) +
                           lh * 8);
  };
  auto wfrag = [&](const uint8_t* st, int kk, int b) -> bf16x8 {
    if constexpr (FP8)
      return e4m3x8_to_bf16(wraw(st, kk, b));
    else
      return *(const bf16x8*)(st + kTileB + (wn * 128 + b * 32) * kRowB + frag_off(kk));
  };
  auto xfrag = [&](const uint8_t* st, int kk, int j) -> bf16x8 {
    return *(const bf16x8*)(st + (wm * 128 + j * 32) * kRowB + frag_off(kk));
  };
  auto rdfrag = [&](const uint8_t* st, int kk, bf16x8 (&wf)[4], bf16x8 (&xf)[4]) {
#pragma unroll
    for (int b = 0; b < 4; ++b) wf[b] = wfrag(st, kk, b);
#pragma unroll
    for (int j = 0; j < 4; ++j) xf[j] = xfrag(st, kk, j);
  };
  auto mfma_row = [&](int b, const bf16x8 (&wf)[4], const bf16x8 (&xf)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[b][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[b], xf[j], acc[b][j], 0, 0, 0);
  };
  auto mfmas = [&](const bf16x8 (&wf)[4], const bf16x8 (&xf)[4]) {
#pragma unroll
    for (int b = 0; b < 4; ++b) mfma_row(b, wf, xf);
  };
  // Spread among a slice's 16 MFMAs: the next slice's 8 fragment reads
  // (FP8: the reads in the first half, then the 16 widening instructions of
  // the codes they brought, so the widening waits on reads issued 8 MFMAs
  // earlier).
  auto group = [&](bool reads) {
    if (FP8 && reads) {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // four LDS reads
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);  // four MFMAs
      }
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);  // eight VALU (widening)
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);  // four MFMAs
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (reads) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // two LDS reads
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);             // four MFMAs
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // One K-step from stage `stage`, four 16-wide K slices.  Slices 0 and 1
  // run in four rounds each: an eighth of the next step's copies (into the
  // other stage, which every wave finished reading before the previous
  // barrier), the next slice's four weight and four activation fragment
  // reads, and one row of four MFMAs, pinned in that order.  Spread this way
  // the copies keep the LDS command queue from filling (issued four at a
  // time in slice 0 alone they measured 6-10 % slower, all over the four
  // slices slower still: the last copies land too late).  Slices 2 and 3
  // interleave their MFMAs with the next slice's reads.  The step ends when
  // this wave's copies have landed and all waves reach the barrier.  FP8:
  // the codes read in a slice's rounds are widened right after them.
  auto step = [&](int stage) {
    const uint8_t* st = smem + stage * W::kStage;
    bf16x8 wa[4], xa[4], wb[4], xb[4];
    uint2 rw[4];  // FP8: codes of the slice read in the rounds
    rdfrag(st, 0, wa, xa);
    __builtin_amdgcn_sched_barrier(0);
    auto rounds = [&](int r0, int kk, const bf16x8(&wc)[4], const bf16x8(&xc)[4],
                      bf16x8(&wn)[4], bf16x8(&xn)[4]) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
#pragma unroll
        for (int c = (r0 + q) * kCopies / 8; c < (r0 + q + 1) * kCopies / 8; ++c)
          copy(stage ^ 1, c);
        if constexpr (FP8)
          rw[q] = wraw(st, kk, q);
        else
          wn[q] = wfrag(st, kk, q);
        xn[q] = xfrag(st, kk, q);
        mfma_row(q, wc, xc);
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (FP8) {
#pragma unroll
        for (int q = 0; q < 4; ++q) wn[q] = e4m3x8_to_bf16(rw[q]);
      }
    };
    rounds(0, 1, wa, xa, wb, xb);  // slice 0; reads slice 1
    rounds(4, 2, wb, xb, wa, xa);  // slice 1; reads slice 2
    advance();
    rdfrag(st, 3, wb, xb);
    mfmas(wa, xa);
    group(true);
    mfmas(wb, xb);
    group(false);
    wait_vm<0>();
    __syncthreads();
  };
#pragma unroll
  for (int q = 0; q < kCopies; ++q) copy(0, q);
  advance();
  wait_vm<0>();
  __syncthreads();

  int stage = 0;
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
    for (int g = 0; g < nk; ++g) {
      step(stage);
      stage ^= 1;
    }

    // Epilogue.  D[n][m]: lane holds token row m = lr32 of each 32 x 32
    // block and weight rows n = 8 (v / 4) + 4 lh + v % 4.  FP8: the row
    // scales follow each expert's codes.
    const float* bias = HAS_BIAS ? p.bias + (long long)e * p.N : nullptr;
    const float* sc1 = nullptr;
    const float* sc3 = nullptr;
    if constexpr (FP8) {
      sc1 = (const float*)((const uint8_t*)p.B1 + (long long)e * p.strideB + (long long)p.N * K);
      if constexpr (S::kSwiglu)
        sc3 = (const float*)((const uint8_t*)p.B3 + (long long)e * p.strideB + (long long)p.N * K);
    }
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
            f32x4 s1 = {1.f, 1.f, 1.f, 1.f}, s3 = {1.f, 1.f, 1.f, 1.f};
            if constexpr (FP8) {
              s1 = *(const f32x4*)(sc1 + gc);
              s3 = *(const f32x4*)(sc3 + gc);
            }
            float f[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const float gv = acc[b][j][4 * q + v] * s1[v], uv = acc[b + 2][j][4 * q + v] * s3[v];
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
            f32x4 s1 = {1.f, 1.f, 1.f, 1.f};
            if constexpr (FP8) s1 = *(const f32x4*)(sc1 + gc);
            float f[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              f[v] = acc[b][j][4 * q + v] * s1[v];
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

template <int EPI, bool HAS_BIAS, bool FP8>
hipError_t launch_t(const GemmBf16Args& a, hipStream_t s) {
  using S = Shape<EPI>;
  using W = WRows<FP8>;
  if (FP8 && a.K % kBK) return hipErrorInvalidValue;  // FP8 codes come in 64-wide K blocks
  // rows through the permutation: 32-bit byte offsets into the whole of A
  if (a.row_token && (long long)a.a_rows * a.lda * 2 > (1LL << 30)) return hipErrorInvalidValue;
  const int nN = (a.N + S::kCols - 1) / S::kCols;
  const long long max_total = (long long)a.max_mtiles * nN;
  if (max_total <= 0) return hipSuccess;
  long long grid = (long long)a.num_cus / kXcds * kXcds;
  if (grid < kXcds) grid = kXcds;
  const long long per = (max_total + kXcds - 1) / kXcds;
  while ((per + grid / kXcds - 1) / (grid / kXcds) > kMaxTilesPerWG) grid += kXcds;
  static const char* const kNames[2][4] = {
      {"ggemm_big_relu", "ggemm_big_swiglu", "ggemm_big_out", "ggemm_big_out"},
      {"ggemm_big_fp8_relu", "ggemm_big_fp8_swiglu", "ggemm_big_fp8_out", "ggemm_big_fp8_out"}};
  ProfScope ps(a.prof_name ? a.prof_name : kNames[FP8 ? 1 : 0][EPI], s);
  ggemm_big_kernel<EPI, HAS_BIAS, FP8><<<dim3((unsigned)grid), dim3(kThreads), 0, s>>>(a);
  return hipGetLastError();
}

template <bool FP8>
hipError_t launch_typed(const GemmBf16Args& a, int epi, hipStream_t s) {
  const bool bias = a.bias != nullptr;
  switch (epi) {
    case EPI_RELU_BF16:
      return bias ? launch_t<EPI_RELU_BF16, true, FP8>(a, s)
                  : launch_t<EPI_RELU_BF16, false, FP8>(a, s);
    case EPI_SWIGLU_BF16:
      return launch_t<EPI_SWIGLU_BF16, false, FP8>(a, s);
    case EPI_IDENT_BF16:
      return bias ? launch_t<EPI_IDENT_BF16, true, FP8>(a, s)
                  : launch_t<EPI_IDENT_BF16, false, FP8>(a, s);
    default:
      return bias ? launch_t<EPI_IDENT_F32, true, FP8>(a, s)
                  : launch_t<EPI_IDENT_F32, false, FP8>(a, s);
  }
}

}  // namespace

hipError_t launch_gemm_big(const GemmBf16Args& a, int epi, hipStream_t s) {
  return a.fp8 ? launch_typed<true>(a, epi, s) : launch_typed<false>(a, epi, s);
}

}  // namespace moe
