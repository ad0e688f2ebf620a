// Grouped GEMM of the expert FFNs on the gfx950 matrix cores
// (v_mfma_f32_32x32x16_bf16: bf16 operands, fp32 accumulation).
//
// One launch covers every expert.  A device-side tile map lists the M-tiles
// (128 rows of one expert's merged batch); the work items are (M-tile,
// N-tile) pairs.  Expert e's weights are W[e] = [N, K] (out x in, K
// contiguous) and the activations X = [rows, K], so both operands stream
// along K.
//
// The expert weights are read once per layer and dominate the bytes, so the
// kernel is shaped for HBM streaming:
//  * persistent: one 8-wave workgroup per CU walks a strided run of tiles
//    inside its XCD's contiguous share of the tile list (N-tiles of one
//    M-tile, which share the activation tile, and M-tiles of one expert,
//    which share its weights, run on the same L2 at about the same time);
//  * K advances 64 at a time, so every row of both operands is read in whole
//    128-byte lines (narrower per-row reads measured about 30% slower);
//  * a ring of kStages LDS buffers is filled by direct global->LDS copies
//    (global_load_lds_dwordx4); step g+2 is copied right after the barrier
//    that opens step g, so two steps are in flight while step g computes;
//    the ring runs on across tile boundaries, so a tile's epilogue overlaps
//    the next tile's loads; one barrier per step;
//  * each lane keeps the global addresses of the rows it copies and updates
//    them only when the copy cursor enters a new tile, so a step's copies
//    are an add and an instruction each;
//  * N-tiles are 256 wide (SwiGLU: 128 columns of both W1 and W3), so each
//    activation tile is fetched from L2 N/256 times; this measured faster than
//    128-wide tiles with a deeper ring (activation re-reads through L2 cost
//    about as much as the weight stream itself);
//  * LDS rows are 128 bytes (8 chunks of 16 bytes); chunk c of row r sits at
//    position c ^ ((r >> 1) & 7), so the 16-byte fragment reads of 16
//    consecutive rows hit 16 distinct bank groups.
// The MFMA computes D = W . X^T (weights as the A operand), so each lane ends
// with 4 consecutive output columns of one row and stores them directly.
// Epilogues: ReLU(+bias) -> bf16 hidden; silu(x.W1^T) * (x.W3^T) -> bf16
// hidden; identity(+bias) -> fp32 or bf16 expert output.
// Rows past a segment's end and columns past N copy clamped (valid) rows and
// are never stored; K-tail chunks copy a 16-byte zero constant.
#include <math.h>

#include "common.h"
#include "launch.h"
#include "lds_dma.h"

namespace moe {
namespace {

constexpr int kBM = kBf16BM;  // rows per M-tile (the tile map's granularity)
constexpr int kBK = 64;       // K per pipeline step
constexpr int kRowB = 128;    // bytes per LDS row (kBK bf16)
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;

__device__ __forceinline__ int swz(int r, int c) { return (c ^ ((r >> 1) & 7)) << 4; }

// HAS_BIAS is a template parameter so that the usual bias-free kernels have
// no global loads in the epilogue (the compiler would otherwise wait there
// for every copy in flight).
//
// FP8: the weights are E4M3 codes in the packed layout of
// moe_pack_fp8_weights (row pairs, 128 bytes per pair and 64-wide K block,
// then one fp32 scale per row).  A weight row takes 64 bytes of LDS per step,
// so a step is 32 KB and the ring is 4 deep; fragments are read as 8 bytes,
// widened to bf16 in registers, and each output row is multiplied by its
// scale in the epilogue.
template <int BN, int EPI, int WGM, bool HAS_BIAS, bool FP8>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void
ggemm_bf16_kernel(const GemmBf16Args p) {
  constexpr int NB = (EPI == EPI_SWIGLU_BF16) ? 2 : 1;  // weight matrices per tile
  constexpr int BROWS = NB * BN;                         // weight rows per tile
  constexpr int kStages = FP8 ? 4 : 3;                   // LDS ring depth
  constexpr int B_ROWB = FP8 ? 64 : kRowB;               // LDS bytes per weight row
  constexpr int A_BYTES = kBM * kRowB, B_BYTES = BROWS * B_ROWB;
  constexpr int STAGE = A_BYTES + B_BYTES;
  constexpr int ADMA = A_BYTES / 1024 / kWaves, BDMA = B_BYTES / 1024 / kWaves;
  constexpr int PER_STEP = ADMA + BDMA;  // copies per thread per step (at most)
  constexpr int WGN = kWaves / WGM;
  constexpr int WM = kBM / WGM, WN = BN / WGN;
  constexpr int FM = WM / 32, FN = WN / 32;
  static_assert(ADMA >= 1 && BDMA >= 1 && FM >= 1 && FN >= 1, "bad tile shape");
  static_assert(BN % 16 == 0, "a copy block must not straddle the two weight matrices");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kStages * STAGE];
  __shared__ int4 meta[kMaxTilesPerWG];  // per tile: expert, first row, end row, first column

  // This workgroup's tiles: XCD x owns tiles [x*per, (x+1)*per); its
  // workgroups take every wpx-th of them.
  const int nN = (p.N + BN - 1) / BN;
  const int total = *p.tile_count * nN;
  // Side by side with the 256 x 256-tile GEMM (this kernel on the side
  // stream): workgroups numbered `used` and up return at once.
  const int used = gemm_used_grid(p, total);
  const int bid = (int)blockIdx.x;
  if (bid >= used) return;
  const int per = (total + kXcds - 1) / kXcds;
  const int xcd = bid % kXcds, slot = bid / kXcds;
  const int wpx = used / kXcds;
  const int first = xcd * per + slot;
  const int last = min(total, (xcd + 1) * per);
  const int ntiles = first < last ? (last - first + wpx - 1) / wpx : 0;
  if (ntiles == 0) return;
  const int tid = threadIdx.x;
  for (int t = tid; t < ntiles; t += kThreads) {
    const int L = first + t * wpx;
    const int mt = L / nN, nt = L % nN;
    const int e = p.tile_expert[mt];
    meta[t] = make_int4(e, p.tile_row0[mt], p.offsets[e + 1], nt * BN);
  }
  __syncthreads();

  const int K = p.K;
  const int nk = (K + kBK - 1) / kBK;
  const int nsteps = ntiles * nk;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;

  // Copy cursor: the next step to copy is step gi (tile it, K-step ikt).
  // Each lane keeps the global address of the 16 bytes it copies for the
  // cursor's tile (both layouts advance 128 bytes per K-step), recomputed
  // only when the cursor enters a new tile.  Activations: row blk*8 +
  // lane/8, chunk (lane%8) swizzled.  bf16 weights: the same.  FP8 weights:
  // row blk*16 + lane/4, 16-byte chunk (lane%4) swizzled.
  const uint8_t* a_src[ADMA];
  const uint8_t* b_src[BDMA];
  int a_chunk[ADMA], b_chunk[BDMA];  // element offset of the lane's chunk (bf16 K tail)
  int gi = 0, it = 0, ikt = 0, islot = 0;  // islot = gi % kStages
  int a_live = 0;                    // copies j < a_live of the activation tile hold real rows
  int cnt_last = 0, cnt_prev = 0;    // copies of the two most recently copied steps
  auto set_tile = [&](int ti) {
    const int4 m = meta[ti];
    // Row groups (8 rows per copy) past the segment's end are not copied:
    // their LDS rows only ever feed output columns that are not stored.
    a_live = 0;
    const int ty = __builtin_amdgcn_readfirstlane(m.y), tz = __builtin_amdgcn_readfirstlane(m.z);
#pragma unroll
    for (int j = 0; j < ADMA; ++j) {
      const int r = (wave + kWaves * j) * 8 + (lane >> 3);
      a_live += m.y + (wave + kWaves * j) * 8 < m.z ? 1 : 0;
      a_chunk[j] = ((lane & 7) ^ ((r >> 1) & 7)) * 8;
      // the merged row (rows past the segment repeat its last one), or its token
      long long arow = min(m.y + r, m.z - 1);
      if (p.row_token)
        arow = row_token8(p.row_token, ty + (wave + kWaves * j) * 8,
                          min(tz, p.row_token_n), lane);
      a_src[j] = (const uint8_t*)(p.A + arow * p.lda + a_chunk[j]);
    }
#pragma unroll
    for (int j = 0; j < BDMA; ++j) {
      if constexpr (FP8) {
        const int r = (wave + kWaves * j) * 16 + (lane >> 2);
        const int which = r / BN, rn = r % BN;
        const int n = min(m.w + rn, p.N - 1);
        const uint8_t* w = (const uint8_t*)(which == 0 ? p.B1 : p.B3) + (long long)m.x * p.strideB;
        const int lc = (lane & 3) ^ ((r >> 1) & 3);  // logical 16-byte chunk of this slot
        b_chunk[j] = 0;
        b_src[j] = w + ((long long)(n >> 1) * (K / 64)) * 128 + (n & 1) * 64 + lc * 16;
      } else {
        const int r = (wave + kWaves * j) * 8 + (lane >> 3);
        const int which = r / BN, rn = r % BN;
        const uint8_t* w = (const uint8_t*)(which == 0 ? p.B1 : p.B3) + (long long)m.x * p.strideB;
        b_chunk[j] = ((lane & 7) ^ ((r >> 1) & 7)) * 8;
        b_src[j] = w + ((long long)min(m.w + rn, p.N - 1) * K + b_chunk[j]) * 2;
      }
    }
  };
  // Copy step gi into ring slot gi % kStages and advance the cursor.  A bf16
  // step that reaches past K copies a 16-byte zero constant for the chunks
  // beyond it (FP8 weights need K % 64 == 0).
  auto issue_next = [&]() {
    const uint32_t sb = lds0 + islot * STAGE;
    const int k0 = ikt * kBK;
    const long long adv = (long long)ikt * 128;
    if (FP8 || k0 + kBK <= K) {
#pragma unroll
      for (int j = 0; j < ADMA; ++j)
        if (j < a_live) dma16(a_src[j] + adv, sb + (wave + kWaves * j) * 1024);
      if (p.b_stream) {
#pragma unroll
        for (int j = 0; j < BDMA; ++j)
          dma16_stream(b_src[j] + adv, sb + A_BYTES + (wave + kWaves * j) * 1024);
      } else {
#pragma unroll
        for (int j = 0; j < BDMA; ++j)
          dma16(b_src[j] + adv, sb + A_BYTES + (wave + kWaves * j) * 1024);
      }
    } else {
#pragma unroll
      for (int j = 0; j < ADMA; ++j)
        if (j < a_live)
          dma16(k0 + a_chunk[j] < K ? (const void*)(a_src[j] + adv) : (const void*)kZeroChunk,
                sb + (wave + kWaves * j) * 1024);
#pragma unroll
      for (int j = 0; j < BDMA; ++j) {
        const void* src =
            k0 + b_chunk[j] < K ? (const void*)(b_src[j] + adv) : (const void*)kZeroChunk;
        if (p.b_stream)
          dma16_stream(src, sb + A_BYTES + (wave + kWaves * j) * 1024);
        else
          dma16(src, sb + A_BYTES + (wave + kWaves * j) * 1024);
      }
    }
    cnt_prev = cnt_last;
    cnt_last = a_live + BDMA;
    ++gi;
    islot = islot == kStages - 1 ? 0 : islot + 1;
    if (++ikt == nk) {
      ikt = 0;
      if (++it < ntiles) set_tile(it);
    }
  };

  const int wm = wave / WGN, wn = wave % WGN;
  const int lr = lane & 31, lh = lane >> 5;

  f32x16 acc[NB][FM][FN];
  auto zero_acc = [&]() {
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[b][i][j][v] = 0.f;
  };
  zero_acc();

  // Finished results of the last tile, stored one step later.
  f32x4 pend_f[EPI == EPI_IDENT_F32 ? FM : 1][EPI == EPI_IDENT_F32 ? FN : 1][4];
  uint2 pend_h[EPI == EPI_IDENT_F32 ? 1 : FM][EPI == EPI_IDENT_F32 ? 1 : FN][4];
  int pend_row = 0, pend_end = 0, pend_col = 0;
  bool pend = false;
  auto store_pending = [&]() {
    if (!pend) return;
    pend = false;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int gr = pend_row + i * 32;
      if (gr >= pend_end) continue;
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int gc = pend_col + j * 32 + q4 * 8;
          if (gc >= p.N) continue;
          if constexpr (EPI == EPI_IDENT_F32)
            *(f32x4*)((float*)p.C + (long long)gr * p.ldc + gc) = pend_f[i][j][q4];
          else
            *(uint2*)((uint16_t*)p.C + (long long)gr * p.ldc + gc) = pend_h[i][j][q4];
        }
    }
  };

  int4 cm = meta[0];  // the computing tile
  set_tile(0);
#pragma unroll
  for (int s = 0; s < kStages - 1; ++s)
    if (gi < nsteps) issue_next();

  // Compute position: tile ct, K-step ck within it, ring slot cslot (kept
  // incrementally: no integer division per step).
  int ct = 0, ck = 0, cslot = 0;
  for (int g = 0; g < nsteps; ++g) {
    // Steps copied after this one (at most kStages-2).  Wait until only
    // their copies may still be in flight; loads complete in order, so
    // step g's copies have then landed.
    const int ahead = min(nsteps, g + kStages - 1) - 1 - g;
    static_assert(kStages == 3 || kStages == 4, "the waits below cover 3- or 4-deep rings");
    wait_vm_upto<(kStages - 2) * PER_STEP>(ahead <= 0 ? 0 : ahead == 1 ? cnt_last
                                                                      : cnt_last + cnt_prev);
    __syncthreads();
    if (ck == 0) cm = meta[ct];
    // Every wave is past step g-1, so its ring slot can take step
    // g+kStages-1 now, while this step computes.
    if (gi < nsteps) issue_next();
    store_pending();
    const uint8_t* As = smem + cslot * STAGE;
    const uint8_t* Bs = As + A_BYTES;
    // A wave whose token rows all lie past the segment's end has nothing to
    // compute this tile.
    if (cm.y + wm * WM < cm.z) {
    // All fragments of the step first (the LDS reads overlap one another),
    // then the MFMAs (FP8: the widening of slice kk runs beside the MFMAs
    // of slice kk-1).
    bf16x8 xf[kBK / 16][FM], wf[kBK / 16][NB][FN];
    uint2 wraw[kBK / 16][NB][FN];
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      const int c = 2 * kk + lh;  // 32x32x16 operand: row lane%32, k = 8*(lane/32)..+7
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int r = wm * WM + i * 32 + lr;
        xf[kk][i] = *(const bf16x8*)(As + r * kRowB + swz(r, c));
      }
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int r = b * BN + wn * WN + j * 32 + lr;
          if constexpr (FP8) {
            wraw[kk][b][j] = *(const uint2*)(Bs + r * 64 + ((kk ^ ((r >> 1) & 3)) << 4) + lh * 8);
          } else {
            wf[kk][b][j] = *(const bf16x8*)(Bs + r * kRowB + swz(r, c));
          }
        }
    }
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      if constexpr (FP8) {
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int j = 0; j < FN; ++j) wf[kk][b][j] = e4m3x8_to_bf16(wraw[kk][b][j]);
      }
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[b][i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[kk][b][j], xf[kk][i],
                                                                   acc[b][i][j], 0, 0, 0);
    }
    // Scheduling groups: every LDS read of the step, then the MFMAs (FP8:
    // each slice's widening, 4 instructions per fragment, then its MFMAs).
    __builtin_amdgcn_sched_group_barrier(0x100, (kBK / 16) * (FM + NB * FN), 0);
    if constexpr (FP8) {
#pragma unroll
      for (int kk = 0; kk < kBK / 16; ++kk) {
        __builtin_amdgcn_sched_group_barrier(0x002, 4 * NB * FN, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, NB * FM * FN, 0);
      }
    } else {
      __builtin_amdgcn_sched_group_barrier(0x008, (kBK / 16) * NB * FM * FN, 0);
    }
    }

    cslot = cslot == kStages - 1 ? 0 : cslot + 1;
    if (++ck == nk) {
      ck = 0;
      ++ct;
      // Tile done.  D[n][m] layout: lane holds column m = lane%32 of each
      // 32x32 block and rows n = 8*(v/4) + 4*(lane/32) + v%4.  The results
      // are finished (scale, bias, activation, bf16 rounding) into registers
      // here and stored at the next step, after its copies are issued, so
      // the stores drain while that step computes.
      const int4 m = cm;
      const int e = m.x;
      const float* bias = HAS_BIAS ? p.bias + (long long)e * p.N : nullptr;
      // FP8: the row scales follow each expert's codes.
      const float* sc1 = FP8 ? (const float*)((const uint8_t*)p.B1 + (long long)e * p.strideB +
                                             (long long)p.N * K)
                             : nullptr;
      const float* sc3 = (FP8 && NB == 2) ? (const float*)((const uint8_t*)p.B3 +
                                                           (long long)e * p.strideB +
                                                           (long long)p.N * K)
                                          : nullptr;
      // FP8: this lane's row scales for every (j, q4), read once per tile;
      // each group of 8 rows comes from a wave-uniform address (scalar loads).
      float s1[FN][4][4], s3[FN][4][4];
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int gc0 = m.w + wn * WN + j * 32 + q4 * 8;  // first of 8 rows (N % 8 == 0)
#pragma unroll
          for (int q = 0; q < 4; ++q) s1[j][q4][q] = s3[j][q4][q] = 1.f;
          if constexpr (FP8) {
            if (gc0 < p.N) {
              float u1[8], u3[8];
#pragma unroll
              for (int q = 0; q < 8; ++q) {
                u1[q] = sc1[gc0 + q];
                u3[q] = NB == 2 ? sc3[gc0 + q] : 1.f;
              }
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                s1[j][q4][q] = lh ? u1[4 + q] : u1[q];
                s3[j][q4][q] = lh ? u3[4 + q] : u3[q];
              }
            }
          }
        }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const int gc = m.w + wn * WN + j * 32 + q4 * 8 + lh * 4;
            float f[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              if constexpr (EPI == EPI_SWIGLU_BF16) {
                const float gv = acc[0][i][j][4 * q4 + q] * s1[j][q4][q];
                const float uv = acc[NB - 1][i][j][4 * q4 + q] * s3[j][q4][q];
                f[q] = gv / (1.f + expf(-gv)) * uv;
              } else {
                f[q] = acc[0][i][j][4 * q4 + q] * s1[j][q4][q];
                if constexpr (HAS_BIAS) f[q] += gc < p.N ? bias[gc + q] : 0.f;
                if constexpr (EPI == EPI_RELU_BF16) f[q] = fmaxf(f[q], 0.f);
              }
            }
            if constexpr (EPI == EPI_IDENT_F32) {
              pend_f[i][j][q4] = f32x4{f[0], f[1], f[2], f[3]};
            } else {
              pend_h[i][j][q4] = make_uint2(bf16x2_bits(f[0], f[1]), bf16x2_bits(f[2], f[3]));
            }
          }
      pend_row = m.y + wm * WM + lr;
      pend_end = m.z;
      pend_col = m.w + wn * WN + lh * 4;
      pend = true;
      zero_acc();
    }
  }
  store_pending();
}

template <int BN, int EPI, int WGM, bool HAS_BIAS, bool FP8>
hipError_t launch_t(const GemmBf16Args& a, hipStream_t s) {
  const int nN = (a.N + BN - 1) / BN;
  const long long max_total = (long long)a.max_mtiles * nN;
  if (max_total <= 0) return hipSuccess;
  // One workgroup per CU, a multiple of the XCD count, and enough of them
  // that no workgroup holds more than kMaxTilesPerWG tiles.
  long long grid = (long long)a.num_cus / kXcds * kXcds;
  if (grid < kXcds) grid = kXcds;
  const long long per = (max_total + kXcds - 1) / kXcds;
  while ((per + grid / kXcds - 1) / (grid / kXcds) > kMaxTilesPerWG) grid += kXcds;
  static const char* const kNames[3][3] = {
      {"ggemm_bf16_relu", "ggemm_bf16_swiglu", "ggemm_bf16_out"},
      {"shared_bf16_relu", "shared_bf16_swiglu", "shared_bf16_out"},
      {"ggemm_fp8_relu", "ggemm_fp8_swiglu", "ggemm_fp8_out"}};
  ProfScope ps(a.prof_name ? a.prof_name
                           : kNames[FP8 ? 2 : a.shared ? 1 : 0][EPI == EPI_RELU_BF16     ? 0
                                                                : EPI == EPI_SWIGLU_BF16 ? 1
                                                                                         : 2],
               s);
  ggemm_bf16_kernel<BN, EPI, WGM, HAS_BIAS, FP8>
      <<<dim3((unsigned)grid), dim3(kThreads), 0, s>>>(a);
  return hipGetLastError();
}

template <bool FP8>
hipError_t launch_typed(const GemmBf16Args& a, int epi, hipStream_t s) {
  const bool bias = a.bias != nullptr;
  switch (epi) {
    case EPI_RELU_BF16:
      return bias ? launch_t<256, EPI_RELU_BF16, 2, true, FP8>(a, s)
                  : launch_t<256, EPI_RELU_BF16, 2, false, FP8>(a, s);
    case EPI_SWIGLU_BF16:
      return launch_t<128, EPI_SWIGLU_BF16, 2, false, FP8>(a, s);
    case EPI_IDENT_BF16:
      return bias ? launch_t<256, EPI_IDENT_BF16, 2, true, FP8>(a, s)
                  : launch_t<256, EPI_IDENT_BF16, 2, false, FP8>(a, s);
    default:
      return bias ? launch_t<256, EPI_IDENT_F32, 2, true, FP8>(a, s)
                  : launch_t<256, EPI_IDENT_F32, 2, false, FP8>(a, s);
  }
}

}  // namespace

hipError_t launch_gemm_bf16(const GemmBf16Args& a, int epi, hipStream_t s) {
  return a.fp8 ? launch_typed<true>(a, epi, s) : launch_typed<false>(a, epi, s);
}

}  // namespace moe
