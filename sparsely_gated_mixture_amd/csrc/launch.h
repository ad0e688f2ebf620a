// Host-side launchers of the gfx950 kernels (internal to libmoe).
// Each returns the HIP error of its launch; none synchronises.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

constexpr int kXcds = 8;  // MI355X: 8 accelerator complex dies, one L2 each

// A grouped GEMM's tile map: tile t covers rows [row0[t], min(row0[t] + bm,
// offsets[expert[t] + 1])) of expert[t]; *count tiles.
struct TileMap {
  int32_t* expert;
  int32_t* row0;
  int32_t* count;
};

// The experts split by size run their two grouped GEMMs side by side when
// the weights are bf16, each on its own share of the compute units: the
// 256 x 256-tile GEMM of the big experts is bound by the matrix units of the
// CUs it holds, while the 128-row GEMM of the small ones streams their
// weights and is bound by HBM on the whole chip, so on fewer CUs it moves
// more bytes per CU (about 30 against 22 GB/s) and the two overlap.  (With
// FP8 weights the 128-row GEMM is bound inside the CU -- the same weights
// per CU-second as bf16 -- and gains nothing; those run one after the
// other.)  The shares are set from the routing on the device, by the kernel
// that writes the two tile maps, one for each product (first: x W1^T and
// x W3^T; second: hidden W2^T), so that the two kernels' chains take about
// as long (below).  Each kernel's cost in CU-seconds:
//   big, first product:  flops over the big experts' rows padded to whole
//     256-row tiles (the 256 x 256 kernel's unit of work: an expert of 130
//     rows costs a whole tile) / kBigFlopsPerCu0, plus the weight bytes of
//     its M-tile groups (each group of kBigGroupM M-tiles of an expert reads
//     the expert's weights once) / kBigWeightBytesPerCu0;
//   big, second product: padded-tile flops / kBigFlopsPerCu1;
//   small: the product's weight and activation bytes / kSmallBytesPerCu.
// The rates were fitted on MI355X to the measured balance points of two
// routings at d = 7168, h = 2048 (31 big experts of up to 16 M-tiles, and 73
// of mostly one or two), each kernel running beside the other.  The share is
// a multiple of kXcds in [kXcds, cus - kXcds] (each XCD then holds as many
// workgroups of each kernel as every other XCD); 0 without big experts,
// every CU without small ones.
constexpr double kBigFlopsPerCu0 = 5.13e12;
constexpr double kBigWeightBytesPerCu0 = 59e9;
constexpr double kBigFlopsPerCu1 = 4.4e12;
constexpr double kSmallBytesPerCu = 30e9;
constexpr int kBigGroupM = 4;  // M-tiles per group of the 256 x 256 kernel's work order
// big_padded_rows: the big experts' rows, each expert's rounded up to a
// multiple of kBigBM; big_groups: sum over the big experts of
// ceil(M-tiles / kBigGroupM).  product: 0 first, 1 second.
//
// The two chains run independently (each kernel waits only for the previous
// one on its own stream), so the step ends with the longer chain.  The first
// product's share balances that product.  The second product's share then
// balances the chains' totals, on the side the first product frees first:
// if the small experts' chain finishes its first product first, the big
// experts' second product may take more CUs than its first (they are free
// by the time it starts), never fewer than the first's, and the other way
// round, so neither kernel's workgroups wait for CUs the other chain holds.
__host__ __device__ inline int expert_cu_split(int cus, long long big_padded_rows,
                                               long long big_groups, long long small_experts,
                                               long long small_rows, int d, int h, int swiglu,
                                               int product) {
  if (big_padded_rows <= 0) return 0;
  if (small_experts <= 0) return cus;
  const int units = cus / kXcds;
  if (units < 2) return cus;
  // Each product's cost in CU-seconds: weight matrices (each d x h) and
  // activation bytes per row.
  double t_big[2], t_small[2];
  for (int q = 0; q < 2; ++q) {
    const double mats = q == 0 && swiglu ? 2.0 : 1.0;
    const double row_bytes = q == 0 ? 2.0 * d + 2.0 * h : 2.0 * h + 4.0 * d;
    const double flops = 2.0 * mats * d * h * (double)big_padded_rows;
    t_big[q] = q == 0 ? flops / kBigFlopsPerCu0 +
                            mats * d * h * 2.0 * (double)big_groups / kBigWeightBytesPerCu0
                      : flops / kBigFlopsPerCu1;
    t_small[q] = (mats * d * h * 2.0 * (double)small_experts + row_bytes * (double)small_rows) /
                 kSmallBytesPerCu;
  }
  int u0 = (int)(units * t_big[0] / (t_big[0] + t_small[0]) + 0.5);
  u0 = u0 < 1 ? 1 : (u0 > units - 1 ? units - 1 : u0);
  if (product == 0) return u0 * kXcds;
  // chain times in units of CU-seconds per XCD row of CUs
  const double b0 = t_big[0] / u0, s0 = t_small[0] / (units - u0);
  const int lo = s0 <= b0 ? u0 : 1, hi = s0 <= b0 ? units - 1 : u0;
  int best = u0;
  double best_t = 1e300;
  for (int u = lo; u <= hi; ++u) {
    const double tb = b0 + t_big[1] / u, ts = s0 + t_small[1] / (units - u);
    const double t = tb > ts ? tb : ts;
    if (t < best_t) best_t = t, best = u;
  }
  return best * kXcds;
}

// Where the tile-map kernels write that share (out == null: no side-by-side
// run) and what it is computed from.
struct CuSplit {
  int32_t* out;  // device int[2]: CUs of the 256 x 256-tile GEMM in each product
  int cus;       // compute units of the device
  int d, h;      // model and hidden widths
  int swiglu;    // 1: W1, W3 and W2 per expert; 0: W1 and W2
};

// Brackets one kernel launch with HIP events while kernel timing is on
// (moe_profile_enable); a no-op otherwise.
struct ProfScope {
  int slot;
  hipStream_t stream;
  ProfScope(const char* name, hipStream_t s);
  ~ProfScope();
  ProfScope(const ProfScope&) = delete;
  ProfScope& operator=(const ProfScope&) = delete;
};

// ---------------------------------------------------------------------------
// fp32 MFMA GEMM:  C[r, c] = epi(sum_k A[r, k] * B[c, k] + bias[c]).
// Flat mode (tile_expert == nullptr): rows 0..M-1.  Grouped mode: M-tiles
// come from a device tile map (expert / group e, first row), rows of tile
// stop at offsets[e+1], and B / bias are offset by e * stride.
// B rows [0, n1) come from B1, rows [n1, N) from B2 (gate: clean | noise).
// A row r is A + (rowmap ? rowmap[r] : r) * lda.
// ---------------------------------------------------------------------------
struct GemmF32Args {
  const float* A;
  long long lda;
  const int32_t* rowmap;
  const float* B1;
  const float* B2;
  long long strideB1, strideB2;  // per-group element strides
  int n1, N, K;
  float* C;
  long long ldc;
  const float* bias;       // per-group bias rows of length N (may be null)
  long long stride_bias;
  int relu;                // 1: max(0, .)
  int M;                   // flat mode rows
  int mtiles;              // flat mode M-tiles (host-known)
  const int32_t* tile_expert;
  const int32_t* tile_row0;
  const int32_t* offsets;
  const int32_t* tile_count;  // device total of M-tiles (grouped mode)
  int max_mtiles;             // upper bound of M-tiles (grid sizing)
  const char* prof_name;      // profiler name of this launch (null: by tile size)
  // K-split (gate GEMM, flat mode only): ksplit > 1 splits K into ksplit
  // ranges of gate_split_len(K, ksplit) (a multiple of 256); split s writes
  // its partial product to C + s * split_stride.  0 or 1: one product to C.
  int ksplit;
  long long split_stride;
  // Flat mode, optional: the items of the first column tile also write A
  // rounded to bf16 (to nearest even: the operand split's high part) to
  // a_bf16 = [M, K] -- the layer forward's token-order bf16 copy of x.
  uint16_t* a_bf16;
};
// Length of each K range of a ksplit-way gate GEMM: ceil(K / ksplit) rounded
// up to the kernel's 256-wide accumulation chunks.
__host__ __device__ inline int gate_split_len(int K, int ksplit) {
  const int per = (K + ksplit - 1) / ksplit;
  return (per + 255) / 256 * 256;
}
// bm: 64 or 128 (BN = bm).
hipError_t launch_gemm_f32(const GemmF32Args& a, int bm, hipStream_t s);
// The same product without bias or ReLU on the bf16 matrix cores, each fp32
// operand split into three bf16 parts (fp32 accuracy), in flat mode (a.mtiles
// M-tiles of bm rows) or grouped mode (a tile map of bm-row tiles, row map,
// per-group weights).  K % 4 == 0.
hipError_t launch_gemm_gate(const GemmF32Args& a, int bm, hipStream_t s);
// Matrix-unit peak probe (probe.hip): `blocks` blocks of 4 waves, `iters`
// iterations of 4 MFMAs each; sink receives blocks * 256 floats.
hipError_t launch_mfma_probe(bool bf16, int blocks, int iters, float* sink, hipStream_t s);
// HBM read-stream probe (probe.hip): reads the first bytes (rounded down to
// 16) of buf; sink receives blocks * 256 floats.
hipError_t launch_hbm_read_probe(const void* buf, long long bytes, int blocks, float* sink,
                                 hipStream_t s);

// ---------------------------------------------------------------------------
// bf16 MFMA grouped GEMM for the expert FFNs.
// ---------------------------------------------------------------------------
// EPI_IDENT_BF16: identity(+bias) rounded to bf16 (the layer forward's expert
// outputs, which only the combine reads).
enum GemmEpi { EPI_RELU_BF16 = 0, EPI_SWIGLU_BF16 = 1, EPI_IDENT_F32 = 2, EPI_IDENT_BF16 = 3 };
struct GemmBf16Args {
  const uint16_t* A;     // [rows, K] bf16, rows contiguous
  long long lda;
  const void* B1;        // [n, N, K] bf16, or n packed FP8 experts (fp8 = 1)
  const void* B3;        // SwiGLU second matrix, same layout
  long long strideB;     // bytes from one expert's weights to the next
  int N, K;
  void* C;               // bf16 [rows, N] or f32 [rows, N]
  long long ldc;
  const float* bias;     // [n, N] or null
  const int32_t* tile_expert;
  const int32_t* tile_row0;
  const int32_t* offsets;
  const int32_t* tile_count;
  int max_mtiles;
  int num_cus;           // compute units of the device (persistent grid size)
  int shared;            // 1: the shared expert (only the profiler name differs)
  int fp8;               // 1: B1/B3 are packed E4M3 weights with per-row scales
  const char* prof_name; // profiler name of this launch (null: by epilogue and kind)
  // Side-by-side run (expert_cu_split): cu_split (device) holds the CUs of
  // the 256 x 256-tile GEMM in this product; this launch keeps that many workgroups
  // (cu_big = 1) or num_cus minus that many (cu_big = 0), at least enough
  // for kMaxTilesPerWG, and the others return at once.  Null: the whole grid.
  const int32_t* cu_split;
  int cu_big;
  // Activation rows through the permutation (null: A holds the merged rows
  // themselves): merged row r is row row_token[r] of A = [a_rows, K] bf16,
  // for r < row_token_n (the layer forward's token-order bf16 copy of x and
  // its perm); the copies look each row up with scalar loads when a tile
  // starts.
  const int32_t* row_token;
  int row_token_n;
  int a_rows;
  // Nonzero: each weight tile is read by one work item only (every expert
  // holds one M-tile), so the 128-row kernel copies weights with the
  // non-temporal hint.
  int b_stream;
};
constexpr int kBf16BM = 128;
constexpr int kMaxTilesPerWG = 512;  // tiles one persistent workgroup can hold
// The 256 x 256-tile grouped GEMM (ggemm_big.hip): same arguments, a tile map
// of kBigBM-row M-tiles, bf16 weights only (no FP8).
constexpr int kBigBM = 256;
hipError_t launch_gemm_big(const GemmBf16Args& a, int epi, hipStream_t s);

// Pack n_experts [N, K] weight matrices (fp32, or bf16 when src_bf16) into
// the FP8 E4M3 layout the grouped GEMM reads (codes by row pair and 64-wide
// K block, then one fp32 scale per row); N*K + 4*N bytes per expert.
hipError_t launch_pack_fp8(int n_experts, int N, int K, int src_bf16, const void* src, void* dst,
                           hipStream_t s);

// Compute units of the current device (queried once per device).
int device_cus();
// Sets the thread's last-error message (moe_last_error) and returns st.
moe_status report_error(moe_status st, const char* msg);
// Workspace bytes moe_gate needs for *cfg (0 when cfg is invalid).
size_t gate_workspace_bytes(const moe_config* cfg);
hipError_t launch_gemm_bf16(const GemmBf16Args& a, int epi, hipStream_t s);

// ---------------------------------------------------------------------------
// bf16 MFMA GEMMs of the expert backward: C[c][m] = sum_k A[k][m] * B(k, c).
// A is K-major (row k holds M contiguous columns; rows k >= k_split come from
// A2 at row k - k_split), offset by e * strideA for expert e.
// BWD_ROWS: c runs over the merged rows of the dispatch's 128-row tiles
//   (tile_expert / tile_row0 / offsets / tile_count); B[c][k] row-major with
//   K contiguous (ldb); K = p.K (a multiple of 64).
// BWD_WGRAD: one [N][M] output per expert e < n_experts; k runs over the
//   expert's merged rows offsets[e] .. offsets[e+1]; B[k][c] K-major.
// Epilogues: BEPI_F32 -> C (+ e*strideC; WGRAD rows c >= c_split go to C2
//   at row c - c_split); BEPI_RELU_MASK -> Cb = bf16(D where aux_h > 0);
//   BEPI_SWIGLU -> Cb[c][m] = bf16(da), Cb[c][c_split + m] = bf16(db) from
//   aux_a / aux_b (fp32 pre-activations, row stride ldaux).
// M and N multiples of 8; every pointer 16-byte aligned.
// ---------------------------------------------------------------------------
enum BwdMode { BWD_ROWS = 0, BWD_WGRAD = 1 };
enum BwdEpi { BEPI_F32 = 0, BEPI_RELU_MASK = 1, BEPI_SWIGLU = 2 };
struct GemmBwdArgs {
  const uint16_t* A;
  const uint16_t* A2;
  const int32_t* rowmap_a;  // fp32 WGRAD only: A's row k is rowmap_a[k] (null: k)
  long long lda, strideA;
  int k_split;
  const uint16_t* B;
  long long ldb;
  int M, N, K;
  float* C;
  float* C2;
  uint16_t* Cb;
  long long ldc, strideC;
  int c_split;
  const uint16_t* aux_h;
  const float* aux_a;
  const float* aux_b;
  long long ldaux;
  const int32_t* tile_expert;
  const int32_t* tile_row0;
  const int32_t* offsets;
  const int32_t* tile_count;
  int max_tiles;
  int tile_rows;  // rows per tile of the tile map (the bf16 kernels: kBf16BM)
  int n_experts;
};
hipError_t launch_gemm_bwd(const GemmBwdArgs& a, int mode, int epi, const char* name,
                           hipStream_t s);
// The same products for fp32 experts (A, A2, B hold fp32; the ReLU mask reads
// the fp32 hidden values from aux_a; no SwiGLU).  tile_rows is a multiple of 64.
hipError_t launch_gemm_bwd_f32(const GemmBwdArgs& a, int mode, int epi, const char* name,
                               hipStream_t s);

// Tile map of a grouped GEMM: for every expert e with rows in
// [offsets[e], offsets[e+1]), ceil(rows/bm) M-tiles in expert order.
hipError_t launch_tilemap(const int32_t* offsets, int n, int bm, int32_t* tile_expert,
                          int32_t* tile_row0, int32_t* tile_count, hipStream_t s);
// The same segments split by size: experts with fewer than big_rows rows in
// bm-row tiles (small), the others in kBigBM-row tiles (big).
hipError_t launch_tilemap_split(const int32_t* offsets, int n, int bm, int big_rows,
                                TileMap small, TileMap big, CuSplit split, hipStream_t s);

// ---------------------------------------------------------------------------
// Gate epilogue: noise, KeepTopK, softmax / Switch, importance/load partials.
// Row r reads clean logits at logits[r*ldl + j] (j < n) and raw noise logits
// at logits[r*ldl + n + j].
// Flat mode: row r is token r; outputs at [r*k + s]; bias b[j]; noise[r*n+j].
// Grouped (two-level secondary) mode: rows are the primary slots dispatched
// by group (row_token[r] = token); tiles of rows never straddle a group; the
// outputs go to the token's combined slots and multiply by the primary
// weight; partial sums are per tile.
// ---------------------------------------------------------------------------
struct TopkArgs {
  int rows, n, k, switch_mode, noisy;
  int sigmoid_mode;         // selection on logit + bias, weights Sigmoid(logit) renormalised
  float* logits;
  long long ldl;
  const float* bias;
  const float* noise;       // flat: [rows, n]; grouped: [T, k1, n] indexed by (token, slot)
  int32_t* topk_idx;
  float* topk_w;
  float* part_imp;          // [nparts, n]
  float* part_load;         // [nparts, n]
  float* part_stats;        // [nparts, 2]: sum of squared pre-softmax logits, sum of gate
                            // entropies over the block's rows (null: not computed)
  int rows_per_block;       // flat mode
  // grouped mode
  const int32_t* row_token;     // perm of the group dispatch
  const int32_t* prim_idx;      // [T, k1] primary group per slot
  const float* prim_w;          // [T, k1]
  int k1;
  const int32_t* tile_expert;   // group of each row tile
  const int32_t* tile_row0;
  const int32_t* offsets;       // group row offsets
  const int32_t* tile_count;
  int max_tiles;
  int tile_rows;
  // Flat mode: the gate GEMM's K-split partials.  nsplit > 1: row r's logits
  // are the sum, in split order, of logits[r] + s * split_stride over s <
  // nsplit; the kernel writes the sums back to logits[r] (split 0), where the
  // backward reads them.  0 or 1: logits[r] as is.
  int nsplit;
  long long split_stride;
};
// Wavefronts (rows in flight) per gate-epilogue block: 16 while a row fits in
// at most 8 registers per lane (n <= 512), else 8 (larger rows need the
// registers).  The host's rows-per-block is a multiple of this.
inline int topk_waves(int n) { return (n + 63) / 64 <= 8 ? 16 : 8; }
hipError_t launch_topk(const TopkArgs& a, hipStream_t s);
// Backward of a gate, one wavefront per row.  Flat mode: row r is token r
// (rows_per_block a multiple of topk_waves(n)); reads the forward's logits
// (clean without the bias | raw, row stride ldl), bias, noise [T, n],
// topk_idx / topk_w [T, k], the slot gradients dG [T, k], dimp [n] (null: 0),
// dload [n] and coef = {c_z, c_ent}; writes dlogits [rows, ldd] (dL/d clean |
// dL/d raw, zero-padded) and, if part_db, per-block column sums of the clean
// part [nblocks, n].  Grouped mode (tile_expert != null: a two-level
// secondary gate): rows are the group dispatch's (token, primary slot)
// pairs in tiles of tile_rows; noise [T, k1, n]; the slots are the token's
// combined slots s*k .. s*k+k-1 of topk_idx [T, k1*k] (ids g*n + e); the
// secondary weights are recomputed from the logits; dG [T, k1, k]; dload
// [groups, n].
struct GateBwdArgs {
  int T, n, k, switch_mode, sigmoid_mode, noisy;
  const float* logits;
  long long ldl;
  const float* bias;
  const float* noise;
  const int32_t* topk_idx;
  const float* topk_w;
  const float* dG;
  const float* dimp;
  const float* dload;
  const float* coef;
  float* dlogits;
  long long ldd;
  float* part_db;
  int rows_per_block;
  // grouped mode
  const int32_t* row_token;
  const int32_t* prim_idx;
  int k1;
  const int32_t* tile_expert;
  const int32_t* tile_row0;
  const int32_t* offsets;
  const int32_t* tile_count;
  int max_tiles;
  int tile_rows;
};
hipError_t launch_gate_bwd(const GateBwdArgs& a, hipStream_t s);
// out[j] = sum over parts p < nparts of part[p*n + j] (double sum, fixed
// order), for up to three (part, n, out) vectors in one launch; a vector with
// a null part is skipped.
struct ColsumVec {
  const float* part;
  int n;
  float* out;
};
hipError_t launch_colsum(int nparts, ColsumVec v0, ColsumVec v1, ColsumVec v2, hipStream_t s);
// Two-level gate statistics: out[0] = prim[0] + sum over the secondary tiles
// of part[t*2], out[1] = sum of part[t*2+1] (the product gate's entropy is
// carried entirely by the secondary rows).
hipError_t launch_hier_stats(const float* prim, const float* part, const int32_t* tile_count,
                             float* out, hipStream_t s);
// Two-level aux vectors: per-tile partials of the secondary gate are summed
// per group (tiles of a group are consecutive), then combined with the
// primary vectors: load[g*b+e] = load_p[g]*load_g[e]/|X_g|.
// load_g (may be null) receives the per-group secondary loads [a, b].
hipError_t launch_hier_finalize(const float* part_imp, const float* part_load,
                                const int32_t* tile_expert, const int32_t* tile_count,
                                const int32_t* group_counts, const float* load_primary, int a,
                                int b, float* importance, float* load, float* load_g,
                                hipStream_t s);

// ---------------------------------------------------------------------------
// Dispatch.
// ---------------------------------------------------------------------------
constexpr int kDispatchChunk = 256;  // assignments per chunk (one wavefront each in the permute)
struct DispatchArgs {
  const int32_t* topk_idx;
  int T, k, n;
  long long cap;
  int32_t* counts_pre;
  int32_t* counts;
  int32_t* offsets;
  int32_t* perm;
  int32_t* slot_pos;
  int32_t* chunk_hist;
  int32_t* chunk_base;
  // Optional: the grouped GEMM's tile map for tile_bm-row M-tiles (0 = none).
  int tile_bm;
  int32_t* tile_expert;
  int32_t* tile_row0;
  int32_t* tile_count;
  // Optional (big_rows > 0, with tile_bm): the same segments split in two
  // maps by size -- experts keeping fewer than big_rows rows in tile_bm-row
  // tiles (small map), the others in kBigBM-row tiles (big map).
  int big_rows;
  TileMap small_map, big_map;
  CuSplit split;  // with big_rows > 0: the side-by-side CU share (split.out may be null)
  // Optional: auxiliary losses from importance / load (load may be null) and
  // the pre-capacity counts (losses == null: none).
  float* losses;
  const float* importance;
  const float* load;
  const float* gate_stats;  // [2] or null: z-loss and entropy sums
  float w_imp, w_load, alpha, w_z, w_ent;
  // Optional: the gate's column sums (its per-block Importance / Load /
  // statistics partials over colsum_nparts parts) run inside the histogram
  // launch instead of a launch of their own (colsum_fused != 0).
  ColsumVec colsum[3];
  int colsum_nparts;
  int colsum_fused;
};
hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t s);
// Scatter each token's row to its kept slots: x_perm[slot_pos[t, s]] =
// convert(x[t]) (bf16 round to nearest even, or an fp32 copy); x_bf16 (may be
// null) also receives every row in token order, in bf16.
hipError_t launch_gather(const float* x, const int32_t* slot_pos, int T, int k, int d,
                         int bf16_out, void* x_perm, uint16_t* x_bf16, hipStream_t s);
// x_bf16[t] = bf16(x[t]) for every token.
hipError_t launch_to_bf16(const float* x, long long elems, uint16_t* out, hipStream_t s);
// Tile map of one segment of T rows (the shared expert): offsets2 = {0, T}.
hipError_t launch_shared_tilemap(int T, int bm, int32_t* offsets2, int32_t* tile_expert,
                                 int32_t* tile_row0, int32_t* tile_count, hipStream_t s);
// Selection-bias controller: bias[i] -= gamma if counts_pre[i]*n > T*k,
// += gamma if counts_pre[i]*n < T*k.
hipError_t launch_bias_update(const int32_t* counts_pre, int n, int T, int k, float gamma,
                              float* bias, hipStream_t s);

// ---------------------------------------------------------------------------
// Combine and aux.
// ---------------------------------------------------------------------------
// The auxiliary losses' inputs (block_aux_losses); losses == null: none.
struct AuxArgs {
  const float* importance;
  const float* load;  // may be null (no Load term)
  const int32_t* counts_pre;
  const float* gate_stats;  // may be null
  int T, k, n;
  float w_imp, w_load, alpha, w_z, w_ent;
  float* losses;
};
// y[t] = y_base[t] (when given) + sum over kept slots, in slot order.  With
// aux (losses non-null) one more block of the launch (its first) computes the
// losses.  y_perm holds fp32 rows, or bf16 rows when y_bf16 is set.
hipError_t launch_combine(const void* y_perm, const int32_t* slot_pos, const float* topk_w,
                          const float* y_base, int T, int k, int d, float* y, hipStream_t s,
                          const AuxArgs* aux = nullptr, bool y_bf16 = false);
hipError_t launch_aux(const float* importance, const float* load, const int32_t* counts_pre,
                      const float* gate_stats, int T, int k, int n, float w_imp, float w_load,
                      float alpha, float w_z, float w_ent, float* losses, hipStream_t s);

// ---------------------------------------------------------------------------
// Backward (backward.hip).
// ---------------------------------------------------------------------------
// Per token, per kept slot: dG[t,s] = <dy_t, y_perm[row]>, dout[row] =
// topk_w[t,s] * dy_t (bf16, or fp32 when dout_f32); dropped slots get dG = 0.
hipError_t launch_combine_bwd(const float* dy, const float* y_perm, const int32_t* slot_pos,
                              const float* topk_w, int T, int k, int d, float* dG, void* dout,
                              int dout_f32, hipStream_t s);
// dimp = dl0 w_imp dCV^2(importance) + dl2 alpha n f / T, dload = dl1 w_load
// dCV^2(load) (skipped when load is null), coef = {dl3 w_z / T, dl4 w_ent / T,
// dl3 w_z / T, 0} (the last pair for a gate without an entropy term of its
// own); dlosses is a device vector of 5.
hipError_t launch_loss_grad(const float* importance, const float* load,
                            const int32_t* counts_pre, const float* dlosses, int T, int k, int n,
                            float w_imp, float w_load, float alpha, float w_z, float w_ent,
                            float* dimp, float* dload, float* coef, hipStream_t s);
// Gate weight gradients: rows m < M of dlogits^T x, split over tokens into
// `splits` partial products of tokens_per_split tokens each (partial holds
// splits * M * d floats), then summed in split order into dw_gate (rows m <
// n) and dw_noise (rows m >= n).  d % 4 == 0, ldd % 4 == 0.
struct GateWgradArgs {
  const float* x;
  const float* dlogits;
  long long ldd;
  int T, d, M, n, splits, tokens_per_split;
  float* partial;
};
int gate_wgrad_splits(int T, int d, int M);
hipError_t launch_gate_wgrad(const GateWgradArgs& a, float* dw_gate, float* dw_noise,
                             hipStream_t s);
// wt [d, ldk] = [w_gate; w_noise (if given)]^T, zero past the stacked rows.
hipError_t launch_transpose_gate(const float* w_gate, const float* w_noise, int n, int d,
                                 int ldk, float* wt, hipStream_t s);
// out[e][c] = sum over rows offsets[e] .. offsets[e+1]-1 of src[row][c] (bf16,
// or fp32 when src_f32).
hipError_t launch_seg_colsum(const void* src, int src_f32, long long ld, const int32_t* offsets,
                             int n_seg, int N, float* out, hipStream_t s);
// dx[t] = dx_gate[t] (+ dx_shared[t]) (+ the two-level secondary gates' rows
// du2[slot2[t, s]], s < k2) + sum over kept slots of du_perm[row].
hipError_t launch_dx_gather(const float* dx_gate, const float* dx_shared, const float* du_perm,
                            const int32_t* slot_pos, int T, int k, int d, const float* du2,
                            const int32_t* slot2, int k2, float* dx, hipStream_t s);
// Two-level layer: the product weights' gradients split into the primary
// slots' dG1 [T, k1] and the secondary slots' dG2 [T, k1, k2] (coef[1] =
// c_ent, dimp over the a*b experts).
hipError_t launch_hier_product_bwd(const int32_t* topk_idx, const float* topk_w,
                                   const float* prim_w, const float* dG, const float* dimp,
                                   const float* coef, int T, int k1, int k2, float* dG1,
                                   float* dG2, hipStream_t s);
// Two-level layer: dLoad_H [a*b] into dLoad_p [a] and dLoad_g [a, b] through
// Load_H = Load_p Load_g / |X_g| (counts = |X_g|).
hipError_t launch_hier_dload(const float* dload_h, const float* load_p, const float* load_g,
                             const int32_t* counts, int a, int b, float* dload_p,
                             float* dload_g, hipStream_t s);
// hid[i] = bf16(silu(a[i]) * b[i]) for i < elems (a multiple of 4).
hipError_t launch_swiglu_hidden(const float* a, const float* b, long long elems, uint16_t* hid,
                                hipStream_t s);

}  // namespace moe
