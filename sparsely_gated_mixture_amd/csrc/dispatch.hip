// Dispatch on gfx950: merge all positions routed to each expert into one
// contiguous batch (the notes on arXiv 1701.06538, "Engineering": all time
// steps merged into one batch; MoE survey, tufusi.com 3.2: expert capacity,
// overflow dropped to the residual).
//
// The T*k (token, slot) assignments are cut into chunks of kDispatchChunk.
//   1. chunk_hist_kernel: per-chunk expert histogram (integer LDS atomics,
//      whose result does not depend on their order).  In the layer forward
//      the gate's fixed-order column sums ride in the same launch
//      (hist_colsum_kernel: the first blocks histogram, the rest sum
//      columns), which saves a launch on the path.
//   2. scan_finalize_kernel, column scan: per expert, exclusive prefix over
//      chunks, and the total count (counts_pre); four threads per expert
//      each walk a quarter of the chunks, and the quarters are joined in
//      order.
//   3. in the same launch, the finalize, run by the scan block that finishes
//      last: counts = min(counts_pre, C), exclusive scan -> offsets; in the
//      layer forward it also writes the grouped GEMMs' tile maps (and the
//      side-by-side CU share) and the auxiliary losses.
//   4. permute_kernel: one wavefront walks its chunk in order, 64 slots at a
//      time; a slot's rank inside its group of 64 is the number of earlier
//      lanes with the same expert (the lanes holding the same id are found
//      with one ballot per bit of the expert id), so the resulting order is
//      exactly (token, slot) order -- stable, and independent of scheduling.
//   5. gather_kernel: one wavefront per token reads its row once and writes
//      it to each kept slot's row, converted to bf16 (RNE) or copied as fp32,
//      and/or once in token order as bf16 (the layer forward's bf16 experts
//      then read their rows through perm and no slot rows are written).
#include <algorithm>

#include "colsum.h"
#include "common.h"
#include "launch.h"

namespace moe {
namespace {

// Histogram of chunk `c` into chunk_hist[c]; any block size.
__device__ inline void chunk_hist_block(const int32_t* __restrict__ idx, long long A, int n,
                                        int32_t* __restrict__ chunk_hist, int c, int32_t* hist) {
  const int nt = (int)blockDim.x;
  for (int e = threadIdx.x; e < n; e += nt) hist[e] = 0;
  __syncthreads();
  const long long a0 = (long long)c * kDispatchChunk;
  for (int i = threadIdx.x; i < kDispatchChunk; i += nt) {
    const long long a = a0 + i;
    if (a < A) {
      const int e = idx[a];
      if ((unsigned)e < (unsigned)n) atomicAdd(&hist[e], 1);  // ids outside [0, n): no expert
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < n; e += nt) chunk_hist[(long long)c * n + e] = hist[e];
}

// `done`: the ticket of the scan + finalize launch that follows, set to 0.
__global__ __launch_bounds__(256) void chunk_hist_kernel(const int32_t* __restrict__ idx,
                                                         long long A, int n,
                                                         int32_t* __restrict__ chunk_hist,
                                                         int32_t* __restrict__ done) {
  extern __shared__ int32_t hist[];
  if (blockIdx.x == 0 && threadIdx.x == 0) *done = 0;
  chunk_hist_block(idx, A, n, chunk_hist, (int)blockIdx.x, hist);
}

// Blocks [0, nchunks) histogram their chunk; block nchunks + b sums columns
// (b % cx) of the gate's vector b / cx (kColThreads threads either way).
__global__ __launch_bounds__(kColThreads) void hist_colsum_kernel(
    const int32_t* __restrict__ idx, long long A, int n, int32_t* __restrict__ chunk_hist,
    int nchunks, const ColsumArgs cs, int nparts, int cx, int32_t* __restrict__ done) {
  extern __shared__ int32_t hist[];
  const int b = (int)blockIdx.x;
  if (b == 0 && threadIdx.x == 0) *done = 0;
  if (b < nchunks) {
    chunk_hist_block(idx, A, n, chunk_hist, b, hist);
    return;
  }
  colsum_block(cs, nparts, (b - nchunks) % cx, (b - nchunks) / cx);
}

// 64 experts per block (256 threads); thread (e, q) covers chunks
// [q*G, (q+1)*G).
__device__ inline void column_scan_block(const int32_t* __restrict__ chunk_hist, int nchunks,
                                         int n, int32_t* __restrict__ chunk_base,
                                         int32_t* __restrict__ counts_pre) {
  __shared__ int32_t qs[4][64];
  const int el = threadIdx.x & 63, q = threadIdx.x >> 6;
  const int e = blockIdx.x * 64 + el;
  const int G = (nchunks + 3) / 4;
  const int c0 = q * G, c1 = min(nchunks, c0 + G);
  int sum = 0;
  if (e < n) {
#pragma unroll 8
    for (int c = c0; c < c1; ++c) sum += chunk_hist[(long long)c * n + e];
  }
  qs[q][el] = sum;
  __syncthreads();
  int run = 0;
  for (int r = 0; r < q; ++r) run += qs[r][el];
  if (e < n) {
#pragma unroll 8
    for (int c = c0; c < c1; ++c) {
      const int h = chunk_hist[(long long)c * n + e];
      chunk_base[(long long)c * n + e] = run;
      run += h;
    }
    if (q == 3) counts_pre[e] = run;
  }
}

// One block of kFinThreads threads; thread t owns the contiguous experts
// [t*per, t*per + per).
constexpr int kFinThreads = 256;
__device__ inline void finalize_block(const DispatchArgs& a) {
  __shared__ int32_t si[kFinThreads / 64];
  __shared__ double sd[kFinThreads / 64];
  const int n = a.n;
  const int per = (n + kFinThreads - 1) / kFinThreads;
  const int b = min(n, (int)threadIdx.x * per), e1 = min(n, b + per);
  int local = 0;
  for (int e = b; e < e1; ++e) {
    const long long c = a.counts_pre[e];
    const int kept = (int)(c < a.cap ? c : a.cap);
    a.counts[e] = kept;
    local += kept;
  }
  const int2 sc = block_exscan<kFinThreads>(local, si);
  int run = sc.x, nt = 0;
  for (int e = b; e < e1; ++e) {
    a.offsets[e] = run;
    const int kept = a.counts[e];
    run += kept;
    if (a.tile_bm > 0) nt += (kept + a.tile_bm - 1) / a.tile_bm;
  }
  if (threadIdx.x == kFinThreads - 1) a.offsets[n] = sc.y;
  if (a.tile_bm > 0) {
    const int2 tc = block_exscan<kFinThreads>(nt, si);
    int t = tc.x;
    int off = sc.x;
    for (int e = b; e < e1; ++e) {
      const int kept = a.counts[e];
      for (int m = 0; m < kept; m += a.tile_bm) {
        a.tile_expert[t] = e;
        a.tile_row0[t] = off + m;
        ++t;
      }
      off += kept;
    }
    if (threadIdx.x == kFinThreads - 1) *a.tile_count = tc.y;
    if (a.big_rows > 0) {
      int ns = 0, nb = 0;
      for (int e = b; e < e1; ++e) {
        const int kept = a.counts[e];
        if (kept >= a.big_rows) nb += (kept + kBigBM - 1) / kBigBM;
        else ns += (kept + a.tile_bm - 1) / a.tile_bm;
      }
      const int2 cs = block_exscan<kFinThreads>(ns, si);
      const int2 cb = block_exscan<kFinThreads>(nb, si);
      int ts = cs.x, tb = cb.x;
      off = sc.x;
      for (int e = b; e < e1; ++e) {
        const int kept = a.counts[e];
        const bool big = kept >= a.big_rows;
        const int bm = big ? kBigBM : a.tile_bm;
        const TileMap& tm = big ? a.big_map : a.small_map;
        int& t2 = big ? tb : ts;
        for (int m = 0; m < kept; m += bm) {
          tm.expert[t2] = e;
          tm.row0[t2] = off + m;
          ++t2;
        }
        off += kept;
      }
      if (threadIdx.x == kFinThreads - 1) {
        *a.small_map.count = cs.y;
        *a.big_map.count = cb.y;
      }
      if (a.split.out) {
        int big_r = 0, big_g = 0, small_e = 0, small_r = 0;
        for (int e = b; e < e1; ++e) {
          const int kept = a.counts[e];
          if (kept >= a.big_rows) {
            const int mt = (kept + kBigBM - 1) / kBigBM;
            big_r += mt * kBigBM;
            big_g += (mt + kBigGroupM - 1) / kBigGroupM;
          } else if (kept > 0) {
            ++small_e, small_r += kept;
          }
        }
        const int tb_rows = block_exscan<kFinThreads>(big_r, si).y;
        const int tb_groups = block_exscan<kFinThreads>(big_g, si).y;
        const int ts_exp = block_exscan<kFinThreads>(small_e, si).y;
        const int ts_rows = block_exscan<kFinThreads>(small_r, si).y;
        if (threadIdx.x < 2)
          a.split.out[threadIdx.x] =
              expert_cu_split(a.split.cus, tb_rows, tb_groups, ts_exp, ts_rows, a.split.d,
                              a.split.h, a.split.swiglu, (int)threadIdx.x);
      }
    }
  }
  if (a.losses)
    block_aux_losses<kFinThreads>(a.importance, a.load, a.counts_pre, a.gate_stats, a.T, a.k, n,
                                  a.w_imp, a.w_load, a.alpha, a.w_z, a.w_ent, a.losses, sd);
}

// The column scan in blocks of 64 experts; the last block to finish then
// runs the finalize, so the two take one launch.  "Last" is a ticket on
// `done` (set to 0 by the histogram launch before): each block makes its
// counts visible device-wide (a device-scope fence: writeback across the
// XCDs' L2s), then takes a ticket; the block that draws the last one fences
// again (invalidating stale lines) and reads every block's counts.  No block
// waits for another.
static_assert(kFinThreads == 256, "the scan and the finalize share the 256-thread block");
__global__ void zero_int_kernel(int32_t* __restrict__ p) { *p = 0; }
__global__ __launch_bounds__(256) void scan_finalize_kernel(const DispatchArgs a, int nchunks,
                                                            int32_t* __restrict__ done) {
  column_scan_block(a.chunk_hist, nchunks, a.n, a.chunk_base, a.counts_pre);
  __shared__ int last;
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) last = atomicAdd(done, 1) == (int)gridDim.x - 1;
  __syncthreads();
  if (!last) return;
  __threadfence();
  finalize_block(a);
}

// One wavefront per chunk.
__global__ __launch_bounds__(64) void permute_kernel(const int32_t* __restrict__ idx, long long A,
                                                     int k, int n, long long cap,
                                                     const int32_t* __restrict__ chunk_base,
                                                     const int32_t* __restrict__ offsets,
                                                     int32_t* __restrict__ perm,
                                                     int32_t* __restrict__ slot_pos) {
  extern __shared__ int32_t fill[];
  constexpr int G = kDispatchChunk / 64;
  const int lane = threadIdx.x;
  const long long c = blockIdx.x;
  const long long a0 = c * kDispatchChunk;
  int ev[G];  // the whole chunk's expert ids, loaded up front
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const long long a = a0 + g * 64 + lane;
    ev[g] = a < A ? idx[a] : -1;
  }
  for (int e = lane; e < n; e += 64) fill[e] = chunk_base[c * n + e];
  __syncthreads();
  // Bits of an expert id (n <= 2^nbits).
  int nbits = 0;
  while ((1 << nbits) < n) ++nbits;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const long long a = a0 + g * 64 + lane;
    const int e = ev[g];
    const bool ok = a < A && (unsigned)e < (unsigned)n;  // ids outside [0, n): dropped
    // Lanes holding the same expert: the valid lanes, narrowed by one ballot
    // per bit of the id; `before` counts those below this lane.
    unsigned long long same_mask = __ballot(ok);
    for (int b = 0; b < nbits; ++b) {
      const unsigned long long ones = __ballot((e >> b) & 1);
      same_mask &= ((e >> b) & 1) ? ones : ~ones;
    }
    const int same = __popcll(same_mask);
    const int before = (int)__builtin_amdgcn_mbcnt_hi(
        (unsigned)(same_mask >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)same_mask, 0u));
    int base = 0;
    if (ok) base = fill[e];
    __syncthreads();  // every lane has read fill[] before the leaders update it
    if (ok && before == 0) fill[e] = base + same;
    __syncthreads();
    if (ok) {
      const long long rank = (long long)base + before;
      if (rank < cap) {
        const int pos = offsets[e] + (int)rank;
        perm[pos] = (int)(a / k);
        slot_pos[a] = pos;
      } else {
        slot_pos[a] = -1;
      }
    } else if (a < A) {
      slot_pos[a] = -1;
    }
  }
}

// One wavefront per token; 8 elements per lane per step.
__global__ __launch_bounds__(256) void gather_kernel(const float* __restrict__ x,
                                                     const int32_t* __restrict__ slot_pos, int T,
                                                     int k, int d, int bf16_out,
                                                     void* __restrict__ out,
                                                     uint16_t* __restrict__ x_bf16) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* src = x + (long long)t * d;
  const int32_t* sp = slot_pos + (long long)t * k;
  for (int c = lane * 8; c < d; c += 64 * 8) {
    const f32x4 v0 = *(const f32x4*)(src + c);
    const f32x4 v1 = *(const f32x4*)(src + c + 4);
    uint4 pk = make_uint4(0u, 0u, 0u, 0u);
    if (bf16_out || x_bf16) {
      pk.x = bf16x2_bits(v0[0], v0[1]);
      pk.y = bf16x2_bits(v0[2], v0[3]);
      pk.z = bf16x2_bits(v1[0], v1[1]);
      pk.w = bf16x2_bits(v1[2], v1[3]);
    }
    if (x_bf16) *(uint4*)(x_bf16 + (long long)t * d + c) = pk;
    for (int s = 0; out && s < k; ++s) {
      const int row = sp[s];
      if (row < 0) continue;
      if (bf16_out) {
        *(uint4*)((uint16_t*)out + (long long)row * d + c) = pk;
      } else {
        float* dst = (float*)out + (long long)row * d + c;
        *(f32x4*)dst = v0;
        *(f32x4*)(dst + 4) = v1;
      }
    }
  }
}

// out[i] = bf16(x[i]), 8 elements per thread (elems is a multiple of 8).
__global__ __launch_bounds__(256) void to_bf16_kernel(const float* __restrict__ x, long long n8,
                                                      uint16_t* __restrict__ out) {
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n8;
       i += (long long)gridDim.x * 256) {
    const f32x4 v0 = *(const f32x4*)(x + i * 8);
    const f32x4 v1 = *(const f32x4*)(x + i * 8 + 4);
    uint4 pk;
    pk.x = bf16x2_bits(v0[0], v0[1]);
    pk.y = bf16x2_bits(v0[2], v0[3]);
    pk.z = bf16x2_bits(v1[0], v1[1]);
    pk.w = bf16x2_bits(v1[2], v1[3]);
    *(uint4*)(out + i * 8) = pk;
  }
}

// One segment of T rows: offsets2 = {0, T} and its M-tiles.
__global__ __launch_bounds__(256) void shared_tilemap_kernel(int T, int bm,
                                                             int32_t* __restrict__ offsets2,
                                                             int32_t* __restrict__ tile_expert,
                                                             int32_t* __restrict__ tile_row0,
                                                             int32_t* __restrict__ tile_count) {
  const int nt = (T + bm - 1) / bm;
  for (int t = threadIdx.x; t < nt; t += 256) {
    tile_expert[t] = 0;
    tile_row0[t] = t * bm;
  }
  if (threadIdx.x == 0) {
    offsets2[0] = 0;
    offsets2[1] = T;
    *tile_count = nt;
  }
}

// One thread per expert.  counts_pre[i] * n against T * k compares the
// count with the even share T*k/n exactly.
__global__ __launch_bounds__(256) void bias_update_kernel(const int32_t* __restrict__ counts_pre,
                                                          int n, long long tk, float gamma,
                                                          float* __restrict__ bias) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const long long c = (long long)counts_pre[i] * n;
  if (c > tk) bias[i] = bias[i] - gamma;
  else if (c < tk) bias[i] = bias[i] + gamma;
}

// Single block: the segments split by size into a small-tile and a
// big-tile map (see launch_tilemap_split).
__global__ __launch_bounds__(1024) void tilemap_split_kernel(const int32_t* __restrict__ offsets,
                                                             int n, int bm, int big_rows,
                                                             TileMap sm, TileMap bg,
                                                             CuSplit split) {
  __shared__ int32_t tsum[2][1024];
  const int per = (n + 1023) / 1024;
  const int b = threadIdx.x * per;
  int ns = 0, nb = 0;
  for (int i = 0; i < per && b + i < n; ++i) {
    const int rows = offsets[b + i + 1] - offsets[b + i];
    if (rows >= big_rows) nb += (rows + kBigBM - 1) / kBigBM;
    else ns += (rows + bm - 1) / bm;
  }
  tsum[0][threadIdx.x] = ns;
  tsum[1][threadIdx.x] = nb;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int v0 = threadIdx.x >= off ? tsum[0][threadIdx.x - off] : 0;
    const int v1 = threadIdx.x >= off ? tsum[1][threadIdx.x - off] : 0;
    __syncthreads();
    tsum[0][threadIdx.x] += v0;
    tsum[1][threadIdx.x] += v1;
    __syncthreads();
  }
  int ts = threadIdx.x ? tsum[0][threadIdx.x - 1] : 0;
  int tb = threadIdx.x ? tsum[1][threadIdx.x - 1] : 0;
  for (int i = 0; i < per && b + i < n; ++i) {
    const int e = b + i;
    const int r0 = offsets[e], rows = offsets[e + 1] - r0;
    const bool big = rows >= big_rows;
    const int tbm = big ? kBigBM : bm;
    const TileMap& tm = big ? bg : sm;
    int& t = big ? tb : ts;
    for (int m = 0; m < rows; m += tbm) {
      tm.expert[t] = e;
      tm.row0[t] = r0 + m;
      ++t;
    }
  }
  if (threadIdx.x == 1023) {
    *sm.count = tsum[0][1023];
    *bg.count = tsum[1][1023];
  }
  if (split.out) {
    // Padded rows and M-tile groups of the big experts, count and rows of the
    // small ones, summed in the same shared arrays (every thread has read its
    // prefix above).
    int v[4] = {0, 0, 0, 0};
    for (int i = 0; i < per && b + i < n; ++i) {
      const int rows = offsets[b + i + 1] - offsets[b + i];
      if (rows >= big_rows) {
        const int mt = (rows + kBigBM - 1) / kBigBM;
        v[0] += mt * kBigBM;
        v[3] += (mt + kBigGroupM - 1) / kBigGroupM;
      } else if (rows > 0) {
        v[1] += 1, v[2] += rows;
      }
    }
    int tot[4];
    for (int q = 0; q < 4; ++q) {
      __syncthreads();
      tsum[0][threadIdx.x] = v[q];
      __syncthreads();
      for (int off = 512; off > 0; off >>= 1) {
        if ((int)threadIdx.x < off) tsum[0][threadIdx.x] += tsum[0][threadIdx.x + off];
        __syncthreads();
      }
      tot[q] = tsum[0][0];
    }
    if (threadIdx.x < 2)
      split.out[threadIdx.x] = expert_cu_split(split.cus, tot[0], tot[3], tot[1], tot[2],
                                               split.d, split.h, split.swiglu, (int)threadIdx.x);
  }
}

// Single block: M-tiles of every expert segment, in expert order.
__global__ __launch_bounds__(1024) void tilemap_kernel(const int32_t* __restrict__ offsets, int n,
                                                       int bm, int32_t* __restrict__ tile_expert,
                                                       int32_t* __restrict__ tile_row0,
                                                       int32_t* __restrict__ tile_count) {
  __shared__ int32_t tsum[1024];
  const int per = (n + 1023) / 1024;
  const int b = threadIdx.x * per;
  int local = 0;
  for (int i = 0; i < per && b + i < n; ++i) {
    const int rows = offsets[b + i + 1] - offsets[b + i];
    local += (rows + bm - 1) / bm;
  }
  tsum[threadIdx.x] = local;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int v = threadIdx.x >= off ? tsum[threadIdx.x - off] : 0;
    __syncthreads();
    tsum[threadIdx.x] += v;
    __syncthreads();
  }
  int t = threadIdx.x ? tsum[threadIdx.x - 1] : 0;
  for (int i = 0; i < per && b + i < n; ++i) {
    const int e = b + i;
    const int r0 = offsets[e], rows = offsets[e + 1] - r0;
    for (int m = 0; m < rows; m += bm) {
      tile_expert[t] = e;
      tile_row0[t] = r0 + m;
      ++t;
    }
  }
  if (threadIdx.x == 1023) *tile_count = tsum[1023];
}

}  // namespace

hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t s) {
  const long long A = (long long)a.T * a.k;
  const int n = a.n;
  const int nchunks = (int)((A + kDispatchChunk - 1) / kDispatchChunk);
  const size_t shm = (size_t)n * sizeof(int32_t);
  // The scan + finalize launch's ticket: the int after the chunk bases,
  // zeroed by the histogram launch (or by a one-thread launch when there is
  // no histogram to take: no assignments and no column sums).
  int32_t* done = a.chunk_base + (long long)(nchunks > 0 ? nchunks : 1) * n;
  bool zeroed = false;
  if (a.colsum_fused) {
    ColsumArgs cs;
    int nmax;
    const int nv = colsum_pack(a.colsum, cs, nmax);
    const int cx = (nmax + 63) / 64;
    const int blocks = nchunks + cx * nv;
    if (blocks > 0) {
      ProfScope ps("dispatch_hist", s);
      hist_colsum_kernel<<<dim3(blocks), dim3(kColThreads), shm, s>>>(
          a.topk_idx, A, n, a.chunk_hist, nchunks, cs, a.colsum_nparts, cx > 0 ? cx : 1, done);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      zeroed = true;
    }
  } else if (nchunks > 0) {
    ProfScope ps("dispatch_hist", s);
    chunk_hist_kernel<<<dim3(nchunks), dim3(256), shm, s>>>(a.topk_idx, A, n, a.chunk_hist,
                                                             done);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    zeroed = true;
  }
  if (!zeroed) {
    zero_int_kernel<<<dim3(1), dim3(1), 0, s>>>(done);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    ProfScope ps("dispatch_scan_finalize", s);
    scan_finalize_kernel<<<dim3((n + 63) / 64), dim3(256), 0, s>>>(a, nchunks, done);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (nchunks > 0) {
    ProfScope ps("dispatch_permute", s);
    permute_kernel<<<dim3(nchunks), dim3(64), shm, s>>>(a.topk_idx, A, a.k, n, a.cap,
                                                         a.chunk_base, a.offsets, a.perm,
                                                         a.slot_pos);
    e = hipGetLastError();
  }
  return e;
}

hipError_t launch_gather(const float* x, const int32_t* slot_pos, int T, int k, int d,
                         int bf16_out, void* x_perm, uint16_t* x_bf16, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  ProfScope ps(x_perm ? "dispatch_gather" : "dispatch_gather_bf16", s);
  gather_kernel<<<dim3((T + 3) / 4), dim3(256), 0, s>>>(x, slot_pos, T, k, d, bf16_out, x_perm,
                                                        x_bf16);
  return hipGetLastError();
}

hipError_t launch_to_bf16(const float* x, long long elems, uint16_t* out, hipStream_t s) {
  const long long n8 = elems / 8;
  if (n8 <= 0) return hipSuccess;
  ProfScope ps("to_bf16", s);
  const long long blocks = std::min<long long>((n8 + 255) / 256, 4096);
  to_bf16_kernel<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(x, n8, out);
  return hipGetLastError();
}

hipError_t launch_shared_tilemap(int T, int bm, int32_t* offsets2, int32_t* tile_expert,
                                 int32_t* tile_row0, int32_t* tile_count, hipStream_t s) {
  ProfScope ps("shared_tilemap", s);
  shared_tilemap_kernel<<<dim3(1), dim3(256), 0, s>>>(T, bm, offsets2, tile_expert, tile_row0,
                                                      tile_count);
  return hipGetLastError();
}

hipError_t launch_bias_update(const int32_t* counts_pre, int n, int T, int k, float gamma,
                              float* bias, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  ProfScope ps("bias_update", s);
  bias_update_kernel<<<dim3((n + 255) / 256), dim3(256), 0, s>>>(counts_pre, n,
                                                                 (long long)T * k, gamma, bias);
  return hipGetLastError();
}

hipError_t launch_tilemap_split(const int32_t* offsets, int n, int bm, int big_rows,
                                TileMap small, TileMap big, CuSplit split, hipStream_t s) {
  ProfScope ps("ffn_tilemap", s);
  tilemap_split_kernel<<<dim3(1), dim3(1024), 0, s>>>(offsets, n, bm, big_rows, small, big,
                                                      split);
  return hipGetLastError();
}

hipError_t launch_tilemap(const int32_t* offsets, int n, int bm, int32_t* tile_expert,
                          int32_t* tile_row0, int32_t* tile_count, hipStream_t s) {
  ProfScope ps("ffn_tilemap", s);
  tilemap_kernel<<<dim3(1), dim3(1024), 0, s>>>(offsets, n, bm, tile_expert, tile_row0,
                                                tile_count);
  return hipGetLastError();
}

}  // namespace moe
