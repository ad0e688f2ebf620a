// Dispatch on gfx950: merge all positions routed to each expert into one
// contiguous batch (the notes on arXiv 1701.06538, "Engineering": all time
// steps merged into one batch; MoE survey, tufusi.com 3.2: expert capacity,
// overflow dropped to the residual).
//
// The T*k (token, slot) assignments are cut into chunks of kDispatchChunk.
//   1. chunk_hist_kernel: per-chunk expert histogram (integer LDS atomics,
//      whose result does not depend on their order).
//   2. column_scan_kernel: per expert, exclusive prefix over chunks, and the
//      total count (counts_pre).
//   3. offsets_kernel: counts = min(counts_pre, C), exclusive scan -> offsets.
//   4. permute_kernel: one wavefront walks its chunk in order, 64 slots at a
//      time; a slot's rank inside its group of 64 is the number of earlier
//      lanes with the same expert (found with wave-uniform readlanes), so
//      the resulting order is exactly (token, slot) order -- stable, and
//      independent of scheduling.
//   5. gather_kernel: x_perm[row] = x[perm[row]], converted to bf16 (RNE)
//      or copied as fp32.
#include "common.h"
#include "launch.h"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void chunk_hist_kernel(const int32_t* __restrict__ idx,
                                                         long long A, int n,
                                                         int32_t* __restrict__ chunk_hist) {
  extern __shared__ int32_t hist[];
  for (int e = threadIdx.x; e < n; e += 256) hist[e] = 0;
  __syncthreads();
  const long long a0 = (long long)blockIdx.x * kDispatchChunk;
  for (int i = threadIdx.x; i < kDispatchChunk; i += 256) {
    const long long a = a0 + i;
    if (a < A) atomicAdd(&hist[idx[a]], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < n; e += 256)
    chunk_hist[(long long)blockIdx.x * n + e] = hist[e];
}

__global__ __launch_bounds__(256) void column_scan_kernel(const int32_t* __restrict__ chunk_hist,
                                                          int nchunks, int n,
                                                          int32_t* __restrict__ chunk_base,
                                                          int32_t* __restrict__ counts_pre) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= n) return;
  int run = 0;
#pragma unroll 8
  for (int c = 0; c < nchunks; ++c) {
    const int h = chunk_hist[(long long)c * n + e];
    chunk_base[(long long)c * n + e] = run;
    run += h;
  }
  counts_pre[e] = run;
}

// Single block: counts = min(counts_pre, cap); offsets = exclusive scan.
__global__ __launch_bounds__(1024) void offsets_kernel(const int32_t* __restrict__ counts_pre,
                                                       int n, long long cap,
                                                       int32_t* __restrict__ counts,
                                                       int32_t* __restrict__ offsets) {
  __shared__ int32_t tsum[1024];
  const int per = (n + 1023) / 1024;
  const int b = threadIdx.x * per;
  int local = 0;
  for (int i = 0; i < per && b + i < n; ++i) {
    const long long c = counts_pre[b + i];
    local += (int)(c < cap ? c : cap);
  }
  tsum[threadIdx.x] = local;
  __syncthreads();
  // Hillis-Steele inclusive scan over the 1024 thread sums.
  for (int off = 1; off < 1024; off <<= 1) {
    const int v = threadIdx.x >= off ? tsum[threadIdx.x - off] : 0;
    __syncthreads();
    tsum[threadIdx.x] += v;
    __syncthreads();
  }
  int run = threadIdx.x ? tsum[threadIdx.x - 1] : 0;
  for (int i = 0; i < per && b + i < n; ++i) {
    const long long c = counts_pre[b + i];
    const int kept = (int)(c < cap ? c : cap);
    counts[b + i] = kept;
    offsets[b + i] = run;
    run += kept;
  }
  if (threadIdx.x == 1023) offsets[n] = tsum[1023];
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
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const long long a = a0 + g * 64 + lane;
    const bool ok = a < A;
    const int e = ev[g];
    int before = 0, same = 0;
    for (int j = 0; j < 64; ++j) {
      const int ej = __builtin_amdgcn_readlane(e, j);
      const int m = (ej == e) ? 1 : 0;
      same += m;
      before += (j < lane) ? m : 0;
    }
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
    }
  }
}

// One wavefront per row; 8 elements per lane per step.
__global__ __launch_bounds__(256) void gather_kernel(const float* __restrict__ x,
                                                     const int32_t* __restrict__ perm,
                                                     const int32_t* __restrict__ rows_dev,
                                                     int d, int bf16_out, void* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= *rows_dev) return;
  const float* src = x + (long long)perm[row] * d;
  for (int c = lane * 8; c < d; c += 64 * 8) {
    const f32x4 v0 = *(const f32x4*)(src + c);
    const f32x4 v1 = *(const f32x4*)(src + c + 4);
    if (bf16_out) {
      uint32_t w[4];
      w[0] = (uint32_t)f32_to_bf16(v0[0]) | ((uint32_t)f32_to_bf16(v0[1]) << 16);
      w[1] = (uint32_t)f32_to_bf16(v0[2]) | ((uint32_t)f32_to_bf16(v0[3]) << 16);
      w[2] = (uint32_t)f32_to_bf16(v1[0]) | ((uint32_t)f32_to_bf16(v1[1]) << 16);
      w[3] = (uint32_t)f32_to_bf16(v1[2]) | ((uint32_t)f32_to_bf16(v1[3]) << 16);
      uint4 pk = make_uint4(w[0], w[1], w[2], w[3]);
      *(uint4*)((uint16_t*)out + (long long)row * d + c) = pk;
    } else {
      float* dst = (float*)out + (long long)row * d + c;
      *(f32x4*)dst = v0;
      *(f32x4*)(dst + 4) = v1;
    }
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

hipError_t launch_dispatch(const int32_t* topk_idx, int T, int k, int n, long long cap,
                           int32_t* counts_pre, int32_t* counts, int32_t* offsets,
                           int32_t* perm, int32_t* slot_pos, int32_t* chunk_hist,
                           int32_t* chunk_base, hipStream_t s) {
  const long long A = (long long)T * k;
  const int nchunks = (int)((A + kDispatchChunk - 1) / kDispatchChunk);
  const size_t shm = (size_t)n * sizeof(int32_t);
  if (nchunks > 0) {
    ProfScope ps("dispatch_hist", s);
    chunk_hist_kernel<<<dim3(nchunks), dim3(256), shm, s>>>(topk_idx, A, n, chunk_hist);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    ProfScope ps("dispatch_colscan", s);
    column_scan_kernel<<<dim3((n + 255) / 256), dim3(256), 0, s>>>(chunk_hist, nchunks, n,
                                                                    chunk_base, counts_pre);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    ProfScope ps("dispatch_offsets", s);
    offsets_kernel<<<dim3(1), dim3(1024), 0, s>>>(counts_pre, n, cap, counts, offsets);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (nchunks > 0) {
    ProfScope ps("dispatch_permute", s);
    permute_kernel<<<dim3(nchunks), dim3(64), shm, s>>>(topk_idx, A, k, n, cap, chunk_base,
                                                         offsets, perm, slot_pos);
    e = hipGetLastError();
  }
  return e;
}

hipError_t launch_gather(const float* x, const int32_t* perm, const int32_t* rows_dev,
                         int max_rows, int d, int bf16_out, void* x_perm, hipStream_t s) {
  if (max_rows <= 0) return hipSuccess;
  ProfScope ps("dispatch_gather", s);
  gather_kernel<<<dim3((max_rows + 3) / 4), dim3(256), 0, s>>>(x, perm, rows_dev, d, bf16_out,
                                                               x_perm);
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
