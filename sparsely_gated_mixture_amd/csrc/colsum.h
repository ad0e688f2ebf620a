// Fixed-order column sums of per-block partial vectors (the gate's
// Importance, Load and statistics partials), as one workgroup's body, so the
// same sums can run in their own launch or inside another small launch.
//
// out[j] = sum of part[p][j] over p.  64 columns per workgroup of 1024
// threads; 16 part-lanes per column each add every 16th partial in ascending
// order (coalesced rows, many loads in flight), then the lane sums are added
// in lane order: the same order on every call, whichever launch runs it.
#pragma once

#include <hip/hip_runtime.h>

#include "launch.h"

namespace moe {

constexpr int kColLanes = 16;
constexpr int kColThreads = 64 * kColLanes;

struct ColsumArgs {
  ColsumVec v[3];
};

// Packs the vectors with a part (in order) into `a`; returns how many there
// are and sets nmax to the longest one's n.
inline int colsum_pack(const ColsumVec* v, ColsumArgs& a, int& nmax) {
  int nv = 0;
  nmax = 0;
  a = ColsumArgs{};
  for (int i = 0; i < 3; ++i)
    if (v[i].part && v[i].n > 0) {
      a.v[nv++] = v[i];
      nmax = v[i].n > nmax ? v[i].n : nmax;
    }
  return nv;
}

// Columns [bx*64, bx*64 + 64) of vector `by`; kColThreads threads.
__device__ inline void colsum_block(const ColsumArgs& a, int nparts, int bx, int by) {
  __shared__ double sh[kColLanes][64];
  const float* part = a.v[by].part;
  float* out = a.v[by].out;
  const int n = a.v[by].n;
  const int c = threadIdx.x & 63, q = threadIdx.x >> 6;
  const int j = bx * 64 + c;
  double s = 0.0;
  if (j < n) {
#pragma unroll 8
    for (int p = q; p < nparts; p += kColLanes) s += (double)part[(long long)p * n + j];
  }
  sh[q][c] = s;
  __syncthreads();
  if (q == 0 && j < n) {
    double t = 0.0;
    for (int r = 0; r < kColLanes; ++r) t += sh[r][c];
    out[j] = (float)t;
  }
}

}  // namespace moe
