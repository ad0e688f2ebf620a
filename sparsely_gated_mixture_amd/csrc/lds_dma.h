// Direct global -> LDS copies and their waits (gfx950), shared by the grouped
// GEMMs of the forward and the backward.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {
namespace {

// A 16-byte zero source for copies that fall outside an operand.
__device__ __attribute__((aligned(16))) const uint32_t kZeroChunk[4] = {0u, 0u, 0u, 0u};

// 16-byte global -> LDS copy.  Lane i of the wave writes LDS bytes
// [lds + 16 i, lds + 16 i + 16); `lds` must be wave-uniform.  The copy has no
// register result; its completion is tracked with vmcnt (wait_vm).
//
// The LDS address goes through m0, which the asm sets itself and lists as
// clobbered.  The compiler builtin for this copy is not used: the compiler
// counts its LDS write as pending at every workgroup barrier and drains all
// copies in flight there (s_waitcnt vmcnt(0) before each s_barrier), which
// would empty the copy ring at every K-step.  m0 is a reserved register that
// the compiler sets right before each instruction that reads it; in the
// kernels that include this header no compiler-generated instruction uses it
// at all (tests/test_isa.py checks the compiled code: every m0 reference is
// this asm's write, directly followed by its copy).  clang warns that a
// reserved register in a clobber list may not be preserved across the asm;
// that is the intent here, so the warning is silenced for this statement.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, off" ::"v"(g),
      "s"(lds)
      : "memory", "m0");
#pragma clang diagnostic pop
}

// dma16 with the non-temporal hint, for lines that no other copy will ask
// for again (a small expert's weight tile): they then do not push reusable
// lines out of L2.
__device__ __forceinline__ void dma16_stream(const void* g, uint32_t lds) {
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, off nt" ::"v"(g),
      "s"(lds)
      : "memory", "m0");
#pragma clang diagnostic pop
}

// 16-byte buffer -> LDS copy through a buffer descriptor (raw addressing
// with the descriptor's range check: an offset past its range copies zeros
// and touches no memory).  voff is the lane's byte offset, soff a
// wave-uniform one added to it; lane i writes LDS bytes [lds + 16 i, +16).
// Same m0 handling and the same reason for not using the compiler builtin
// as dma16; in addition, after such builtin copies the compiler inserts full
// vmcnt waits before LDS reads it cannot prove disjoint from the copies'
// destination, which would serialise a copy stream with the reads of the
// other LDS stage.
typedef uint32_t rsrc_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void bdma16(rsrc_t rsrc, int voff, int soff, uint32_t lds) {
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, %3 offen lds" ::"s"(lds),
      "v"(voff), "s"(rsrc), "s"(soff)
      : "memory", "m0");
#pragma clang diagnostic pop
}

// A raw buffer descriptor (byte addressing, range check) over `bytes` bytes
// from `base`, in scalar registers; `bytes` above 2^30 are clamped to 2^30.
__device__ __forceinline__ rsrc_t buffer_rsrc(const void* base, long long bytes) {
  const uint64_t b = (uint64_t)(uintptr_t)base;
  rsrc_t r;
  r.x = __builtin_amdgcn_readfirstlane((uint32_t)b);
  r.y = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32) & 0xffffu);
  r.z = __builtin_amdgcn_readfirstlane((uint32_t)(bytes < (1LL << 30) ? bytes : (1LL << 30)));
  r.w = 0x00020000u;
  return r;
}

// Wait until at most N vector memory operations of this wave are in flight.
// Loads complete in order, so this covers every copy issued more than N
// loads ago.
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// wait_vm<n>() for a run-time n in [0, MAX] (a wave-uniform value).
template <int MAX>
__device__ __forceinline__ void wait_vm_upto(int n) {
  if constexpr (MAX > 0) {
    if (n >= MAX) {
      wait_vm<MAX>();
      return;
    }
    wait_vm_upto<MAX - 1>(n);
  } else {
    wait_vm<0>();
  }
}

}  // namespace
}  // namespace moe
