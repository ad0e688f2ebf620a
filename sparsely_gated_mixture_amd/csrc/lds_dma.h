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
