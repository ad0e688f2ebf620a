// moe_gate_static: the flat gate (moe_gate) with the library's own scratch
// memory instead of a caller-supplied workspace, for callers that cannot
// allocate (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc).
//
// The scratch is a file-scope device array of kScratchBytes.  Every GPU the
// library runs on holds its own copy, at its own address, from the first use
// on that device until the process ends.  Host code never passes the array's
// name to a kernel (on the host it is a stand-in, not a device address): the
// first call on a device, with that device current, asks the runtime for the
// device address (hipGetSymbolAddress) and keeps it per device; the gate's
// kernels receive that address as their workspace.
//
// The call allocates nothing: no hipMalloc / hipFree and no allocating
// library routine.  The gate writes every scratch byte it later reads within
// the same call (the logits, the per-block Importance / Load / statistics
// partials), so nothing needs clearing between calls.  All calls on one GPU
// share its array: calls that overlap on one GPU (two streams, two threads)
// race on it, and the caller must order them.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "../../include/moe.h"
#include "launch.h"

namespace moe {
namespace {

// 48 MiB: the gate's logits [T, 2n] fp32 (one copy per K range when K is
// split) and its partial sums -- e.g. T = 8192 tokens with a noisy gate over
// 256 experts needs 16.8 MB; T = 4096 at d = 7168 over 256 experts (K in
// four ranges) 34 MB.
constexpr size_t kScratchBytes = (size_t)48 << 20;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

void* g_scratch[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];

}  // namespace
}  // namespace moe

extern "C" moe_status moe_gate_static(const moe_config* cfg, const float* x,
                                      const float* w_gate, const float* b_gate,
                                      const float* w_noise, const float* noise,
                                      int32_t* topk_idx, float* topk_w, float* importance,
                                      float* load, float* gate_stats, void* stream) {
  using namespace moe;
  const size_t need = gate_workspace_bytes(cfg);
  if (need == 0)  // an invalid config: moe_gate reports why, before any launch
    return moe_gate(cfg, x, w_gate, b_gate, w_noise, noise, topk_idx, topk_w, importance, load,
                    gate_stats, nullptr, 0, stream);
  char msg[256];
  if (need > kScratchBytes) {
    snprintf(msg, sizeof msg,
             "moe_gate_static: this config needs %zu bytes of scratch; the static scratch holds "
             "%zu (call moe_gate with a workspace instead)",
             need, kScratchBytes);
    return report_error(MOE_ERR_WORKSPACE, msg);
  }
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    snprintf(msg, sizeof msg, "moe_gate_static: hipGetDevice: %s", hipGetErrorString(e));
    return report_error(MOE_ERR_HIP, msg);
  }
  if (dev < 0 || dev >= kMaxDevices) {
    snprintf(msg, sizeof msg, "moe_gate_static: device %d is beyond the %d the scratch covers",
             dev, kMaxDevices);
    return report_error(MOE_ERR_UNSUPPORTED, msg);
  }
  // Once per device, with that device current: the device address of this
  // device's copy of the array.
  std::call_once(g_scratch_once[dev], [dev] {
    g_scratch_err[dev] = hipGetSymbolAddress(&g_scratch[dev], HIP_SYMBOL(scratch));
  });
  if (g_scratch_err[dev] != hipSuccess || g_scratch[dev] == nullptr) {
    snprintf(msg, sizeof msg, "moe_gate_static: hipGetSymbolAddress of the scratch: %s",
             hipGetErrorString(g_scratch_err[dev]));
    return report_error(MOE_ERR_HIP, msg);
  }
  return moe_gate(cfg, x, w_gate, b_gate, w_noise, noise, topk_idx, topk_w, importance, load,
                  gate_stats, g_scratch[dev], kScratchBytes, stream);
}
