// C ABI of the MoE layer (forward and backward): argument validation,
// workspace layout and the launch sequence of each stage.  Validation runs before any HIP call,
// so a failing call enqueues nothing.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "../../include/moe.h"
#include "launch.h"

using namespace moe;

namespace {

thread_local char g_err[512] = "";

moe_status fail(moe_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

#define HIP_TRY(expr)                                                              \
  do {                                                                             \
    hipError_t e_ = (expr);                                                        \
    if (e_ != hipSuccess)                                                          \
      return fail(MOE_ERR_HIP, "%s: %s", #expr, hipGetErrorString(e_));            \
  } while (0)

constexpr int kMaxGateN = 2048;     // experts per gate (64 lanes x 32 registers)
constexpr int kMaxExperts = 16384;  // dispatch histogram in LDS
constexpr int kMaxK = 64;           // one slot per lane
constexpr int kSecondaryBM = 64;    // row tile of the two-level secondary gate
constexpr int kF32ExpertBM = 64;
constexpr int kSplitRows = 128;    // experts with at least this many rows: the 256 x 256 GEMM

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Required pointer.  A buffer that holds no element (empty == true, e.g. a
// per-token array when T == 0) may be NULL.
moe_status need(const void* p, const char* name, bool empty = false) {
  if (!p && empty) return MOE_OK;
  if (!p) return fail(MOE_ERR_INVALID_ARG, "%s must not be NULL", name);
  if (!aligned16(p)) return fail(MOE_ERR_INVALID_ARG, "%s must be 16-byte aligned", name);
  return MOE_OK;
}
moe_status optional(const void* p, const char* name) {
  if (p && !aligned16(p)) return fail(MOE_ERR_INVALID_ARG, "%s must be 16-byte aligned", name);
  return MOE_OK;
}

#define CHECK(expr)                     \
  do {                                  \
    moe_status s_ = (expr);             \
    if (s_ != MOE_OK) return s_;        \
  } while (0)

moe_status validate(const moe_config* c) {
  if (!c) return fail(MOE_ERR_INVALID_ARG, "cfg must not be NULL");
  if (c->T < 0) return fail(MOE_ERR_INVALID_ARG, "T must be >= 0 (got %d)", c->T);
  if (c->d_model <= 0 || c->d_hidden <= 0)
    return fail(MOE_ERR_INVALID_ARG, "d_model and d_hidden must be positive");
  if (c->d_model % 8 || c->d_hidden % 8)
    return fail(MOE_ERR_UNSUPPORTED, "d_model (%d) and d_hidden (%d) must be multiples of 8",
                c->d_model, c->d_hidden);
  if (c->n_experts < 1) return fail(MOE_ERR_INVALID_ARG, "n_experts must be >= 1");
  if (c->k < 1 || c->k > c->n_experts)
    return fail(MOE_ERR_INVALID_ARG, "k must be in [1, n_experts] (k=%d, n=%d)", c->k,
                c->n_experts);
  if (c->k > kMaxK) return fail(MOE_ERR_UNSUPPORTED, "k must be <= %d", kMaxK);
  if (c->gate != MOE_GATE_TOPK_SOFTMAX && c->gate != MOE_GATE_SWITCH_TOP1 &&
      c->gate != MOE_GATE_SIGMOID_BIAS)
    return fail(MOE_ERR_INVALID_ARG, "unknown gate kind %d", c->gate);
  if (c->act != MOE_ACT_RELU && c->act != MOE_ACT_SWIGLU)
    return fail(MOE_ERR_INVALID_ARG, "unknown activation %d", c->act);
  if (c->expert_dtype != MOE_F32 && c->expert_dtype != MOE_BF16 && c->expert_dtype != MOE_FP8)
    return fail(MOE_ERR_INVALID_ARG, "unknown expert dtype %d", c->expert_dtype);
  if (c->expert_dtype == MOE_FP8 && (c->d_model % 64 || c->d_hidden % 64))
    return fail(MOE_ERR_UNSUPPORTED, "FP8 experts need d_model (%d) and d_hidden (%d) to be "
                "multiples of 64", c->d_model, c->d_hidden);
  if (c->gate == MOE_GATE_SWITCH_TOP1 && c->k != 1)
    return fail(MOE_ERR_INVALID_ARG, "the Switch router needs k = 1");
  if (c->act == MOE_ACT_SWIGLU && c->expert_dtype == MOE_F32)
    return fail(MOE_ERR_UNSUPPORTED, "SwiGLU experts are implemented for bf16 and FP8 only");
  if (!std::isfinite(c->capacity_factor))
    return fail(MOE_ERR_INVALID_ARG, "capacity_factor must be finite");
  if (c->d_hidden_shared < 0 || c->d_hidden_shared % 8)
    return fail(MOE_ERR_INVALID_ARG, "d_hidden_shared must be a non-negative multiple of 8");
  if (c->d_hidden_shared > 0 && c->expert_dtype != MOE_BF16)
    return fail(MOE_ERR_UNSUPPORTED, "the shared expert is implemented for bf16 experts only");
  if (c->n_experts > kMaxExperts)
    return fail(MOE_ERR_UNSUPPORTED, "n_experts must be <= %d", kMaxExperts);
  if ((long long)c->T * c->k > (1LL << 30))
    return fail(MOE_ERR_UNSUPPORTED, "T*k must be <= 2^30");
  if (c->n_groups < 0) return fail(MOE_ERR_INVALID_ARG, "n_groups must be >= 0");
  if (c->n_groups > 0) {
    const int a = c->n_groups;
    if (c->n_experts % a)
      return fail(MOE_ERR_INVALID_ARG, "n_experts (%d) must be a multiple of n_groups (%d)",
                  c->n_experts, a);
    if (c->gate != MOE_GATE_TOPK_SOFTMAX)
      return fail(MOE_ERR_INVALID_ARG, "the two-level layer uses the top-k softmax gate");
    if (c->d_hidden_shared > 0)
      return fail(MOE_ERR_UNSUPPORTED, "the shared expert is implemented for flat layers");
    if (c->k_groups < 1 || c->k_groups > a || c->k % c->k_groups)
      return fail(MOE_ERR_INVALID_ARG, "k_groups must be in [1, n_groups] and divide k");
    const int b = c->n_experts / a, k2 = c->k / c->k_groups;
    if (k2 > b) return fail(MOE_ERR_INVALID_ARG, "k / k_groups must be <= experts per group");
    if (a > kMaxGateN || b > kMaxGateN)
      return fail(MOE_ERR_UNSUPPORTED, "gates are limited to %d experts", kMaxGateN);
  } else if (c->n_experts > kMaxGateN) {
    return fail(MOE_ERR_UNSUPPORTED, "a flat gate is limited to %d experts", kMaxGateN);
  }
  return MOE_OK;
}

long long capacity(const moe_config& c) {
  if (!(c.capacity_factor > 0.f)) return (long long)1 << 62;
  // No expert can receive more than T*k slots, so a larger capacity is the
  // same as T*k; clamping first keeps the conversion defined for any finite
  // factor.
  const double all = (double)c.T * (double)c.k;
  const double cap = std::floor((double)c.capacity_factor * all / (double)c.n_experts);
  return (long long)std::min(cap, all);
}

long long round_up(long long v, long long m) { return (v + m - 1) / m * m; }

}  // namespace

moe_status moe::report_error(moe_status st, const char* msg) { return fail(st, "%s", msg); }

int moe::device_cus() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = 256;
    cache[dev] = cus;
  }
  return cache[dev];
}

namespace {

// A second stream per device and the two events that fork work onto it from
// the caller's stream and join it back (created on first use, kept until the
// process ends; default priority).
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  // Held from the fork to the join, so that calls from several host threads
  // on one device do not interleave their uses of the shared events (their
  // side-stream work runs one call after the other).
  std::mutex m;
};
// The current device's side stream, or null: it is created on first use,
// but not while `caller` is being captured into a graph (that call then runs
// the two classes one after the other).
SideStream* side_stream(hipStream_t caller) {
  static SideStream cache[64];
  static std::mutex init;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  SideStream& ss = cache[dev];
  std::lock_guard<std::mutex> lock(init);
  if (!ss.s) {
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(caller, &cap) != hipSuccess || cap != hipStreamCaptureStatusNone)
      return nullptr;
    hipStream_t st = nullptr;
    if (hipStreamCreateWithFlags(&st, hipStreamNonBlocking) != hipSuccess) return nullptr;
    if (hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&ss.join, hipEventDisableTiming) != hipSuccess)
      return nullptr;
    ss.s = st;
  }
  return &ss;
}

// The side-by-side share's inputs for config c, written to `out` (device);
// out stays null (no side-by-side run) unless the weights are bf16.
CuSplit cu_split_of(const moe_config& c, int32_t* out) {
  CuSplit sp{};
  sp.out = c.expert_dtype == MOE_BF16 ? out : nullptr;
  sp.cus = device_cus();
  sp.d = c.d_model;
  sp.h = c.d_hidden;
  sp.swiglu = c.act == MOE_ACT_SWIGLU;
  return sp;
}

// ---------------------------------------------------------------------------
// Workspace layout.  [stage scratch: max over gate / dispatch / ffn]
// [forward intermediates].  Stage calls use only the first part.
// ---------------------------------------------------------------------------
struct Region {
  size_t off = 0, bytes = 0;
};

struct Plan {
  // gate (flat or primary)
  int n_gate = 0, ldl = 0, gemm_bm = 128, rows_per_block = 16, nparts = 0;
  int gate_splits = 1;  // K-split of the flat / primary gate GEMM
  Region logits, part_imp, part_load, part_stats, prim_stats;
  // two-level extras
  int a = 0, b = 0, k1 = 0, k2 = 0, ldl2 = 0, max_tiles2 = 0;
  Region prim_idx, prim_w, prim_imp, prim_load, g_counts_pre, g_counts, g_offsets, g_perm,
      g_slot, g_chunk_hist, g_chunk_base, t2_expert, t2_row0, t2_count, part2_imp, part2_load,
      part2_stats;
  // dispatch
  int nchunks = 0;
  Region chunk_hist, chunk_base;
  // ffn
  int ffn_bm = 128, max_mtiles = 0;
  Region t_expert, t_row0, t_count, hidden;
  // experts split by size (big_rows > 0): fewer rows -> 128-row tiles of the
  // streaming GEMM (small map), more -> 256 x 256 tiles (big map)
  int big_rows = 0, max_mtiles_s = 0, max_mtiles_b = 0;
  Region ts_expert, ts_row0, ts_count, tb_expert, tb_row0, tb_count, t_split;
  size_t gate_bytes = 0, dispatch_bytes = 0, ffn_bytes = 0, stage_bytes = 0;
  // forward intermediates
  Region f_idx, f_w, f_imp, f_load, f_counts_pre, f_counts, f_offsets, f_perm, f_slot, f_xperm,
      f_yperm, f_tile_expert, f_tile_row0, f_tile_count, f_stats, f_ts_expert, f_ts_row0,
      f_ts_count, f_tb_expert, f_tb_row0, f_tb_count, f_split;
  // shared expert (d_hidden_shared > 0): bf16 copy of x, hidden, output, tile map
  int sh_tiles = 0;
  Region sh_xb, sh_hidden, sh_y, sh_te, sh_tr, sh_tc, sh_off;
  size_t total = 0;
};

struct Cursor {
  size_t at;
  Region take(size_t bytes) {
    Region r;
    r.off = at;
    r.bytes = bytes;
    at += (size_t)round_up((long long)bytes, 256);
    return r;
  }
};

// Experts that keep at least this many rows run on the 256 x 256-tile GEMM,
// the others on the 128-row one; 0: every expert on the 128-row GEMM.  The
// split pays where both products are long (K >= 2048 each: the fine-grained
// layer measured 17 % faster, 4.9 against 5.9 ms for the two GEMMs); with
// short K (d = 512, h = 1024) every split measured slower.  bf16 and FP8
// weights (fp32 experts run on their own GEMM).
int split_rows(const moe_config& c) {
  if (c.expert_dtype != MOE_BF16 && c.expert_dtype != MOE_FP8) return 0;
  return (c.d_model >= 2048 && c.d_hidden >= 2048) ? kSplitRows : 0;
}

// K-split of the flat (or primary) gate GEMM.  While its tiles number fewer
// than three per CU (the 64 x 64 kernel's occupancy on 256 CUs; one per CU
// for the 128 x 128 kernel), K is split into up to ceil(768 / tiles) (256 /
// tiles) ranges of at least 1024, every range non-empty, with the partial
// logits (one [T, ldl] copy per range) within 32 MiB.
int gate_splits(long long T, long long d, int n_gate, int bm, int ldl) {
  const long long tiles = ((T + bm - 1) / bm) * ((n_gate + bm - 1) / bm);
  const long long target = bm == 128 ? 256 : 768;
  if (tiles <= 0 || tiles >= target) return 1;
  long long s = (target + tiles - 1) / tiles;
  s = std::min(s, d / 1024);
  s = std::min(s, std::max(1LL, (32LL << 20) / (T * ldl * 4)));
  s = std::max(1LL, std::min(s, 8LL));
  while (s > 1 && (long long)gate_split_len((int)d, (int)s) * (s - 1) >= d) --s;
  return (int)s;
}

Plan make_plan(const moe_config& c) {
  Plan p;
  const long long T = c.T, d = c.d_model, h = c.d_hidden, n = c.n_experts, k = c.k;
  const long long A = T * k;
  const bool hier = c.n_groups > 0;
  p.n_gate = hier ? c.n_groups : c.n_experts;
  const int ncols = 2 * p.n_gate;  // clean | raw (the raw half is unused when noiseless)
  p.ldl = (int)round_up(ncols, 4);
  {
    // 128x128 tiles (8 waves) once they give every CU a tile, or at d >= 2048
    // where the K-split makes up the count (fewer re-reads of x and fewer
    // fragment reads per MFMA than 64x64); 64x64 otherwise.
    const long long t128 = ((T + 127) / 128) * ((ncols + 127) / 128);
    p.gemm_bm = t128 >= 256 || d >= 2048 ? 128 : 64;
    p.gate_splits = gate_splits(T, d, p.n_gate, p.gemm_bm, p.ldl);
  }
  {
    // one partial vector per block; at most 256 blocks (one per CU) once T
    // is large, so the column sums stay short; below that one row per wave,
    // so the blocks still reach every CU (fine-grained layer, T = 4096: 256
    // blocks, top-k 24 -> 17 us; with two rows per wave, 128 blocks)
    const long long w = topk_waves(p.n_gate);
    long long rpb = std::max(w, round_up((T + 255) / 256, w));
    p.rows_per_block = (int)rpb;
    p.nparts = (int)((T + rpb - 1) / rpb);
  }
  // gate scratch
  Cursor g{0};
  if (hier) {
    p.a = c.n_groups;
    p.b = c.n_experts / c.n_groups;
    p.k1 = c.k_groups;
    p.k2 = c.k / c.k_groups;
    p.ldl2 = (int)round_up(2 * p.b, 4);
    p.max_tiles2 = (int)((T * p.k1 + kSecondaryBM - 1) / kSecondaryBM + p.a);
    const long long logit_elems = std::max(p.gate_splits * T * p.ldl, T * p.k1 * p.ldl2);
    p.logits = g.take(logit_elems * 4);
    p.part_imp = g.take((size_t)p.nparts * p.a * 4);
    p.part_load = g.take((size_t)p.nparts * p.a * 4);
    p.part_stats = g.take((size_t)p.nparts * 2 * 4);
    p.prim_stats = g.take(2 * 4);
    p.prim_idx = g.take(T * p.k1 * 4);
    p.prim_w = g.take(T * p.k1 * 4);
    p.prim_imp = g.take(p.a * 4);
    p.prim_load = g.take(p.a * 4);
    p.g_counts_pre = g.take(p.a * 4);
    p.g_counts = g.take(p.a * 4);
    p.g_offsets = g.take((p.a + 1) * 4);
    p.g_perm = g.take(std::max(1LL, T * p.k1) * 4);
    p.g_slot = g.take(std::max(1LL, T * p.k1) * 4);
    const long long gchunks = (T * p.k1 + kDispatchChunk - 1) / kDispatchChunk;
    p.g_chunk_hist = g.take(std::max(1LL, gchunks) * p.a * 4);
    p.g_chunk_base = g.take((std::max(1LL, gchunks) * p.a + 1) * 4);  // + the scan's ticket
    p.t2_expert = g.take((size_t)p.max_tiles2 * 4);
    p.t2_row0 = g.take((size_t)p.max_tiles2 * 4);
    p.t2_count = g.take(4);
    p.part2_imp = g.take((size_t)p.max_tiles2 * p.b * 4);
    p.part2_load = g.take((size_t)p.max_tiles2 * p.b * 4);
    p.part2_stats = g.take((size_t)p.max_tiles2 * 2 * 4);
  } else {
    p.logits = g.take(p.gate_splits * T * p.ldl * 4);
    p.part_imp = g.take((size_t)p.nparts * n * 4);
    p.part_load = g.take((size_t)p.nparts * n * 4);
    p.part_stats = g.take((size_t)p.nparts * 2 * 4);
  }
  p.gate_bytes = g.at;
  // dispatch scratch
  Cursor dsp{0};
  p.nchunks = (int)((A + kDispatchChunk - 1) / kDispatchChunk);
  p.chunk_hist = dsp.take(std::max(1LL, (long long)p.nchunks) * n * 4);
  p.chunk_base = dsp.take((std::max(1LL, (long long)p.nchunks) * n + 1) * 4);  // + the ticket
  p.dispatch_bytes = dsp.at;
  // ffn scratch
  Cursor f{0};
  p.ffn_bm = c.expert_dtype != MOE_F32 ? kBf16BM : kF32ExpertBM;
  p.max_mtiles = (int)((A + p.ffn_bm - 1) / p.ffn_bm + n);
  p.t_expert = f.take((size_t)p.max_mtiles * 4);
  p.t_row0 = f.take((size_t)p.max_mtiles * 4);
  p.t_count = f.take(4);
  p.big_rows = split_rows(c);
  if (p.big_rows > 0) {
    p.max_mtiles_s = (int)((A + kBf16BM - 1) / kBf16BM + n);
    p.max_mtiles_b = (int)((A + kBigBM - 1) / kBigBM + n);
    p.ts_expert = f.take((size_t)p.max_mtiles_s * 4);
    p.ts_row0 = f.take((size_t)p.max_mtiles_s * 4);
    p.ts_count = f.take(4);
    p.tb_expert = f.take((size_t)p.max_mtiles_b * 4);
    p.tb_row0 = f.take((size_t)p.max_mtiles_b * 4);
    p.tb_count = f.take(4);
    p.t_split = f.take(2 * 4);  // one share per product
  }
  p.hidden = f.take(std::max(1LL, A) * h * (c.expert_dtype != MOE_F32 ? 2 : 4));
  p.ffn_bytes = f.at;
  p.stage_bytes = std::max(p.gate_bytes, std::max(p.dispatch_bytes, p.ffn_bytes));
  // forward intermediates
  Cursor w{p.stage_bytes};
  const long long A1 = std::max(1LL, A);
  p.f_idx = w.take(A1 * 4);
  p.f_w = w.take(A1 * 4);
  p.f_imp = w.take(n * 4);
  p.f_load = w.take(n * 4);
  p.f_counts_pre = w.take(n * 4);
  p.f_counts = w.take(n * 4);
  p.f_offsets = w.take((n + 1) * 4);
  p.f_perm = w.take(A1 * 4);
  p.f_slot = w.take(A1 * 4);
  p.f_xperm = w.take(A1 * d * (c.expert_dtype != MOE_F32 ? 2 : 4));
  p.f_yperm = w.take(A1 * d * 4);
  p.f_tile_expert = w.take((size_t)p.max_mtiles * 4);
  p.f_tile_row0 = w.take((size_t)p.max_mtiles * 4);
  p.f_tile_count = w.take(4);
  p.f_stats = w.take(2 * 4);
  if (p.big_rows > 0) {
    p.f_ts_expert = w.take((size_t)p.max_mtiles_s * 4);
    p.f_ts_row0 = w.take((size_t)p.max_mtiles_s * 4);
    p.f_ts_count = w.take(4);
    p.f_tb_expert = w.take((size_t)p.max_mtiles_b * 4);
    p.f_tb_row0 = w.take((size_t)p.max_mtiles_b * 4);
    p.f_tb_count = w.take(4);
    p.f_split = w.take(2 * 4);
  }
  if (c.d_hidden_shared > 0) {
    const long long hs = c.d_hidden_shared;
    p.sh_tiles = (int)((T + kBf16BM - 1) / kBf16BM + 1);
    p.sh_xb = w.take(std::max(1LL, T) * d * 2);
    p.sh_hidden = w.take(std::max(1LL, T) * hs * 2);
    p.sh_y = w.take(std::max(1LL, T) * d * 4);
    p.sh_te = w.take((size_t)p.sh_tiles * 4);
    p.sh_tr = w.take((size_t)p.sh_tiles * 4);
    p.sh_tc = w.take(4);
    p.sh_off = w.take(2 * 4);
  }
  p.total = w.at;
  return p;
}

template <typename Tp>
Tp* at(void* ws, const Region& r) {
  return (Tp*)((char*)ws + r.off);
}

moe_status check_ws(void* ws, size_t ws_bytes, size_t need_bytes, const char* what) {
  if (need_bytes == 0) return MOE_OK;
  if (!ws) return fail(MOE_ERR_WORKSPACE, "%s: ws must not be NULL", what);
  if (!aligned16(ws)) return fail(MOE_ERR_INVALID_ARG, "%s: ws must be 16-byte aligned", what);
  if (ws_bytes < need_bytes)
    return fail(MOE_ERR_WORKSPACE, "%s: workspace of %zu bytes is too small (needs %zu)", what,
                ws_bytes, need_bytes);
  return MOE_OK;
}

// ---------------------------------------------------------------------------
// Stages (arguments already validated).
// ---------------------------------------------------------------------------
moe_status run_gate(const moe_config& c, const Plan& p, const float* x, const float* w_gate,
                    const float* b_gate, const float* w_noise, const float* noise,
                    int32_t* topk_idx, float* topk_w, float* importance, float* load,
                    float* gate_stats, void* ws, hipStream_t s, ColsumVec* defer = nullptr,
                    uint16_t* x_bf16 = nullptr) {
  const int n = c.n_experts;
  const bool noisy = w_noise != nullptr;
  float* logits = at<float>(ws, p.logits);
  if (c.T > 0) {
    GemmF32Args g{};
    g.A = x;
    g.a_bf16 = x_bf16;  // optional: x in bf16, token order, as a by-product
    g.lda = c.d_model;
    g.B1 = w_gate;
    g.B2 = w_noise;
    g.n1 = n;
    g.N = noisy ? 2 * n : n;
    g.K = c.d_model;
    g.C = logits;
    g.ldc = p.ldl;
    g.M = c.T;
    g.mtiles = (c.T + p.gemm_bm - 1) / p.gemm_bm;
    g.max_mtiles = g.mtiles;
    g.ksplit = p.gate_splits;
    g.split_stride = (long long)c.T * p.ldl;
    HIP_TRY(launch_gemm_gate(g, p.gemm_bm, s));
  }
  TopkArgs t{};
  t.rows = c.T;
  t.n = n;
  t.k = c.k;
  t.switch_mode = c.gate == MOE_GATE_SWITCH_TOP1;
  t.sigmoid_mode = c.gate == MOE_GATE_SIGMOID_BIAS;
  t.noisy = noisy;
  t.logits = logits;
  t.ldl = p.ldl;
  t.bias = b_gate;
  t.noise = noise;
  t.topk_idx = topk_idx;
  t.topk_w = topk_w;
  t.part_imp = at<float>(ws, p.part_imp);
  t.part_load = noisy ? at<float>(ws, p.part_load) : nullptr;
  t.part_stats = gate_stats ? at<float>(ws, p.part_stats) : nullptr;
  t.rows_per_block = p.rows_per_block;
  t.nsplit = p.gate_splits;
  t.split_stride = (long long)c.T * p.ldl;
  HIP_TRY(launch_topk(t, s));
  const ColsumVec sums[3] = {ColsumVec{t.part_imp, n, importance}, ColsumVec{t.part_load, n, load},
                             ColsumVec{t.part_stats, 2, gate_stats}};
  if (defer) {  // the caller's dispatch runs them inside its histogram launch
    for (int i = 0; i < 3; ++i) defer[i] = sums[i];
    return MOE_OK;
  }
  HIP_TRY(launch_colsum(p.nparts, sums[0], sums[1], sums[2], s));
  return MOE_OK;
}

// logits2 (null: the primary's buffer, overwritten) receives the secondary
// logits; load_g (null: not kept) the per-group secondary loads [a, b].
moe_status run_gate_hier(const moe_config& c, const Plan& p, const float* x, const float* w_gate,
                         const float* b_gate, const float* w_noise, const float* noise,
                         const float* w_gate2, const float* w_noise2, const float* noise2,
                         int32_t* topk_idx, float* topk_w, float* importance, float* load,
                         float* gate_stats, void* ws, hipStream_t s, float* logits2 = nullptr,
                         float* load_g = nullptr) {
  const bool noisy = w_noise != nullptr;
  const int a = p.a, b = p.b, k1 = p.k1;
  float* logits = at<float>(ws, p.logits);
  if (!logits2) logits2 = logits;
  int32_t* prim_idx = at<int32_t>(ws, p.prim_idx);
  float* prim_w = at<float>(ws, p.prim_w);
  // 1. primary gate over the a groups
  if (c.T > 0) {
    GemmF32Args g{};
    g.A = x;
    g.lda = c.d_model;
    g.B1 = w_gate;
    g.B2 = w_noise;
    g.n1 = a;
    g.N = noisy ? 2 * a : a;
    g.K = c.d_model;
    g.C = logits;
    g.ldc = p.ldl;
    g.M = c.T;
    g.mtiles = (c.T + p.gemm_bm - 1) / p.gemm_bm;
    g.max_mtiles = g.mtiles;
    g.ksplit = p.gate_splits;
    g.split_stride = (long long)c.T * p.ldl;
    HIP_TRY(launch_gemm_gate(g, p.gemm_bm, s));
  }
  TopkArgs t{};
  t.rows = c.T;
  t.n = a;
  t.k = k1;
  t.noisy = noisy;
  t.logits = logits;
  t.ldl = p.ldl;
  t.bias = b_gate;
  t.noise = noise;
  t.topk_idx = prim_idx;
  t.topk_w = prim_w;
  t.part_imp = at<float>(ws, p.part_imp);
  t.part_load = noisy ? at<float>(ws, p.part_load) : nullptr;
  t.part_stats = gate_stats ? at<float>(ws, p.part_stats) : nullptr;
  t.rows_per_block = p.rows_per_block;
  t.nsplit = p.gate_splits;
  t.split_stride = (long long)c.T * p.ldl;
  HIP_TRY(launch_topk(t, s));
  HIP_TRY(launch_colsum(p.nparts, ColsumVec{t.part_imp, a, at<float>(ws, p.prim_imp)},
                        ColsumVec{t.part_load, a, at<float>(ws, p.prim_load)},
                        ColsumVec{t.part_stats, 2, at<float>(ws, p.prim_stats)}, s));
  // 2. rows of each group (tokens ascending)
  int32_t* g_counts_pre = at<int32_t>(ws, p.g_counts_pre);
  int32_t* g_offsets = at<int32_t>(ws, p.g_offsets);
  int32_t* g_perm = at<int32_t>(ws, p.g_perm);
  int32_t* t2e = at<int32_t>(ws, p.t2_expert);
  int32_t* t2r = at<int32_t>(ws, p.t2_row0);
  int32_t* t2c = at<int32_t>(ws, p.t2_count);
  {
    DispatchArgs da{};
    da.topk_idx = prim_idx;
    da.T = c.T;
    da.k = k1;
    da.n = a;
    da.cap = (long long)1 << 62;
    da.counts_pre = g_counts_pre;
    da.counts = at<int32_t>(ws, p.g_counts);
    da.offsets = g_offsets;
    da.perm = g_perm;
    da.slot_pos = at<int32_t>(ws, p.g_slot);
    da.chunk_hist = at<int32_t>(ws, p.g_chunk_hist);
    da.chunk_base = at<int32_t>(ws, p.g_chunk_base);
    da.tile_bm = kSecondaryBM;
    da.tile_expert = t2e;
    da.tile_row0 = t2r;
    da.tile_count = t2c;
    HIP_TRY(launch_dispatch(da, s));
  }
  // 3. secondary logits: each group's own gate over its rows
  {
    GemmF32Args g{};
    g.A = x;
    g.lda = c.d_model;
    g.rowmap = g_perm;
    g.B1 = w_gate2;
    g.B2 = w_noise2;
    g.strideB1 = (long long)b * c.d_model;
    g.strideB2 = (long long)b * c.d_model;
    g.n1 = b;
    g.N = w_noise2 ? 2 * b : b;
    g.K = c.d_model;
    g.C = logits2;
    g.ldc = p.ldl2;
    g.tile_expert = t2e;
    g.tile_row0 = t2r;
    g.offsets = g_offsets;
    g.tile_count = t2c;
    g.max_mtiles = p.max_tiles2;
    g.prof_name = "gate2_gemm_bf16x6";
    HIP_TRY(launch_gemm_gate(g, kSecondaryBM, s));
  }
  // 4. secondary top-k per (token, primary slot) row
  TopkArgs u{};
  u.n = b;
  u.k = p.k2;
  u.noisy = w_noise2 != nullptr;
  u.logits = logits2;
  u.ldl = p.ldl2;
  u.noise = noise2;
  u.topk_idx = topk_idx;
  u.topk_w = topk_w;
  u.part_imp = at<float>(ws, p.part2_imp);
  u.part_load = u.noisy ? at<float>(ws, p.part2_load) : nullptr;
  u.part_stats = gate_stats ? at<float>(ws, p.part2_stats) : nullptr;
  u.row_token = g_perm;
  u.prim_idx = prim_idx;
  u.prim_w = prim_w;
  u.k1 = k1;
  u.tile_expert = t2e;
  u.tile_row0 = t2r;
  u.offsets = g_offsets;
  u.tile_count = t2c;
  u.max_tiles = p.max_tiles2;
  u.tile_rows = kSecondaryBM;
  HIP_TRY(launch_topk(u, s));
  // 5. two-level importance / load vectors
  const bool both_noisy = noisy && w_noise2 != nullptr;
  HIP_TRY(launch_hier_finalize(u.part_imp, both_noisy ? u.part_load : nullptr, t2e, t2c,
                               g_counts_pre, at<float>(ws, p.prim_load), a, b, importance,
                               both_noisy ? load : nullptr, both_noisy ? load_g : nullptr, s));
  if (gate_stats)
    HIP_TRY(launch_hier_stats(at<float>(ws, p.prim_stats), u.part_stats, t2c, gate_stats, s));
  return MOE_OK;
}

// Optional extras of the layer forward (fused into the dispatch finalize):
// the grouped GEMM's tile map and the auxiliary losses.
struct ForwardExtras {
  int32_t* tile_expert = nullptr;
  int32_t* tile_row0 = nullptr;
  int32_t* tile_count = nullptr;
  int big_rows = 0;  // > 0: the dispatch also writes the size-split maps
  TileMap small_map{}, big_map{};
  int32_t* cu_split = nullptr;  // with big_rows: where the dispatch writes the CU share
  float* losses = nullptr;
  const float* importance = nullptr;
  const float* load = nullptr;
  const float* gate_stats = nullptr;
  uint16_t* x_bf16 = nullptr;  // x in bf16, token order, written by the gather
  bool x_bf16_written = false;  // ... or already by the gate GEMM
  // Non-null: GEMM 1 reads merged row r as row row_token[r] (= perm) of the
  // token-order x_bf16, and the gather writes no x_perm.
  const int32_t* row_token = nullptr;
  // The gate's column sums, deferred into the histogram launch (run_gate's
  // `defer`), when colsum_fused.
  ColsumVec colsum[3] = {};
  bool colsum_fused = false;
};

moe_status run_dispatch(const moe_config& c, const Plan& p, const int32_t* topk_idx,
                        const float* x, int32_t* counts_pre, int32_t* counts, int32_t* offsets,
                        int32_t* perm, int32_t* slot_pos, void* x_perm, void* ws, hipStream_t s,
                        const ForwardExtras* fx = nullptr) {
  DispatchArgs da{};
  da.topk_idx = topk_idx;
  da.T = c.T;
  da.k = c.k;
  da.n = c.n_experts;
  da.cap = capacity(c);
  da.counts_pre = counts_pre;
  da.counts = counts;
  da.offsets = offsets;
  da.perm = perm;
  da.slot_pos = slot_pos;
  da.chunk_hist = at<int32_t>(ws, p.chunk_hist);
  da.chunk_base = at<int32_t>(ws, p.chunk_base);
  if (fx) {
    da.tile_bm = p.ffn_bm;
    da.tile_expert = fx->tile_expert;
    da.tile_row0 = fx->tile_row0;
    da.tile_count = fx->tile_count;
    da.big_rows = fx->big_rows;
    da.small_map = fx->small_map;
    da.big_map = fx->big_map;
    if (fx->big_rows > 0) da.split = cu_split_of(c, fx->cu_split);
    da.losses = fx->losses;
    da.importance = fx->importance;
    da.load = fx->load;
    da.gate_stats = fx->gate_stats;
    da.w_imp = c.w_importance;
    da.w_load = c.w_load;
    da.alpha = c.alpha_switch;
    da.w_z = c.w_z;
    da.w_ent = c.w_entropy;
    if (fx->colsum_fused) {
      for (int i = 0; i < 3; ++i) da.colsum[i] = fx->colsum[i];
      da.colsum_nparts = p.nparts;
      da.colsum_fused = 1;
    }
  }
  HIP_TRY(launch_dispatch(da, s));
  uint16_t* xb = fx && !fx->x_bf16_written ? fx->x_bf16 : nullptr;
  if (x_perm || xb)
    HIP_TRY(launch_gather(x, slot_pos, c.T, c.k, c.d_model, c.expert_dtype != MOE_F32, x_perm, xb,
                          s));
  return MOE_OK;
}

// GEMM 1 of the layer forward reading its rows through perm (`x_perm` is then
// the token-order bf16 x).
void set_row_token(GemmBf16Args& g, const moe_config& c, const ForwardExtras* fx) {
  if (!fx || !fx->row_token) return;
  g.row_token = fx->row_token;
  g.row_token_n = (int)((long long)c.T * c.k);
  g.a_rows = c.T;
}

// `fx` (layer forward) carries a tile map the dispatch already wrote;
// otherwise the tile map is built here from `offsets`.
moe_status run_ffn(const moe_config& c, const Plan& p, const void* x_perm,
                   const int32_t* offsets, const void* w1, const float* b1, const void* w3,
                   const void* w2, const float* b2, float* y_perm, void* ws, hipStream_t s,
                   const ForwardExtras* fx = nullptr, bool y_bf16 = false) {
  const int n = c.n_experts, d = c.d_model, h = c.d_hidden;
  int32_t* te = fx ? fx->tile_expert : at<int32_t>(ws, p.t_expert);
  int32_t* tr = fx ? fx->tile_row0 : at<int32_t>(ws, p.t_row0);
  int32_t* tc = fx ? fx->tile_count : at<int32_t>(ws, p.t_count);
  void* hidden = at<void>(ws, p.hidden);
  if (p.big_rows > 0) {
    // Experts split by size: the 128-row GEMM over the small map, the 256 x
    // 256 GEMM over the big map; the two cover disjoint rows.
    TileMap sm{at<int32_t>(ws, p.ts_expert), at<int32_t>(ws, p.ts_row0),
               at<int32_t>(ws, p.ts_count)};
    TileMap bg{at<int32_t>(ws, p.tb_expert), at<int32_t>(ws, p.tb_row0),
               at<int32_t>(ws, p.tb_count)};
    int32_t* share = at<int32_t>(ws, p.t_split);
    if (fx && fx->big_rows > 0) {
      sm = fx->small_map;
      bg = fx->big_map;
      share = fx->cu_split;
    } else {
      HIP_TRY(launch_tilemap_split(offsets, n, kBf16BM, p.big_rows, sm, bg,
                                   cu_split_of(c, share), s));
    }
    const bool fp8 = c.expert_dtype == MOE_FP8;
    GemmBf16Args g{};
    g.A = (const uint16_t*)x_perm;
    g.lda = d;
    g.B1 = w1;
    g.B3 = w3;
    g.strideB = fp8 ? (long long)h * d + 4LL * h : (long long)h * d * 2;
    g.fp8 = fp8;
    g.N = h;
    g.K = d;
    g.C = hidden;
    g.ldc = h;
    g.bias = b1;
    g.offsets = offsets;
    g.num_cus = device_cus();
    set_row_token(g, c, fx);
    GemmBf16Args g2 = g;
    g2.row_token = nullptr;
    g2.A = (const uint16_t*)hidden;
    g2.lda = h;
    g2.B1 = w2;
    g2.B3 = nullptr;
    g2.strideB = fp8 ? (long long)d * h + 4LL * d : (long long)d * h * 2;
    g2.N = d;
    g2.K = h;
    g2.C = y_perm;
    g2.ldc = d;
    g2.bias = b2;
    const int epi1 = c.act == MOE_ACT_SWIGLU ? EPI_SWIGLU_BF16 : EPI_RELU_BF16;
    const int epi2 = y_bf16 ? EPI_IDENT_BF16 : EPI_IDENT_F32;
    // bf16 weights: the small experts' chain runs on the side stream beside
    // the big experts' chain on `s`, each kernel on its share of the CUs.
    // FP8 weights (or no side stream): one after the other, each on the
    // whole grid.
    SideStream* ss = c.expert_dtype == MOE_BF16 ? side_stream(s) : nullptr;
    std::unique_lock<std::mutex> side_lock;
    if (ss) {
      side_lock = std::unique_lock<std::mutex>(ss->m);
      HIP_TRY(hipEventRecord(ss->fork, s));
      HIP_TRY(hipStreamWaitEvent(ss->s, ss->fork, 0));
    }
    for (int prod = 0; prod < 2; ++prod) {
      const GemmBf16Args* a = prod == 0 ? &g : &g2;
      GemmBf16Args as = *a, ab = *a;
      as.tile_expert = sm.expert;
      as.tile_row0 = sm.row0;
      as.tile_count = sm.count;
      as.max_mtiles = p.max_mtiles_s;
      as.b_stream = 1;  // the small map's experts hold fewer rows than one M-tile
      ab.tile_expert = bg.expert;
      ab.tile_row0 = bg.row0;
      ab.tile_count = bg.count;
      ab.max_mtiles = p.max_mtiles_b;
      if (ss) {
        as.cu_split = ab.cu_split = share + prod;
        as.cu_big = 0;
        ab.cu_big = 1;
      }
      const int epi = prod == 0 ? epi1 : epi2;
      HIP_TRY(launch_gemm_bf16(as, epi, ss ? ss->s : s));
      HIP_TRY(launch_gemm_big(ab, epi, s));
    }
    if (ss) {
      HIP_TRY(hipEventRecord(ss->join, ss->s));
      HIP_TRY(hipStreamWaitEvent(s, ss->join, 0));
    }
    return MOE_OK;
  }
  if (!fx) HIP_TRY(launch_tilemap(offsets, n, p.ffn_bm, te, tr, tc, s));
  if (c.expert_dtype != MOE_F32) {
    const bool fp8 = c.expert_dtype == MOE_FP8;
    GemmBf16Args g{};
    g.A = (const uint16_t*)x_perm;
    g.lda = d;
    g.B1 = w1;
    g.B3 = w3;
    g.strideB = fp8 ? (long long)h * d + 4LL * h : (long long)h * d * 2;
    g.fp8 = fp8;
    g.N = h;
    g.K = d;
    g.C = hidden;
    g.ldc = h;
    g.bias = b1;
    g.tile_expert = te;
    g.tile_row0 = tr;
    g.offsets = offsets;
    g.tile_count = tc;
    g.max_mtiles = p.max_mtiles;
    g.num_cus = device_cus();
    set_row_token(g, c, fx);
    HIP_TRY(launch_gemm_bf16(g, c.act == MOE_ACT_SWIGLU ? EPI_SWIGLU_BF16 : EPI_RELU_BF16, s));
    GemmBf16Args g2 = g;
    g2.row_token = nullptr;
    g2.A = (const uint16_t*)hidden;
    g2.lda = h;
    g2.B1 = w2;
    g2.B3 = nullptr;
    g2.strideB = fp8 ? (long long)d * h + 4LL * d : (long long)d * h * 2;
    g2.N = d;
    g2.K = h;
    g2.C = y_perm;
    g2.ldc = d;
    g2.bias = b2;
    HIP_TRY(launch_gemm_bf16(g2, y_bf16 ? EPI_IDENT_BF16 : EPI_IDENT_F32, s));
  } else {
    GemmF32Args g{};
    g.A = (const float*)x_perm;
    g.lda = d;
    g.B1 = (const float*)w1;
    g.strideB1 = (long long)h * d;
    g.n1 = h;
    g.N = h;
    g.K = d;
    g.C = (float*)hidden;
    g.ldc = h;
    g.bias = b1;
    g.stride_bias = h;
    g.relu = 1;
    g.tile_expert = te;
    g.tile_row0 = tr;
    g.offsets = offsets;
    g.tile_count = tc;
    g.max_mtiles = p.max_mtiles;
    HIP_TRY(launch_gemm_f32(g, kF32ExpertBM, s));
    GemmF32Args g2 = g;
    g2.A = (const float*)hidden;
    g2.lda = h;
    g2.B1 = (const float*)w2;
    g2.strideB1 = (long long)d * h;
    g2.n1 = d;
    g2.N = d;
    g2.K = h;
    g2.C = y_perm;
    g2.ldc = d;
    g2.bias = b2;
    g2.stride_bias = d;
    g2.relu = 0;
    HIP_TRY(launch_gemm_f32(g2, kF32ExpertBM, s));
  }
  return MOE_OK;
}

// The shared expert over all T rows of x_bf16: a one-segment tile map, then
// the same grouped GEMMs as the routed experts.
moe_status run_shared_ffn(const moe_config& c, const Plan& p, const uint16_t* xb,
                          const void* ws1, const void* ws3, const void* ws2, float* y_shared,
                          void* ws, hipStream_t s) {
  if (c.T == 0) return MOE_OK;
  const int d = c.d_model, hs = c.d_hidden_shared;
  int32_t* off = at<int32_t>(ws, p.sh_off);
  int32_t* te = at<int32_t>(ws, p.sh_te);
  int32_t* tr = at<int32_t>(ws, p.sh_tr);
  int32_t* tc = at<int32_t>(ws, p.sh_tc);
  uint16_t* hidden = at<uint16_t>(ws, p.sh_hidden);
  // One segment of T rows: the 256 x 256 GEMM where both products are long
  // (as for the routed experts, split_rows), else the 128-row one.
  const bool big = c.d_model >= 2048 && hs >= 2048;
  HIP_TRY(launch_shared_tilemap(c.T, big ? kBigBM : kBf16BM, off, te, tr, tc, s));
  GemmBf16Args g{};
  g.A = xb;
  g.lda = d;
  g.B1 = ws1;
  g.B3 = ws3;
  g.strideB = 0;
  g.N = hs;
  g.K = d;
  g.C = hidden;
  g.ldc = hs;
  g.tile_expert = te;
  g.tile_row0 = tr;
  g.offsets = off;
  g.tile_count = tc;
  g.max_mtiles = p.sh_tiles;
  g.num_cus = device_cus();
  g.shared = 1;
  const int epi1 = c.act == MOE_ACT_SWIGLU ? EPI_SWIGLU_BF16 : EPI_RELU_BF16;
  if (big) {
    g.prof_name = c.act == MOE_ACT_SWIGLU ? "shared_big_swiglu" : "shared_big_relu";
    HIP_TRY(launch_gemm_big(g, epi1, s));
  } else {
    HIP_TRY(launch_gemm_bf16(g, epi1, s));
  }
  GemmBf16Args g2 = g;
  g2.A = hidden;
  g2.lda = hs;
  g2.B1 = ws2;
  g2.B3 = nullptr;
  g2.N = d;
  g2.K = hs;
  g2.C = y_shared;
  g2.ldc = d;
  if (big) {
    g2.prof_name = "shared_big_out";
    HIP_TRY(launch_gemm_big(g2, EPI_IDENT_F32, s));
  } else {
    HIP_TRY(launch_gemm_bf16(g2, EPI_IDENT_F32, s));
  }
  return MOE_OK;
}

moe_status check_shared_ptrs(const moe_config& c, const void* ws1, const void* ws3,
                             const void* ws2) {
  CHECK(need(ws1, "ws1 (shared expert)"));
  CHECK(need(ws2, "ws2 (shared expert)"));
  if (c.act == MOE_ACT_SWIGLU) CHECK(need(ws3, "ws3 (shared SwiGLU expert)"));
  else CHECK(optional(ws3, "ws3"));
  return MOE_OK;
}

moe_status check_gate_ptrs(const moe_config& c, const float* x, const float* w_gate,
                           const float* b_gate, const float* w_noise, const float* noise) {
  CHECK(need(x, "x", c.T == 0));
  CHECK(need(w_gate, "w_gate"));
  CHECK(optional(b_gate, "b_gate"));
  CHECK(optional(w_noise, "w_noise"));
  if (w_noise) CHECK(need(noise, "noise (required with w_noise)", c.T == 0));
  if (w_noise && c.gate == MOE_GATE_SWITCH_TOP1)
    return fail(MOE_ERR_INVALID_ARG, "the Switch router is noiseless (w_noise must be NULL)");
  if (w_noise && c.gate == MOE_GATE_SIGMOID_BIAS)
    return fail(MOE_ERR_INVALID_ARG, "the sigmoid gate is noiseless (w_noise must be NULL)");
  return MOE_OK;
}


// ---------------------------------------------------------------------------
// Backward workspace: the forward's plan, with the gate logits and the hidden
// activations moved out of the stage scratch (the backward reads them after
// later stages ran), followed by the backward's own buffers.
// ---------------------------------------------------------------------------
struct BwdPlan {
  Plan f;  // forward plan (logits / hidden relocated)
  int M = 0, ldk = 0, splits = 0, tps = 0, hw = 0, hws = 0;
  Region losses, dG, dout, dimp, dload, coef, dlogits, part_db, dpre, a_pre, b_pre, du_perm,
      dx_gate, wt, wpart, a_s, b_s, dout_s, dpre_s, du_s;
  // two-level layer: secondary logits and their gradients, the split slot
  // gradients, the factorised load's parts, the secondary rows' dx
  Region logits2, dlogits2, dG1, dG2, dload_p, dload_g, load_g, du2;
  size_t total = 0;
};

BwdPlan make_bwd_plan(const moe_config& c) {
  BwdPlan b;
  b.f = make_plan(c);
  const long long T = c.T, d = c.d_model, h = c.d_hidden, n = c.n_experts;
  const long long A1 = std::max(1LL, (long long)T * c.k);
  const long long T1 = std::max(1LL, T);
  const bool swiglu = c.act == MOE_ACT_SWIGLU;
  Cursor w{b.f.total};
  const long long esz = c.expert_dtype == MOE_F32 ? 4 : 2;  // activations and their gradients
  b.f.logits = w.take(b.f.gate_splits * T1 * b.f.ldl * 4);
  b.f.hidden = w.take(A1 * h * esz);
  b.losses = w.take(8 * 4);
  b.dG = w.take(A1 * 4);
  b.dout = w.take(A1 * d * esz);
  const long long ng = b.f.n_gate;  // the flat or primary gate's width
  b.dimp = w.take(n * 4);
  b.dload = w.take(n * 4);
  b.coef = w.take(4 * 4);
  b.dlogits = w.take(T1 * b.f.ldl * 4);
  b.part_db = w.take((size_t)std::max(1, b.f.nparts) * ng * 4);
  b.hw = swiglu ? 2 * (int)h : (int)h;  // width of the hidden-layer gradient rows
  b.dpre = w.take(A1 * b.hw * esz);
  if (swiglu) {
    b.a_pre = w.take(A1 * h * 4);
    b.b_pre = w.take(A1 * h * 4);
  }
  b.du_perm = w.take(A1 * d * 4);
  b.dx_gate = w.take(T1 * d * 4);
  b.M = (int)ng * 2;  // dclean | draw columns of dlogits (draw unused when noiseless)
  b.ldk = (int)round_up(b.M, 4);
  b.wt = w.take(d * b.ldk * 4);
  b.splits = gate_wgrad_splits((int)T, (int)d, b.M);
  b.tps = (int)std::max(1LL, (T + b.splits - 1) / b.splits);
  b.wpart = w.take((size_t)b.splits * b.M * d * 4);
  if (c.n_groups > 0) {
    const long long rows2 = std::max(1LL, T * b.f.k1);
    b.logits2 = w.take(rows2 * b.f.ldl2 * 4);
    b.dlogits2 = w.take(rows2 * b.f.ldl2 * 4);
    b.dG1 = w.take(rows2 * 4);
    b.dG2 = w.take(A1 * 4);
    b.dload_p = w.take(ng * 4);
    b.dload_g = w.take(n * 4);
    b.load_g = w.take(n * 4);
    b.du2 = w.take(rows2 * d * 4);
  }
  if (c.d_hidden_shared > 0) {
    const long long hs = c.d_hidden_shared;
    b.hws = swiglu ? 2 * (int)hs : (int)hs;
    if (swiglu) {
      b.a_s = w.take(T1 * hs * 4);
      b.b_s = w.take(T1 * hs * 4);
    }
    b.dout_s = w.take(T1 * d * 2);
    b.dpre_s = w.take(T1 * b.hws * 2);
    b.du_s = w.take(T1 * d * 4);
  }
  b.total = w.at;
  return b;
}

moe_status validate_bwd(const moe_config& c) {
  if (c.expert_dtype == MOE_FP8)
    return fail(MOE_ERR_UNSUPPORTED, "the backward pass needs bf16 or fp32 experts");
  if (c.d_model % 64 || c.d_hidden % 64 || c.d_hidden_shared % 64)
    return fail(MOE_ERR_UNSUPPORTED,
                "the backward pass needs d_model, d_hidden and d_hidden_shared multiples of 64");
  return MOE_OK;
}

// First GEMM of an expert FFN for the backward: the hidden activations (bf16)
// and, for SwiGLU, the two fp32 pre-activations they come from.
moe_status bwd_hidden(const moe_config& c, GemmBf16Args g, int h, uint16_t* hidden, float* a_pre,
                      float* b_pre, long long elems, hipStream_t s) {
  g.N = h;
  g.ldc = h;
  if (c.act == MOE_ACT_SWIGLU) {
    const void* w3 = g.B3;
    g.B3 = nullptr;
    g.prof_name = g.shared ? "bwd_shared_preact" : "bwd_ggemm_preact";
    g.C = a_pre;
    HIP_TRY(launch_gemm_bf16(g, EPI_IDENT_F32, s));
    g.B1 = w3;
    g.C = b_pre;
    HIP_TRY(launch_gemm_bf16(g, EPI_IDENT_F32, s));
    HIP_TRY(launch_swiglu_hidden(a_pre, b_pre, elems, hidden, s));
  } else {
    g.C = hidden;
    HIP_TRY(launch_gemm_bf16(g, EPI_RELU_BF16, s));
  }
  return MOE_OK;
}

// The four products of one FFN's backward over merged rows (routed experts:
// the dispatch's tile map; shared expert: a one-segment map).
struct FfnBwd {
  const uint16_t* u;       // inputs [rows, d] bf16 (fp32 experts: fp32)
  const uint16_t* hidden;  // [rows, h], same type
  const float* a_pre;      // SwiGLU pre-activations [rows, h]
  const float* b_pre;
  const uint16_t* gout;    // output gradient rows [rows, d], same type
  uint16_t* dpre;          // [rows, hw], same type
  float* du;               // [rows, d]
  const void* w1;
  const void* w3;
  const void* w2;
  long long stride1, stride2;  // elements between experts' w1 (and w3) / w2
  float* dw1;
  float* dw3;
  float* dw2;
  const int32_t* tile_expert;
  const int32_t* tile_row0;
  const int32_t* offsets;
  const int32_t* tile_count;
  int max_tiles, tile_rows, n_experts, h;
  bool f32;  // fp32 experts (activations and gradient rows in fp32)
  const char* names[4];
};

moe_status ffn_bwd(const moe_config& c, const FfnBwd& f, hipStream_t s) {
  const int d = c.d_model, h = f.h;
  const bool swiglu = c.act == MOE_ACT_SWIGLU;
  const int hw = swiglu ? 2 * h : h;
  GemmBwdArgs g{};
  g.tile_expert = f.tile_expert;
  g.tile_row0 = f.tile_row0;
  g.offsets = f.offsets;
  g.tile_count = f.tile_count;
  g.max_tiles = f.max_tiles;
  g.tile_rows = f.tile_rows;
  g.n_experts = f.n_experts;
  auto launch = [&](const GemmBwdArgs& a, int mode, int epi, const char* name) {
    return f.f32 ? launch_gemm_bwd_f32(a, mode, epi, name, s)
                 : launch_gemm_bwd(a, mode, epi, name, s);
  };
  // (i) dhid = gout . W2 -> dpre (ReLU mask or SwiGLU da | db)
  g.A = (const uint16_t*)f.w2;
  g.lda = h;
  g.strideA = f.stride2;
  g.k_split = d;
  g.B = f.gout;
  g.ldb = d;
  g.M = h;
  g.N = 0;
  g.K = d;
  g.Cb = f.dpre;
  g.ldc = hw;
  g.c_split = h;
  g.aux_h = f.hidden;
  g.aux_a = f.f32 ? (const float*)f.hidden : f.a_pre;
  g.aux_b = f.b_pre;
  g.ldaux = h;
  if (f.f32) g.C = (float*)f.dpre;  // fp32 gradient rows
  // (ii) du = dpre . [W1; W3]
  GemmBwdArgs g2{};
  g2.tile_expert = f.tile_expert;
  g2.tile_row0 = f.tile_row0;
  g2.offsets = f.offsets;
  g2.tile_count = f.tile_count;
  g2.max_tiles = f.max_tiles;
  g2.tile_rows = f.tile_rows;
  g2.A = (const uint16_t*)f.w1;
  g2.A2 = swiglu ? (const uint16_t*)f.w3 : nullptr;
  g2.lda = d;
  g2.strideA = f.stride1;
  g2.k_split = h;
  g2.B = f.dpre;
  g2.ldb = hw;
  g2.M = d;
  g2.K = hw;
  g2.C = f.du;
  g2.ldc = d;
  // (iii) dW2[e] = gout^T . hidden over the expert's rows
  GemmBwdArgs g3{};
  g3.offsets = f.offsets;
  g3.n_experts = f.n_experts;
  g3.A = f.hidden;
  g3.lda = h;
  g3.B = f.gout;
  g3.ldb = d;
  g3.M = h;
  g3.N = d;
  g3.C = f.dw2;
  g3.ldc = h;
  g3.strideC = (long long)d * h;
  g3.c_split = d;
  // (iv) [dW1; dW3][e] = dpre^T . u
  GemmBwdArgs g4{};
  g4.offsets = f.offsets;
  g4.n_experts = f.n_experts;
  g4.A = f.u;
  g4.lda = d;
  g4.B = f.dpre;
  g4.ldb = hw;
  g4.M = d;
  g4.N = hw;
  g4.C = f.dw1;
  g4.C2 = f.dw3;
  g4.ldc = d;
  g4.strideC = (long long)h * d;
  g4.c_split = h;
  // Launch order: dW2 first, while the output-gradient rows written by the
  // combine backward are fresh in cache; then dhid, dW1 while dpre is fresh,
  // and the input gradients last.  The four products are independent apart
  // from dpre, and each writes its own output, so the order changes no
  // result; at T=8192, d=512, h=1024, n=256, k=4 it measured about 1 %
  // faster than (i)-(iv) in turn.
  HIP_TRY(launch(g3, BWD_WGRAD, BEPI_F32, f.names[2]));
  HIP_TRY(launch(g, BWD_ROWS, swiglu ? BEPI_SWIGLU : BEPI_RELU_MASK, f.names[0]));
  HIP_TRY(launch(g4, BWD_WGRAD, BEPI_F32, f.names[3]));
  HIP_TRY(launch(g2, BWD_ROWS, BEPI_F32, f.names[1]));
  return MOE_OK;
}

// Pointer checks of the training entry points (gr == null: forward only).
moe_status check_bwd_args(const moe_config& c, const moe_weights* wt, const float* x,
                          const float* noise, const float* noise2, const float* dy,
                          const float* dlosses, const moe_grads* gr) {
  if (!wt) return fail(MOE_ERR_INVALID_ARG, "weights must not be NULL");
  CHECK(check_gate_ptrs(c, x, wt->w_gate, wt->b_gate, wt->w_noise, noise));
  const bool swiglu = c.act == MOE_ACT_SWIGLU;
  const bool shared = c.d_hidden_shared > 0;
  const bool noisy = wt->w_noise != nullptr;
  const bool hier = c.n_groups > 0;
  const bool noisy2 = hier && wt->w_noise2 != nullptr;
  const bool has_load = hier ? (noisy && noisy2) : noisy;
  if (hier) {
    CHECK(need(wt->w_gate2, "weights->w_gate2"));
    CHECK(optional(wt->w_noise2, "weights->w_noise2"));
    if (noisy2) CHECK(need(noise2, "noise2 (required with w_noise2)", c.T == 0));
    const int b2 = c.n_experts / c.n_groups;
    if ((noisy2 ? 2 * b2 : b2) % 16)
      return fail(MOE_ERR_UNSUPPORTED,
                  "the two-level backward needs the secondary gate's logit columns (b, or 2b "
                  "with noise) to be a multiple of 16");
  }
  CHECK(need(wt->w1, "weights->w1"));
  CHECK(need(wt->w2, "weights->w2"));
  if (swiglu) {
    CHECK(need(wt->w3, "weights->w3 (required for SwiGLU)"));
    if (wt->b1 || wt->b2) return fail(MOE_ERR_UNSUPPORTED, "SwiGLU experts take no biases");
  }
  CHECK(optional(wt->b1, "weights->b1"));
  CHECK(optional(wt->b2, "weights->b2"));
  if (shared) CHECK(check_shared_ptrs(c, wt->ws1, wt->ws3, wt->ws2));
  if (!gr) return MOE_OK;  // forward only
  CHECK(need(dy, "dy", c.T == 0));
  CHECK(need(dlosses, "dlosses"));
  CHECK(need(gr->dx, "grads->dx", c.T == 0));
  CHECK(need(gr->dw_gate, "grads->dw_gate"));
  const bool want_db = wt->b_gate && c.gate != MOE_GATE_SIGMOID_BIAS;
  if (want_db) CHECK(need(gr->db_gate, "grads->db_gate"));
  if (noisy) CHECK(need(gr->dw_noise, "grads->dw_noise"));
  CHECK(need(gr->dw1, "grads->dw1"));
  CHECK(need(gr->dw2, "grads->dw2"));
  if (swiglu) CHECK(need(gr->dw3, "grads->dw3"));
  if (wt->b1) CHECK(need(gr->db1, "grads->db1"));
  if (wt->b2) CHECK(need(gr->db2, "grads->db2"));
  if (hier) {
    CHECK(need(gr->dw_gate2, "grads->dw_gate2"));
    if (noisy2) CHECK(need(gr->dw_noise2, "grads->dw_noise2"));
  }
  if (shared) {
    CHECK(need(gr->dws1, "grads->dws1"));
    CHECK(need(gr->dws2, "grads->dws2"));
    if (swiglu) CHECK(need(gr->dws3, "grads->dws3"));
  }
  return MOE_OK;
}

// The training path over the backward's workspace layout (every intermediate
// the backward reads survives the forward).  do_fwd: the layer forward (y
// and losses may be null); do_bwd: the gradients from the intermediates the
// forward left in ws.
moe_status train_run(const moe_config& c, const moe_weights* wt, const float* x,
                     const float* noise, const float* noise2, const float* dy,
                     const float* dlosses, const moe_grads* gr, float* y, float* losses,
                     void* ws, size_t ws_bytes, hipStream_t s, bool do_fwd, bool do_bwd,
                     const char* what) {
  const bool swiglu = c.act == MOE_ACT_SWIGLU;
  const bool shared = c.d_hidden_shared > 0;
  const bool noisy = wt->w_noise != nullptr;
  const bool hier = c.n_groups > 0;
  const bool noisy2 = hier && wt->w_noise2 != nullptr;
  const bool has_load = hier ? (noisy && noisy2) : noisy;
  const bool want_db = wt->b_gate && c.gate != MOE_GATE_SIGMOID_BIAS;
  const BwdPlan b = make_bwd_plan(c);
  const Plan& p = b.f;
  CHECK(check_ws(ws, ws_bytes, b.total, what));
  const int T = c.T, d = c.d_model, h = c.d_hidden, n = c.n_experts, k = c.k;
  const long long A = (long long)T * k;
  int32_t* idx = at<int32_t>(ws, p.f_idx);
  float* w = at<float>(ws, p.f_w);
  float* imp = at<float>(ws, p.f_imp);
  float* ld = at<float>(ws, p.f_load);
  int32_t* counts_pre = at<int32_t>(ws, p.f_counts_pre);
  int32_t* counts = at<int32_t>(ws, p.f_counts);
  int32_t* offsets = at<int32_t>(ws, p.f_offsets);
  int32_t* perm = at<int32_t>(ws, p.f_perm);
  int32_t* slot = at<int32_t>(ws, p.f_slot);
  uint16_t* xperm = at<uint16_t>(ws, p.f_xperm);
  float* yperm = at<float>(ws, p.f_yperm);
  float* stats = at<float>(ws, p.f_stats);
  uint16_t* hidden = at<uint16_t>(ws, p.hidden);
  float* a_pre = swiglu ? at<float>(ws, b.a_pre) : nullptr;
  float* b_pre = swiglu ? at<float>(ws, b.b_pre) : nullptr;
  float* logits2 = hier ? at<float>(ws, b.logits2) : nullptr;
  float* load_g = hier ? at<float>(ws, b.load_g) : nullptr;
  ForwardExtras fx;
  fx.tile_expert = at<int32_t>(ws, p.f_tile_expert);
  fx.tile_row0 = at<int32_t>(ws, p.f_tile_row0);
  fx.tile_count = at<int32_t>(ws, p.f_tile_count);
  fx.losses = losses ? losses : at<float>(ws, b.losses);
  fx.importance = imp;
  fx.load = has_load ? ld : nullptr;
  fx.gate_stats = stats;
  fx.x_bf16 = shared ? at<uint16_t>(ws, p.sh_xb) : nullptr;
  const bool f32 = c.expert_dtype == MOE_F32;
  const int hs = c.d_hidden_shared;
  uint16_t* xb = shared ? at<uint16_t>(ws, p.sh_xb) : nullptr;
  uint16_t* hid_s = shared ? at<uint16_t>(ws, p.sh_hidden) : nullptr;
  int32_t* sh_off = shared ? at<int32_t>(ws, p.sh_off) : nullptr;
  int32_t* sh_te = shared ? at<int32_t>(ws, p.sh_te) : nullptr;
  int32_t* sh_tr = shared ? at<int32_t>(ws, p.sh_tr) : nullptr;
  int32_t* sh_tc = shared ? at<int32_t>(ws, p.sh_tc) : nullptr;
  float* a_s = shared && swiglu ? at<float>(ws, b.a_s) : nullptr;
  float* b_s = shared && swiglu ? at<float>(ws, b.b_s) : nullptr;

  if (do_fwd) {
  if (hier) {
    CHECK(run_gate_hier(c, p, x, wt->w_gate, wt->b_gate, wt->w_noise, noise, wt->w_gate2,
                        wt->w_noise2, noise2, idx, w, imp, ld, stats, ws, s, logits2, load_g));
  } else {
    CHECK(run_gate(c, p, x, wt->w_gate, wt->b_gate, wt->w_noise, noise, idx, w, imp, ld, stats,
                   ws, s, fx.colsum));
    fx.colsum_fused = true;
  }
  CHECK(run_dispatch(c, p, idx, x, counts_pre, counts, offsets, perm, slot, xperm, ws, s, &fx));
  if (f32) {
    // fp32 experts: the forward's own expert stage (hidden goes to the
    // relocated region of this plan)
    CHECK(run_ffn(c, p, xperm, offsets, wt->w1, wt->b1, wt->w3, wt->w2, wt->b2, yperm, ws, s,
                  &fx));
  } else {
  GemmBf16Args g1{};
  g1.A = xperm;
  g1.lda = d;
  g1.B1 = wt->w1;
  g1.B3 = wt->w3;
  g1.strideB = (long long)h * d * 2;
  g1.K = d;
  g1.bias = wt->b1;
  g1.tile_expert = fx.tile_expert;
  g1.tile_row0 = fx.tile_row0;
  g1.offsets = offsets;
  g1.tile_count = fx.tile_count;
  g1.max_mtiles = p.max_mtiles;
  g1.num_cus = device_cus();
  CHECK(bwd_hidden(c, g1, h, hidden, a_pre, b_pre, A * h, s));
  GemmBf16Args g2 = g1;
  g2.A = hidden;
  g2.lda = h;
  g2.B1 = wt->w2;
  g2.B3 = nullptr;
  g2.strideB = (long long)d * h * 2;
  g2.N = d;
  g2.K = h;
  g2.C = yperm;
  g2.ldc = d;
  g2.bias = wt->b2;
  HIP_TRY(launch_gemm_bf16(g2, EPI_IDENT_F32, s));
  }
  if (shared) {
    HIP_TRY(launch_shared_tilemap(T, kBf16BM, sh_off, sh_te, sh_tr, sh_tc, s));
    GemmBf16Args gs{};
    gs.A = xb;
    gs.lda = d;
    gs.B1 = wt->ws1;
    gs.B3 = wt->ws3;
    gs.K = d;
    gs.tile_expert = sh_te;
    gs.tile_row0 = sh_tr;
    gs.offsets = sh_off;
    gs.tile_count = sh_tc;
    gs.max_mtiles = p.sh_tiles;
    gs.num_cus = device_cus();
    gs.shared = 1;
    CHECK(bwd_hidden(c, gs, hs, hid_s, a_s, b_s, (long long)T * hs, s));
  }
  if (y) {
    float* ysh = nullptr;
    if (shared && T > 0) {
      // the shared expert's output (its hidden values are kept above)
      ysh = at<float>(ws, p.sh_y);
      GemmBf16Args go{};
      go.A = hid_s;
      go.lda = hs;
      go.B1 = wt->ws2;
      go.N = d;
      go.K = hs;
      go.C = ysh;
      go.ldc = d;
      go.tile_expert = sh_te;
      go.tile_row0 = sh_tr;
      go.offsets = sh_off;
      go.tile_count = sh_tc;
      go.max_mtiles = p.sh_tiles;
      go.num_cus = device_cus();
      go.shared = 1;
      HIP_TRY(launch_gemm_bf16(go, EPI_IDENT_F32, s));
    }
    HIP_TRY(launch_combine(yperm, slot, w, ysh, T, k, d, y, s));
  }
  }
  if (!do_bwd) return MOE_OK;

  // ---- backward ---------------------------------------------------------
  float* dG = at<float>(ws, b.dG);
  uint16_t* dout = at<uint16_t>(ws, b.dout);
  float* dimp = at<float>(ws, b.dimp);
  float* dload = at<float>(ws, b.dload);
  float* coef = at<float>(ws, b.coef);
  float* dlogits = at<float>(ws, b.dlogits);
  HIP_TRY(launch_combine_bwd(dy, yperm, slot, w, T, k, d, dG, dout, f32, s));
  HIP_TRY(launch_loss_grad(imp, has_load ? ld : nullptr, counts_pre, dlosses, T, k, n,
                           c.w_importance, c.w_load, c.alpha_switch, c.w_z, c.w_entropy, dimp,
                           dload, coef, s));
  // The flat gate, or the two-level layer's primary gate (whose slots carry
  // the product weights' split gradients and no Importance or entropy term).
  const int ng = p.n_gate;
  const int kg = hier ? p.k1 : k;
  float* dG1 = hier ? at<float>(ws, b.dG1) : nullptr;
  float* dG2 = hier ? at<float>(ws, b.dG2) : nullptr;
  float* dload_p = hier && has_load ? at<float>(ws, b.dload_p) : nullptr;
  float* dload_g = hier && has_load ? at<float>(ws, b.dload_g) : nullptr;
  if (hier) {
    HIP_TRY(launch_hier_product_bwd(idx, w, at<float>(ws, p.prim_w), dG, dimp, coef, T, p.k1,
                                    p.k2, dG1, dG2, s));
    if (has_load)
      HIP_TRY(launch_hier_dload(dload, at<float>(ws, p.prim_load), load_g,
                                at<int32_t>(ws, p.g_counts_pre), p.a, p.b, dload_p, dload_g, s));
  }
  GateBwdArgs gb{};
  gb.T = T;
  gb.n = ng;
  gb.switch_mode = c.gate == MOE_GATE_SWITCH_TOP1;
  gb.sigmoid_mode = c.gate == MOE_GATE_SIGMOID_BIAS;
  gb.noisy = noisy;
  gb.logits = at<float>(ws, p.logits);
  gb.ldl = p.ldl;
  gb.bias = wt->b_gate;
  gb.noise = noise;
  gb.k = kg;
  gb.topk_idx = hier ? at<int32_t>(ws, p.prim_idx) : idx;
  gb.topk_w = hier ? at<float>(ws, p.prim_w) : w;
  gb.dG = hier ? dG1 : dG;
  gb.dimp = hier ? nullptr : dimp;
  gb.dload = hier ? dload_p : (noisy ? dload : nullptr);
  gb.coef = hier ? coef + 2 : coef;
  gb.dlogits = dlogits;
  gb.ldd = p.ldl;
  gb.part_db = want_db ? at<float>(ws, b.part_db) : nullptr;
  gb.rows_per_block = p.rows_per_block;
  HIP_TRY(launch_gate_bwd(gb, s));
  if (want_db)
    HIP_TRY(launch_colsum(p.nparts, ColsumVec{gb.part_db, ng, gr->db_gate},
                          ColsumVec{nullptr, 0, nullptr}, ColsumVec{nullptr, 0, nullptr}, s));
  const int M = noisy ? 2 * ng : ng;
  GateWgradArgs gw{};
  gw.x = x;
  gw.dlogits = dlogits;
  gw.ldd = p.ldl;
  gw.T = T;
  gw.d = d;
  gw.M = M;
  gw.n = ng;
  gw.splits = b.splits;
  gw.tokens_per_split = b.tps;
  gw.partial = at<float>(ws, b.wpart);
  HIP_TRY(launch_gate_wgrad(gw, gr->dw_gate, gr->dw_noise, s));
  float* dx_gate = at<float>(ws, b.dx_gate);
  if (T > 0) {
    const int ldk = (int)round_up(M, 4);
    float* wtr = at<float>(ws, b.wt);
    HIP_TRY(launch_transpose_gate(wt->w_gate, wt->w_noise, ng, d, ldk, wtr, s));
    GemmF32Args gx{};
    gx.A = dlogits;
    gx.lda = p.ldl;
    gx.B1 = wtr;
    gx.B2 = wtr;
    gx.n1 = d;
    gx.N = d;
    gx.K = ldk;
    gx.C = dx_gate;
    gx.ldc = d;
    gx.M = T;
    gx.mtiles = (T + p.gemm_bm - 1) / p.gemm_bm;
    gx.max_mtiles = gx.mtiles;
    gx.prof_name = "bwd_gate_dx";
    HIP_TRY(launch_gemm_gate(gx, p.gemm_bm, s));
  }
  FfnBwd fb{};
  fb.u = xperm;
  fb.hidden = hidden;
  fb.a_pre = a_pre;
  fb.b_pre = b_pre;
  fb.gout = dout;
  fb.dpre = at<uint16_t>(ws, b.dpre);
  fb.du = at<float>(ws, b.du_perm);
  fb.w1 = wt->w1;
  fb.w3 = wt->w3;
  fb.w2 = wt->w2;
  fb.stride1 = (long long)h * d;
  fb.stride2 = (long long)d * h;
  fb.dw1 = gr->dw1;
  fb.dw3 = gr->dw3;
  fb.dw2 = gr->dw2;
  fb.tile_expert = fx.tile_expert;
  fb.tile_row0 = fx.tile_row0;
  fb.offsets = offsets;
  fb.tile_count = fx.tile_count;
  fb.max_tiles = p.max_mtiles;
  fb.tile_rows = p.ffn_bm;
  fb.n_experts = n;
  fb.h = h;
  fb.f32 = f32;
  fb.names[0] = "bwd_ggemm_dhidden";
  fb.names[1] = "bwd_ggemm_dinput";
  fb.names[2] = "bwd_ggemm_dw2";
  fb.names[3] = "bwd_ggemm_dw1";
  CHECK(ffn_bwd(c, fb, s));
  if (wt->b2) HIP_TRY(launch_seg_colsum(dout, f32, d, offsets, n, d, gr->db2, s));
  if (wt->b1) HIP_TRY(launch_seg_colsum(fb.dpre, f32, h, offsets, n, h, gr->db1, s));
  float* du_s = nullptr;
  if (shared) {
    uint16_t* dout_s = at<uint16_t>(ws, b.dout_s);
    du_s = at<float>(ws, b.du_s);
    HIP_TRY(launch_to_bf16(dy, (long long)T * d, dout_s, s));
    FfnBwd fs{};
    fs.u = xb;
    fs.hidden = hid_s;
    fs.a_pre = a_s;
    fs.b_pre = b_s;
    fs.gout = dout_s;
    fs.dpre = at<uint16_t>(ws, b.dpre_s);
    fs.du = du_s;
    fs.w1 = wt->ws1;
    fs.w3 = wt->ws3;
    fs.w2 = wt->ws2;
    fs.dw1 = gr->dws1;
    fs.dw3 = gr->dws3;
    fs.dw2 = gr->dws2;
    fs.tile_expert = sh_te;
    fs.tile_row0 = sh_tr;
    fs.offsets = sh_off;
    fs.tile_count = sh_tc;
    fs.max_tiles = p.sh_tiles;
    fs.tile_rows = kBf16BM;
    fs.n_experts = 1;
    fs.h = hs;
    fs.names[0] = "bwd_shared_dhidden";
    fs.names[1] = "bwd_shared_dinput";
    fs.names[2] = "bwd_shared_dw2";
    fs.names[3] = "bwd_shared_dw1";
    CHECK(ffn_bwd(c, fs, s));
  }
  float* du2 = nullptr;
  if (hier) {
    // Each group's secondary gate over the rows routed to it.
    const int bb = p.b;
    float* dlogits2 = at<float>(ws, b.dlogits2);
    const int32_t* g_perm = at<int32_t>(ws, p.g_perm);
    const int32_t* g_offsets = at<int32_t>(ws, p.g_offsets);
    GateBwdArgs g2{};
    g2.T = T;
    g2.n = bb;
    g2.k = p.k2;
    g2.noisy = noisy2;
    g2.logits = logits2;
    g2.ldl = p.ldl2;
    g2.noise = noise2;
    g2.topk_idx = idx;
    g2.dG = dG2;
    g2.dload = dload_g;
    g2.coef = coef + 2;
    g2.dlogits = dlogits2;
    g2.ldd = p.ldl2;
    g2.row_token = g_perm;
    g2.prim_idx = at<int32_t>(ws, p.prim_idx);
    g2.k1 = p.k1;
    g2.tile_expert = at<int32_t>(ws, p.t2_expert);
    g2.tile_row0 = at<int32_t>(ws, p.t2_row0);
    g2.offsets = g_offsets;
    g2.tile_count = at<int32_t>(ws, p.t2_count);
    g2.max_tiles = p.max_tiles2;
    g2.tile_rows = kSecondaryBM;
    HIP_TRY(launch_gate_bwd(g2, s));
    const int K2 = noisy2 ? 2 * bb : bb;
    // dW_gate2 | dW_noise2 [g] = dlogits2^T x over the group's rows
    GemmBwdArgs gw2{};
    gw2.A = (const uint16_t*)x;
    gw2.lda = d;
    gw2.rowmap_a = g_perm;
    gw2.B = (const uint16_t*)dlogits2;
    gw2.ldb = p.ldl2;
    gw2.M = d;
    gw2.N = K2;
    gw2.C = gr->dw_gate2;
    gw2.C2 = gr->dw_noise2;
    gw2.ldc = d;
    gw2.strideC = (long long)bb * d;
    gw2.c_split = bb;
    gw2.offsets = g_offsets;
    gw2.n_experts = p.a;
    HIP_TRY(launch_gemm_bwd_f32(gw2, BWD_WGRAD, BEPI_F32, "bwd_gate2_wgrad", s));
    // the rows' input gradients dlogits2 . [W_gate2; W_noise2][g]
    du2 = at<float>(ws, b.du2);
    GemmBwdArgs gx2{};
    gx2.A = (const uint16_t*)wt->w_gate2;
    gx2.A2 = (const uint16_t*)wt->w_noise2;
    gx2.lda = d;
    gx2.strideA = (long long)bb * d;
    gx2.k_split = bb;
    gx2.B = (const uint16_t*)dlogits2;
    gx2.ldb = p.ldl2;
    gx2.M = d;
    gx2.K = K2;
    gx2.C = du2;
    gx2.ldc = d;
    gx2.tile_expert = g2.tile_expert;
    gx2.tile_row0 = g2.tile_row0;
    gx2.offsets = g_offsets;
    gx2.tile_count = g2.tile_count;
    gx2.max_tiles = p.max_tiles2;
    gx2.tile_rows = kSecondaryBM;
    HIP_TRY(launch_gemm_bwd_f32(gx2, BWD_ROWS, BEPI_F32, "bwd_gate2_dx", s));
  }
  HIP_TRY(launch_dx_gather(dx_gate, du_s, fb.du, slot, T, k, d, du2,
                           hier ? at<int32_t>(ws, p.g_slot) : nullptr, p.k1, gr->dx, s));
  return MOE_OK;
}

}  // namespace

extern "C" {

size_t moe_fp8_weight_bytes(int32_t n_experts, int32_t N, int32_t K) {
  if (n_experts < 0 || N <= 0 || K <= 0 || N % 8 || K % 64) return 0;
  return (size_t)n_experts * ((size_t)N * K + 4 * (size_t)N);
}

moe_status moe_pack_fp8_weights(int32_t n_experts, int32_t N, int32_t K, int32_t src_dtype,
                                const void* src, void* dst, void* stream) {
  g_err[0] = 0;
  if (n_experts < 0 || N <= 0 || K <= 0)
    return fail(MOE_ERR_INVALID_ARG, "n_experts >= 0, N > 0 and K > 0 required");
  if (N % 8 || K % 64)
    return fail(MOE_ERR_UNSUPPORTED, "FP8 packing needs N %% 8 == 0 and K %% 64 == 0 (N=%d, K=%d)",
                N, K);
  if (src_dtype != MOE_F32 && src_dtype != MOE_BF16)
    return fail(MOE_ERR_INVALID_ARG, "src_dtype must be MOE_F32 or MOE_BF16");
  if (n_experts > 65535) return fail(MOE_ERR_UNSUPPORTED, "at most 65535 experts per call");
  CHECK(need(src, "src", n_experts == 0));
  CHECK(need(dst, "dst", n_experts == 0));
  HIP_TRY(launch_pack_fp8(n_experts, N, K, src_dtype == MOE_BF16, src, dst, (hipStream_t)stream));
  return MOE_OK;
}

size_t moe_workspace_size(const moe_config* cfg) {
  if (validate(cfg) != MOE_OK) return 0;
  return make_plan(*cfg).total;
}

int32_t moe_expert_split_rows(const moe_config* cfg) {
  if (validate(cfg) != MOE_OK) return 0;
  return split_rows(*cfg);
}

int32_t moe_gate_k_splits(const moe_config* cfg) {
  if (validate(cfg) != MOE_OK) return 0;
  return make_plan(*cfg).gate_splits;
}

int32_t moe_expert_cu_split(const moe_config* cfg, const int32_t* counts, int32_t cus,
                            int32_t product) {
  if (validate(cfg) != MOE_OK || !counts || cus < 0 || (product != 0 && product != 1)) return -1;
  const int big_rows = split_rows(*cfg);
  if (big_rows <= 0) return 0;
  long long br = 0, bg = 0, se = 0, sr = 0;
  for (int e = 0; e < cfg->n_experts; ++e) {
    const int kept = counts[e];
    if (kept >= big_rows) {
      const long long mt = (kept + kBigBM - 1) / kBigBM;
      br += mt * kBigBM;
      bg += (mt + kBigGroupM - 1) / kBigGroupM;
    } else if (kept > 0) {
      ++se, sr += kept;
    }
  }
  if (cfg->expert_dtype != MOE_BF16) return 0;
  const CuSplit sp = cu_split_of(*cfg, nullptr);
  return expert_cu_split(cus > 0 ? cus : sp.cus, br, bg, se, sr, sp.d, sp.h, sp.swiglu, product);
}

}  // extern "C"

size_t moe::gate_workspace_bytes(const moe_config* cfg) {
  if (validate(cfg) != MOE_OK) return 0;
  return make_plan(*cfg).gate_bytes;
}

extern "C" {

moe_status moe_gate(const moe_config* cfg, const float* x, const float* w_gate,
                    const float* b_gate, const float* w_noise, const float* noise,
                    int32_t* topk_idx, float* topk_w, float* importance, float* load,
                    float* gate_stats, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  CHECK(validate(cfg));
  const moe_config& c = *cfg;
  if (c.n_groups > 0) return fail(MOE_ERR_INVALID_ARG, "moe_gate is the flat gate; use moe_gate_hier");
  CHECK(check_gate_ptrs(c, x, w_gate, b_gate, w_noise, noise));
  CHECK(need(topk_idx, "topk_idx", c.T == 0));
  CHECK(need(topk_w, "topk_w", c.T == 0));
  CHECK(need(importance, "importance"));
  if (w_noise) CHECK(need(load, "load (required for a noisy gate)"));
  CHECK(optional(gate_stats, "gate_stats"));
  const Plan p = make_plan(c);
  CHECK(check_ws(ws, ws_bytes, p.gate_bytes, "moe_gate"));
  return run_gate(c, p, x, w_gate, b_gate, w_noise, noise, topk_idx, topk_w, importance, load,
                  gate_stats, ws, (hipStream_t)stream);
}

moe_status moe_gate_hier(const moe_config* cfg, const float* x, const float* w_gate,
                         const float* b_gate, const float* w_noise, const float* noise,
                         const float* w_gate2, const float* w_noise2, const float* noise2,
                         int32_t* topk_idx, float* topk_w, float* importance, float* load,
                         float* gate_stats, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  CHECK(validate(cfg));
  const moe_config& c = *cfg;
  if (c.n_groups <= 0) return fail(MOE_ERR_INVALID_ARG, "moe_gate_hier needs n_groups > 0");
  CHECK(check_gate_ptrs(c, x, w_gate, b_gate, w_noise, noise));
  CHECK(need(w_gate2, "w_gate2"));
  CHECK(optional(w_noise2, "w_noise2"));
  if (w_noise2) CHECK(need(noise2, "noise2 (required with w_noise2)", c.T == 0));
  CHECK(need(topk_idx, "topk_idx", c.T == 0));
  CHECK(need(topk_w, "topk_w", c.T == 0));
  CHECK(need(importance, "importance"));
  if (w_noise && w_noise2) CHECK(need(load, "load (required for noisy gates)"));
  CHECK(optional(gate_stats, "gate_stats"));
  const Plan p = make_plan(c);
  CHECK(check_ws(ws, ws_bytes, p.gate_bytes, "moe_gate_hier"));
  return run_gate_hier(c, p, x, w_gate, b_gate, w_noise, noise, w_gate2, w_noise2, noise2,
                       topk_idx, topk_w, importance, load, gate_stats, ws, (hipStream_t)stream);
}

moe_status moe_dispatch(const moe_config* cfg, const int32_t* topk_idx, const float* x,
                        int32_t* counts_pre, int32_t* counts, int32_t* offsets, int32_t* perm,
                        int32_t* slot_pos, void* x_perm, void* ws, size_t ws_bytes,
                        void* stream) {
  g_err[0] = 0;
  CHECK(validate(cfg));
  const moe_config& c = *cfg;
  CHECK(need(topk_idx, "topk_idx", c.T == 0));
  CHECK(need(x, "x", c.T == 0));
  CHECK(need(counts_pre, "counts_pre"));
  CHECK(need(counts, "counts"));
  CHECK(need(offsets, "offsets"));
  CHECK(need(perm, "perm", c.T == 0));
  CHECK(need(slot_pos, "slot_pos", c.T == 0));
  CHECK(need(x_perm, "x_perm", c.T == 0));
  const Plan p = make_plan(c);
  CHECK(check_ws(ws, ws_bytes, p.dispatch_bytes, "moe_dispatch"));
  return run_dispatch(c, p, topk_idx, x, counts_pre, counts, offsets, perm, slot_pos, x_perm, ws,
                      (hipStream_t)stream);
}

moe_status moe_expert_ffn(const moe_config* cfg, const void* x_perm, const int32_t* offsets,
                          const void* w1, const float* b1, const void* w3, const void* w2,
                          const float* b2, float* y_perm, void* ws, size_t ws_bytes,
                          void* stream) {
  g_err[0] = 0;
  CHECK(validate(cfg));
  const moe_config& c = *cfg;
  CHECK(need(x_perm, "x_perm", c.T == 0));
  CHECK(need(offsets, "offsets"));
  CHECK(need(w1, "w1"));
  CHECK(need(w2, "w2"));
  CHECK(need(y_perm, "y_perm", c.T == 0));
  if (c.act == MOE_ACT_SWIGLU) {
    CHECK(need(w3, "w3 (required for SwiGLU)"));
    if (b1 || b2) return fail(MOE_ERR_UNSUPPORTED, "SwiGLU experts take no biases");
  } else {
    CHECK(optional(w3, "w3"));
  }
  CHECK(optional(b1, "b1"));
  CHECK(optional(b2, "b2"));
  const Plan p = make_plan(c);
  CHECK(check_ws(ws, ws_bytes, p.ffn_bytes, "moe_expert_ffn"));
  return run_ffn(c, p, x_perm, offsets, w1, b1, w3, w2, b2, y_perm, ws, (hipStream_t)stream);
}

moe_status moe_shared_ffn(const moe_config* cfg, const float* x, const void* ws1,
                          const void* ws3, const void* ws2, float* y_shared, void* ws,
                          size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  CHECK(validate(cfg));
  const moe_config& c = *cfg;
  if (c.d_hidden_shared <= 0)
    return fail(MOE_ERR_INVALID_ARG, "moe_shared_ffn needs d_hidden_shared > 0");
  CHECK(need(x, "x", c.T == 0));
  CHECK(check_shared_ptrs(c, ws1, ws3, ws2));
  CHECK(need(y_shared, "y_shared", c.T == 0));
  const Plan p = make_plan(c);
  CHECK(check_ws(ws, ws_bytes, p.total, "moe_shared_ffn"));
  hipStream_t s = (hipStream_t)stream;
  uint16_t* xb = at<uint16_t>(ws, p.sh_xb);
  HIP_TRY(launch_to_bf16(x, (long long)c.T * c.d_model, xb, s));
  return run_shared_ffn(c, p, xb, ws1, ws3, ws2, y_shared, ws, s);
}

moe_status moe_combine(const moe_config* cfg, const float* y_perm, const int32_t* slot_pos,
                       const float* topk_w, const float* y_base, float* y, void* stream) {
  g_err[0] = 0;
  CHECK(validate(cfg));
  const moe_config& c = *cfg;
  CHECK(need(y_perm, "y_perm", c.T == 0));
  CHECK(need(slot_pos, "slot_pos", c.T == 0));
  CHECK(need(topk_w, "topk_w", c.T == 0));
  CHECK(optional(y_base, "y_base"));
  CHECK(need(y, "y", c.T == 0));
  HIP_TRY(launch_combine(y_perm, slot_pos, topk_w, y_base, c.T, c.k, c.d_model, y,
                         (hipStream_t)stream));
  return MOE_OK;
}

moe_status moe_aux_loss(const moe_config* cfg, const float* importance, const float* load,
                        const int32_t* counts_pre, const float* gate_stats, float* losses,
                        void* stream) {
  g_err[0] = 0;
  CHECK(validate(cfg));
  const moe_config& c = *cfg;
  CHECK(need(importance, "importance"));
  CHECK(optional(load, "load"));
  CHECK(need(counts_pre, "counts_pre"));
  CHECK(optional(gate_stats, "gate_stats"));
  CHECK(need(losses, "losses"));
  HIP_TRY(launch_aux(importance, load, counts_pre, gate_stats, c.T, c.k, c.n_experts,
                     c.w_importance, c.w_load, c.alpha_switch, c.w_z, c.w_entropy, losses,
                     (hipStream_t)stream));
  return MOE_OK;
}

moe_status moe_router_bias_update(const moe_config* cfg, const int32_t* counts_pre, float* bias,
                                  float gamma, void* stream) {
  g_err[0] = 0;
  CHECK(validate(cfg));
  const moe_config& c = *cfg;
  if (!std::isfinite(gamma)) return fail(MOE_ERR_INVALID_ARG, "gamma must be finite");
  CHECK(need(counts_pre, "counts_pre"));
  CHECK(need(bias, "bias"));
  HIP_TRY(launch_bias_update(counts_pre, c.n_experts, c.T, c.k, gamma, bias,
                             (hipStream_t)stream));
  return MOE_OK;
}

moe_status moe_forward(const moe_config* cfg, const moe_weights* wt, const float* x,
                       const float* noise, const float* noise2, float* y, float* losses,
                       const moe_diag* diag, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  CHECK(validate(cfg));
  const moe_config& c = *cfg;
  if (!wt) return fail(MOE_ERR_INVALID_ARG, "weights must not be NULL");
  const bool hier = c.n_groups > 0;
  CHECK(check_gate_ptrs(c, x, wt->w_gate, wt->b_gate, wt->w_noise, noise));
  if (hier) {
    CHECK(need(wt->w_gate2, "weights->w_gate2"));
    CHECK(optional(wt->w_noise2, "weights->w_noise2"));
    if (wt->w_noise2) CHECK(need(noise2, "noise2 (required with w_noise2)", c.T == 0));
  }
  CHECK(need(wt->w1, "weights->w1"));
  CHECK(need(wt->w2, "weights->w2"));
  if (c.act == MOE_ACT_SWIGLU) {
    CHECK(need(wt->w3, "weights->w3 (required for SwiGLU)"));
    if (wt->b1 || wt->b2) return fail(MOE_ERR_UNSUPPORTED, "SwiGLU experts take no biases");
  }
  CHECK(optional(wt->b1, "weights->b1"));
  CHECK(optional(wt->b2, "weights->b2"));
  if (c.d_hidden_shared > 0) CHECK(check_shared_ptrs(c, wt->ws1, wt->ws3, wt->ws2));
  CHECK(need(y, "y", c.T == 0));
  CHECK(need(losses, "losses"));
  moe_diag dg{};
  if (diag) {
    dg = *diag;
    CHECK(optional(dg.topk_idx, "diag->topk_idx"));
    CHECK(optional(dg.topk_w, "diag->topk_w"));
    CHECK(optional(dg.importance, "diag->importance"));
    CHECK(optional(dg.load, "diag->load"));
    CHECK(optional(dg.counts_pre, "diag->counts_pre"));
    CHECK(optional(dg.counts, "diag->counts"));
    CHECK(optional(dg.offsets, "diag->offsets"));
    CHECK(optional(dg.perm, "diag->perm"));
    CHECK(optional(dg.slot_pos, "diag->slot_pos"));
  }
  const Plan p = make_plan(c);
  CHECK(check_ws(ws, ws_bytes, p.total, "moe_forward"));
  hipStream_t s = (hipStream_t)stream;
  int32_t* idx = dg.topk_idx ? dg.topk_idx : at<int32_t>(ws, p.f_idx);
  float* w = dg.topk_w ? dg.topk_w : at<float>(ws, p.f_w);
  float* imp = dg.importance ? dg.importance : at<float>(ws, p.f_imp);
  float* ld = dg.load ? dg.load : at<float>(ws, p.f_load);
  int32_t* counts_pre = dg.counts_pre ? dg.counts_pre : at<int32_t>(ws, p.f_counts_pre);
  int32_t* counts = dg.counts ? dg.counts : at<int32_t>(ws, p.f_counts);
  int32_t* offsets = dg.offsets ? dg.offsets : at<int32_t>(ws, p.f_offsets);
  int32_t* perm = dg.perm ? dg.perm : at<int32_t>(ws, p.f_perm);
  int32_t* slot = dg.slot_pos ? dg.slot_pos : at<int32_t>(ws, p.f_slot);
  void* xperm = at<void>(ws, p.f_xperm);
  float* yperm = at<float>(ws, p.f_yperm);
  const bool has_load = hier ? (wt->w_noise && wt->w_noise2) : (wt->w_noise != nullptr);
  float* stats = at<float>(ws, p.f_stats);
  ForwardExtras fx;
  const bool shared = c.d_hidden_shared > 0;
  fx.x_bf16 = shared ? at<uint16_t>(ws, p.sh_xb) : nullptr;
  // bf16 and FP8 experts: x is rounded to bf16 once, in token order (into the
  // x_perm region unless the shared expert's copy exists), and GEMM 1 reads
  // each merged row through perm, instead of k copies of every row.  The flat
  // gate GEMM writes that copy as a by-product of splitting x (the two-level
  // layer's gather writes it).
  const bool via_perm =
      c.expert_dtype != MOE_F32 && (long long)c.T * c.d_model * 2 <= (1LL << 30);
  if (via_perm) {
    fx.row_token = perm;
    if (!fx.x_bf16) fx.x_bf16 = (uint16_t*)xperm;
  }
  if (hier) {
    CHECK(run_gate_hier(c, p, x, wt->w_gate, wt->b_gate, wt->w_noise, noise, wt->w_gate2,
                        wt->w_noise2, noise2, idx, w, imp, ld, stats, ws, s));
  } else {
    CHECK(run_gate(c, p, x, wt->w_gate, wt->b_gate, wt->w_noise, noise, idx, w, imp, ld, stats,
                   ws, s, fx.colsum, fx.x_bf16));
    fx.colsum_fused = true;
    fx.x_bf16_written = fx.x_bf16 != nullptr;
  }
  fx.tile_expert = at<int32_t>(ws, p.f_tile_expert);
  fx.tile_row0 = at<int32_t>(ws, p.f_tile_row0);
  fx.tile_count = at<int32_t>(ws, p.f_tile_count);
  if (p.big_rows > 0) {
    fx.big_rows = p.big_rows;
    fx.small_map = TileMap{at<int32_t>(ws, p.f_ts_expert), at<int32_t>(ws, p.f_ts_row0),
                           at<int32_t>(ws, p.f_ts_count)};
    fx.big_map = TileMap{at<int32_t>(ws, p.f_tb_expert), at<int32_t>(ws, p.f_tb_row0),
                         at<int32_t>(ws, p.f_tb_count)};
    fx.cu_split = at<int32_t>(ws, p.f_split);
  }
  // The losses are not needed before the combine: one extra block of the
  // combine launch computes them, off the dispatch's serial finalize.
  fx.losses = nullptr;
  fx.importance = imp;
  fx.load = has_load ? ld : nullptr;
  fx.gate_stats = stats;
  CHECK(run_dispatch(c, p, idx, x, counts_pre, counts, offsets, perm, slot,
                     via_perm ? nullptr : xperm, ws, s, &fx));
  // bf16 / FP8 experts: their output rows are rounded to bf16 (only the
  // combine reads them); fp32 experts keep fp32 rows.
  const bool y_bf16 = c.expert_dtype != MOE_F32;
  CHECK(run_ffn(c, p, via_perm ? (const void*)fx.x_bf16 : xperm, offsets, wt->w1, wt->b1, wt->w3,
                wt->w2, wt->b2, yperm, ws, s, &fx, y_bf16));
  float* ysh = shared ? at<float>(ws, p.sh_y) : nullptr;
  if (shared) CHECK(run_shared_ffn(c, p, fx.x_bf16, wt->ws1, wt->ws3, wt->ws2, ysh, ws, s));
  const AuxArgs aux{imp,       fx.load,   counts_pre,     stats,       c.T,
                    c.k,       c.n_experts, c.w_importance, c.w_load, c.alpha_switch,
                    c.w_z,     c.w_entropy, losses};
  HIP_TRY(launch_combine(yperm, slot, w, ysh, c.T, c.k, c.d_model, y, s, &aux, y_bf16));
  return MOE_OK;
}

size_t moe_backward_workspace_size(const moe_config* cfg) {
  if (validate(cfg) != MOE_OK || validate_bwd(*cfg) != MOE_OK) return 0;
  return make_bwd_plan(*cfg).total;
}

moe_status moe_backward(const moe_config* cfg, const moe_weights* wt, const float* x,
                        const float* noise, const float* noise2, const float* dy,
                        const float* dlosses, const moe_grads* gr, void* ws, size_t ws_bytes,
                        void* stream) {
  g_err[0] = 0;
  CHECK(validate(cfg));
  CHECK(validate_bwd(*cfg));
  if (!gr) return fail(MOE_ERR_INVALID_ARG, "grads must not be NULL");
  CHECK(check_bwd_args(*cfg, wt, x, noise, noise2, dy, dlosses, gr));
  return train_run(*cfg, wt, x, noise, noise2, dy, dlosses, gr, nullptr, nullptr, ws, ws_bytes,
                   (hipStream_t)stream, true, true, "moe_backward");
}

moe_status moe_forward_train(const moe_config* cfg, const moe_weights* wt, const float* x,
                             const float* noise, const float* noise2, float* y, float* losses,
                             void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  CHECK(validate(cfg));
  CHECK(validate_bwd(*cfg));
  CHECK(check_bwd_args(*cfg, wt, x, noise, noise2, nullptr, nullptr, nullptr));
  CHECK(need(y, "y", cfg->T == 0));
  CHECK(need(losses, "losses"));
  return train_run(*cfg, wt, x, noise, noise2, nullptr, nullptr, nullptr, y, losses, ws,
                   ws_bytes, (hipStream_t)stream, true, false, "moe_forward_train");
}

moe_status moe_backward_saved(const moe_config* cfg, const moe_weights* wt, const float* x,
                              const float* noise, const float* noise2, const float* dy,
                              const float* dlosses, const moe_grads* gr, void* ws,
                              size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  CHECK(validate(cfg));
  CHECK(validate_bwd(*cfg));
  if (!gr) return fail(MOE_ERR_INVALID_ARG, "grads must not be NULL");
  CHECK(check_bwd_args(*cfg, wt, x, noise, noise2, dy, dlosses, gr));
  return train_run(*cfg, wt, x, noise, noise2, dy, dlosses, gr, nullptr, nullptr, ws, ws_bytes,
                   (hipStream_t)stream, false, true, "moe_backward_saved");
}

moe_status moe_probe_mfma(int32_t dtype, int32_t blocks, int32_t iters, float* sink,
                          double* flops, void* stream) {
  g_err[0] = 0;
  if (dtype != MOE_BF16 && dtype != MOE_F32)
    return fail(MOE_ERR_INVALID_ARG, "moe_probe_mfma: dtype must be MOE_BF16 or MOE_F32");
  if (blocks <= 0 || iters <= 0)
    return fail(MOE_ERR_INVALID_ARG, "moe_probe_mfma: blocks and iters must be positive");
  CHECK(need(sink, "sink"));
  if (flops)
    *flops = (double)blocks * 4 * (double)iters * 4 * (dtype == MOE_BF16 ? 32768.0 : 4096.0);
  HIP_TRY(launch_mfma_probe(dtype == MOE_BF16, blocks, iters, sink, (hipStream_t)stream));
  return MOE_OK;
}

moe_status moe_probe_hbm_read(const void* buf, size_t bytes, int32_t blocks, float* sink,
                              void* stream) {
  g_err[0] = 0;
  if (blocks <= 0) return fail(MOE_ERR_INVALID_ARG, "moe_probe_hbm_read: blocks must be positive");
  if (bytes < 16) return fail(MOE_ERR_INVALID_ARG, "moe_probe_hbm_read: bytes must be >= 16");
  CHECK(need(buf, "buf"));
  CHECK(need(sink, "sink"));
  HIP_TRY(launch_hbm_read_probe(buf, (long long)bytes, blocks, sink, (hipStream_t)stream));
  return MOE_OK;
}

const char* moe_status_string(moe_status status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported configuration";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_HIP: return "HIP launch failure";
  }
  return "unknown status";
}

const char* moe_last_error(void) { return g_err; }

}  // extern "C"
