/*
 * moe.h -- C ABI of the MI355X (gfx950) Sparsely-Gated Mixture-of-Experts
 * layer: forward and backward.
 *
 * The layer computes y = sum_i G(x)_i * E_i(x) over n experts, with the
 * noisy top-k gate G(x) = Softmax(KeepTopK(H(x), k)),
 *   H(x)_i = (x . W_g)_i + StandardNormal() * Softplus((x . W_noise)_i),
 * and the importance / load auxiliary losses w * CV(.)^2.
 *   Source: arXiv 1701.06538 summary page (xyznot.com), section
 *   "Method and key formulas" (layer output, Noisy Top-K gating, load
 *   balancing losses); reading notes on the same paper (chenshi221.pages.dev),
 *   sections "Sparsely-Gated MoE layer architecture", "Noisy Top-K Gating",
 *   "Balancing expert utilization", "Hierarchical MoE".
 * Also supported: the Switch top-1 router with expert capacity and its
 * n * sum f_i P_i loss (MoE survey, tufusi.com, sections 3.1 and 3.2),
 * renormalised top-k over a gated (SwiGLU) expert FFN (same survey, section
 * 6.2, fine-grained routed experts), the sigmoid gate with a selection-only
 * bias, its bias controller and an always-active shared expert (same survey,
 * sections 5.2, 6.2, 6.3), and the router z-loss and gate-entropy losses
 * (MoE algorithm introduction, wkbse.com, part 2).
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Data pointers are DEVICE pointers (HIP device memory of the current
 *    device), caller-owned.  The library never allocates, frees, copies to
 *    the host or synchronises; scratch memory is the caller's workspace `ws`.
 *  - `stream` is a hipStream_t (NULL = the null stream).  All work is
 *    enqueued on it; calls return after enqueueing.
 *  - Validation is synchronous and complete before anything is enqueued:
 *    a status other than MOE_OK means nothing was launched.  The detail of the
 *    last failure on the calling thread is in moe_last_error().  Device faults
 *    surface at the caller's next synchronisation.
 *  - Required pointers must be non-NULL and 16-byte aligned.  Optional
 *    pointers may be NULL, meaning "absent" (zero bias, noiseless gate, ...).
 *  - All matrices are row-major and contiguous.  Weights are stored out-by-in
 *    (like a PyTorch Linear): w_gate[i][c] multiplies x[t][c] for expert i.
 *  - bf16 tensors are passed as raw 16-bit patterns (uint16_t storage).
 *  - Results are bitwise deterministic for identical inputs on one device:
 *    no floating-point atomics, fixed-order reductions.
 *  - The calls are stateless and reentrant; concurrent calls need distinct
 *    workspaces.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* NULL / misaligned pointer, bad size or enum */
  MOE_ERR_UNSUPPORTED = 2, /* valid but outside what the kernels implement */
  MOE_ERR_WORKSPACE = 3,   /* ws NULL or ws_bytes too small */
  MOE_ERR_HIP = 4          /* a HIP launch failed */
} moe_status;

typedef enum {
  MOE_GATE_TOPK_SOFTMAX = 0, /* G = Softmax(KeepTopK(H, k)); noisy iff w_noise != NULL */
  MOE_GATE_SWITCH_TOP1 = 1,  /* p = softmax(h) over all n; top-1 with weight p_argmax; k = 1 */
  MOE_GATE_SIGMOID_BIAS = 2  /* top-k of h + b_gate; g = Sigmoid(h) / sum over the kept of
                                Sigmoid(h); no noise; flat layers only */
} moe_gate_kind;

typedef enum {
  MOE_ACT_RELU = 0,  /* E(u) = max(0, u W1^T + b1) W2^T + b2 */
  MOE_ACT_SWIGLU = 1 /* E(u) = (silu(u W1^T) * (u W3^T)) W2^T; bf16 experts only */
} moe_act;

typedef enum {
  MOE_F32 = 0,
  MOE_BF16 = 1,
  MOE_FP8 = 2 /* expert weights only: packed E4M3 codes with a per-row scale (see
                 moe_pack_fp8_weights); activations stay bf16 */
} moe_dtype;

/* Layer shape and options.  All fields are 4 bytes. */
typedef struct {
  int32_t T;              /* tokens (all positions merged into one batch), >= 0 */
  int32_t d_model;        /* d, multiple of 8 */
  int32_t d_hidden;       /* expert hidden width h, multiple of 8 */
  int32_t n_experts;      /* n (two-level layer: a*b) */
  int32_t k;              /* experts per token, 1..min(n,64) (two-level: k1*k2) */
  int32_t gate;           /* moe_gate_kind */
  int32_t act;            /* moe_act */
  int32_t expert_dtype;   /* moe_dtype of w1/w3/w2; x_perm is fp32 for MOE_F32, else bf16.
                             MOE_FP8 needs d_model and d_hidden multiples of 64 */
  int32_t n_groups;       /* two-level layer: a groups of b = n/a experts; 0 = flat */
  int32_t k_groups;       /* two-level layer: k1 groups per token, k = k1*k2 */
  float capacity_factor;  /* > 0: expert capacity min(floor(cf*T*k/n), T*k); <= 0: none */
  float w_importance;     /* weight of CV(Importance)^2 */
  float w_load;           /* weight of CV(Load)^2 */
  float alpha_switch;     /* weight of n * sum_i f_i P_i */
  float w_z;              /* weight of the router z-loss */
  float w_entropy;        /* weight of the gate-entropy loss */
  int32_t d_hidden_shared;/* hidden width of the shared expert, multiple of 8; 0 = none.
                             The shared expert uses `act` and needs bf16 experts. */
} moe_config;

/* Weight pointers for moe_forward (a host struct holding device pointers). */
typedef struct {
  const float* w_gate;   /* [n_gate, d] fp32; n_gate = n (flat) or a (two-level) */
  const float* b_gate;   /* [n_gate] fp32 per-expert logit bias, optional */
  const float* w_noise;  /* [n_gate, d] fp32, optional (NULL = noiseless gate) */
  const float* w_gate2;  /* two-level only: [a, b, d] secondary gates */
  const float* w_noise2; /* two-level only: [a, b, d], optional */
  const void* w1;        /* [n, h, d] expert_dtype */
  const float* b1;       /* [n, h] fp32, optional (ReLU only) */
  const void* w3;        /* [n, h, d] expert_dtype, SwiGLU only */
  const void* w2;        /* [n, d, h] expert_dtype */
  const float* b2;       /* [n, d] fp32, optional (ReLU only) */
  const void* ws1;       /* shared expert [h_s, d] bf16 (h_s = d_hidden_shared) */
  const void* ws3;       /* shared expert [h_s, d] bf16, SwiGLU only */
  const void* ws2;       /* shared expert [d, h_s] bf16 */
} moe_weights;

/* Optional intermediate outputs of moe_forward; every field may be NULL
 * (the forward then keeps that intermediate in the workspace). */
typedef struct {
  int32_t* topk_idx;   /* [T, k] */
  float* topk_w;       /* [T, k] */
  float* importance;   /* [n] */
  float* load;         /* [n]; written only for a noisy gate */
  int32_t* counts_pre; /* [n] */
  int32_t* counts;     /* [n] */
  int32_t* offsets;    /* [n+1] */
  int32_t* perm;       /* [T*k] */
  int32_t* slot_pos;   /* [T, k] */
} moe_diag;

/* FP8 expert weights.  Definition: the MoE survey's DeepSeek-V3 summary
 * (tufusi.com, section 9: FP8 for the main computation), read as E4M3 codes
 * (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; largest finite 448;
 * the "e4m3fn" variant) with one fp32 scale per output row:
 *   scale = amax(row) / 448 (1 for an all-zero row), code = E4M3(w / scale),
 * both divisions in IEEE single precision, nearest code with ties to an
 * even mantissa, saturating at 448.  The expert computes with the value
 * decode(code) * scale; activations stay bf16.
 * Packed layout of one [N, K] matrix (N % 8 == 0, K % 64 == 0), N*K + 4*N bytes:
 * the codes of rows 2p, 2p+1 over columns 64b..64b+63 are the 128 bytes at
 * offset (p*(K/64) + b)*128 (row 2p first), then the N fp32 scales.
 * n_experts such matrices follow one another.
 * moe_fp8_weight_bytes: bytes of n_experts packed [N, K] matrices (0 on
 * invalid sizes).  moe_pack_fp8_weights: src [n_experts, N, K] of src_dtype
 * (MOE_F32 or MOE_BF16) -> dst (that many bytes, 16-byte aligned), on
 * `stream`.  Pack w1 and w3 as [n, h, d] and w2 as [n, d, h]. */
size_t moe_fp8_weight_bytes(int32_t n_experts, int32_t N, int32_t K);
moe_status moe_pack_fp8_weights(int32_t n_experts, int32_t N, int32_t K, int32_t src_dtype,
                                const void* src, void* dst, void* stream);

/* Bytes of workspace that every call below accepts as sufficient (the
 * forward's need; each stage needs at most this).  0 on an invalid config. */
size_t moe_workspace_size(const moe_config* cfg);

/* How moe_expert_ffn / moe_forward split the experts between their two
 * grouped GEMMs: experts keeping at least this many rows run on 256 x 256
 * tiles, the others on 128-row tiles (0: every expert on 128-row tiles).
 * Depends on the config only (bf16 or FP8 weights with d_model and d_hidden
 * both >= 2048 split); the results do not depend on it.  0 on an invalid
 * config. */
int32_t moe_expert_split_rows(const moe_config* cfg);

/* Into how many K ranges moe_gate, moe_gate_hier (its primary gate) and
 * moe_forward split the gate's logit GEMM: 1 (none) unless its tiles number
 * fewer than three per CU and d_model >= 2048.  Each range's fp32 partial
 * logits take [T, 2 * n_gate] of the workspace; the gate adds them in range
 * order.  Depends on the config only; 0 on an invalid config. */
int32_t moe_gate_k_splits(const moe_config* cfg);

/* When experts are split by size (moe_expert_split_rows > 0) and the
 * weights are bf16, the two grouped GEMMs run side by side: the small
 * experts' 128-row GEMM, which streams their weights from HBM, on a second
 * stream of the library's own, beside the big experts' 256 x 256-tile GEMM
 * on the caller's stream, each on its own share of the compute units; the
 * caller's stream waits for both before the combine.  (FP8 weights: one
 * after the other.)  Calls on one device from several host threads take
 * turns on that second stream; a call captured into a graph before any
 * uncaptured call on its device has created the stream runs the two one
 * after the other.  The shares are computed on the device from the
 * routing; this call computes the same share on the host.
 *   counts: host array [n_experts] of the rows each expert keeps (the
 *           dispatch's counts); cus: compute units of the GPU (0: the
 *           current device's).
 * Returns the compute units of the 256 x 256-tile GEMM (the other GEMM
 * gets the rest): 0 without experts of at least moe_expert_split_rows rows,
 * without the split or with FP8 weights, every CU without smaller non-empty
 * experts, else a
 * multiple of 8 (the XCD count) in [8, cus - 8].  Each product has its own
 * share (product 0: x W1^T, with x W3^T for SwiGLU; 1: hidden W2^T): the
 * 256 x 256 GEMM runs at another rate per CU on K = d_model than on K =
 * d_hidden.  -1 on an invalid config, null counts, cus < 0 or a product
 * other than 0 and 1.  The results of the layer do not depend on it. */
int32_t moe_expert_cu_split(const moe_config* cfg, const int32_t* counts, int32_t cus,
                            int32_t product);

/* Flat gating network: logits, noise, KeepTopK, softmax, and the two
 * auxiliary-loss vectors.
 *   Definition: xyznot.com summary, "Method and key formulas", Noisy Top-K
 *   gating (H, KeepTopK, G) and the Importance / P(x,i) / Load equations;
 *   Switch router: tufusi.com survey, section 3.1.
 * In:  x [T, d], w_gate [n, d], b_gate [n] (optional; added to the clean
 *      logit), w_noise [n, d] (optional), noise [T, n] (the StandardNormal
 *      draws; required iff w_noise != NULL), all fp32.
 * Out: topk_idx [T, k] int32 -- slot s holds the expert of rank s: descending
 *      H, lower index first on equal H (-0.0 == +0.0);
 *      topk_w [T, k] fp32 -- softmax over the kept H (Switch: p_argmax);
 *      importance [n] fp32 -- sum over tokens of the dense gate G (Switch:
 *      of the full softmax p);
 *      load [n] fp32 -- sum over tokens of P(x,i) = Phi((clean_i - thr_i) /
 *      Softplus(raw_i)), thr_i = H_(k+1) if i is kept else H_(k); required iff
 *      w_noise != NULL, ignored otherwise (may be NULL);
 *      gate_stats [2] fp32, optional -- [0] = sum over tokens of the squared
 *      L2 norm of the logits the gate's softmax sees (H; the sigmoid gate:
 *      the bias-free logits h), [1] = sum over tokens of the entropy of the
 *      gate distribution (the kept weights; Switch: the full softmax p).
 *      Definition: wkbse.com MoE introduction, part 2 (router z-loss, gate
 *      entropy loss).
 * MOE_GATE_SIGMOID_BIAS (tufusi.com survey 6.2, 6.3): b_gate only moves the
 * selection (top-k of h + b); the weights are Sigmoid(h) renormalised over
 * the kept experts; w_noise must be NULL.
 * Flat configs only (n_groups == 0); n <= 2048. */
moe_status moe_gate(const moe_config* cfg, const float* x, const float* w_gate,
                    const float* b_gate, const float* w_noise, const float* noise,
                    int32_t* topk_idx, float* topk_w, float* importance, float* load,
                    float* gate_stats, void* ws, size_t ws_bytes, void* stream);

/* moe_gate without a workspace argument, for callers that cannot allocate
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments (minus ws, ws_bytes), same kernels, same
 * results as moe_gate.
 * Scratch: a static device array of 48 MiB inside the library, one copy per
 * GPU, held from the first call on that GPU until the process ends; the call
 * itself allocates nothing.  A config whose gate needs more scratch than
 * that (moe_gate's workspace: the logits [T, 2n] fp32 plus per-block partial
 * sums) returns MOE_ERR_WORKSPACE before any launch.
 * Calls that overlap on one GPU (other streams, other threads) share that
 * GPU's array and race: the caller must order them.  Consecutive calls need
 * no clearing between them (every scratch byte read is written earlier in
 * the same call). */
moe_status moe_gate_static(const moe_config* cfg, const float* x, const float* w_gate,
                           const float* b_gate, const float* w_noise, const float* noise,
                           int32_t* topk_idx, float* topk_w, float* importance, float* load,
                           float* gate_stats, void* stream);

/* Two-level gate: a primary gate picks k1 of a groups, then each chosen
 * group's own secondary gate picks k2 of its b experts.
 *   Definition: chenshi221.pages.dev notes, section "Hierarchical MoE"; the
 *   xyznot.com summary's key-term entry on hierarchical mixtures of experts.
 * In:  x [T, d]; w_gate/w_noise [a, d], b_gate [a] (optional), noise [T, a];
 *      w_gate2/w_noise2 [a, b, d]; noise2 [T, k1, b] (draws of the secondary
 *      gate for the token's primary slot s).  Noise pointers are required
 *      iff the matching w_noise is given.
 * Out: topk_idx [T, k1*k2]: slot s*k2+s2 = g_s*b + e (g_s primary slot s,
 *      e the secondary slot s2); topk_w = w_primary[s] * w_secondary[s2];
 *      importance [a*b] = sum of those products per expert;
 *      load [a*b] = Load_primary[g] * Load_g[e] / |X_g| (0 when no token
 *      reaches g), Load_g the secondary gate's load over the tokens X_g routed
 *      to g; required iff w_noise != NULL (both levels must then be noisy);
 *      gate_stats [2], optional: [0] = squared logit norms of both levels'
 *      gates summed over tokens, [1] = entropy of the product distribution
 *      summed over tokens.
 * cfg->n_groups = a, cfg->k_groups = k1, cfg->k = k1*k2, n = a*b. */
moe_status moe_gate_hier(const moe_config* cfg, const float* x, const float* w_gate,
                         const float* b_gate, const float* w_noise, const float* noise,
                         const float* w_gate2, const float* w_noise2, const float* noise2,
                         int32_t* topk_idx, float* topk_w, float* importance, float* load,
                         float* gate_stats, void* ws, size_t ws_bytes, void* stream);

/* Merge every position routed to an expert into one contiguous batch.
 *   Definition: chenshi221.pages.dev notes, "Engineering" (all time steps
 *   merged into one batch); tufusi.com survey 3.2 (expert capacity C =
 *   tokens/E * capacity factor; overflow passes through the residual).
 * In:  topk_idx [T, k], x [T, d] fp32.
 * Out: counts_pre [n] (slots routed to each expert), counts [n] =
 *      min(counts_pre, C) with C = floor(cf*T*k/n) (no limit if cf <= 0),
 *      offsets [n+1] = exclusive scan of counts (offsets[n] = kept rows),
 *      perm [T*k] (row -> token; tokens ascend within each expert; rows >=
 *      offsets[n] untouched), slot_pos [T, k] (row of each slot, -1 when the
 *      slot was over capacity; over-capacity slots are dropped first come
 *      first served in (token, slot) order),
 *      x_perm [T*k, d] = x[perm[row]] converted to expert_dtype (bf16 round
 *      to nearest even).
 * topk_idx entries should lie in [0, n); an entry outside it is treated like a
 * slot dropped for capacity (slot_pos -1, counted in no expert). */
moe_status moe_dispatch(const moe_config* cfg, const int32_t* topk_idx, const float* x,
                        int32_t* counts_pre, int32_t* counts, int32_t* offsets, int32_t* perm,
                        int32_t* slot_pos, void* x_perm, void* ws, size_t ws_bytes,
                        void* stream);

/* All experts on their merged batches (one grouped launch per layer).
 *   Definition: chenshi221.pages.dev notes, "Sparsely-Gated MoE layer
 *   architecture" (identical one-hidden-layer ReLU FFNs, own parameters);
 *   tufusi.com survey 6.2 (fine-grained routed experts, d_ff = 2048).
 * In:  x_perm [T*k, d] expert_dtype; offsets [n+1] (rows of expert e are
 *      offsets[e] .. offsets[e+1]-1); w1 [n, h, d], w3 [n, h, d] (SwiGLU),
 *      w2 [n, d, h] in expert_dtype; b1 [n, h], b2 [n, d] fp32 optional
 *      (ReLU only).  bf16 experts accumulate in fp32; the hidden activations
 *      are rounded to bf16 before the second product.
 * Out: y_perm [T*k, d] fp32 (rows >= offsets[n] untouched). */
moe_status moe_expert_ffn(const moe_config* cfg, const void* x_perm, const int32_t* offsets,
                          const void* w1, const float* b1, const void* w3, const void* w2,
                          const float* b2, float* y_perm, void* ws, size_t ws_bytes,
                          void* stream);

/* The shared expert on every token: y_shared[t] = E_shared(x[t]) with
 * E(u) = ReLU(u ws1^T) ws2^T or (silu(u ws1^T) * (u ws3^T)) ws2^T (cfg->act),
 * bf16 weights, fp32 accumulation, hidden activations rounded to bf16.
 *   Definition: tufusi.com survey, sections 5.2 (shared experts, always
 *   active) and 6.2 (one shared expert of the routed experts' width).
 * In:  x [T, d] fp32; ws1 [h_s, d], ws3 [h_s, d] (SwiGLU), ws2 [d, h_s] bf16,
 *      h_s = cfg->d_hidden_shared > 0.
 * Out: y_shared [T, d] fp32. */
moe_status moe_shared_ffn(const moe_config* cfg, const float* x, const void* ws1,
                          const void* ws3, const void* ws2, float* y_shared, void* ws,
                          size_t ws_bytes, void* stream);

/* y[t] = y_base[t] (optional; e.g. the shared expert's output) + the sum over
 * the token's slots s (in slot order) of topk_w[t,s] * y_perm[slot_pos[t,s]];
 * slots with slot_pos < 0 add nothing.  A gather: every output row is written
 * exactly once, no atomics.
 *   Definition: xyznot.com summary, "Method and key formulas" (layer output);
 *   tufusi.com survey 6.2 (shared expert added to the routed sum).
 * In: y_perm [*, d] fp32, slot_pos [T, k], topk_w [T, k], y_base [T, d] or
 * NULL.  Out: y [T, d] fp32. */
moe_status moe_combine(const moe_config* cfg, const float* y_perm, const int32_t* slot_pos,
                       const float* topk_w, const float* y_base, float* y, void* stream);

/* Auxiliary losses, losses[5] fp32 on the device:
 *   losses[0] = w_importance * CV(importance)^2
 *   losses[1] = w_load * CV(load)^2 (0 when load == NULL)
 *   losses[2] = alpha_switch * n * sum_i f_i P_i, f_i = counts_pre[i]/(T*k),
 *               P_i = importance[i]/T (0 when T == 0)
 *   losses[3] = w_z * gate_stats[0] / T        (router z-loss)
 *   losses[4] = -w_entropy * gate_stats[1] / T (minus the mean gate entropy)
 *               (both 0 when gate_stats == NULL or T == 0)
 * CV uses the population variance; CV^2 = 0 when the mean is 0.
 *   Definition: xyznot.com summary, "Method and key formulas" (L_importance,
 *   L_load); tufusi.com survey 3.2 (Switch auxiliary loss); wkbse.com MoE
 *   introduction, part 2 (z-loss on the L2 norm of the pre-softmax logits,
 *   read as its square; entropy loss rewarding a high gate entropy). */
moe_status moe_aux_loss(const moe_config* cfg, const float* importance, const float* load,
                        const int32_t* counts_pre, const float* gate_stats, float* losses,
                        void* stream);

/* Non-gradient selection-bias controller of the sigmoid gate: for every
 * expert, bias[i] -= gamma if counts_pre[i] > T*k/n (overloaded),
 * bias[i] += gamma if counts_pre[i] < T*k/n, unchanged at the even share.
 *   Definition: tufusi.com survey, section 6.3.
 * In: counts_pre [n] int32 (e.g. from moe_dispatch or the forward's diag).
 * In/out: bias [n] fp32 (the b_gate of the next step). */
moe_status moe_router_bias_update(const moe_config* cfg, const int32_t* counts_pre, float* bias,
                                  float gamma, void* stream);

/* The whole layer: gate (flat or two-level), dispatch, experts, the shared
 * expert (cfg->d_hidden_shared > 0), combine, losses, all on `stream` with no
 * host synchronisation.
 * In:  weights (see moe_weights), x [T, d], noise [T, n_gate] (required iff
 *      weights->w_noise), noise2 [T, k1, b] (two-level, iff w_noise2).
 * Out: y [T, d] fp32 (no residual added), losses [5] fp32 (as moe_aux_loss),
 *      diag: optional intermediates (may be NULL).
 * Precision: with bf16 or FP8 experts each expert's output row is rounded to
 * bf16 before the combine weights and sums it in fp32 (moe_expert_ffn and
 * the training forward keep those rows in fp32). */
moe_status moe_forward(const moe_config* cfg, const moe_weights* weights, const float* x,
                       const float* noise, const float* noise2, float* y, float* losses,
                       const moe_diag* diag, void* ws, size_t ws_bytes, void* stream);

/* Gradient outputs of moe_backward (a host struct holding device pointers),
 * all fp32, shaped like the matching weights.  A gradient is written iff its
 * weight is present (then the pointer is required); db_gate also needs a
 * softmax or Switch gate (the sigmoid gate's bias only moves the selection
 * and receives no gradient; db_gate must then be NULL). */
typedef struct {
  float* dx;       /* [T, d] */
  float* dw_gate;  /* [n, d] */
  float* db_gate;  /* [n] */
  float* dw_noise; /* [n, d] */
  float* dw1;      /* [n, h, d] */
  float* db1;      /* [n, h] */
  float* dw3;      /* [n, h, d] */
  float* dw2;      /* [n, d, h] */
  float* db2;      /* [n, d] */
  float* dws1;     /* [h_s, d] */
  float* dws3;     /* [h_s, d] */
  float* dws2;     /* [d, h_s] */
  float* dw_gate2; /* [a, b, d] (two-level layer) */
  float* dw_noise2;/* [a, b, d] (two-level layer with w_noise2) */
} moe_grads;

/* Bytes of workspace moe_backward needs (0 on an invalid or unsupported
 * config). */
size_t moe_backward_workspace_size(const moe_config* cfg);

/* Backward pass of the layer: the gradients of
 *   L = sum_t <dy_t, y_t> + sum_j dlosses[j] * losses[j]
 * (y and losses[5] as moe_forward computes them) with respect to x and every
 * weight, the routing (the top-k selection and the capacity drops) held
 * fixed.  The forward's routing and activations are recomputed first with
 * the forward's kernels, so they are the forward's bit for bit.
 *   Definition: xyznot.com summary, FAQ on training through the top-k (the
 *   selection precedes the softmax, so the kept gate values are
 *   differentiable in the gate's weights); chenshi221.pages.dev notes,
 *   "Noisy Top-K Gating" (the noise term lets the load loss pass gradients,
 *   through P(x,i) into the clean logit, the noise scale and the
 *   threshold's logit).  The bf16 roundings of the forward pass gradients
 *   unchanged.
 * Arithmetic: for bf16 experts the expert gradients are bf16 MFMA products
 * with fp32 accumulation (the gradient rows entering them are rounded to
 * bf16); for fp32 experts everything is fp32; the gate's gradients are fp32.
 * Two-level layer (chenshi221.pages.dev notes, "Hierarchical MoE"): a
 * combined slot's weight is w1_s * w2_{s,s2}, Importance and the entropy
 * are over these products and Load is the factorised form (see
 * moe_gate_hier); the chain runs through both gates, each group's over the
 * rows routed to it.
 * In:  weights, x [T, d], noise [T, n_gate], noise2 [T, k1, b] as for
 *      moe_forward; dy [T, d] fp32; dlosses [5] fp32 device vector.
 * Out: every gradient of `grads` (see moe_grads).
 * Supported: expert_dtype MOE_BF16 or MOE_F32; d_model, d_hidden and
 * d_hidden_shared multiples of 64; for the two-level layer the secondary
 * gate's logit columns (b, or 2b with w_noise2) a multiple of 16;
 * MOE_ERR_UNSUPPORTED otherwise.  ws: moe_backward_workspace_size(cfg)
 * bytes. */
moe_status moe_backward(const moe_config* cfg, const moe_weights* weights, const float* x,
                        const float* noise, const float* noise2, const float* dy,
                        const float* dlosses, const moe_grads* grads, void* ws, size_t ws_bytes,
                        void* stream);

/* A training step in two calls, with no forward recomputation: the layer
 * forward of moe_forward that also keeps, in ws, every intermediate the
 * backward reads (routing, merged batches, hidden activations, gate logits).
 * Same definition and arguments as moe_forward (no diag); the routing and
 * losses are moe_forward's bit for bit; y agrees with moe_forward's to fp32
 * rounding (for SwiGLU bf16 experts the hidden value comes from the two fp32
 * pre-activations kept for the backward).
 * ws: moe_backward_workspace_size(cfg) bytes, owned by the caller and kept
 * untouched until the matching moe_backward_saved. */
moe_status moe_forward_train(const moe_config* cfg, const moe_weights* weights, const float* x,
                             const float* noise, const float* noise2, float* y, float* losses,
                             void* ws, size_t ws_bytes, void* stream);

/* The gradients of moe_backward from the intermediates the last
 * moe_forward_train left in ws.  Precondition (not checkable here): the
 * same cfg, weights, x, noise, noise2 and ws as that call, none modified
 * since, and the call ordered after it (same stream, or synchronised).  The
 * result is then moe_backward's bit for bit.  Arguments and errors as
 * moe_backward. */
moe_status moe_backward_saved(const moe_config* cfg, const moe_weights* weights, const float* x,
                              const float* noise, const float* noise2, const float* dy,
                              const float* dlosses, const moe_grads* grads, void* ws,
                              size_t ws_bytes, void* stream);

/* Kernel timing, a tracing aid (off by default).  moe_profile_enable(1)
 * clears earlier results and starts bracketing every kernel launch of the
 * library with two HIP events recorded on that launch's stream;
 * moe_profile_enable(0) stops recording.  moe_profile_collect() waits for the
 * recorded events, folds them into per-kernel totals and returns the number
 * of distinct kernels; moe_profile_entry(i, ...) copies kernel i's name
 * (NUL-terminated, truncated to name_len), its total milliseconds and its
 * launch count, or returns MOE_ERR_INVALID_ARG for a bad index or NULL
 * output.  Process-wide state, safe to call from several threads. */
moe_status moe_profile_enable(int on);
int moe_profile_collect(void);
moe_status moe_profile_entry(int i, char* name, size_t name_len, double* total_ms,
                             long long* launches);

/* Matrix-unit peak probe, a measurement aid (not part of the layer): a loop
 * of MFMA instructions on register operands, nothing else, so that the
 * attainable bf16 (dtype MOE_BF16, v_mfma_f32_32x32x16_bf16) or fp32
 * (MOE_F32, v_mfma_f32_32x32x2f32) matrix rate can be measured beside the
 * datasheet peaks.  Launches `blocks` blocks of 4 waves; each wave runs
 * `iters` iterations of 4 independent MFMAs.  sink: device buffer of at least
 * blocks * 256 floats (overwritten with a checksum per lane); *flops (host,
 * may be NULL) receives the launch's flop count.  Asynchronous on `stream`;
 * time it with events around the call. */
moe_status moe_probe_mfma(int32_t dtype, int32_t blocks, int32_t iters, float* sink,
                          double* flops, void* stream);

/* HBM read-bandwidth probe, a measurement aid (not part of the layer): reads
 * the first floor(bytes / 16) * 16 bytes of the device buffer `buf` (16-byte
 * aligned) once; each of `blocks` blocks of 256 threads streams its own
 * contiguous segment with eight 16-byte loads per thread in flight, and
 * writes a checksum per thread to `sink` (device, at least blocks * 256
 * floats).  Asynchronous on `stream`; time it with
 * events around the call. */
moe_status moe_probe_hbm_read(const void* buf, size_t bytes, int32_t blocks, float* sink,
                              void* stream);

/* Static text for a status code. */
const char* moe_status_string(moe_status status);

/* Detail of the last failure on the calling thread ("" if none). */
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
