/*
 * Plain CPU oracle for the Sparsely-Gated Mixture-of-Experts layer, forward
 * and backward.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this library: only the test suite, the package's smoke check and the
 * benchmark's CPU-baseline leg use it.  It shares no code, header, table or
 * constant with the HIP implementation.
 *
 * Everything is computed in double precision from the definitions on the
 * pages, one stage at a time, with no blocking, fusion or reordering beyond
 * what those definitions state.  Per-element loops run in a fixed order; the
 * only parallelism is an OpenMP split over independent tokens / rows, which
 * does not change any result.
 *
 * Sources (cited by page title and section):
 *   [NOTES]  "Outrageously Large Neural Networks: The Sparsely-Gated
 *            Mixture-of-Experts Layer", reading notes (chenshi221.pages.dev),
 *            sections "Sparsely-Gated MoE 层架构", "Noisy Top-K Gating",
 *            "负载均衡", "分层 MoE".
 *   [PAPER]  arXiv 1701.06538 summary page (xyznot.com), section
 *            "方法（與關鍵公式）": the layer output, Noisy Top-K gating
 *            (H, KeepTopK, G) and the load-balancing losses
 *            (Importance, L_importance, P(x,i), Load, L_load).
 *   [SURVEY] "MoE 稀疏架构深度解析" (tufusi.com), section 3.1 (Switch router)
 *            and 3.2 (auxiliary loss, expert capacity).
 *   [WIKI]   "MoE (Mixture-of-Experts) 算法介绍" (wkbse.com), part 2 (top-k
 *            weights renormalised to sum to one; router z-loss and gate
 *            entropy among the auxiliary losses).
 *   [SURVEY] sections 5.2 (shared expert), 6.2 (sigmoid affinities
 *            normalised over the top k) and 6.3 (selection-only bias and its
 *            non-gradient update).
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *   - KeepTopK ties: the lower expert index wins; -0.0 equals +0.0.
 *   - Slot order: descending H, lower index first on equal H.
 *   - kth_excluding(H,k,i): the k-th largest of {H_j : j != i}; it equals
 *     H_(k+1) when i is kept and H_(k) otherwise; -inf when no such value.
 *   - CV uses the population variance; CV^2 = 0 when the mean is 0.
 *   - Capacity C = floor(cf*T*k/n); slots over capacity are dropped first
 *     come first served in (token, slot) order and contribute zero.
 *   - bf16 experts: inputs and hidden activations are rounded to bf16
 *     (round to nearest, ties to even) before each product; sums in double.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_GATE_TOPK_SOFTMAX 0
#define ORACLE_GATE_SWITCH_TOP1 1
#define ORACLE_GATE_SIGMOID_BIAS 2
#define ORACLE_ACT_RELU 0
#define ORACLE_ACT_SWIGLU 1

/* Threads the OpenMP loops below use (for reporting the baseline's cores). */
int oracle_num_threads(void) { return omp_get_max_threads(); }

/* Sets the thread count of later OpenMP loops (n >= 1).  The results do not
 * depend on it: every per-element loop writes disjoint outputs in a fixed
 * order and every sum over tokens is serial. */
void oracle_set_num_threads(int n) {
  if (n >= 1) omp_set_num_threads(n);
}

/* ------------------------------------------------------------------------ */
/* Scalar helpers                                                            */
/* ------------------------------------------------------------------------ */

/* Softplus(z) = log(1 + e^z), written in the overflow-safe form
 * max(z,0) + log1p(e^-|z|).  [PAPER] Noisy Top-K gating uses it as the
 * per-expert noise scale. */
double oracle_softplus(double z) {
  double a = fabs(z);
  return (z > 0.0 ? z : 0.0) + log1p(exp(-a));
}

/* Standard normal CDF, Phi(z) = erfc(-z / sqrt 2) / 2.  [PAPER] smooth load
 * estimator P(x,i). */
double oracle_phi(double z) { return 0.5 * erfc(-z / sqrt(2.0)); }

/* Round a real number to the nearest bfloat16 value (8 significant bits,
 * exponent range of binary32), ties to even.  Written from the format's
 * definition: scale the value so that its 8 significant bits sit left of the
 * binary point, round to the nearest integer with ties to even (rint in the
 * default rounding mode), scale back.  Below the normal range the spacing is
 * fixed at 2^-133 (the bf16 subnormal step).  Values past the largest finite
 * bf16 become infinities. */
double oracle_bf16_round(double v) {
  if (!(v == v) || v == 0.0 || isinf(v)) return v;
  int e;
  frexp(v, &e); /* v = f * 2^e with 0.5 <= |f| < 1 */
  int shift = 8 - e; /* 2^(e-8) is the spacing of 8-bit significands */
  if (e - 8 < -133) shift = 133; /* subnormal spacing */
  double r = ldexp(rint(ldexp(v, shift)), -shift);
  /* largest finite bf16 = (2 - 2^-7) * 2^127 */
  const double maxb = ldexp(255.0, 120);
  if (fabs(r) > maxb) r = v > 0 ? INFINITY : -INFINITY;
  return r;
}

void oracle_bf16_round_array(int64_t count, const double* in, double* out) {
  for (int64_t i = 0; i < count; ++i) out[i] = oracle_bf16_round(in[i]);
}

/* ------------------------------------------------------------------------ */
/* Gating network                                                            */
/* ------------------------------------------------------------------------ */

/* O1 + O2.  [PAPER] Noisy Top-K gating:
 *   clean_i = (x . W_g)_i (+ b_i, the per-expert logit bias of a workload),
 *   sp_i    = Softplus((x . W_noise)_i),
 *   H_i     = clean_i + z_i * sp_i, z_i ~ StandardNormal (supplied as input).
 * Weights are stored out-by-in: w_gate[i][c] is (W_g)_{c,i}.
 * w_noise == NULL means a noiseless gate: H = clean and sp is not written. */
void oracle_gate_logits(int T, int d, int n, const double* x, const double* w_gate,
                        const double* b_gate, const double* w_noise, const double* noise,
                        double* clean, double* sp, double* H) {
#pragma omp parallel for schedule(static)
  for (int t = 0; t < T; ++t) {
    const double* xt = x + (size_t)t * d;
    for (int i = 0; i < n; ++i) {
      double c = 0.0;
      for (int j = 0; j < d; ++j) c += xt[j] * w_gate[(size_t)i * d + j];
      if (b_gate) c += b_gate[i];
      clean[(size_t)t * n + i] = c;
      double h = c;
      if (w_noise) {
        double r = 0.0;
        for (int j = 0; j < d; ++j) r += xt[j] * w_noise[(size_t)i * d + j];
        double s = oracle_softplus(r);
        if (sp) sp[(size_t)t * n + i] = s;
        h = c + (noise ? noise[(size_t)t * n + i] : 0.0) * s;
      }
      H[(size_t)t * n + i] = h;
    }
  }
}

/* O3.  [PAPER] KeepTopK(v,k)_i = v_i if v_i is among the top k of v, else -inf.
 * Expert i's rank is the number of experts that beat it: a strictly larger H,
 * or an equal H and a lower index.  Expert i is kept iff rank_i < k, and slot
 * s of the token holds the expert of rank s.
 * Also returns H_(k) (the k-th largest, the smallest kept value) and
 * H_(k+1) (the largest dropped value, -inf when k == n): these are the two
 * values kth_excluding(H,k,i) can take. */
void oracle_keep_topk(int T, int n, int k, const double* H, int32_t* topk_idx, double* h_k,
                      double* h_k1) {
#pragma omp parallel for schedule(static)
  for (int t = 0; t < T; ++t) {
    const double* v = H + (size_t)t * n;
    int32_t* out = topk_idx + (size_t)t * k;
    int kth_owner = -1, k1_owner = -1;
    for (int i = 0; i < n; ++i) {
      int rank = 0;
      for (int j = 0; j < n; ++j) {
        if (v[j] > v[i] || (v[j] == v[i] && j < i)) ++rank;
      }
      if (rank < k) out[rank] = i;
      if (rank == k - 1) kth_owner = i;
      if (rank == k) k1_owner = i;
    }
    if (h_k) h_k[t] = v[kth_owner];
    if (h_k1) h_k1[t] = k1_owner >= 0 ? v[k1_owner] : -INFINITY;
  }
}

/* O4.  Gate weights of the kept slots, and the dense gate vector probs[T][n].
 *  TOPK_SOFTMAX: [PAPER] G(x) = Softmax(KeepTopK(H(x),k)); the -inf entries
 *    vanish, so G is the softmax over the kept values.  This equals the
 *    renormalised top-k weights of [WIKI] part 2.
 *  SWITCH_TOP1: [SURVEY] 3.1 p = softmax(h) over all experts; the token goes
 *    to argmax p with weight p_selected (not renormalised); probs = p. */
void oracle_gate_weights(int T, int n, int k, int mode, const double* H,
                         const int32_t* topk_idx, double* topk_w, double* probs) {
#pragma omp parallel for schedule(static)
  for (int t = 0; t < T; ++t) {
    const double* v = H + (size_t)t * n;
    const int32_t* idx = topk_idx + (size_t)t * k;
    double* w = topk_w + (size_t)t * k;
    double* g = probs ? probs + (size_t)t * n : NULL;
    if (mode == ORACLE_GATE_SWITCH_TOP1) {
      double m = v[idx[0]];
      double z = 0.0;
      for (int j = 0; j < n; ++j) z += exp(v[j] - m);
      for (int s = 0; s < k; ++s) w[s] = exp(v[idx[s]] - m) / z;
      if (g)
        for (int j = 0; j < n; ++j) g[j] = exp(v[j] - m) / z;
    } else {
      double m = v[idx[0]];
      double z = 0.0;
      for (int s = 0; s < k; ++s) z += exp(v[idx[s]] - m);
      for (int s = 0; s < k; ++s) w[s] = exp(v[idx[s]] - m) / z;
      if (g) {
        for (int j = 0; j < n; ++j) g[j] = 0.0;
        for (int s = 0; s < k; ++s) g[idx[s]] = w[s];
      }
    }
  }
}

/* O4 for the sigmoid gate.  [SURVEY] 6.2: s_i = Sigmoid(h_i(x)) and the kept
 * experts get g_i = s_i / sum over the kept j of s_j.  [SURVEY] 6.3: the
 * per-expert bias enters only the selection score h_i + b_i, so the caller
 * selects on h + b and passes the bias-free logits h here.  probs[T][n] is
 * the dense gate vector (g on the kept experts, 0 elsewhere). */
void oracle_sigmoid_gate_weights(int T, int n, int k, const double* h,
                                 const int32_t* topk_idx, double* topk_w, double* probs) {
#pragma omp parallel for schedule(static)
  for (int t = 0; t < T; ++t) {
    const double* v = h + (size_t)t * n;
    const int32_t* idx = topk_idx + (size_t)t * k;
    double* w = topk_w + (size_t)t * k;
    double z = 0.0;
    for (int s = 0; s < k; ++s) {
      w[s] = 1.0 / (1.0 + exp(-v[idx[s]]));
      z += w[s];
    }
    for (int s = 0; s < k; ++s) w[s] /= z;
    if (probs) {
      double* g = probs + (size_t)t * n;
      for (int j = 0; j < n; ++j) g[j] = 0.0;
      for (int s = 0; s < k; ++s) g[idx[s]] = w[s];
    }
  }
}

/* ------------------------------------------------------------------------ */
/* FP8 expert weights                                                        */
/* ------------------------------------------------------------------------ */

/* [SURVEY] section 9 (DeepSeek-V3 summary): the main computation runs in FP8.
 * Read here as FP8 E4M3 expert weights with one scale per output row (the
 * activations stay bf16).  The E4M3 format (the "e4m3fn" variant): 1 sign, 4
 * exponent bits with bias 7, 3 mantissa bits; exponent field 1..15 gives
 * (1 + m/8) 2^(e-7), field 0 gives the subnormals (m/8) 2^-6; the code
 * S.1111.111 is NaN; there are no infinities; the largest finite value is
 * 448 = 1.75 * 2^8. */
double oracle_e4m3_decode(int code) {
  int e = (code >> 3) & 15, m = code & 7;
  if (e == 15 && m == 7) return NAN;
  double v = e == 0 ? ldexp(m / 8.0, -6) : ldexp(1.0 + m / 8.0, e - 7);
  return (code & 0x80) ? -v : v;
}

/* Nearest E4M3 value, ties to the even code (round to nearest even):
 * the finite magnitudes, in code order 0..0x7e, increase; bisect for the
 * first one >= |v| and take the nearer of it and its predecessor (the even
 * code on a tie).  Magnitudes beyond 448 give 448 (saturation); NaN gives
 * 0x7f; the sign of zero is kept. */
static double e4m3_mag[0x7f]; /* decode(c) for the finite codes 0..0x7e */
static int e4m3_mag_ready = 0;

static void e4m3_table(void) {
  if (e4m3_mag_ready) return;
  for (int c = 0; c <= 0x7e; ++c) e4m3_mag[c] = oracle_e4m3_decode(c);
  e4m3_mag_ready = 1;
}

int oracle_e4m3_encode(double v) {
  if (v != v) return 0x7f;
  e4m3_table();
  int sign = signbit(v) ? 0x80 : 0;
  double a = fabs(v);
  if (a >= 448.0) return sign | 0x7e;
  int lo = 0, hi = 0x7e; /* find the first code with decode >= a */
  while (lo < hi) {
    int mid = (lo + hi) / 2;
    if (e4m3_mag[mid] < a) lo = mid + 1;
    else hi = mid;
  }
  int c = lo; /* decode(c) >= a, decode(c - 1) < a (or c == 0) */
  if (c > 0) {
    double up = e4m3_mag[c] - a, down = a - e4m3_mag[c - 1];
    if (down < up || (down == up && ((c - 1) & 1) == 0)) c = c - 1;
  }
  return sign | c;
}

/* Per-row quantization of a weight matrix w[rows][K] (fp32 or bf16 values):
 * scale s = amax / 448 and code = E4M3(w / s), both divisions in IEEE single
 * precision (a zero row gets s = 1); the value a code stands for is
 * decode(code) * s.  The single-precision arithmetic is part of the format's
 * definition here, so that the codes are reproducible bit for bit. */
void oracle_quantize_fp8_rows(int rows, int K, const double* w, uint8_t* codes,
                              double* scales) {
  e4m3_table();
#pragma omp parallel for schedule(static)
  for (int r = 0; r < rows; ++r) {
    double amax = 0.0;
    for (int k = 0; k < K; ++k) {
      double a = fabs(w[(size_t)r * K + k]);
      if (a > amax) amax = a;
    }
    float s = amax > 0.0 ? (float)amax / 448.0f : 1.0f;
    scales[r] = s;
    for (int k = 0; k < K; ++k) {
      float q = (float)w[(size_t)r * K + k] / s;
      codes[(size_t)r * K + k] = (uint8_t)oracle_e4m3_encode(q);
    }
  }
}

/* Router z-loss statistic.  [WIKI] part 2: the z-loss penalises the L2 norm
 * of the logits the gate feeds to its softmax.  Read as the squared norm,
 * summed over tokens: sum_t sum_j Z[t][j]^2 (the caller divides by T). */
double oracle_zloss_sum(int T, int n, const double* Z) {
  double acc = 0.0;
  for (int t = 0; t < T; ++t) {
    double r = 0.0;
    for (int j = 0; j < n; ++j) r += Z[(size_t)t * n + j] * Z[(size_t)t * n + j];
    acc += r;
  }
  return acc;
}

/* Gate entropy statistic.  [WIKI] part 2: the gate-entropy loss rewards a
 * high entropy of the gate's output distribution.  Sum over tokens of
 * -sum_j G[t][j] ln G[t][j], with 0 ln 0 = 0. */
double oracle_entropy_sum(int T, int n, const double* G) {
  double acc = 0.0;
  for (int t = 0; t < T; ++t) {
    double r = 0.0;
    for (int j = 0; j < n; ++j) {
      double g = G[(size_t)t * n + j];
      if (g > 0.0) r -= g * log(g);
    }
    acc += r;
  }
  return acc;
}

/* [SURVEY] 6.3 non-gradient bias controller: an expert that received more
 * than its even share of the step's assignments (counts_pre[i] > T*k/n)
 * loses gamma from its selection bias, one that received fewer gains gamma,
 * one exactly at the share keeps it. */
void oracle_bias_update(int n, int T, int k, const int32_t* counts_pre, double gamma,
                        double* bias) {
  double share = (double)T * (double)k / (double)n;
  for (int i = 0; i < n; ++i) {
    if ((double)counts_pre[i] > share) bias[i] -= gamma;
    else if ((double)counts_pre[i] < share) bias[i] += gamma;
  }
}

/* [PAPER] Importance(X) = sum over x in X of G(x): column sums of probs,
 * summed over tokens in ascending order. */
void oracle_importance(int T, int n, const double* probs, double* importance) {
  for (int i = 0; i < n; ++i) importance[i] = 0.0;
  for (int t = 0; t < T; ++t)
    for (int i = 0; i < n; ++i) importance[i] += probs[(size_t)t * n + i];
}

/* [PAPER] P(x,i) = Phi(((x.W_g)_i - kth_excluding(H(x),k,i)) /
 * Softplus((x.W_noise)_i)),  Load(X)_i = sum over x of P(x,i).
 * The numerator uses the clean logit (with the workload's logit bias); the
 * threshold is H_(k+1) for a kept expert and H_(k) otherwise (-inf when
 * k == n, which makes P = 1).  P may be NULL; load may be NULL. */
void oracle_load(int T, int n, int k, const double* clean, const double* sp,
                 const int32_t* topk_idx, const double* h_k, const double* h_k1, double* P,
                 double* load) {
  double* prob = P ? P : (double*)malloc(sizeof(double) * (size_t)T * n);
#pragma omp parallel for schedule(static)
  for (int t = 0; t < T; ++t) {
    const int32_t* idx = topk_idx + (size_t)t * k;
    for (int i = 0; i < n; ++i) {
      int kept = 0;
      for (int s = 0; s < k; ++s) kept |= (idx[s] == i);
      double thr = kept ? h_k1[t] : h_k[t];
      double z = (clean[(size_t)t * n + i] - thr) / sp[(size_t)t * n + i];
      prob[(size_t)t * n + i] = oracle_phi(z);
    }
  }
  if (load) {
    for (int i = 0; i < n; ++i) load[i] = 0.0;
    for (int t = 0; t < T; ++t)
      for (int i = 0; i < n; ++i) load[i] += prob[(size_t)t * n + i];
  }
  if (!P) free(prob);
}

/* ------------------------------------------------------------------------ */
/* Dispatch                                                                  */
/* ------------------------------------------------------------------------ */

/* O6.  [NOTES] engineering: all positions are merged into one batch per
 * expert; [SURVEY] 3.2 expert capacity C = tokens/E * capacity factor, with
 * overflow tokens passed on through the residual.
 * Walk the (token, slot) pairs in order; the r-th pair routed to expert e
 * becomes row offsets[e] + r of the merged batch if r < C, else it is dropped
 * (slot_pos = -1).  counts_pre counts every pair, counts the kept ones,
 * offsets[n+1] is the exclusive scan of counts, perm[row] = token.
 * cf <= 0 means no capacity limit.  Returns the number of kept rows. */
int oracle_dispatch(int T, int k, int n, double cf, const int32_t* topk_idx, int32_t* counts_pre,
                    int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* slot_pos) {
  int64_t cap = INT64_MAX;
  /* An expert receives at most T*k pairs, so any capacity above that is no
   * limit; clamping before the conversion keeps it defined for every finite
   * cf. */
  if (cf > 0.0) cap = (int64_t)fmin(floor(cf * (double)T * (double)k / (double)n), (double)T * k);
  for (int e = 0; e < n; ++e) counts_pre[e] = 0;
  for (int64_t a = 0; a < (int64_t)T * k; ++a) counts_pre[topk_idx[a]] += 1;
  for (int e = 0; e < n; ++e) counts[e] = (int32_t)(counts_pre[e] < cap ? counts_pre[e] : cap);
  offsets[0] = 0;
  for (int e = 0; e < n; ++e) offsets[e + 1] = offsets[e] + counts[e];
  int32_t* fill = (int32_t*)calloc((size_t)n, sizeof(int32_t));
  for (int t = 0; t < T; ++t) {
    for (int s = 0; s < k; ++s) {
      int64_t a = (int64_t)t * k + s;
      int e = topk_idx[a];
      int32_t r = fill[e]++;
      if (r < cap) {
        slot_pos[a] = offsets[e] + r;
        perm[offsets[e] + r] = t;
      } else {
        slot_pos[a] = -1;
      }
    }
  }
  free(fill);
  return offsets[n];
}

/* ------------------------------------------------------------------------ */
/* Experts                                                                   */
/* ------------------------------------------------------------------------ */

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* O7.  [NOTES] each expert is a feed-forward network with one ReLU hidden
 * layer, with its own parameters.  For one expert and its `rows` merged input
 * rows u[rows][d]:
 *   RELU:   hid_j = max(0, u . w1[j] + b1[j]),   y_i = hid . w2[i] + b2[i]
 *   SWIGLU: hid_j = silu(u . w1[j]) * (u . w3[j])  (the gated FFN of the
 *           fine-grained workload; no biases)
 * w1, w3: [h][d]; w2: [d][h]; b1: [h]; b2: [d] (biases may be NULL).
 * With bf16 != 0 the product inputs u and hid are rounded to bf16 first; the
 * weights are expected to hold bf16 values already. */
void oracle_expert_ffn(int rows, int d, int h, int act, int bf16, const double* u,
                       const double* w1, const double* b1, const double* w3, const double* w2,
                       const double* b2, double* y) {
#pragma omp parallel for schedule(static)
  for (int r = 0; r < rows; ++r) {
    double* ur = (double*)malloc(sizeof(double) * (size_t)d);
    double* hid = (double*)malloc(sizeof(double) * (size_t)h);
    for (int c = 0; c < d; ++c) {
      double v = u[(size_t)r * d + c];
      ur[c] = bf16 ? oracle_bf16_round(v) : v;
    }
    for (int j = 0; j < h; ++j) {
      double a = 0.0;
      for (int c = 0; c < d; ++c) a += ur[c] * w1[(size_t)j * d + c];
      double hj;
      if (act == ORACLE_ACT_SWIGLU) {
        double b = 0.0;
        for (int c = 0; c < d; ++c) b += ur[c] * w3[(size_t)j * d + c];
        hj = silu(a) * b;
      } else {
        if (b1) a += b1[j];
        hj = a > 0.0 ? a : 0.0;
      }
      hid[j] = bf16 ? oracle_bf16_round(hj) : hj;
    }
    for (int i = 0; i < d; ++i) {
      double a = 0.0;
      for (int j = 0; j < h; ++j) a += hid[j] * w2[(size_t)i * h + j];
      if (b2) a += b2[i];
      y[(size_t)r * d + i] = a;
    }
    free(ur);
    free(hid);
  }
}

/* ------------------------------------------------------------------------ */
/* Combine                                                                   */
/* ------------------------------------------------------------------------ */

/* O8.  [PAPER] y = sum_i G(x)_i E_i(x): for each token, the gate-weighted sum
 * of its kept slots' expert outputs, in slot order.  A dropped slot
 * (slot_pos < 0) adds nothing (the residual is the caller's). */
void oracle_combine(int T, int k, int d, const double* y_perm, const int32_t* slot_pos,
                    const double* topk_w, double* y) {
#pragma omp parallel for schedule(static)
  for (int t = 0; t < T; ++t) {
    double* yt = y + (size_t)t * d;
    for (int c = 0; c < d; ++c) yt[c] = 0.0;
    for (int s = 0; s < k; ++s) {
      int32_t p = slot_pos[(size_t)t * k + s];
      if (p < 0) continue;
      double w = topk_w[(size_t)t * k + s];
      for (int c = 0; c < d; ++c) yt[c] += w * y_perm[(size_t)p * d + c];
    }
  }
}

/* ------------------------------------------------------------------------ */
/* Auxiliary losses                                                          */
/* ------------------------------------------------------------------------ */

/* Squared coefficient of variation, population variance, two passes:
 * CV^2 = ((1/n) sum (v_i - mean)^2) / mean^2, and 0 when the mean is 0.
 * [NOTES] "负载均衡": both losses are squared CVs; [PAPER] L = w * CV(.)^2. */
double oracle_cv2(int n, const double* v) {
  double s = 0.0;
  for (int i = 0; i < n; ++i) s += v[i];
  double mean = s / n;
  if (mean == 0.0) return 0.0;
  double q = 0.0;
  for (int i = 0; i < n; ++i) q += (v[i] - mean) * (v[i] - mean);
  return (q / n) / (mean * mean);
}

/* O9 final.  losses[0] = w_importance * CV(Importance)^2,
 *            losses[1] = w_load * CV(Load)^2 (0 when load is NULL),
 *            losses[2] = alpha * n * sum_i f_i * P_i  ([SURVEY] 3.2), with
 *              f_i = counts_pre[i] / (T*k) (fraction of routed slots) and
 *              P_i = Importance_i / T (mean router probability),
 *            losses[3] = w_z * zsum / T, losses[4] = -w_entropy * entsum / T
 *              (zsum, entsum: oracle_zloss_sum / oracle_entropy_sum). */
void oracle_aux(int T, int k, int n, const double* importance, const double* load,
                const int32_t* counts_pre, double w_importance, double w_load, double alpha,
                double zsum, double entsum, double w_z, double w_entropy, double* losses) {
  losses[0] = w_importance * oracle_cv2(n, importance);
  losses[1] = load ? w_load * oracle_cv2(n, load) : 0.0;
  double acc = 0.0;
  if (T > 0) {
    for (int i = 0; i < n; ++i) {
      double f = (double)counts_pre[i] / ((double)T * (double)k);
      double p = importance[i] / (double)T;
      acc += f * p;
    }
  }
  losses[2] = alpha * (double)n * acc;
  /* [WIKI] part 2: mean squared logit norm (z-loss) and minus the mean gate
   * entropy (minimising it raises the entropy); 0 when T == 0. */
  losses[3] = T > 0 ? w_z * zsum / (double)T : 0.0;
  losses[4] = T > 0 ? -w_entropy * entsum / (double)T : 0.0;
}

/* O10 aux part.  Hierarchical load: for primary group g and expert e of that
 * group, Load_H[g*b+e] = Load_primary[g] * Load_g[e] / |X_g|, where Load_g is
 * the secondary gate's smooth load over the |X_g| tokens routed to group g
 * (0 when |X_g| = 0).  Reading of [NOTES] "分层 MoE" (the pages give the
 * structure only; this is the factorised expected count). */
void oracle_hier_load(int a, int b, const double* load_primary, const double* load_secondary,
                      const int32_t* group_tokens, double* load) {
  for (int g = 0; g < a; ++g)
    for (int e = 0; e < b; ++e)
      load[(size_t)g * b + e] =
          group_tokens[g] > 0
              ? load_primary[g] * load_secondary[(size_t)g * b + e] / (double)group_tokens[g]
              : 0.0;
}

/* ------------------------------------------------------------------------ */
/* Backward                                                                  */
/* ------------------------------------------------------------------------ */

/* The backward pass differentiates the scalar objective
 *   L = sum_t <dy_t, y_t> + sum_j dl_j * losses_j
 * (dy and dl are the upstream gradients) by the chain rule, one stage at a
 * time in reverse.  [PAPER] FAQ on back-propagating through the discrete
 * top-k: the selection happens before the softmax, so the kept gate values
 * stay differentiable functions of the gate's weights while the selection
 * itself is held fixed; [NOTES] "Noisy Top-K Gating": the noise term is what
 * lets the load-balancing loss pass gradients (through the smooth P(x,i)).
 * The bf16 roundings of the forward are taken as the identity (their
 * rounded values are used wherever the forward used them). */

/* d CV(v)^2 / d v_i with the population variance: writing m for the mean and
 * var for the variance, CV^2 = var / m^2, d var / d v_i = 2 (v_i - m) / n and
 * d m / d v_i = 1 / n, so the derivative is
 *   (2 / (n m^2)) * ((v_i - m) - var / m),
 * times `scale`; 0 where CV^2 is defined as 0 (mean 0). */
void oracle_cv2_grad(int n, const double* v, double scale, double* out) {
  double s = 0.0;
  for (int i = 0; i < n; ++i) s += v[i];
  double m = s / n;
  if (m == 0.0) {
    for (int i = 0; i < n; ++i) out[i] = 0.0;
    return;
  }
  double q = 0.0;
  for (int i = 0; i < n; ++i) q += (v[i] - m) * (v[i] - m);
  double var = q / n;
  for (int i = 0; i < n; ++i) out[i] = scale * (2.0 / (n * m * m)) * ((v[i] - m) - var / m);
}

/* Standard normal density, the derivative of Phi. */
static double std_normal_pdf(double z) { return exp(-0.5 * z * z) / sqrt(2.0 * acos(-1.0)); }

/* Gate backward for every token, the selection held fixed.
 * In (per token t, n experts):
 *   Hsel    the values the selection ranks (H; sigmoid gate: h + b),
 *   Zs      the logits the gate's softmax / sigmoid sees (H; sigmoid: h),
 *   clean, sp, z, raw   the noisy gate's parts (sp/z/raw NULL when
 *           noiseless): H = clean + z * Softplus(raw),
 *   topk_idx, topk_w, probs (the forward's outputs), h_k, h_k1 (H_(k) and
 *           H_(k+1)),
 *   dG      [T][k] gradient of L with respect to topk_w from the combine,
 *   dImp    [n] gradient of L with respect to Importance,
 *   dLoad   [n] gradient of L with respect to Load (NULL: none),
 *   c_z     dL / d(sum over tokens and experts of Zs^2),
 *   c_ent   dL / d(sum over tokens and experts of g ln g).
 * Out: dclean [T][n] = dL / d clean (sigmoid gate: dL / d h), and, for a
 *      noisy gate, draw [T][n] = dL / d raw.
 * Steps, per token:
 *  1. gradient on the gate distribution: the combine's dG on the kept
 *     slots, dImp (Importance sums the distribution), and c_ent (ln g + 1)
 *     from the entropy statistic (0 ln 0 terms contribute nothing);
 *  2. through the normalisation: softmax over the kept values (top-k),
 *     over all n (Switch), or Sigmoid then division by the kept sum;
 *  3. the z statistic adds 2 c_z Zs_j for every expert;
 *  4. Load: P_i = Phi((clean_i - thr_i) / sp_i) moves with clean_i, with
 *     sp_i and with its threshold thr_i, which is the H of another expert:
 *     the expert of rank k (H_(k+1)) for a kept i, the one of rank k-1
 *     (H_(k)) otherwise; no gradient where the threshold is -inf;
 *  5. H = clean + z sp: d clean += dH, d sp += z dH, and
 *     d raw = d sp * Sigmoid(raw) (the derivative of Softplus). */
void oracle_gate_backward(int T, int n, int k, int mode, const double* Hsel, const double* Zs,
                          const double* clean, const double* sp, const double* z,
                          const double* raw, const int32_t* topk_idx, const double* topk_w,
                          const double* probs, const double* h_k, const double* h_k1,
                          const double* dG, const double* dImp, const double* dLoad,
                          double c_z, double c_ent, double* dclean, double* draw) {
#pragma omp parallel for schedule(static)
  for (int t = 0; t < T; ++t) {
    const double* hs = Hsel + (size_t)t * n;
    const double* zs = Zs + (size_t)t * n;
    const int32_t* idx = topk_idx + (size_t)t * k;
    const double* w = topk_w + (size_t)t * k;
    const double* p = probs + (size_t)t * n;
    const double* dg = dG + (size_t)t * k;
    double* dH = (double*)calloc((size_t)n, sizeof(double));
    double* dsp = (double*)calloc((size_t)n, sizeof(double));
    double* dc = dclean + (size_t)t * n;
    for (int j = 0; j < n; ++j) dc[j] = 0.0;

    /* 1 + 2: the gate distribution and its normalisation. */
    if (mode == ORACLE_GATE_SWITCH_TOP1) {
      double* gp = (double*)malloc(sizeof(double) * (size_t)n);
      for (int j = 0; j < n; ++j) {
        gp[j] = dImp[j];
        if (p[j] > 0.0) gp[j] += c_ent * (log(p[j]) + 1.0);
      }
      gp[idx[0]] += dg[0];
      double dot = 0.0;
      for (int j = 0; j < n; ++j) dot += p[j] * gp[j];
      for (int j = 0; j < n; ++j) dH[j] += p[j] * (gp[j] - dot);
      free(gp);
    } else {
      double* gg = (double*)malloc(sizeof(double) * (size_t)k);
      for (int s = 0; s < k; ++s) {
        gg[s] = dg[s] + dImp[idx[s]];
        if (w[s] > 0.0) gg[s] += c_ent * (log(w[s]) + 1.0);
      }
      double dot = 0.0;
      for (int s = 0; s < k; ++s) dot += w[s] * gg[s];
      if (mode == ORACLE_GATE_SIGMOID_BIAS) {
        /* g_s = sig_s / S: d g_s / d h_j = sig'_j / S * ([s == j] - g_s). */
        double S = 0.0;
        for (int s = 0; s < k; ++s) S += 1.0 / (1.0 + exp(-zs[idx[s]]));
        for (int s = 0; s < k; ++s) {
          double sg = 1.0 / (1.0 + exp(-zs[idx[s]]));
          dH[idx[s]] += sg * (1.0 - sg) / S * (gg[s] - dot);
        }
      } else {
        for (int s = 0; s < k; ++s) dH[idx[s]] += w[s] * (gg[s] - dot);
      }
      free(gg);
    }

    /* 3: the z statistic. */
    for (int j = 0; j < n; ++j) dH[j] += 2.0 * c_z * zs[j];

    /* 4: the smooth load estimator. */
    if (dLoad && sp) {
      int owner_k = -1; /* the expert of rank k: largest H outside the kept set */
      for (int j = 0; j < n; ++j) {
        int kept = 0;
        for (int s = 0; s < k; ++s) kept |= (idx[s] == j);
        if (kept) continue;
        if (owner_k < 0 || hs[j] > hs[owner_k]) owner_k = j;
      }
      for (int i = 0; i < n; ++i) {
        int kept = 0;
        for (int s = 0; s < k; ++s) kept |= (idx[s] == i);
        double thr = kept ? h_k1[t] : h_k[t];
        if (isinf(thr)) continue;
        double spi = sp[(size_t)t * n + i];
        double zeta = (clean[(size_t)t * n + i] - thr) / spi;
        double q = dLoad[i] * std_normal_pdf(zeta) / spi;
        dc[i] += q;
        dsp[i] -= q * zeta;
        dH[kept ? owner_k : idx[k - 1]] -= q;
      }
    }

    /* 5: back to clean and raw. */
    for (int j = 0; j < n; ++j) dc[j] += dH[j];
    if (draw && sp) {
      for (int j = 0; j < n; ++j) {
        double zz = z ? z[(size_t)t * n + j] : 0.0;
        double r = raw[(size_t)t * n + j];
        draw[(size_t)t * n + j] = (dsp[j] + zz * dH[j]) / (1.0 + exp(-r));
      }
    }
    free(dH);
    free(dsp);
  }
}
