/*
 * sv_oracle.c -- plain, slow, sequential CPU oracle for the speculative-
 * sampling verify step.  TEST INFRASTRUCTURE ONLY: it is linked or called by
 * the tests, by the package's smoke check and by the CPU-baseline leg of the
 * benchmark, never by the product path.  It shares no code, header, table or
 * constant with the HIP library.
 *
 * Everything is double precision and sequential, in the order the pages state
 * the algorithm.  Sources (page title, section):
 *
 *   [P1] "深入推测解码：从概念到实现" (Exploring Speculative Decoding: From
 *        Concept to Implementation), section "保证原始分布": sample x from the
 *        draft q, accept with probability min(1, p(x)/q(x)) (case a p>=q
 *        accept, case b p<q accept with p/q), on rejection resample from
 *        max(0, p - q); worked example q=0.4, p=0.2 -> accept half the time.
 *   [P2] "RTP-LLM Speculative Engine 深度解析", section "拒绝采样算法"
 *        (SpeculativeSampler::stochasticSample): per proposed position compare
 *        a Uniform(0,1) draw with p_score/p_draft, on rejection sample from
 *        normalize(max(0, p_score - p_draft)) and stop.
 *   [P3] "投机采样" (razer666.cn), section "投机解码算法", steps 3-5: the
 *        accepted count n, the adjusted distribution norm(max(0, p_{n+1} -
 *        q_{n+1})), the extra token from p_{gamma+1} when every guess passes,
 *        output length in [1, gamma+1]; section "验证阶段的策略 / 精确匹配":
 *        greedy exact match against the max-probability token.
 *
 * Readings where the pages are silent (each is listed with its reason in the
 * design notes of the repository):
 *   - p = softmax(l / T) for target logits, and the same T for draft logits;
 *   - T that is not a positive, normal, finite float selects greedy: accept
 *     iff the draft's logit equals the row maximum (ties accepted), the
 *     emitted token is the lowest index attaining the maximum, no uniforms;
 *   - acceptance is the strict test u < ratio with u in [0,1);
 *   - q(x) = 0 gives ratio +inf when p(x) > 0, else 0;
 *   - one-hot (n-gram) drafts: ratio = p(x), residual = p with p(x) zeroed;
 *   - a draft id outside [0, V) is never accepted and zeroes nothing;
 *   - inverse CDF: smallest i with C_i > u * S, C_i the running sum;
 *     if none, the largest i with r_i > 0; if S = 0, draw from p instead;
 *   - uniforms from Philox4x64-10 with key (seed, 0) and counter
 *     (offset, b, j, 0); word 0 -> acceptance uniform, word 1 -> draw
 *     uniform; u = (w >> 40) * 2^-24.
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define SVO_F32 0
#define SVO_BF16 1

#define SVO_MODE_PROB 0
#define SVO_MODE_ONEHOT 1

#define SVO_FLAG_BAD_DRAFT_ID 1u
#define SVO_FLAG_BAD_NUM_DRAFTS 2u
#define SVO_FLAG_ZERO_RESIDUAL 4u

/* ------------------------------------------------------------------------ */
/* Philox4x64-10: Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As   */
/* Easy as 1, 2, 3" (SC'11).  Ten rounds; each round multiplies counter      */
/* words 0 and 2 by the two round multipliers, mixes the high halves with    */
/* the other words and the key, and the key is bumped by the two Weyl        */
/* constants between rounds.                                                 */
/* ------------------------------------------------------------------------ */
static void mul_hilo64(uint64_t a, uint64_t b, uint64_t *hi, uint64_t *lo) {
  unsigned __int128 prod = (unsigned __int128)a * (unsigned __int128)b;
  *hi = (uint64_t)(prod >> 64);
  *lo = (uint64_t)prod;
}

void svo_philox4x64_10(const uint64_t ctr_in[4], const uint64_t key_in[2],
                       uint64_t out[4]) {
  const uint64_t mult0 = 0xD2E7470EE14C6C93ULL, mult1 = 0xCA5A826395121157ULL;
  const uint64_t weyl0 = 0x9E3779B97F4A7C15ULL, weyl1 = 0xBB67AE8584CAA73BULL;
  uint64_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
  uint64_t k0 = key_in[0], k1 = key_in[1];
  for (int round = 0; round < 10; ++round) {
    uint64_t hi0, lo0, hi1, lo1;
    mul_hilo64(mult0, c0, &hi0, &lo0);
    mul_hilo64(mult1, c2, &hi1, &lo1);
    uint64_t n0 = hi1 ^ c1 ^ k0;
    uint64_t n1 = lo1;
    uint64_t n2 = hi0 ^ c3 ^ k1;
    uint64_t n3 = lo0;
    c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    k0 += weyl0;
    k1 += weyl1;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* The two uniforms of request b at position j (see the header comment). */
void svo_uniforms(uint64_t seed, uint64_t offset, uint64_t b, uint64_t j,
                  double *u_acc, double *u_rec) {
  uint64_t ctr[4] = {offset, b, j, 0};
  uint64_t key[2] = {seed, 0};
  uint64_t w[4];
  svo_philox4x64_10(ctr, key, w);
  *u_acc = (double)(w[0] >> 40) * 0x1p-24;
  *u_rec = (double)(w[1] >> 40) * 0x1p-24;
}

/* ------------------------------------------------------------------------ */
/* Element access: bf16 is the top half of an IEEE float.                    */
/* ------------------------------------------------------------------------ */
static double load_elem(const void *base, int dtype, size_t idx) {
  if (dtype == SVO_BF16) {
    uint16_t bits = ((const uint16_t *)base)[idx];
    uint32_t wide = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &wide, sizeof f);
    return (double)f;
  }
  return (double)((const float *)base)[idx];
}

static void load_row(const void *base, int dtype, size_t row, int V,
                     double *dst) {
  for (int i = 0; i < V; ++i) dst[i] = load_elem(base, dtype, row * (size_t)V + i);
}

/* Sampling is selected by a positive, normal, finite temperature. */
int svo_is_sampling(float T) { return isnormal(T) && T > 0.0f; }

/* Neumaier-compensated sequential sum. */
static double sum_compensated(const double *v, int n) {
  double s = 0.0, c = 0.0;
  for (int i = 0; i < n; ++i) {
    double t = s + v[i];
    if (fabs(s) >= fabs(v[i]))
      c += (s - t) + v[i];
    else
      c += (v[i] - t) + s;
    s = t;
  }
  return s + c;
}

/* p_i = exp((l_i - m) / T) / sum_k exp((l_k - m) / T), m = max_i l_i. */
void svo_softmax(const double *logits, int V, double T, double *p) {
  double m = -INFINITY;
  for (int i = 0; i < V; ++i)
    if (logits[i] > m) m = logits[i];
  for (int i = 0; i < V; ++i) p[i] = exp((logits[i] - m) / T);
  double Z = sum_compensated(p, V);
  for (int i = 0; i < V; ++i) p[i] /= Z;
}

/* Lowest index attaining the maximum. */
int svo_argmax(const double *v, int V) {
  int best = 0;
  for (int i = 1; i < V; ++i)
    if (v[i] > v[best]) best = i;
  return best;
}

/* Acceptance ratio p(x)/q(x) with q(x) = 0 read as +inf (p(x) > 0) or 0. */
double svo_accept_ratio(double px, double qx) {
  if (qx > 0.0) return px / qx;
  return px > 0.0 ? INFINITY : 0.0;
}

/* Residual law after a rejection of draft x (unnormalized):
 *   probabilistic draft: r_i = max(0, p_i - q_i)   [P1 step 4, P2, P3 step 4]
 *   one-hot draft:       r_i = p_i, r_x = 0        (q is the point mass at x)
 * x outside [0, V) zeroes nothing. */
void svo_residual(const double *p, const double *q, int mode, int x, int V,
                  double *r) {
  if (mode == SVO_MODE_PROB) {
    for (int i = 0; i < V; ++i) {
      double d = p[i] - q[i];
      r[i] = d > 0.0 ? d : 0.0;
    }
  } else {
    for (int i = 0; i < V; ++i) r[i] = p[i];
    if (x >= 0 && x < V) r[x] = 0.0;
  }
}

/* Inverse-CDF draw from the unnormalized law r with uniform u in [0, 1).
 * Returns the token, or -1 when S = sum r is not positive.  *margin is the
 * distance of u*S to the nearer CDF boundary of the chosen token, over S. */
int svo_draw(const double *r, int V, double u, double *margin) {
  double S = sum_compensated(r, V);
  if (!(S > 0.0)) {
    *margin = 0.0;
    return -1;
  }
  double theta = u * S;
  double below = 0.0, C = 0.0;
  int y = -1;
  for (int i = 0; i < V; ++i) {
    below = C;
    C += r[i];
    if (C > theta) {
      y = i;
      break;
    }
  }
  if (y < 0) { /* rounding left theta past the last boundary */
    for (int i = V - 1; i >= 0; --i)
      if (r[i] > 0.0) { y = i; break; }
    *margin = 0.0;
    return y;
  }
  double lo = theta - below, hi = C - theta;
  *margin = (lo < hi ? lo : hi) / S;
  return y;
}

/* Where token y sits in the inverse CDF of svo_draw: with the same running
 * sums C and total S, *lo = C_{y-1} / S and *hi = C_y / S, so a uniform u
 * selects y iff lo <= u < hi (u * S against C).  Returns r_y / S; for y
 * outside [0, V) or S not positive returns 0 and sets lo = hi = NaN. */
double svo_draw_interval(const double *r, int V, int y, double *lo,
                         double *hi) {
  double S = sum_compensated(r, V);
  *lo = NAN;
  *hi = NAN;
  if (!(S > 0.0) || y < 0 || y >= V) return 0.0;
  double C = 0.0;
  for (int i = 0; i < y; ++i) C += r[i];
  *lo = C / S;
  *hi = (C + r[y]) / S;
  return r[y] / S;
}

/* ------------------------------------------------------------------------ */
/* The verify step, driven by explicit uniforms.                              */
/*                                                                          */
/*   target      [B][K+1][V] logits, target_dtype                            */
/*   draft       [B][K][V] draft logits (draft_is_probs = 0) or normalized   */
/*               probabilities (draft_is_probs = 1); NULL = all one-hot      */
/*   draft_mode  [B] 0 = probabilistic, 1 = one-hot; NULL = all probabilistic*/
/*   draft_ids   [B][K]; num_drafts [B]; temperatures [B]                    */
/*   u_acc,u_rec [B][K+1]                                                     */
/*   out_tokens  [B][K+1]: accepted drafts, the emitted token, then -1       */
/*   out_num_accepted [B]                                                     */
/*   out_p,out_q [B][K] or NULL: p_j(x_j), q_j(x_j) for every j < n_b of a   */
/*               sampling request (q = 1 for one-hot), NaN elsewhere         */
/*   out_margin_acc [B][K] or NULL: |u - ratio| of each evaluated sampling   */
/*               decision, +inf for greedy decisions, NaN if not evaluated   */
/*   out_margin_rec [B] or NULL: draw margin (+inf for greedy)               */
/* Returns the OR of the SVO_FLAG_* conditions met.                          */
/* ------------------------------------------------------------------------ */
uint32_t svo_verify_with_uniforms(
    int B, int K, int V, int target_dtype, const void *target, int draft_dtype,
    const void *draft, int draft_is_probs, const uint8_t *draft_mode,
    const int32_t *draft_ids, const int32_t *num_drafts,
    const float *temperatures, const double *u_acc, const double *u_rec,
    int32_t *out_tokens, int32_t *out_num_accepted, double *out_p,
    double *out_q, double *out_margin_acc, double *out_margin_rec) {
  uint32_t flags = 0;
  double *tl = malloc(sizeof(double) * (size_t)V); /* target logits row */
  double *dl = malloc(sizeof(double) * (size_t)V); /* draft row */
  double *p = malloc(sizeof(double) * (size_t)V);
  double *q = malloc(sizeof(double) * (size_t)V);
  double *r = malloc(sizeof(double) * (size_t)V);

  for (int b = 0; b < B; ++b) {
    int n = num_drafts[b];
    if (n < 0 || n > K) {
      flags |= SVO_FLAG_BAD_NUM_DRAFTS;
      n = n < 0 ? 0 : K;
    }
    const float T = temperatures[b];
    const int sampling = svo_is_sampling(T);
    int mode = SVO_MODE_PROB;
    if (draft == NULL || (draft_mode != NULL && draft_mode[b] != 0))
      mode = SVO_MODE_ONEHOT;
    const size_t trow0 = (size_t)b * (K + 1); /* target row index of j = 0 */
    const size_t drow0 = (size_t)b * K;

    for (int j = 0; j < K; ++j) {
      if (out_p) out_p[(size_t)b * K + j] = NAN;
      if (out_q) out_q[(size_t)b * K + j] = NAN;
      if (out_margin_acc) out_margin_acc[(size_t)b * K + j] = NAN;
    }

    /* Sequential decisions, stopping at the first rejection. */
    int n_acc = 0, rejected = 0;
    for (int j = 0; j < n; ++j) {
      const int x = draft_ids[(size_t)b * K + j];
      const int valid = x >= 0 && x < V;
      if (!valid) flags |= SVO_FLAG_BAD_DRAFT_ID;
      load_row(target, target_dtype, trow0 + j, V, tl);
      int accept;
      if (!sampling) {
        double m = tl[svo_argmax(tl, V)];
        accept = valid && tl[x] == m;
        if (out_margin_acc) out_margin_acc[(size_t)b * K + j] = INFINITY;
      } else {
        svo_softmax(tl, V, (double)T, p);
        double px = valid ? p[x] : 0.0, qx;
        if (mode == SVO_MODE_PROB) {
          load_row(draft, draft_dtype, drow0 + j, V, dl);
          if (draft_is_probs)
            memcpy(q, dl, sizeof(double) * (size_t)V);
          else
            svo_softmax(dl, V, (double)T, q);
          qx = valid ? q[x] : 0.0;
        } else {
          qx = 1.0;
        }
        double ratio = valid ? svo_accept_ratio(px, qx) : 0.0;
        double u = u_acc[(size_t)b * (K + 1) + j];
        accept = u < ratio;
        if (out_margin_acc)
          out_margin_acc[(size_t)b * K + j] = fabs(u - ratio);
      }
      if (!accept) {
        rejected = 1;
        break;
      }
      n_acc++;
    }

    /* The emitted token: correction at the rejected position, else bonus. */
    const int jemit = n_acc; /* == rejected position, or n when all passed */
    int y;
    double margin_rec = INFINITY;
    load_row(target, target_dtype, trow0 + jemit, V, tl);
    if (!sampling) {
      y = svo_argmax(tl, V);
    } else {
      svo_softmax(tl, V, (double)T, p);
      if (rejected) {
        const int x = draft_ids[(size_t)b * K + jemit];
        if (mode == SVO_MODE_PROB) {
          load_row(draft, draft_dtype, drow0 + jemit, V, dl);
          if (draft_is_probs)
            memcpy(q, dl, sizeof(double) * (size_t)V);
          else
            svo_softmax(dl, V, (double)T, q);
        }
        svo_residual(p, q, mode, x, V, r);
      } else {
        memcpy(r, p, sizeof(double) * (size_t)V);
      }
      double u = u_rec[(size_t)b * (K + 1) + jemit];
      y = svo_draw(r, V, u, &margin_rec);
      if (y < 0) { /* no residual mass: draw from p itself */
        flags |= SVO_FLAG_ZERO_RESIDUAL;
        y = svo_draw(p, V, u, &margin_rec);
        margin_rec = 0.0;
      }
    }

    for (int j = 0; j < K + 1; ++j) {
      int32_t tok = -1;
      if (j < n_acc) tok = draft_ids[(size_t)b * K + j];
      else if (j == n_acc) tok = y;
      out_tokens[(size_t)b * (K + 1) + j] = tok;
    }
    out_num_accepted[b] = n_acc;
    if (out_margin_rec) out_margin_rec[b] = margin_rec;

    /* Diagnostics: p_j(x_j) and q_j(x_j) for every drafted position. */
    if (sampling && (out_p || out_q)) {
      for (int j = 0; j < n; ++j) {
        const int x = draft_ids[(size_t)b * K + j];
        if (x < 0 || x >= V) continue;
        load_row(target, target_dtype, trow0 + j, V, tl);
        svo_softmax(tl, V, (double)T, p);
        double qx = 1.0;
        if (mode == SVO_MODE_PROB) {
          load_row(draft, draft_dtype, drow0 + j, V, dl);
          if (draft_is_probs)
            qx = dl[x];
          else {
            svo_softmax(dl, V, (double)T, q);
            qx = q[x];
          }
        }
        if (out_p) out_p[(size_t)b * K + j] = p[x];
        if (out_q) out_q[(size_t)b * K + j] = qx;
      }
    }
  }
  free(tl); free(dl); free(p); free(q); free(r);
  return flags;
}

/* The verify step with uniforms from the Philox stream (seed, offset). */
uint32_t svo_verify(int B, int K, int V, int target_dtype, const void *target,
                    int draft_dtype, const void *draft, int draft_is_probs,
                    const uint8_t *draft_mode, const int32_t *draft_ids,
                    const int32_t *num_drafts, const float *temperatures,
                    uint64_t seed, uint64_t offset, int32_t *out_tokens,
                    int32_t *out_num_accepted, double *out_p, double *out_q,
                    double *out_margin_acc, double *out_margin_rec) {
  size_t n = (size_t)(B > 0 ? B : 1) * (K + 1);
  double *ua = malloc(sizeof(double) * n), *ur = malloc(sizeof(double) * n);
  for (int b = 0; b < B; ++b)
    for (int j = 0; j <= K; ++j)
      svo_uniforms(seed, offset, (uint64_t)b, (uint64_t)j,
                   &ua[(size_t)b * (K + 1) + j], &ur[(size_t)b * (K + 1) + j]);
  uint32_t flags = svo_verify_with_uniforms(
      B, K, V, target_dtype, target, draft_dtype, draft, draft_is_probs,
      draft_mode, draft_ids, num_drafts, temperatures, ua, ur, out_tokens,
      out_num_accepted, out_p, out_q, out_margin_acc, out_margin_rec);
  free(ua);
  free(ur);
  return flags;
}

/* ------------------------------------------------------------------------ */
/* Draft-token sampler: the step that produces the drafts the verify step    */
/* checks.  [P1] section "引言", the propose pseudo-code: every draft step    */
/* samples one token from the draft model's logits and appends it.  [P3]     */
/* section "投机解码算法", 第一步 - 采样: for each guess i, q_i is the draft     */
/* model's distribution given the prefix and the earlier guesses, and x_i is */
/* sampled from q_i.                                                         */
/*                                                                          */
/* Readings: q_j = softmax(l_j / T_b), the temperature the verify step also  */
/* applies to draft logits; a greedy temperature takes the lowest argmax;    */
/* the draw is the verify step's inverse CDF with a uniform of its own: word */
/* 0 of the Philox block at counter (offset, b, j, 1), key (seed, 0).  The   */
/* verify step's counters have word 3 = 0, so no uniform is shared.          */
/* ------------------------------------------------------------------------ */
double svo_draft_uniform(uint64_t seed, uint64_t offset, uint64_t b, uint64_t j) {
  uint64_t ctr[4] = {offset, b, j, 1};
  uint64_t key[2] = {seed, 0};
  uint64_t w[4];
  svo_philox4x64_10(ctr, key, w);
  return (double)(w[0] >> 40) * 0x1p-24;
}

/*   draft       [B][K][V] draft logits, dtype                                */
/*   num_drafts  [B]: rows j < n_b are sampled; NULL samples all K rows.      */
/*               Counts outside [0, K] are clamped and flagged.               */
/*   out_ids     [B][K]: x_j, or -1 for j >= n_b                              */
/*   out_q       [B][K] or NULL: q_j(x_j); 1 for greedy rows, NaN if unused   */
/*   out_margin  [B][K] or NULL: draw margin; +inf greedy, NaN if unused      */
/* Returns the OR of the SVO_FLAG_* conditions met.                          */
uint32_t svo_draft_sample(int B, int K, int V, int dtype, const void *draft,
                          const int32_t *num_drafts, const float *temperatures,
                          uint64_t seed, uint64_t offset, int32_t *out_ids,
                          double *out_q, double *out_margin) {
  uint32_t flags = 0;
  double *l = malloc(sizeof(double) * (size_t)(V > 0 ? V : 1));
  double *q = malloc(sizeof(double) * (size_t)(V > 0 ? V : 1));
  for (int b = 0; b < B; ++b) {
    int n = num_drafts ? num_drafts[b] : K;
    if (n < 0 || n > K) {
      flags |= SVO_FLAG_BAD_NUM_DRAFTS;
      n = n < 0 ? 0 : K;
    }
    const float T = temperatures[b];
    for (int j = 0; j < K; ++j) {
      const size_t o = (size_t)b * K + j;
      int32_t x = -1;
      double qx = NAN, margin = NAN;
      if (j < n) {
        load_row(draft, dtype, o, V, l);
        if (!svo_is_sampling(T)) {
          x = svo_argmax(l, V);
          qx = 1.0;
          margin = INFINITY;
        } else {
          svo_softmax(l, V, (double)T, q);
          x = svo_draw(q, V, svo_draft_uniform(seed, offset, (uint64_t)b, (uint64_t)j),
                       &margin);
          qx = q[x];
        }
      }
      out_ids[o] = x;
      if (out_q) out_q[o] = qx;
      if (out_margin) out_margin[o] = margin;
    }
  }
  free(l);
  free(q);
  return flags;
}

/* ------------------------------------------------------------------------ */
/* n-gram prompt-lookup proposer.  [P1] section "n-gram": take the last n    */
/* tokens of the sequence, find where they occurred before, and propose the  */
/* k tokens that followed that earlier occurrence; the match is the longest  */
/* one with n in [min_n, max_n] (prompt_lookup_min / max), and proposals     */
/* stop at max_model_len.                                                    */
/*                                                                          */
/* Readings where the page is silent: the earlier occurrence must end before */
/* the last token (it may overlap the suffix); among occurrences of the      */
/* longest matching n-gram the most recent one is taken (the one a search    */
/* over the reversed sequence meets first); the count is                     */
/* min(k, tokens after the occurrence, max_model_len - N); no match gives no */
/* drafts.  This is the definition written out: every n from the longest    */
/* down, every end position from the latest down.                           */
/*                                                                          */
/*   context   [B][stride] int32; lens [B] (clamped into [0, stride])        */
/*   out_drafts [B][k]: the proposed tokens, then -1; out_num [B]            */
/* ------------------------------------------------------------------------ */
void svo_ngram_propose(int B, const int32_t *context, int stride,
                       const int32_t *lens, int min_n, int max_n, int k,
                       int max_model_len, int32_t *out_drafts, int32_t *out_num) {
  for (int b = 0; b < B; ++b) {
    const int32_t *t = context + (size_t)b * stride;
    int N = lens[b];
    if (N < 0) N = 0;
    if (N > stride) N = stride;
    int count = 0, start = -1;
    for (int n = max_n; n >= min_n && start < 0; --n) {
      if (n > N - 1) continue;
      for (int e = N - 2; e >= n - 1; --e) { /* occurrence t[e-n+1 .. e] */
        int match = 1;
        for (int i = 0; i < n; ++i)
          if (t[e - i] != t[N - 1 - i]) { match = 0; break; }
        if (match) { start = e + 1; break; }
      }
    }
    if (start >= 0) {
      count = k;
      if (count > N - start) count = N - start;
      if (count > max_model_len - N) count = max_model_len - N;
      if (count < 0) count = 0;
    }
    for (int i = 0; i < k; ++i)
      out_drafts[(size_t)b * k + i] = i < count ? t[start + i] : -1;
    out_num[b] = count;
  }
}

/* ------------------------------------------------------------------------ */
/* Typical acceptance.  [P3] section 验收标准, Typical Acceptance: a draft    */
/* token is accepted when its probability exceeds a hard threshold; the      */
/* threshold can be relaxed through a top-k constraint; the tokens that form */
/* the longest accepted run are kept and the rest discarded.                 */
/*                                                                          */
/* Readings: the probability is the target's p_j = softmax(l_j / T_b); x_j  */
/* is accepted iff p_j(x_j) > eps or x_j ranks among the top_k of row j,    */
/* i.e. #{i : l_i > l_x} < top_k (top_k = 0: the threshold alone; ties at   */
/* the k-th value are all in); the walk stops at the first rejection; the    */
/* token at that position, or the bonus token after n_b acceptances, is     */
/* drawn from p itself with the verify step's draw uniform (no residual:    */
/* there is no q); greedy requests keep the exact-match rule.               */
/* Outputs as svo_verify; out_p[b][j] = p_j(x_j) for every drafted j of a    */
/* sampling request; margins: |p(x) - eps| (+inf when the rank decides, or  */
/* for greedy requests; NaN past the first rejection).                      */
/* ------------------------------------------------------------------------ */
uint32_t svo_verify_typical(int B, int K, int V, int target_dtype,
                            const void *target, const int32_t *draft_ids,
                            const int32_t *num_drafts,
                            const float *temperatures, double eps, int top_k,
                            uint64_t seed, uint64_t offset, int32_t *out_tokens,
                            int32_t *out_num_accepted, double *out_p,
                            double *out_margin_acc, double *out_margin_rec) {
  uint32_t flags = 0;
  double *l = malloc(sizeof(double) * (size_t)V);
  double *p = malloc(sizeof(double) * (size_t)V);
  for (int b = 0; b < B; ++b) {
    int n = num_drafts[b];
    if (n < 0 || n > K) {
      flags |= SVO_FLAG_BAD_NUM_DRAFTS;
      n = n < 0 ? 0 : K;
    }
    const float T = temperatures[b];
    const int sampling = svo_is_sampling(T);
    const size_t row0 = (size_t)b * (K + 1);
    for (int j = 0; j < K; ++j) {
      if (out_p) out_p[(size_t)b * K + j] = NAN;
      if (out_margin_acc) out_margin_acc[(size_t)b * K + j] = NAN;
    }
    int n_acc = 0;
    for (int j = 0; j < n; ++j) {
      const int x = draft_ids[(size_t)b * K + j];
      const int valid = x >= 0 && x < V;
      if (!valid) flags |= SVO_FLAG_BAD_DRAFT_ID;
      load_row(target, target_dtype, row0 + j, V, l);
      int accept;
      double margin = INFINITY;
      if (!sampling) {
        accept = valid && l[x] == l[svo_argmax(l, V)];
      } else {
        svo_softmax(l, V, (double)T, p);
        int above = 0;
        if (valid)
          for (int i = 0; i < V; ++i) above += l[i] > l[x];
        const double px = valid ? p[x] : 0.0;
        if (valid && above < top_k) {
          accept = 1;
        } else {
          accept = valid && px > eps;
          margin = fabs(px - eps);
        }
      }
      if (out_margin_acc) out_margin_acc[(size_t)b * K + j] = margin;
      if (!accept) break;
      n_acc++;
    }
    int y;
    double margin_rec = INFINITY;
    load_row(target, target_dtype, row0 + n_acc, V, l);
    if (!sampling) {
      y = svo_argmax(l, V);
    } else {
      double ua, ur;
      svo_uniforms(seed, offset, (uint64_t)b, (uint64_t)n_acc, &ua, &ur);
      svo_softmax(l, V, (double)T, p);
      y = svo_draw(p, V, ur, &margin_rec);
    }
    for (int j = 0; j < K + 1; ++j) {
      int32_t tok = -1;
      if (j < n_acc) tok = draft_ids[(size_t)b * K + j];
      else if (j == n_acc) tok = y;
      out_tokens[(size_t)b * (K + 1) + j] = tok;
    }
    out_num_accepted[b] = n_acc;
    if (out_margin_rec) out_margin_rec[b] = margin_rec;

    /* Diagnostics: p_j(x_j) for every drafted position, as in svo_verify. */
    if (sampling && out_p) {
      for (int j = 0; j < n; ++j) {
        const int x = draft_ids[(size_t)b * K + j];
        if (x < 0 || x >= V) continue;
        load_row(target, target_dtype, row0 + j, V, l);
        svo_softmax(l, V, (double)T, p);
        out_p[(size_t)b * K + j] = p[x];
      }
    }
  }
  free(l);
  free(p);
  return flags;
}

/* ------------------------------------------------------------------------ */
/* Token-tree verification.  [P3] section 验证阶段的策略 / 验证方案: draft     */
/* sequences with shared prefixes are merged into a token tree (a trie),     */
/* and the target scores every node in one pass (tree attention); SpecInfer  */
/* and Spectr are named for the multi-branch rule, which the page does not   */
/* give.                                                                     */
/*                                                                          */
/* Reading: the page's chain rule applied child by child, keeping the       */
/* target law (multi-step speculative sampling).  At node v the children    */
/* (nodes whose parent is v, in index order) are tested in turn; the k-th   */
/* test uses the law left by the k earlier rejections:                      */
/*   probabilistic tree: p'_k = max(0, p - c_k q) / Z_k, c_0 = 0, Z_0 = 1,   */
/*     c_{k+1} = c_k + Z_k, Z_k = sum_i max(0, p_i - c_k q_i); child x is    */
/*     accepted iff u < p'_k(x) / q(x)  (k = 0 is the chain's p(x)/q(x));    */
/*   one-hot tree (no draft rows): p'_k = p with the rejected siblings'     */
/*     tokens removed, renormalized; accepted iff u < p'_k(x);              */
/*   greedy: the first child whose token attains the row maximum.           */
/* An accepted child becomes v.  When every child is rejected, or v has     */
/* none, one token is drawn at v from p'_k (from p at a leaf), the emitted  */
/* token.  p at node i = softmax(target[i] / T_b), q = softmax(draft[i] /   */
/* T_b), the law node i's children were drawn from.  Uniforms: the block at */
/* counter (offset, b, i, 0) gives in word 0 the acceptance uniform of node */
/* i + 1 and in word 1 the draw uniform at node i, so a chain-shaped tree   */
/* (parent of i = i - 1) reproduces the verify step exactly.  A child with  */
/* an id outside [0, V) is never accepted (counted as a rejection); nodes  */
/* whose parent is not an earlier node are never visited; both are flagged. */
/*                                                                          */
/*   target [B][N][V], draft [B][N][V] logits (or normalized q with         */
/*   draft_is_probs) or NULL; tokens, parents [B][N];                       */
/*   num_nodes [B] (clamped into [1, N]); out_tokens [B][N]: the accepted   */
/*   path's tokens, the emitted token, then -1; out_num_accepted [B];       */
/*   out_last_node [B]: the deepest accepted node (0 = root);               */
/*   out_margin_acc [B]: smallest |u - ratio| of the sampling tests made    */
/*   (+inf if none); out_margin_rec [B]: the draw margin (+inf greedy).     */
/* ------------------------------------------------------------------------ */
#define SVO_FLAG_BAD_TREE 16u

uint32_t svo_verify_tree(int B, int N, int V, int target_dtype,
                         const void *target, int draft_dtype, const void *draft,
                         int draft_is_probs, const int32_t *tokens,
                         const int32_t *parents,
                         const int32_t *num_nodes, const float *temperatures,
                         uint64_t seed, uint64_t offset, int32_t *out_tokens,
                         int32_t *out_num_accepted, int32_t *out_last_node,
                         double *out_margin_acc, double *out_margin_rec) {
  uint32_t flags = 0;
  double *l = malloc(sizeof(double) * (size_t)V);
  double *p = malloc(sizeof(double) * (size_t)V);
  double *q = malloc(sizeof(double) * (size_t)V);
  double *r = malloc(sizeof(double) * (size_t)V);
  int *removed = malloc(sizeof(int) * (size_t)V);
  for (int b = 0; b < B; ++b) {
    int n = num_nodes[b];
    if (n < 1 || n > N) {
      flags |= SVO_FLAG_BAD_NUM_DRAFTS;
      n = n < 1 ? 1 : N;
    }
    const int32_t *tok = tokens + (size_t)b * N, *par = parents + (size_t)b * N;
    for (int i = 1; i < n; ++i)
      if (par[i] < 0 || par[i] >= i) flags |= SVO_FLAG_BAD_TREE;
    const float T = temperatures[b];
    const int sampling = svo_is_sampling(T);
    const int onehot = draft == NULL;
    double margin_acc = INFINITY, margin_rec = INFINITY;
    int v = 0, n_acc = 0, y = -1;
    int32_t *out = out_tokens + (size_t)b * N;
    for (int i = 0; i < N; ++i) out[i] = -1;
    for (;;) {
      load_row(target, target_dtype, (size_t)b * N + v, V, l);
      if (sampling) svo_softmax(l, V, (double)T, p);
      if (sampling && !onehot) {
        load_row(draft, draft_dtype, (size_t)b * N + v, V, q);
        if (!draft_is_probs) svo_softmax(q, V, (double)T, q);
      }
      double ck = 0.0, Zk = 1.0;   /* probabilistic residual after k rejections */
      int nrej = 0;
      for (int i = 0; i < V; ++i) removed[i] = 0;
      int next = -1;
      for (int c = v + 1; c < n && next < 0; ++c) {
        if (par[c] != v) continue;
        const int x = tok[c];
        const int valid = x >= 0 && x < V;
        if (!valid) flags |= SVO_FLAG_BAD_DRAFT_ID;
        int accept;
        if (!sampling) {
          accept = valid && l[x] == l[svo_argmax(l, V)];
        } else {
          double ua, ur, ratio = 0.0;
          svo_uniforms(seed, offset, (uint64_t)b, (uint64_t)(c - 1), &ua, &ur);
          if (valid && onehot) {
            ratio = removed[x] ? 0.0 : p[x] / Zk;
          } else if (valid) {
            const double num = p[x] - ck * q[x];
            ratio = svo_accept_ratio((num > 0.0 ? num : 0.0) / Zk, q[x]);
          }
          accept = ua < ratio;
          const double m = fabs(ua - ratio);
          if (m < margin_acc) margin_acc = m;
        }
        if (accept) {
          next = c;
          break;
        }
        nrej++;
        if (sampling && onehot) {
          if (valid && !removed[x]) {
            removed[x] = 1;
            Zk -= p[x];
          }
        } else if (sampling) {
          ck += Zk;
          for (int i = 0; i < V; ++i) {
            const double d = p[i] - ck * q[i];
            r[i] = d > 0.0 ? d : 0.0;
          }
          Zk = sum_compensated(r, V);
        }
      }
      if (next >= 0) {
        out[n_acc++] = tok[next];
        v = next;
        continue;
      }
      /* every child rejected, or a leaf: the emitted token is drawn at v */
      if (!sampling) {
        y = svo_argmax(l, V);
      } else {
        double ua, ur;
        svo_uniforms(seed, offset, (uint64_t)b, (uint64_t)v, &ua, &ur);
        if (onehot) {
          for (int i = 0; i < V; ++i) r[i] = removed[i] ? 0.0 : p[i];
        } else if (nrej > 0) {
          for (int i = 0; i < V; ++i) {
            const double d = p[i] - ck * q[i];
            r[i] = d > 0.0 ? d : 0.0;
          }
        } else {
          memcpy(r, p, sizeof(double) * (size_t)V);
        }
        y = svo_draw(r, V, ur, &margin_rec);
        if (y < 0) { /* no residual mass: draw from p itself */
          flags |= SVO_FLAG_ZERO_RESIDUAL;
          y = svo_draw(p, V, ur, &margin_rec);
          margin_rec = 0.0;
        }
      }
      break;
    }
    out[n_acc] = y;
    out_num_accepted[b] = n_acc;
    out_last_node[b] = v;
    if (out_margin_acc) out_margin_acc[b] = margin_acc;
    if (out_margin_rec) out_margin_rec[b] = margin_rec;
  }
  free(l); free(p); free(q); free(r); free(removed);
  return flags;
}

/* ------------------------------------------------------------------------ */
/* Outputs along a given path.  A decision whose uniform lies within        */
/* rounding of its threshold, or a draw within rounding of a CDF boundary,  */
/* may go the other way in an implementation that rounds differently.  Its  */
/* output then follows another path through the same method: the functions  */
/* below evaluate the method along a path the caller names, with the same   */
/* arithmetic as the walks above, so that every step of that output can be  */
/* checked (each step either agrees with this arithmetic or lies within the */
/* caller's band of its threshold).  They decide nothing themselves.        */
/* ------------------------------------------------------------------------ */

/* Shared output of a path's emitted token: the oracle's own token there and
 * its draw margin, and where a given token y sits in that draw's law. */
static void path_emit(const double *r, int V, double u, int y, int32_t *tok,
                      double *margin_rec, double *out_y) {
  double m = 0.0;
  *tok = svo_draw(r, V, u, &m);
  *margin_rec = m;
  double lo, hi;
  const double mass = svo_draw_interval(r, V, y, &lo, &hi);
  out_y[0] = lo;
  out_y[1] = hi;
  out_y[2] = mass;
  out_y[3] = u;
}

/* The verify step of one request along the path "the first n_path drafts
 * accepted, then the token at position n_path emitted": the correction
 * drawn after a rejection at n_path when n_path < n_b, else the bonus token.
 *
 *   target [K+1][V], draft [K][V] or NULL (one-hot; also when onehot != 0),
 *   draft_ids [K], num_drafts (clamped into [0, K]), T, u_acc / u_rec [K+1]
 *   as in svo_verify_with_uniforms; 0 <= n_path <= n_b.
 *   out_accept[j], out_margin[j], j < K: for every position the path
 *     decides (j <= n_path and j < n_b) the oracle's decision there (1
 *     accept, 0 reject) and |u - ratio| (+inf for greedy); NaN elsewhere.
 *   *out_tok, *out_margin_rec: the oracle's emitted token at n_path and its
 *     draw margin (greedy: the lowest argmax, +inf).
 *   out_y[4] for token y: (lo, hi, mass, u) of y in that draw's law (see
 *     svo_draw_interval) and the draw uniform; greedy: NaN.
 * Returns the SVO_FLAG_* conditions met on the path. */
uint32_t svo_verify_path(int K, int V, int target_dtype, const void *target,
                         int draft_dtype, const void *draft,
                         int draft_is_probs, int onehot,
                         const int32_t *draft_ids, int num_drafts, float T,
                         const double *u_acc, const double *u_rec, int n_path,
                         int y, double *out_accept, double *out_margin,
                         int32_t *out_tok, double *out_margin_rec,
                         double *out_y) {
  uint32_t flags = 0;
  int n = num_drafts;
  if (n < 0 || n > K) {
    flags |= SVO_FLAG_BAD_NUM_DRAFTS;
    n = n < 0 ? 0 : K;
  }
  const int sampling = svo_is_sampling(T);
  const int mode = (draft == NULL || onehot) ? SVO_MODE_ONEHOT : SVO_MODE_PROB;
  for (int j = 0; j < K; ++j) out_accept[j] = out_margin[j] = NAN;
  for (int i = 0; i < 4; ++i) out_y[i] = NAN;
  *out_tok = -1;
  *out_margin_rec = NAN;
  if (n_path < 0 || n_path > n) return flags;
  double *tl = malloc(sizeof(double) * (size_t)V);
  double *dl = malloc(sizeof(double) * (size_t)V);
  double *p = malloc(sizeof(double) * (size_t)V);
  double *q = malloc(sizeof(double) * (size_t)V);
  double *r = malloc(sizeof(double) * (size_t)V);

  /* every decision the path makes: accepts at 0..n_path-1, the stop at n_path */
  for (int j = 0; j <= n_path && j < n; ++j) {
    const int x = draft_ids[j];
    const int valid = x >= 0 && x < V;
    if (!valid) flags |= SVO_FLAG_BAD_DRAFT_ID;
    load_row(target, target_dtype, (size_t)j, V, tl);
    if (!sampling) {
      out_accept[j] = valid && tl[x] == tl[svo_argmax(tl, V)];
      out_margin[j] = INFINITY;
      continue;
    }
    svo_softmax(tl, V, (double)T, p);
    double px = valid ? p[x] : 0.0, qx = 1.0;
    if (mode == SVO_MODE_PROB) {
      load_row(draft, draft_dtype, (size_t)j, V, dl);
      if (draft_is_probs)
        memcpy(q, dl, sizeof(double) * (size_t)V);
      else
        svo_softmax(dl, V, (double)T, q);
      qx = valid ? q[x] : 0.0;
    }
    const double ratio = valid ? svo_accept_ratio(px, qx) : 0.0;
    out_accept[j] = u_acc[j] < ratio;
    out_margin[j] = fabs(u_acc[j] - ratio);
  }

  /* the emitted token at n_path */
  load_row(target, target_dtype, (size_t)n_path, V, tl);
  if (!sampling) {
    *out_tok = svo_argmax(tl, V);
    *out_margin_rec = INFINITY;
  } else {
    svo_softmax(tl, V, (double)T, p);
    if (n_path < n) {
      if (mode == SVO_MODE_PROB) {
        load_row(draft, draft_dtype, (size_t)n_path, V, dl);
        if (draft_is_probs)
          memcpy(q, dl, sizeof(double) * (size_t)V);
        else
          svo_softmax(dl, V, (double)T, q);
      }
      svo_residual(p, q, mode, draft_ids[n_path], V, r);
    } else {
      memcpy(r, p, sizeof(double) * (size_t)V);
    }
    if (!(sum_compensated(r, V) > 0.0)) { /* no residual mass: from p */
      flags |= SVO_FLAG_ZERO_RESIDUAL;
      memcpy(r, p, sizeof(double) * (size_t)V);
      path_emit(r, V, u_rec[n_path], y, out_tok, out_margin_rec, out_y);
      *out_margin_rec = 0.0;
    } else {
      path_emit(r, V, u_rec[n_path], y, out_tok, out_margin_rec, out_y);
    }
  }
  free(tl); free(dl); free(p); free(q); free(r);
  return flags;
}

/* Typical acceptance of one request along the path "n_path drafts
 * accepted, then the token at n_path drawn from p_{n_path}" (see
 * svo_verify_typical for the rule).  Arguments and outputs as in
 * svo_verify_path, without draft rows; out_margin[j] is |p(x) - eps|, or
 * +inf where the rank decides or the request is greedy. */
uint32_t svo_verify_typical_path(int K, int V, int target_dtype,
                                 const void *target, const int32_t *draft_ids,
                                 int num_drafts, float T, double eps,
                                 int top_k, const double *u_rec, int n_path,
                                 int y, double *out_accept, double *out_margin,
                                 int32_t *out_tok, double *out_margin_rec,
                                 double *out_y) {
  uint32_t flags = 0;
  int n = num_drafts;
  if (n < 0 || n > K) {
    flags |= SVO_FLAG_BAD_NUM_DRAFTS;
    n = n < 0 ? 0 : K;
  }
  const int sampling = svo_is_sampling(T);
  for (int j = 0; j < K; ++j) out_accept[j] = out_margin[j] = NAN;
  for (int i = 0; i < 4; ++i) out_y[i] = NAN;
  *out_tok = -1;
  *out_margin_rec = NAN;
  if (n_path < 0 || n_path > n) return flags;
  double *l = malloc(sizeof(double) * (size_t)V);
  double *p = malloc(sizeof(double) * (size_t)V);
  for (int j = 0; j <= n_path && j < n; ++j) {
    const int x = draft_ids[j];
    const int valid = x >= 0 && x < V;
    if (!valid) flags |= SVO_FLAG_BAD_DRAFT_ID;
    load_row(target, target_dtype, (size_t)j, V, l);
    double margin = INFINITY;
    int accept;
    if (!sampling) {
      accept = valid && l[x] == l[svo_argmax(l, V)];
    } else {
      svo_softmax(l, V, (double)T, p);
      int above = 0;
      if (valid)
        for (int i = 0; i < V; ++i) above += l[i] > l[x];
      const double px = valid ? p[x] : 0.0;
      if (valid && above < top_k) {
        accept = 1;
      } else {
        accept = valid && px > eps;
        margin = fabs(px - eps);
      }
    }
    out_accept[j] = accept;
    out_margin[j] = margin;
  }
  load_row(target, target_dtype, (size_t)n_path, V, l);
  if (!sampling) {
    *out_tok = svo_argmax(l, V);
    *out_margin_rec = INFINITY;
  } else {
    svo_softmax(l, V, (double)T, p);
    path_emit(p, V, u_rec[n_path], y, out_tok, out_margin_rec, out_y);
  }
  free(l);
  free(p);
  return flags;
}

/* Token-tree verification of one request along a given walk: path[0] = 0
 * (the root), path[1..a] the accepted nodes in order (each a child of the
 * one before), and the emitted token drawn at path[a] after every child of
 * path[a] was rejected.  At each path node the children are tested in index
 * order as in svo_verify_tree: those before the next path node are
 * rejected, the next path node is accepted, and at the last node all are
 * rejected; the law after each rejection is updated as there.
 *
 *   target [N][V], draft [N][V] or NULL, tokens / parents [N], num_nodes
 *   (clamped into [1, N]), T; ua[i] / ur[i] = words 0 / 1 of the Philox
 *   block of node index i (ua[c - 1] tests child c, ur[v] draws at v).
 *   out_tests[4 k + 0..3] for the k-th test on the walk: the child tested,
 *     the walk's outcome there (1 accepted, 0 rejected), the oracle's
 *     decision, and |u - ratio| (+inf for greedy); *n_tests = k.
 *   *out_tok, *out_margin_rec, out_y[4]: as in svo_verify_path, for the
 *     draw at path[a].
 * Returns the SVO_FLAG_* conditions met on the walk, and -1 in *n_tests
 * for a path that is not a walk of this tree. */
uint32_t svo_verify_tree_path(int N, int V, int target_dtype,
                              const void *target, int draft_dtype,
                              const void *draft, int draft_is_probs,
                              const int32_t *tokens, const int32_t *parents,
                              int num_nodes, float T, const double *ua,
                              const double *ur, int a, const int32_t *path,
                              int y, double *out_tests, int *n_tests,
                              int32_t *out_tok, double *out_margin_rec,
                              double *out_y) {
  uint32_t flags = 0;
  int n = num_nodes;
  if (n < 1 || n > N) {
    flags |= SVO_FLAG_BAD_NUM_DRAFTS;
    n = n < 1 ? 1 : N;
  }
  *n_tests = 0;
  *out_tok = -1;
  *out_margin_rec = NAN;
  for (int i = 0; i < 4; ++i) out_y[i] = NAN;
  if (a < 0 || a >= n || path[0] != 0) {
    *n_tests = -1;
    return flags;
  }
  for (int k = 1; k <= a; ++k)
    if (path[k] <= path[k - 1] || path[k] >= n || parents[path[k]] != path[k - 1]) {
      *n_tests = -1;
      return flags;
    }
  const int sampling = svo_is_sampling(T);
  const int onehot = draft == NULL;
  double *l = malloc(sizeof(double) * (size_t)V);
  double *p = malloc(sizeof(double) * (size_t)V);
  double *q = malloc(sizeof(double) * (size_t)V);
  double *r = malloc(sizeof(double) * (size_t)V);
  int *removed = malloc(sizeof(int) * (size_t)V);
  int nt = 0;
  for (int k = 0; k <= a; ++k) {
    const int v = path[k];
    const int next = k < a ? path[k + 1] : -1;
    load_row(target, target_dtype, (size_t)v, V, l);
    if (sampling) svo_softmax(l, V, (double)T, p);
    if (sampling && !onehot) {
      load_row(draft, draft_dtype, (size_t)v, V, q);
      if (!draft_is_probs) svo_softmax(q, V, (double)T, q);
    }
    double ck = 0.0, Zk = 1.0;
    int nrej = 0;
    for (int i = 0; i < V; ++i) removed[i] = 0;
    for (int c = v + 1; c < n; ++c) {
      if (parents[c] != v) continue;
      const int x = tokens[c];
      const int valid = x >= 0 && x < V;
      if (!valid) flags |= SVO_FLAG_BAD_DRAFT_ID;
      int accept;
      double m = INFINITY;
      if (!sampling) {
        accept = valid && l[x] == l[svo_argmax(l, V)];
      } else {
        double ratio = 0.0;
        if (valid && onehot) {
          ratio = removed[x] ? 0.0 : p[x] / Zk;
        } else if (valid) {
          const double num = p[x] - ck * q[x];
          ratio = svo_accept_ratio((num > 0.0 ? num : 0.0) / Zk, q[x]);
        }
        accept = ua[c - 1] < ratio;
        m = fabs(ua[c - 1] - ratio);
      }
      out_tests[4 * nt + 0] = c;
      out_tests[4 * nt + 1] = c == next;
      out_tests[4 * nt + 2] = accept;
      out_tests[4 * nt + 3] = m;
      nt++;
      if (c == next) break; /* the walk moves on to the next path node */
      nrej++;
      if (sampling && onehot) {
        if (valid && !removed[x]) {
          removed[x] = 1;
          Zk -= p[x];
        }
      } else if (sampling) {
        ck += Zk;
        for (int i = 0; i < V; ++i) {
          const double d = p[i] - ck * q[i];
          r[i] = d > 0.0 ? d : 0.0;
        }
        Zk = sum_compensated(r, V);
      }
    }
    if (k < a) continue;
    /* the draw at the last node */
    if (!sampling) {
      *out_tok = svo_argmax(l, V);
      *out_margin_rec = INFINITY;
    } else {
      if (onehot) {
        for (int i = 0; i < V; ++i) r[i] = removed[i] ? 0.0 : p[i];
      } else if (nrej > 0) {
        for (int i = 0; i < V; ++i) {
          const double d = p[i] - ck * q[i];
          r[i] = d > 0.0 ? d : 0.0;
        }
      } else {
        memcpy(r, p, sizeof(double) * (size_t)V);
      }
      if (!(sum_compensated(r, V) > 0.0)) { /* no residual mass: from p */
        flags |= SVO_FLAG_ZERO_RESIDUAL;
        memcpy(r, p, sizeof(double) * (size_t)V);
        path_emit(r, V, ur[v], y, out_tok, out_margin_rec, out_y);
        *out_margin_rec = 0.0;
      } else {
        path_emit(r, V, ur[v], y, out_tok, out_margin_rec, out_y);
      }
    }
  }
  *n_tests = nt;
  free(l); free(p); free(q); free(r); free(removed);
  return flags;
}
