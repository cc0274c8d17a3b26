/*
 * oracle.c -- plain fp64 CPU oracle for bf16 causal grouped-query attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load or call this file.  It shares no code,
 * header, table or helper with the HIP library; neither includes the other.
 *
 * What it computes.  The h3.c issue "Qwen text encoder: sequence exceeds Metal
 * threadgroup memory with reference video + ref images (>=150 frames)"
 * (sections "Error" and "Suggested fix directions") names the operation: the
 * text encoder's bf16 causal GQA, which forms, for every query token, the
 * causal attention score row over all earlier tokens and takes its softmax.
 * The tiled scheme that the same section proposes is only a faster way to the
 * same numbers, so this oracle writes the plain definition out, query row by
 * query row, in double precision:
 *
 *   g        = h / G,  G = Hq / Hkv       (heads g*G .. g*G+G-1 share KV head g)
 *   x_j      = scale * sum_d Q[i,h,d] * K[j,g,d]      for j = 0 .. i (local)
 *   m        = max_j x_j
 *   l        = sum_j exp(x_j - m)
 *   O[i,h,:] = sum_j exp(x_j - m) / l * V[j,g,:]
 *   LSE[h,i] = m + log(l)                               (natural log)
 *
 * Readings taken where the pages say nothing (they are listed, with reasons,
 * in the design notes): the contiguous head grouping g = h / G; the diagonal
 * is visible (key j is seen by query i iff j <= i); the softmax scale is the
 * caller's fp32 value widened to double; LSE is the natural log of the sum of
 * exponentials of the scaled scores; in a packed (varlen) batch positions are
 * local to each sequence and no query sees another sequence's keys.
 *
 * Inputs are bf16 bit patterns (uint16); decoding bf16 to double is exact, so
 * the only rounding is fp64's own.  Outputs stay in double.
 *
 * Split-KV partials (the first fix direction of the same section: the score
 * row computed in pieces, with intermediate results in global memory) are
 * attention restricted to a key range: oracle_gqa_causal_keyrange evaluates
 * the same definition over keys j in [key_begin, key_end) with j <= i, giving
 * O = 0 and LSE = -inf where that set is empty.  Merging partials is done in
 * oracle/__init__.py (merge_partials), in double precision with numpy.
 *
 * The DiT's attention on the vpipe page and in the h3.c project README is the
 * same softmax without the causal mask: oracle_gqa_bidirectional lets every
 * query of a sequence see all S keys (j = 0 .. S-1), nothing else changes.
 *
 * The step before attention: the h3.c project README ("Checkpoint layout and
 * media pipeline") runs a fused QK-normalization / RoPE kernel on the DiT's
 * Q and K rows.  The pages give no formulas; oracle_qk_norm_rope takes the
 * plainest reading, the Qwen-family convention:
 *   RMS norm of one (token, head) row x[0..D):  y_d = x_d / sqrt(mean_d(x_d^2) + eps) * w_d
 *   rotary embedding (rotate-half pairs (i, i + D/2), i < D/2), position p:
 *     a_i = p * theta^(-2i/D)
 *     z_i       = y_i * cos(a_i) - y_{i+D/2} * sin(a_i)
 *     z_{i+D/2} = y_{i+D/2} * cos(a_i) + y_i * sin(a_i)
 * either step optional, all in double.
 *
 * Parallelism: (token, KV head) items are independent; OpenMP spreads them
 * over threads.  One item evaluates the G query heads that share the KV head,
 * reading each key and value row once for all G; each head's sums still run
 * in the order the definition above writes them, whatever the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double bf16_bits_to_double(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* Attention of the G query heads h = g*G .. g*G+G-1 of one query token over
 * keys [first_key, last_key] (packed token indices, inclusive), i.e. the causal
 * prefix of its own sequence.  The G heads share KV head g, so each key row is
 * read once for all of them; every head's arithmetic is the plain definition
 * on its own, sums in key (or dimension) order exactly as for a single row:
 *   dot  = ((q_0 k_0 + q_1 k_1) + q_2 k_2) + ...        (d = 0, 1, ..)
 *   m    = max over keys, l = sum_t exp(x_t - m)        (t = 0, 1, ..)
 *   o[d] = sum_t (exp(x_t - m) / l) v_t[d]              (t = 0, 1, ..)
 * q_rows: the G rows Q[pos, g*G + hh, :] (D values each, stride D).
 * Writes G rows of D doubles to out_o (stride o_stride) and G log-sum-exps to
 * out_lse (stride lse_stride).  scores: caller scratch of at least
 * G * (last_key - first_key + 1) doubles; dot, mx, sum: scratch of G doubles
 * each; qt: G * D doubles; vd: D doubles. */
static void attend_group(const uint16_t* q_rows, int64_t G,
                         const uint16_t* k, const uint16_t* v,
                         int64_t kv_token_stride,     /* Hkv * D */
                         int64_t g, int64_t D, double scale,
                         int64_t first_key, int64_t last_key,
                         double* scores, double* dot, double* qt, double* mx, double* sum,
                         double* vd,
                         double* out_o, int64_t o_stride,
                         double* out_lse, int64_t lse_stride) {
  const int64_t n = last_key - first_key + 1;

  /* the G query rows decoded once, dimension-major: qt[d * G + hh] */
  for (int64_t hh = 0; hh < G; ++hh)
    for (int64_t d = 0; d < D; ++d) qt[d * G + hh] = bf16_bits_to_double(q_rows[hh * D + d]);

  /* scores of the causal rows: scores[hh * n + t] */
  for (int64_t t = 0; t < n; ++t) {
    const uint16_t* k_row = k + (first_key + t) * kv_token_stride + g * D;
    for (int64_t hh = 0; hh < G; ++hh) dot[hh] = 0.0;
    for (int64_t d = 0; d < D; ++d) {
      const double kd = bf16_bits_to_double(k_row[d]);
      for (int64_t hh = 0; hh < G; ++hh) dot[hh] += qt[d * G + hh] * kd;
    }
    for (int64_t hh = 0; hh < G; ++hh) scores[hh * n + t] = scale * dot[hh];
  }

  /* per head: the max, then the sum of shifted exponentials */
  for (int64_t hh = 0; hh < G; ++hh) {
    const double* x = scores + hh * n;
    double m = x[0];
    for (int64_t t = 1; t < n; ++t)
      if (x[t] > m) m = x[t];
    double l = 0.0;
    for (int64_t t = 0; t < n; ++t) l += exp(x[t] - m);
    mx[hh] = m;
    sum[hh] = l;
    for (int64_t d = 0; d < D; ++d) out_o[hh * o_stride + d] = 0.0;
  }

  /* probability-weighted sums of the value rows, each value row decoded once */
  for (int64_t t = 0; t < n; ++t) {
    const uint16_t* v_row = v + (first_key + t) * kv_token_stride + g * D;
    for (int64_t d = 0; d < D; ++d) vd[d] = bf16_bits_to_double(v_row[d]);
    for (int64_t hh = 0; hh < G; ++hh) {
      const double p = exp(scores[hh * n + t] - mx[hh]) / sum[hh];
      double* o = out_o + hh * o_stride;
      for (int64_t d = 0; d < D; ++d) o[d] += p * vd[d];
    }
  }
  for (int64_t hh = 0; hh < G; ++hh) out_lse[hh * lse_stride] = mx[hh] + log(sum[hh]);
}

/*
 * Packed-batch form; the fixed-length call is the case num_seqs = 1,
 * cu_seqlens = {0, S}.
 *
 * q: [T, Hq, D] bf16 bits; k, v: [T, Hkv, D] bf16 bits; T = cu_seqlens[num_seqs].
 * cu_seqlens: host int64[num_seqs + 1], cu[0] = 0, non-decreasing.
 * tokens: the ntok packed query positions to evaluate (any order, repeats ok).
 * o_out: [ntok, Hq, D] doubles; lse_out: [Hq, ntok] doubles.
 * threads <= 0 means "OpenMP default".
 * Returns 0, or a negative code for invalid arguments (nothing is written).
 */
int oracle_gqa_causal_varlen(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                             const int64_t* cu_seqlens, int64_t num_seqs,
                             int64_t Hq, int64_t Hkv, int64_t D, float scale_f32,
                             const int64_t* tokens, int64_t ntok,
                             double* o_out, double* lse_out, int threads) {
  if (!q || !k || !v || !cu_seqlens || !o_out || !lse_out || (ntok > 0 && !tokens)) return -1;
  if (num_seqs < 1 || Hq < 1 || Hkv < 1 || D < 1 || Hq % Hkv != 0) return -2;
  if (cu_seqlens[0] != 0) return -3;
  for (int64_t s = 0; s < num_seqs; ++s)
    if (cu_seqlens[s + 1] < cu_seqlens[s]) return -3;
  const int64_t T = cu_seqlens[num_seqs];
  for (int64_t t = 0; t < ntok; ++t)
    if (tokens[t] < 0 || tokens[t] >= T) return -4;

  const int64_t G = Hq / Hkv;
  const double scale = (double)scale_f32;
  const int64_t n_items = ntok * Hkv;
  int status = 0;

#ifdef _OPENMP
  if (threads > 0) omp_set_num_threads(threads);
#else
  (void)threads;
#endif

#pragma omp parallel
  {
    int64_t longest = 0;
    for (int64_t s = 0; s < num_seqs; ++s)
      if (cu_seqlens[s + 1] - cu_seqlens[s] > longest) longest = cu_seqlens[s + 1] - cu_seqlens[s];
    double* scores = (double*)malloc(sizeof(double) * (size_t)(G * (longest > 0 ? longest : 1) + 3 * G + G * D + D));
    if (!scores) {
#pragma omp atomic write
      status = -5;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t item = 0; item < n_items; ++item) {
      if (!scores) continue;
      const int64_t ti = item / Hkv;
      const int64_t g = item % Hkv;
      const int64_t pos = tokens[ti];
      /* the sequence holding this packed position */
      int64_t s = 0;
      while (!(cu_seqlens[s] <= pos && pos < cu_seqlens[s + 1])) ++s;
      const int64_t h0 = g * G;
      attend_group(q + (pos * Hq + h0) * D, G, k, v, Hkv * D, g, D, scale, cu_seqlens[s], pos,
                   scores + 3 * G + G * D + D, scores, scores + G, scores + G + G * D,
                   scores + 2 * G + G * D, scores + 3 * G + G * D, o_out + (ti * Hq + h0) * D, D,
                   lse_out + h0 * ntok + ti, ntok);
    }
    free(scores);
  }
  return status;
}

/* Fixed-length form: one sequence of S tokens. */
int oracle_gqa_causal(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t S,
                      int64_t Hq, int64_t Hkv, int64_t D, float scale_f32,
                      const int64_t* tokens, int64_t ntok, double* o_out, double* lse_out,
                      int threads) {
  if (S < 0) return -2;
  const int64_t cu[2] = {0, S};
  return oracle_gqa_causal_varlen(q, k, v, cu, 1, Hq, Hkv, D, scale_f32, tokens, ntok, o_out,
                                  lse_out, threads);
}

/*
 * Key-range form (one sequence of S tokens): query token i attends to the keys
 * j with key_begin <= j < key_end and j <= i.  Where no key qualifies the row's
 * output is O = 0, LSE = -inf.  Same layouts and return codes as above.
 */
int oracle_gqa_causal_keyrange(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                               int64_t S, int64_t Hq, int64_t Hkv, int64_t D, float scale_f32,
                               int64_t key_begin, int64_t key_end,
                               const int64_t* tokens, int64_t ntok,
                               double* o_out, double* lse_out, int threads) {
  if (!q || !k || !v || !o_out || !lse_out || (ntok > 0 && !tokens)) return -1;
  if (S < 0 || Hq < 1 || Hkv < 1 || D < 1 || Hq % Hkv != 0) return -2;
  for (int64_t t = 0; t < ntok; ++t)
    if (tokens[t] < 0 || tokens[t] >= S) return -4;

  const int64_t G = Hq / Hkv;
  const double scale = (double)scale_f32;
  const int64_t n_items = ntok * Hkv;
  int status = 0;

#ifdef _OPENMP
  if (threads > 0) omp_set_num_threads(threads);
#else
  (void)threads;
#endif

#pragma omp parallel
  {
    double* scores = (double*)malloc(sizeof(double) * (size_t)(G * (S > 0 ? S : 1) + 3 * G + G * D + D));
    if (!scores) {
#pragma omp atomic write
      status = -5;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t item = 0; item < n_items; ++item) {
      if (!scores) continue;
      const int64_t ti = item / Hkv;
      const int64_t g = item % Hkv;
      const int64_t pos = tokens[ti];
      const int64_t h0 = g * G;
      const int64_t first = key_begin > 0 ? key_begin : 0;
      const int64_t last = (key_end - 1 < pos) ? key_end - 1 : pos;
      if (first > last) {
        for (int64_t hh = 0; hh < G; ++hh) {
          double* o_row = o_out + (ti * Hq + h0 + hh) * D;
          for (int64_t d = 0; d < D; ++d) o_row[d] = 0.0;
          lse_out[(h0 + hh) * ntok + ti] = -INFINITY;
        }
        continue;
      }
      attend_group(q + (pos * Hq + h0) * D, G, k, v, Hkv * D, g, D, scale, first, last,
                   scores + 3 * G + G * D + D, scores, scores + G, scores + G + G * D,
                   scores + 2 * G + G * D, scores + 3 * G + G * D, o_out + (ti * Hq + h0) * D, D,
                   lse_out + h0 * ntok + ti, ntok);
    }
    free(scores);
  }
  return status;
}

/*
 * Bidirectional (non-causal) form, one sequence of S tokens: every query token
 * attends to all S keys.  Same layouts and return codes as above.
 */
int oracle_gqa_bidirectional(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                             int64_t S, int64_t Hq, int64_t Hkv, int64_t D, float scale_f32,
                             const int64_t* tokens, int64_t ntok,
                             double* o_out, double* lse_out, int threads) {
  if (!q || !k || !v || !o_out || !lse_out || (ntok > 0 && !tokens)) return -1;
  if (S < 1 || Hq < 1 || Hkv < 1 || D < 1 || Hq % Hkv != 0) return -2;
  for (int64_t t = 0; t < ntok; ++t)
    if (tokens[t] < 0 || tokens[t] >= S) return -4;

  const int64_t G = Hq / Hkv;
  const double scale = (double)scale_f32;
  const int64_t n_items = ntok * Hkv;
  int status = 0;

#ifdef _OPENMP
  if (threads > 0) omp_set_num_threads(threads);
#else
  (void)threads;
#endif

#pragma omp parallel
  {
    double* scores = (double*)malloc(sizeof(double) * (size_t)(G * S + 3 * G + G * D + D));
    if (!scores) {
#pragma omp atomic write
      status = -5;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t item = 0; item < n_items; ++item) {
      if (!scores) continue;
      const int64_t ti = item / Hkv;
      const int64_t g = item % Hkv;
      const int64_t pos = tokens[ti];
      const int64_t h0 = g * G;
      attend_group(q + (pos * Hq + h0) * D, G, k, v, Hkv * D, g, D, scale, 0, S - 1,
                   scores + 3 * G + G * D + D, scores, scores + G, scores + G + G * D,
                   scores + 2 * G + G * D, scores + 3 * G + G * D, o_out + (ti * Hq + h0) * D, D,
                   lse_out + h0 * ntok + ti, ntok);
    }
    free(scores);
  }
  return status;
}

/*
 * Q/K prologue: x [S, H, D] bf16 bits -> out [S, H, D] doubles.
 * weight: D bf16 bits of the norm weight, or NULL for no norm.  rope: 0 or 1.
 * positions: S int64 positions, or NULL for p = token index.  D must be even when
 * rope is set.  Returns 0 or a negative code for invalid arguments.
 */
int oracle_qk_norm_rope(const uint16_t* x, int64_t S, int64_t H, int64_t D,
                        const uint16_t* weight, double eps, int rope, double theta,
                        const int64_t* positions, double* out) {
  if (!x || !out) return -1;
  if (S < 0 || H < 1 || D < 1 || (rope && (D % 2 != 0 || !(theta > 0.0)))) return -2;
  if (weight && !(eps >= 0.0)) return -2;
  const int64_t half = D / 2;
#pragma omp parallel for schedule(static)
  for (int64_t row = 0; row < S * H; ++row) {
    const int64_t t = row / H;
    const uint16_t* xr = x + row * D;
    double* o = out + row * D;
    for (int64_t d = 0; d < D; ++d) o[d] = bf16_bits_to_double(xr[d]);
    if (weight) {
      double ss = 0.0;
      for (int64_t d = 0; d < D; ++d) ss += o[d] * o[d];
      const double inv = 1.0 / sqrt(ss / (double)D + eps);
      for (int64_t d = 0; d < D; ++d) o[d] = o[d] * inv * bf16_bits_to_double(weight[d]);
    }
    if (rope) {
      const double p = positions ? (double)positions[t] : (double)t;
      for (int64_t i = 0; i < half; ++i) {
        const double a = p * pow(theta, -2.0 * (double)i / (double)D);
        const double c = cos(a), sn = sin(a);
        const double lo = o[i], hi = o[i + half];
        o[i] = lo * c - hi * sn;
        o[i + half] = hi * c + lo * sn;
      }
    }
  }
  return 0;
}

/* Threads an OpenMP region would use with the given request (<= 0: default). */
int oracle_threads(int threads) {
#ifdef _OPENMP
  if (threads > 0) return threads;
  return omp_get_max_threads();
#else
  (void)threads;
  return 1;
#endif
}
