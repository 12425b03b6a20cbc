/*
 * CPU oracle for the one-pass row statistics of a diffusion-LM denoise step
 * and for the top-K logprobs of converged slots.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may load, call or
 * link this file: only the tests, the smoke check and the benchmark's CPU
 * baseline use it. It shares no code with the HIP library.
 *
 * Source of the semantics: the vLLM API page "diffusion_gemma_sampler"
 * (DiffusionGemma sampler):
 *   - module docstring: for each canvas row, the argmax of the logits divided
 *     by the temperature, a Gumbel-max sample, the softmax entropy and the
 *     softmax;
 *   - sample_row_stats (docstring): row i takes its temperature from
 *     temps[i // canvas_len]; T = 0 means greedy, and for the entropy the
 *     temperature is clamped at 1e-10;
 *   - sample_row_stats_reference: scaled = logits / clamp(T, 1e-10),
 *     Gumbel noise applied only where T > 0, entropy over p > 0 only;
 *   - _lp_topk_kernel docstring: keys order by value, then by lower index;
 *   - stash_converged_logprobs docstring: rows of slots not kept are skipped,
 *     the kept rows are divided by their temperature, the top-k is taken with
 *     ties going to the lower id.
 *
 * Readings where the page leaves a step open (each one is listed with its
 * reason in the design notes of the repository):
 *   - noise: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random
 *     Numbers: As Easy as 1, 2, 3", SC'11) with counter
 *     (col >> 2, 0, lo32(row), hi32(row)) and key (lo32(seed), hi32(seed));
 *     column col takes output word col & 3; u = (w + 0.5) * 2^-32 and
 *     g = -log(-log u), both in double;
 *   - the temperature divide is one IEEE fp32 division; every later
 *     reduction is in double;
 *   - the entropy is log S - sum_c p_c (s_c - m), the identity
 *     H = log Z - sum p * s written relative to the row maximum m;
 *   - probs are rounded to bf16 / fp16 once, to nearest-even, from the double
 *     probability, subnormals kept;
 *   - the top-K logprob of column c is s_c - log Z with the same clamp on T,
 *     evaluated as (s_c - m) - log sum exp(s - m).
 *
 * Plain C99, no fast-math, no FMA contraction; OpenMP only splits rows.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_OK 0
#define OR_ERR_ARG (-1)
#define OR_ERR_NOMEM (-2)

/* ------------------------------------------------------------------------ */
/* Philox4x32-10 (Salmon et al., SC'11): two 32x32->64 multiplies per round,  */
/* Weyl-sequence key schedule, 10 rounds.                                     */
/* ------------------------------------------------------------------------ */
static const uint32_t PHILOX_M0 = 0xD2511F53u;
static const uint32_t PHILOX_M1 = 0xCD9E8D57u;
static const uint32_t PHILOX_W0 = 0x9E3779B9u;
static const uint32_t PHILOX_W1 = 0xBB67AE85u;

void oracle_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2],
                          uint32_t out[4]) {
  uint32_t c[4] = {ctr_in[0], ctr_in[1], ctr_in[2], ctr_in[3]};
  uint32_t k0 = key_in[0], k1 = key_in[1];
  for (int round = 0; round < 10; ++round) {
    if (round > 0) {
      k0 += PHILOX_W0;
      k1 += PHILOX_W1;
    }
    uint64_t p0 = (uint64_t)PHILOX_M0 * (uint64_t)c[0];
    uint64_t p1 = (uint64_t)PHILOX_M1 * (uint64_t)c[2];
    uint32_t n0 = (uint32_t)(p1 >> 32) ^ c[1] ^ k0;
    uint32_t n1 = (uint32_t)p1;
    uint32_t n2 = (uint32_t)(p0 >> 32) ^ c[3] ^ k1;
    uint32_t n3 = (uint32_t)p0;
    c[0] = n0;
    c[1] = n1;
    c[2] = n2;
    c[3] = n3;
  }
  out[0] = c[0];
  out[1] = c[1];
  out[2] = c[2];
  out[3] = c[3];
}

/* The 32-bit word that the noise of (seed, row, col) is drawn from. */
static uint32_t noise_word(uint64_t seed, int64_t row, int64_t col) {
  uint32_t ctr[4], key[2], out[4];
  uint64_t q = (uint64_t)col >> 2;
  ctr[0] = (uint32_t)q;
  ctr[1] = (uint32_t)(q >> 32);
  ctr[2] = (uint32_t)((uint64_t)row);
  ctr[3] = (uint32_t)((uint64_t)row >> 32);
  key[0] = (uint32_t)seed;
  key[1] = (uint32_t)(seed >> 32);
  oracle_philox4x32_10(ctr, key, out);
  return out[col & 3];
}

/* u in (0, 1), then the standard Gumbel variate -log(-log u). */
void oracle_uniform_gumbel(uint32_t w, double *u_out, double *g_out) {
  double u = ((double)w + 0.5) * (1.0 / 4294967296.0);
  *u_out = u;
  *g_out = -log(-log(u));
}

uint32_t oracle_noise_word(uint64_t seed, int64_t row, int64_t col) {
  return noise_word(seed, row, col);
}

/* ------------------------------------------------------------------------ */
/* Temperature rule (sample_row_stats docstring, reference form).           */
/* ------------------------------------------------------------------------ */
static float clamp_temp(float t) {
  const float lo = 1e-10f;
  return (t > lo) ? t : lo; /* clamp(min=1e-10) of a non-NaN fp32 value */
}

static int is_greedy(float t) { return !(t > 0.0f); }

/* s[c] = x[c] / Tc, one IEEE fp32 division per element. */
void oracle_scale_row(const float *x, int64_t n, float t, float *s) {
  float tc = clamp_temp(t);
  for (int64_t c = 0; c < n; ++c) s[c] = x[c] / tc;
}

/* ------------------------------------------------------------------------ */
/* Round-to-nearest-even from double into bf16 / fp16 bit patterns.          */
/* Only p in [0, 1] is ever rounded here (probabilities).                    */
/* ------------------------------------------------------------------------ */
/* Round v >= 0 to a binary format with `mant` stored mantissa bits and     */
/* smallest normal exponent emin (value 2^emin); subnormals keep the         */
/* spacing 2^(emin - mant).                                                  */
static double round_to_format(double v, int mant, int emin) {
  if (v == 0.0) return 0.0;
  int e2;
  (void)frexp(v, &e2);          /* v = f * 2^e2, f in [0.5, 1) */
  int e = e2 - 1;               /* v in [2^e, 2^(e+1)) */
  if (e < emin) e = emin;       /* subnormal range shares the smallest quantum */
  double quantum = ldexp(1.0, e - mant);
  double r = nearbyint(v / quantum); /* default rounding mode: ties to even */
  return r * quantum;
}

uint16_t oracle_bf16_bits(double p) {
  double v = round_to_format(p, 7, -126);
  float f = (float)v; /* exact: every bf16 value is an fp32 value */
  uint32_t b;
  memcpy(&b, &f, sizeof b);
  return (uint16_t)(b >> 16);
}

uint16_t oracle_fp16_bits(double p) {
  double v = round_to_format(p, 10, -14);
  if (v == 0.0) return 0;
  int e2;
  double f = frexp(v, &e2); /* v = f * 2^e2 */
  int e = e2 - 1;
  if (e < -14) { /* subnormal: v = k * 2^-24 */
    return (uint16_t)(uint32_t)ldexp(v, 24);
  }
  uint32_t mant = (uint32_t)((ldexp(f, 1) - 1.0) * 1024.0);
  return (uint16_t)(((uint32_t)(e + 15) << 10) | mant);
}

/* ------------------------------------------------------------------------ */
/* Row statistics.                                                            */
/* ------------------------------------------------------------------------ */
typedef struct {
  int64_t argmax;
  int64_t sample;
  double entropy;      /* log S - sum p (s - m) */
  double entropy_plogp;/* -sum_{p>0} p log p, the reference's form */
  double gap;          /* best z - second z over columns; +inf if greedy */
} row_result;

static int one_row(const float *x, int64_t vocab, int64_t row, float t,
                   uint64_t seed, int probs_dtype, float *s, uint16_t *probs,
                   row_result *res) {
  float tc = clamp_temp(t);
  for (int64_t c = 0; c < vocab; ++c) s[c] = x[c] / tc;

  /* max and the lowest index attaining it (IEEE compare: -0 == +0) */
  float m = s[0];
  int64_t am = 0;
  for (int64_t c = 1; c < vocab; ++c) {
    if (s[c] > m) {
      m = s[c];
      am = c;
    }
  }
  res->argmax = am;

  /* S = sum exp(s - m) in double */
  double md = (double)m;
  double S = 0.0;
  for (int64_t c = 0; c < vocab; ++c) S += exp((double)s[c] - md);
  double logS = log(S);

  /* entropy, both forms, over p > 0 only (the -inf columns drop out) */
  double sum_pd = 0.0, sum_plogp = 0.0;
  for (int64_t c = 0; c < vocab; ++c) {
    double d = (double)s[c] - md;
    double p = exp(d) / S;
    if (p > 0.0) {
      sum_pd += p * d;
      sum_plogp += p * (d - logS);
    }
    if (probs) {
      probs[c] = (probs_dtype == 2) ? oracle_fp16_bits(p) : oracle_bf16_bits(p);
    }
  }
  res->entropy = logS - sum_pd;
  res->entropy_plogp = -sum_plogp;

  /* Gumbel-max sample; greedy rows take the argmax (noise times 0). */
  if (is_greedy(t)) {
    res->sample = am;
    res->gap = INFINITY;
    return OR_OK;
  }
  double best = -INFINITY, second = -INFINITY;
  int64_t best_c = -1;
  uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  uint32_t words[4];
  for (int64_t c = 0; c < vocab; ++c) {
    if ((c & 3) == 0) {
      uint64_t q = (uint64_t)c >> 2;
      uint32_t ctr[4] = {(uint32_t)q, (uint32_t)(q >> 32), (uint32_t)(uint64_t)row,
                         (uint32_t)((uint64_t)row >> 32)};
      oracle_philox4x32_10(ctr, key, words);
    }
    double u, g;
    oracle_uniform_gumbel(words[c & 3], &u, &g);
    double z = (double)s[c] + g;
    if (best_c < 0 || z > best) {
      second = best;
      best = z;
      best_c = c;
    } else if (z > second || z == best) {
      /* an exact tie keeps the lower index as winner; it is also the gap 0 */
      second = z;
    }
  }
  res->sample = best_c;
  res->gap = best - second;
  return OR_OK;
}

static int nthreads_used = 1;

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/*
 * Row statistics of the selected rows.
 *   x        host fp32, n_sel rows with stride ld (x[i*ld + c] is row_ids[i])
 *   row_ids  global row index of each selected row (temperature slot and noise)
 *   temps    per-slot fp32 temperatures, n_temps of them
 *   probs    NULL or n_sel*vocab uint16 (bf16 if probs_dtype==1, fp16 if 2)
 * Outputs are indexed by the selection index i.
 */
int oracle_rowstats(const float *x, int64_t ld, int64_t n_sel,
                    const int64_t *row_ids, int64_t vocab, const float *temps,
                    int64_t n_temps, int64_t canvas_len, uint64_t seed,
                    int probs_dtype, int64_t *argmax, int64_t *sample,
                    double *entropy, double *entropy_plogp, double *gap,
                    uint16_t *probs) {
  if (!x || !row_ids || !temps || !argmax || !sample || !entropy || !gap)
    return OR_ERR_ARG;
  if (n_sel < 0 || vocab < 1 || ld < vocab || canvas_len < 1) return OR_ERR_ARG;
  if (probs && probs_dtype != 1 && probs_dtype != 2) return OR_ERR_ARG;
  for (int64_t i = 0; i < n_sel; ++i) {
    if (row_ids[i] < 0 || row_ids[i] / canvas_len >= n_temps) return OR_ERR_ARG;
  }
  int err = OR_OK;
#pragma omp parallel
  {
    float *s = (float *)malloc(sizeof(float) * (size_t)vocab);
    if (!s) {
#pragma omp atomic write
      err = OR_ERR_NOMEM;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t i = 0; i < n_sel; ++i) {
      if (!s) continue;
      int64_t row = row_ids[i];
      float t = temps[row / canvas_len];
      row_result res;
      one_row(x + i * ld, vocab, row, t, seed, probs_dtype, s,
              probs ? probs + i * vocab : NULL, &res);
      argmax[i] = res.argmax;
      sample[i] = res.sample;
      entropy[i] = res.entropy;
      if (entropy_plogp) entropy_plogp[i] = res.entropy_plogp;
      gap[i] = res.gap;
    }
    free(s);
  }
  nthreads_used = oracle_num_threads();
  return err;
}

/* ------------------------------------------------------------------------ */
/* Top-K logprobs of kept rows: full sort by (value desc, index asc).        */
/* ------------------------------------------------------------------------ */
typedef struct {
  float s;
  int32_t c;
} entry;

static int cmp_entry(const void *a, const void *b) {
  const entry *x = (const entry *)a, *y = (const entry *)b;
  if (x->s > y->s) return -1;
  if (x->s < y->s) return 1;
  /* equal values (including -0 vs +0): the lower index ranks first */
  return (x->c < y->c) ? -1 : (x->c > y->c);
}

/*
 * For every selected row whose slot is kept: out_idx[i*K + k] is the column
 * of rank k and out_vals[i*K + k] = s - log Z at that column. Rows of slots
 * not kept are left untouched.
 */
int oracle_topk_logprobs(const float *x, int64_t ld, int64_t n_sel,
                         const int64_t *row_ids, int64_t vocab,
                         const float *temps, int64_t n_temps, int64_t canvas_len,
                         const uint8_t *keep_mask, int32_t K, float *out_vals,
                         int64_t *out_idx) {
  if (!x || !row_ids || !temps || !keep_mask || !out_vals || !out_idx)
    return OR_ERR_ARG;
  if (n_sel < 0 || vocab < 1 || ld < vocab || canvas_len < 1) return OR_ERR_ARG;
  if (K < 1 || K > vocab) return OR_ERR_ARG;
  for (int64_t i = 0; i < n_sel; ++i) {
    if (row_ids[i] < 0 || row_ids[i] / canvas_len >= n_temps) return OR_ERR_ARG;
  }
  int err = OR_OK;
#pragma omp parallel
  {
    entry *e = (entry *)malloc(sizeof(entry) * (size_t)vocab);
    if (!e) {
#pragma omp atomic write
      err = OR_ERR_NOMEM;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t i = 0; i < n_sel; ++i) {
      if (!e) continue;
      int64_t row = row_ids[i];
      int64_t slot = row / canvas_len;
      if (!keep_mask[slot]) continue;
      float tc = clamp_temp(temps[slot]);
      const float *xr = x + i * ld;
      float m = -INFINITY;
      for (int64_t c = 0; c < vocab; ++c) {
        e[c].s = xr[c] / tc;
        e[c].c = (int32_t)c;
        if (c == 0 || e[c].s > m) m = e[c].s;
      }
      double S = 0.0;
      for (int64_t c = 0; c < vocab; ++c) S += exp((double)e[c].s - (double)m);
      /* s - log Z written as (s - m) - log S: s - m is exact in double, so
         the result keeps its precision when |m| is large (T clamped to
         1e-10 scales the logits by 1e10) */
      double logS = log(S);
      qsort(e, (size_t)vocab, sizeof(entry), cmp_entry);
      for (int32_t k = 0; k < K; ++k) {
        out_idx[i * K + k] = e[k].c;
        out_vals[i * K + k] = (float)(((double)e[k].s - (double)m) - logS);
      }
    }
    free(e);
  }
  nthreads_used = oracle_num_threads();
  return err;
}

int oracle_last_threads(void) { return nthreads_used; }
