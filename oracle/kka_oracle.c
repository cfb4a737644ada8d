/*
 * CPU oracle for Key-Key Semantic Affinity (KKA) block selection.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this file's library.  The GPU
 * library never calls it and shares no code, header or constant with it.
 *
 * Plain, single-threaded C; every sum is taken in double precision from the
 * exact bf16/fp32 inputs and each output is rounded once to fp32.  The
 * method is described on the page "Key-Key Semantic Affinity: Key vectors
 * replace attention scores for KV-cache importance" (10100.com); each
 * function names the section it follows.  Where that page is silent or its
 * formulas were lost in extraction, the readings are:
 *   - affinity = (1 + cos(v_anchor, v_b)) / 2, clamped to [0, 1], with
 *     cos = 0 when either vector has zero norm;
 *   - head weight = temporal variance of that (layer, KV head)'s keys
 *     (per-dimension population variance over the sequence's tokens,
 *     averaged over dimensions), normalised to sum 1 (uniform when every
 *     variance is 0), rounded to fp32 before use;
 *   - chunk vector = mean of its present page vectors, grid vector = mean of
 *     its present chunk vectors;
 *   - children of an unselected parent score exactly +0 and stay eligible;
 *     every ordering is (score descending, index ascending).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  const uint16_t* k; /* bf16 bit patterns */
  int32_t L, H, D, B;
  int64_t P;
  int64_t sL, sB, sT, sH; /* element strides; dimension stride is 1 */
} oracle_kpool;

static double bf16_value(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

static const uint16_t* key_row(const oracle_kpool* kp, int32_t l, int64_t p, int32_t t, int32_t h) {
  return kp->k + (int64_t)l * kp->sL + p * kp->sB + (int64_t)t * kp->sT + (int64_t)h * kp->sH;
}

static int kpool_ok(const oracle_kpool* kp) {
  return kp && kp->k && kp->L > 0 && kp->H > 0 && kp->D > 0 && kp->B > 0 && kp->P > 0;
}

/*
 * Head weights for one sequence (section 3.3 "experimental validation":
 * weight each attention head by its variance; section 6.1 repeats that
 * low-variance heads behave like positional bias).  A head is one
 * (layer, KV head) pair.  For each head and dimension d, the population
 * variance over the sequence's T tokens is taken with the two-pass formula
 * (mean first, then mean squared deviation); the head's variance is the
 * average over d.  Weights are variances over their sum, rounded to fp32.
 * table: physical block of each logical block of the sequence.
 */
int oracle_head_weights(const oracle_kpool* kp, const int32_t* table, int32_t T, float* w_out) {
  if (!kpool_ok(kp) || !table || !w_out || T < 0) return 1;
  const int32_t L = kp->L, H = kp->H, D = kp->D, B = kp->B;
  double* mean = (double*)malloc(sizeof(double) * (size_t)D);
  double* sq = (double*)malloc(sizeof(double) * (size_t)D);
  double* var = (double*)malloc(sizeof(double) * (size_t)L * (size_t)H);
  double total = 0.0;
  for (int32_t l = 0; l < L; ++l) {
    for (int32_t h = 0; h < H; ++h) {
      for (int32_t d = 0; d < D; ++d) mean[d] = 0.0;
      for (int32_t tau = 0; tau < T; ++tau) {
        const uint16_t* r = key_row(kp, l, table[tau / B], tau % B, h);
        for (int32_t d = 0; d < D; ++d) mean[d] += bf16_value(r[d]);
      }
      for (int32_t d = 0; d < D; ++d) mean[d] = T > 0 ? mean[d] / (double)T : 0.0;
      for (int32_t d = 0; d < D; ++d) sq[d] = 0.0;
      for (int32_t tau = 0; tau < T; ++tau) {
        const uint16_t* r = key_row(kp, l, table[tau / B], tau % B, h);
        for (int32_t d = 0; d < D; ++d) {
          double x = bf16_value(r[d]) - mean[d];
          sq[d] += x * x;
        }
      }
      double acc = 0.0;
      for (int32_t d = 0; d < D; ++d) acc += T > 0 ? sq[d] / (double)T : 0.0;
      var[l * H + h] = acc / (double)D;
      total += var[l * H + h];
    }
  }
  for (int32_t i = 0; i < L * H; ++i)
    w_out[i] = total > 0.0 ? (float)(var[i] / total) : (float)(1.0 / (double)(L * H));
  free(mean);
  free(sq);
  free(var);
  return 0;
}

/*
 * Mean-pool of keys over a set of (block, slot) token positions, all layers
 * and all KV heads (section 2.2 step 1 and section 5.2 step 3: mean-pool
 * over every token, KV head and layer into one head_dim vector).
 * Tokens are given as physical block `phys[i]` and slot `slot[i]`,
 * i < n_tok.  With weights w (fp32, [L*H]) the result is
 * sum_{l,h} w[l*H+h] * mean_t K[l][.][t][h][:]; without, the plain mean
 * over all n_tok * L * H key vectors.  Empty token set -> zero vector.
 */
static int pool_tokens(const oracle_kpool* kp, const int64_t* phys, const int32_t* slot, int32_t n_tok,
                       const float* w, float* out) {
  const int32_t L = kp->L, H = kp->H, D = kp->D;
  double* acc = (double*)calloc((size_t)D, sizeof(double));
  double* head = (double*)malloc(sizeof(double) * (size_t)D);
  if (n_tok > 0) {
    for (int32_t l = 0; l < L; ++l) {
      for (int32_t h = 0; h < H; ++h) {
        for (int32_t d = 0; d < D; ++d) head[d] = 0.0;
        for (int32_t i = 0; i < n_tok; ++i) {
          const uint16_t* r = key_row(kp, l, phys[i], slot[i], h);
          for (int32_t d = 0; d < D; ++d) head[d] += bf16_value(r[d]);
        }
        if (w) {
          double wl = (double)w[l * H + h];
          for (int32_t d = 0; d < D; ++d) acc[d] += wl * (head[d] / (double)n_tok);
        } else {
          for (int32_t d = 0; d < D; ++d) acc[d] += head[d];
        }
      }
    }
    if (!w)
      for (int32_t d = 0; d < D; ++d) acc[d] /= (double)n_tok * (double)L * (double)H;
  }
  for (int32_t d = 0; d < D; ++d) out[d] = (float)acc[d];
  free(acc);
  free(head);
  return 0;
}

/*
 * Block representation v_b (section 2.2 step 1; section 5.2 step 2: one
 * head_dim float vector per block, computed when the block is written).
 * Pools the first n_valid token slots of physical block `phys`.
 */
int oracle_pool_block(const oracle_kpool* kp, int64_t phys, int32_t n_valid, const float* w, float* out) {
  if (!kpool_ok(kp) || !out || phys < 0 || phys >= kp->P || n_valid < 0 || n_valid > kp->B) return 1;
  int64_t* ph = (int64_t*)malloc(sizeof(int64_t) * (size_t)(kp->B > 0 ? kp->B : 1));
  int32_t* sl = (int32_t*)malloc(sizeof(int32_t) * (size_t)(kp->B > 0 ? kp->B : 1));
  for (int32_t t = 0; t < n_valid; ++t) {
    ph[t] = phys;
    sl[t] = t;
  }
  int rc = pool_tokens(kp, ph, sl, n_valid, w, out);
  free(ph);
  free(sl);
  return rc;
}

/*
 * Query anchor v_anchor (section 2.2 step 2; section 5.2 step 1): the same
 * pooling over the sequence's last min(W, T) tokens, which may span two
 * or more blocks.  table: physical block of each logical block.
 */
int oracle_pool_anchor(const oracle_kpool* kp, const int32_t* table, int32_t T, int32_t W, const float* w,
                       float* out) {
  if (!kpool_ok(kp) || !table || !out || T < 0 || W < 0) return 1;
  int32_t n = W < T ? W : T;
  int64_t* ph = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n > 0 ? n : 1));
  int32_t* sl = (int32_t*)malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1));
  for (int32_t i = 0; i < n; ++i) {
    int32_t tau = T - n + i;
    ph[i] = table[tau / kp->B];
    sl[i] = tau % kp->B;
  }
  int rc = pool_tokens(kp, ph, sl, n, w, out);
  free(ph);
  free(sl);
  return rc;
}

/* Mean of rows [lo, hi) of an fp32 [n][D] table, in double, rounded once. */
static void mean_rows(const float* rows, int64_t lo, int64_t hi, int32_t D, float* out) {
  for (int32_t d = 0; d < D; ++d) {
    double s = 0.0;
    for (int64_t r = lo; r < hi; ++r) s += (double)rows[r * D + d];
    out[d] = hi > lo ? (float)(s / (double)(hi - lo)) : 0.0f;
  }
}

/*
 * Grid -> Chunk -> Page representations (section 5.1): a chunk is the mean
 * of its (at most ppc) page vectors, a grid is the mean of its (at most cpg)
 * chunk vectors.  n_c = ceil(n_p / ppc), n_g = ceil(n_c / cpg).
 */
int oracle_build_levels(const float* pages, int32_t n_p, int32_t D, int32_t ppc, int32_t cpg, float* chunks,
                        float* grids) {
  if (!pages || n_p < 0 || D <= 0 || ppc <= 0 || cpg <= 0) return 1;
  int32_t n_c = (n_p + ppc - 1) / ppc;
  int32_t n_g = (n_c + cpg - 1) / cpg;
  if ((n_c && !chunks) || (n_g && !grids)) return 1;
  for (int32_t j = 0; j < n_c; ++j) {
    int64_t hi = (int64_t)(j + 1) * ppc;
    mean_rows(pages, (int64_t)j * ppc, hi < n_p ? hi : n_p, D, chunks + (int64_t)j * D);
  }
  for (int32_t g = 0; g < n_g; ++g) {
    int64_t hi = (int64_t)(g + 1) * cpg;
    mean_rows(chunks, (int64_t)g * cpg, hi < n_c ? hi : n_c, D, grids + (int64_t)g * D);
  }
  return 0;
}

/*
 * Semantic affinity (section 2.2 step 3, section 3.2, section 5.2 step 3):
 * cosine of v_anchor and each row, mapped to [0, 1] as (1 + cos) / 2.
 */
int oracle_affinity(const float* rows, int64_t n, int32_t D, const float* anchor, float* aff) {
  if ((n > 0 && (!rows || !aff)) || !anchor || D <= 0) return 1;
  double na = 0.0;
  for (int32_t d = 0; d < D; ++d) na += (double)anchor[d] * (double)anchor[d];
  for (int64_t r = 0; r < n; ++r) {
    double dot = 0.0, nr = 0.0;
    for (int32_t d = 0; d < D; ++d) {
      double x = (double)rows[r * D + d];
      dot += x * (double)anchor[d];
      nr += x * x;
    }
    double c = (nr > 0.0 && na > 0.0) ? dot / (sqrt(nr) * sqrt(na)) : 0.0;
    double a = 0.5 * (1.0 + c);
    if (!(a > 0.0)) a = 0.0;
    if (a > 1.0) a = 1.0;
    float f = (float)a;
    aff[r] = f == 0.0f ? 0.0f : f;
  }
  return 0;
}

typedef struct {
  float score;
  int32_t idx;
} scored;

static int by_score_then_index(const void* a, const void* b) {
  const scored* x = (const scored*)a;
  const scored* y = (const scored*)b;
  if (x->score > y->score) return -1;
  if (x->score < y->score) return 1;
  return (x->idx > y->idx) - (x->idx < y->idx);
}

/* Sort (score, index) pairs by score descending, index ascending; keep k. */
static int32_t top_k(const float* score, int32_t n, int32_t k, int32_t* idx_out, float* score_out) {
  scored* v = (scored*)malloc(sizeof(scored) * (size_t)(n > 0 ? n : 1));
  for (int32_t i = 0; i < n; ++i) {
    v[i].score = score[i];
    v[i].idx = i;
  }
  qsort(v, (size_t)n, sizeof(scored), by_score_then_index);
  int32_t ke = k < n ? k : n;
  if (ke < 0) ke = 0;
  for (int32_t i = 0; i < ke; ++i) {
    idx_out[i] = v[i].idx;
    if (score_out) score_out[i] = v[i].score;
  }
  free(v);
  return ke;
}

/*
 * Top-K block selection (section 5.2 step 4) through the Grid -> Chunk ->
 * Page hierarchy of section 5.1: all levels are scored, the top k_g grids
 * are kept, a chunk's score is its affinity when its grid was kept and 0
 * otherwise, the top k_c chunks are kept, and a page's score is its affinity
 * when its chunk was kept and 0 otherwise.  The result is the top k_p pages
 * by (score descending, index ascending), with their (masked) scores.
 * Flat mode (hierarchical == 0) takes the top k_p pages directly.
 * Writes min(k_p, n_p) entries and returns that count in *count_out.
 */
int oracle_select(const float* aff_pages, const float* aff_chunks, const float* aff_grids, int32_t n_p, int32_t ppc,
                  int32_t cpg, int32_t hierarchical, int32_t k_g, int32_t k_c, int32_t k_p, int32_t* idx_out,
                  float* score_out, int32_t* count_out) {
  if (n_p < 0 || (n_p > 0 && !aff_pages) || !count_out || k_p < 0 || (k_p > 0 && !idx_out)) return 1;
  if (!hierarchical) {
    *count_out = top_k(aff_pages, n_p, k_p, idx_out, score_out);
    return 0;
  }
  if (ppc <= 0 || cpg <= 0 || k_g < 0 || k_c < 0) return 1;
  int32_t n_c = (n_p + ppc - 1) / ppc;
  int32_t n_g = (n_c + cpg - 1) / cpg;
  if ((n_c && !aff_chunks) || (n_g && !aff_grids)) return 1;
  char* grid_kept = (char*)calloc((size_t)(n_g > 0 ? n_g : 1), 1);
  char* chunk_kept = (char*)calloc((size_t)(n_c > 0 ? n_c : 1), 1);
  int32_t* tmp = (int32_t*)malloc(sizeof(int32_t) * (size_t)(n_p + n_c + n_g + 1));
  float* sc = (float*)malloc(sizeof(float) * (size_t)(n_p + n_c + 1));

  int32_t kg = top_k(aff_grids, n_g, k_g, tmp, NULL);
  for (int32_t i = 0; i < kg; ++i) grid_kept[tmp[i]] = 1;

  for (int32_t j = 0; j < n_c; ++j) sc[j] = grid_kept[j / cpg] ? aff_chunks[j] : 0.0f;
  int32_t kc = top_k(sc, n_c, k_c, tmp, NULL);
  for (int32_t i = 0; i < kc; ++i) chunk_kept[tmp[i]] = 1;

  for (int32_t i = 0; i < n_p; ++i) sc[i] = chunk_kept[i / ppc] ? aff_pages[i] : 0.0f;
  *count_out = top_k(sc, n_p, k_p, idx_out, score_out);

  free(grid_kept);
  free(chunk_kept);
  free(tmp);
  free(sc);
  return 0;
}

/*
 * Stability score (section 5.3 "stability filtering"): over the last W
 * decode steps, the fraction of steps in which a block's affinity was high.
 * The page gives the window W (usually 20), the per-step threshold theta
 * (usually 0.5) and two worked values; its formula was lost in extraction.
 * Readings: a step is high when aff > theta (strict); a step before the
 * first one, or before the block existed (the caller passes an affinity at
 * or below theta for it), is not high; the score is count / W from the
 * first step on (fp64 division rounded once to fp32).
 * aff_hist: [n_steps][n] affinities of n blocks, oldest step first.
 * bits_out (optional, W <= 32): the same window as a word, bit i set when
 * the step i steps before the newest was high.
 */
int oracle_stability(const float* aff_hist, int32_t n_steps, int64_t n, int32_t W, float theta, float* score_out,
                     uint32_t* bits_out) {
  if (n_steps < 0 || n < 0 || W < 1 || (bits_out && W > 32) || (n > 0 && (!score_out || (n_steps > 0 && !aff_hist))))
    return 1;
  int32_t first = n_steps > W ? n_steps - W : 0; /* oldest step still in the window */
  for (int64_t b = 0; b < n; ++b) {
    int32_t count = 0;
    uint32_t bits = 0u;
    for (int32_t t = first; t < n_steps; ++t) {
      int high = (double)aff_hist[(int64_t)t * n + b] > (double)theta;
      count += high;
      if (high) bits |= 1u << (n_steps - 1 - t);
    }
    score_out[b] = (float)((double)count / (double)W);
    if (bits_out) bits_out[b] = bits;
  }
  return 0;
}

/*
 * Attention mass per block for one decode query (section 3.3 "experimental
 * validation": the reference selection is the top-K blocks by real
 * attention, QK^T averaged over every layer and head).  Readings: the
 * attention of query head hq in layer l is softmax over the sequence's T
 * tokens of scale * (q[l][hq] . k[l][t][h]) with KV head h = hq / (Hq / H)
 * (consecutive query heads share a KV head); the probabilities are averaged
 * over the L * Hq (layer, query head) pairs and summed over each block's
 * tokens.  Softmax is taken with the maximum subtracted, in double.
 * q: [L][Hq][D] fp32.  out: ceil(T / B) block scores (fp32, rounded once).
 */
int oracle_attention_blocks(const oracle_kpool* kp, const int32_t* table, int32_t T, int32_t Hq, const float* q,
                            double scale, float* out) {
  if (!kpool_ok(kp) || T < 0 || Hq < kp->H || Hq % kp->H != 0 || !q || (T > 0 && (!table || !out))) return 1;
  const int32_t G = Hq / kp->H;
  const int32_t nb = (T + kp->B - 1) / kp->B;
  double* logit = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
  double* acc = (double*)calloc((size_t)(nb > 0 ? nb : 1), sizeof(double));
  for (int32_t l = 0; l < kp->L; ++l) {
    for (int32_t hq = 0; hq < Hq; ++hq) {
      const int32_t h = hq / G;
      const float* qv = q + ((int64_t)l * Hq + hq) * kp->D;
      double mx = -INFINITY;
      for (int32_t t = 0; t < T; ++t) {
        const uint16_t* kr = key_row(kp, l, table[t / kp->B], t % kp->B, h);
        double dot = 0.0;
        for (int32_t d = 0; d < kp->D; ++d) dot += (double)qv[d] * bf16_value(kr[d]);
        logit[t] = scale * dot;
        if (logit[t] > mx) mx = logit[t];
      }
      double z = 0.0;
      for (int32_t t = 0; t < T; ++t) z += exp(logit[t] - mx);
      for (int32_t t = 0; t < T; ++t) acc[t / kp->B] += exp(logit[t] - mx) / z;
    }
  }
  for (int32_t b = 0; b < nb; ++b) out[b] = (float)(acc[b] / ((double)kp->L * Hq));
  free(logit);
  free(acc);
  return 0;
}
