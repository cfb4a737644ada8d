/*
 * Seeded synthetic inputs for the Key-Key Semantic Affinity workloads.
 *
 * This module only draws random numbers and lays them out in memory: paged
 * bf16 key pools, block tables, permutations, topic assignments and fp32
 * block-vector tables.  It holds none of the method's arithmetic (no pooling,
 * no variance, no affinity, no selection), so both the oracle side and the
 * HIP side of the tests can consume its output without sharing any code of
 * the method.
 *
 * Random numbers are counter based: value i of stream k is
 * SplitMix64(k + (i + 1) * golden), the SplitMix64 output function of
 * Steele, Lea and Flood ("Fast splittable pseudorandom number generators",
 * OOPSLA 2014).  Uniforms take the top 53 bits; normals use the Box-Muller
 * transform (Box and Muller 1958), one (cos, sin) pair per two uniforms.
 * Any element can be regenerated on its own from (seed, stream tag, index).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL
#define TWO_PI 6.283185307179586476925286766559

static inline uint64_t sm64_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

/* Stream key for (seed, tag): distinct tags give unrelated streams. */
uint64_t synth_stream(uint64_t seed, uint64_t tag) {
  return sm64_mix(sm64_mix(seed + GOLDEN) ^ (tag * 0xD1B54A32D192ED03ULL + 0x8CB92BA72F3D8DD7ULL));
}

static inline uint64_t ctr_u64(uint64_t stream, uint64_t i) {
  return sm64_mix(stream + (i + 1) * GOLDEN);
}

/* Uniform on the open interval (0, 1). */
static inline double ctr_unif(uint64_t stream, uint64_t i) {
  return ((double)(ctr_u64(stream, i) >> 11) + 0.5) * 0x1.0p-53;
}

/* Standard normal pair number `pair` of a stream: elements 2*pair, 2*pair+1. */
static inline void ctr_normal_pair(uint64_t stream, uint64_t pair, double* z0, double* z1) {
  double u1 = ctr_unif(stream, 2 * pair);
  double u2 = ctr_unif(stream, 2 * pair + 1);
  double r = sqrt(-2.0 * log(u1));
  double a = TWO_PI * u2;
  *z0 = r * cos(a);
  *z1 = r * sin(a);
}

/* Standard normal element i of a stream. */
static inline double ctr_normal(uint64_t stream, uint64_t i) {
  double z0, z1;
  ctr_normal_pair(stream, i >> 1, &z0, &z1);
  return (i & 1) ? z1 : z0;
}

/* fp32 -> bf16 bit pattern, round to nearest, ties to even. */
static inline uint16_t f32_to_bf16(float f) {
  uint32_t x;
  memcpy(&x, &f, 4);
  if ((x & 0x7F800000u) == 0x7F800000u && (x & 0x007FFFFFu)) return (uint16_t)((x >> 16) | 0x40u);
  x += 0x7FFFu + ((x >> 16) & 1u);
  return (uint16_t)(x >> 16);
}

/* ------------------------------------------------------------------ scalars */

uint64_t synth_u64(uint64_t seed, uint64_t tag, uint64_t i) { return ctr_u64(synth_stream(seed, tag), i); }

double synth_normal(uint64_t seed, uint64_t tag, uint64_t i) { return ctr_normal(synth_stream(seed, tag), i); }

double synth_uniform(uint64_t seed, uint64_t tag, uint64_t i) { return ctr_unif(synth_stream(seed, tag), i); }

void synth_f32_to_bf16(const float* in, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = f32_to_bf16(in[i]);
}

/* Integers uniform on [lo, hi] (inclusive), by 128-bit multiply-high. */
void synth_uniform_int(uint64_t seed, uint64_t tag, int64_t n, int64_t lo, int64_t hi, int64_t* out) {
  uint64_t st = synth_stream(seed, tag);
  uint64_t span = (uint64_t)(hi - lo) + 1;
  for (int64_t i = 0; i < n; ++i) {
    unsigned __int128 m = (unsigned __int128)ctr_u64(st, (uint64_t)i) * span;
    out[i] = lo + (int64_t)(uint64_t)(m >> 64);
  }
}

/* Uniform doubles on (0, 1). */
void synth_uniform_f64(uint64_t seed, uint64_t tag, int64_t n, double* out) {
  uint64_t st = synth_stream(seed, tag);
  for (int64_t i = 0; i < n; ++i) out[i] = ctr_unif(st, (uint64_t)i);
}

/* Normals N(mean, std) as doubles. */
void synth_normal_f64(uint64_t seed, uint64_t tag, int64_t n, double mean, double std, double* out) {
  uint64_t st = synth_stream(seed, tag);
  for (int64_t i = 0; i < n; ++i) out[i] = mean + std * ctr_normal(st, (uint64_t)i);
}

/* Fisher-Yates shuffle of 0..n-1 (Durstenfeld's in-place form). */
void synth_permutation(uint64_t seed, uint64_t tag, int64_t n, int32_t* out) {
  uint64_t st = synth_stream(seed, tag);
  for (int64_t i = 0; i < n; ++i) out[i] = (int32_t)i;
  for (int64_t i = n - 1; i > 0; --i) {
    unsigned __int128 m = (unsigned __int128)ctr_u64(st, (uint64_t)i) * (uint64_t)(i + 1);
    int64_t j = (int64_t)(uint64_t)(m >> 64);
    int32_t t = out[i];
    out[i] = out[j];
    out[j] = t;
  }
}

/* n_vec random unit directions of length dim (normalised Gaussian vectors),
 * rows of `out` [n_vec][dim]. */
void synth_unit_dirs(uint64_t seed, uint64_t tag, int64_t n_vec, int32_t dim, float* out) {
  uint64_t st = synth_stream(seed, tag);
  double* tmp = (double*)malloc(sizeof(double) * (size_t)dim);
  for (int64_t v = 0; v < n_vec; ++v) {
    double ss = 0.0;
    for (int32_t d = 0; d < dim; ++d) {
      tmp[d] = ctr_normal(st, (uint64_t)v * (uint64_t)dim + (uint64_t)d);
      ss += tmp[d] * tmp[d];
    }
    double inv = ss > 0.0 ? 1.0 / sqrt(ss) : 0.0;
    for (int32_t d = 0; d < dim; ++d) out[v * dim + d] = (float)(tmp[d] * inv);
  }
  free(tmp);
}

/* ------------------------------------------------------------------ threads */

typedef void (*range_fn)(void* ctx, int64_t lo, int64_t hi);
typedef struct {
  range_fn fn;
  void* ctx;
  int64_t lo, hi;
} range_job;

static void* range_thread(void* p) {
  range_job* j = (range_job*)p;
  j->fn(j->ctx, j->lo, j->hi);
  return NULL;
}

static void parallel_range(range_fn fn, void* ctx, int64_t n, int n_threads) {
  if (n_threads < 1) n_threads = 1;
  if (n_threads > 256) n_threads = 256;
  if ((int64_t)n_threads > n) n_threads = (int)(n > 0 ? n : 1);
  if (n_threads == 1) {
    fn(ctx, 0, n);
    return;
  }
  pthread_t th[256];
  range_job jobs[256];
  for (int t = 0; t < n_threads; ++t) {
    jobs[t].fn = fn;
    jobs[t].ctx = ctx;
    jobs[t].lo = n * t / n_threads;
    jobs[t].hi = n * (t + 1) / n_threads;
    pthread_create(&th[t], NULL, range_thread, &jobs[t]);
  }
  for (int t = 0; t < n_threads; ++t) pthread_join(th[t], NULL);
}

/* ------------------------------------------------------------------ key pool */

/*
 * Paged key pool.  Element (layer l, physical block p, token slot t, head h,
 * dim d) lives at out[l*sL + p*sB + t*sT + h*sH + d].  Logical block b of the
 * CSR batch sits in physical block block_table[b]; token slot t of logical
 * block i of sequence s is sequence position tau = i*B + t.
 *
 * For tau < gen_len[s] the key is
 *     amp * g * dir[topic][l][h][:] + bias[l][h][:] + noise_std[l*H+h] * n
 * where topic = block_topic[b] (no signal term when it is negative or when
 * block_topic is NULL), g ~ N(1, jitter) per (token, l, h) (g = 1 when
 * jitter == 0), and n is standard normal per element.  Slots with
 * tau >= gen_len[s] are written as zero.  The value is rounded once to bf16.
 * Counter indices use the global token number block_offsets[s]*B + tau.
 */
typedef struct {
  int32_t L, H, D, B;
  int64_t P;
  int64_t sL, sB, sT, sH;
  int32_t S;
  const int32_t* gen_len;
  const int32_t* block_offsets;
  const int32_t* block_table;
  const int32_t* block_topic;
  const float* topic_dir; /* [n_topics][L][H][D] */
  int32_t n_topics;
  float amp;
  float jitter;
  const float* noise_std; /* [L*H] */
  const float* bias;      /* [L][H][D] or NULL */
  uint64_t seed;
} synth_kpool_spec;

typedef struct {
  const synth_kpool_spec* sp;
  uint16_t* out;
  const int32_t* seq_of_block;
  uint64_t st_noise, st_jit;
} kpool_ctx;

static void kpool_range(void* vctx, int64_t lo, int64_t hi) {
  kpool_ctx* c = (kpool_ctx*)vctx;
  const synth_kpool_spec* sp = c->sp;
  const int32_t L = sp->L, H = sp->H, D = sp->D, B = sp->B;
  float* row = (float*)malloc(sizeof(float) * (size_t)D);
  for (int64_t item = lo; item < hi; ++item) {
    int64_t b = item / L;
    int32_t l = (int32_t)(item % L);
    int32_t s = c->seq_of_block[b];
    int64_t i = b - sp->block_offsets[s];
    int64_t p = sp->block_table[b];
    int32_t topic = sp->block_topic ? sp->block_topic[b] : -1;
    for (int32_t t = 0; t < B; ++t) {
      int64_t tau = i * B + t;
      uint64_t g_tok = (uint64_t)sp->block_offsets[s] * (uint64_t)B + (uint64_t)tau;
      for (int32_t h = 0; h < H; ++h) {
        uint16_t* dst = c->out + l * sp->sL + p * sp->sB + t * sp->sT + h * sp->sH;
        if (tau >= sp->gen_len[s]) {
          memset(dst, 0, sizeof(uint16_t) * (size_t)D);
          continue;
        }
        uint64_t lh = ((g_tok * (uint64_t)L + (uint64_t)l) * (uint64_t)H + (uint64_t)h);
        double nstd = sp->noise_std ? sp->noise_std[l * H + h] : 0.0;
        uint64_t base = lh * (uint64_t)D; /* D is even: pairs never straddle rows */
        for (int32_t d = 0; d < D; d += 2) {
          double z0, z1;
          ctr_normal_pair(c->st_noise, (base + (uint64_t)d) >> 1, &z0, &z1);
          row[d] = (float)(nstd * z0);
          row[d + 1] = (float)(nstd * z1);
        }
        if (topic >= 0 && topic < sp->n_topics && sp->amp != 0.0f) {
          double g = 1.0;
          if (sp->jitter != 0.0f) g = 1.0 + (double)sp->jitter * ctr_normal(c->st_jit, lh);
          const float* u = sp->topic_dir + (((int64_t)topic * L + l) * H + h) * D;
          for (int32_t d = 0; d < D; ++d) row[d] = (float)((double)row[d] + (double)sp->amp * g * (double)u[d]);
        }
        if (sp->bias) {
          const float* bv = sp->bias + ((int64_t)l * H + h) * D;
          for (int32_t d = 0; d < D; ++d) row[d] = (float)((double)row[d] + (double)bv[d]);
        }
        for (int32_t d = 0; d < D; ++d) dst[d] = f32_to_bf16(row[d]);
      }
    }
  }
  free(row);
}

int synth_kpool(const synth_kpool_spec* sp, uint16_t* out, int n_threads) {
  if (!sp || !out || sp->D % 2 != 0) return 1;
  int64_t total = sp->block_offsets[sp->S];
  int32_t* sob = (int32_t*)malloc(sizeof(int32_t) * (size_t)(total > 0 ? total : 1));
  for (int32_t s = 0; s < sp->S; ++s)
    for (int64_t b = sp->block_offsets[s]; b < sp->block_offsets[s + 1]; ++b) sob[b] = s;
  kpool_ctx c;
  c.sp = sp;
  c.out = out;
  c.seq_of_block = sob;
  c.st_noise = synth_stream(sp->seed, 0x4E4F495345ULL); /* "NOISE" */
  c.st_jit = synth_stream(sp->seed, 0x4A4954ULL);       /* "JIT" */
  parallel_range(kpool_range, &c, total * sp->L, n_threads);
  free(sob);
  return 0;
}

/* --------------------------------------------------------- block-vector table */

/*
 * Rows of fp32 vectors out[r][:] = amp * dir[topic[r]][:] + std * n for
 * r < n_rows (no signal term when topic[r] < 0); n standard normal with
 * counter index r*D + d of stream (seed, tag).  Used for block-vector tables
 * written directly and for anchors.
 */
typedef struct {
  const int32_t* topic;
  const float* dir;
  int32_t n_topics, D;
  float amp, std;
  uint64_t st;
  float* out;
} rows_ctx;

static void rows_range(void* vctx, int64_t lo, int64_t hi) {
  rows_ctx* c = (rows_ctx*)vctx;
  const int32_t D = c->D;
  for (int64_t r = lo; r < hi; ++r) {
    float* dst = c->out + r * D;
    int32_t tp = c->topic ? c->topic[r] : -1;
    for (int32_t d = 0; d < D; d += 2) {
      double z0, z1;
      ctr_normal_pair(c->st, ((uint64_t)r * (uint64_t)D + (uint64_t)d) >> 1, &z0, &z1);
      double v0 = (double)c->std * z0, v1 = (double)c->std * z1;
      if (tp >= 0 && tp < c->n_topics) {
        v0 += (double)c->amp * (double)c->dir[(int64_t)tp * D + d];
        v1 += (double)c->amp * (double)c->dir[(int64_t)tp * D + d + 1];
      }
      dst[d] = (float)v0;
      dst[d + 1] = (float)v1;
    }
  }
}

int synth_rows(uint64_t seed, uint64_t tag, int64_t n_rows, int32_t D, const int32_t* topic, const float* dir,
               int32_t n_topics, float amp, float std, float* out, int n_threads) {
  if (D % 2 != 0 || !out) return 1;
  rows_ctx c = {topic, dir, n_topics, D, amp, std, synth_stream(seed, tag), out};
  parallel_range(rows_range, &c, n_rows, n_threads);
  return 0;
}
