/*
 * Seeded synthetic inputs for long-context GQA decode attention.
 *
 * This module only draws random numbers and lays them out; it holds none of
 * the attention, quantisation or token-selection arithmetic.  Both the CPU
 * oracle's tests and the GPU tests/bench read their inputs from here.
 *
 * Generator: splitmix64 (Steele, Lea and Flood, "Fast splittable pseudorandom
 * number generators", OOPSLA 2014) used as a counter-based stream:
 *   key(seed, tensor) = mix(mix(seed) ^ (tensor * GOLDEN + 1))
 *   word(i)           = mix(key + (i + 1) * GOLDEN)
 * uniform(i) = ((word(i) >> 11) + 1) * 2^-53, in (0, 1].
 * Normals by Box-Muller (Box and Muller 1958) on the pair (2p, 2p+1):
 *   r = sqrt(-2 ln u0), z(2p) = r cos(2 pi u1), z(2p+1) = r sin(2 pi u1).
 * fp64 -> fp32 (round to nearest even) -> bf16 (round to nearest even).
 *
 * The counter of K/V element (b, kh, t, d) is ((b*KH + kh) << 40) + t*D + d,
 * so a value does not depend on the memory layout it is written into.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

/* The public splitmix64 step: state += gamma; return mix(state). */
uint64_t synth_splitmix64_next(uint64_t *state) {
  *state += GOLDEN;
  return mix64(*state);
}

uint64_t synth_key(uint64_t seed, uint32_t tensor) {
  return mix64(mix64(seed) ^ ((uint64_t)tensor * GOLDEN + 1ULL));
}

static inline uint64_t word_at(uint64_t key, uint64_t i) { return mix64(key + (i + 1ULL) * GOLDEN); }

static inline double uniform_at(uint64_t key, uint64_t i) {
  return (double)((word_at(key, i) >> 11) + 1ULL) * (1.0 / 9007199254740992.0);
}

double synth_uniform(uint64_t seed, uint32_t tensor, uint64_t i) {
  return uniform_at(synth_key(seed, tensor), i);
}

uint64_t synth_word(uint64_t seed, uint32_t tensor, uint64_t i) {
  return word_at(synth_key(seed, tensor), i);
}

/* Standard normal number i of the stream. */
static inline double normal_at(uint64_t key, uint64_t i) {
  uint64_t p = i >> 1;
  double u0 = uniform_at(key, 2 * p);
  double u1 = uniform_at(key, 2 * p + 1);
  double r = sqrt(-2.0 * log(u0));
  double a = 6.283185307179586476925286766559 * u1;
  return (i & 1) ? r * sin(a) : r * cos(a);
}

double synth_normal(uint64_t seed, uint32_t tensor, uint64_t i) {
  return normal_at(synth_key(seed, tensor), i);
}

/* fp32 -> bf16 bits, round to nearest even (inputs are finite). */
static inline uint16_t f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

enum { SYNTH_F32 = 0, SYNTH_BF16 = 1 };
enum { SYNTH_NORMAL = 0, SYNTH_UNIT_DIR_LOGNORMAL = 1 };

typedef struct {
  uint64_t key, norm_key;
  int32_t B, KH, D, kind, fmt;
  const int32_t *lens;
  const int64_t *seq_offset;
  int64_t stride_h, stride_t;
  const float *chan_mult; /* [KH][D] multipliers or NULL */
  void *out;
  int64_t total_rows;     /* sum over (b, kh) of lens[b] */
  const int64_t *row_start; /* [B*KH + 1] prefix of rows */
  int nthreads, tid;
} job_t;

static void gen_row(const job_t *j, int b, int kh, int64_t t, double *tmp) {
  const int D = j->D;
  uint64_t base = ((uint64_t)(b * j->KH + kh) << 40) + (uint64_t)t * (uint64_t)D;
  for (int d = 0; d < D; ++d) tmp[d] = normal_at(j->key, base + (uint64_t)d);
  if (j->kind == SYNTH_UNIT_DIR_LOGNORMAL) {
    double ss = 0.0;
    for (int d = 0; d < D; ++d) ss += tmp[d] * tmp[d];
    double nrm = sqrt(ss);
    uint64_t nidx = ((uint64_t)(b * j->KH + kh) << 40) + (uint64_t)t;
    double scale = exp(normal_at(j->norm_key, nidx)) / nrm;
    for (int d = 0; d < D; ++d) tmp[d] *= scale;
  }
  if (j->chan_mult) {
    const float *m = j->chan_mult + (size_t)kh * D;
    for (int d = 0; d < D; ++d) tmp[d] *= (double)m[d];
  }
  int64_t off = j->seq_offset[b] + (int64_t)kh * j->stride_h + t * j->stride_t;
  if (j->fmt == SYNTH_F32) {
    float *o = (float *)j->out + off;
    for (int d = 0; d < D; ++d) o[d] = (float)tmp[d];
  } else {
    uint16_t *o = (uint16_t *)j->out + off;
    for (int d = 0; d < D; ++d) o[d] = f32_to_bf16((float)tmp[d]);
  }
}

static void *worker(void *arg) {
  const job_t *j = (const job_t *)arg;
  double *tmp = (double *)malloc(sizeof(double) * (size_t)j->D);
  int64_t per = (j->total_rows + j->nthreads - 1) / j->nthreads;
  int64_t r0 = per * j->tid, r1 = r0 + per;
  if (r1 > j->total_rows) r1 = j->total_rows;
  int nbk = j->B * j->KH;
  int bk = 0;
  for (int64_t r = r0; r < r1; ++r) {
    while (bk < nbk - 1 && j->row_start[bk + 1] <= r) ++bk;
    int b = bk / j->KH, kh = bk % j->KH;
    gen_row(j, b, kh, r - j->row_start[bk], tmp);
  }
  free(tmp);
  return NULL;
}

/*
 * Fill a KV-shaped tensor: for every sequence b < B, head kh < KH and token
 * t < lens[b], the D values of row (b, kh, t) are written at element offset
 * seq_offset[b] + kh*stride_h + t*stride_t.  kind selects i.i.d. N(0,1) or a
 * unit N(0,1) direction scaled by exp(N(0,1)) drawn from tensor `norm_tensor`.
 * chan_mult (may be NULL) multiplies channel d of head kh before rounding.
 * Returns 0 on success.
 */
int synth_fill(uint64_t seed, uint32_t tensor, uint32_t norm_tensor, int32_t B, int32_t KH, int32_t D,
               const int32_t *lens, const int64_t *seq_offset, int64_t stride_h, int64_t stride_t,
               int32_t kind, const float *chan_mult, int32_t fmt, void *out, int32_t nthreads) {
  if (B < 0 || KH < 1 || D < 2 || (D & 1) || nthreads < 1 || !out) return 1;
  int nbk = B * KH;
  int64_t *row_start = (int64_t *)malloc(sizeof(int64_t) * (size_t)(nbk + 1));
  row_start[0] = 0;
  for (int i = 0; i < nbk; ++i) row_start[i + 1] = row_start[i] + (lens[i / KH] > 0 ? lens[i / KH] : 0);
  job_t base;
  memset(&base, 0, sizeof(base));
  base.key = synth_key(seed, tensor);
  base.norm_key = synth_key(seed, norm_tensor);
  base.B = B; base.KH = KH; base.D = D; base.kind = kind; base.fmt = fmt;
  base.lens = lens; base.seq_offset = seq_offset; base.stride_h = stride_h; base.stride_t = stride_t;
  base.chan_mult = chan_mult; base.out = out; base.total_rows = row_start[nbk];
  base.row_start = row_start; base.nthreads = nthreads;
  if (base.total_rows == 0) { free(row_start); return 0; }
  pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
  job_t *jobs = (job_t *)malloc(sizeof(job_t) * (size_t)nthreads);
  for (int i = 0; i < nthreads; ++i) {
    jobs[i] = base;
    jobs[i].tid = i;
    pthread_create(&th[i], NULL, worker, &jobs[i]);
  }
  for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
  free(jobs); free(th); free(row_start);
  return 0;
}
