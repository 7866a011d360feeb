/*
 * synth.c -- seeded synthetic inputs for the KV-cache eviction path.
 *
 * This file holds only input generation: a counter-based random number
 * generator, normal variates, bf16 encoding and the placement of generated
 * rows into a paged cache.  It contains none of the eviction method's
 * arithmetic (no attention, no scores, no selection, no compaction).  Both the
 * CPU oracle and the GPU path consume the bytes written here.
 *
 * Random numbers: SplitMix64 (Steele, Lea and Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014) used as a counter-based
 * generator: value(seed, stream, i) = mix64(key(seed, stream) + (i + 1) * gamma)
 * with gamma = 0x9e3779b97f4a7c15.  Uniforms take the top 53 bits, offset by
 * one half so they lie strictly inside (0, 1).  Normals use the Box-Muller
 * transform (Box and Muller, 1958) on the uniforms at counters 2i and 2i+1.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define SYNTH_GAMMA 0x9e3779b97f4a7c15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
  return z ^ (z >> 31);
}

static inline uint64_t stream_key(uint64_t seed, uint64_t stream) {
  return mix64(mix64(seed + SYNTH_GAMMA) ^ (stream * 0xd1b54a32d192ed03ULL));
}

static inline uint64_t draw_u64(uint64_t key, uint64_t i) {
  return mix64(key + (i + 1) * SYNTH_GAMMA);
}

static inline double draw_uniform(uint64_t key, uint64_t i) {
  return ((double)(draw_u64(key, i) >> 11) + 0.5) * (1.0 / 9007199254740992.0);
}

static inline double draw_normal(uint64_t key, uint64_t i) {
  const double two_pi = 6.283185307179586476925286766559;
  double u1 = draw_uniform(key, 2 * i);
  double u2 = draw_uniform(key, 2 * i + 1);
  return sqrt(-2.0 * log(u1)) * cos(two_pi * u2);
}

/* float -> bf16 bits, round to nearest even; NaN stays a quiet NaN. */
static inline uint16_t f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

uint64_t synth_u64(uint64_t seed, uint64_t stream, uint64_t i) {
  return draw_u64(stream_key(seed, stream), i);
}

void synth_uniform(double *out, int64_t n, uint64_t seed, uint64_t stream, int64_t offset) {
  uint64_t key = stream_key(seed, stream);
  for (int64_t i = 0; i < n; ++i) out[i] = draw_uniform(key, (uint64_t)(offset + i));
}

void synth_normal(double *out, int64_t n, uint64_t seed, uint64_t stream, int64_t offset) {
  uint64_t key = stream_key(seed, stream);
  for (int64_t i = 0; i < n; ++i) out[i] = draw_normal(key, (uint64_t)(offset + i));
}

void synth_f32_to_bf16(const float *in, uint16_t *out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = f32_to_bf16(in[i]);
}

void synth_f64_to_bf16(const double *in, uint16_t *out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = f32_to_bf16((float)in[i]);
}

void synth_bf16_to_f32(const uint16_t *in, float *out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) {
    uint32_t u = (uint32_t)in[i] << 16;
    memcpy(&out[i], &u, 4);
  }
}

/* In-place Fisher-Yates shuffle of perm[0..n) driven by the counter stream. */
void synth_shuffle_i32(int32_t *perm, int64_t n, uint64_t seed, uint64_t stream) {
  uint64_t key = stream_key(seed, stream);
  for (int64_t i = n - 1; i > 0; --i) {
    int64_t j = (int64_t)(draw_uniform(key, (uint64_t)i) * (double)(i + 1));
    if (j > i) j = i;
    int32_t t = perm[i];
    perm[i] = perm[j];
    perm[j] = t;
  }
}

/*
 * Fill the live rows of a paged pool.  Logical row (unit u = b*kv_heads + h,
 * slot s) gets, for d in [0, dim):
 *     x = row_scale[u][s] * N(seed, stream, (u*rows + s)*dim + d)
 *         + plant[u][s] * plant_amp * plant_dir[u][d]
 * written to physical row block_table[u][s/16]*16 + s%16 of `pool` as fp32
 * (is_bf16 = 0) or bf16 (is_bf16 = 1).  row_scale, plant and plant_dir may be
 * NULL (1, 0 and unused).  The normal index does not depend on the block
 * table, so a shuffled table stores the same logical values.
 */
typedef struct {
  void *pool;
  int is_bf16;
  const int32_t *block_table;
  int64_t units, max_blocks, rows, dim;
  const int32_t *n_rows; /* live rows per unit */
  uint64_t key;
  const float *row_scale;
  const uint8_t *plant;
  const float *plant_dir;
  float plant_amp;
  int64_t u0, u1;
} fill_job;

static void *fill_worker(void *arg) {
  fill_job *j = (fill_job *)arg;
  for (int64_t u = j->u0; u < j->u1; ++u) {
    int64_t n = j->n_rows[u];
    for (int64_t s = 0; s < n; ++s) {
      int64_t blk = j->block_table[u * j->max_blocks + s / 16];
      int64_t prow = blk * 16 + s % 16;
      float rs = j->row_scale ? j->row_scale[u * j->rows + s] : 1.0f;
      int pl = j->plant ? j->plant[u * j->rows + s] : 0;
      for (int64_t d = 0; d < j->dim; ++d) {
        double x = (double)rs * draw_normal(j->key, (uint64_t)((u * j->rows + s) * j->dim + d));
        if (pl) x += (double)j->plant_amp * (double)j->plant_dir[u * j->dim + d];
        if (j->is_bf16)
          ((uint16_t *)j->pool)[prow * j->dim + d] = f32_to_bf16((float)x);
        else
          ((float *)j->pool)[prow * j->dim + d] = (float)x;
      }
    }
  }
  return NULL;
}

int synth_fill_paged(void *pool, int is_bf16, const int32_t *block_table, int64_t units,
                     int64_t max_blocks, int64_t rows, int64_t dim, const int32_t *n_rows,
                     uint64_t seed, uint64_t stream, const float *row_scale,
                     const uint8_t *plant, const float *plant_dir, float plant_amp,
                     int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 64) nthreads = 64;
  if (nthreads > units) nthreads = (int)(units > 0 ? units : 1);
  pthread_t th[64];
  fill_job jobs[64];
  for (int t = 0; t < nthreads; ++t) {
    fill_job j = {pool, is_bf16, block_table, units, max_blocks, rows, dim, n_rows,
                  stream_key(seed, stream), row_scale, plant, plant_dir, plant_amp,
                  units * t / nthreads, units * (t + 1) / nthreads};
    jobs[t] = j;
  }
  for (int t = 1; t < nthreads; ++t) pthread_create(&th[t], NULL, fill_worker, &jobs[t]);
  fill_worker(&jobs[0]);
  for (int t = 1; t < nthreads; ++t) pthread_join(th[t], NULL);
  return 0;
}

/*
 * Dense rows: out[i*dim + d] = row_scale[i] * N(seed, stream, i*dim + d)
 *                              + plant_amp * plant_dir[dir_of_row[i]*dim + d]
 * for i in [0, n_rows); plant_dir/dir_of_row may be NULL.  Output as fp32 or bf16.
 */
int synth_fill_rows(void *out, int is_bf16, int64_t n_rows, int64_t dim, uint64_t seed,
                    uint64_t stream, const float *row_scale, const int32_t *dir_of_row,
                    const float *plant_dir, float plant_amp) {
  uint64_t key = stream_key(seed, stream);
  for (int64_t i = 0; i < n_rows; ++i) {
    float rs = row_scale ? row_scale[i] : 1.0f;
    for (int64_t d = 0; d < dim; ++d) {
      double x = (double)rs * draw_normal(key, (uint64_t)(i * dim + d));
      if (plant_dir && dir_of_row && dir_of_row[i] >= 0)
        x += (double)plant_amp * (double)plant_dir[(int64_t)dir_of_row[i] * dim + d];
      if (is_bf16)
        ((uint16_t *)out)[i * dim + d] = f32_to_bf16((float)x);
      else
        ((float *)out)[i * dim + d] = (float)x;
    }
  }
  return 0;
}
