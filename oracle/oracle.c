/*
 * oracle.c -- plain CPU reference of attention-score KV-cache eviction.
 *
 * TEST INFRASTRUCTURE (see oracle.h).  Scalar loops, double precision, no
 * blocking and no reordering beyond what each definition states.  Threads are
 * used only across independent KV heads (b, h).
 */
#include "oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- helpers */

static double widen(const void *base, int is_bf16, int64_t idx) {
  if (is_bf16) {
    uint32_t u = (uint32_t)((const uint16_t *)base)[idx] << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
  }
  return (double)((const float *)base)[idx];
}

/* Physical row of slot s of unit u ([VTOK] section 3.4, Eq. 2 with S = 16). */
static int64_t phys_row(const orc_cache *c, int64_t u, int64_t s) {
  return (int64_t)c->block_table[u * c->max_blocks + s / 16] * 16 + s % 16;
}

typedef void (*unit_fn)(void *ctx, int64_t unit);
typedef struct {
  unit_fn fn;
  void *ctx;
  const uint8_t *mask;
  int64_t units;
  int tid, nthreads;
} par_job;

static void *par_worker(void *arg) {
  par_job *j = (par_job *)arg;
  for (int64_t u = j->tid; u < j->units; u += j->nthreads)
    if (!j->mask || j->mask[u]) j->fn(j->ctx, u);
  return NULL;
}

static void parallel_units(unit_fn fn, void *ctx, int64_t units, const uint8_t *mask,
                           int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if (nthreads > units) nthreads = (int)(units > 0 ? units : 1);
  pthread_t th[256];
  par_job jobs[256];
  for (int t = 0; t < nthreads; ++t) {
    par_job j = {fn, ctx, mask, units, t, nthreads};
    jobs[t] = j;
  }
  for (int t = 1; t < nthreads; ++t) pthread_create(&th[t], NULL, par_worker, &jobs[t]);
  par_worker(&jobs[0]);
  for (int t = 1; t < nthreads; ++t) pthread_join(th[t], NULL);
}

/* q.k_s of one window query row against slot s of unit u, d ascending. */
static double dot_qk(const orc_cache *c, const orc_window *w, int64_t qrow, int64_t u, int64_t s) {
  int64_t D = c->head_dim, prow = phys_row(c, u, s);
  double acc = 0.0;
  for (int64_t d = 0; d < D; ++d)
    acc += widen(w->q, c->is_bf16, qrow * D + d) * widen(c->k_pool, c->is_bf16, prow * D + d);
  return acc;
}

/* ---------------------------------------------- LSE and output (inputs) */
/*
 * The log-sum-exp of a query's scaled logits over the keys it attends, and the
 * attention output a = sum_j p_j v_j.  A forward pass produces both ([DROP]
 * Jargon, "Log-sum-exp"); here they are built from their definitions,
 * max-shifted, to feed the scoring step.
 */
typedef struct {
  const orc_cache *c;
  const orc_window *w;
  double *lse, *a;
} lse_ctx;

static void lse_unit(void *vctx, int64_t u) {
  lse_ctx *x = (lse_ctx *)vctx;
  const orc_cache *c = x->c;
  const orc_window *w = x->w;
  int64_t G = w->group, W = w->obs_window, D = c->head_dim;
  int64_t b = u / c->kv_heads, h = u % c->kv_heads, Hq = (int64_t)c->kv_heads * G;
  int64_t n = c->seq_len[u];
  const int32_t *pos = c->pos + u * (int64_t)c->max_blocks * 16;
  double *s = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
  for (int64_t g = 0; g < G; ++g) {
    int64_t hq = h * G + g;
    for (int64_t wi = 0; wi < W; ++wi) {
      int64_t qrow = (b * Hq + hq) * W + wi;
      int32_t qp = w->q_pos[b * W + wi];
      double mx = -INFINITY;
      for (int64_t j = 0; j < n; ++j) {
        if (pos[j] > qp) continue;
        s[j] = w->scale * dot_qk(c, w, qrow, u, j);
        if (s[j] > mx) mx = s[j];
      }
      double z = 0.0;
      for (int64_t j = 0; j < n; ++j)
        if (pos[j] <= qp) z += exp(s[j] - mx);
      double lse = (z > 0.0) ? mx + log(z) : -INFINITY;
      x->lse[qrow] = lse;
      if (x->a) {
        double *arow = x->a + qrow * D;
        for (int64_t d = 0; d < D; ++d) arow[d] = 0.0;
        if (z > 0.0) {
          for (int64_t j = 0; j < n; ++j) {
            if (pos[j] > qp) continue;
            double p = exp(s[j] - lse);
            int64_t prow = phys_row(c, u, j);
            for (int64_t d = 0; d < D; ++d) arow[d] += p * widen(c->v_pool, c->is_bf16, prow * D + d);
          }
        }
      }
    }
  }
  free(s);
}

int orc_lse_a(const orc_cache *c, const orc_window *w, double *lse_out, double *a_out,
              const uint8_t *unit_mask, int nthreads) {
  if (!c || !w || !lse_out || !w->q || !w->q_pos || w->group < 1 || w->obs_window < 1) return -1;
  lse_ctx ctx = {c, w, lse_out, a_out};
  parallel_units(lse_unit, &ctx, (int64_t)c->batch * c->kv_heads, unit_mask, nthreads);
  return 0;
}

/* ------------------------------------------------------------- scoring */
/*
 * Attention probability of window query (g, w) for slot j:
 *     p = exp(scale * q.k_j - LSE)     if pos_j <= q_pos_w, else 0
 * ([H2O] "The Existence of Heavy Hitters": A = softmax(QK^T / sqrt(d)); the
 * LSE form of the same softmax per [DROP] Jargon).  The diagonal is included,
 * so each row is the full softmax.
 *
 * SUM: S_j = sum_w sum_g p  -- the accumulated attention of [H2O]
 *   "Formulating Cumulative Attention Scores", summed over the query heads of
 *   the KV head's GQA group ([H2O] FAQ, GQA) and over the window, which is
 *   also the SnapKV window sum ([SNAP] "How it works").  In ACCUMULATE mode
 *   the previous score is added ([H2O] lifecycle step "Score Accumulation").
 * POOL: P_j = max of S_i for i in [j - r, j + r] clamped to [0, n-1],
 *   r = (pool_kernel - 1) / 2 ([SNAP] "How it works").
 * DROP: sum_w sum_g p / (1 - p) * ||a - v_j||  ([DROP] Lemma 1: the output
 *   shift from removing j is p_j/(1-p_j)(a - v_j); the score is its length,
 *   summed over the window).  1 - p is -expm1(x); when x >= 0 (p >= 1) the
 *   removal is undefined and the term is +inf.
 */
typedef struct {
  const orc_cache *c;
  const orc_window *w;
  int flags, pool_kernel;
  const float *prev;
  double *sum, *pooled, *drop;
} score_ctx;

static void score_unit(void *vctx, int64_t u) {
  score_ctx *x = (score_ctx *)vctx;
  const orc_cache *c = x->c;
  const orc_window *w = x->w;
  int64_t G = w->group, W = w->obs_window, D = c->head_dim;
  int64_t b = u / c->kv_heads, h = u % c->kv_heads, Hq = (int64_t)c->kv_heads * G;
  int64_t n = c->seq_len[u], max_slots = (int64_t)c->max_blocks * 16;
  const int32_t *pos = c->pos + u * max_slots;
  double *S = (double *)calloc((size_t)(n > 0 ? n : 1), sizeof(double));
  double *R = (double *)calloc((size_t)(n > 0 ? n : 1), sizeof(double));

  for (int64_t wi = 0; wi < W; ++wi) {
    int32_t qp = w->q_pos[b * W + wi];
    for (int64_t g = 0; g < G; ++g) {
      int64_t hq = h * G + g;
      int64_t qrow = (b * Hq + hq) * W + wi;
      double lse = (double)w->lse[qrow];
      for (int64_t j = 0; j < n; ++j) {
        if (pos[j] > qp) continue;
        double xv = w->scale * dot_qk(c, w, qrow, u, j) - lse;
        double p = exp(xv);
        S[j] += p;
        if (x->flags & ORC_DROP) {
          int64_t prow = phys_row(c, u, j);
          double r2 = 0.0;
          for (int64_t d = 0; d < D; ++d) {
            double diff = (double)w->a[qrow * D + d] -
                          widen(c->v_pool, c->is_bf16, prow * D + d);
            r2 += diff * diff;
          }
          double term = (xv >= 0.0) ? INFINITY : p / (-expm1(xv)) * sqrt(r2);
          R[j] += term;
        }
      }
    }
  }
  double *sum_row = x->sum ? x->sum + u * max_slots : NULL;
  if (x->flags & ORC_ACCUMULATE)
    for (int64_t j = 0; j < n; ++j) S[j] += (double)x->prev[u * max_slots + j];
  if (sum_row)
    for (int64_t j = 0; j < n; ++j) sum_row[j] = S[j];
  if (x->flags & ORC_POOL) {
    int64_t r = (x->pool_kernel - 1) / 2;
    double *P = x->pooled + u * max_slots;
    for (int64_t j = 0; j < n; ++j) {
      int64_t lo = j - r < 0 ? 0 : j - r, hi = j + r > n - 1 ? n - 1 : j + r;
      double m = S[lo];
      for (int64_t i = lo + 1; i <= hi; ++i)
        if (S[i] > m) m = S[i];
      P[j] = m;
    }
  }
  if (x->flags & ORC_DROP) {
    double *Dr = x->drop + u * max_slots;
    for (int64_t j = 0; j < n; ++j) Dr[j] = R[j];
  }
  free(S);
  free(R);
}

int orc_score(const orc_cache *c, const orc_window *w, int flags, int pool_kernel,
              const float *prev_sum, double *sum, double *pooled, double *drop,
              const uint8_t *unit_mask, int nthreads) {
  if (!c || !w || !w->q || !w->lse || !w->q_pos) return -1;
  if (w->group < 1 || w->obs_window < 1) return -1;
  if (!(flags & (ORC_SUM | ORC_POOL | ORC_DROP))) return -1;
  if ((flags & ORC_SUM) && !sum) return -1;
  if ((flags & ORC_POOL) && (!pooled || pool_kernel < 1 || pool_kernel % 2 == 0)) return -1;
  if ((flags & ORC_DROP) && (!drop || !w->a)) return -1;
  if ((flags & ORC_ACCUMULATE) && (!prev_sum || (flags & (ORC_POOL | ORC_DROP)))) return -1;
  score_ctx ctx = {c, w, flags, pool_kernel, prev_sum, (flags & ORC_SUM) ? sum : NULL, pooled, drop};
  parallel_units(score_unit, &ctx, (int64_t)c->batch * c->kv_heads, unit_mask, nthreads);
  return 0;
}

/* ----------------------------------------------------------- selection */
/*
 * Victims of one KV head ([H2O] "Step-by-Step Eviction Lifecycle" and
 * "Dual-Pool Budget Partitioning"; [SNAP] "How it works", "Tie-breaking",
 * "Parameters"; [DROP] greedy bottom-k):
 *   m = max(0, n - budget) tokens go; the budget counts the recent window.
 *   Candidates are slots [0, n - R): the last R slots are protected.
 *   Order candidates by (score, position); equal scores evict the lower
 *   position first.  -0 equals +0; NaN ranks above +inf.
 *   The m first candidates are returned in ascending position order.
 */
typedef struct {
  float v;
  int32_t slot;
} cand;

static int score_class(float v) { return isnan(v) ? 1 : 0; }

static int cand_cmp(const void *pa, const void *pb) {
  const cand *a = (const cand *)pa, *b = (const cand *)pb;
  int ca = score_class(a->v), cb = score_class(b->v);
  if (ca != cb) return ca < cb ? -1 : 1;
  if (!ca) {
    if (a->v < b->v) return -1; /* numeric compare: -0 == +0 */
    if (a->v > b->v) return 1;
  }
  return (a->slot > b->slot) - (a->slot < b->slot);
}

static int int_cmp(const void *pa, const void *pb) {
  int32_t a = *(const int32_t *)pa, b = *(const int32_t *)pb;
  return (a > b) - (a < b);
}

int orc_select(const float *scores, const int32_t *seq_len, int32_t units, int32_t max_slots,
               int32_t budget, int32_t recent_window, int32_t *victims, int32_t *n_victims) {
  if (!scores || !seq_len || !victims || !n_victims) return -1;
  if (budget <= 0 || recent_window < 0 || recent_window >= budget) return -1;
  cand *buf = (cand *)malloc(sizeof(cand) * (size_t)(max_slots > 0 ? max_slots : 1));
  for (int64_t u = 0; u < units; ++u) {
    int64_t n = seq_len[u];
    int64_t m = n - budget > 0 ? n - budget : 0;
    int64_t nc = n - recent_window > 0 ? n - recent_window : 0;
    for (int64_t j = 0; j < nc; ++j) {
      buf[j].v = scores[u * (int64_t)max_slots + j];
      buf[j].slot = (int32_t)j;
    }
    qsort(buf, (size_t)nc, sizeof(cand), cand_cmp);
    int32_t *out = victims + u * (int64_t)max_slots;
    for (int64_t i = 0; i < m; ++i) out[i] = buf[i].slot;
    qsort(out, (size_t)m, sizeof(int32_t), int_cmp);
    n_victims[u] = (int32_t)m;
  }
  free(buf);
  return 0;
}

/* ---------------------------------------------------------- compaction */
/*
 * Order-preserving, in-place left-pack of each KV head's kept rows within its
 * own blocks ([H2O] "PagedAttention Memory Integration": in-place overwrite
 * within existing pages; [VTOK] section 3.3 stage 3: fill destinations fully,
 * keep logical order).  Kept slots in ascending order take ranks 0, 1, ...;
 * row r <- row s for K, V, pos and the optional score row.  Blocks at logical
 * indices [ceil(n'/16), ceil(n/16)) are then empty: they are appended to the
 * free list in (b, h, logical block) order and their table entries set to -1
 * ([VTOK] section 1: whole emptied blocks return to the free pool).
 * Rank <= slot, so an ascending sequential copy never overwrites a row that is
 * still to be read.
 */
int orc_compact(void *k_pool, void *v_pool, int32_t elem_bytes, int32_t head_dim,
                int32_t *block_table, int32_t *seq_len, int32_t *pos, float *score,
                int32_t units, int32_t max_blocks, const int32_t *victims,
                const int32_t *n_victims, int32_t *free_list, int32_t *free_count,
                int32_t free_capacity, int64_t *stats) {
  if (!k_pool || !v_pool || !block_table || !seq_len || !pos || !victims || !n_victims ||
      !free_list || !free_count || !stats)
    return -1;
  if (elem_bytes != 2 && elem_bytes != 4) return -1;
  int64_t max_slots = (int64_t)max_blocks * 16;
  int64_t row_bytes = (int64_t)head_dim * elem_bytes;
  int64_t total_free = 0;
  for (int64_t u = 0; u < units; ++u) {
    int64_t n = seq_len[u], m = n_victims[u];
    if (m < 0 || m > n) return -1;
    total_free += (n + 15) / 16 - (n - m + 15) / 16;
  }
  if (*free_count + total_free > free_capacity) return -2;

  int64_t blocks_freed = 0, rows_moved = 0, at_risk = 0;
  for (int64_t u = 0; u < units; ++u) {
    int64_t n = seq_len[u], m = n_victims[u], n2 = n - m;
    const int32_t *vic = victims + u * max_slots;
    int32_t *bt = block_table + u * max_blocks;
    int32_t *ps = pos + u * max_slots;
    float *sc = score ? score + u * max_slots : NULL;
    int64_t vi = 0, r = 0;
    for (int64_t s = 0; s < n; ++s) {
      if (vi < m && vic[vi] == s) {
        ++vi;
        continue;
      }
      if (r != s) {
        int64_t dst = (int64_t)bt[r / 16] * 16 + r % 16;
        int64_t src = (int64_t)bt[s / 16] * 16 + s % 16;
        memcpy((char *)k_pool + dst * row_bytes, (char *)k_pool + src * row_bytes, (size_t)row_bytes);
        memcpy((char *)v_pool + dst * row_bytes, (char *)v_pool + src * row_bytes, (size_t)row_bytes);
        ps[r] = ps[s];
        if (sc) sc[r] = sc[s];
        ++rows_moved;
        if (s < n2) ++at_risk;
      }
      ++r;
    }
    for (int64_t lb = (n2 + 15) / 16; lb < (n + 15) / 16; ++lb) {
      free_list[(*free_count)++] = bt[lb];
      bt[lb] = -1;
      ++blocks_freed;
    }
    seq_len[u] = (int32_t)n2;
  }
  stats[0] = blocks_freed;
  stats[1] = rows_moved;
  stats[2] = rows_moved * 2 * row_bytes * 2; /* K and V rows, each read once and written once */
  stats[3] = at_risk;
  stats[4] = 0;
  return 0;
}

/* --------------------------------------------------------- measurement */
/*
 * Intra-block waste F = 1 - sum_i n_i / (N * S) over the N allocated blocks
 * ([VTOK] section 2, Eq. 1), and the fraction of allocated blocks at or below
 * 50% use ([VTOK] Fig. 1).  "naive": victims are only marked dead, every block
 * stays allocated; "after": the kept tokens are packed and emptied blocks freed.
 */
int orc_measure(const int32_t *seq_len_before, const int32_t *victims, const int32_t *n_victims,
                int32_t units, int32_t max_slots, double *out) {
  if (!seq_len_before || !victims || !n_victims || !out) return -1;
  double live = 0, blocks_naive = 0, blocks_after = 0, half_naive = 0, half_after = 0;
  for (int64_t u = 0; u < units; ++u) {
    int64_t n = seq_len_before[u], m = n_victims[u], n2 = n - m;
    const int32_t *vic = victims + u * (int64_t)max_slots;
    int64_t vi = 0;
    for (int64_t lb = 0; lb < (n + 15) / 16; ++lb) {
      int64_t live_b = 0;
      for (int64_t s = lb * 16; s < lb * 16 + 16 && s < n; ++s) {
        while (vi < m && vic[vi] < s) ++vi;
        if (!(vi < m && vic[vi] == s)) ++live_b;
      }
      blocks_naive += 1;
      if (2 * live_b <= 16) half_naive += 1;
    }
    for (int64_t lb = 0; lb < (n2 + 15) / 16; ++lb) {
      int64_t live_b = (lb + 1) * 16 <= n2 ? 16 : n2 - lb * 16;
      blocks_after += 1;
      if (2 * live_b <= 16) half_after += 1;
    }
    live += (double)n2;
  }
  out[0] = blocks_naive > 0 ? 1.0 - live / (blocks_naive * 16.0) : 0.0;
  out[1] = blocks_after > 0 ? 1.0 - live / (blocks_after * 16.0) : 0.0;
  out[2] = blocks_naive > 0 ? half_naive / blocks_naive : 0.0;
  out[3] = blocks_after > 0 ? half_after / blocks_after : 0.0;
  out[4] = blocks_naive;
  out[5] = blocks_after;
  out[6] = live;
  out[7] = blocks_naive - blocks_after;
  return 0;
}

/* ----------------------------------------------------- H2O decode step */
/*
 * [H2O] "Step-by-Step Eviction Lifecycle": the new token's query attends to
 * the cached tokens and to itself; the attention weights, summed over the G
 * query heads of the KV head (GQA), are added to the running scores; if the
 * cache holds more tokens than the budget, the token with the smallest
 * running score outside the recent window is pruned.  [H2O] "PagedAttention
 * Memory Integration": the pruned token's slot is overwritten in place by the
 * new token, so the cache never grows past the budget.  The recent window is
 * the `recent` most recent positions t - recent + 1 .. t; ties on the score
 * evict the lower position.  Heads are processed in (b, h) order, so the
 * blocks taken from the free list (top of the stack first) go to the heads in
 * that order.
 */
static void copy_row(void *pool, int64_t row, const void *src, int64_t row_bytes) {
  memcpy((char *)pool + row * row_bytes, src, (size_t)row_bytes);
}

int orc_h2o_step(void *k_pool, void *v_pool, int32_t is_bf16, int32_t head_dim,
                 int32_t *block_table, int32_t *seq_len, int32_t *pos, float *score,
                 int32_t batch, int32_t kv_heads, int32_t max_blocks, int32_t num_blocks,
                 int32_t group, const void *q, const void *k_new, const void *v_new,
                 const int32_t *t_pos, double scale, int32_t budget, int32_t recent,
                 int32_t *free_list, int32_t *free_count, int32_t *evicted_pos,
                 double *attn_out, double *attn_abs) {
  if (!k_pool || !v_pool || !block_table || !seq_len || !pos || !score || !q || !k_new || !v_new ||
      !t_pos || !free_list || !free_count || !evicted_pos)
    return -1;
  if (group < 1 || budget <= 0 || recent < 0 || recent >= budget) return -1;
  if (budget > max_blocks * 16) return -1;
  const int64_t D = head_dim, G = group, max_slots = (int64_t)max_blocks * 16;
  const int64_t row_bytes = D * (is_bf16 ? 2 : 4);
  double *s = (double *)malloc(sizeof(double) * (size_t)(G * (budget + 1)));
  double *lse = (double *)malloc(sizeof(double) * (size_t)G);
  for (int64_t u = 0; u < (int64_t)batch * kv_heads; ++u) {
    const int64_t b = u / kv_heads, h = u % kv_heads;
    const int64_t n = seq_len[u], t = t_pos[b];
    int32_t *bt = block_table + u * max_blocks;
    int32_t *ps = pos + u * max_slots;
    float *sc = score + u * max_slots;
    if (n < 0 || n > budget) {
      evicted_pos[u] = -2;
      continue;
    }
    int bad = 0;
    for (int64_t lb = 0; lb < (n + 15) / 16; ++lb)
      if (bt[lb] < 0 || bt[lb] >= num_blocks) bad = 1;
    const int need_block = n < budget && n % 16 == 0 && bt[n / 16] < 0;
    if (!need_block && n < budget && bt[n / 16] >= num_blocks) bad = 1;
    if (bad) {
      evicted_pos[u] = -4;
      continue;
    }
    if (need_block) {
      if (*free_count <= 0) {
        evicted_pos[u] = -3;
        continue;
      }
      const int32_t blk = free_list[--*free_count]; /* taken even if it is out of range */
      if (blk < 0 || blk >= num_blocks) {
        evicted_pos[u] = -4;
        continue;
      }
      bt[n / 16] = blk;
    }
    /* logits of the G query rows: cached tokens (slot j), then the new token (index n) */
    const char *knew = (const char *)k_new + u * row_bytes;
    for (int64_t g = 0; g < G; ++g) {
      const int64_t qrow = (b * kv_heads + h) * G + g;
      double mx = -INFINITY;
      for (int64_t j = 0; j <= n; ++j) {
        double acc = 0.0;
        if (j < n && ps[j] > t) {
          s[g * (budget + 1) + j] = -INFINITY; /* a later position is not attended */
          continue;
        }
        const int64_t prow = j < n ? (int64_t)bt[j / 16] * 16 + j % 16 : -1;
        for (int64_t d = 0; d < D; ++d) {
          const double kd = j < n ? widen(k_pool, is_bf16, prow * D + d) : widen(knew, is_bf16, d);
          acc += widen(q, is_bf16, qrow * D + d) * kd;
        }
        s[g * (budget + 1) + j] = scale * acc;
        if (s[g * (budget + 1) + j] > mx) mx = s[g * (budget + 1) + j];
      }
      double z = 0.0;
      for (int64_t j = 0; j <= n; ++j) z += exp(s[g * (budget + 1) + j] - mx);
      lse[g] = mx + log(z);
    }
    /* the step's attention output: the same weights on the values */
    if (attn_out || attn_abs) {
      const char *vnew = (const char *)v_new + u * row_bytes;
      for (int64_t g = 0; g < G; ++g) {
        const int64_t qrow = (b * kv_heads + h) * G + g;
        for (int64_t d = 0; d < D; ++d) {
          double acc = 0.0, aabs = 0.0;
          for (int64_t j = 0; j <= n; ++j) {
            const double p = exp(s[g * (budget + 1) + j] - lse[g]);
            const double vd = j < n ? widen(v_pool, is_bf16, ((int64_t)bt[j / 16] * 16 + j % 16) * D + d)
                                    : widen(vnew, is_bf16, d);
            acc += p * vd;
            aabs += p * fabs(vd);
          }
          if (attn_out) attn_out[qrow * D + d] = acc;
          if (attn_abs) attn_abs[qrow * D + d] = aabs;
        }
      }
    }
    /* the running scores after this step's attention (g ascending) */
    float s_new;
    {
      double pn = 0.0;
      for (int64_t g = 0; g < G; ++g) pn += exp(s[g * (budget + 1) + n] - lse[g]);
      s_new = (float)pn;
    }
    for (int64_t j = 0; j < n; ++j) {
      double pj = 0.0;
      for (int64_t g = 0; g < G; ++g) pj += exp(s[g * (budget + 1) + j] - lse[g]);
      sc[j] = (float)((double)sc[j] + pj);
    }
    int64_t dst;
    if (n < budget) {
      dst = n;
      seq_len[u] = (int32_t)(n + 1);
      evicted_pos[u] = -1;
    } else {
      /* argmin of (score, position) over the tokens outside the recent window */
      int64_t best = -2; /* -2: none yet, -1: the new token, >= 0: a slot */
      float bv = 0.f;
      int64_t bp = 0;
      for (int64_t j = 0; j <= n; ++j) {
        const int64_t pj = j < n ? ps[j] : t;
        if (t - pj < recent) continue;
        const float v = j < n ? sc[j] : s_new;
        const cand a = {v, 0}, c = {bv, 0};
        int less;
        if (best == -2) {
          less = 1;
        } else {
          const int cmp = cand_cmp(&a, &c); /* value order, NaN above every number */
          less = cmp < 0 || (cmp == 0 && pj < bp);
        }
        if (less) {
          best = j < n ? j : -1;
          bv = v;
          bp = pj;
        }
      }
      if (best < 0) {
        /* the new token itself is dropped (or, with positions that leave no
         * candidate at all, cannot be placed) */
        evicted_pos[u] = (int32_t)t;
        continue;
      }
      dst = best;
      evicted_pos[u] = ps[dst];
    }
    const int64_t row = (int64_t)bt[dst / 16] * 16 + dst % 16;
    copy_row(k_pool, row, knew, row_bytes);
    copy_row(v_pool, row, (const char *)v_new + u * row_bytes, row_bytes);
    ps[dst] = (int32_t)t;
    sc[dst] = s_new;
  }
  free(lse);
  free(s);
  return 0;
}

/* --------------------------------------------- vToken lazy reclamation */
/*
 * [VTOK] section 3.2: a token table keeps, per token, its physical place and
 * a liveness bit; evicting a token only clears the bit.  Section 3.3: the
 * reclamation backend later packs the live tokens of several under-used
 * blocks into fewer destination blocks taken from the free pool (out of
 * place), fills each destination completely, keeps the logical order, and
 * returns the emptied source blocks; it refuses plans that would not free
 * anything (section 3.5, I4).  Here the token table of a head is its block
 * list plus the per-slot liveness and position, so a relocation rewrites the
 * block list entries of the sources.
 */
int orc_vtok_evict(const int32_t *block_table, const int32_t *seq_len, uint8_t *live,
                   int32_t *block_live, int32_t units, int32_t max_blocks,
                   const int32_t *victims, const int32_t *n_victims, int32_t *status) {
  if (!block_table || !seq_len || !live || !block_live || !victims || !n_victims || !status)
    return -1;
  const int64_t max_slots = (int64_t)max_blocks * 16;
  *status = 0;
  for (int64_t u = 0; u < units; ++u) {
    const int64_t n = seq_len[u];
    int64_t m = n_victims[u];
    if (m > max_slots) { /* the list holds max_slots entries */
      *status |= 1;
      m = max_slots;
    }
    for (int64_t i = 0; i < m; ++i) {
      const int64_t v = victims[u * max_slots + i];
      if (v < 0 || v >= n || v >= max_slots || block_table[u * max_blocks + v / 16] < 0 ||
          !live[u * max_slots + v]) {
        *status |= 1;
        continue;
      }
      live[u * max_slots + v] = 0;
      block_live[u * max_blocks + v / 16] -= 1;
    }
  }
  return 0;
}

int orc_vtok_reclaim(void *k_pool, void *v_pool, int32_t elem_bytes, int32_t head_dim,
                     int32_t *block_table, const int32_t *seq_len, int32_t *pos, float *score,
                     uint8_t *live, int32_t *block_live, int32_t units, int32_t max_blocks,
                     int32_t num_blocks, double theta_f, int32_t max_sources,
                     int32_t *free_list, int32_t *free_count, int32_t free_capacity,
                     int64_t *stats) {
  if (!k_pool || !v_pool || !block_table || !seq_len || !pos || !live || !block_live ||
      !free_list || !free_count || !stats || max_sources < 1)
    return -1;
  if (elem_bytes != 2 && elem_bytes != 4) return -1;
  if (*free_count < 0 || *free_count > free_capacity) return -1;
  const int64_t max_slots = (int64_t)max_blocks * 16, row_bytes = (int64_t)head_dim * elem_bytes;
  for (int i = 0; i < 10; ++i) stats[i] = 0;
  /* every head's plan: sources and the destination count */
  int32_t *src = (int32_t *)malloc(sizeof(int32_t) * (size_t)(units * (int64_t)max_sources + 1));
  int32_t *nsrc = (int32_t *)calloc((size_t)units + 1, sizeof(int32_t));
  int32_t *ndst = (int32_t *)calloc((size_t)units + 1, sizeof(int32_t));
  int64_t total_free = *free_count;
  for (int64_t u = 0; u < units; ++u) {
    const int64_t n = seq_len[u];
    const int32_t *bt = block_table + u * max_blocks;
    if (n < 0 || n > max_slots) {
      stats[9] |= 2;
      continue;
    }
    const int64_t nb = (n + 15) / 16;
    int64_t alloc = 0, livec = 0, bad = 0;
    for (int64_t lb = 0; lb < nb; ++lb)
      if (bt[lb] >= 0) {
        ++alloc;
        livec += block_live[u * max_blocks + lb];
        if (bt[lb] >= num_blocks || block_live[u * max_blocks + lb] < 0 ||
            block_live[u * max_blocks + lb] > 16)
          bad = 1;
      }
    if (bad) {
      stats[9] |= 4;
      continue;
    }
    stats[6] += livec;
    stats[7] += alloc;
    const double F = alloc > 0 ? 1.0 - (double)livec / (16.0 * (double)alloc) : 0.0;
    if (!(F > theta_f)) {
      ++stats[2];
      continue;
    }
    int64_t k = 0, T = 0;
    for (int64_t lb = 0; lb + 1 < nb && k < max_sources; ++lb) {
      if (bt[lb] < 0 || block_live[u * max_blocks + lb] >= 16) continue;
      src[u * max_sources + k++] = (int32_t)lb;
      T += block_live[u * max_blocks + lb];
    }
    const int64_t D = (T + 15) / 16;
    if (k < 2 || D >= k) {
      ++stats[2]; /* nothing to gain: counted with the heads left as they are */
      continue;
    }
    nsrc[u] = (int32_t)k;
    ndst[u] = (int32_t)D;
  }
  /* headroom: destinations from the top of the free list, heads in order */
  int64_t fc = *free_count, taken = 0, pushed = 0;
  int64_t *dst_off = (int64_t *)calloc((size_t)units + 1, sizeof(int64_t));
  for (int64_t u = 0; u < units; ++u) {
    if (!nsrc[u]) continue;
    if (taken + ndst[u] > fc) {
      ++stats[1];
      nsrc[u] = 0;
      continue;
    }
    dst_off[u] = taken;
    taken += ndst[u];
    pushed += nsrc[u];
  }
  if (fc - taken + pushed > free_capacity) {
    free(src); free(nsrc); free(ndst); free(dst_off);
    return -2;
  }
  (void)total_free;
  /* moves, in head order; destinations are free_list[fc - 1 - dst_off - d] */
  int32_t *dst_ids = (int32_t *)malloc(sizeof(int32_t) * (size_t)(taken + 1));
  for (int64_t i = 0; i < taken; ++i) dst_ids[i] = free_list[fc - 1 - i];
  int64_t top = fc - taken;
  int32_t *tpos = (int32_t *)malloc(sizeof(int32_t) * (size_t)(max_sources * 16 + 1));
  float *tsc = (float *)malloc(sizeof(float) * (size_t)(max_sources * 16 + 1));
  for (int64_t u = 0; u < units; ++u) {
    const int64_t k = nsrc[u];
    if (!k) continue;
    int32_t *bt = block_table + u * max_blocks;
    int32_t *ps = pos + u * max_slots;
    uint8_t *lv = live + u * max_slots;
    int32_t *bl = block_live + u * max_blocks;
    float *sc = score ? score + u * max_slots : NULL;
    const int32_t *sv = src + u * max_sources;
    const int64_t D = ndst[u];
    int64_t i = 0;
    for (int64_t j = 0; j < k; ++j) {
      const int64_t lb = sv[j];
      for (int64_t o = 0; o < 16; ++o) {
        const int64_t s = lb * 16 + o;
        if (!lv[s]) continue;
        const int64_t from = (int64_t)bt[lb] * 16 + o;
        const int64_t to = (int64_t)dst_ids[dst_off[u] + i / 16] * 16 + i % 16;
        memcpy((char *)k_pool + to * row_bytes, (char *)k_pool + from * row_bytes, (size_t)row_bytes);
        memcpy((char *)v_pool + to * row_bytes, (char *)v_pool + from * row_bytes, (size_t)row_bytes);
        tpos[i] = ps[s];
        if (sc) tsc[i] = sc[s];
        ++i;
      }
    }
    const int64_t T = i;
    /* the block list and the per-slot table of the source positions */
    for (int64_t j = 0; j < k; ++j) {
      const int64_t lb = sv[j];
      free_list[top++] = bt[lb];
      bt[lb] = j < D ? dst_ids[dst_off[u] + j] : -1;
      const int64_t cnt = j < D ? (T - 16 * j < 16 ? T - 16 * j : 16) : 0;
      bl[lb] = (int32_t)cnt;
      for (int64_t o = 0; o < 16; ++o) {
        const int64_t s = lb * 16 + o, t = 16 * j + o;
        lv[s] = o < cnt ? 1 : 0;
        if (o < cnt) {
          ps[s] = tpos[t];
          if (sc) sc[s] = tsc[t];
        }
      }
    }
    ++stats[0];
    stats[3] += k - D;
    stats[4] += T;
    stats[5] += T * 2 * row_bytes * 2;
    stats[8] -= k - D;
  }
  stats[8] += stats[7];
  *free_count = (int32_t)top;
  free(tpos); free(tsc); free(dst_ids); free(src); free(nsrc); free(ndst); free(dst_off);
  return 0;
}



/* ---- online checks of I1 and I2 ([VTOK] section 3.5) ---- */

/* MurmurHash3's 64-bit finalizer (Appleby): xor-shift, multiply, twice. */
uint64_t orc_fmix64(uint64_t k) {
  k ^= k >> 33;
  k *= 0xff51afd7ed558ccdULL;
  k ^= k >> 33;
  k *= 0xc4ceb9fe1a85ec53ULL;
  k ^= k >> 33;
  return k;
}

static uint64_t row_word(const void *pool, int64_t row, int32_t row_bytes, int64_t i) {
  uint64_t w;
  memcpy(&w, (const char *)pool + row * row_bytes + i * 8, 8);
  return w;
}

int orc_vtok_digest(const void *k_pool, const void *v_pool, int32_t row_bytes,
                    const int32_t *block_table, const int32_t *seq_len, const int32_t *pos,
                    const uint8_t *live, int32_t units, int32_t max_blocks, int32_t num_blocks,
                    uint64_t *digest) {
  if (!k_pool || !v_pool || !block_table || !seq_len || !pos || !live || !digest ||
      row_bytes <= 0 || row_bytes % 8)
    return -1;
  const uint64_t G = 0x9E3779B97F4A7C15ULL;
  const int64_t max_slots = (int64_t)max_blocks * 16, nw = row_bytes / 8;
  for (int64_t u = 0; u < units; ++u) {
    int64_t n = seq_len[u];
    if (n < 0) n = 0;
    if (n > max_slots) n = max_slots;
    uint64_t d = 0;
    for (int64_t s = 0; s < n; ++s) {
      const int64_t blk = block_table[u * max_blocks + s / 16];
      if (blk < 0 || blk >= num_blocks || !live[u * max_slots + s]) continue;
      const int64_t row = blk * 16 + s % 16;
      uint64_t t = orc_fmix64((uint64_t)(uint32_t)pos[u * max_slots + s] ^ G);
      for (int64_t i = 0; i < nw; ++i) {
        t += orc_fmix64(row_word(k_pool, row, row_bytes, i) ^ ((uint64_t)(2 * i + 1) * G));
        t += orc_fmix64(row_word(v_pool, row, row_bytes, i) ^ ((uint64_t)(2 * i + 2) * G));
      }
      d += orc_fmix64(t);
    }
    digest[u] = d;
  }
  return 0;
}

int orc_vtok_check(const int32_t *block_table, const uint8_t *live, const int32_t *block_live,
                   int32_t units, int32_t max_blocks, int32_t num_blocks,
                   const int32_t *free_list, int32_t free_count, int64_t *out) {
  if (!block_table || !live || !block_live || !free_list || !out || num_blocks < 1 ||
      free_count < 0)
    return -1;
  int32_t *held = (int32_t *)calloc((size_t)num_blocks, sizeof(int32_t));
  out[0] = out[1] = out[2] = out[3] = 0;
  for (int64_t u = 0; u < units; ++u)
    for (int64_t lb = 0; lb < max_blocks; ++lb) {
      const int64_t e = block_table[u * max_blocks + lb];
      if (e < 0) continue;
      if (e >= num_blocks) {
        ++out[2];
      } else {
        ++held[e];
      }
      int64_t c = 0;
      for (int64_t o = 0; o < 16; ++o) c += live[(u * max_blocks + lb) * 16 + o] != 0;
      if (c != block_live[u * max_blocks + lb]) ++out[3];
    }
  for (int64_t i = 0; i < free_count; ++i) {
    const int64_t e = free_list[i];
    if (e < 0 || e >= num_blocks) {
      ++out[2];
    } else {
      ++held[e];
    }
  }
  for (int64_t b = 0; b < num_blocks; ++b) {
    if (held[b] > 1) ++out[0];
    if (held[b] == 0) ++out[1];
  }
  free(held);
  return 0;
}


/* ---- shared scores across the KV heads of a sequence ([H2O] Eq. for S_j) ---- */

int orc_select_shared(const float *scores, const int32_t *seq_len, const int32_t *pos, int32_t B,
                      int32_t Hkv, int32_t max_slots, int32_t budget, int32_t recent_window,
                      int32_t *victims, int32_t *n_victims) {
  if (!scores || !seq_len || !pos || !victims || !n_victims || B < 0 || Hkv < 1 ||
      max_slots < 1)
    return -1;
  if (budget <= 0 || recent_window < 0 || recent_window >= budget) return -1;
  float *row = (float *)malloc(sizeof(float) * (size_t)max_slots);
  int32_t *vic = (int32_t *)malloc(sizeof(int32_t) * (size_t)max_slots);
  for (int64_t b = 0; b < B; ++b) {
    const int64_t u0 = b * Hkv;
    const int32_t n = seq_len[u0];
    int ok = n >= 0 && n <= max_slots;
    for (int64_t h = 1; h < Hkv; ++h) ok = ok && seq_len[u0 + h] == n;
    for (int64_t s = 0; ok && s < n; ++s) {
      float acc = scores[u0 * max_slots + s];
      for (int64_t h = 1; h < Hkv; ++h) {
        acc = acc + scores[(u0 + h) * max_slots + s];
        if (pos[(u0 + h) * max_slots + s] != pos[u0 * max_slots + s]) ok = 0;
      }
      row[s] = acc;
    }
    int32_t m = -1;
    if (ok) orc_select(row, &n, 1, max_slots, budget, recent_window, vic, &m);
    for (int64_t h = 0; h < Hkv; ++h) {
      n_victims[u0 + h] = m;
      for (int64_t i = 0; i < m; ++i) victims[(u0 + h) * max_slots + i] = vic[i];
    }
  }
  free(row);
  free(vic);
  return 0;
}


/* ---- per-unit budgets ([H2O] asymmetric layer allocation) ---- */

int orc_select_budgets(const float *scores, const int32_t *seq_len, int32_t units,
                       int32_t max_slots, const int32_t *budget, const int32_t *recent_window,
                       int32_t *victims, int32_t *n_victims) {
  if (!scores || !seq_len || !budget || !recent_window || !victims || !n_victims) return -1;
  for (int64_t u = 0; u < units; ++u) {
    const int32_t b = budget[u], r = recent_window[u], n = seq_len[u];
    if (b <= 0 || r < 0 || r >= b || n < 0 || n > max_slots) {
      n_victims[u] = -1;
      continue;
    }
    orc_select(scores + u * (int64_t)max_slots, seq_len + u, 1, max_slots, b, r,
               victims + u * (int64_t)max_slots, n_victims + u);
  }
  return 0;
}


/* ---- SnapKV's decode-time ring buffer ([SNAP] "How it works") ---- */

typedef struct {
  int32_t pos;
  int64_t idx; /* slot, or -1 for the new token */
} by_pos;

static int by_pos_cmp(const void *a, const void *b) {
  const by_pos *x = (const by_pos *)a, *y = (const by_pos *)b;
  return (x->pos > y->pos) - (x->pos < y->pos);
}

int orc_ring_step(void *k_pool, void *v_pool, int32_t is_bf16, int32_t head_dim,
                  int32_t *block_table, int32_t *seq_len, int32_t *pos, float *hist,
                  int32_t *ring, int32_t *rank, int32_t batch, int32_t kv_heads,
                  int32_t max_blocks, int32_t num_blocks, int32_t group, const void *q,
                  const void *k_new, const void *v_new, const int32_t *t_pos,
                  const int32_t *observe, double scale, int32_t budget, int32_t recent,
                  int32_t obs_window, int32_t pool_kernel, int32_t *free_list,
                  int32_t *free_count, int32_t *evicted_pos) {
  if (!k_pool || !v_pool || !block_table || !seq_len || !pos || !hist || !ring || !rank || !q ||
      !k_new || !v_new || !t_pos || !observe || !free_list || !free_count || !evicted_pos)
    return -1;
  if (group < 1 || budget <= 0 || recent < 0 || recent >= budget || obs_window < 1) return -1;
  if (pool_kernel < 1 || pool_kernel % 2 == 0 || budget > max_blocks * 16) return -1;
  const int64_t D = head_dim, G = group, W = obs_window, max_slots = (int64_t)max_blocks * 16;
  const int64_t row_bytes = D * (is_bf16 ? 2 : 4), r = (pool_kernel - 1) / 2;
  double *s = (double *)malloc(sizeof(double) * (size_t)(G * (budget + 1)));
  double *lse = (double *)malloc(sizeof(double) * (size_t)G);
  float *S = (float *)malloc(sizeof(float) * (size_t)(budget + 1));
  float *pooled = (float *)malloc(sizeof(float) * (size_t)(budget + 1));
  by_pos *order = (by_pos *)malloc(sizeof(by_pos) * (size_t)(budget + 1));
  for (int64_t u = 0; u < (int64_t)batch * kv_heads; ++u) {
    const int64_t b = u / kv_heads, h = u % kv_heads;
    const int64_t n = seq_len[u], t = t_pos[b];
    int32_t *bt = block_table + u * max_blocks;
    int32_t *ps = pos + u * max_slots;
    float *hs = hist + u * W * max_slots; /* [W][max_slots] per head */
    if (n < 0 || n > budget || ring[u] < 0 || ring[u] >= W) {
      evicted_pos[u] = -2;
      continue;
    }
    int bad = 0;
    for (int64_t lb = 0; lb < (n + 15) / 16; ++lb)
      if (bt[lb] < 0 || bt[lb] >= num_blocks) bad = 1;
    const int need_block = n < budget && n % 16 == 0 && bt[n / 16] < 0;
    if (!need_block && n < budget && bt[n / 16] >= num_blocks) bad = 1;
    if (bad) {
      evicted_pos[u] = -4;
      continue;
    }
    if (need_block) {
      if (*free_count <= 0) {
        evicted_pos[u] = -3;
        continue;
      }
      const int32_t blk = free_list[--*free_count];
      if (blk < 0 || blk >= num_blocks) {
        evicted_pos[u] = -4;
        continue;
      }
      bt[n / 16] = blk;
    }
    /* the step's softmax over the cached tokens (pos <= t) and the new token */
    const char *knew = (const char *)k_new + u * row_bytes;
    for (int64_t g = 0; g < G; ++g) {
      const int64_t qrow = (b * kv_heads + h) * G + g;
      double mx = -INFINITY;
      for (int64_t j = 0; j <= n; ++j) {
        if (j < n && ps[j] > t) {
          s[g * (budget + 1) + j] = -INFINITY;
          continue;
        }
        const int64_t prow = j < n ? (int64_t)bt[j / 16] * 16 + j % 16 : -1;
        double acc = 0.0;
        for (int64_t d = 0; d < D; ++d) {
          const double kd = j < n ? widen(k_pool, is_bf16, prow * D + d) : widen(knew, is_bf16, d);
          acc += widen(q, is_bf16, qrow * D + d) * kd;
        }
        s[g * (budget + 1) + j] = scale * acc;
        if (s[g * (budget + 1) + j] > mx) mx = s[g * (budget + 1) + j];
      }
      double z = 0.0;
      for (int64_t j = 0; j <= n; ++j) z += exp(s[g * (budget + 1) + j] - mx);
      lse[g] = mx + log(z);
    }
    /* on_decode_step: the cached slots' weights into the ring, then advance */
    if (observe[b]) {
      for (int64_t j = 0; j < n; ++j) {
        double pj = 0.0;
        for (int64_t g = 0; g < G; ++g) pj += exp(s[g * (budget + 1) + j] - lse[g]);
        hs[(int64_t)ring[u] * max_slots + j] = (float)pj;
      }
      ring[u] = (int32_t)((ring[u] + 1) % W);
    }
    /* admit the new token with a zero ring; evict when over the budget */
    int64_t dst;
    int64_t kept_new = 1;
    if (n < budget) {
      dst = n;
      seq_len[u] = (int32_t)(n + 1);
      evicted_pos[u] = -1;
    } else {
      for (int64_t j = 0; j <= n; ++j) {
        float acc = 0.f;
        if (j < n)
          for (int64_t w = 0; w < W; ++w) acc = acc + hs[w * max_slots + j];
        S[j] = acc;
        order[j].pos = j < n ? ps[j] : (int32_t)t;
        order[j].idx = j < n ? j : -1;
      }
      qsort(order, (size_t)(n + 1), sizeof(by_pos), by_pos_cmp);
      /* max-pool over the neighbours in position order, clamped at both ends */
      for (int64_t k = 0; k <= n; ++k) {
        const int64_t lo = k - r > 0 ? k - r : 0, hi = k + r < n ? k + r : n;
        float m = S[order[lo].idx < 0 ? n : order[lo].idx];
        for (int64_t k2 = lo + 1; k2 <= hi; ++k2) {
          const float v = S[order[k2].idx < 0 ? n : order[k2].idx];
          if (v > m) m = v;
        }
        pooled[order[k].idx < 0 ? n : order[k].idx] = m;
      }
      int64_t best = -2;
      float bv = 0.f;
      int64_t bp = 0;
      for (int64_t j = 0; j <= n; ++j) {
        const int64_t pj = j < n ? ps[j] : t;
        if (t - pj < recent) continue;
        const cand a = {pooled[j], 0}, c = {bv, 0};
        int less;
        if (best == -2) {
          less = 1;
        } else {
          const int cmp = cand_cmp(&a, &c);
          less = cmp < 0 || (cmp == 0 && pj < bp);
        }
        if (less) {
          best = j < n ? j : -1;
          bv = pooled[j];
          bp = pj;
        }
      }
      if (best < 0) {
        evicted_pos[u] = (int32_t)t;
        kept_new = 0;
        dst = -1;
      } else {
        dst = best;
        evicted_pos[u] = ps[dst];
      }
    }
    if (kept_new) {
      const int64_t row = (int64_t)bt[dst / 16] * 16 + dst % 16;
      copy_row(k_pool, row, knew, row_bytes);
      copy_row(v_pool, row, (const char *)v_new + u * row_bytes, row_bytes);
      ps[dst] = (int32_t)t;
      for (int64_t w = 0; w < W; ++w) hs[w * max_slots + dst] = 0.f;
    }
    /* each slot's index in position order */
    const int64_t n2 = seq_len[u];
    for (int64_t j = 0; j < n2; ++j) {
      int32_t c = 0;
      for (int64_t i = 0; i < n2; ++i) c += ps[i] < ps[j];
      rank[u * max_slots + j] = c;
    }
  }
  free(order);
  free(pooled);
  free(S);
  free(lse);
  free(s);
  return 0;
}


/* ---- vToken's sync_new_tokens and slot mapping ([VTOK] section 3.2, Eq. 2) ---- */

int orc_vtok_sync(const int32_t *block_table, int32_t *seq_len, int32_t *pos, uint8_t *live,
                  int32_t *block_live, int32_t batch, int32_t kv_heads, int32_t max_blocks,
                  int32_t num_blocks, const int32_t *new_len, const int32_t *pos0,
                  int32_t *status) {
  if (!block_table || !seq_len || !pos || !live || !block_live || !new_len || !pos0 || !status)
    return -1;
  const int64_t max_slots = (int64_t)max_blocks * 16;
  for (int64_t u = 0; u < (int64_t)batch * kv_heads; ++u) {
    const int64_t b = u / kv_heads, n = seq_len[u], m = new_len[u];
    const int32_t *bt = block_table + u * max_blocks;
    if (n < 0 || m < n || m > max_slots) {
      status[u] = -2;
      continue;
    }
    int bad = 0;
    for (int64_t s = n; s < m; ++s)
      if (bt[s / 16] < 0 || bt[s / 16] >= num_blocks) bad = 1;
    if (bad) {
      status[u] = -4;
      continue;
    }
    for (int64_t s = n; s < m; ++s) {
      live[u * max_slots + s] = 1;
      pos[u * max_slots + s] = (int32_t)(pos0[b] + (s - n));
      block_live[u * max_blocks + s / 16] += 1;
    }
    seq_len[u] = (int32_t)m;
    status[u] = 0;
  }
  return 0;
}

int orc_vtok_slot_mapping(const int32_t *block_table, const int32_t *seq_len, const int32_t *pos,
                          const uint8_t *live, int32_t units, int32_t max_blocks,
                          int32_t num_blocks, int32_t *slots, int32_t *positions,
                          int32_t *count) {
  if (!block_table || !seq_len || !pos || !live || !slots || !positions || !count) return -1;
  const int64_t max_slots = (int64_t)max_blocks * 16;
  for (int64_t u = 0; u < units; ++u) {
    const int64_t n = seq_len[u];
    if (n < 0 || n > max_slots) {
      count[u] = -1;
      continue;
    }
    int64_t k = 0;
    for (int64_t s = 0; s < n; ++s) {
      const int64_t blk = block_table[u * max_blocks + s / 16];
      if (blk < 0 || blk >= num_blocks || !live[u * max_slots + s]) continue;
      slots[u * max_slots + k] = (int32_t)(blk * 16 + s % 16); /* Eq. 2 */
      positions[u * max_slots + k] = pos[u * max_slots + s];
      ++k;
    }
    count[u] = (int32_t)k;
  }
  return 0;
}
