/*
 * oracle.h -- plain CPU reference of attention-score KV-cache eviction.
 *
 * TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may call this library.  The product path (the HIP library
 * and its Python binding) never links, loads or calls it, and it shares no
 * code, header or table with that path.
 *
 * Everything is computed with scalar loops in double precision.  bf16 inputs
 * are widened exactly (bits << 16), fp32 inputs exactly.  Sources:
 *   [H2O]   "H2O Guide: Heavy Hitter Oracle KV Cache Eviction for LLMs"
 *   [SNAP]  "SnapKV" (policy book entry, decode-time adaptation)
 *   [VTOK]  "vToken: Turning Token-Level KV Eviction into Actually Reusable GPU Memory"
 *   [DROP]  "DropKV paper -- Residual-output perturbation scoring for KV-cache eviction"
 *
 * Cache layout (one layer): K and V pools of [num_blocks][16][head_dim]; the
 * slot s of KV head (b, h) lives in physical row
 *     block_table[b][h][s / 16] * 16 + s % 16          ([VTOK] section 3.4, Eq. 2)
 * pos[b][h][s] is the original position of slot s; slots are kept in
 * ascending position order.
 */
#ifndef KVEV_ORACLE_H
#define KVEV_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORC_SUM 1
#define ORC_POOL 2
#define ORC_DROP 4
#define ORC_ACCUMULATE 8

typedef struct {
  int32_t batch, kv_heads, head_dim, max_blocks, num_blocks, is_bf16;
  const void *k_pool, *v_pool;   /* [num_blocks][16][head_dim], fp32 or bf16 bits */
  const int32_t *block_table;    /* [batch][kv_heads][max_blocks] */
  const int32_t *seq_len;        /* [batch][kv_heads] */
  const int32_t *pos;            /* [batch][kv_heads][max_blocks*16] */
} orc_cache;

typedef struct {
  int32_t group, obs_window;     /* G query heads per KV head, W window queries */
  const void *q;                 /* [batch][kv_heads*group][W][head_dim], cache dtype */
  const float *lse;              /* [batch][kv_heads*group][W] */
  const float *a;                /* [batch][kv_heads*group][W][head_dim], fp32 (the
                                    forward pass's output, whatever the cache dtype) */
  const int32_t *q_pos;          /* [batch][W] */
  double scale;                  /* multiplies q.k before the LSE is subtracted (the
                                    callers pass the fp32 value the library gets) */
} orc_window;

/* Input builder (not the method): LSE and attention output of each window
 * query over the keys it attends (pos <= q_pos).  lse_out [B][Hq][W],
 * a_out [B][Hq][W][D] (may be NULL).  unit_mask [B*Hkv] selects KV heads (NULL = all). */
int orc_lse_a(const orc_cache *c, const orc_window *w, double *lse_out, double *a_out,
              const uint8_t *unit_mask, int nthreads);

/* Per-token scores of every live slot; outputs [B][Hkv][max_blocks*16] in
 * double, entries at slots >= seq_len untouched.  prev_sum (fp32) is read in
 * ACCUMULATE mode.  Returns 0, or -1 on invalid arguments. */
int orc_score(const orc_cache *c, const orc_window *w, int flags, int pool_kernel,
              const float *prev_sum, double *sum, double *pooled, double *drop,
              const uint8_t *unit_mask, int nthreads);

/* Victims of every KV head from fp32 scores [B][Hkv][max_slots].
 * victims [B][Hkv][max_slots] (first n_victims entries valid, ascending slots). */
int orc_select(const float *scores, const int32_t *seq_len, int32_t units, int32_t max_slots,
               int32_t budget, int32_t recent_window, int32_t *victims, int32_t *n_victims);

/* Selection with one score per token shared by all KV heads of a sequence
 * ([H2O] "Formulating Cumulative Attention Scores": S_j sums the attention
 * of every head of the layer).  scores: fp32 [B][Hkv][max_slots] per-head
 * rows.  The shared row of sequence b adds its heads' rows in fp32, heads in
 * ascending order (the precision and order in which the library takes the
 * same decision), then orc_select runs on it; every head of the sequence gets
 * its victims.  Heads of a sequence whose seq_len differ, or whose pos differ
 * at a slot below it, or a length outside [0, max_slots]: n_victims = -1 on
 * every head of the sequence.  Returns 0 or -1 (invalid arguments). */
int orc_select_shared(const float *scores, const int32_t *seq_len, const int32_t *pos, int32_t B,
                      int32_t Hkv, int32_t max_slots, int32_t budget, int32_t recent_window,
                      int32_t *victims, int32_t *n_victims);

/* orc_select with a (budget, recent_window) pair per unit; a unit whose pair
 * is invalid (budget <= 0, recent < 0, recent >= budget) or whose seq_len is
 * outside [0, max_slots] gets n_victims = -1.  Returns 0 or -1. */
int orc_select_budgets(const float *scores, const int32_t *seq_len, int32_t units,
                       int32_t max_slots, const int32_t *budget, const int32_t *recent_window,
                       int32_t *victims, int32_t *n_victims);

/* One decode step of SnapKV's ring-buffer adaptation for every KV head
 * ([SNAP] "How it works", "On the adaptation", "Parameters").  Per slot the
 * cache keeps a ring of the last obs_window observed attention weights,
 * hist [batch][kv_heads][obs_window][max_blocks*16] fp32 (ring index major,
 * so one index of every slot is contiguous), and ring
 * [batch][kv_heads] the ring index written next.  The new token of sequence
 * b (position t_pos[b]; k_new, v_new, q as in orc_h2o_step) attends to the
 * cached tokens with pos <= t and to itself; the weight of cached token j is
 * the group sum of its softmax probabilities, rounded to fp32.  When
 * observe[b] is nonzero, every cached slot's weight goes to its ring at
 * index ring[u] and the index advances modulo obs_window; a null step
 * (observe[b] == 0) writes nothing and leaves the index.  The new token is
 * then admitted with an all-zero ring.  Below the budget it is appended (a
 * block popped from the free list when needed).  At the budget one of the
 * n + 1 tokens is dropped: with sums S = the fp32 sum of each ring, index 0
 * upward (0 for the new token), and the tokens taken in position order,
 * pooled = the max of S over the poolKernel tokens centred on each (clamped
 * at both ends); the victim is the smallest (pooled, position) among the
 * tokens at least `recent` positions older than t (the new token included
 * when recent == 0).  A cached victim's slot receives the new token (K, V,
 * pos, a zero ring); a dropped new token leaves the cache as it was.
 * rank [batch][kv_heads][max_blocks*16] is written for the slots below the
 * new length: each slot's index in position order.  evicted_pos as in
 * orc_h2o_step (-1 appended, the dropped position, or -2 / -3 / -4 with the
 * head unchanged, rings included).  Returns 0, or -1 on invalid arguments
 * (recent >= budget, obs_window < 1, an even or non-positive pool_kernel). */
int orc_ring_step(void *k_pool, void *v_pool, int32_t is_bf16, int32_t head_dim,
                  int32_t *block_table, int32_t *seq_len, int32_t *pos, float *hist,
                  int32_t *ring, int32_t *rank, int32_t batch, int32_t kv_heads,
                  int32_t max_blocks, int32_t num_blocks, int32_t group, const void *q,
                  const void *k_new, const void *v_new, const int32_t *t_pos,
                  const int32_t *observe, double scale, int32_t budget, int32_t recent,
                  int32_t obs_window, int32_t pool_kernel, int32_t *free_list,
                  int32_t *free_count, int32_t *evicted_pos);

/* In-place, order-preserving compaction of every KV head; frees emptied tail
 * blocks to the free list.  elem_bytes is 4 (fp32) or 2 (bf16).  score may be
 * NULL.  stats[5] = {blocks_freed, rows_moved, bytes_moved, at_risk_rows, status}.
 * Returns 0, -1 (invalid) or -2 (free list too small; nothing modified). */
int orc_compact(void *k_pool, void *v_pool, int32_t elem_bytes, int32_t head_dim,
                int32_t *block_table, int32_t *seq_len, int32_t *pos, float *score,
                int32_t units, int32_t max_blocks, const int32_t *victims,
                const int32_t *n_victims, int32_t *free_list, int32_t *free_count,
                int32_t free_capacity, int64_t *stats);

/* Block-level waste of an eviction ([VTOK] section 2, Eq. 1 and Fig. 1).
 * out[8] = {F_naive, F_after, frac_le_half_naive, frac_le_half_after,
 *           blocks_naive, blocks_after, live_tokens, blocks_freed}. */
int orc_measure(const int32_t *seq_len_before, const int32_t *victims, const int32_t *n_victims,
                int32_t units, int32_t max_slots, double *out);

/* One H2O decode step of every KV head ([H2O] "Step-by-Step Eviction
 * Lifecycle" and "PagedAttention Memory Integration").  The new token of
 * sequence b sits at position t_pos[b]; its key and value k_new / v_new are
 * [batch][kv_heads][head_dim] and its G query rows q [batch][kv_heads*G][head_dim]
 * (cache dtype).  The query attends to every cached token with pos <= t and to
 * itself; score [batch][kv_heads][max_blocks*16] is the running fp32 score.
 * Below the budget the token is appended (a block popped from the free list
 * when its logical block has none); at the budget the smallest (score, pos)
 * among the tokens at least `recent` positions older than t (the new token
 * included when recent == 0) is evicted and the new token overwrites its
 * slot.  evicted_pos[u] = -1 (appended), the evicted position (t when the
 * new token itself was dropped, or no cached token is a candidate), or -2
 * (n < 0 or n > budget), -3 (no free block), -4 (block id out of range; a
 * bad id taken from the free list stays taken): on a negative code other
 * than -1 the head is left unchanged.  attn_out (may be NULL): the step's
 * attention output of each query row, sum_j p_j v_j over the same keys and
 * the new token ([B][kv_heads*G][head_dim], double, written for the heads
 * that are not refused); attn_abs (may be NULL): sum_j p_j |v_j| alike, the
 * scale of its rounding error.  Returns 0, or -1 on invalid arguments. */
int orc_h2o_step(void *k_pool, void *v_pool, int32_t is_bf16, int32_t head_dim,
                 int32_t *block_table, int32_t *seq_len, int32_t *pos, float *score,
                 int32_t batch, int32_t kv_heads, int32_t max_blocks, int32_t num_blocks,
                 int32_t group, const void *q, const void *k_new, const void *v_new,
                 const int32_t *t_pos, double scale, int32_t budget, int32_t recent,
                 int32_t *free_list, int32_t *free_count, int32_t *evicted_pos,
                 double *attn_out, double *attn_abs);

/* vToken liveness ([VTOK] section 3.2): mark the victim slots of every head
 * dead.  live [units][max_blocks*16] (1 live, 0 dead), block_live
 * [units][max_blocks] (live slots per logical block).  A victim that is out
 * of range, not live or in a block without a physical block sets bit 0 of
 * *status and is skipped. */
int orc_vtok_evict(const int32_t *block_table, const int32_t *seq_len, uint8_t *live,
                   int32_t *block_live, int32_t units, int32_t max_blocks,
                   const int32_t *victims, const int32_t *n_victims, int32_t *status);

/* vToken lazy reclamation ([VTOK] section 3.3, stages 1-3, and section 3.5,
 * I1, I2, I4), one call over every head in (b, h) order:
 *   - eligibility: the head's waste F = 1 - live / (16 * allocated blocks)
 *     (Eq. 1 over the head) above theta_f;
 *   - sources: the first max_sources allocated, not full blocks in logical
 *     order, the block holding the head's last slot excluded (it still takes
 *     appends);
 *   - T = their live tokens; the plan needs D = ceil(T / 16) destination
 *     blocks and proceeds only if D < the number of sources;
 *   - headroom: D blocks from the top of the free list while enough remain;
 *     a head that does not fit is deferred;
 *   - moves: the sources' live tokens in logical order fill the destination
 *     blocks completely, one after the other; the first D source positions of
 *     the block list take the destination blocks, the other source positions
 *     become -1 (so the moved tokens keep their relative order, passing over
 *     any full block between two sources); K, V, pos, live, block_live and
 *     the optional score row follow; after every head has planned, the source
 *     blocks are appended to the free list in (b, h, block) order.
 * stats[10] = {heads reclaimed, heads deferred, heads left as they are (waste
 * at or below theta_f, or no plan that frees a block), blocks freed, rows
 * moved, bytes moved (K+V read+write), live tokens, allocated blocks before,
 * after, status (an OR of 2: a seq_len out of range, 4: a block id past the
 * pool or a live count outside [0, 16]; such heads are skipped and not
 * counted)}.  Returns 0, -1 (invalid),
 * -2 (free list capacity too small; nothing modified). */
int orc_vtok_reclaim(void *k_pool, void *v_pool, int32_t elem_bytes, int32_t head_dim,
                     int32_t *block_table, const int32_t *seq_len, int32_t *pos, float *score,
                     uint8_t *live, int32_t *block_live, int32_t units, int32_t max_blocks,
                     int32_t num_blocks, double theta_f, int32_t max_sources,
                     int32_t *free_list, int32_t *free_count, int32_t free_capacity,
                     int64_t *stats);

/* vToken's sync_new_tokens ([VTOK] section 3.2: the scheduler passes the
 * current block list and length; the table gives the new tokens sequential
 * logical IDs at their physical positions).  For every head u with
 * n = seq_len[u] and m = new_len[u]: the slots [n, m) become live, slot s
 * takes position pos0[b] + (s - n), each block's live count grows by its new
 * slots, and seq_len[u] = m.  status[u] = 0, or -2 (m < n or m above the
 * capacity), -4 (a block of [n, m) without an id in [0, num_blocks)); a head
 * with a nonzero status is left unchanged.  Returns 0 or -1. */
int orc_vtok_sync(const int32_t *block_table, int32_t *seq_len, int32_t *pos, uint8_t *live,
                  int32_t *block_live, int32_t batch, int32_t kv_heads, int32_t max_blocks,
                  int32_t num_blocks, const int32_t *new_len, const int32_t *pos0,
                  int32_t *status);

/* vToken's BuildSlotMapping ([VTOK] Eq. 2 and Algorithm 1, step 4): for every
 * head, the live tokens below seq_len in logical order, each as its physical
 * slot block_id * 16 + offset (slots [units][max_slots]) and its position
 * (positions [units][max_slots]); count[u] of them.  Slots in blocks without
 * an id in [0, num_blocks) are skipped; a seq_len outside [0, max_slots]
 * gives count -1.  Returns 0 or -1. */
int orc_vtok_slot_mapping(const int32_t *block_table, const int32_t *seq_len, const int32_t *pos,
                          const uint8_t *live, int32_t units, int32_t max_blocks,
                          int32_t num_blocks, int32_t *slots, int32_t *positions,
                          int32_t *count);

/* The online checks of I1 and I2 ([VTOK] section 3.5: token conservation and
 * unique mapping are verified at every relocation by hashing and comparing).
 *
 * orc_vtok_digest: per head, an order-independent digest of its live tokens:
 * the sum (mod 2^64) over live slots s < seq_len (seq_len clamped to
 * [0, max_blocks*16]) in blocks whose id lies in [0, num_blocks) of
 * fmix64(t), where
 *   t = fmix64(pos ^ G) + sum_i fmix64(k_i ^ (2i+1) G) + sum_i fmix64(v_i ^ (2i+2) G)
 * (mod 2^64), pos zero-extended from 32 bits, k_i and v_i the row's
 * little-endian 64-bit words, G = 0x9E3779B97F4A7C15, and fmix64 the
 * 64-bit finalizer of Appleby's MurmurHash3.  A token keeps its digest
 * wherever it is stored; any change of a live token's position, K or V
 * changes the head's digest with overwhelming probability.
 *
 * orc_vtok_check: out[4] = {pool blocks held more than once, pool blocks held
 * by nobody, references out of range, live-count mismatches}, counting as
 * holders every table entry >= 0 of every head (all max_blocks entries) and
 * free_list[0, *free_count).  A table entry >= num_blocks or a list entry
 * outside [0, num_blocks) is out of range.  A mismatch is an entry >= 0 whose
 * block_live differs from its number of nonzero live bytes.  I2 holds when
 * the first three are 0.  Returns 0, or -1 for invalid arguments. */
uint64_t orc_fmix64(uint64_t k);
int orc_vtok_digest(const void *k_pool, const void *v_pool, int32_t row_bytes,
                    const int32_t *block_table, const int32_t *seq_len, const int32_t *pos,
                    const uint8_t *live, int32_t units, int32_t max_blocks, int32_t num_blocks,
                    uint64_t *digest);
int orc_vtok_check(const int32_t *block_table, const uint8_t *live, const int32_t *block_live,
                   int32_t units, int32_t max_blocks, int32_t num_blocks,
                   const int32_t *free_list, int32_t free_count, int64_t *out);

#ifdef __cplusplus
}
#endif
#endif
