/*
 * kvev.h -- attention-score KV-cache eviction on MI355X (gfx950): score,
 * select and compact one layer's paged KV cache.
 *
 * Sources (cited by page title and section):
 *   [H2O]  "H2O Guide: Heavy Hitter Oracle KV Cache Eviction for LLMs"
 *   [SNAP] "SnapKV" (policy book entry)
 *   [VTOK] "vToken: Turning Token-Level KV Eviction into Actually Reusable GPU Memory"
 *   [DROP] "DropKV paper -- Residual-output perturbation scoring for KV-cache eviction"
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every data pointer is a DEVICE pointer owned by the caller (for example a
 *   torch tensor's data_ptr()).  The library allocates nothing, frees nothing
 *   and keeps no state of its own (what persists between calls lives in the
 *   caller's workspace); calls on different workspaces are independent.  The
 *   one exception is kvev_evict_noalloc, whose workspace is a static device
 *   array per GPU (its address is looked up once per device and kept).
 * - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Each
 *   call only enqueues work on that stream and never synchronises.  Calls that
 *   share a workspace or touch the same cache must be ordered on one stream.
 * - Return value: KVEV_OK, or a negative kvev_status.  Argument errors are
 *   detected on the host BEFORE anything is enqueued, so a refused call leaves
 *   every buffer untouched.  Inconsistent device-resident data (for example a
 *   seq_len above the head's capacity, or victims not strictly ascending) is
 *   detected by the kernels: the affected head is left unchanged and a bit is
 *   set in stats[4] of kvev_compact; kvev_score skips the head and kvev_select
 *   sets its n_victims to -1.
 * - Block size is fixed at 16 tokens ([VTOK] section 2 and section 5's block
 *   size sensitivity; [H2O] "PagedAttention Memory Integration").
 * - Workspace: one caller-owned device buffer of kvev_workspace_bytes() bytes
 *   serves every entry point of a cache shape.  ZERO-FILL IT ONCE before its
 *   first use: its leading part holds state (selection histograms, per-head
 *   compaction accumulators) that kvev_select, kvev_compact and kvev_evict
 *   expect to be zero and leave zero when their work completes; the rest is
 *   scratch.  Do not modify it between calls; calls sharing it must be
 *   ordered on one stream.  After a KVEV_EDEVICE return, zero it again.
 *   The vToken entry points size their workspace with their own queries
 *   (kvev_vtok_*_workspace_bytes) and write only past that state part, so
 *   one buffer of the larger size may serve both; kvev_h2o_step's workspace
 *   is its own (see there).
 *
 * Cache layout (one layer)
 * ------------------------
 * k_pool, v_pool: [num_blocks][16][head_dim] in the cache dtype (fp32 or
 * bf16).  Each (batch b, KV head h) owns a list of blocks; logical slot s of
 * that head lives in physical row
 *     block_table[b][h][s / 16] * 16 + s % 16          ([VTOK] section 3.4, Eq. 2)
 * seq_len[b][h] = n live slots; pos[b][h][s] = original token position of slot
 * s.  Slots are in ascending position order (compaction keeps it), except
 * after kvev_h2o_step, which places each new token in the slot it frees.
 */
#ifndef KVEV_H
#define KVEV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVEV_BLOCK_SIZE 16
#define KVEV_ABI_VERSION 17
/* bytes of the static device array kvev_evict_noalloc works in, per GPU */
#define KVEV_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)

typedef enum {
  KVEV_OK = 0,
  KVEV_EINVAL = -1,       /* bad argument: NULL, bad shape, refused parameter */
  KVEV_ENOSPACE = -2,     /* workspace or free list too small */
  KVEV_EUNSUPPORTED = -3, /* dtype / head_dim / row count the kernels lack */
  KVEV_EDEVICE = -4       /* a HIP launch or query failed */
} kvev_status;

typedef enum { KVEV_F32 = 0, KVEV_BF16 = 1 } kvev_dtype;

/* score kinds (flags of kvev_score) */
enum {
  KVEV_SUM = 1,        /* H2O accumulated attention / SnapKV window sum */
  KVEV_POOL = 2,       /* SnapKV window sum followed by the 1-D max-pool */
  KVEV_DROP = 4,       /* DropKV residual score */
  KVEV_ACCUMULATE = 8  /* add the window sum to the values already in `sum` */
};

typedef struct kvev_cache {
  int32_t batch;        /* B */
  int32_t kv_heads;     /* Hkv */
  int32_t head_dim;     /* D: 64 or 128 */
  int32_t block_size;   /* must be 16 */
  int32_t max_blocks;   /* block-table entries per head; capacity = max_blocks*16 slots */
  int32_t num_blocks;   /* physical blocks in each pool */
  int32_t dtype;        /* kvev_dtype of k_pool, v_pool, q and a */
  void *k_pool;         /* [num_blocks][16][head_dim] */
  void *v_pool;         /* [num_blocks][16][head_dim] */
  int32_t *block_table; /* [batch][kv_heads][max_blocks]; -1 = no block */
  int32_t *seq_len;     /* [batch][kv_heads] live slots per head */
  int32_t *pos;         /* [batch][kv_heads][max_blocks*16] original positions */
} kvev_cache;

typedef struct kvev_window {
  int32_t group;        /* G query heads per KV head (GQA), >= 1 */
  int32_t obs_window;   /* W window queries per query head, >= 1 */
  const void *q;        /* [batch][kv_heads*group][W][head_dim], cache dtype */
  const float *lse;     /* [batch][kv_heads*group][W]: log-sum-exp of scale*q.k */
  const float *a;       /* [batch][kv_heads*group][W][head_dim], fp32 (the forward
                           pass's attention output, whatever the cache dtype); DROP only */
  const int32_t *q_pos; /* [batch][W] positions of the window queries (causal mask) */
  float scale;          /* softmax scale applied to q.k, usually 1/sqrt(head_dim) */
} kvev_window;

/*
 * kvev_score -- per-token scores of every live slot of every KV head.
 *
 * Attention probability of window query (g, w) of KV head (b, h) for slot j
 * ([H2O] "The Existence of Heavy Hitters"; [DROP] Jargon, "Log-sum-exp"):
 *     p = exp(scale * q.k_j - lse)   if pos[j] <= q_pos[w], else 0.
 * The sums run over the G query heads of the group ([H2O] FAQ on GQA) and the
 * W window queries:
 *   KVEV_SUM:  sum[j]  = sum_{w,g} p          ([H2O] "Formulating Cumulative
 *              Attention Scores"; [SNAP] window sums)
 *              with KVEV_ACCUMULATE: sum[j] += sum_{w,g} p ([H2O] lifecycle,
 *              "Score Accumulation"); then sum must hold the previous scores.
 *   KVEV_POOL: pooled[j] = max over i in [j-r, j+r] clamped to [0, n-1] of
 *              sum_{w,g} p at i, r = (pool_kernel-1)/2 ([SNAP] "How it works").
 *   KVEV_DROP: drop[j] = sum_{w,g} p/(1-p) * ||a_{g,w} - v_j|| ([DROP] Lemma 1
 *              and the window sum), +inf for a term with p >= 1.  Terms
 *              with p >= 1/4 are computed in double from the rows (the
 *              term's rounding error grows as 1/(1-p)); the others in fp32,
 *              a.v from a's bf16 high and low parts on bf16 caches.
 * Outputs are fp32 [batch][kv_heads][max_blocks*16]; only slots [0, n) are
 * written.  Pass NULL for kinds not requested.  Reductions use a fixed order:
 * results are bitwise reproducible run to run.
 * Errors (KVEV_EINVAL): NULL cache/window/q/lse/q_pos; head_dim not 64/128;
 * block_size != 16; group < 1; obs_window < 1 ([SNAP] Parameters: a zero
 * window is refused); flags empty or unknown; POOL without `pooled`, or
 * pool_kernel < 1 or even ([SNAP] Parameters); DROP without `a` or `drop`;
 * SUM without `sum`; ACCUMULATE without SUM or combined with POOL or DROP.
 * KVEV_EUNSUPPORTED: group*obs_window above 4096.  Window rows that do not
 * fit a workgroup's 160 KB of LDS beside a 16-block tile (bf16, head_dim
 * 128: about 540 rows, 180 with DROP) are split over several workgroups per
 * tile; their raw sums then go to `workspace` past the part the other entry
 * points use (16-byte aligned, kvev_workspace_bytes(cache, group,
 * obs_window) bytes, else KVEV_ENOSPACE).  Windows that fit use no
 * workspace; `workspace` may then be NULL.
 */
int kvev_score(const kvev_cache *cache, const kvev_window *win, int32_t flags,
               int32_t pool_kernel, float *sum, float *pooled, float *drop, void *workspace,
               size_t ws_bytes, void *stream);

/*
 * kvev_select -- each KV head's victims under a budget.
 *
 * With n = seq_len[b][h]: m = max(0, n - budget) tokens are evicted (the
 * budget counts the recent window: [H2O] "Dual-Pool Budget Partitioning").
 * Candidates are slots [0, n - recent_window): the newest recent_window slots
 * are protected ([H2O] lifecycle; [SNAP] "drop the lowest outside the recent
 * window").  The m candidates with the smallest (score, position) are chosen:
 * equal scores evict the lower position ([SNAP] "Tie-breaking"), -0 equals +0
 * and NaN ranks above +inf.  victims[b][h][0..m) receives their slot indices
 * in ascending order, n_victims[b][h] = m.  score: fp32 [batch][kv_heads]
 * [max_blocks*16], 16-byte aligned (for example `pooled` of kvev_score); victims: int32 with
 * the same shape; n_victims: int32 [batch][kv_heads].  Bit-exact: the result
 * depends only on the score bits.
 * Errors (KVEV_EINVAL): NULL pointers; a score pointer not 16-byte aligned; budget <= 0; recent_window < 0 or
 * recent_window >= budget ([SNAP] Parameters); KVEV_ENOSPACE for a missing or
 * short workspace; KVEV_EUNSUPPORTED above 1M slots per head.
 */
int kvev_select(const kvev_cache *cache, const float *score, int32_t budget,
                int32_t recent_window, int32_t *victims, int32_t *n_victims, void *workspace,
                size_t ws_bytes, void *stream);

/*
 * kvev_select_budgets -- kvev_select with a budget and a recent window per
 * KV head: budget and recent_window are int32 [batch][kv_heads] on the
 * device.  For asymmetric allocations across layers ([H2O] "Asymmetric
 * Layer Allocation": larger recent windows in early layers, larger heavy
 * hitter pools in deep ones), the layers of a model can be stacked along the
 * batch axis of one cache so that a single call serves them all, each with
 * its own pair.  A head whose pair is invalid (budget <= 0, recent_window < 0
 * or recent_window >= budget) gets n_victims -1, as does an inconsistent
 * seq_len.  Same workspace as kvev_select (kvev_workspace_bytes).
 * Errors: KVEV_EINVAL for NULL pointers, a bad cache or a misaligned score;
 * KVEV_EUNSUPPORTED above 1M slots per head; KVEV_ENOSPACE.
 */
int kvev_select_budgets(const kvev_cache *cache, const float *score, const int32_t *budget,
                        const int32_t *recent_window, int32_t *victims, int32_t *n_victims,
                        void *workspace, size_t ws_bytes, void *stream);

/*
 * kvev_select_shared -- victim selection with one score shared by all KV
 * heads of a sequence ([H2O] "Formulating Cumulative Attention Scores": a
 * token's cumulative score sums the attention of every head of the layer;
 * the page's cache class keeps one score per token for the batch row).
 * score: fp32 [batch][kv_heads][max_blocks*16] per-head scores (each
 * already summed over its GQA group, e.g. from kvev_score), 16-byte
 * aligned.  For every sequence b the shared row is
 *   S_b[s] = score[b][0][s] + score[b][1][s] + ... + score[b][kv_heads-1][s]
 * in fp32, heads in ascending order, and kvev_select's rule runs on it once
 * (m = max(0, n - budget) victims among the slots [0, n - recent_window), the
 * m smallest (S, slot) pairs, ascending).  Every head of the sequence
 * receives the same victims: victims int32 [batch][kv_heads][max_blocks*16]
 * and n_victims int32 [batch][kv_heads], ready for kvev_compact.  The heads
 * of a sequence must hold the same tokens in the same slots: when their
 * seq_len differ, or their pos differ at any slot below it, n_victims is -1
 * on every head of the sequence.  Workspace: kvev_select_shared_workspace_bytes
 * (scratch only; no clearing needed), 16-byte aligned.  Six kernels on
 * `stream`.
 * Errors: as kvev_select (KVEV_EINVAL, KVEV_EUNSUPPORTED above 1M slots per
 * head, KVEV_ENOSPACE).
 */
int kvev_select_shared(const kvev_cache *cache, const float *score, int32_t budget,
                       int32_t recent_window, int32_t *victims, int32_t *n_victims,
                       void *workspace, size_t ws_bytes, void *stream);

/* Workspace bytes of kvev_select_shared; 0 for a bad cache. */
size_t kvev_select_shared_workspace_bytes(const kvev_cache *cache);

/*
 * kvev_compact -- remove the victims and repack each KV head in place.
 *
 * Kept slots keep their order: kept slot s with rank r moves to slot r (K row,
 * V row, pos, and score_or_null's entry), n becomes n' = n - n_victims
 * ([H2O] "PagedAttention Memory Integration": in-place overwrite within the
 * existing pages; [VTOK] section 3.3, stage 3: fill destinations fully, keep
 * logical order).  The blocks at logical indices [ceil(n'/16), ceil(n/16))
 * are then empty: their ids are appended to free_list in (b, h, logical
 * block) order at free_list[*free_count ...], *free_count grows by their
 * number, and their block_table entries become -1 ([VTOK] section 1: emptied
 * blocks return to the free pool).  Slots [n', ceil(n'/16)*16) hold
 * unspecified data afterwards.
 * victims/n_victims: as written by kvev_select (ascending, inside [0, n)).
 * free_list: int32 [free_capacity] device array; free_count: one int32 on
 * the device.  At most 4096 KV heads (batch * kv_heads) per call.  stats: int64[5] on the device = {blocks_freed, rows_moved,
 * bytes_moved (K and V rows moved, read + write), at_risk_rows (kept rows
 * whose source lies inside the compacted range), status (0, or a bit set per
 * inconsistent head: bit 0 victims not ascending / out of range, bit 1
 * seq_len above capacity)}.  The at-risk rows of a head are staged through
 * the workspace when there are at most 4096 of them; a head with more is
 * moved by one workgroup in ascending rounds of destination ranks, each
 * round's rows all read before any is written, so the workspace holds at
 * most 4096 staged rows a head.
 * Errors: KVEV_EINVAL for NULL pointers or a bad cache; KVEV_ENOSPACE when
 * free_capacity < num_blocks (the list must be able to hold the whole pool)
 * or ws_bytes < kvev_workspace_bytes(cache, 1, 1); KVEV_EUNSUPPORTED above 4096
 * KV heads or 1M slots per head.
 */
int kvev_compact(const kvev_cache *cache, const int32_t *victims, const int32_t *n_victims,
                 float *score_or_null, int32_t *free_list, int32_t *free_count,
                 int32_t free_capacity, int64_t *stats, void *workspace, size_t ws_bytes,
                 void *stream);

/*
 * kvev_evict -- one whole eviction step: kvev_score with `flags`, then
 * kvev_select on that score, then kvev_compact with the score as
 * score_or_null, with the same results as those three calls ([SNAP] "How it
 * works": score the window, keep the top budget, drop the rest; [VTOK]
 * section 3.3 for the repack).  Two launches: the scoring pass (which also
 * builds each head's selection histogram), then one launch that finds each
 * head's exact threshold, writes the victims and compacts the head in place
 * without staging any row.
 * flags: exactly one of KVEV_SUM, KVEV_POOL, KVEV_DROP (KVEV_ACCUMULATE with
 * KVEV_SUM); score: fp32 [batch][kv_heads][max_blocks*16], 16-byte aligned.
 * On entry it matters only with ACCUMULATE (the running sums).  On return its
 * slots [0, n') hold the kept tokens' scores in their compacted order; its
 * slots from n' on are unspecified.  victims, n_victims, free_list,
 * free_count, stats: as written by kvev_select and kvev_compact (stats[3]
 * counts the kept rows below n' that move, as kvev_compact does, though
 * none is staged), plus status bit 8 if a wait between workgroups reached
 * its spin limit (never expected).  Errors: the union of those three calls'
 * (KVEV_EINVAL also for several score kinds in flags or a workspace off 16
 * bytes); workspace: kvev_workspace_bytes(cache, 0, 0) bytes, as for
 * kvev_compact.  The workspace's state part also holds the pass's ticket and
 * arrival counters: after a KVEV_EDEVICE return, zero it again.
 */
int kvev_evict(const kvev_cache *cache, const kvev_window *win, int32_t flags,
               int32_t pool_kernel, int32_t budget, int32_t recent_window, float *score,
               int32_t *victims, int32_t *n_victims, int32_t *free_list, int32_t *free_count,
               int32_t free_capacity, int64_t *stats, void *workspace, size_t ws_bytes,
               void *stream);

/*
 * kvev_evict_noalloc -- kvev_evict for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments (minus the workspace), results and errors
 * as kvev_evict; the same two kernels run, plus one fill kernel first.
 * It allocates nothing: its workspace is a static device array of
 * KVEV_NOALLOC_SCRATCH_BYTES (128 MiB) that every GPU the library runs on
 * holds until the process ends.  The array keeps the last call's contents;
 * each call zeroes the part that must start at zero (the selection state and
 * the pass's counters) with the fill kernel, so no earlier call, failed or
 * not, leaves anything behind.
 * Limit: the pass needs its state plus 12 bytes per slot of every head
 * (batch * kv_heads * max_blocks * 16 slots), plus 4 * P more per slot when
 * the window's rows are too many for one workgroup's LDS and are split over
 * P workgroups per tile (large DropKV windows, as kvev_score describes); a
 * shape that needs more than the array returns KVEV_ENOSPACE before any work
 * is enqueued.  Example: 32 heads of 32768 slots need 12.6 MB.
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (two streams, two host threads) race and corrupt each other's results,
 * so order them.  The device current at the call must be the stream's; the
 * first call on a device looks the array's address up (hipGetSymbolAddress)
 * and keeps it: make that first call outside graph capture.
 */
int kvev_evict_noalloc(const kvev_cache *cache, const kvev_window *win, int32_t flags,
                       int32_t pool_kernel, int32_t budget, int32_t recent_window, float *score,
                       int32_t *victims, int32_t *n_victims, int32_t *free_list,
                       int32_t *free_count, int32_t free_capacity, int64_t *stats,
                       void *stream);

/*
 * kvev_measure -- block-level waste of an eviction ([VTOK] section 2, Eq. 1
 * and Fig. 1: F = 1 - live tokens / (blocks * 16), and the share of blocks at
 * half use or less).
 *
 * For every KV head u with a consistent record (0 <= n <= max_slots, 0 <= m
 * <= n, where n = seq_len_before[u] and m = n_victims[u]):
 *   before compaction ("naive" eviction, emptied slots stay in their blocks)
 *   block b of [0, ceil(n/16)) holds min(16, n - 16b) slots, minus the victims
 *   among them; after compaction the n' = n - m kept tokens fill
 *   ceil(n'/16) blocks from the front.
 * out: int64[6] on the device = {live tokens (sum of n'), blocks before,
 * blocks after, blocks before with 2 * live <= 16, blocks after with
 * 2 * live <= 16, blocks freed}.  F_naive = 1 - out[0] / (16 * out[1]),
 * F_after = 1 - out[0] / (16 * out[2]).  Heads with an inconsistent record
 * add nothing.  seq_len_before: int32 [units] (the lengths before
 * kvev_compact or kvev_evict); victims: int32 [units][max_slots], ascending
 * per head as kvev_select writes them; n_victims: int32 [units].  All device
 * pointers; the call only enqueues (two kernels) on `stream`.
 * Errors: KVEV_EINVAL for NULL pointers, units < 0 or max_slots not a
 * positive multiple of 16.
 */
int kvev_measure(const int32_t *seq_len_before, const int32_t *victims,
                 const int32_t *n_victims, int32_t units, int32_t max_slots, int64_t *out,
                 void *stream);

/*
 * kvev_h2o_step -- one H2O decode step of every KV head ([H2O] "Step-by-Step
 * Eviction Lifecycle"; "PagedAttention Memory Integration" for the in-place
 * overwrite).  Sequence b's new token sits at position t_pos[b].  For each KV
 * head u = (b, h) with n = seq_len[u] tokens:
 *   - the token's G query rows attend to every cached token with pos <= t
 *     and to the token itself: p_g,j = exp(scale * q_g.k_j - lse_g), lse_g
 *     the log-sum-exp over those keys (computed here, fp32);
 *   - score[u][j] += sum_g p_g,j for each cached slot j (g ascending, fp32),
 *     and the new token's score is sum_g p_g,new;
 *   - if n < budget the token is appended at slot n (seq_len becomes n + 1);
 *     when slot n opens a logical block whose table entry is -1, one block
 *     is taken from the top of the free list (free_list[free_count - 1],
 *     free_count decremented atomically; heads taking blocks in the same call
 *     get them in an unspecified order);
 *   - if n == budget, among the cached tokens with t - pos >= recent_window
 *     (and the new token itself when recent_window == 0) the one with the
 *     smallest score is pruned, ties to the lower position (scores compared
 *     as numbers, -0 == +0, NaN above every number); the new token's K, V,
 *     position and score overwrite the pruned slot.  If the new token itself
 *     is the smallest it is dropped and the cache keeps its tokens.
 * Slot order then no longer follows position order: do not pool (KVEV_POOL)
 * or compact such a cache expecting positional neighbours.
 * attn_out (may be NULL): fp32 [batch][kv_heads*group][head_dim], the step's
 * attention output sum_j p_g,j v_j over the same keys and the new token (the
 * value rows are read only when it is given), so one pass over the cache
 * serves the decode attention and the eviction ([H2O] "Score Accumulation":
 * the scores come from the attention softmax itself); not written for a
 * refused head.
 * q: [batch][kv_heads*group][head_dim], k_new / v_new:
 * [batch][kv_heads][head_dim], all in the cache dtype; t_pos: int32 [batch];
 * score: fp32 [batch][kv_heads][max_blocks*16], the running scores (read and
 * written); evicted_pos: int32 [batch][kv_heads] out = -1 (appended), the
 * pruned token's position (t when the new token was dropped), or, with the
 * head left unchanged, -2 (seq_len < 0 or > budget), -3 (free list empty),
 * -4 (a block id of the head, or the one taken from the free list, outside
 * [0, num_blocks); a bad free-list entry stays taken).  Device pointers; one
 * kernel on `stream`.  Workspace: at least kvev_h2o_workspace_bytes(cache,
 * group, budget) bytes, zero-filled once before its first use (its leading
 * part holds per-head counters that every call leaves zero); it is separate
 * from, and may not alias, the workspace of the other entry points while
 * both are in use.  Each KV head is split over several workgroups that hand
 * their partial results to the last one through the workspace.
 * Errors: KVEV_EINVAL for NULL pointers, a bad cache, group < 1,
 * budget <= 0 or above max_blocks * 16, recent_window < 0 or >= budget;
 * KVEV_EUNSUPPORTED for group > 16, budget > 4096 or group * budget (rounded
 * up to 16) > 16384, or, with attn_out, a shape whose workgroup would need
 * more than 156 KiB of LDS (large groups with large budgets and few heads);
 * KVEV_ENOSPACE for a missing or short workspace.
 */
int kvev_h2o_step(const kvev_cache *cache, const void *q, const void *k_new, const void *v_new,
                  const int32_t *t_pos, int32_t group, float scale, float *score,
                  int32_t budget, int32_t recent_window, int32_t *free_list,
                  int32_t *free_count, int32_t *evicted_pos, float *attn_out,
                  void *workspace, size_t ws_bytes, void *stream);

/* Workspace bytes kvev_h2o_step needs for this cache, group and budget; 0
 * for a bad cache or a group / budget it refuses. */
size_t kvev_h2o_workspace_bytes(const kvev_cache *cache, int32_t group, int32_t budget);

/*
 * kvev_ring_step -- one decode step of SnapKV's ring-buffer adaptation for
 * every KV head ([SNAP] "How it works", "On the adaptation", "Parameters",
 * "Tie-breaking").  State beside the cache (device, caller-owned):
 *   hist: fp32 [batch][kv_heads][obs_window][max_blocks*16], each slot's
 *         ring of its last obs_window observed weights (ring index major);
 *   ring: int32 [batch][kv_heads], the ring index written next;
 *   rank: int32 [batch][kv_heads][max_blocks*16], each slot's index in
 *         position order (below seq_len); kvev_ring_init sets all three.
 * The new token of sequence b sits at position t_pos[b]; k_new, v_new are
 * [batch][kv_heads][head_dim] and q [batch][kv_heads*group][head_dim] in the
 * cache dtype.  Its query rows attend to the cached tokens with pos <= t and
 * to itself; a cached token's weight is the sum over the group of its
 * softmax probabilities (fp32).  observe: int32 [batch]; nonzero writes every
 * cached slot's weight at its ring index and advances the index modulo
 * obs_window; 0 (a null attention vector) writes nothing and leaves it.  The
 * new token enters with a zero ring.  Below the budget it is appended (a
 * block popped from the free list when its logical block has none; heads
 * appending in the same step may take the blocks in any order).  At the
 * budget one token is dropped: ring sums S (fp32; 0 for the new token),
 * max-pooled over the pool_kernel tokens centred on each in position order
 * (clamped at both ends); the smallest (pooled, position) among the tokens
 * at least recent_window positions older than t (the new token included
 * when recent_window == 0) is dropped, and the new token overwrites a
 * dropped cached token's slot (K, V, pos, a zero ring).  S is summed as:
 * the entries other than the one the step writes, index 0 upward, then the
 * step's weight (a null step: all entries, index 0 upward).
 * evicted_pos: int32 [batch][kv_heads], -1 appended, else the dropped
 * position; -2 (seq_len outside [0, budget], ring index or a rank out of
 * range), -3 (no free block), -4 (a block id out of range) leave the head
 * unchanged.  Positions of a head must be distinct.  One launch on
 * `stream`; each head is split over several 1024-thread workgroups that
 * hand their partial results to the last one through the workspace.
 * Workspace: at least kvev_ring_workspace_bytes(cache, group, budget)
 * bytes, zero-filled once before its first use (its leading part holds
 * per-head arrival counters that every call leaves zero); it may not alias
 * another entry point's workspace while both are in use.
 * Errors: KVEV_EINVAL for NULL pointers, a bad cache, group < 1,
 * recent_window outside [0, budget), obs_window < 1, an even or
 * non-positive pool_kernel, budget above the capacity; KVEV_EUNSUPPORTED
 * for group > 8, budget > 4096, group * (budget + 1) > 16384 or pool_kernel
 * > 2 * budget + 1; KVEV_ENOSPACE for a missing or short workspace.
 */
int kvev_ring_step(const kvev_cache *cache, float *hist, int32_t *ring, int32_t *rank,
                   const void *q, const void *k_new, const void *v_new, const int32_t *t_pos,
                   const int32_t *observe, int32_t group, float scale, int32_t budget,
                   int32_t recent_window, int32_t obs_window, int32_t pool_kernel,
                   int32_t *free_list, int32_t *free_count, int32_t *evicted_pos,
                   void *workspace, size_t ws_bytes, void *stream);

/* Workspace bytes kvev_ring_step needs for this cache, group and budget; 0
 * for a bad cache or a group / budget it refuses. */
size_t kvev_ring_workspace_bytes(const kvev_cache *cache, int32_t group, int32_t budget);

/*
 * kvev_ring_init -- the ring state of a cache for kvev_ring_step: every
 * ring zero, every ring index 0, and each slot's rank (its index in position
 * order among the head's seq_len slots; heads longer than 4096 are left
 * without ranks, which the step refuses anyway).  One workgroup per head.
 * Errors: KVEV_EINVAL for NULL pointers, a bad cache or obs_window < 1.
 */
int kvev_ring_init(const kvev_cache *cache, float *hist, int32_t *ring, int32_t *rank,
                   int32_t obs_window, void *stream);

/*
 * kvev_vtok_evict -- vToken's evict_token for a batch ([VTOK] section 3.2:
 * evicting a token only marks it dead in the token table; no KV memory moves
 * or is freed).  The token table of a head is its block list, pos, and
 * live: uint8 [batch][kv_heads][max_blocks*16] (nonzero live, 0 dead), with
 * block_live: int32 [batch][kv_heads][max_blocks] the live slots of each
 * logical block.  For every head u and i < n_victims[u], slot victims[u][i]
 * (int32 [batch][kv_heads][max_blocks*16], any order) is marked dead, and
 * the live count of each block holding a victim is set to the number of its
 * live slots afterwards.  A victim that is out of [0, seq_len), in a block
 * whose table entry is -1, or already dead (a repeat within the call
 * included), and a count n_victims[u] above max_blocks*16, set *status
 * (int32 on the device, written by the call: 0 or 1); such victims are
 * skipped.  Device pointers; live and the workspace 16-byte aligned; the
 * workspace (kvev_vtok_evict_workspace_bytes, scratch only, no clearing
 * needed) holds a claim word per slot.  Four kernels on `stream`, plain
 * loads and stores (no atomics on the table).
 * Errors: KVEV_EINVAL for NULL pointers, a bad cache or a misaligned live or
 * workspace; KVEV_ENOSPACE for a missing or short workspace.
 */
int kvev_vtok_evict(const kvev_cache *cache, uint8_t *live, int32_t *block_live,
                    const int32_t *victims, const int32_t *n_victims, int32_t *status,
                    void *workspace, size_t ws_bytes, void *stream);

/* Workspace bytes of kvev_vtok_evict (4 per slot); 0 for a bad cache. */
size_t kvev_vtok_evict_workspace_bytes(const kvev_cache *cache);

/*
 * kvev_vtok_reclaim -- vToken's lazy reclamation ([VTOK] section 3.3, stages
 * 1-3, and section 3.5: I1 conservation, I2 unique mapping, I4 strictly
 * fewer blocks), over every head in (b, h) order:
 *   - a head is eligible when its waste F = 1 - live / (16 * allocated
 *     blocks) (Eq. 1 over the head's blocks whose entry is not -1) exceeds
 *     theta_f;
 *   - its sources are its first max_sources allocated blocks that are not
 *     full, in logical order, excluding the block of slot seq_len - 1 (it
 *     still takes appends); T = their live tokens; the plan needs
 *     D = ceil(T / 16) destination blocks and goes ahead only if D is less
 *     than the number of sources;
 *   - heads take their D destinations from the top of the free list in
 *     (b, h) order while enough remain; a head that does not fit is deferred;
 *   - the sources' live tokens, in logical order, fill the destinations
 *     completely one after the other (K, V, pos, the optional score row);
 *     the first D source entries of the block list take the destination
 *     blocks and the others become -1, so moved tokens keep their relative
 *     order (passing over any full block between two sources); live and
 *     block_live follow; the source blocks are appended to the free list in
 *     (b, h, block) order after every head has taken its destinations.
 * seq_len does not change: slots in a -1 block are holes.  The copies run on
 * `stream`; a caller that overlaps them with decoding issues the call on a
 * stream of its own and makes the next attention wait for an event recorded
 * after it ([VTOK] section 3.3, stage 4).
 * stats: int64[10] on the device = {heads reclaimed, heads deferred, heads
 * left as they are (F at or below theta_f, or no plan that frees a block),
 * blocks freed, rows moved, bytes moved (K and V, read + write), live
 * tokens, allocated blocks before, after, status (an OR of 2: a seq_len
 * out of range, 4: a block id past the pool or a live count outside
 * [0, 16] -- such heads are skipped and not counted; 8: a free count outside
 * [0, min(free_capacity, num_blocks)] -- nothing is admitted -- or a list
 * too small for the returned sources, whose excess is dropped)}.
 * Workspace: at least kvev_vtok_workspace_bytes(cache, max_sources) bytes
 * (scratch only).  live, the cache's pos, score_or_null and the workspace:
 * 16-byte aligned.
 * Errors: KVEV_EINVAL for NULL pointers, a bad cache, a misaligned pointer,
 * theta_f outside [0, 1) or max_sources outside [2, 4096]; KVEV_EUNSUPPORTED above 8192 KV
 * heads; KVEV_ENOSPACE when free_capacity < num_blocks or the workspace is
 * missing or short.
 */
int kvev_vtok_reclaim(const kvev_cache *cache, uint8_t *live, int32_t *block_live,
                      float *score_or_null, double theta_f, int32_t max_sources,
                      int32_t *free_list, int32_t *free_count, int32_t free_capacity,
                      int64_t *stats, void *workspace, size_t ws_bytes, void *stream);

/* Workspace bytes of kvev_vtok_reclaim; 0 for a bad cache or max_sources. */
size_t kvev_vtok_workspace_bytes(const kvev_cache *cache, int32_t max_sources);

/*
 * kvev_vtok_sync -- vToken's sync_new_tokens ([VTOK] section 3.2: the
 * scheduler passes the current block list and length; the table registers
 * the new tokens at their physical positions with sequential logical IDs).
 * For every head u with n = seq_len[u] and m = new_len[u] (int32
 * [batch][kv_heads], device): the slots [n, m) become live, slot s takes
 * position pos0[b] + (s - n) (pos0: int32 [batch], device), each block's
 * live count grows by its new slots, and seq_len[u] = m.  The caller has
 * already written the new K/V rows and the block ids of [n, m) (from its
 * allocator).  status[u] (int32 [batch][kv_heads], device) = 0, -2 (m < n
 * or m above the capacity) or -4 (a block of [n, m) without an id in
 * [0, num_blocks)); a head with a nonzero status is left unchanged.  One
 * workgroup per head on `stream`.
 * Errors: KVEV_EINVAL for NULL pointers or a bad cache.
 */
int kvev_vtok_sync(const kvev_cache *cache, uint8_t *live, int32_t *block_live,
                   const int32_t *new_len, const int32_t *pos0, int32_t *status, void *stream);

/*
 * kvev_vtok_slot_mapping -- vToken's BuildSlotMapping ([VTOK] Algorithm 1,
 * step 4, and Eq. 2: slot = block_id * block_size + offset for every live
 * token).  For every head, the live slots below seq_len in logical order go
 * to slots (int32 [batch][kv_heads][max_blocks*16], the physical row of the
 * pools) with their positions (same shape); count[u] (int32
 * [batch][kv_heads]) of them, or -1 for a seq_len outside [0, max_blocks*16].
 * Slots in blocks without an id in [0, num_blocks) are skipped.  An attention
 * kernel reads a reclaimed head through this mapping.  Workspace:
 * kvev_vtok_map_workspace_bytes (scratch: live slots per 4096-slot chunk).
 * Two launches over 4096-slot chunks of every head on `stream`.
 * Errors: KVEV_EINVAL for NULL pointers or a bad cache; KVEV_ENOSPACE for a
 * missing or short workspace.
 */
int kvev_vtok_slot_mapping(const kvev_cache *cache, const uint8_t *live, int32_t *slots,
                           int32_t *positions, int32_t *count, void *workspace, size_t ws_bytes,
                           void *stream);

/* Workspace bytes of kvev_vtok_slot_mapping; 0 for a bad cache. */
size_t kvev_vtok_map_workspace_bytes(const kvev_cache *cache);

/*
 * kvev_vtok_digest -- the online check of vToken's I1, token conservation
 * ([VTOK] section 3.5: the set of live tokens and their K/V contents survive
 * every relocation; checked by hashing and comparing).  For every head u,
 * digest[u] (uint64 on the device, written by the call) is the sum mod 2^64,
 * over the live slots s < seq_len (clamped to [0, max_blocks*16]) in blocks
 * whose id lies in [0, num_blocks), of fmix64(t) with
 *   t = fmix64(pos ^ G) + sum_i fmix64(k_i ^ (2i+1)*G) + sum_i fmix64(v_i ^ (2i+2)*G),
 * pos zero-extended, k_i / v_i the little-endian 64-bit words of the token's
 * K and V rows, G = 0x9E3779B97F4A7C15, fmix64 MurmurHash3's 64-bit
 * finalizer.  A token's contribution does not depend on where it is stored,
 * so equal digests before and after kvev_vtok_reclaim confirm I1 (with
 * overwhelming probability).  live: 16-byte aligned.  Two kernels on
 * `stream` (one reads every live K and V row once).
 * Errors: KVEV_EINVAL for NULL pointers, a bad cache or misaligned pointers.
 */
int kvev_vtok_digest(const kvev_cache *cache, const uint8_t *live, uint64_t *digest,
                     void *stream);

/*
 * kvev_vtok_check -- the online check of vToken's I2, unique mapping
 * ([VTOK] section 3.5), and of the live counts of section 3.3 stage 1.
 * out: int64[4] on the device = {pool blocks held more than once, pool
 * blocks held by nobody, references out of range, live-count mismatches}.
 * Holders are every table entry >= 0 of every head (all max_blocks entries)
 * and free_list[0, *free_count); a table entry >= num_blocks, a list entry
 * outside [0, num_blocks) and a free count outside [0, free_capacity] are out
 * of range.  A mismatch is a table entry >= 0 whose block_live differs from
 * the number of its nonzero live bytes.  I2 holds when the first three are
 * 0.  Workspace: kvev_vtok_check_workspace_bytes (scratch, a holder count per
 * pool block).  live and the workspace 16-byte aligned.  Five kernels on
 * `stream`.
 * Errors: KVEV_EINVAL for NULL pointers, a bad cache, misaligned pointers or
 * a negative capacity; KVEV_ENOSPACE for a missing or short workspace.
 */
int kvev_vtok_check(const kvev_cache *cache, const uint8_t *live, const int32_t *block_live,
                    const int32_t *free_list, const int32_t *free_count, int32_t free_capacity,
                    int64_t *out, void *workspace, size_t ws_bytes, void *stream);

/* Workspace bytes of kvev_vtok_check; 0 for a bad cache. */
size_t kvev_vtok_check_workspace_bytes(const kvev_cache *cache);

/*
 * kvev_window_attn -- helper outside the eviction step: the log-sum-exp and
 * (optionally) the attention output of each window query, which a
 * FlashAttention-style forward pass would produce ([DROP] Jargon,
 * "Log-sum-exp"; "Why does the Triton kernel matter").
 *     lse_out[b][hq][w] = log sum_{pos_j <= q_pos[w]} exp(scale * q.k_j)   (fp32)
 *     a_out[b][hq][w][:] = sum_j exp(scale * q.k_j - lse) v_j           (fp32, may be NULL)
 * q.k on the MFMA (cache-dtype inputs, fp32 sums); for the output the
 * weights enter the MFMA as a bf16 high part plus a bf16 low part (bf16
 * caches: each weight to a relative 2^-16) or in fp32 (fp32 caches), with
 * fp32 sums; the chunks of keys are merged in fp32.  A query that attends no
 * key gets lse = -inf and a = 0; the slots of a block id outside the pool
 * are skipped (attended by no query).  Bitwise reproducible.  Workspace: at
 * least kvev_workspace_bytes(cache, group, W).  Errors as for kvev_score;
 * KVEV_ENOSPACE for a short workspace.
 */
int kvev_window_attn(const kvev_cache *cache, const kvev_window *win, float *lse_out,
                     float *a_out, void *workspace, size_t ws_bytes, void *stream);

/* Workspace bytes needed by kvev_select, kvev_compact, kvev_evict, kvev_score
 * and kvev_window_attn on this cache shape with this window shape (group,
 * obs_window); pass 0, 0 for calls without a window (kvev_select,
 * kvev_compact).  Windows too large for one workgroup's LDS add room for
 * their split rows' raw sums.  0 for a bad cache. */
size_t kvev_workspace_bytes(const kvev_cache *cache, int32_t group, int32_t obs_window);

/* Static description of a status code. */
const char *kvev_strerror(int status);

/* KVEV_ABI_VERSION of the loaded library. */
int kvev_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* KVEV_H */
