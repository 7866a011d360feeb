// kvev_kernels.h -- argument blocks and host-side launchers of the libkvev
// kernels.  Internal to the library; the public interface is include/kvev.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kvev {

// Per-head selection state and outputs of the select kernels
// (kvev_select_head.h).
struct SelHead {
  int32_t *n_victims;
  uint32_t *hist;         // state [units][2048]: top 11 key bits (zero between calls)
  uint32_t *hist2;        // state [units][2048]: key bits 20..10 of the bucket's keys (zero between calls)
  uint32_t *head_sel;     // scratch [units][4]: T, cut slot, bucket, keys below the bucket
  uint32_t *chunk_off;    // scratch [units][chunks]: first victim index of each chunk
  uint32_t *chunk_below;  // scratch [units][chunks]: keys below the bucket per chunk
  uint2 *cand;            // scratch [units][nwg][4096]: (key, slot) pairs of the bucket
  uint32_t *ccount;       // scratch [units][nwg]: pairs in each collect region
  int32_t budget, recent, chunks, nwg;  // chunks: 1024-slot chunks; nwg: 4096-slot regions
  const int32_t *budget_u, *recent_u;  // per-unit budgets and recent windows, or null
};

// The budget and recent window of unit u; false when the pair is invalid
// (the unit is then treated as an inconsistent head: n_victims -1).
__device__ __forceinline__ bool unit_budget(const SelHead &S, int u, int &budget, int &recent) {
  budget = S.budget_u ? S.budget_u[u] : S.budget;
  recent = S.recent_u ? S.recent_u[u] : S.recent;
  return budget > 0 && recent >= 0 && recent < budget;
}

struct ScoreArgs {
  const uint8_t *k_pool, *v_pool;
  const int32_t *block_table, *seq_len, *pos;
  const uint8_t *q;
  const float *a;                // DROP: fp32 [B][Hq][W][D]
  const float *lse;
  const int32_t *q_pos;
  float *sum, *pooled, *drop;
  const float *prev;             // ACCUMULATE: the running sums added to (normally `sum`)
  uint32_t *head_err;            // optional [units]: set to 1 when a block id is outside the pool
  // optional [units][2048]: the top 11 key bits of the written score over each
  // head's candidate slots [0, n - sel_recent), for heads with n > sel_budget
  uint32_t *hist;
  int32_t sel_budget, sel_recent;
  int32_t units, Hkv, G, W, max_blocks, num_blocks;
  int32_t rows, row_tiles;       // G*W and ceil(rows / 16)
  int32_t flags, pool_r, halo_blocks, tile_blocks, tiles_per_head, threads;
  float c1;                      // scale * log2(e)
  float scale;                   // the softmax scale itself (exact DropKV terms)
  // rows split over row_parts workgroups per tile, rt_part row tiles each;
  // with row_parts > 1 the parts' raw sums go to part_sum / part_drop
  // [row_parts][units][max_slots] (workspace) and a combine pass finishes
  int32_t row_parts, rt_part;
  float *part_sum, *part_drop;
};

struct SelectArgs {
  const float *score;
  const int32_t *seq_len;
  int32_t *victims;
  SelHead sel;
  int32_t units, max_slots;
};

struct CompactArgs {
  uint8_t *k_pool, *v_pool;
  int32_t *block_table, *seq_len, *pos;
  float *score;                 // optional score row moved with the tokens
  const int32_t *victims, *n_victims;
  int32_t *free_list, *free_count;
  int64_t *stats;
  // workspace regions
  int32_t *src_of;              // [units][max_slots]: source of each destination rank
  int32_t *src_row;             // [units][max_slots]: pool row of each moved rank's source (-1: stays)
  int32_t *new_pos;             // [units][max_slots]: pos of each kept rank
  float *new_score;             // [units][max_slots]: score of each kept rank
  uint8_t *stage_k, *stage_v;   // [units][stage_rows][row_bytes]: at-risk rows
  int32_t *head_info;           // [units][8]: n, m, error, blocks freed, rows moved, staged,
                                // in order (more at-risk rows than stage_rows)
  unsigned long long *head_acc; // [units] persistent state (zero between calls): prep
                                // chunks done, chunks with errors, rows moved, staged
  int32_t *fc0;                 // free_count before the call
  int32_t units, max_blocks, max_slots, num_blocks, row_bytes, stage_rows, chunks,
      free_capacity, rows_per_item;
  int32_t rows_cap;             // kept rows per head are at most this (sizes the gather grid)
};

// The fused eviction pass after scoring (finish.hip): exact threshold,
// victims and in-place compaction of every head in one launch.
struct FinishArgs {
  uint8_t *k_pool, *v_pool;
  int32_t *block_table, *seq_len, *pos;
  const float *sc;              // [units][max_slots] this pass's scores (workspace)
  float *score_out;             // [units][max_slots] receives the compacted scores
  int32_t *victims, *n_victims;
  int32_t *free_list, *free_count;
  int64_t *stats;
  // state (zero between calls): bad-block flags and key histograms the
  // scoring pass set, the bucket's second-level histograms, member counts
  // and arrivals per head, per-batch "sources read" marks, workgroups done
  // per head, the ticket and done counters, and the stat accumulators
  uint32_t *head_err, *hist, *hist2, *nmem, *arrive, *marks, *head_done, *ctr;
  uint32_t *bctr;  // per head: batch tickets of the compaction
  unsigned long long *acc;      // [4]: blocks freed, rows moved, at-risk rows, status bits
  // scratch: the bucket's (key, slot) members [units][max_slots], keys below
  // the bucket per 1024-slot chunk [units][chunks]
  uint2 *mem;
  uint32_t *gbelow;
  int32_t chunks;               // 1024-slot chunks per head
  int32_t units, max_blocks, max_slots, num_blocks, row_bytes, budget, recent;
  int32_t kh;                   // workgroups per head
  int32_t marks_per_head;       // batches of 256 ranks a head can have
  int32_t free_capacity;
};
hipError_t launch_finish(const FinishArgs &a, hipStream_t s);
size_t finish_lds_bytes();
int finish_parts(int units, int rows_cap);  // workgroups per head

struct MeasureArgs {
  const int32_t *seq_len_before, *victims, *n_victims;
  int64_t *out;  // [6]
  int32_t units, max_slots;
};
hipError_t launch_measure(const MeasureArgs &a, hipStream_t s);

struct H2oArgs {
  uint8_t *k_pool, *v_pool;
  int32_t *block_table, *seq_len, *pos;
  float *score;                        // running scores [units][max_slots]
  const uint8_t *q, *k_new, *v_new;    // [B][Hq][D], [B][Hkv][D], [B][Hkv][D]
  const int32_t *t_pos;                // [B]
  int32_t *free_list, *free_count;
  int32_t *evicted;                    // [units]
  float *attn;                         // optional attention output [B][Hq][D] (fp32)
  // workspace: e values [units][G][np], part maxima and sums [units][8][32],
  // parts' attention shares [units][8][G][D], state (zero between calls)
  // arrival counters and error flags [units]
  uint32_t *e, *ml, *arrive, *err;
  float *o;
  int32_t units, Hkv, G, max_blocks, max_slots, num_blocks, budget, recent;
  int32_t np;                          // budget rounded up to 16, plus 16 (the new token's e)
  int32_t split;                       // workgroups per head
  float c1;                            // scale * log2(e)
};
hipError_t launch_h2o_step(const H2oArgs &a, int bf16, int head_dim, hipStream_t s);
size_t h2o_lds_bytes(const H2oArgs &a, int head_dim);  // dynamic LDS of one workgroup

struct VtokArgs {
  uint8_t *k_pool, *v_pool;
  int32_t *block_table;
  int32_t *seq_len;                    // written by sync_new_tokens only
  int32_t *pos;
  float *score;                        // optional score row moved with the tokens
  uint8_t *live;                       // [units][max_slots] liveness bytes
  int32_t *block_live;                 // [units][max_blocks] live slots per block
  const int32_t *victims, *n_victims;  // marks
  int32_t *status;                     // marks: bit 0, a victim that was not live
  int32_t *free_list, *free_count;
  int64_t *stats;                      // reclamation [10]
  // workspace: plan records [units][8], sources, their live offsets and the
  // destination ids of the first D source positions [units][max_sources],
  // destination / push offsets [units], staged positions and scores
  // [units][max_sources*16], misc [8]; for the marks, a claim word per slot
  // [units][max_slots]
  int32_t *plan, *src, *srcoff, *dstw, *dst_off, *push_off, *tpos, *misc, *claim;
  float *tscore;
  // sync_new_tokens: new lengths [units], first positions [B]; slot mapping
  // outputs: slots and positions [units][max_slots], counts [units]
  const int32_t *new_len, *pos0;
  int32_t *map_slots, *map_pos, *map_count;
  int32_t *map_chunk, map_chunks;      // workspace: live slots per 1024-slot chunk [units][chunks]
  int32_t units, Hkv, max_blocks, max_slots, num_blocks, row_bytes, max_sources, free_capacity;
  double theta_f;
};
hipError_t launch_vtok_evict(const VtokArgs &a, hipStream_t s);
hipError_t launch_vtok_reclaim(const VtokArgs &a, hipStream_t s);
hipError_t launch_vtok_digest(const VtokArgs &a, uint64_t *digest, hipStream_t s);
hipError_t launch_vtok_sync(const VtokArgs &a, hipStream_t s);
hipError_t launch_vtok_slot_mapping(const VtokArgs &a, hipStream_t s);
hipError_t launch_vtok_check(const VtokArgs &a, int32_t *held, int64_t *out, hipStream_t s);

// Shared scores across the KV heads of a sequence (policy.hip).
struct SharedArgs {
  const float *score;          // [B][Hkv][max_slots] per-head scores
  const int32_t *seq_len, *pos;
  float *row;                  // workspace [B][max_slots]: the shared rows
  int32_t *vseq;               // workspace [B]: the shared rows' lengths (zeroed first)
  int32_t *vvict, *vnv;        // workspace: the selection's victims [B][max_slots], counts [B]
  int32_t *victims, *n_victims;  // outputs [B][Hkv][max_slots], [B][Hkv]
  uint32_t *zero;              // the words cleared first: vseq and the selection histograms
  size_t zero_words;
  SelectArgs sel;              // the selection over the B shared rows
  int32_t B, Hkv, max_slots;
};
hipError_t launch_select_shared(const SharedArgs &a, hipStream_t s);

// SnapKV's decode-time ring buffer (ring_step.hip).
constexpr int kRingMaxGroup = 8;
constexpr int kRingMaxBudget = 4096;
constexpr int kRingMaxBlocks = kRingMaxBudget / 16 + 1;
constexpr int kRingMaxSplit = 8;       // workgroups per head
struct RingArgs {
  uint8_t *k_pool, *v_pool;
  int32_t *block_table, *seq_len, *pos;
  float *hist;                         // [units][W][max_slots] rings
  int32_t *ring, *rank;                // [units] next ring index; [units][max_slots] position order
  const uint8_t *q, *k_new, *v_new;    // [B][Hq][D], [B][Hkv][D], [B][Hkv][D]
  const int32_t *t_pos, *observe;      // [B]
  int32_t *free_list, *free_count;
  int32_t *evicted;                    // [units]
  // workspace: e values [units][G][np], the other ring entries' sums
  // [units][np], part maxima and sums [units][8][32]; state (zero between
  // calls): arrival counters [units]
  uint32_t *e, *rsum, *ml, *arrive;
  int32_t units, Hkv, G, W, max_blocks, max_slots, num_blocks, budget, recent, pool_kernel;
  int32_t split, cb, nbmax, np;        // parts per head, blocks per part, budget blocks, e stride
  float c1;                            // softmax scale * log2(e)
};
hipError_t launch_ring_step(const RingArgs &a, int bf16, int head_dim, hipStream_t s);
hipError_t launch_ring_init(const RingArgs &a, hipStream_t s);
size_t ring_lds_bytes(const RingArgs &a);  // dynamic LDS of one workgroup

struct WindowAttnArgs {
  const uint8_t *k_pool, *v_pool;
  const int32_t *block_table, *seq_len, *pos;
  const uint8_t *q;
  const int32_t *q_pos;
  float *lse_out;
  float *a_out;                        // fp32 [B][Hq][W][D]
  float *part_m, *part_l, *part_acc;   // workspace partials
  int32_t units, Hkv, G, W, max_blocks, num_blocks, rows, chunk_slots, chunks, want_a;
  int32_t threads, rt_wave, row_parts;  // workgroup size, row tiles per wave, workgroups per chunk
  float scale;
};

hipError_t launch_score(const ScoreArgs &a, int bf16, int head_dim, int drop, hipStream_t s);
hipError_t launch_select(const SelectArgs &a, hipStream_t s);
hipError_t launch_compact(const CompactArgs &a, hipStream_t s);
hipError_t launch_window_attn(const WindowAttnArgs &a, int bf16, int head_dim, hipStream_t s);

constexpr int kSelectChunk = 1024;      // victim offsets are kept per chunk of slots
constexpr int kSelectBins = 2048;       // histogram bins (top 11 key bits)
constexpr int kSelectMaxChunks = 1024;  // chunks per head: up to 1M slots
constexpr int kHistChunk = 4096;        // slots per select histogram workgroup
constexpr int kCompactMaxUnits = 4096;  // compact.hip gather limit
constexpr int kCompactChunk = 1024;     // compact.hip prep chunk (slots)
constexpr int kCompactStageRows = 4096; // compact.hip: at-risk rows staged per head at most
// Prep packs a head's chunk arrivals into 11 bits.
static_assert(kSelectMaxChunks * kSelectChunk / kCompactChunk < 2048,
              "chunk arrivals are counted in 11 bits");
constexpr int kH2oMaxBudget = 4096;    // h2o_step.hip: tokens per head
constexpr int kH2oMaxLogits = 16384;   // h2o_step.hip: G * budget (64 KB of LDS)
constexpr int kH2oMaxSplit = 8;        // h2o_step.hip: workgroups per head
constexpr int kVtokMaxUnits = 8192;    // vtoken.hip: heads per reclamation call (admission in LDS)
constexpr int kVtokMaxSources = 4096;  // vtoken.hip: sources per head and call
// score.hip: DropKV terms with p >= 1/4 queued for the exact pass, per staged
// window row (weights of one row sum to 1: at most four reach 1/4)
constexpr int kExactPerRow = 4;

// LDS bytes of one window-attention workgroup (chunk_slots keys per chunk).
__host__ __device__ size_t window_attn_lds_bytes(int bf16, int head_dim, int want_a,
                                                 int chunk_slots);

// LDS bytes of one score workgroup (hist: with the tile's key histogram).
__host__ __device__ size_t score_lds_bytes(int bf16, int head_dim, int drop, int row_tiles,
                                            int tile_blocks, int halo_blocks, int hist);

}  // namespace kvev
