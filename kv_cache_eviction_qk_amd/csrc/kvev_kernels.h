// kvev_kernels.h -- argument blocks and host-side launchers of the libkvev
// kernels.  Internal to the library; the public interface is include/kvev.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kvev {

struct ScoreArgs {
  const uint8_t *k_pool, *v_pool;
  const int32_t *block_table, *seq_len, *pos;
  const uint8_t *q, *a;
  const float *lse;
  const int32_t *q_pos;
  float *sum, *pooled, *drop;
  int32_t units, Hkv, G, W, max_blocks, num_blocks;
  int32_t rows, row_tiles;       // G*W and ceil(rows / 16)
  int32_t flags, pool_r, halo_blocks, tile_blocks, tiles_per_head, threads;
  float c1;                      // scale * log2(e)
};

struct SelectArgs {
  const float *score;
  const int32_t *seq_len;
  int32_t *victims, *n_victims;
  // workspace: persistent state (zero between calls)
  uint32_t *hist;         // [units][2048] histogram of the top 11 key bits
  // workspace: scratch
  uint2 *cand;            // [units][subs][256] (key, slot) of the threshold bucket
  uint32_t *ccount;       // [units][subs] candidates of each 256-slot sub-chunk
  int32_t *cnt_lt;        // [units][subs] keys below the threshold bucket
  uint32_t *chunk_off;    // [units][chunks] output offset of each 1024-slot chunk
  uint32_t *head_sel;     // [units][4] threshold key, tie-cut slot
  int32_t units, max_slots, budget, recent, chunks;
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
  int32_t *new_pos;             // [units][max_slots]: pos of each kept rank
  float *new_score;             // [units][max_slots]: score of each kept rank
  uint8_t *stage_k, *stage_v;   // [units][stage_rows][row_bytes]: at-risk rows
  int32_t *head_info;           // [units][4]: n before the call, -, error, blocks freed
  uint32_t *head_err;           // [units] persistent state (zero between calls)
  int32_t *chunk_mv;            // [units][chunks][2]: rows moved, rows staged
  int32_t *fc0;                 // free_count before the call
  int32_t units, max_blocks, max_slots, num_blocks, row_bytes, stage_rows, chunks,
      free_capacity, rows_per_item;
};

struct WindowAttnArgs {
  const uint8_t *k_pool, *v_pool;
  const int32_t *block_table, *seq_len, *pos;
  const uint8_t *q;
  const int32_t *q_pos;
  float *lse_out;
  uint8_t *a_out;
  float *part_m, *part_l, *part_acc;   // workspace partials
  int32_t units, Hkv, G, W, max_blocks, num_blocks, rows, chunk_slots, chunks, want_a;
  float scale;
};

hipError_t launch_score(const ScoreArgs &a, int bf16, int head_dim, int drop, hipStream_t s);
hipError_t launch_select(const SelectArgs &a, hipStream_t s);
hipError_t launch_compact(const CompactArgs &a, hipStream_t s);
hipError_t launch_window_attn(const WindowAttnArgs &a, int bf16, int head_dim, hipStream_t s);

// LDS bytes of one score workgroup (0 when the row count does not fit).
constexpr int kSelectChunk = 1024;      // select.hip chunk (slots)
constexpr int kSelectBins = 2048;       // select.hip histogram bins
constexpr int kSelectMaxChunks = 1024;  // select.hip refine step limit
constexpr int kCompactMaxUnits = 4096;  // compact.hip gather limit
constexpr int kCompactChunk = 1024;     // compact.hip prep chunk (slots)

size_t score_lds_bytes(int bf16, int head_dim, int drop, int row_tiles, int tile_blocks,
                       int halo_blocks);

}  // namespace kvev
