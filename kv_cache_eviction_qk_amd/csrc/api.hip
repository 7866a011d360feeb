// api.hip -- the C ABI of libkvev (declared in include/kvev.h).
//
// Host side only: argument validation (every refusal happens before any
// work is enqueued), launch geometry, workspace layout and error mapping.
// All arithmetic runs in the kernels of score.hip, select.hip, compact.hip
// and window_attn.hip.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstddef>
#include <cstdint>
#include <mutex>

#include "kvev.h"
#include "kvev_kernels.h"

namespace {

constexpr int kWaMaxChunk = 8192;     // keys per window-attention chunk, at most
constexpr size_t kMaxLds = 160 * 1024;
#ifndef KV_TILE_MAX
#define KV_TILE_MAX 256
#endif
#ifndef KV_THREADS_MAX
#define KV_THREADS_MAX 512  // score workgroups: 256 or 512 threads
#endif
constexpr int kMaxPoolKernel = 2049;  // halo of at most 64 blocks per side

bool valid_cache(const kvev_cache *c) {
  if (!c) return false;
  if (c->batch < 1 || c->kv_heads < 1 || c->max_blocks < 1 || c->num_blocks < 1) return false;
  if (c->block_size != KVEV_BLOCK_SIZE) return false;
  if (c->head_dim != 64 && c->head_dim != 128) return false;
  if (c->dtype != KVEV_F32 && c->dtype != KVEV_BF16) return false;
  if (!c->k_pool || !c->v_pool || !c->block_table || !c->seq_len || !c->pos) return false;
  if ((int64_t)c->max_blocks * KVEV_BLOCK_SIZE > INT32_MAX / 2) return false;
  if ((int64_t)c->num_blocks * KVEV_BLOCK_SIZE > INT32_MAX / 2) return false;
  if ((int64_t)c->batch * c->kv_heads > 65535) return false;
  return true;
}

int elem_bytes(const kvev_cache *c) { return c->dtype == KVEV_BF16 ? 2 : 4; }

size_t a256(size_t x) { return (x + 255) & ~(size_t)255; }

// Zeroes n16 16-byte words (a fill kernel, not a memset, so that callers
// may capture it in a graph).
__global__ __launch_bounds__(256) void clear16_kernel(uint4 *p, size_t n16) {
  for (size_t i = blockIdx.x * (size_t)256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// Workspace = [persistent state | scratch].  The state (selection
// histograms, per-head compaction accumulators) must be zero before
// the first call; every call leaves it zero.  The scratch part is shared by
// all entry points; selection and compaction use disjoint parts of it, so
// the fused call can pass the threshold from one to the other.
struct StateLayout {
  size_t hist, hist2, head_acc, fin_err, fin_nmem, fin_arrive, fin_marks, fin_done, fin_bctr, fin_ctr,
      fin_acc, total;
  int marks_per_head;
};

StateLayout state_layout(const kvev_cache *c) {
  StateLayout L{};
  const size_t units = (size_t)c->batch * c->kv_heads;
  const size_t max_slots = (size_t)c->max_blocks * KVEV_BLOCK_SIZE;
  L.marks_per_head = (int)((max_slots + 255) / 256);
  size_t off = 0;
  L.hist = off; off = a256(off + units * kvev::kSelectBins * 4);
  L.hist2 = off; off = a256(off + units * kvev::kSelectBins * 4);
  L.head_acc = off; off = a256(off + units * 8);
  // kvev_evict's pass after scoring (it also uses hist and hist2): bad-block
  // flags, bucket member counts, arrivals, batch marks, heads' workgroups
  // done, ticket and done counters, stat accumulators
  L.fin_err = off; off = a256(off + units * 4);
  L.fin_nmem = off; off = a256(off + units * 4);
  L.fin_arrive = off; off = a256(off + units * 4);
  L.fin_marks = off; off = a256(off + units * (size_t)L.marks_per_head * 4);
  L.fin_done = off; off = a256(off + units * 4);
  L.fin_bctr = off; off = a256(off + units * 4);
  L.fin_ctr = off; off = a256(off + 4 * 4);
  L.fin_acc = off; off = a256(off + 4 * 8);
  L.total = off;
  return L;
}

// kvev_evict's scratch after the state: the scores of the pass, the bucket
// members and the keys below the bucket per 1024-slot chunk, per head.
struct EvictLayout {
  size_t sc, mem, gbelow, total;
  int chunks;
};

EvictLayout evict_layout(const kvev_cache *c) {
  EvictLayout L{};
  const size_t units = (size_t)c->batch * c->kv_heads;
  const size_t max_slots = (size_t)c->max_blocks * KVEV_BLOCK_SIZE;
  L.chunks = (int)((max_slots + 1023) / 1024);
  size_t off = state_layout(c).total;
  L.sc = off; off = a256(off + units * max_slots * 4);
  L.mem = off; off = a256(off + units * max_slots * 8);
  L.gbelow = off; off = a256(off + units * (size_t)L.chunks * 4);
  L.total = off;
  return L;
}

size_t evict_layout_total(const kvev_cache *c) { return evict_layout(c).total; }

size_t compact_layout_total(const kvev_cache *c);

// The workspace kvev_select, kvev_compact and kvev_evict share.
size_t main_layout_total(const kvev_cache *c) {
  return std::max(compact_layout_total(c), evict_layout_total(c));
}

struct SelectLayout {
  size_t chunk_off, chunk_below, head_sel, cand, ccount, total;
  int chunks, nwg;
};

SelectLayout select_layout(const kvev_cache *c) {
  SelectLayout L{};
  const size_t units = (size_t)c->batch * c->kv_heads;
  const size_t max_slots = (size_t)c->max_blocks * KVEV_BLOCK_SIZE;
  L.chunks = (int)((max_slots + kvev::kSelectChunk - 1) / kvev::kSelectChunk);
  L.nwg = (int)((max_slots + kvev::kHistChunk - 1) / kvev::kHistChunk);
  size_t off = state_layout(c).total;
  L.chunk_off = off; off = a256(off + units * (size_t)L.chunks * 4);
  L.chunk_below = off; off = a256(off + units * (size_t)L.chunks * 4);
  L.head_sel = off; off = a256(off + units * 16);
  L.cand = off; off = a256(off + units * (size_t)L.nwg * kvev::kHistChunk * 8);
  L.ccount = off; off = a256(off + units * (size_t)L.nwg * 4);
  L.total = off;
  return L;
}

struct CompactLayout {
  size_t src_of, src_row, new_pos, new_score, stage_k, stage_v, head_info, fc0, total;
  int chunks, stage_rows;
};

CompactLayout compact_layout(const kvev_cache *c) {
  CompactLayout L{};
  const size_t units = (size_t)c->batch * c->kv_heads;
  const size_t max_slots = (size_t)c->max_blocks * KVEV_BLOCK_SIZE;
  const size_t row_bytes = (size_t)c->head_dim * elem_bytes(c);
  L.chunks = (int)((max_slots + kvev::kCompactChunk - 1) / kvev::kCompactChunk);
  // At-risk rows are staged up to kCompactStageRows a head (a head with more
  // is compacted in rank order by one workgroup, staging nothing).
  L.stage_rows = (int)std::min<size_t>(max_slots, kvev::kCompactStageRows);
  size_t off = select_layout(c).total;
  L.src_of = off; off = a256(off + units * max_slots * 4);
  L.src_row = off; off = a256(off + units * max_slots * 4);
  L.new_pos = off; off = a256(off + units * max_slots * 4);
  L.new_score = off; off = a256(off + units * max_slots * 4);
  L.stage_k = off; off = a256(off + units * (size_t)L.stage_rows * row_bytes);
  L.stage_v = off; off = a256(off + units * (size_t)L.stage_rows * row_bytes);
  L.head_info = off; off = a256(off + units * 8 * 4);
  L.fc0 = off; off = a256(off + 4);
  L.total = off;
  return L;
}

size_t compact_layout_total(const kvev_cache *c) { return compact_layout(c).total; }

// Window attention's launch shape: 256 threads with one row tile per wave up
// to 4 tiles, two per wave up to 8, then 512 threads with two per wave and
// as many workgroups per chunk as 16 tiles need; chunks of a multiple of 32
// keys, for about 512 workgroups, of at least 256 keys and 8 per window row
// (so that the partials stay small beside the keys), at most kWaMaxChunk.
struct WaShape {
  int threads, rt_wave, row_parts, chunk_slots, chunks;
};

WaShape wa_shape(const kvev_cache *c, int rows) {
  WaShape s{};
  const int T = (rows + 15) / 16;
  s.threads = T <= 8 ? 256 : 512;
  s.rt_wave = T <= 4 ? 1 : 2;
  const int tiles_per_wg = (s.threads / 64) * s.rt_wave;
  s.row_parts = (T + tiles_per_wg - 1) / tiles_per_wg;
  const int64_t units = (int64_t)c->batch * c->kv_heads;
  const int64_t max_slots = (int64_t)c->max_blocks * KVEV_BLOCK_SIZE;
  const int64_t want = (512 + units * s.row_parts - 1) / (units * s.row_parts);
  int64_t cs = (max_slots + want - 1) / want;
  cs = std::max<int64_t>(cs, std::max<int64_t>(256, (int64_t)rows * 8));
  cs = std::min<int64_t>(cs, kWaMaxChunk);
  cs = (cs + 31) / 32 * 32;
  s.chunk_slots = (int)cs;
  s.chunks = (int)((max_slots + cs - 1) / cs);
  return s;
}

struct WaLayout {
  size_t part_m, part_l, part_acc, total;
  int chunks;
};

WaLayout wa_layout(const kvev_cache *c, int group, int obs_window) {
  WaLayout L{};
  const size_t units = (size_t)c->batch * c->kv_heads;
  const int rows = group * obs_window;
  L.chunks = wa_shape(c, rows).chunks;
  const size_t parts = units * (size_t)rows * L.chunks;
  size_t off = state_layout(c).total;
  L.part_m = off; off = a256(off + parts * 4);
  L.part_l = off; off = a256(off + parts * 4);
  L.part_acc = off; off = a256(off + parts * (size_t)c->head_dim * 4);
  L.total = off;
  return L;
}

int map_err(hipError_t e) { return e == hipSuccess ? KVEV_OK : KVEV_EDEVICE; }

// Window rows a score workgroup stages: split over several workgroups per
// tile when they do not fit in LDS beside a 16-block tile (DropKV stages a
// second and, for bf16, a third copy of each row).  Returns the parts;
// *rt_part receives the row tiles of each.
int score_row_parts(int bf16, int head_dim, int drop, int row_tiles, int *rt_part) {
  int parts = 1, rtp = row_tiles;
  while (rtp > 1 &&
         kvev::score_lds_bytes(bf16, head_dim, drop, rtp, 16, 0, 1) > kMaxLds - 1024) {
    ++parts;
    rtp = (row_tiles + parts - 1) / parts;
  }
  *rt_part = rtp;
  return (row_tiles + rtp - 1) / rtp;
}

// Workspace bytes of the split windows' raw sums (0 when the rows fit).
size_t score_parts_bytes(const kvev_cache *c, int32_t group, int32_t obs_window, int drop,
                         int want_sum) {
  if (group < 1 || obs_window < 1) return 0;
  int rtp;
  const int parts = score_row_parts(c->dtype == KVEV_BF16, c->head_dim, drop,
                                    (group * obs_window + 15) / 16, &rtp);
  if (parts == 1) return 0;
  const size_t row = (size_t)c->batch * c->kv_heads * c->max_blocks * KVEV_BLOCK_SIZE * 4;
  return a256((size_t)parts * row * ((want_sum ? 1 : 0) + (drop ? 1 : 0)));
}

int check_window(const kvev_cache *c, const kvev_window *w) {
  if (!w || !w->q || !w->lse || !w->q_pos) return KVEV_EINVAL;
  if (w->group < 1 || w->obs_window < 1) return KVEV_EINVAL;
  if ((int64_t)w->group * w->obs_window > 4096) return KVEV_EUNSUPPORTED;
  if (!std::isfinite(w->scale)) return KVEV_EINVAL;
  (void)c;
  return KVEV_OK;
}

// Workspace of kvev_h2o_step: [arrival counters | error flags] (state, zero
// between calls) then the parts' e values and (max, sum) per row.
struct H2oLayout {
  size_t arrive, err, e, ml, o, total;
  int np, nbmax;
};

H2oLayout h2o_layout(const kvev_cache *c, int32_t group, int32_t budget) {
  H2oLayout L{};
  const size_t units = (size_t)c->batch * c->kv_heads;
  L.nbmax = (budget + KVEV_BLOCK_SIZE - 1) / KVEV_BLOCK_SIZE;
  L.np = (L.nbmax + 1) * KVEV_BLOCK_SIZE;  // every slot, then the new token's e
  size_t off = 0;
  L.arrive = off; off = a256(off + units * 4);
  L.err = off; off = a256(off + units * 4);
  L.e = off; off = a256(off + units * (size_t)group * L.np * 4);
  L.ml = off; off = a256(off + units * (size_t)kvev::kH2oMaxSplit * 32 * 4);
  L.o = off; off = a256(off + units * (size_t)kvev::kH2oMaxSplit * group * c->head_dim * 4);
  L.total = off;
  return L;
}

// Workspace of kvev_ring_step: [arrival counters] (state, zero between
// calls) then the parts' e values, the other ring entries' sums and (max,
// sum) per row.
struct RingLayout {
  size_t arrive, e, rsum, ml, total;
  int np, nbmax;
};

RingLayout ring_layout(const kvev_cache *c, int32_t group, int32_t budget) {
  RingLayout L{};
  const size_t units = (size_t)c->batch * c->kv_heads;
  L.nbmax = (budget + KVEV_BLOCK_SIZE - 1) / KVEV_BLOCK_SIZE;
  L.np = L.nbmax * KVEV_BLOCK_SIZE;
  size_t off = 0;
  L.arrive = off; off = a256(off + units * 4);
  L.e = off; off = a256(off + units * (size_t)group * L.np * 4);
  L.rsum = off; off = a256(off + units * (size_t)L.np * 4);
  L.ml = off; off = a256(off + units * (size_t)kvev::kRingMaxSplit * 32 * 4);
  L.total = off;
  return L;
}

}  // namespace

extern "C" {

int kvev_measure(const int32_t *seq_len_before, const int32_t *victims,
                 const int32_t *n_victims, int32_t units, int32_t max_slots, int64_t *out,
                 void *stream) {
  if (!seq_len_before || !victims || !n_victims || !out || units < 0 || max_slots <= 0 ||
      max_slots % KVEV_BLOCK_SIZE != 0)
    return KVEV_EINVAL;
  if ((int64_t)max_slots / KVEV_BLOCK_SIZE > (int64_t)65535 * 256 || units > 65535)
    return KVEV_EUNSUPPORTED;
  kvev::MeasureArgs a{};
  a.seq_len_before = seq_len_before;
  a.victims = victims;
  a.n_victims = n_victims;
  a.out = out;
  a.units = units;
  a.max_slots = max_slots;
  return map_err(kvev::launch_measure(a, static_cast<hipStream_t>(stream)));
}

size_t kvev_h2o_workspace_bytes(const kvev_cache *cache, int32_t group, int32_t budget) {
  if (!valid_cache(cache) || group < 1 || group > 16 || budget <= 0 ||
      budget > kvev::kH2oMaxBudget)
    return 0;
  return h2o_layout(cache, group, budget).total;
}

int kvev_h2o_step(const kvev_cache *cache, const void *q, const void *k_new, const void *v_new,
                  const int32_t *t_pos, int32_t group, float scale, float *score,
                  int32_t budget, int32_t recent_window, int32_t *free_list,
                  int32_t *free_count, int32_t *evicted_pos, float *attn_out, void *workspace,
                  size_t ws_bytes, void *stream) {
  if (!valid_cache(cache) || !q || !k_new || !v_new || !t_pos || !score || !free_list ||
      !free_count || !evicted_pos)
    return KVEV_EINVAL;
  if (group < 1 || budget <= 0 || recent_window < 0 || recent_window >= budget)
    return KVEV_EINVAL;
  if ((int64_t)budget > (int64_t)cache->max_blocks * KVEV_BLOCK_SIZE) return KVEV_EINVAL;
  if (group > 16 || budget > kvev::kH2oMaxBudget ||
      (int64_t)group * ((budget + KVEV_BLOCK_SIZE - 1) / KVEV_BLOCK_SIZE * KVEV_BLOCK_SIZE) >
          kvev::kH2oMaxLogits)
    return KVEV_EUNSUPPORTED;
  const H2oLayout L = h2o_layout(cache, group, budget);
  if (!workspace || ws_bytes < L.total) return KVEV_ENOSPACE;
  uint8_t *ws = static_cast<uint8_t *>(workspace);
  kvev::H2oArgs a{};
  a.k_pool = static_cast<uint8_t *>(cache->k_pool);
  a.v_pool = static_cast<uint8_t *>(cache->v_pool);
  a.block_table = cache->block_table;
  a.seq_len = cache->seq_len;
  a.pos = cache->pos;
  a.score = score;
  a.q = static_cast<const uint8_t *>(q);
  a.k_new = static_cast<const uint8_t *>(k_new);
  a.v_new = static_cast<const uint8_t *>(v_new);
  a.t_pos = t_pos;
  a.free_list = free_list;
  a.free_count = free_count;
  a.evicted = evicted_pos;
  a.arrive = reinterpret_cast<uint32_t *>(ws + L.arrive);
  a.err = reinterpret_cast<uint32_t *>(ws + L.err);
  a.e = reinterpret_cast<uint32_t *>(ws + L.e);
  a.ml = reinterpret_cast<uint32_t *>(ws + L.ml);
  a.o = reinterpret_cast<float *>(ws + L.o);
  a.attn = attn_out;
  a.units = cache->batch * cache->kv_heads;
  a.Hkv = cache->kv_heads;
  a.G = group;
  a.max_blocks = cache->max_blocks;
  a.max_slots = cache->max_blocks * KVEV_BLOCK_SIZE;
  a.num_blocks = cache->num_blocks;
  a.budget = budget;
  a.recent = recent_window;
  a.np = L.np;
  // enough workgroups to cover the CUs, at most one per block of the budget
  const int want = (256 + a.units - 1) / a.units;
  a.split = std::max(1, std::min({want, kvev::kH2oMaxSplit, L.nbmax}));
  a.c1 = scale * 1.4426950408889634f;
  // the shapes the limits above admit can still need more LDS with the
  // attention output (rows rounded up to 4, few parts): refuse those
  if (kvev::h2o_lds_bytes(a, cache->head_dim) > kMaxLds - 4096) return KVEV_EUNSUPPORTED;
  return map_err(kvev::launch_h2o_step(a, cache->dtype == KVEV_BF16, cache->head_dim,
                                       static_cast<hipStream_t>(stream)));
}

int kvev_abi_version(void) { return KVEV_ABI_VERSION; }

const char *kvev_strerror(int status) {
  switch (status) {
    case KVEV_OK: return "ok";
    case KVEV_EINVAL: return "invalid argument";
    case KVEV_ENOSPACE: return "workspace or free list too small";
    case KVEV_EUNSUPPORTED: return "shape or dtype not supported by the kernels";
    case KVEV_EDEVICE: return "HIP launch failed";
    default: return "unknown status";
  }
}

size_t kvev_workspace_bytes(const kvev_cache *cache, int32_t group, int32_t obs_window) {
  if (!valid_cache(cache)) return 0;
  // the main workspace, then (large windows) the split rows' raw sums
  size_t need = main_layout_total(cache) + score_parts_bytes(cache, group, obs_window, 1, 1);
  if (group >= 1 && obs_window >= 1) {
    const size_t wa = wa_layout(cache, group, obs_window).total;
    if (wa > need) need = wa;
  }
  return need;
}

}  // extern "C"

namespace {

// Validates the score arguments and fills the kernel's argument block and
// its LDS size.  Nothing is enqueued.
int build_score_args(const kvev_cache *cache, const kvev_window *win, int32_t flags,
                     int32_t pool_kernel, float *sum, float *pooled, float *drop, int hist,
                     kvev::ScoreArgs &a) {
  // (split windows: the caller points part_sum / part_drop at its workspace)
  if (!valid_cache(cache)) return KVEV_EINVAL;
  int rc = check_window(cache, win);
  if (rc) return rc;
  if (flags == 0 || (flags & ~(KVEV_SUM | KVEV_POOL | KVEV_DROP | KVEV_ACCUMULATE))) return KVEV_EINVAL;
  if (!(flags & (KVEV_SUM | KVEV_POOL | KVEV_DROP))) return KVEV_EINVAL;
  if ((flags & KVEV_SUM) && !sum) return KVEV_EINVAL;
  if (flags & KVEV_POOL) {
    if (!pooled || pool_kernel < 1 || pool_kernel % 2 == 0) return KVEV_EINVAL;
    if (pool_kernel > kMaxPoolKernel) return KVEV_EUNSUPPORTED;
  }
  if ((flags & KVEV_DROP) && (!drop || !win->a)) return KVEV_EINVAL;
  if ((flags & KVEV_ACCUMULATE) && (!(flags & KVEV_SUM) || (flags & (KVEV_POOL | KVEV_DROP))))
    return KVEV_EINVAL;

  a = kvev::ScoreArgs{};
  a.k_pool = static_cast<const uint8_t *>(cache->k_pool);
  a.v_pool = static_cast<const uint8_t *>(cache->v_pool);
  a.block_table = cache->block_table;
  a.seq_len = cache->seq_len;
  a.pos = cache->pos;
  a.q = static_cast<const uint8_t *>(win->q);
  a.a = win->a;
  a.lse = win->lse;
  a.q_pos = win->q_pos;
  a.sum = sum;
  a.pooled = pooled;
  a.drop = drop;
  a.prev = sum;
  a.head_err = nullptr;
  a.units = cache->batch * cache->kv_heads;
  a.Hkv = cache->kv_heads;
  a.G = win->group;
  a.W = win->obs_window;
  a.max_blocks = cache->max_blocks;
  a.num_blocks = cache->num_blocks;
  a.rows = win->group * win->obs_window;
  a.row_tiles = (a.rows + 15) / 16;
  a.flags = flags & (KVEV_SUM | KVEV_POOL | KVEV_ACCUMULATE);
  a.pool_r = (flags & KVEV_POOL) ? (pool_kernel - 1) / 2 : 0;
  const int bf16 = cache->dtype == KVEV_BF16;
  const int is_drop = (flags & KVEV_DROP) ? 1 : 0;
  a.row_parts = score_row_parts(bf16, cache->head_dim, is_drop, a.row_tiles, &a.rt_part);
  if (a.row_parts > 1) hist = 0;  // the combine pass builds the histogram
  // split windows pool in the combine pass: no halo blocks
  a.halo_blocks =
      a.row_parts > 1 ? 0 : (a.pool_r + KVEV_BLOCK_SIZE - 1) / KVEV_BLOCK_SIZE;
  // Up to 8 waves (512 threads) share one staging of the window rows and
  // split a tile of up to 256 blocks; smaller tiles when the tiles would not
  // cover the 256 CUs, and down to two tiles per CU while what each tile
  // stages besides its own keys (the window rows, with the attention output
  // for DropKV, and the halo blocks) stays within a sixteenth of its key
  // bytes (one CU pulls more bytes at once with two workgroups; a
  // single-query decode window tiles finer, a 32-query prefill window does
  // not); smaller again when the staged window rows plus the tile's score
  // rows exceed a workgroup's LDS (large G*W windows); fewer waves for small
  // tiles.
  auto lds_of = [&](int t) {
    return kvev::score_lds_bytes(bf16, cache->head_dim, is_drop, a.rt_part, t, a.halo_blocks,
                                 hist);
  };
  // fp32 DropKV at head_dim 128: two stages of key and value fragments fill
  // 256 registers, so one wave per SIMD (4 waves, 512 registers each)
  const int max_threads = (!bf16 && cache->head_dim == 128 && is_drop) ? 256 : KV_THREADS_MAX;
  int tb = KV_TILE_MAX, threads = max_threads;
  auto tiles_of = [&](int t) {
    return (int64_t)a.units * ((cache->max_blocks + t - 1) / t) * a.row_parts;
  };
  while (tb > 16 && tiles_of(tb) < 256) tb /= 2;
  const int64_t row_bytes = (int64_t)cache->head_dim * (bf16 ? 2 : 4);
  const int64_t block_bytes = (int64_t)KVEV_BLOCK_SIZE * row_bytes * (is_drop ? 2 : 1);
  const int64_t staged = (int64_t)a.rt_part * 16 * row_bytes * (is_drop ? (bf16 ? 3 : 2) : 1) +
                         2 * (int64_t)a.halo_blocks * block_bytes;
  while (tb > 16 && tiles_of(tb) < 512 && staged * 16 <= (int64_t)(tb / 2) * block_bytes) tb /= 2;
  while (tb > 1 && lds_of(tb) > kMaxLds - 1024) tb /= 2;
  if (lds_of(tb) > kMaxLds - 1024) return KVEV_EUNSUPPORTED;
  while (threads > 256 && tb < 16 * (threads / 64)) threads /= 2;
  // a wave indexes its block range by lane: at most 64 blocks per wave
  while (tb > 1 && (tb + 2 * a.halo_blocks + threads / 64 - 1) / (threads / 64) > 64) tb /= 2;
  a.tile_blocks = tb;
  a.threads = threads;
  a.tiles_per_head = (cache->max_blocks + tb - 1) / tb;
  a.c1 = win->scale * 1.4426950408889634f;
  a.scale = win->scale;
  if ((int64_t)a.units * a.tiles_per_head * a.row_parts > INT32_MAX) return KVEV_EUNSUPPORTED;
  return KVEV_OK;
}

// Points a split window's raw sums at `ws` (the caller checked its size).
void set_score_parts(kvev::ScoreArgs &a, const kvev_cache *c, uint8_t *ws) {
  if (a.row_parts == 1) return;
  const size_t row = (size_t)a.units * c->max_blocks * KVEV_BLOCK_SIZE;
  float *p = reinterpret_cast<float *>(ws);
  const bool want_sum = (a.flags & (KVEV_SUM | KVEV_POOL)) != 0;
  a.part_sum = want_sum ? p : nullptr;
  a.part_drop = a.drop ? p + (want_sum ? (size_t)a.row_parts * row : 0) : nullptr;
}

// Fills the compaction argument block (workspace pointers included).
void fill_compact_args(kvev_cache *cache, float *score_or_null, int32_t *free_list,
                       int32_t *free_count, int32_t free_capacity, int64_t *stats,
                       void *workspace, kvev::CompactArgs &a) {
  uint8_t *ws = static_cast<uint8_t *>(workspace);
  const CompactLayout L = compact_layout(cache);
  const StateLayout S = state_layout(cache);
  a.k_pool = static_cast<uint8_t *>(cache->k_pool);
  a.v_pool = static_cast<uint8_t *>(cache->v_pool);
  a.block_table = cache->block_table;
  a.seq_len = cache->seq_len;
  a.pos = cache->pos;
  a.score = score_or_null;
  a.free_list = free_list;
  a.free_count = free_count;
  a.stats = stats;
  a.src_of = reinterpret_cast<int32_t *>(ws + L.src_of);
  a.src_row = reinterpret_cast<int32_t *>(ws + L.src_row);
  a.new_pos = reinterpret_cast<int32_t *>(ws + L.new_pos);
  a.new_score = reinterpret_cast<float *>(ws + L.new_score);
  a.stage_k = ws + L.stage_k;
  a.stage_v = ws + L.stage_v;
  a.head_info = reinterpret_cast<int32_t *>(ws + L.head_info);
  a.head_acc = reinterpret_cast<unsigned long long *>(ws + S.head_acc);
  a.fc0 = reinterpret_cast<int32_t *>(ws + L.fc0);
  a.units = cache->batch * cache->kv_heads;
  a.max_blocks = cache->max_blocks;
  a.max_slots = cache->max_blocks * KVEV_BLOCK_SIZE;
  a.num_blocks = cache->num_blocks;
  a.row_bytes = cache->head_dim * elem_bytes(cache);
  a.stage_rows = L.stage_rows;
  a.chunks = L.chunks;
  a.free_capacity = free_capacity;
  a.rows_per_item = 4 * 256 / (a.row_bytes / 16);  // compact.hip: 4 rows per thread
  a.rows_cap = a.max_slots;
}

kvev::SelHead sel_head(const kvev_cache *cache, int32_t *n_victims, int32_t budget,
                       int32_t recent_window, void *workspace) {
  uint8_t *ws = static_cast<uint8_t *>(workspace);
  const StateLayout S = state_layout(cache);
  const SelectLayout L = select_layout(cache);
  kvev::SelHead h{};
  h.n_victims = n_victims;
  h.hist = reinterpret_cast<uint32_t *>(ws + S.hist);
  h.hist2 = reinterpret_cast<uint32_t *>(ws + S.hist2);
  h.head_sel = reinterpret_cast<uint32_t *>(ws + L.head_sel);
  h.chunk_off = reinterpret_cast<uint32_t *>(ws + L.chunk_off);
  h.chunk_below = reinterpret_cast<uint32_t *>(ws + L.chunk_below);
  h.cand = reinterpret_cast<uint2 *>(ws + L.cand);
  h.ccount = reinterpret_cast<uint32_t *>(ws + L.ccount);
  h.budget = budget;
  h.recent = recent_window;
  h.chunks = L.chunks;
  h.nwg = L.nwg;
  return h;
}

}  // namespace

namespace {

// The vToken entry points' scratch starts past the state part, so that a
// buffer shared with kvev_select / kvev_compact / kvev_evict keeps its
// zero state.
size_t vtok_base(const kvev_cache *c) { return state_layout(c).total; }

// Workspace of kvev_vtok_reclaim (scratch only).
struct VtokLayout {
  size_t plan, src, srcoff, dstw, dst_off, push_off, tpos, tscore, misc, total;
};

VtokLayout vtok_layout(const kvev_cache *c, int32_t max_sources) {
  VtokLayout L{};
  const size_t units = (size_t)c->batch * c->kv_heads, ms = (size_t)max_sources;
  size_t off = vtok_base(c);
  L.plan = off; off = a256(off + units * 8 * 4);
  L.src = off; off = a256(off + units * ms * 4);
  L.srcoff = off; off = a256(off + units * ms * 4);
  L.dstw = off; off = a256(off + units * ms * 4);
  L.dst_off = off; off = a256(off + units * 4);
  L.push_off = off; off = a256(off + units * 4);
  L.tpos = off; off = a256(off + units * ms * KVEV_BLOCK_SIZE * 4);
  L.tscore = off; off = a256(off + units * ms * KVEV_BLOCK_SIZE * 4);
  L.misc = off; off = a256(off + 8 * 4);
  L.total = off;
  return L;
}

// Workspace of kvev_vtok_evict: a claim word per slot, past the state part.
size_t vtok_evict_ws(const kvev_cache *c) {
  return vtok_base(c) + a256((size_t)c->batch * c->kv_heads * c->max_blocks * KVEV_BLOCK_SIZE * 4);
}

bool misaligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) != 0; }

kvev::VtokArgs vtok_args(const kvev_cache *cache, uint8_t *live, int32_t *block_live) {
  kvev::VtokArgs a{};
  a.k_pool = static_cast<uint8_t *>(cache->k_pool);
  a.v_pool = static_cast<uint8_t *>(cache->v_pool);
  a.block_table = cache->block_table;
  a.seq_len = cache->seq_len;
  a.pos = cache->pos;
  a.live = live;
  a.block_live = block_live;
  a.units = cache->batch * cache->kv_heads;
  a.Hkv = cache->kv_heads;
  a.max_blocks = cache->max_blocks;
  a.max_slots = cache->max_blocks * KVEV_BLOCK_SIZE;
  a.num_blocks = cache->num_blocks;
  a.row_bytes = cache->head_dim * elem_bytes(cache);
  return a;
}

// Workspace of kvev_select_shared: the selection's regions for a view of
// the cache with one head per sequence, then the shared rows and victims.
struct SharedLayout {
  StateLayout S;
  SelectLayout L;
  size_t row, vvict, vnv, total;
};

kvev_cache shared_view(const kvev_cache *c) {
  kvev_cache v = *c;
  v.kv_heads = 1;
  return v;
}

SharedLayout shared_layout(const kvev_cache *c) {
  const kvev_cache v = shared_view(c);
  SharedLayout X{};
  X.S = state_layout(&v);
  X.L = select_layout(&v);
  const size_t ms = (size_t)c->max_blocks * KVEV_BLOCK_SIZE, B = (size_t)c->batch;
  size_t off = X.L.total;
  X.row = off; off = a256(off + B * ms * 4);
  X.vvict = off; off = a256(off + B * ms * 4);
  X.vnv = off; off = a256(off + B * 4);
  X.total = off;
  return X;
}

}  // namespace

extern "C" {

size_t kvev_vtok_evict_workspace_bytes(const kvev_cache *cache) {
  return valid_cache(cache) ? vtok_evict_ws(cache) : 0;
}

int kvev_vtok_evict(const kvev_cache *cache, uint8_t *live, int32_t *block_live,
                    const int32_t *victims, const int32_t *n_victims, int32_t *status,
                    void *workspace, size_t ws_bytes, void *stream) {
  if (!valid_cache(cache) || !live || !block_live || !victims || !n_victims || !status)
    return KVEV_EINVAL;
  if (misaligned16(live)) return KVEV_EINVAL;
  if (!workspace || ws_bytes < vtok_evict_ws(cache)) return KVEV_ENOSPACE;
  if (misaligned16(workspace)) return KVEV_EINVAL;
  kvev::VtokArgs a = vtok_args(cache, live, block_live);
  a.victims = victims;
  a.n_victims = n_victims;
  a.status = status;
  a.claim = reinterpret_cast<int32_t *>(static_cast<uint8_t *>(workspace) + vtok_base(cache));
  return map_err(kvev::launch_vtok_evict(a, static_cast<hipStream_t>(stream)));
}

size_t kvev_vtok_workspace_bytes(const kvev_cache *cache, int32_t max_sources) {
  if (!valid_cache(cache) || max_sources < 2 || max_sources > kvev::kVtokMaxSources) return 0;
  return vtok_layout(cache, max_sources).total;
}

int kvev_vtok_reclaim(const kvev_cache *cache, uint8_t *live, int32_t *block_live,
                      float *score_or_null, double theta_f, int32_t max_sources,
                      int32_t *free_list, int32_t *free_count, int32_t free_capacity,
                      int64_t *stats, void *workspace, size_t ws_bytes, void *stream) {
  if (!valid_cache(cache) || !live || !block_live || !free_list || !free_count || !stats)
    return KVEV_EINVAL;
  if (misaligned16(live) || misaligned16(cache->pos) || misaligned16(score_or_null))
    return KVEV_EINVAL;
  if (!(theta_f >= 0.0 && theta_f < 1.0)) return KVEV_EINVAL;  // NaN refused too
  if (max_sources < 2 || max_sources > kvev::kVtokMaxSources) return KVEV_EINVAL;
  if ((int64_t)cache->batch * cache->kv_heads > kvev::kVtokMaxUnits) return KVEV_EUNSUPPORTED;
  if (free_capacity < cache->num_blocks) return KVEV_ENOSPACE;
  const VtokLayout L = vtok_layout(cache, max_sources);
  if (!workspace || ws_bytes < L.total) return KVEV_ENOSPACE;
  if (misaligned16(workspace)) return KVEV_EINVAL;
  uint8_t *ws = static_cast<uint8_t *>(workspace);
  kvev::VtokArgs a = vtok_args(cache, live, block_live);
  a.score = score_or_null;
  a.free_list = free_list;
  a.free_count = free_count;
  a.stats = stats;
  a.max_sources = max_sources;
  a.free_capacity = free_capacity;
  a.theta_f = theta_f;
  a.plan = reinterpret_cast<int32_t *>(ws + L.plan);
  a.src = reinterpret_cast<int32_t *>(ws + L.src);
  a.srcoff = reinterpret_cast<int32_t *>(ws + L.srcoff);
  a.dstw = reinterpret_cast<int32_t *>(ws + L.dstw);
  a.dst_off = reinterpret_cast<int32_t *>(ws + L.dst_off);
  a.push_off = reinterpret_cast<int32_t *>(ws + L.push_off);
  a.tpos = reinterpret_cast<int32_t *>(ws + L.tpos);
  a.tscore = reinterpret_cast<float *>(ws + L.tscore);
  a.misc = reinterpret_cast<int32_t *>(ws + L.misc);
  return map_err(kvev::launch_vtok_reclaim(a, static_cast<hipStream_t>(stream)));
}

int kvev_vtok_digest(const kvev_cache *cache, const uint8_t *live, uint64_t *digest,
                     void *stream) {
  if (!valid_cache(cache) || !live || !digest) return KVEV_EINVAL;
  if (misaligned16(live) || (reinterpret_cast<uintptr_t>(digest) & 7)) return KVEV_EINVAL;
  kvev::VtokArgs a = vtok_args(cache, const_cast<uint8_t *>(live), nullptr);
  return map_err(kvev::launch_vtok_digest(a, digest, static_cast<hipStream_t>(stream)));
}

size_t kvev_vtok_check_workspace_bytes(const kvev_cache *cache) {
  return valid_cache(cache) ? vtok_base(cache) + a256(((size_t)cache->num_blocks + 1) / 2 * 8) : 0;
}

int kvev_vtok_check(const kvev_cache *cache, const uint8_t *live, const int32_t *block_live,
                    const int32_t *free_list, const int32_t *free_count, int32_t free_capacity,
                    int64_t *out, void *workspace, size_t ws_bytes, void *stream) {
  if (!valid_cache(cache) || !live || !block_live || !free_list || !free_count || !out)
    return KVEV_EINVAL;
  if (misaligned16(live) || (reinterpret_cast<uintptr_t>(out) & 7) || free_capacity < 0)
    return KVEV_EINVAL;
  if (!workspace || ws_bytes < kvev_vtok_check_workspace_bytes(cache)) return KVEV_ENOSPACE;
  if (misaligned16(workspace)) return KVEV_EINVAL;
  kvev::VtokArgs a = vtok_args(cache, const_cast<uint8_t *>(live),
                               const_cast<int32_t *>(block_live));
  a.free_list = const_cast<int32_t *>(free_list);
  a.free_count = const_cast<int32_t *>(free_count);
  a.free_capacity = free_capacity;
  return map_err(kvev::launch_vtok_check(
      a, reinterpret_cast<int32_t *>(static_cast<uint8_t *>(workspace) + vtok_base(cache)), out,
      static_cast<hipStream_t>(stream)));
}

int kvev_score(const kvev_cache *cache, const kvev_window *win, int32_t flags,
               int32_t pool_kernel, float *sum, float *pooled, float *drop, void *workspace,
               size_t ws_bytes, void *stream) {
  kvev::ScoreArgs a;
  const int rc = build_score_args(cache, win, flags, pool_kernel, sum, pooled, drop, 0, a);
  if (rc) return rc;
  if (a.row_parts > 1) {
    // the split rows' raw sums go to the workspace past its main part (whose
    // state the other entry points keep)
    const size_t need = main_layout_total(cache) +
                        score_parts_bytes(cache, win->group, win->obs_window, a.drop != nullptr,
                                          (a.flags & (KVEV_SUM | KVEV_POOL)) != 0);
    if (!workspace || ws_bytes < need) return KVEV_ENOSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) & 15) return KVEV_EINVAL;
    set_score_parts(a, cache, static_cast<uint8_t *>(workspace) + main_layout_total(cache));
  }
  return map_err(kvev::launch_score(a, cache->dtype == KVEV_BF16, cache->head_dim,
                                    (flags & KVEV_DROP) ? 1 : 0, static_cast<hipStream_t>(stream)));
}

int kvev_select(const kvev_cache *cache, const float *score, int32_t budget,
                int32_t recent_window, int32_t *victims, int32_t *n_victims, void *workspace,
                size_t ws_bytes, void *stream) {
  if (!valid_cache(cache) || !score || !victims || !n_victims) return KVEV_EINVAL;
  if (reinterpret_cast<uintptr_t>(score) & 15) return KVEV_EINVAL;
  if (budget <= 0 || recent_window < 0 || recent_window >= budget) return KVEV_EINVAL;
  const SelectLayout L = select_layout(cache);
  if (L.chunks > kvev::kSelectMaxChunks) return KVEV_EUNSUPPORTED;
  if (!workspace || ws_bytes < L.total) return KVEV_ENOSPACE;
  kvev::SelectArgs a{};
  a.score = score;
  a.seq_len = cache->seq_len;
  a.victims = victims;
  a.sel = sel_head(cache, n_victims, budget, recent_window, workspace);
  a.units = cache->batch * cache->kv_heads;
  a.max_slots = cache->max_blocks * KVEV_BLOCK_SIZE;
  return map_err(kvev::launch_select(a, static_cast<hipStream_t>(stream)));
}

int kvev_compact(const kvev_cache *cache, const int32_t *victims, const int32_t *n_victims,
                 float *score_or_null, int32_t *free_list, int32_t *free_count,
                 int32_t free_capacity, int64_t *stats, void *workspace, size_t ws_bytes,
                 void *stream) {
  if (!valid_cache(cache) || !victims || !n_victims || !free_list || !free_count || !stats)
    return KVEV_EINVAL;
  if (free_capacity < cache->num_blocks) return KVEV_ENOSPACE;
  if (cache->batch * cache->kv_heads > kvev::kCompactMaxUnits) return KVEV_EUNSUPPORTED;
  const CompactLayout L = compact_layout(cache);
  if (L.chunks > kvev::kSelectMaxChunks) return KVEV_EUNSUPPORTED;  // 1M slots per head
  if (!workspace || ws_bytes < L.total) return KVEV_ENOSPACE;
  kvev::CompactArgs a{};
  fill_compact_args(const_cast<kvev_cache *>(cache), score_or_null, free_list, free_count,
                    free_capacity, stats, workspace, a);
  a.victims = victims;
  a.n_victims = n_victims;
  return map_err(kvev::launch_compact(a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// kvev_evict on the workspace `workspace` (ws_bytes long), a split window's
// raw sums at parts_off (past the pass's own layout); clear_state first
// zeroes the state part with a fill kernel (the no-allocation entry point,
// whose static array keeps the last call's contents).
int evict_impl(const kvev_cache *cache, const kvev_window *win, int32_t flags,
               int32_t pool_kernel, int32_t budget, int32_t recent_window, float *score,
               int32_t *victims, int32_t *n_victims, int32_t *free_list, int32_t *free_count,
               int32_t free_capacity, int64_t *stats, void *workspace, size_t ws_bytes,
               size_t parts_off, bool clear_state, void *stream) {
  if (!valid_cache(cache) || !score || !victims || !n_victims || !free_list || !free_count ||
      !stats)
    return KVEV_EINVAL;
  if (reinterpret_cast<uintptr_t>(score) & 15) return KVEV_EINVAL;
  const int kind = flags & (KVEV_SUM | KVEV_POOL | KVEV_DROP);
  if (kind != KVEV_SUM && kind != KVEV_POOL && kind != KVEV_DROP) return KVEV_EINVAL;
  if (budget <= 0 || recent_window < 0 || recent_window >= budget) return KVEV_EINVAL;
  if (reinterpret_cast<uintptr_t>(workspace) & 15) return KVEV_EINVAL;
  const StateLayout S = state_layout(cache);
  const EvictLayout E = evict_layout(cache);
  // this pass's scores go to the workspace row; the output row receives them
  // compacted (the address is formed before the workspace is checked, and
  // used only after)
  float *sc = reinterpret_cast<float *>(reinterpret_cast<uintptr_t>(workspace) + E.sc);
  kvev::ScoreArgs a;
  int rc = build_score_args(cache, win, flags, pool_kernel, kind == KVEV_SUM ? sc : nullptr,
                            kind == KVEV_POOL ? sc : nullptr, kind == KVEV_DROP ? sc : nullptr, 1,
                            a);
  if (rc) return rc;
  if (free_capacity < cache->num_blocks) return KVEV_ENOSPACE;
  if ((size_t)cache->max_blocks * KVEV_BLOCK_SIZE >
      (size_t)kvev::kSelectMaxChunks * kvev::kSelectChunk)
    return KVEV_EUNSUPPORTED;  // 1M slots per head
  const size_t parts_bytes = score_parts_bytes(cache, win->group, win->obs_window,
                                               kind == KVEV_DROP, kind != KVEV_DROP);
  // the pass uses the state, its own scratch (E) and the split rows' sums
  if (parts_off < E.total) return KVEV_EINVAL;
  if (!workspace || ws_bytes < parts_off + parts_bytes) return KVEV_ENOSPACE;
  uint8_t *ws = static_cast<uint8_t *>(workspace);
  set_score_parts(a, cache, ws + parts_off);
  a.prev = score;  // ACCUMULATE: the running sums are in the output row
  a.head_err = reinterpret_cast<uint32_t *>(ws + S.fin_err);
  a.hist = reinterpret_cast<uint32_t *>(ws + S.hist);
  a.sel_budget = budget;
  a.sel_recent = recent_window;
  kvev::FinishArgs f{};
  f.k_pool = static_cast<uint8_t *>(cache->k_pool);
  f.v_pool = static_cast<uint8_t *>(cache->v_pool);
  f.block_table = cache->block_table;
  f.seq_len = cache->seq_len;
  f.pos = cache->pos;
  f.sc = sc;
  f.score_out = score;
  f.victims = victims;
  f.n_victims = n_victims;
  f.free_list = free_list;
  f.free_count = free_count;
  f.stats = stats;
  f.head_err = a.head_err;
  f.hist = a.hist;
  f.hist2 = reinterpret_cast<uint32_t *>(ws + S.hist2);
  f.nmem = reinterpret_cast<uint32_t *>(ws + S.fin_nmem);
  f.arrive = reinterpret_cast<uint32_t *>(ws + S.fin_arrive);
  f.mem = reinterpret_cast<uint2 *>(ws + E.mem);
  f.gbelow = reinterpret_cast<uint32_t *>(ws + E.gbelow);
  f.chunks = E.chunks;
  f.marks = reinterpret_cast<uint32_t *>(ws + S.fin_marks);
  f.head_done = reinterpret_cast<uint32_t *>(ws + S.fin_done);
  f.ctr = reinterpret_cast<uint32_t *>(ws + S.fin_ctr);
  f.bctr = reinterpret_cast<uint32_t *>(ws + S.fin_bctr);
  f.acc = reinterpret_cast<unsigned long long *>(ws + S.fin_acc);
  f.units = cache->batch * cache->kv_heads;
  f.max_blocks = cache->max_blocks;
  f.max_slots = cache->max_blocks * KVEV_BLOCK_SIZE;
  f.num_blocks = cache->num_blocks;
  f.row_bytes = cache->head_dim * elem_bytes(cache);
  f.budget = budget;
  f.recent = recent_window;
  f.kh = kvev::finish_parts(f.units, std::min(budget, f.max_slots));
  f.marks_per_head = S.marks_per_head;
  f.free_capacity = free_capacity;
  if ((int64_t)f.units * f.kh > INT32_MAX) return KVEV_EUNSUPPORTED;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (clear_state) {
    const size_t n16 = S.total / 16;  // S.total is a multiple of 256
    hipLaunchKernelGGL(clear16_kernel, dim3((unsigned)std::min<size_t>((n16 + 255) / 256, 1024)),
                       dim3(256), 0, st, reinterpret_cast<uint4 *>(ws), n16);
    rc = map_err(hipGetLastError());
    if (rc) return rc;
  }
  rc = map_err(kvev::launch_score(a, cache->dtype == KVEV_BF16, cache->head_dim,
                                  kind == KVEV_DROP, st));
  if (rc) return rc;
  return map_err(kvev::launch_finish(f, st));
}

// The no-allocation entry point's scratch: one static array per GPU.  Host
// code never passes the array's name to a kernel (on the host it is only a
// stand-in): each device's address is looked up once, with that device
// current, and kept.
constexpr size_t kNoAllocBytes = KVEV_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kNoAllocBytes];
constexpr int kMaxDevices = 64;
std::atomic<uint8_t *> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

int scratch_of_current_device(uint8_t **out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return KVEV_EDEVICE;
  if (dev < 0 || dev >= kMaxDevices) return KVEV_EUNSUPPORTED;
  uint8_t *p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      void *addr = nullptr;
      if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || !addr)
        return KVEV_EDEVICE;
      p = static_cast<uint8_t *>(addr);
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return KVEV_OK;
}

}  // namespace

extern "C" {

int kvev_evict(const kvev_cache *cache, const kvev_window *win, int32_t flags,
               int32_t pool_kernel, int32_t budget, int32_t recent_window, float *score,
               int32_t *victims, int32_t *n_victims, int32_t *free_list, int32_t *free_count,
               int32_t free_capacity, int64_t *stats, void *workspace, size_t ws_bytes,
               void *stream) {
  return evict_impl(cache, win, flags, pool_kernel, budget, recent_window, score, victims,
                    n_victims, free_list, free_count, free_capacity, stats, workspace, ws_bytes,
                    valid_cache(cache) ? main_layout_total(cache) : 0, false, stream);
}

int kvev_evict_noalloc(const kvev_cache *cache, const kvev_window *win, int32_t flags,
                       int32_t pool_kernel, int32_t budget, int32_t recent_window, float *score,
                       int32_t *victims, int32_t *n_victims, int32_t *free_list,
                       int32_t *free_count, int32_t free_capacity, int64_t *stats,
                       void *stream) {
  if (!valid_cache(cache)) return KVEV_EINVAL;
  uint8_t *ws = nullptr;
  const int rc = scratch_of_current_device(&ws);
  if (rc) return rc;
  return evict_impl(cache, win, flags, pool_kernel, budget, recent_window, score, victims,
                    n_victims, free_list, free_count, free_capacity, stats, ws, kNoAllocBytes,
                    evict_layout(cache).total, true, stream);
}


int kvev_window_attn(const kvev_cache *cache, const kvev_window *win, float *lse_out,
                     float *a_out, void *workspace, size_t ws_bytes, void *stream) {
  if (!valid_cache(cache) || !win || !win->q || !win->q_pos || !lse_out) return KVEV_EINVAL;
  if (win->group < 1 || win->obs_window < 1) return KVEV_EINVAL;
  if ((int64_t)win->group * win->obs_window > 4096) return KVEV_EUNSUPPORTED;
  if (!std::isfinite(win->scale)) return KVEV_EINVAL;
  const WaLayout L = wa_layout(cache, win->group, win->obs_window);
  if (!workspace || ws_bytes < L.total) return KVEV_ENOSPACE;
  uint8_t *ws = static_cast<uint8_t *>(workspace);
  kvev::WindowAttnArgs a{};
  a.k_pool = static_cast<const uint8_t *>(cache->k_pool);
  a.v_pool = static_cast<const uint8_t *>(cache->v_pool);
  a.block_table = cache->block_table;
  a.seq_len = cache->seq_len;
  a.pos = cache->pos;
  a.q = static_cast<const uint8_t *>(win->q);
  a.q_pos = win->q_pos;
  a.lse_out = lse_out;
  a.a_out = a_out;
  a.part_m = reinterpret_cast<float *>(ws + L.part_m);
  a.part_l = reinterpret_cast<float *>(ws + L.part_l);
  a.part_acc = reinterpret_cast<float *>(ws + L.part_acc);
  a.units = cache->batch * cache->kv_heads;
  a.Hkv = cache->kv_heads;
  a.G = win->group;
  a.W = win->obs_window;
  a.max_blocks = cache->max_blocks;
  a.num_blocks = cache->num_blocks;
  a.rows = win->group * win->obs_window;
  const WaShape sh = wa_shape(cache, a.rows);
  a.chunk_slots = sh.chunk_slots;
  a.chunks = sh.chunks;
  a.threads = sh.threads;
  a.rt_wave = sh.rt_wave;
  a.row_parts = sh.row_parts;
  if ((int64_t)a.units * a.row_parts > 65535) return KVEV_EUNSUPPORTED;  // grid rows
  a.want_a = a_out ? 1 : 0;
  if (kvev::window_attn_lds_bytes(cache->dtype == KVEV_BF16, cache->head_dim, a.want_a,
                                  a.chunk_slots) > kMaxLds - 1024)
    return KVEV_EUNSUPPORTED;
  a.scale = win->scale;
  return map_err(kvev::launch_window_attn(a, cache->dtype == KVEV_BF16, cache->head_dim,
                                          static_cast<hipStream_t>(stream)));
}


size_t kvev_select_shared_workspace_bytes(const kvev_cache *cache) {
  return valid_cache(cache) ? shared_layout(cache).total : 0;
}

int kvev_select_shared(const kvev_cache *cache, const float *score, int32_t budget,
                       int32_t recent_window, int32_t *victims, int32_t *n_victims,
                       void *workspace, size_t ws_bytes, void *stream) {
  if (!valid_cache(cache) || !score || !victims || !n_victims) return KVEV_EINVAL;
  if (misaligned16(score) || misaligned16(workspace)) return KVEV_EINVAL;
  if (budget <= 0 || recent_window < 0 || recent_window >= budget) return KVEV_EINVAL;
  const SharedLayout X = shared_layout(cache);
  if (X.L.chunks > kvev::kSelectMaxChunks) return KVEV_EUNSUPPORTED;
  if (!workspace || ws_bytes < X.total) return KVEV_ENOSPACE;
  uint8_t *ws = static_cast<uint8_t *>(workspace);
  const kvev_cache v = shared_view(cache);
  kvev::SharedArgs a{};
  a.score = score;
  a.seq_len = cache->seq_len;
  a.pos = cache->pos;
  a.row = reinterpret_cast<float *>(ws + X.row);
  a.vseq = reinterpret_cast<int32_t *>(ws + X.S.head_acc);  // unused by a selection
  a.vvict = reinterpret_cast<int32_t *>(ws + X.vvict);
  a.vnv = reinterpret_cast<int32_t *>(ws + X.vnv);
  a.victims = victims;
  a.n_victims = n_victims;
  a.zero = reinterpret_cast<uint32_t *>(ws);  // histograms and lengths
  a.zero_words = X.S.total / 4;
  a.B = cache->batch;
  a.Hkv = cache->kv_heads;
  a.max_slots = cache->max_blocks * KVEV_BLOCK_SIZE;
  a.sel.score = a.row;
  a.sel.seq_len = a.vseq;
  a.sel.victims = a.vvict;
  a.sel.sel = sel_head(&v, a.vnv, budget, recent_window, workspace);
  a.sel.units = cache->batch;
  a.sel.max_slots = a.max_slots;
  return map_err(kvev::launch_select_shared(a, static_cast<hipStream_t>(stream)));
}


int kvev_select_budgets(const kvev_cache *cache, const float *score, const int32_t *budget,
                        const int32_t *recent_window, int32_t *victims, int32_t *n_victims,
                        void *workspace, size_t ws_bytes, void *stream) {
  if (!valid_cache(cache) || !score || !budget || !recent_window || !victims || !n_victims)
    return KVEV_EINVAL;
  if (misaligned16(score)) return KVEV_EINVAL;
  const SelectLayout L = select_layout(cache);
  if (L.chunks > kvev::kSelectMaxChunks) return KVEV_EUNSUPPORTED;
  if (!workspace || ws_bytes < L.total) return KVEV_ENOSPACE;
  kvev::SelectArgs a{};
  a.score = score;
  a.seq_len = cache->seq_len;
  a.victims = victims;
  a.sel = sel_head(cache, n_victims, 1, 0, workspace);
  a.sel.budget_u = budget;
  a.sel.recent_u = recent_window;
  a.units = cache->batch * cache->kv_heads;
  a.max_slots = cache->max_blocks * KVEV_BLOCK_SIZE;
  return map_err(kvev::launch_select(a, static_cast<hipStream_t>(stream)));
}


int kvev_ring_init(const kvev_cache *cache, float *hist, int32_t *ring, int32_t *rank,
                   int32_t obs_window, void *stream) {
  if (!valid_cache(cache) || !hist || !ring || !rank || obs_window < 1) return KVEV_EINVAL;
  kvev::RingArgs a{};
  a.seq_len = cache->seq_len;
  a.pos = cache->pos;
  a.hist = hist;
  a.ring = ring;
  a.rank = rank;
  a.units = cache->batch * cache->kv_heads;
  a.W = obs_window;
  a.max_slots = cache->max_blocks * KVEV_BLOCK_SIZE;
  return map_err(kvev::launch_ring_init(a, static_cast<hipStream_t>(stream)));
}

size_t kvev_ring_workspace_bytes(const kvev_cache *cache, int32_t group, int32_t budget) {
  if (!valid_cache(cache) || group < 1 || group > kvev::kRingMaxGroup || budget < 1 ||
      budget > kvev::kRingMaxBudget)
    return 0;
  return ring_layout(cache, group, budget).total;
}

int kvev_ring_step(const kvev_cache *cache, float *hist, int32_t *ring, int32_t *rank,
                   const void *q, const void *k_new, const void *v_new, const int32_t *t_pos,
                   const int32_t *observe, int32_t group, float scale, int32_t budget,
                   int32_t recent_window, int32_t obs_window, int32_t pool_kernel,
                   int32_t *free_list, int32_t *free_count, int32_t *evicted_pos,
                   void *workspace, size_t ws_bytes, void *stream) {
  if (!valid_cache(cache) || !hist || !ring || !rank || !q || !k_new || !v_new || !t_pos ||
      !observe || !free_list || !free_count || !evicted_pos)
    return KVEV_EINVAL;
  if (group < 1 || budget < 1 || recent_window < 0 || recent_window >= budget ||
      obs_window < 1 || pool_kernel < 1 || pool_kernel % 2 == 0 ||
      budget > cache->max_blocks * KVEV_BLOCK_SIZE)
    return KVEV_EINVAL;
  if (group > kvev::kRingMaxGroup || budget > kvev::kRingMaxBudget ||
      (int64_t)group * (budget + 1) > 16384 || pool_kernel > 2 * budget + 1)
    return KVEV_EUNSUPPORTED;
  const RingLayout L = ring_layout(cache, group, budget);
  if (!workspace || ws_bytes < L.total) return KVEV_ENOSPACE;
  uint8_t *ws = static_cast<uint8_t *>(workspace);
  kvev::RingArgs a{};
  a.k_pool = static_cast<uint8_t *>(cache->k_pool);
  a.v_pool = static_cast<uint8_t *>(cache->v_pool);
  a.block_table = cache->block_table;
  a.seq_len = cache->seq_len;
  a.pos = cache->pos;
  a.hist = hist;
  a.ring = ring;
  a.rank = rank;
  a.q = static_cast<const uint8_t *>(q);
  a.k_new = static_cast<const uint8_t *>(k_new);
  a.v_new = static_cast<const uint8_t *>(v_new);
  a.t_pos = t_pos;
  a.observe = observe;
  a.free_list = free_list;
  a.free_count = free_count;
  a.evicted = evicted_pos;
  a.units = cache->batch * cache->kv_heads;
  a.Hkv = cache->kv_heads;
  a.G = group;
  a.W = obs_window;
  a.max_blocks = cache->max_blocks;
  a.max_slots = cache->max_blocks * KVEV_BLOCK_SIZE;
  a.num_blocks = cache->num_blocks;
  a.budget = budget;
  a.recent = recent_window;
  a.pool_kernel = pool_kernel;
  a.e = reinterpret_cast<uint32_t *>(ws + L.e);
  a.rsum = reinterpret_cast<uint32_t *>(ws + L.rsum);
  a.ml = reinterpret_cast<uint32_t *>(ws + L.ml);
  a.arrive = reinterpret_cast<uint32_t *>(ws + L.arrive);
  a.nbmax = L.nbmax;
  a.np = L.np;
  // enough workgroups to cover the CUs, at most one per block of the budget
  const int want = (256 + a.units - 1) / a.units;
  a.split = std::max(1, std::min({want, kvev::kRingMaxSplit, L.nbmax}));
  a.cb = (L.nbmax + a.split - 1) / a.split;
  a.c1 = scale * 1.4426950408889634f;
  return map_err(kvev::launch_ring_step(a, cache->dtype == KVEV_BF16, cache->head_dim,
                                        static_cast<hipStream_t>(stream)));
}


int kvev_vtok_sync(const kvev_cache *cache, uint8_t *live, int32_t *block_live,
                   const int32_t *new_len, const int32_t *pos0, int32_t *status, void *stream) {
  if (!valid_cache(cache) || !live || !block_live || !new_len || !pos0 || !status)
    return KVEV_EINVAL;
  kvev::VtokArgs a = vtok_args(cache, live, block_live);
  a.new_len = new_len;
  a.pos0 = pos0;
  a.status = status;
  return map_err(kvev::launch_vtok_sync(a, static_cast<hipStream_t>(stream)));
}

size_t kvev_vtok_map_workspace_bytes(const kvev_cache *cache) {
  if (!valid_cache(cache)) return 0;
  const size_t chunks = ((size_t)cache->max_blocks * KVEV_BLOCK_SIZE + 4095) / 4096;
  return vtok_base(cache) + a256((size_t)cache->batch * cache->kv_heads * chunks * 4);
}

int kvev_vtok_slot_mapping(const kvev_cache *cache, const uint8_t *live, int32_t *slots,
                           int32_t *positions, int32_t *count, void *workspace, size_t ws_bytes,
                           void *stream) {
  if (!valid_cache(cache) || !live || !slots || !positions || !count) return KVEV_EINVAL;
  if (!workspace || ws_bytes < kvev_vtok_map_workspace_bytes(cache)) return KVEV_ENOSPACE;
  kvev::VtokArgs a = vtok_args(cache, const_cast<uint8_t *>(live), nullptr);
  a.map_slots = slots;
  a.map_pos = positions;
  a.map_count = count;
  a.map_chunk = reinterpret_cast<int32_t *>(static_cast<uint8_t *>(workspace) + vtok_base(cache));
  a.map_chunks = (a.max_slots + 4095) / 4096;
  return map_err(kvev::launch_vtok_slot_mapping(a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
