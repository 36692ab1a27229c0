// C ABI of libpkv.so (declared and documented in include/pkv.h).
//
// Every entry point validates its arguments on the host and returns a status
// before touching the HIP runtime, so a refused call enqueues nothing.  Launch
// geometry comes from host shapes only (max_blocks_per_row, never the device
// lengths): nanoserve "Day 60" page, "Why it matters" -- reading lengths back
// would be a device sync on every call.
#include <limits.h>

#include <algorithm>
#include <mutex>

#include "pkv.h"
#include "pkv_internal.h"

namespace {

constexpr int32_t kDefaultPartition = 512;
constexpr int64_t kTargetWorkgroups = 512;
constexpr int32_t kStreamMinGroups = 4;  // 128 positions
constexpr int32_t kMaxGroup = 16;
using pkv::kMaxPartitionBlocks;  // LDS holds one partition's block ids (16 KB)

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
bool dtype_ok(int32_t d) { return d == PKV_F32 || d == PKV_BF16; }
bool head_dim_ok(int32_t h) { return h == 16 || h == 64 || h == 128; }
bool block_size_ok(int32_t b) { return b == 8 || b == 16 || b == 32; }
int64_t elem_bytes(int32_t d) { return d == PKV_F32 ? 4 : 2; }
int32_t log2i(int32_t x) {
  int32_t l = 0;
  while ((1 << l) < x) ++l;
  return l;
}

// Pool bytes fit in int64 and in the addressable range.
bool pool_fits(int64_t num_blocks, int32_t bs, int32_t n_kv, int32_t hd, int32_t dtype) {
  const int64_t per_block = (int64_t)bs * n_kv * hd * elem_bytes(dtype);
  return num_blocks >= 1 && num_blocks <= INT64_MAX / per_block;
}

// Default partition length where the caller gives none and no other rule
// applies (the stream path, which only keeps it for the record): long
// enough to amortise a workgroup (at most kDefaultPartition positions),
// short enough that the grid of (partition, kv head, row) workgroups reaches
// kTargetWorkgroups when rows are few.  From host shapes only.
int32_t default_partition(const pkv_attn_desc *d, int32_t cap) {
  const int64_t pairs = (int64_t)d->n_kv_heads * (d->rows > 0 ? d->rows : 1);
  const int64_t want_parts = (kTargetWorkgroups + pairs - 1) / pairs;
  int64_t part = (cap + want_parts - 1) / want_parts;
  part = (part + d->block_size - 1) / d->block_size * d->block_size;
  if (part > kDefaultPartition) part = kDefaultPartition;
  if (part < d->block_size) part = d->block_size;
  return (int32_t)part;
}

// Default partition of the MFMA partition kernel (bf16, head_dim 64/128: small
// batches over short tables, and batches too large for the stream plan): as
// few partitions as give one workgroup per compute unit, none shorter than
// kMfmaMinPartition positions unless the table is -- a split costs a merge
// launch, worth about six 32-position groups per wave -- and none longer
// than kMfmaMaxPartition, so that a long row is still cut.  Measured on the
// 8B-shaped layer (us, default before / after): 32 rows x 768 positions 22.5
// / 19.2, 16 x 768 15.6 / 13.5, 8 x 2048 19.9 / 18.3, 32 x 2048 43.8 / 39.2,
// 16 x 4096 43.6 / 40.0 (4096-position partitions: 44.2).
constexpr int64_t kMfmaTargetWorkgroups = 256;
constexpr int32_t kMfmaMinPartition = 768;
constexpr int32_t kMfmaMaxPartition = 2048;
int32_t default_partition_mfma(const pkv_attn_desc *d, int32_t cap) {
  const int64_t pairs = (int64_t)d->n_kv_heads * (d->rows > 0 ? d->rows : 1);
  const int64_t want_parts = (kMfmaTargetWorkgroups + pairs - 1) / pairs;
  int64_t part = (cap + want_parts - 1) / want_parts;
  part = std::min<int64_t>(std::max<int64_t>(part, kMfmaMinPartition), kMfmaMaxPartition);
  part = (part + d->block_size - 1) / d->block_size * d->block_size;
  return (int32_t)part;
}

// Default partition of the VALU partition kernel (fp32, and bf16 head_dim
// 16): about kValuPartitionBytes of K and V per partition, whatever the
// batch.  Its workgroups are latency-bound, so they want many in flight;
// the merge wants few partitions.  Measured (us, former default / this):
// fp32 8 rows x 2 kv heads x hd 64 over 1024 positions 21.5 / 16.6 (128
// positions), the same at 16 positions 10.3 / 6.5 (one partition), fp32 64
// x 8 x hd 128 over 2048 276 / 253 (64), bf16 hd 16 32 x 8 over 4096 16.7 /
// 15.5 (1024).
constexpr int64_t kValuPartitionBytes = 64 << 10;
int32_t default_partition_valu(const pkv_attn_desc *d, int32_t cap) {
  int64_t part = kValuPartitionBytes / (2 * (int64_t)d->head_dim * elem_bytes(d->dtype));
  part = std::max<int64_t>(part / d->block_size * d->block_size, d->block_size);
  return (int32_t)std::min<int64_t>(part, cap);
}

constexpr int64_t kSmallBatchPairs = 256;   // (kv head, row) pairs
constexpr int64_t kSmallBatchTable = 4096;  // positions a row's table can hold
constexpr int64_t kShortTable = 1024;       // positions: the partition kernel at any batch
struct Plan {
  int32_t group, partition, max_parts, log2_bs;
  int32_t stream, cg_min;
  size_t ws_bytes;
};

int plan_decode(const pkv_attn_desc *d, Plan *pl) {
  if (!d) return PKV_ERR_NULL;
  if (!dtype_ok(d->dtype) || !dtype_ok(d->out_dtype)) return PKV_ERR_DTYPE;
  if (d->rows < 0 || d->rows > 65535) return PKV_ERR_SHAPE;
  if (d->n_heads < 1 || d->n_kv_heads < 1 || d->n_kv_heads > 65535) return PKV_ERR_HEADS;
  if (d->n_heads % d->n_kv_heads != 0 || d->n_heads / d->n_kv_heads > kMaxGroup) return PKV_ERR_HEADS;
  if (!head_dim_ok(d->head_dim)) return PKV_ERR_HEAD_DIM;
  if (!block_size_ok(d->block_size)) return PKV_ERR_BLOCK_SIZE;
  if (d->max_blocks_per_row < 1 || (int64_t)d->max_blocks_per_row * d->block_size > INT_MAX)
    return PKV_ERR_SHAPE;
  if (d->num_blocks > INT_MAX ||
      !pool_fits(d->num_blocks, d->block_size, d->n_kv_heads, d->head_dim, d->dtype))
    return PKV_ERR_SHAPE;
  const int32_t cap = d->max_blocks_per_row * d->block_size;
  // bf16 with head_dim 64/128 runs the balanced stream decomposition when the
  // plan kernel can hold the rows and the group count fits in 31 bits;
  // everything else runs one workgroup per (partition, kv head, row).  So
  // does a table of at most kShortTable positions, and a small batch over a
  // table of at most kSmallBatchTable: there the partition kernel, one
  // launch with at most a few workgroups per row, beats the stream's fixed
  // start-up and merge, while long tables keep the stream's balance.
  // Measured on the 8B-shaped layer (us, stream / partition): 128 rows x 768
  // positions 72.4 / 62.7, 96 x 1024 63.0 / 55.0, 32 x 4096 65.2 / 64.8;
  // 64 x 2048 86.6 / 90.9, 48 x 4096 83.2 / 100.7, 64 x 4096 106 / 125,
  // 32 x 8192 154 / 179, 4 x 32768 100 / 128.
  const int64_t cap_groups = (cap + pkv::kGroupPositions - 1) / pkv::kGroupPositions;
  const bool small_batch = cap <= kShortTable ||
                           ((int64_t)d->rows * d->n_kv_heads <= kSmallBatchPairs && cap <= kSmallBatchTable);
  const bool mfma = d->dtype == PKV_BF16 && (d->head_dim == 64 || d->head_dim == 128);
  pl->stream = mfma && d->rows <= pkv::kPlanMaxRows && !small_batch &&
               cap_groups * d->n_kv_heads * d->rows < (int64_t)INT_MAX;
  int32_t part = d->partition_tokens;
  if (part == 0)
    part = pl->stream ? default_partition(d, cap) : (mfma ? default_partition_mfma(d, cap) : default_partition_valu(d, cap));
  if (part < 0 || part % d->block_size != 0) return PKV_ERR_PARTITION;
  if (part > cap) part = cap;  // one partition covers every row: no split
  if (part / d->block_size > kMaxPartitionBlocks) return PKV_ERR_PARTITION;
  pl->group = d->n_heads / d->n_kv_heads;
  pl->partition = part;
  pl->log2_bs = log2i(d->block_size);
  pl->ws_bytes = 0;
  if (pl->stream) {
    // slices of at least cg_min groups: the caller's partition length, else
    // kStreamMinGroups, short enough that a small batch still fills every wave
    pl->cg_min = d->partition_tokens ? (part + pkv::kGroupPositions - 1) / pkv::kGroupPositions
                                     : kStreamMinGroups;
    pl->max_parts = (int32_t)((cap_groups + pl->cg_min - 1) / pl->cg_min + 1);
    if (d->rows > 0) pl->ws_bytes = pkv::stream_layout(d->rows, pl->group, d->head_dim).total * sizeof(int32_t);
    return PKV_OK;
  }
  pl->cg_min = 0;
  pl->max_parts = (cap + part - 1) / part;
  // one workgroup per (partition, kv head, row) in a 1-D grid
  if ((int64_t)pl->max_parts * d->n_kv_heads * d->rows > INT_MAX) return PKV_ERR_SHAPE;
  if (pl->max_parts > 1 && d->rows > 0)
    pl->ws_bytes =
        pkv::ws_layout(d->rows, d->n_heads, pl->max_parts, d->head_dim).total_floats * sizeof(float);
  return PKV_OK;
}

// Multi-query read: bf16, head_dim 64/128.  Partitions are whole 32-position
// groups, at most kMultiMaxPartition positions: the caller's partition_tokens
// rounded up to a group (and capped), else the power of two (256 .. 2048)
// nearest below the one that makes the largest possible grid about one
// workgroup per slot of the GPU (kComputeUnits compute units times the
// workgroups of this shape one unit holds), and 1024 at most for two-wave
// workgroups.  Larger partitions mean fewer start-ups and partial results.
// Measured on the 8B shape (lengths uniform in [512, 4096]), us per call
// for partitions of 256 / 512 / 1024 / 2048 positions (* = this rule):
//   16 rows x 64 queries  207.5 / 142.3 / 120.4 / 105.8*
//   64 rows x 64 queries  736.9 / 517.0 / 391.3 / 355.6*
//    4 rows x 64 queries   60.5 /  43.6* /  57.3 /  90.2
//   64 rows x 32 queries  442.0 / 321.4 / 271.2 / 253.9*
//   16 rows x 16 queries   73.8 /  58.6 /  52.1* /  81.4
//   64 rows x 16 queries  244.0 / 199.6 / 171.6* / 180.3
//   64 rows x  8 queries  205.2 / 176.2 / 158.9* / 171.1
constexpr int64_t kComputeUnits = 256;
constexpr int64_t kStreamMultiGroups = 32;
// Balanced multi-query read (one query block per (row, kv head), at most
// kWindowRows rows): slices of at least this many 32-position groups by
// default (the caller's partition_tokens, rounded up to whole groups,
// replaces it), one per persistent workgroup.
constexpr int64_t kMultiSliceMinGroups = 16;
// ... and only for at least this many (row, kv head) pairs: below, the
// partition kernel's workgroups start at once and the balanced read's fixed
// costs do not pay (8B shape, 64 queries: 4 rows 44.8 vs 49.5 us, 8 rows
// 62.5 vs 63.6; 16 rows 97.1 vs 90.3, 64 rows 321.4 vs 265.9).
constexpr int64_t kMultiBalancedMinPairs = 128;
struct MultiPlan {
  int32_t q_tiles, q_per_tile, q_blocks;
  int32_t stream;  // 1: query_len * group <= 16 columns on the stream path
  int32_t stream_waves;  // balanced multi-query read: persistent workgroups
};
int plan_multi(const pkv_attn_desc *d, int32_t query_len, Plan *pl, MultiPlan *mp) {
  if (!d) return PKV_ERR_NULL;
  if (d->partition_tokens < 0) return PKV_ERR_PARTITION;
  // The shapes are checked as for the one-query read, without its partition
  // rule: this read rounds the caller's length to whole groups itself.
  pkv_attn_desc dd = *d;
  dd.partition_tokens = 0;
  const int st = plan_decode(&dd, pl);
  if (st != PKV_OK) return st;
  if (d->dtype != PKV_BF16) return PKV_ERR_DTYPE;
  if (d->head_dim != 64 && d->head_dim != 128) return PKV_ERR_HEAD_DIM;
  if (query_len < 1 || query_len > 65535) return PKV_ERR_SHAPE;
  // A chunk whose (query, head) pairs fit the 16 columns of the one-query
  // read's score tile runs on that read's stream decomposition -- the same
  // bytes, in columns the one-query read leaves empty -- when the table can
  // hold at least kStreamMultiGroups groups per persistent wave.  Below
  // that the stream is latency-bound and the workgroup kernel is faster
  // (8B-shaped layer, 4 queries: 16 rows 54 vs 60 us, 64 rows 179 vs 129 us).
  const int64_t cap_groups = ((int64_t)d->max_blocks_per_row * d->block_size + pkv::kGroupPositions - 1) /
                             pkv::kGroupPositions;
  mp->stream = pl->stream && (int64_t)query_len * pl->group <= 16 &&
               (int64_t)d->rows * d->n_kv_heads * cap_groups >= kStreamMultiGroups * pkv::kStreamWaves;
  if (mp->stream) {
    mp->q_tiles = mp->q_per_tile = mp->q_blocks = 0;
    if (d->partition_tokens)  // the minimum slice, in whole groups, as on the one-query read
      pl->cg_min = (int32_t)std::min<int64_t>((d->partition_tokens + pkv::kGroupPositions - 1) / pkv::kGroupPositions,
                                              cap_groups);
    pl->ws_bytes =
        d->rows > 0 ? pkv::stream_layout(d->rows, query_len * pl->group, d->head_dim).total * sizeof(int32_t) : 0;
    return PKV_OK;
  }
  const int32_t cap = d->max_blocks_per_row * d->block_size;
  mp->q_per_tile = 32 / pl->group;  // group <= 16
  mp->q_tiles = (query_len + mp->q_per_tile - 1) / mp->q_per_tile;
  const int32_t waves = pkv::multi_waves(mp->q_tiles);
  mp->q_blocks = (mp->q_tiles + waves - 1) / waves;
  const int64_t g32 = pkv::kGroupPositions;
  const int64_t per_cu = std::max<int64_t>(1, (d->head_dim == 128 ? 4 : 8) / waves);  // registers, LDS
  mp->stream_waves = 0;
  if (mp->q_blocks == 1 && d->rows <= pkv::kWindowRows &&
      (int64_t)d->rows * d->n_kv_heads >= kMultiBalancedMinPairs) {
    // balanced: one slice of the (kv head, row) group stream per persistent
    // workgroup, as many workgroups as the GPU holds at once
    mp->stream_waves = (int32_t)(kComputeUnits * per_cu);
    pl->stream = 2;
    pl->cg_min = (int32_t)(d->partition_tokens ? (d->partition_tokens + g32 - 1) / g32 : kMultiSliceMinGroups);
    pl->partition = 0;
    pl->max_parts = 0;
    if ((int64_t)d->rows * query_len * d->n_heads > INT_MAX) return PKV_ERR_SHAPE;
    pl->ws_bytes = d->rows > 0 ? pkv::stream_layout(d->rows, query_len * pl->group, d->head_dim, mp->stream_waves).total *
                                     sizeof(int32_t)
                               : 0;
    return PKV_OK;
  }
  int64_t part;
  if (d->partition_tokens) {
    part = (d->partition_tokens + g32 - 1) / g32 * g32;
  } else {
    const int64_t blocks = (int64_t)mp->q_blocks * d->n_kv_heads * (d->rows > 0 ? d->rows : 1);
    const int64_t want = (int64_t)cap * blocks / (kComputeUnits * per_cu);
    // two-wave workgroups (at most two tiles) stop at 1024 positions
    const int64_t top = waves <= 2 ? 1024 : 2048;
    part = 256;
    while (part < top && part * 2 <= want) part *= 2;
  }
  if (part > pkv::kMultiMaxPartition) part = pkv::kMultiMaxPartition;
  if (part < g32) part = g32;
  const int64_t cap32 = (cap + g32 - 1) / g32 * g32;
  if (part > cap32) part = cap32;
  pl->partition = (int32_t)part;
  pl->max_parts = (int32_t)((cap + part - 1) / part);
  const int64_t units = (int64_t)pl->max_parts * mp->q_blocks * d->n_kv_heads * d->rows;
  const int64_t vrows = (int64_t)d->rows * query_len;
  if (units > INT_MAX || vrows * d->n_heads > INT_MAX) return PKV_ERR_SHAPE;
  pl->stream = 0;
  pl->ws_bytes = 0;
  if (pl->max_parts > 1 && d->rows > 0)
    pl->ws_bytes =
        pkv::ws_layout((int32_t)vrows, d->n_heads, pl->max_parts, d->head_dim).total_floats * sizeof(float);
  return PKV_OK;
}

int check_scatter(const void *k, const void *v, const int64_t *slot_mapping, int64_t num_tokens,
                  const void *k_pool, const void *v_pool, int64_t num_blocks, int32_t block_size,
                  int32_t n_kv_heads, int32_t head_dim, int32_t dtype);

// Every host-side check of a read, before anything is enqueued.
int check_attention_args(const pkv_attn_desc *d, const void *q, const void *k_pool, const void *v_pool,
                         const int32_t *block_table, const int32_t *context_lens, const void *out, Plan *pl) {
  const int st = plan_decode(d, pl);
  if (st != PKV_OK) return st;
  if (!q || !k_pool || !v_pool || !block_table || !context_lens || !out) return PKV_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(out, 16) ||
      !aligned(block_table, 4) || !aligned(context_lens, 4))
    return PKV_ERR_ALIGN;
  return PKV_OK;
}

int check_attention(const pkv_attn_desc *d, const void *q, const void *k_pool, const void *v_pool,
                    const int32_t *block_table, const int32_t *context_lens, const void *out,
                    const void *workspace, size_t workspace_bytes, Plan *pl) {
  const int st = check_attention_args(d, q, k_pool, v_pool, block_table, context_lens, out, pl);
  if (st != PKV_OK) return st;
  if (pl->ws_bytes > 0) {
    if (!workspace || workspace_bytes < pl->ws_bytes) return PKV_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return PKV_ERR_ALIGN;
  }
  return PKV_OK;
}

int launch_attention(const pkv_attn_desc *d, const Plan &pl, const void *q, const void *k_pool,
                     const void *v_pool, const int32_t *block_table, const int32_t *context_lens,
                     float scale, void *out, void *workspace, hipStream_t stream,
                     const void *k_new = nullptr, const void *v_new = nullptr,
                     const int64_t *slot_new = nullptr) {
  if (d->rows == 0) return PKV_OK;
  pkv::DecodeArgs a = {};
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_table = block_table;
  a.context_lens = context_lens;
  a.out = out;
  a.ws = pl.ws_bytes ? static_cast<float *>(workspace) : nullptr;
  a.rows = d->rows;
  a.n_heads = d->n_heads;
  a.n_kv_heads = d->n_kv_heads;
  a.group = pl.group;
  a.head_dim = d->head_dim;
  a.block_size = d->block_size;
  a.log2_bs = pl.log2_bs;
  a.max_blocks_per_row = d->max_blocks_per_row;
  a.partition_tokens = pl.partition;
  a.max_parts = pl.max_parts;
  a.stream = pl.stream;
  a.cg_min = pl.cg_min;
  a.stream_waves = pkv::kStreamWaves;
  a.inplan = pl.stream && d->rows <= pkv::kWindowRows;
  a.num_blocks = d->num_blocks;
  a.dtype = d->dtype;
  a.out_dtype = d->out_dtype;
  a.scale = scale;
  a.query_len = 1;
  a.cols = pl.group;
  a.k_new = k_new;
  a.v_new = v_new;
  a.slot_new = slot_new;
  return pkv::launch_decode(a, stream) == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int pkv_version(void) { return 300; }

const char *pkv_strerror(int status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_ERR_NULL: return "a required pointer is NULL";
    case PKV_ERR_ALIGN: return "a buffer is not aligned (16 bytes for K/V/q/out/workspace)";
    case PKV_ERR_DTYPE: return "unsupported dtype (0 = f32, 1 = bf16)";
    case PKV_ERR_HEADS: return "n_heads must be a multiple of n_kv_heads with group <= 16";
    case PKV_ERR_HEAD_DIM: return "head_dim must be 16, 64 or 128";
    case PKV_ERR_BLOCK_SIZE: return "block_size must be 8, 16 or 32";
    case PKV_ERR_SHAPE: return "a size is out of range or overflows";
    case PKV_ERR_WORKSPACE: return "workspace missing or smaller than pkv_paged_attention_workspace_size";
    case PKV_ERR_PARTITION: return "partition_tokens must be a positive multiple of block_size";
    case PKV_ERR_LAUNCH: return "the HIP runtime refused a kernel launch";
    case PKV_ERR_MODE: return "read counters of different reads (mode or block differ)";
    case PKV_ERR_EXHAUSTED: return "the pool has fewer free blocks than asked for";
    case PKV_ERR_SCRATCH: return "the read needs more scratch than the library's static buffer holds";
    default: return "unknown status";
  }
}

int pkv_reshape_and_cache(const void *k, const void *v, const int64_t *slot_mapping,
                          int64_t num_tokens, void *k_pool, void *v_pool, int64_t num_blocks,
                          int32_t block_size, int32_t n_kv_heads, int32_t head_dim, int32_t dtype,
                          void *stream) {
  const int st = check_scatter(k, v, slot_mapping, num_tokens, k_pool, v_pool, num_blocks, block_size,
                               n_kv_heads, head_dim, dtype);
  if (st != PKV_OK) return st;
  if (num_tokens == 0) return PKV_OK;
  const hipError_t e = pkv::launch_scatter(k, v, slot_mapping, num_tokens, k_pool, v_pool,
                                           num_blocks, block_size, n_kv_heads, head_dim, dtype,
                                           static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}

}  // extern "C"

namespace {

int check_scatter(const void *k, const void *v, const int64_t *slot_mapping, int64_t num_tokens,
                  const void *k_pool, const void *v_pool, int64_t num_blocks, int32_t block_size,
                  int32_t n_kv_heads, int32_t head_dim, int32_t dtype) {
  if (!k || !v || !slot_mapping || !k_pool || !v_pool) return PKV_ERR_NULL;
  if (!dtype_ok(dtype)) return PKV_ERR_DTYPE;
  if (!head_dim_ok(head_dim)) return PKV_ERR_HEAD_DIM;
  if (!block_size_ok(block_size)) return PKV_ERR_BLOCK_SIZE;
  if (num_tokens < 0 || num_tokens > INT_MAX || n_kv_heads < 1 || n_kv_heads > 4096)
    return PKV_ERR_SHAPE;
  if (!pool_fits(num_blocks, block_size, n_kv_heads, head_dim, dtype)) return PKV_ERR_SHAPE;
  if (!aligned(k, 16) || !aligned(v, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) ||
      !aligned(slot_mapping, 8))
    return PKV_ERR_ALIGN;
  return PKV_OK;
}

}  // namespace

extern "C" {

size_t pkv_paged_attention_workspace_size(const pkv_attn_desc *d) {
  Plan pl;
  if (plan_decode(d, &pl) != PKV_OK) return 0;
  return pl.ws_bytes;
}

int pkv_paged_attention(const pkv_attn_desc *d, const void *q, const void *k_pool,
                        const void *v_pool, const int32_t *block_table,
                        const int32_t *context_lens, float scale, void *out, void *workspace,
                        size_t workspace_bytes, void *stream) {
  Plan pl;
  const int st = check_attention(d, q, k_pool, v_pool, block_table, context_lens, out, workspace,
                                 workspace_bytes, &pl);
  if (st != PKV_OK) return st;
  return launch_attention(d, pl, q, k_pool, v_pool, block_table, context_lens, scale, out, workspace,
                          static_cast<hipStream_t>(stream));
}

}  // extern "C"

// ---------------------------------------------------------------------------
// The read for callers that cannot allocate (HIP graph capture, tight serving
// loops): its scratch -- the partial slots and plan words the kernels would
// otherwise keep in the caller's workspace -- is this file-scope device
// array.  Every GPU the library runs on holds its own copy from the module's
// load until the process ends.  In host code `scratch` names a host-side
// stand-in, never the device copy: host code only ever uses the address
// hipGetSymbolAddress returns for the current device, kept per device below.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[PKV_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];  // device address of `scratch` on each device, once looked up

// Device address of `scratch` on the current device, looked up on the first
// call made with that device current.
int scratch_of_current_device(void **ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PKV_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return PKV_ERR_LAUNCH;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return PKV_OK;
}

}  // namespace

extern "C" {

int pkv_paged_attention_noalloc(const pkv_attn_desc *d, const void *q, const void *k_pool, const void *v_pool,
                                const int32_t *block_table, const int32_t *context_lens, float scale, void *out,
                                void *stream) {
  Plan pl;
  int st = check_attention_args(d, q, k_pool, v_pool, block_table, context_lens, out, &pl);
  if (st != PKV_OK) return st;
  if (pl.ws_bytes > (size_t)PKV_NOALLOC_SCRATCH_BYTES) return PKV_ERR_SCRATCH;
  if (d->rows == 0) return PKV_OK;
  void *ws = nullptr;
  if (pl.ws_bytes > 0) {
    st = scratch_of_current_device(&ws);
    if (st != PKV_OK) return st;
  }
  // The kernels need no zeroed scratch: every partial slot and plan word a
  // call reads is written earlier in the same call.
  return launch_attention(d, pl, q, k_pool, v_pool, block_table, context_lens, scale, out, ws,
                          static_cast<hipStream_t>(stream));
}

size_t pkv_paged_attention_multi_workspace_size(const pkv_attn_desc *d, int32_t query_len) {
  Plan pl;
  MultiPlan mp;
  if (plan_multi(d, query_len, &pl, &mp) != PKV_OK) return 0;
  return pl.ws_bytes;
}

int pkv_paged_attention_multi(const pkv_attn_desc *d, int32_t query_len, const void *q, const void *k_pool,
                              const void *v_pool, const int32_t *block_table, const int32_t *context_lens,
                              float scale, void *out, void *workspace, size_t workspace_bytes, void *stream) {
  Plan pl;
  MultiPlan mp;
  const int st = plan_multi(d, query_len, &pl, &mp);
  if (st != PKV_OK) return st;
  if (!q || !k_pool || !v_pool || !block_table || !context_lens || !out) return PKV_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(out, 16) ||
      !aligned(block_table, 4) || !aligned(context_lens, 4))
    return PKV_ERR_ALIGN;
  if (pl.ws_bytes > 0) {
    if (!workspace || workspace_bytes < pl.ws_bytes) return PKV_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return PKV_ERR_ALIGN;
  }
  if (d->rows == 0) return PKV_OK;
  if (mp.stream) {  // the one-query read's kernels, query_len * group columns
    pkv::DecodeArgs a = {};
    a.q = q;
    a.k_pool = k_pool;
    a.v_pool = v_pool;
    a.block_table = block_table;
    a.context_lens = context_lens;
    a.out = out;
    a.ws = pl.ws_bytes ? static_cast<float *>(workspace) : nullptr;
    a.rows = d->rows;
    a.n_heads = d->n_heads;
    a.n_kv_heads = d->n_kv_heads;
    a.group = pl.group;
    a.head_dim = d->head_dim;
    a.block_size = d->block_size;
    a.log2_bs = pl.log2_bs;
    a.max_blocks_per_row = d->max_blocks_per_row;
    a.partition_tokens = pl.partition;
    a.max_parts = pl.max_parts;
    a.stream = 1;
    a.cg_min = pl.cg_min;
    a.stream_waves = pkv::kStreamWaves;
    a.inplan = d->rows <= pkv::kWindowRows;
    a.num_blocks = d->num_blocks;
    a.dtype = d->dtype;
    a.out_dtype = d->out_dtype;
    a.scale = scale;
    a.query_len = query_len;
    a.cols = query_len * pl.group;
    return pkv::launch_decode(a, static_cast<hipStream_t>(stream)) == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
  }
  pkv::DecodeArgs a = {};
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_table = block_table;
  a.context_lens = context_lens;
  a.out = out;
  a.ws = pl.ws_bytes ? static_cast<float *>(workspace) : nullptr;
  a.rows = d->rows;
  a.n_heads = d->n_heads;
  a.n_kv_heads = d->n_kv_heads;
  a.group = pl.group;
  a.head_dim = d->head_dim;
  a.block_size = d->block_size;
  a.log2_bs = pl.log2_bs;
  a.max_blocks_per_row = d->max_blocks_per_row;
  a.partition_tokens = pl.partition;
  a.max_parts = pl.max_parts;
  a.num_blocks = d->num_blocks;
  a.dtype = d->dtype;
  a.out_dtype = d->out_dtype;
  a.scale = scale;
  a.query_len = query_len;
  a.q_tiles = mp.q_tiles;
  a.q_per_tile = mp.q_per_tile;
  a.q_blocks = mp.q_blocks;
  a.stream = pl.stream;  // 2: the balanced multi-query read
  a.cg_min = pl.cg_min;
  a.stream_waves = mp.stream_waves;
  a.cols = query_len * pl.group;
  return pkv::launch_multi(a, static_cast<hipStream_t>(stream)) == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}

int pkv_decode_step(const pkv_attn_desc *d, const void *k_new, const void *v_new,
                    const int64_t *slot_mapping, const void *q, void *k_pool, void *v_pool,
                    const int32_t *block_table, const int32_t *context_lens, float scale, void *out,
                    void *workspace, size_t workspace_bytes, void *stream) {
  Plan pl;
  int st = check_attention(d, q, k_pool, v_pool, block_table, context_lens, out, workspace,
                           workspace_bytes, &pl);
  if (st != PKV_OK) return st;
  st = check_scatter(k_new, v_new, slot_mapping, d->rows, k_pool, v_pool, d->num_blocks, d->block_size,
                     d->n_kv_heads, d->head_dim, d->dtype);
  if (st != PKV_OK) return st;
  if (d->rows == 0) return PKV_OK;
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  // Every read kernel appends the new tokens itself: one launch less than a
  // scatter followed by a read.
  return launch_attention(d, pl, q, k_pool, v_pool, block_table, context_lens, scale, out, workspace, hs,
                          k_new, v_new, slot_mapping);
}

int pkv_read_stats_init(pkv_read_stats *s, int32_t mode, int32_t block) {
  if (!s) return PKV_ERR_NULL;
  if ((mode != PKV_READ_GATHERED && mode != PKV_READ_STREAMED) || block < 1) return PKV_ERR_SHAPE;
  s->mode = mode;
  s->block = block;
  s->calls = s->rows = s->score_cells = s->held_cells = 0;
  return PKV_OK;
}

int pkv_read_stats_record(pkv_read_stats *s, int32_t rows, int32_t heads, int32_t query_len, int32_t width) {
  if (!s) return PKV_ERR_NULL;
  if (rows < 0 || heads < 0 || query_len < 0 || width < 0) return PKV_ERR_SHAPE;
  // rows * heads * query_len <= 2^93 in theory: bound each product in 63 bits
  const int64_t lanes = (int64_t)rows * heads;
  if (query_len && lanes > INT64_MAX / query_len) return PKV_ERR_SHAPE;
  const int64_t q = lanes * query_len;
  if (width && q > INT64_MAX / width) return PKV_ERR_SHAPE;
  const int64_t cells = q * width;
  const int64_t held = s->mode == PKV_READ_STREAMED ? q * (width < s->block ? width : s->block) : cells;
  if (s->score_cells > INT64_MAX - cells || s->held_cells > INT64_MAX - held) return PKV_ERR_SHAPE;
  s->calls += 1;
  s->rows += rows;
  s->score_cells += cells;
  s->held_cells += held;
  return PKV_OK;
}

int32_t pkv_read_tile(const pkv_attn_desc *d) {
  Plan pl;
  if (plan_decode(d, &pl) != PKV_OK) return 0;
  if (pl.stream) return pkv::kGroupPositions;  // one wave, one group
  if (d->dtype == PKV_BF16 && (d->head_dim == 64 || d->head_dim == 128))  // decode_partition_mfma: a group per wave
    return pkv::mfma_partition_waves(pl.max_parts, d->n_kv_heads, d->rows) * pkv::kGroupPositions;
  // decode_partition: four waves x four 16-byte loads per lane, each load
  // covering 64 / (head_dim / (16 / elem)) positions
  return (int32_t)(1024 * (16 / elem_bytes(d->dtype)) / d->head_dim);
}

int pkv_read_stats_record_read(pkv_read_stats *s, const pkv_attn_desc *d) {
  if (!s || !d) return PKV_ERR_NULL;
  const int32_t tile = pkv_read_tile(d);
  if (tile == 0 || d->rows < 0) return PKV_ERR_SHAPE;
  if (s->mode == PKV_READ_STREAMED && s->block != tile) return PKV_ERR_MODE;
  return pkv_read_stats_record(s, d->rows, d->n_heads, 1, d->max_blocks_per_row * d->block_size);
}

int pkv_read_stats_since(const pkv_read_stats *now, const pkv_read_stats *earlier, pkv_read_stats *window) {
  if (!now || !earlier || !window) return PKV_ERR_NULL;
  if (now->mode != earlier->mode || now->block != earlier->block) return PKV_ERR_MODE;
  if (now->calls < earlier->calls || now->rows < earlier->rows || now->score_cells < earlier->score_cells ||
      now->held_cells < earlier->held_cells)
    return PKV_ERR_SHAPE;  // not an earlier reading of the same counters
  window->mode = now->mode;
  window->block = now->block;
  window->calls = now->calls - earlier->calls;
  window->rows = now->rows - earlier->rows;
  window->score_cells = now->score_cells - earlier->score_cells;
  window->held_cells = now->held_cells - earlier->held_cells;
  return PKV_OK;
}

double pkv_read_stats_saving(const pkv_read_stats *s) {
  if (!s || s->held_cells <= 0) return 1.0;
  return (double)s->score_cells / (double)s->held_cells;
}

}  // extern "C"
