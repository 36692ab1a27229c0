// Internal launcher interface between the C ABI (abi.hip) and the kernels.
// Everything here has already been validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

enum : int { kF32 = 0, kBF16 = 1 };

struct DecodeArgs {
  const void *q;
  const void *k_pool;
  const void *v_pool;
  const int32_t *block_table;
  const int32_t *context_lens;
  void *out;
  float *ws;  // workspace: partition layout (ws_layout) or stream layout (stream_layout)
  int32_t rows, n_heads, n_kv_heads, group, head_dim, block_size, log2_bs;
  int32_t max_blocks_per_row, partition_tokens, max_parts;
  int32_t stream;  // 1: balanced stream decomposition (bf16, head_dim 64/128); 2: the
                   // multi-query read's balanced decomposition (decode_multi_stream)
  int32_t cg_min;  // stream paths: minimum 32-position groups per slice
  int32_t stream_waves;  // stream paths: slices at most (persistent waves or workgroups)
  int32_t inplan;  // stream path: rows <= kWindowRows, each wave plans for itself
  int64_t num_blocks;
  int32_t dtype, out_dtype;
  float scale;
  // multi-query read: queries per row, 32-column tiles per (row, kv head),
  // queries per tile, query blocks (one workgroup each) per (row, kv head)
  int32_t query_len, q_tiles, q_per_tile, q_blocks;
  // stream path: score columns per (kv head, row), (query, head) pairs in
  // that order: group for the one-query read, query_len * group (<= 16)
  // for a multi-query read on the stream path
  int32_t cols;
  // decode step fused into the stream read: the step's new token of every
  // row (k_new, v_new [rows, n_kv_heads, head_dim], slot_new [rows]),
  // appended by the read itself.  Null: a plain read.
  const void *k_new, *v_new;
  const int64_t *slot_new;
};

// Multi-query read: a workgroup of multi_waves(tiles) waves, one 32-column
// score tile each, covers that many tiles of one (row, kv head) and shares
// every staged K/V group among them.
__host__ __device__ inline int32_t multi_waves(int32_t tiles) { return tiles > 4 ? 8 : (tiles > 2 ? 4 : 2); }
// LDS ring depth of the multi-query read, in 32-position groups: eight for
// a workgroup that has its compute unit to itself (eight waves), four where
// two workgroups share one.
__host__ __device__ constexpr int multi_ring(int waves) { return waves >= 8 ? 8 : 4; }
constexpr int kMultiMaxPartition = 4096;   // positions per multi-query partition, at most
constexpr int32_t kMaxPartitionBlocks = 4096;  // block ids of one partition of the partition kernels, at most
// Balanced multi-query read: each (kv head, row) enters the stream with this
// many extra groups of no work ahead of its own, which charge a slice for
// what every (kv head, row) it starts costs beyond its groups (the restart:
// block ids, queries, the ring's first groups; and the output or partial
// written at its end), so that slices balance time, not groups.  Measured
// on the 8B shape (us per call, 0 / 4 / 8 / 12 / 16 / 24 / 32 groups):
// 16 rows x 64 queries 109.6 / 103.0 / 98.9 / 90.3 / 90.0 / 92.4 / 96.1,
// 64 x 64 316.7 / 297.7 / 281.3 / 265.9 / 264.3 / 266.6 / 271.7.
constexpr int kMultiSegmentCost = 12;
// Waves per workgroup of the matrix-core partition read: eight (two per
// SIMD) when the grid is at most one workgroup per compute unit, so that a
// short read has two waves per SIMD to hide its load latency; else four.
__host__ __device__ inline int mfma_partition_waves(int32_t max_parts, int32_t n_kv_heads, int32_t rows) {
  return (long long)max_parts * n_kv_heads * rows <= 256 ? 8 : 4;
}

// Workspace of the split-context read, in floats: running max m and sum l
// per (row, query head, partition), then the fp32 partial output rows.
struct WsLayout {
  size_t m_off, l_off, acc_off, total_floats;
};
__host__ __device__ inline WsLayout ws_layout(int32_t rows, int32_t n_heads, int32_t max_parts,
                                              int32_t head_dim) {
  WsLayout w;
  const size_t slots = (size_t)rows * n_heads * max_parts;
  w.m_off = 0;
  w.l_off = slots;
  w.acc_off = (2 * slots + 3) & ~(size_t)3;  // 16-byte aligned
  w.total_floats = w.acc_off + slots * head_dim;
  return w;
}

// Stream decomposition of the bf16 read: the groups of 32 positions of all
// (kv head, row) pairs, in that order, are cut into equal contiguous slices,
// one per persistent wave (at most kStreamWaves of them; the multi-query
// read's balanced form cuts at most one slice per persistent workgroup).
// Workspace, in 4-byte words, for at most `waves` slices:
//   hdr[4]                 groups per kv head, waves used, two words unused
//   first_pos[2 * waves]   (kv head * rows + row, group) where each wave starts
//   gpre[rows + 1]         exclusive prefix of groups per row
//   partials[2 * waves][slot]  fp32 acc[cols][hd], m[cols], l[cols]
// The plan words (hdr, first_pos, gpre) are written by decode_plan; a batch
// of at most kWindowRows rows is planned inside every wave and leaves them
// unused.
//
// Partial slots belong to waves, not to (kv head, row) pairs.  Inside one
// wave's slice only the first and the last segment can be pieces of a pair
// cut by a slice boundary (every segment in between is a whole pair, which
// the wave writes to `out` itself).  A cut pair's first piece is the last
// segment of the slice it starts in, and each later piece is the first
// segment of the next slices.  So a wave owns two slots: 2w + 1 for a piece
// that starts a cut pair, 2w for a later piece; a pair whose first piece is
// in slice f keeps piece k at stream_piece_slot(f, k).  The workspace grows
// with the number of waves, not with the table width.
constexpr int kStreamWaves = 1024;  // one persistent wave per SIMD (4 per CU)
constexpr int kWindowRows = 256;  // rows a wave keeps (and, if that is all, plans) in LDS
constexpr int kPlanMaxRows = 8192;
constexpr int kGroupPositions = 32;
struct StreamLayout {
  size_t hdr, first_pos, gpre, partials, total;
  size_t slot_stride;
};
__host__ __device__ inline size_t align4(size_t x) { return (x + 3) & ~(size_t)3; }
__host__ __device__ inline StreamLayout stream_layout(int32_t rows, int32_t cols, int32_t head_dim,
                                                      int32_t waves = kStreamWaves) {
  StreamLayout L;
  L.hdr = 0;
  L.first_pos = 4;
  L.gpre = L.first_pos + 2 * (size_t)waves;
  L.partials = align4(L.gpre + (size_t)rows + 1);
  L.slot_stride = align4((size_t)cols * (head_dim + 2));
  L.total = L.partials + 2 * (size_t)waves * L.slot_stride;
  return L;
}
// Slot of piece k of a cut pair whose first piece lies in slice `first`.
__host__ __device__ inline size_t stream_piece_slot(long long first, int k) {
  return k == 0 ? (size_t)(2 * first + 1) : (size_t)(2 * (first + k));
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream);
hipError_t launch_multi(const DecodeArgs &a, hipStream_t stream);

hipError_t launch_scatter(const void *k, const void *v, const int64_t *slots, int64_t num_tokens,
                          void *k_pool, void *v_pool, int64_t num_blocks, int32_t block_size,
                          int32_t n_kv_heads, int32_t head_dim, int32_t dtype, hipStream_t stream);

}  // namespace pkv
