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
  float *ws;  // [3 regions] m, l, acc; null when max_parts == 1
  int32_t rows, n_heads, n_kv_heads, group, head_dim, block_size, log2_bs;
  int32_t max_blocks_per_row, partition_tokens, max_parts;
  int64_t num_blocks;
  int32_t dtype, out_dtype;
  float scale;
};

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

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream);

hipError_t launch_scatter(const void *k, const void *v, const int64_t *slots, int64_t num_tokens,
                          void *k_pool, void *v_pool, int64_t num_blocks, int32_t block_size,
                          int32_t n_kv_heads, int32_t head_dim, int32_t dtype, hipStream_t stream);

}  // namespace pkv
