// Slot-mapping scatter (reshape_and_cache) for gfx950.
//
// Each new token's K and V rows, for every kv head, are copied bit for bit
// into the pool slot its slot id names: block slot / block_size, offset
// slot % block_size (nanoserve "Day 25" page, "What I learned", item 1: the
// scatter is exact; "Day 17" page, "Post angle": a pool of fixed-size blocks).
//
// One workgroup per token.  Reads of a token's [n_kv_heads, head_dim] K and V
// are contiguous runs.  K lands as whole head rows (16-byte chunks) in the
// (block, kv head) tiles of [num_blocks, n_kv_heads, block_size, head_dim];
// V is stored dimension-major inside a block, [num_blocks, n_kv_heads,
// head_dim, block_size], so each V element is its own store, block_size
// elements apart.
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kThreads = 256;

template <typename E>
__global__ __launch_bounds__(kThreads) void scatter_kv(const uint4 *__restrict__ k,
                                                       const E *__restrict__ v,
                                                       const int64_t *__restrict__ slots,
                                                       uint4 *__restrict__ k_pool,
                                                       E *__restrict__ v_pool, int64_t num_slots,
                                                       int32_t log2_bs, int32_t n_kv_heads,
                                                       int32_t head_dim) {
  const int64_t t = blockIdx.x;
  const int64_t s = slots[t];
  if (s < 0 || s >= num_slots) return;  // padding (or out of the pool: skipped)
  const int64_t blk = s >> log2_bs;
  const int64_t off = s & ((1 << log2_bs) - 1);
  // K: 16-byte chunks of whole head rows
  const int row_chunks = head_dim * (int)sizeof(E) / 16;
  const int k_chunks = n_kv_heads * row_chunks;
  for (int c = threadIdx.x; c < k_chunks; c += kThreads) {
    const int head = c / row_chunks;
    const int cc = c - head * row_chunks;
    const size_t dst = ((((size_t)blk * n_kv_heads + head) << log2_bs) + off) * row_chunks + cc;
    k_pool[dst] = k[(size_t)t * k_chunks + c];
  }
  // V: element (head, d) goes to [blk][head][d][off]
  const int v_elems = n_kv_heads * head_dim;
  for (int e = threadIdx.x; e < v_elems; e += kThreads) {
    const size_t dst = (((size_t)blk * n_kv_heads * head_dim + e) << log2_bs) + off;
    v_pool[dst] = v[(size_t)t * v_elems + e];
  }
}

}  // namespace

hipError_t launch_scatter(const void *k, const void *v, const int64_t *slots, int64_t num_tokens,
                          void *k_pool, void *v_pool, int64_t num_blocks, int32_t block_size,
                          int32_t n_kv_heads, int32_t head_dim, int32_t dtype, hipStream_t stream) {
  int log2_bs = 0;
  while ((1 << log2_bs) < block_size) ++log2_bs;
  if (dtype == kF32)
    hipLaunchKernelGGL(scatter_kv<uint32_t>, dim3((unsigned)num_tokens), dim3(kThreads), 0, stream,
                       static_cast<const uint4 *>(k), static_cast<const uint32_t *>(v), slots,
                       static_cast<uint4 *>(k_pool), static_cast<uint32_t *>(v_pool),
                       num_blocks * block_size, log2_bs, n_kv_heads, head_dim);
  else
    hipLaunchKernelGGL(scatter_kv<uint16_t>, dim3((unsigned)num_tokens), dim3(kThreads), 0, stream,
                       static_cast<const uint4 *>(k), static_cast<const uint16_t *>(v), slots,
                       static_cast<uint4 *>(k_pool), static_cast<uint16_t *>(v_pool),
                       num_blocks * block_size, log2_bs, n_kv_heads, head_dim);
  return hipGetLastError();
}

}  // namespace pkv
