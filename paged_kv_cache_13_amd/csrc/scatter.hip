// Slot-mapping scatter (reshape_and_cache) for gfx950.
//
// Each new token's K and V rows, for every kv head, are copied bit for bit
// into the pool slot its slot id names: block slot / block_size, offset
// slot % block_size (nanoserve "Day 25" page, "What I learned", item 1: the
// scatter is exact; "Day 17" page, "Post angle": a pool of fixed-size blocks).
//
// One workgroup per token; each thread moves 16-byte chunks.  Reads of a
// token's [n_kv_heads, head_dim] K (then V) are one contiguous run; writes
// land as whole head rows (head_dim * elem bytes each) in the (block, kv head)
// tiles of the pool layout [num_blocks, n_kv_heads, block_size, head_dim].
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void scatter_kv(const uint4 *__restrict__ k,
                                                       const uint4 *__restrict__ v,
                                                       const int64_t *__restrict__ slots,
                                                       uint4 *__restrict__ k_pool,
                                                       uint4 *__restrict__ v_pool, int64_t num_slots,
                                                       int32_t log2_bs, int32_t n_kv_heads,
                                                       int32_t row_chunks) {
  const int64_t t = blockIdx.x;
  const int64_t s = slots[t];
  if (s < 0 || s >= num_slots) return;  // padding (or out of the pool: skipped)
  const int64_t blk = s >> log2_bs;
  const int64_t off = s & ((1 << log2_bs) - 1);
  const int per_token = n_kv_heads * row_chunks;  // 16-byte chunks of one tensor
  for (int i = threadIdx.x; i < 2 * per_token; i += kThreads) {
    const bool is_v = i >= per_token;
    const int c = is_v ? i - per_token : i;
    const int head = c / row_chunks;
    const int cc = c - head * row_chunks;
    const size_t dst = ((((size_t)blk * n_kv_heads + head) << log2_bs) + off) * row_chunks + cc;
    const size_t src = (size_t)t * per_token + c;
    if (is_v)
      v_pool[dst] = v[src];
    else
      k_pool[dst] = k[src];
  }
}

}  // namespace

hipError_t launch_scatter(const void *k, const void *v, const int64_t *slots, int64_t num_tokens,
                          void *k_pool, void *v_pool, int64_t num_blocks, int32_t block_size,
                          int32_t n_kv_heads, int32_t head_dim, int32_t dtype, hipStream_t stream) {
  const int es = dtype == kF32 ? 4 : 2;
  const int row_chunks = head_dim * es / 16;
  int log2_bs = 0;
  while ((1 << log2_bs) < block_size) ++log2_bs;
  hipLaunchKernelGGL(scatter_kv, dim3((unsigned)num_tokens), dim3(kThreads), 0, stream,
                     static_cast<const uint4 *>(k), static_cast<const uint4 *>(v), slots,
                     static_cast<uint4 *>(k_pool), static_cast<uint4 *>(v_pool),
                     num_blocks * block_size, log2_bs, n_kv_heads, row_chunks);
  return hipGetLastError();
}

}  // namespace pkv
