// Slot-mapping scatter (reshape_and_cache) for gfx950.
//
// Each new token's K and V rows, for every kv head, are copied bit for bit
// into the pool slot its slot id names: block slot / block_size, offset
// slot % block_size (nanoserve "Day 25" page, "What I learned", item 1: the
// scatter is exact; "Day 17" page, "Post angle": a pool of fixed-size blocks).
//
// Few tokens (a decode step): one workgroup per token.  Reads of a token's [n_kv_heads, head_dim] K and V
// are contiguous runs.  K lands as whole head rows (16-byte chunks) in the
// (block, kv head) tiles of [num_blocks, n_kv_heads, block_size, head_dim];
// V is stored dimension-major inside a block, [num_blocks, n_kv_heads,
// head_dim, block_size], so each V element is its own store, block_size
// elements apart.
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kThreads = 256;
constexpr int64_t kTiledMinTokens = 1024;  // below: one workgroup per token

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

// Many tokens (a prompt): one workgroup per tile of kTileTokens consecutive
// tokens.  K is copied as above.  V goes through LDS: the tile's rows are
// read whole, then written out transposed, lane i carrying token i of the
// tile for one (kv head, dimension) -- tokens that fill consecutive offsets
// of one block (the prompt case) land as one contiguous run per element.
constexpr int kTileTokens = 32;
constexpr int kTileLdsBytes = 64 * 1024;

template <typename E>
__global__ __launch_bounds__(kThreads) void scatter_kv_tiled(const uint4 *__restrict__ k,
                                                             const E *__restrict__ v,
                                                             const int64_t *__restrict__ slots,
                                                             uint4 *__restrict__ k_pool,
                                                             E *__restrict__ v_pool, int64_t num_tokens,
                                                             int64_t num_slots, int32_t log2_bs,
                                                             int32_t n_kv_heads, int32_t head_dim) {
  constexpr int EC = kTileLdsBytes / kTileTokens / (int)sizeof(E) - 16;  // elements per chunk of a row
  constexpr int ROW = EC + 16 / (int)sizeof(E) + 1;  // padded LDS row: consecutive tokens on other banks
  __shared__ E s_v[kTileTokens * ROW];
  __shared__ int64_t s_slot[kTileTokens];
  const int64_t t0 = (int64_t)blockIdx.x * kTileTokens;
  const int nt = (int)min<int64_t>(kTileTokens, num_tokens - t0);
  if (threadIdx.x < kTileTokens) {
    int64_t s = threadIdx.x < nt ? slots[t0 + threadIdx.x] : -1;
    s_slot[threadIdx.x] = (s < 0 || s >= num_slots) ? -1 : s;  // padding or out of the pool: skipped
  }
  __syncthreads();
  const int row_chunks = head_dim * (int)sizeof(E) / 16;
  const int k_chunks = n_kv_heads * row_chunks;
  for (int f = threadIdx.x; f < nt * k_chunks; f += kThreads) {
    const int i = f / k_chunks, c = f - i * k_chunks;
    const int64_t s = s_slot[i];
    if (s < 0) continue;
    const int head = c / row_chunks, cc = c - head * row_chunks;
    const size_t dst = ((((size_t)(s >> log2_bs) * n_kv_heads + head) << log2_bs) + (s & ((1 << log2_bs) - 1))) *
                           row_chunks + cc;
    k_pool[dst] = k[(size_t)(t0 + i) * k_chunks + c];
  }
  const int v_elems = n_kv_heads * head_dim;
  constexpr int VEC = 16 / (int)sizeof(E);
  for (int e0 = 0; e0 < v_elems; e0 += EC) {
    const int ec = min(EC, v_elems - e0);  // a multiple of VEC: head_dim is
    __syncthreads();                        // the LDS tile is free again
    for (int f = threadIdx.x; f < nt * (ec / VEC); f += kThreads) {
      const int i = f / (ec / VEC), c = f - i * (ec / VEC);
      const uint4 x = reinterpret_cast<const uint4 *>(v + (size_t)(t0 + i) * v_elems + e0)[c];
      const E *xe = reinterpret_cast<const E *>(&x);
#pragma unroll
      for (int u = 0; u < VEC; ++u) s_v[i * ROW + c * VEC + u] = xe[u];
    }
    __syncthreads();
    for (int f = threadIdx.x; f < kTileTokens * ec; f += kThreads) {
      const int i = f % kTileTokens, e = f / kTileTokens;
      if (i >= nt) continue;
      const int64_t s = s_slot[i];
      if (s < 0) continue;
      const size_t dst = (((size_t)(s >> log2_bs) * v_elems + e0 + e) << log2_bs) + (s & ((1 << log2_bs) - 1));
      v_pool[dst] = s_v[i * ROW + e];
    }
  }
}

}  // namespace

hipError_t launch_scatter(const void *k, const void *v, const int64_t *slots, int64_t num_tokens,
                          void *k_pool, void *v_pool, int64_t num_blocks, int32_t block_size,
                          int32_t n_kv_heads, int32_t head_dim, int32_t dtype, hipStream_t stream) {
  int log2_bs = 0;
  while ((1 << log2_bs) < block_size) ++log2_bs;
  if (num_tokens >= kTiledMinTokens) {
    const dim3 grid((unsigned)((num_tokens + kTileTokens - 1) / kTileTokens));
    if (dtype == kF32)
      hipLaunchKernelGGL(scatter_kv_tiled<uint32_t>, grid, dim3(kThreads), 0, stream,
                         static_cast<const uint4 *>(k), static_cast<const uint32_t *>(v), slots,
                         static_cast<uint4 *>(k_pool), static_cast<uint32_t *>(v_pool), num_tokens,
                         num_blocks * block_size, log2_bs, n_kv_heads, head_dim);
    else
      hipLaunchKernelGGL(scatter_kv_tiled<uint16_t>, grid, dim3(kThreads), 0, stream,
                         static_cast<const uint4 *>(k), static_cast<const uint16_t *>(v), slots,
                         static_cast<uint4 *>(k_pool), static_cast<uint16_t *>(v_pool), num_tokens,
                         num_blocks * block_size, log2_bs, n_kv_heads, head_dim);
    return hipGetLastError();
  }
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
