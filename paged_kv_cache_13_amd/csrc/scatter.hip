// Slot-mapping scatter (reshape_and_cache) for gfx950.
//
// Each new token's K and V rows, for every kv head, are copied bit for bit
// into the pool slot its slot id names: block slot / block_size, offset
// slot % block_size (nanoserve "Day 25" page, "What I learned", item 1: the
// scatter is exact; "Day 17" page, "Post angle": a pool of fixed-size blocks).
// Both pools are [num_blocks, n_kv_heads, block_size, head_dim]: a token's
// row of one kv head is one contiguous run in the pool, as in the input, so
// K and V move the same way, in 16-byte chunks.
//
// Few tokens (a decode step): one workgroup per token.
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kThreads = 256;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int64_t kTiledMinTokens = 1024;  // below: one workgroup per token

__global__ __launch_bounds__(kThreads) void scatter_kv(const uint4 *__restrict__ k, const uint4 *__restrict__ v,
                                                       const int64_t *__restrict__ slots,
                                                       uint4 *__restrict__ k_pool, uint4 *__restrict__ v_pool,
                                                       int64_t num_slots, int32_t log2_bs, int32_t n_kv_heads,
                                                       int32_t row_chunks) {
  const int64_t t = blockIdx.x;
  const int64_t s = slots[t];
  if (s < 0 || s >= num_slots) return;  // padding (or out of the pool: skipped)
  const int64_t blk = s >> log2_bs;
  const int64_t off = s & ((1 << log2_bs) - 1);
  const int chunks = n_kv_heads * row_chunks;  // 16-byte chunks of one token's K (and of its V)
  for (int c = threadIdx.x; c < 2 * chunks; c += kThreads) {
    const bool is_v = c >= chunks;
    const int cc = is_v ? c - chunks : c;
    const int head = cc / row_chunks;
    const size_t dst = ((((size_t)blk * n_kv_heads + head) << log2_bs) + off) * row_chunks + (cc - head * row_chunks);
    (is_v ? v_pool : k_pool)[dst] = (is_v ? v : k)[(size_t)t * chunks + cc];
  }
}

// Many tokens (a prompt): one workgroup per (tile of kTileTokens consecutive
// tokens, kv head).  Every load a thread makes -- its K and V chunks and
// (first threads) the tile's slots -- is issued before any is waited for,
// so a workgroup costs one round trip to memory; then the chunks are stored
// at their slots.  Non-temporal loads and stores: prompt K/V is read once
// and the pool tiles written here are not read again by this call.
constexpr int kTileTokens = 32;
// 16-byte chunks per thread for one of K or V at head_dim 128 (the largest)
template <typename E>
constexpr int tile_chunks_per_thread() { return kTileTokens * 128 * (int)sizeof(E) / 16 / kThreads; }

__device__ __forceinline__ uint4 ntload(const uint4 *p) {
  const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
  return make_uint4(x[0], x[1], x[2], x[3]);
}
__device__ __forceinline__ void ntstore(uint4 *p, uint4 v) {
  const u32x4 x = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(x, reinterpret_cast<u32x4 *>(p));
}

template <typename E>
__global__ __launch_bounds__(kThreads) void scatter_kv_tiled(const uint4 *__restrict__ k, const uint4 *__restrict__ v,
                                                             const int64_t *__restrict__ slots,
                                                             uint4 *__restrict__ k_pool, uint4 *__restrict__ v_pool,
                                                             int64_t num_tokens, int64_t num_slots, int32_t log2_bs,
                                                             int32_t n_kv_heads, int32_t row_chunks) {
  constexpr int CPT = tile_chunks_per_thread<E>();
  __shared__ int64_t s_slot[kTileTokens];
  const int64_t t0 = (int64_t)blockIdx.x * kTileTokens;
  const int h = blockIdx.y;
  const int nt = (int)min<int64_t>(kTileTokens, num_tokens - t0);
  const int chunks = n_kv_heads * row_chunks;
  // chunk f of the tile: token f / row_chunks, chunk f % row_chunks of its row
  uint4 kx[CPT], vx[CPT];
#pragma unroll
  for (int u = 0; u < CPT; ++u) {
    const int f = threadIdx.x + u * kThreads;
    const int i = f / row_chunks, c = f - i * row_chunks;
    const size_t src = (size_t)(t0 + i) * chunks + h * row_chunks + c;
    const bool live = i < nt;
    kx[u] = live ? ntload(k + src) : make_uint4(0, 0, 0, 0);
    vx[u] = live ? ntload(v + src) : make_uint4(0, 0, 0, 0);
  }
  if (threadIdx.x < kTileTokens) {
    const int64_t s = threadIdx.x < nt ? slots[t0 + threadIdx.x] : -1;
    s_slot[threadIdx.x] = (s < 0 || s >= num_slots) ? -1 : s;  // padding or out of the pool: skipped
  }
  __syncthreads();  // the tile's slots are in LDS
  const int bmask = (1 << log2_bs) - 1;
#pragma unroll
  for (int u = 0; u < CPT; ++u) {
    const int f = threadIdx.x + u * kThreads;
    const int i = f / row_chunks, c = f - i * row_chunks;
    if (i < nt) {
      const int64_t s = s_slot[i];
      if (s >= 0) {
        const size_t dst = ((((size_t)(s >> log2_bs) * n_kv_heads + h) << log2_bs) + (s & bmask)) * row_chunks + c;
        ntstore(k_pool + dst, kx[u]);
        ntstore(v_pool + dst, vx[u]);
      }
    }
  }
}

}  // namespace

hipError_t launch_scatter(const void *k, const void *v, const int64_t *slots, int64_t num_tokens,
                          void *k_pool, void *v_pool, int64_t num_blocks, int32_t block_size,
                          int32_t n_kv_heads, int32_t head_dim, int32_t dtype, hipStream_t stream) {
  int log2_bs = 0;
  while ((1 << log2_bs) < block_size) ++log2_bs;
  const int32_t row_chunks = head_dim * (dtype == kF32 ? 4 : 2) / 16;
  const uint4 *k4 = static_cast<const uint4 *>(k), *v4 = static_cast<const uint4 *>(v);
  uint4 *kp4 = static_cast<uint4 *>(k_pool), *vp4 = static_cast<uint4 *>(v_pool);
  if (num_tokens >= kTiledMinTokens) {
    const dim3 grid((unsigned)((num_tokens + kTileTokens - 1) / kTileTokens), (unsigned)n_kv_heads);
    if (dtype == kF32)
      hipLaunchKernelGGL(scatter_kv_tiled<uint32_t>, grid, dim3(kThreads), 0, stream, k4, v4, slots, kp4, vp4,
                         num_tokens, num_blocks * block_size, log2_bs, n_kv_heads, row_chunks);
    else
      hipLaunchKernelGGL(scatter_kv_tiled<uint16_t>, grid, dim3(kThreads), 0, stream, k4, v4, slots, kp4, vp4,
                         num_tokens, num_blocks * block_size, log2_bs, n_kv_heads, row_chunks);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(scatter_kv, dim3((unsigned)num_tokens), dim3(kThreads), 0, stream, k4, v4, slots, kp4, vp4,
                     num_blocks * block_size, log2_bs, n_kv_heads, row_chunks);
  return hipGetLastError();
}

}  // namespace pkv
