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
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
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

// Many tokens (a prompt): one workgroup per (tile of kTileTokens consecutive
// tokens, kv head).  Every load a thread makes -- its K chunks, its V chunks
// and (first threads) the tile's slots -- is issued before any is waited
// for, so a workgroup costs one round trip to memory.  K chunks are then
// stored as above.  V: the tile's [tokens][head_dim] rows, loaded in 16-byte
// chunks, are written into LDS transposed, [head_dim][tokens] (bf16: a token
// pair per 32-bit word, packed with a byte permute).  Each run of 8 tokens
// of one dimension is stored with one 16-byte store (bf16; two for fp32)
// wherever those tokens fill 8 consecutive offsets of one block starting at
// a multiple of 8 -- what a prompt's rows do -- and element by element
// otherwise (padding, out-of-pool slots and scattered tokens included).
constexpr int kTileTokens = 32;

// Streaming accesses: prompt K/V is read once and the pool tiles written
// here are not read again by this call, so neither is kept in the caches.
__device__ __forceinline__ uint4 ntload(const uint4 *p) {
  const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
  return make_uint4(x[0], x[1], x[2], x[3]);
}
__device__ __forceinline__ void ntstore(uint4 *p, uint4 v) {
  const u32x4 x = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(x, reinterpret_cast<u32x4 *>(p));
}

template <typename E>
struct VTile {
  // 32-bit words per LDS row of one dimension: bf16 16 (token pairs), fp32
  // 32, plus 4 of padding (rows stay 16-byte aligned, and consecutive rows
  // start on other banks)
  static constexpr int kPitch = (sizeof(E) == 2 ? kTileTokens / 2 : kTileTokens) + 4;
  // per thread at head_dim 128 (the largest): 16-byte K chunks, and V items
  // (bf16: a token pair, two chunks; fp32: one chunk)
  static constexpr int kKPerThread = kTileTokens * 128 * (int)sizeof(E) / 16 / kThreads;
  static constexpr int kVPerThread = (sizeof(E) == 2 ? kTileTokens / 2 * (128 / 8) : kTileTokens * (128 / 4)) / kThreads;
};

template <typename E>
__global__ __launch_bounds__(kThreads) void scatter_kv_tiled(const uint4 *__restrict__ k,
                                                             const E *__restrict__ v,
                                                             const int64_t *__restrict__ slots,
                                                             uint4 *__restrict__ k_pool,
                                                             E *__restrict__ v_pool, int64_t num_tokens,
                                                             int64_t num_slots, int32_t log2_bs,
                                                             int32_t n_kv_heads, int32_t head_dim) {
  constexpr bool kBF16 = sizeof(E) == 2;
  constexpr int PITCH = VTile<E>::kPitch, KPT = VTile<E>::kKPerThread, VPT = VTile<E>::kVPerThread;
  __shared__ uint32_t s_t[128 * PITCH];  // head_dim <= 128
  __shared__ int64_t s_slot[kTileTokens];
  __shared__ int s_run[kTileTokens / 8];
  const int64_t t0 = (int64_t)blockIdx.x * kTileTokens;
  const int h = blockIdx.y;
  const int nt = (int)min<int64_t>(kTileTokens, num_tokens - t0);
  const int row_chunks = head_dim * (int)sizeof(E) / 16;
  const int k_chunks = n_kv_heads * row_chunks;
  const int v_elems = n_kv_heads * head_dim;
  // -- loads: K chunks (token f / row_chunks, chunk f % row_chunks) --
  uint4 kx[KPT];
#pragma unroll
  for (int u = 0; u < KPT; ++u) {
    const int f = threadIdx.x + u * kThreads;
    const int i = f / row_chunks, c = f - i * row_chunks;
    kx[u] = i < nt ? ntload(k + (size_t)(t0 + i) * k_chunks + h * row_chunks + c) : make_uint4(0, 0, 0, 0);
  }
  // -- V chunks: bf16 item f = token pair f % 16, dimensions 8 (f / 16) .. + 8;
  //    fp32 item f = token f % 32, dimensions 4 (f / 32) .. + 4 --
  constexpr int VL = kBF16 ? 2 : 1;
  const int v_items = kBF16 ? (kTileTokens / 2) * (head_dim / 8) : kTileTokens * (head_dim / 4);
  uint4 vx[VPT][VL];
#pragma unroll
  for (int u = 0; u < VPT; ++u) {
    const int f = threadIdx.x + u * kThreads;
#pragma unroll
    for (int l = 0; l < VL; ++l) {
      int i, col;
      if constexpr (kBF16) {
        i = 2 * (f % (kTileTokens / 2)) + l;
        col = 8 * (f / (kTileTokens / 2));
      } else {
        i = f % kTileTokens;
        col = 4 * (f / kTileTokens);
      }
      vx[u][l] = (f < v_items && i < nt)
                     ? ntload(reinterpret_cast<const uint4 *>(v + (size_t)(t0 + i) * v_elems + (size_t)h * head_dim + col))
                     : make_uint4(0, 0, 0, 0);
    }
  }
  if (threadIdx.x < kTileTokens) {
    const int64_t s = threadIdx.x < nt ? slots[t0 + threadIdx.x] : -1;
    s_slot[threadIdx.x] = (s < 0 || s >= num_slots) ? -1 : s;  // padding or out of the pool: skipped
  }
  // -- V into LDS, transposed --
#pragma unroll
  for (int u = 0; u < VPT; ++u) {
    const int f = threadIdx.x + u * kThreads;
    if (f < v_items) {
      if constexpr (kBF16) {
        const int p = f % (kTileTokens / 2), c = f / (kTileTokens / 2);
        const uint32_t a0[4] = {vx[u][0].x, vx[u][0].y, vx[u][0].z, vx[u][0].w};
        const uint32_t a1[4] = {vx[u][1].x, vx[u][1].y, vx[u][1].z, vx[u][1].w};
#pragma unroll
        for (int w = 0; w < 4; ++w) {  // dimensions 8c + 2w (low halves) and 8c + 2w + 1 (high halves)
          s_t[(8 * c + 2 * w) * PITCH + p] = __builtin_amdgcn_perm(a1[w], a0[w], 0x05040100u);
          s_t[(8 * c + 2 * w + 1) * PITCH + p] = __builtin_amdgcn_perm(a1[w], a0[w], 0x07060302u);
        }
      } else {
        const int i = f % kTileTokens, c = f / kTileTokens;
        s_t[(4 * c) * PITCH + i] = vx[u][0].x;
        s_t[(4 * c + 1) * PITCH + i] = vx[u][0].y;
        s_t[(4 * c + 2) * PITCH + i] = vx[u][0].z;
        s_t[(4 * c + 3) * PITCH + i] = vx[u][0].w;
      }
    }
  }
  __syncthreads();  // slots and the transposed tile are in LDS
  if (threadIdx.x < kTileTokens / 8) {  // tokens 8g .. 8g+7 fill offsets 8m .. 8m+7 of one block
    const int g = threadIdx.x;
    const int64_t s0 = s_slot[8 * g];
    bool run = s0 >= 0 && (s0 & 7) == 0;
    for (int j = 1; j < 8; ++j) run = run && s_slot[8 * g + j] == s0 + j;
    s_run[g] = run;
  }
  // -- K stores --
#pragma unroll
  for (int u = 0; u < KPT; ++u) {
    const int f = threadIdx.x + u * kThreads;
    const int i = f / row_chunks, c = f - i * row_chunks;
    if (i < nt) {
      const int64_t s = s_slot[i];
      if (s >= 0) {
        const size_t dst = ((((size_t)(s >> log2_bs) * n_kv_heads + h) << log2_bs) + (s & ((1 << log2_bs) - 1))) *
                               row_chunks + c;
        ntstore(k_pool + dst, kx[u]);
      }
    }
  }
  __syncthreads();  // run flags
  // -- V stores: dimension d, tokens 8g .. 8g+7 (g fastest: a row's runs side by side) --
  const int bmask = (1 << log2_bs) - 1;
  for (int f = threadIdx.x; f < head_dim * (kTileTokens / 8); f += kThreads) {
    const int g = f & 3, d = f >> 2;
    const uint32_t *row = s_t + d * PITCH;
    if (s_run[g]) {
      const int64_t s0 = s_slot[8 * g];
      E *dst = v_pool + ((((size_t)(s0 >> log2_bs) * n_kv_heads + h) * head_dim + d) << log2_bs) + (s0 & bmask);
      if constexpr (kBF16) {
        ntstore(reinterpret_cast<uint4 *>(dst), *reinterpret_cast<const uint4 *>(row + 4 * g));
      } else {
        ntstore(reinterpret_cast<uint4 *>(dst), *reinterpret_cast<const uint4 *>(row + 8 * g));
        ntstore(reinterpret_cast<uint4 *>(dst) + 1, *reinterpret_cast<const uint4 *>(row + 8 * g + 4));
      }
    } else {
      for (int j = 0; j < 8; ++j) {
        const int i = 8 * g + j;
        const int64_t s = s_slot[i];
        if (s < 0) continue;
        const E e = kBF16 ? (E)(row[i >> 1] >> (16 * (i & 1))) : (E)row[i];
        v_pool[((((size_t)(s >> log2_bs) * n_kv_heads + h) * head_dim + d) << log2_bs) + (s & bmask)] = e;
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
  if (num_tokens >= kTiledMinTokens) {
    const dim3 grid((unsigned)((num_tokens + kTileTokens - 1) / kTileTokens), (unsigned)n_kv_heads);
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
