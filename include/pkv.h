/*
 * pkv.h -- C ABI of libpkv.so: the slot-mapping scatter and the paged decode
 * read of a block-paged KV cache, as hand-written HIP kernels for gfx950.
 *
 * The operations are the ones the nanoserve dev log builds its paged cache
 * around:
 *   - "Day 17: paging under the sampling path, free-and-reuse closes Week 5",
 *     section "Post angle": K/V live in a pool of fixed-size blocks, and a
 *     block table maps each token position of a sequence to a block;
 *   - "Day 25: the fused read dispatches to the kernel backend", section
 *     "What I added today": the cache's read is handed the layer's K/V pools
 *     and the whole history's slot mapping and returns attention over the
 *     assembled slots; section "Why it matters": the kernel streams an online
 *     softmax instead of materialising the history; section "Diagram": the
 *     result goes back to grouped-query attention;
 *   - "Day 60: the read becomes a choice, and a counter is what can see it",
 *     section "What I added today": the streamed read never builds the
 *     [rows, heads, 1, ctx] score rectangle; section "Why it matters": the
 *     read must not read device values back on the host (no sync).
 *
 * Layout (all buffers device memory, row-major, contiguous, 16-byte aligned):
 *   k_pool         : [num_blocks, n_kv_heads, block_size, head_dim]
 *   v_pool         : [num_blocks, n_kv_heads, head_dim, block_size]
 *                    (each (block, kv head) tile is one contiguous run; inside
 *                    it K is position-major and V dimension-major, so both
 *                    contractions of the read find their reduction index
 *                    contiguous: head_dim for q.K, positions for p.V)
 *   q, out         : [rows, n_heads, head_dim]
 *   k, v (scatter) : [num_tokens, n_kv_heads, head_dim]
 *   slot_mapping   : [num_tokens] int64; slot s = block * block_size + offset
 *   block_table    : [rows, max_blocks_per_row] int32
 *   context_lens   : [rows] int32, number of positions row r holds
 * Query head h reads kv head h / (n_heads / n_kv_heads).
 *
 * Ownership: the caller owns every buffer, the workspace included; the
 * library allocates no device memory, keeps no state between calls and is
 * reentrant.  Every call enqueues its kernels on `stream` (a hipStream_t,
 * NULL = the default stream) and returns without waiting for them.
 *
 * Errors: every entry point returns a pkv_status and never aborts.  Shapes,
 * pointers, alignment, dtypes and the workspace size are checked on the host
 * before anything is enqueued; a refused call enqueues nothing.  Values that
 * live in device memory (block ids, lengths, slots) are never read back: they
 * are the caller's contract (see each function).  Kernels clamp lengths into
 * [0, max_blocks_per_row * block_size] and block ids into [0, num_blocks) so
 * that a broken table cannot make them read outside the buffers; the result
 * for such input is unspecified.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pkv_status {
  PKV_OK = 0,
  PKV_ERR_NULL = 1,          /* a required pointer is NULL */
  PKV_ERR_ALIGN = 2,         /* a buffer is not 16-byte aligned */
  PKV_ERR_DTYPE = 3,         /* unsupported dtype code */
  PKV_ERR_HEADS = 4,         /* n_heads % n_kv_heads != 0, or group > 16 */
  PKV_ERR_HEAD_DIM = 5,      /* head_dim not in {16, 64, 128} */
  PKV_ERR_BLOCK_SIZE = 6,    /* block_size not in {8, 16, 32} */
  PKV_ERR_SHAPE = 7,         /* a size is negative, zero where it may not be, or overflows */
  PKV_ERR_WORKSPACE = 8,     /* workspace NULL or smaller than pkv_paged_attention_workspace_size */
  PKV_ERR_PARTITION = 9,     /* partition_tokens not a positive multiple of block_size */
  PKV_ERR_LAUNCH = 10        /* the HIP runtime refused a launch (hipGetLastError) */
} pkv_status;

typedef enum pkv_dtype {
  PKV_F32 = 0,               /* IEEE binary32 */
  PKV_BF16 = 1               /* bfloat16 */
} pkv_dtype;

/* Shape and type of one paged decode read.  All fields are host scalars. */
typedef struct pkv_attn_desc {
  int32_t rows;               /* decode rows (sequences) in the batch, >= 0 */
  int32_t n_heads;            /* query heads */
  int32_t n_kv_heads;         /* kv heads; n_heads % n_kv_heads == 0, group <= 16 */
  int32_t head_dim;           /* 16, 64 or 128 */
  int32_t block_size;         /* positions per pool block: 8, 16 or 32 */
  int32_t max_blocks_per_row; /* width of block_table, >= 1 */
  int64_t num_blocks;         /* blocks in each pool, >= 1 */
  int32_t dtype;              /* pkv_dtype of q, k_pool, v_pool */
  int32_t out_dtype;          /* pkv_dtype of out (normally == dtype) */
  int32_t partition_tokens;   /* split-context partition length in positions,
                                 a positive multiple of block_size, or 0 for the
                                 library default: bf16 head_dim 64/128 reads cut
                                 rows into slices of at least 128 positions;
                                 other reads use partitions of at most 512
                                 positions, shorter when rows x kv heads are
                                 too few to fill the GPU */
} pkv_attn_desc;

/*
 * pkv_reshape_and_cache -- append new tokens' K/V into the pools.
 * ("Day 25" page, "What I learned", item 1: scatter and gather are exact.)
 *
 * For each token t with s = slot_mapping[t] >= 0: for every kv head g,
 * k_pool[s / block_size, g, s % block_size, :] = k[t, g, :] and
 * v_pool[s / block_size, g, :, s % block_size] = v[t, g, :], copied bit for
 * bit.  Tokens with a negative slot are skipped (padding).
 *
 *   k, v          device [num_tokens, n_kv_heads, head_dim] of `dtype`
 *   slot_mapping  device [num_tokens] int64
 *   k_pool        device [num_blocks, n_kv_heads, block_size, head_dim]
 *   v_pool        device [num_blocks, n_kv_heads, head_dim, block_size]
 *   num_tokens >= 0 (0 enqueues nothing); num_blocks >= 1
 * Caller contract (not checked on device): slots < num_blocks * block_size
 * (larger ones are skipped) and distinct within one call (duplicates race).
 */
int pkv_reshape_and_cache(const void *k, const void *v, const int64_t *slot_mapping,
                          int64_t num_tokens, void *k_pool, void *v_pool,
                          int64_t num_blocks, int32_t block_size, int32_t n_kv_heads,
                          int32_t head_dim, int32_t dtype, void *stream);

/*
 * pkv_paged_attention -- the paged decode read with grouped-query heads.
 *
 * For each row r with n = context_lens[r] and each query head h (kv head
 * g = h / (n_heads / n_kv_heads)): position t < n is read from block
 * block_table[r, t / block_size] at offset t % block_size;
 *   s_t = scale * <q[r,h,:], K_t>,  out[r,h,:] = sum_t softmax(s)_t * V_t,
 * with scores and sums in fp32 and the softmax streamed online over the
 * positions ("Day 25" page, "Why it matters").  A row with n == 0 reads zeros.
 * Rows longer than `partition_tokens` are split into partitions that are
 * read in parallel and merged (running max, rescaled sums) in a second pass.
 * Positions >= n and table entries past cdiv(n, block_size) are never read,
 * so they may hold anything, NaN included.
 *
 *   d             shapes and dtypes (host struct, read during the call only)
 *   q             device [rows, n_heads, head_dim] of d->dtype
 *   k_pool        device [num_blocks, n_kv_heads, block_size, head_dim]
 *   v_pool        device [num_blocks, n_kv_heads, head_dim, block_size]
 *   block_table   device [rows, max_blocks_per_row] int32
 *   context_lens  device [rows] int32
 *   scale         softmax scale applied to the fp32 dot product
 *   out           device [rows, n_heads, head_dim] of d->out_dtype;
 *                 fp32 -> bf16 rounds to nearest even
 *   workspace     device scratch of >= pkv_paged_attention_workspace_size(d)
 *                 bytes (may be NULL when that size is 0); the caller must not
 *                 touch it until the call's work on `stream` has finished
 * Caller contract (not checked on device): 0 <= context_lens[r] <=
 * max_blocks_per_row * block_size; block ids in [0, num_blocks).
 */
int pkv_paged_attention(const pkv_attn_desc *d, const void *q, const void *k_pool,
                        const void *v_pool, const int32_t *block_table,
                        const int32_t *context_lens, float scale, void *out,
                        void *workspace, size_t workspace_bytes, void *stream);

/* Workspace bytes pkv_paged_attention needs for `d`: per row, query head and
 * partition, fp32 partial sums of head_dim values plus the running max and
 * sum.  0 when no row can span more than one partition.  Returns 0 for a
 * NULL descriptor. */
size_t pkv_paged_attention_workspace_size(const pkv_attn_desc *d);

/* Static text for a status code ("unknown status" for anything else). */
const char *pkv_strerror(int status);

/* Version of this ABI: major * 10000 + minor * 100 + patch. */
int pkv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
