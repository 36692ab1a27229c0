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
 *     section "What I added today": where the gathered read scores a whole
 *     rows x heads x 1 x ctx rectangle at once, the streamed read keeps one
 *     tile of scores per row and head; section "Why it matters": the read
 *     must not read device values back on the host (no sync).
 *
 * Layout (all buffers device memory, row-major, contiguous, 16-byte aligned):
 *   k_pool, v_pool : [num_blocks, n_kv_heads, block_size, head_dim] each
 *                    (position-major: a slot's K or V row for one kv head is
 *                    head_dim contiguous elements, and each (block, kv head)
 *                    tile is one contiguous run of block_size rows)
 *   q, out         : [rows, n_heads, head_dim]
 *   k, v (scatter) : [num_tokens, n_kv_heads, head_dim]
 *   slot_mapping   : [num_tokens] int64; slot s = block * block_size + offset
 *   block_table    : [rows, max_blocks_per_row] int32
 *   context_lens   : [rows] int32, number of positions row r holds
 * Query head h reads kv head h / (n_heads / n_kv_heads).
 *
 * Ownership: the caller owns every buffer, the workspace included; the
 * library allocates no device memory, keeps no state between calls and is
 * reentrant -- except pkv_paged_attention_noalloc, whose static scratch buffer
 * is loaded with the library's code on each GPU and shared by its calls.
 * Every call enqueues its kernels on `stream` (a hipStream_t, NULL = the
 * default stream) and returns without waiting for them.
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
  PKV_ERR_LAUNCH = 10,       /* the HIP runtime refused a launch (hipGetLastError) */
  PKV_ERR_MODE = 11,         /* read counters of different reads (mode or block differ) */
  PKV_ERR_EXHAUSTED = 12,    /* the pool has fewer free blocks than asked for */
  PKV_ERR_SCRATCH = 13       /* pkv_paged_attention_noalloc: the read needs more scratch
                                than PKV_NOALLOC_SCRATCH_BYTES */
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
                                 library default, which depends on the path the
                                 read takes (host shapes only; "table" below is
                                 max_blocks_per_row * block_size positions):
                                 - bf16, head_dim 64/128, at most 8192 rows and
                                   not a small batch: the stream read, whose 1024
                                   persistent waves each take an equal slice of
                                   the batch's (kv head, row, position) stream, at
                                   least 128 positions long (an explicit value
                                   sets that minimum instead);
                                 - bf16, head_dim 64/128, a small batch (at most
                                   256 row x kv head pairs over a table of at
                                   most 4096 positions, or any batch over a table
                                   of at most 1024) or more than 8192 rows: the
                                   matrix-core partition read, partitions of
                                   cdiv(table, cdiv(256, rows x kv heads))
                                   positions clamped to [768, 2048] and rounded
                                   up to block_size (never longer than the table);
                                 - fp32, and bf16 head_dim 16: the VALU partition
                                   read, partitions of about 64 KiB of K and V
                                   (65536 / (2 head_dim elem) positions: fp32 hd
                                   64: 128, fp32 hd 128: 64, fp32 hd 16: 512, bf16
                                   hd 16: 1024), rounded down to block_size and
                                   never longer than the table */
} pkv_attn_desc;

/*
 * pkv_reshape_and_cache -- append new tokens' K/V into the pools.
 * ("Day 25" page, "What I learned", item 1: scatter and gather are exact.)
 *
 * For each token t with s = slot_mapping[t] >= 0: for every kv head g,
 * k_pool[s / block_size, g, s % block_size, :] = k[t, g, :] and
 * v_pool[s / block_size, g, s % block_size, :] = v[t, g, :], copied bit for
 * bit.  Tokens with a negative slot are skipped (padding).
 *
 *   k, v          device [num_tokens, n_kv_heads, head_dim] of `dtype`
 *   slot_mapping  device [num_tokens] int64
 *   k_pool        device [num_blocks, n_kv_heads, block_size, head_dim]
 *   v_pool        device [num_blocks, n_kv_heads, block_size, head_dim]
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
 *   v_pool        device [num_blocks, n_kv_heads, block_size, head_dim]
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

/* Workspace bytes pkv_paged_attention needs for `d` (0 for a NULL or invalid
 * descriptor, and for rows == 0).
 *   - The stream read (see partition_tokens): always non-zero.  4-byte words:
 *     a 4-word header, 2048 words of wave starts, rows + 1 group prefixes
 *     (aligned to 4), then two partial slots per persistent wave (1024 waves)
 *     of align4(G * (head_dim + 2)) fp32 values, G = n_heads / n_kv_heads --
 *     whatever the table width: 4.3 MB for G = 4, head_dim 128.
 *   - The partition reads: per row, query head and partition, fp32 partial
 *     sums of head_dim values plus the running max and sum; 0 when one
 *     partition covers the table. */
size_t pkv_paged_attention_workspace_size(const pkv_attn_desc *d);

/*
 * pkv_paged_attention_noalloc -- pkv_paged_attention for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, results and errors,
 * bit for bit the same output, minus the workspace: the read keeps its
 * partial slots and plan words in a static device buffer of
 * PKV_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on
 * until the process ends.  No device memory is allocated or freed by the
 * call.  A read whose pkv_paged_attention_workspace_size exceeds that size is
 * refused with PKV_ERR_SCRATCH before anything is enqueued.  The buffer is
 * looked up on the first call made with a device current, so `stream` must
 * belong to the current device.  Every call on one GPU shares that GPU's
 * buffer: two calls whose work overlaps on one GPU (another stream, or
 * another thread) race and return garbage; calls in order on one stream do
 * not.  The buffer keeps the last call's contents; no call needs it zeroed.
 */
#define PKV_NOALLOC_SCRATCH_BYTES (32u << 20)
int pkv_paged_attention_noalloc(const pkv_attn_desc *d, const void *q, const void *k_pool,
                                const void *v_pool, const int32_t *block_table,
                                const int32_t *context_lens, float scale, void *out, void *stream);

/*
 * pkv_paged_attention_multi -- the paged read for a chunk of query_len
 * queries per row (chunked prefill over the pool): the rectangle's query_len
 * axis of the "Day 60" page, "What I added today", with a causal mask inside
 * the chunk.
 *
 * The chunk is each row's last query_len positions, already scattered into
 * the pool and counted in context_lens[r] = n.  Query i (0 <= i < query_len)
 * sits at position p = n - query_len + i and attends to positions 0 .. p:
 *   s_t = scale * <q[r,i,h,:], K_t>,  out[r,i,h,:] = sum_{t<=p} softmax(s)_t V_t.
 * A query with p < 0 (a row shorter than the chunk) reads zeros.  With
 * query_len = 1 this is pkv_paged_attention.
 *
 * Precision: scores, softmax and sums in fp32.  For a bf16 out the weights
 * enter the P.V product rounded to bf16 (a change of at most 2^-9 max|V|,
 * the size of the output's own rounding); for an fp32 out they keep 16
 * significant bits (a bf16 hi + lo pair).
 *
 *   d             as for pkv_paged_attention; dtype must be PKV_BF16 and
 *                 head_dim 64 or 128 (else PKV_ERR_DTYPE / PKV_ERR_HEAD_DIM).
 *                 The read takes one of three decompositions (host shapes
 *                 only), and partition_tokens means:
 *                 - query_len * (n_heads / n_kv_heads) <= 16 over a table of
 *                   at least 32 * 1024 groups of 32 positions (rows x kv
 *                   heads x table width): pkv_paged_attention's stream
 *                   decomposition; partition_tokens is the minimum slice
 *                   length as there;
 *                 - else, when one workgroup holds all of a row's queries
 *                   (query_len * group <= 256 columns of 32-column tiles, at
 *                   most 8 tiles), rows <= 256 and rows x kv heads >= 128:
 *                   the balanced read, equal slices of the (kv head, row)
 *                   stream of 32-position groups, one per persistent
 *                   workgroup (every (kv head, row) also charged 12 groups
 *                   for its start); partition_tokens, rounded up to whole
 *                   groups, is the minimum slice (0: 16 groups);
 *                 - else partitions of whole 32-position groups, one
 *                   workgroup per (partition, query block, kv head, row);
 *                   partition_tokens is rounded up to a multiple of 32 and
 *                   capped at 4096 (0: chosen from the shapes).
 *   query_len     1 .. 65535
 *   q, out        device [rows, query_len, n_heads, head_dim]
 *   workspace     >= pkv_paged_attention_multi_workspace_size(d, query_len)
 *                 bytes (NULL allowed when that is 0)
 */
int pkv_paged_attention_multi(const pkv_attn_desc *d, int32_t query_len, const void *q,
                              const void *k_pool, const void *v_pool, const int32_t *block_table,
                              const int32_t *context_lens, float scale, void *out, void *workspace,
                              size_t workspace_bytes, void *stream);

/* Workspace bytes of pkv_paged_attention_multi (0 for an invalid request). */
size_t pkv_paged_attention_multi_workspace_size(const pkv_attn_desc *d, int32_t query_len);

/*
 * pkv_decode_step -- one decode step of every row: append the step's new
 * token, then read.  ("Day 60" page, "Tomorrow": with the streamed read a
 * decode step presents a shape of rows and nothing else.)
 *
 * Equivalent to pkv_reshape_and_cache(k_new, v_new, slot_mapping, d->rows,
 * ...) followed by pkv_paged_attention(d, q, ...), enqueued on `stream`,
 * after every check of both has passed (a refused call enqueues nothing).
 * The new token of row r is counted in context_lens[r] and lives at
 * slot_mapping[r]: it is position context_lens[r] - 1 of the row.  The
 * read kernels append the tokens themselves (the wave or workgroup that
 * reads a row's last position stores the row's token first), so the step is
 * one read launch.  Results and pools are bit for bit those of the two
 * calls.  The kernels' launch shapes depend on the descriptor
 * only (rows, heads, head_dim, block size, table width), never on lengths or
 * block ids, so a captured graph of this call replays for any lengths.
 *
 *   k_new, v_new  device [rows, n_kv_heads, head_dim] of d->dtype
 *   slot_mapping  device [rows] int64 (negative: no token this step)
 *   other arguments as for pkv_paged_attention (k_pool, v_pool written)
 */
int pkv_decode_step(const pkv_attn_desc *d, const void *k_new, const void *v_new,
                    const int64_t *slot_mapping, const void *q, void *k_pool, void *v_pool,
                    const int32_t *block_table, const int32_t *context_lens, float scale, void *out,
                    void *workspace, size_t workspace_bytes, void *stream);

/*
 * Read counters, kept by the caller for the read it runs ("Day 60" page,
 * "What I added today": calls, rows, score cells, held cells and their
 * quotient; "Why it matters": the cells come from shapes, so counting costs
 * no device synchronisation; "What I learned", item 3: a window between two
 * readings of different reads is refused).  Host arithmetic only.
 *
 * A read of `rows` rows, `heads` query heads and `query_len` queries per row
 * over a context `width` positions wide is charged rows*heads*query_len*width
 * score cells (the [rows, heads, query_len, width] rectangle).  The gathered
 * read holds them all; the streamed read holds one tile of min(block, width)
 * positions per (row, head, query).
 */
typedef enum pkv_read_mode {
  PKV_READ_GATHERED = 0,      /* materialises the score rectangle */
  PKV_READ_STREAMED = 1       /* walks tiles of `block` positions */
} pkv_read_mode;

typedef struct pkv_read_stats {
  int32_t mode;               /* pkv_read_mode */
  int32_t block;              /* tile width of a streamed read, >= 1 */
  int64_t calls, rows, score_cells, held_cells;
} pkv_read_stats;

/* Zero the counters of a read of `mode` and tile width `block` (>= 1). */
int pkv_read_stats_init(pkv_read_stats *s, int32_t mode, int32_t block);
/* Count one read of the given shape (all >= 0); PKV_ERR_SHAPE on overflow. */
int pkv_read_stats_record(pkv_read_stats *s, int32_t rows, int32_t heads, int32_t query_len,
                          int32_t width);
/* Positions of one (row, head) whose scores a workgroup of the library's read
 * of `d` holds at once: 32 on the stream read (one wave, one 32-position
 * group), 128 on the matrix-core partition read (four waves of one group
 * each), 1024 * (16 / elem) / head_dim on the VALU partition read (four
 * waves, each scoring four 16-byte-per-lane loads' worth of positions; fp32
 * hd 64: 64, fp32 hd 128: 32, fp32 hd 16: 256, bf16 hd 16: 512); elem is
 * the dtype's size in bytes.  0 for an invalid `d`.  A row cut into
 * partitions holds one such tile per partition. */
int32_t pkv_read_tile(const pkv_attn_desc *d);
/* Count one pkv_paged_attention call of descriptor d on a streamed counter
 * whose block is pkv_read_tile(d) (else PKV_ERR_MODE: the counter is of
 * another read), or on a gathered counter: one query per row.  The library
 * never reads the lengths, so the context width charged is the table's,
 * max_blocks_per_row * block_size, an upper bound of the longest row; a
 * caller that knows the longest row counts it with pkv_read_stats_record. */
int pkv_read_stats_record_read(pkv_read_stats *s, const pkv_attn_desc *d);
/* window = now - earlier; PKV_ERR_MODE if the two readings are of reads with
 * a different mode or block, PKV_ERR_SHAPE if `earlier` is not earlier. */
int pkv_read_stats_since(const pkv_read_stats *now, const pkv_read_stats *earlier,
                         pkv_read_stats *window);
/* score_cells / held_cells; 1.0 when nothing is held (the gathered read
 * holds everything it is charged: its saving is 1, not "unmeasured"). */
double pkv_read_stats_saving(const pkv_read_stats *s);

/*
 * Block allocator of the shared pool (host memory only).  ("Day 17" page,
 * "What I added today" and "Post angle": a pool of fixed blocks handed out to
 * sequences and taken back when they finish, free-and-reuse; running out is
 * an error the caller sees.)  The caller owns the struct and its storage of
 * pkv_allocator_storage_bytes(num_blocks) bytes (4-byte aligned); nothing is
 * allocated.  Not thread-safe: one owner at a time.
 */
typedef struct pkv_block_allocator {
  int32_t *free_ids;          /* stack of free block ids (inside the storage) */
  uint8_t *in_use;            /* one byte per block (inside the storage) */
  int64_t num_blocks, num_free;
} pkv_block_allocator;

size_t pkv_allocator_storage_bytes(int64_t num_blocks);  /* 0 if num_blocks is out of 1..2^31-1 */
/* Every block free.  seed 0 hands out blocks 0, 1, 2, ...; any other seed a
 * shuffled order (splitmix64 + Fisher-Yates), so tables come out fragmented. */
int pkv_allocator_init(pkv_block_allocator *a, void *storage, size_t storage_bytes, int64_t num_blocks,
                       uint64_t seed);
/* Take n blocks into ids[0..n): all or nothing, PKV_ERR_EXHAUSTED if fewer
 * than n are free. */
int pkv_allocator_alloc(pkv_block_allocator *a, int64_t n, int32_t *ids);
/* Give blocks back.  PKV_ERR_SHAPE, with nothing freed, if an id is out of
 * range or not in use (a double free). */
int pkv_allocator_free(pkv_block_allocator *a, const int32_t *ids, int64_t n);
int64_t pkv_allocator_num_free(const pkv_block_allocator *a);
/* Slots of `count` positions appended to a sequence of `length` positions
 * whose block table row is table_row[0..max_blocks): blocks are taken from
 * the allocator as the length crosses block boundaries (written into the
 * row), then slots[i] = block * block_size + offset of position length + i.
 * All or nothing: PKV_ERR_EXHAUSTED takes no block, PKV_ERR_SHAPE if the row
 * would overflow max_blocks. */
int pkv_append_slots(pkv_block_allocator *a, int32_t *table_row, int32_t max_blocks, int32_t block_size,
                     int32_t length, int32_t count, int64_t *slots);

/* Static text for a status code ("unknown status" for anything else). */
const char *pkv_strerror(int status);

/* Version of this ABI: major * 10000 + minor * 100 + patch. */
int pkv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
