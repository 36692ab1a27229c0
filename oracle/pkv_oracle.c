/*
 * pkv_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow CPU oracle for the two operations of a block-paged KV cache:
 * the slot-mapping scatter that appends new K/V into a pool of fixed-size
 * blocks, and the decode read in which each row's single query attends over
 * its whole history.  Only tests, the smoke check and the benchmark's CPU
 * baseline may load this library; the product path never does, and this file
 * shares no code, header or constant with the HIP library.
 *
 * Sources (nanoserve dev log):
 *  - "Day 25: the fused read dispatches to the kernel backend", section
 *    "What I added today": the reference read is SDPA over the slots the
 *    history was assembled from; section "What I learned", item 1: that
 *    reference runs the causal softmax by exact index, and the scatter and
 *    gather are exact (same K/V, same slots).
 *  - "Day 17: paging under the sampling path ...", section "Post angle": a
 *    pool of fixed KV blocks and a block table mapping tokens to blocks.
 *  - "Day 60: the read becomes a choice ...", section "What I added today":
 *    the gathered read scores a [rows, heads, 1, ctx] rectangle through the
 *    whole [rows, max_ctx] slot mapping; the streamed read walks tiles.
 *
 * Arithmetic is IEEE double throughout.  The pages state that their reference
 * softmax runs in fp32; double is the closer stand-in for the exact
 * definition, and the GPU's fp32 result is compared against it under the
 * pages' tolerance (Day 25 page, "What I learned", item 2).
 *
 * Layout conventions (the pages leave the pool layout open; this is the
 * reading adopted for both sides of the test):
 *   k_pool         : [num_blocks, n_kv_heads, block_size, head_dim]
 *   v_pool         : [num_blocks, n_kv_heads, block_size, head_dim]
 *                    (the same position-major layout as K)
 *   q              : [rows, n_heads, head_dim]
 *   k, v (scatter) : [num_tokens, n_kv_heads, head_dim]
 *   slot s         : block s / block_size, offset s % block_size
 *   query head h   : reads kv head h / (n_heads / n_kv_heads)
 * Element types: 0 = IEEE binary32, 1 = bfloat16 (upper half of a binary32).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F32 0
#define ORC_BF16 1

#define ORC_OK 0
#define ORC_EBADARG 1
#define ORC_ERANGE 2
#define ORC_ENOMEM 3

static size_t elem_bytes(int32_t dtype) { return dtype == ORC_F32 ? 4u : 2u; }

/* Widen one stored element to double.  bf16 -> binary32 is a 16-bit shift,
 * binary32 -> double is exact, so this loses nothing. */
static double widen(const void *base, int64_t idx, int32_t dtype) {
  float f;
  if (dtype == ORC_F32) {
    memcpy(&f, (const unsigned char *)base + 4 * idx, 4);
  } else {
    uint16_t h;
    uint32_t bits;
    memcpy(&h, (const unsigned char *)base + 2 * idx, 2);
    bits = (uint32_t)h << 16;
    memcpy(&f, &bits, 4);
  }
  return (double)f;
}

/* ------------------------------------------------------------------------ */
/* Scatter: for each new token t in ascending order, its slot s picks       */
/* (block s / bs, offset s % bs); the token's K and V rows for every kv     */
/* head are copied there bit for bit.  A negative slot is padding and is    */
/* skipped.                                                                 */
/* Duplicate slots leave the last writer (never relied upon).               */
/* ------------------------------------------------------------------------ */
int oracle_reshape_and_cache(const void *k, const void *v,
                             const int64_t *slot_mapping, int64_t num_tokens,
                             void *k_pool, void *v_pool, int64_t num_blocks,
                             int32_t block_size, int32_t n_kv_heads,
                             int32_t head_dim, int32_t dtype) {
  size_t row_bytes, es;
  int64_t t;
  int32_t g;
  if (!k || !v || !slot_mapping || !k_pool || !v_pool) return ORC_EBADARG;
  if (num_tokens < 0 || num_blocks <= 0 || block_size <= 0 || n_kv_heads <= 0 ||
      head_dim <= 0 || (dtype != ORC_F32 && dtype != ORC_BF16))
    return ORC_EBADARG;
  es = elem_bytes(dtype);
  row_bytes = (size_t)head_dim * es;
  for (t = 0; t < num_tokens; ++t) {
    int64_t s = slot_mapping[t];
    int64_t blk, off;
    if (s < 0) continue;
    if (s >= num_blocks * (int64_t)block_size) return ORC_ERANGE;
    blk = s / block_size;
    off = s % block_size;
    for (g = 0; g < n_kv_heads; ++g) {
      size_t src = ((size_t)t * n_kv_heads + g) * row_bytes;
      size_t dst = (((size_t)blk * n_kv_heads + g) * block_size + off) * row_bytes;
      memcpy((unsigned char *)k_pool + dst, (const unsigned char *)k + src, row_bytes);
      memcpy((unsigned char *)v_pool + dst, (const unsigned char *)v + src, row_bytes);
    }
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Softmax attention of one query row over an assembled contiguous history. */
/*   s[t] = scale * sum_d q[d] * K[t][d]          (d ascending)             */
/*   m = max_t s[t];  p[t] = exp(s[t] - m);  l = sum_t p[t]                 */
/*   out[d] = (sum_t p[t] * V[t][d]) / l          (t ascending)             */
/* K and V are [n][stride] doubles, the head's slice starting at column 0.  */
/* ------------------------------------------------------------------------ */
static void attend_one(const double *qv, const double *Kc, const double *Vc,
                       int64_t n, int64_t stride, int32_t head_dim,
                       double scale, double *s, double *out) {
  int64_t t;
  int32_t d;
  double m = -INFINITY, l = 0.0;
  for (t = 0; t < n; ++t) {
    double dot = 0.0;
    for (d = 0; d < head_dim; ++d) dot += qv[d] * Kc[t * stride + d];
    s[t] = scale * dot;
    if (s[t] > m) m = s[t];
  }
  for (t = 0; t < n; ++t) {
    s[t] = exp(s[t] - m);
    l += s[t];
  }
  for (d = 0; d < head_dim; ++d) {
    double acc = 0.0;
    for (t = 0; t < n; ++t) acc += s[t] * Vc[t * stride + d];
    out[d] = acc / l;
  }
}

/* Shared by both gathered entry points: given each row's per-position slot
 * (already resolved), assemble the history and attend.  slot_of(r, t) is
 * provided by the caller through the `slots` array of width `width`. */
static int gathered_read(int32_t rows, int32_t n_heads, int32_t n_kv_heads,
                         int32_t head_dim, int32_t block_size,
                         int64_t num_blocks, int32_t dtype, const void *q,
                         const void *k_pool, const void *v_pool,
                         const int64_t *slots, int64_t width,
                         const int32_t *context_lens, double scale,
                         double *out) {
  int32_t r, h, g, d;
  int32_t group;
  int64_t t;
  double *Kc, *Vc, *s, *qv;
  if (!q || !k_pool || !v_pool || !slots || !context_lens || !out)
    return ORC_EBADARG;
  if (rows < 0 || n_heads <= 0 || n_kv_heads <= 0 || head_dim <= 0 ||
      block_size <= 0 || num_blocks <= 0 || width < 0 ||
      n_heads % n_kv_heads != 0 || (dtype != ORC_F32 && dtype != ORC_BF16))
    return ORC_EBADARG;
  group = n_heads / n_kv_heads;
  Kc = (double *)malloc(sizeof(double) * (size_t)(width > 0 ? width : 1) * n_kv_heads * head_dim);
  Vc = (double *)malloc(sizeof(double) * (size_t)(width > 0 ? width : 1) * n_kv_heads * head_dim);
  s = (double *)malloc(sizeof(double) * (size_t)(width > 0 ? width : 1));
  qv = (double *)malloc(sizeof(double) * (size_t)head_dim);
  if (!Kc || !Vc || !s || !qv) {
    free(Kc); free(Vc); free(s); free(qv);
    return ORC_ENOMEM;
  }
  for (r = 0; r < rows; ++r) {
    int64_t n = context_lens[r];
    if (n < 0 || n > width) {
      free(Kc); free(Vc); free(s); free(qv);
      return ORC_ERANGE;
    }
    if (n == 0) {
      /* No history: the read returns zeros (the pages do not say; this is
       * the reading adopted for an empty row). */
      for (h = 0; h < n_heads; ++h)
        for (d = 0; d < head_dim; ++d)
          out[((size_t)r * n_heads + h) * head_dim + d] = 0.0;
      continue;
    }
    /* Assemble the row's history by exact index: position t lives in the
     * pool at slot slots[r][t]. Positions at or past n are never touched. */
    for (t = 0; t < n; ++t) {
      int64_t sl = slots[(size_t)r * width + t];
      int64_t blk, off;
      if (sl < 0 || sl >= num_blocks * (int64_t)block_size) {
        free(Kc); free(Vc); free(s); free(qv);
        return ORC_ERANGE;
      }
      blk = sl / block_size;
      off = sl % block_size;
      for (g = 0; g < n_kv_heads; ++g) {
        int64_t src = (((int64_t)blk * n_kv_heads + g) * block_size + off) * head_dim;
        for (d = 0; d < head_dim; ++d) {
          Kc[((size_t)t * n_kv_heads + g) * head_dim + d] = widen(k_pool, src + d, dtype);
          Vc[((size_t)t * n_kv_heads + g) * head_dim + d] = widen(v_pool, src + d, dtype);
        }
      }
    }
    for (h = 0; h < n_heads; ++h) {
      int32_t kvh = h / group;
      for (d = 0; d < head_dim; ++d)
        qv[d] = widen(q, ((int64_t)r * n_heads + h) * head_dim + d, dtype);
      attend_one(qv, Kc + (size_t)kvh * head_dim, Vc + (size_t)kvh * head_dim, n,
                 (int64_t)n_kv_heads * head_dim, head_dim, scale, s,
                 out + ((size_t)r * n_heads + h) * head_dim);
    }
  }
  free(Kc); free(Vc); free(s); free(qv);
  return ORC_OK;
}

/* The gathered read, driven by slots instead of a block table: row r's
 * position t lives at pool slot slot_mapping[r * width + t] ("Day 25: the
 * fused read dispatches to the kernel backend", "What I added today").
 * *score_cells receives the number of scores this read holds at once,
 * rows * n_heads * 1 * width ("Day 60: the read becomes a choice, and a
 * counter is what can see it", "What I added today"; one query per row in
 * decode). */
int oracle_paged_attention_slots(int32_t rows, int32_t n_heads,
                                 int32_t n_kv_heads, int32_t head_dim,
                                 int32_t block_size, int64_t num_blocks,
                                 int32_t dtype, const void *q,
                                 const void *k_pool, const void *v_pool,
                                 const int64_t *slot_mapping, int64_t width,
                                 const int32_t *context_lens, double scale,
                                 double *out, int64_t *score_cells) {
  int rc = gathered_read(rows, n_heads, n_kv_heads, head_dim, block_size,
                         num_blocks, dtype, q, k_pool, v_pool, slot_mapping,
                         width, context_lens, scale, out);
  if (rc == ORC_OK && score_cells)
    *score_cells = (int64_t)rows * n_heads * 1 * width;
  return rc;
}

/* The gathered read addressed through a block table [rows,
 * max_blocks_per_row]: position t of row r is in block
 * block_table[r][t / block_size] at offset t % block_size, i.e. slot
 * block_table[r][t / block_size] * block_size + t % block_size. */
int oracle_paged_attention(int32_t rows, int32_t n_heads, int32_t n_kv_heads,
                           int32_t head_dim, int32_t block_size,
                           int32_t max_blocks_per_row, int64_t num_blocks,
                           int32_t dtype, const void *q, const void *k_pool,
                           const void *v_pool, const int32_t *block_table,
                           const int32_t *context_lens, double scale,
                           double *out) {
  int64_t width, t;
  int32_t r;
  int64_t *slots;
  int rc;
  if (!block_table || !context_lens || max_blocks_per_row < 0 || rows < 0 ||
      block_size <= 0)
    return ORC_EBADARG;
  width = (int64_t)max_blocks_per_row * block_size;
  slots = (int64_t *)malloc(sizeof(int64_t) * (size_t)(rows > 0 ? rows : 1) *
                            (size_t)(width > 0 ? width : 1));
  if (!slots) return ORC_ENOMEM;
  for (r = 0; r < rows; ++r) {
    int64_t n = context_lens[r];
    for (t = 0; t < width; ++t) {
      /* Only positions the row actually holds are resolved; the rest of the
       * table may hold anything and is never read. */
      if (t < n)
        slots[(size_t)r * width + t] =
            (int64_t)block_table[(size_t)r * max_blocks_per_row + t / block_size] *
                block_size + t % block_size;
      else
        slots[(size_t)r * width + t] = -1;
    }
  }
  rc = gathered_read(rows, n_heads, n_kv_heads, head_dim, block_size,
                     num_blocks, dtype, q, k_pool, v_pool, slots, width,
                     context_lens, scale, out);
  free(slots);
  return rc;
}

/* ------------------------------------------------------------------------ */
/* The streamed read: one program per (row, head) walks the row's history   */
/* in tiles of `tile` positions and never holds more than one tile of       */
/* scores (Day 60 page, "Why it matters": tiles walked is cdiv over the     */
/* context lengths).  Online softmax per tile:                              */
/*   m' = max(m, max_t s[t]);  a = exp(m - m')                              */
/*   l  = l * a + sum_t exp(s[t] - m')                                      */
/*   acc = acc * a + sum_t exp(s[t] - m') * V[t]                            */
/* out = acc / l.  *held_cells receives the sum over programs of the widest */
/* score tile each held, the quantity the Day 60 table calls "held".        */
/* ------------------------------------------------------------------------ */
int oracle_paged_attention_streamed(int32_t rows, int32_t n_heads,
                                    int32_t n_kv_heads, int32_t head_dim,
                                    int32_t block_size,
                                    int32_t max_blocks_per_row,
                                    int64_t num_blocks, int32_t dtype,
                                    const void *q, const void *k_pool,
                                    const void *v_pool,
                                    const int32_t *block_table,
                                    const int32_t *context_lens, double scale,
                                    int32_t tile, double *out,
                                    int64_t *held_cells) {
  int32_t r, h, d;
  int32_t group;
  double *qv, *st, *acc;
  int64_t held = 0;
  if (!q || !k_pool || !v_pool || !block_table || !context_lens || !out)
    return ORC_EBADARG;
  if (rows < 0 || n_heads <= 0 || n_kv_heads <= 0 || head_dim <= 0 ||
      block_size <= 0 || num_blocks <= 0 || tile <= 0 ||
      max_blocks_per_row < 0 || n_heads % n_kv_heads != 0 ||
      (dtype != ORC_F32 && dtype != ORC_BF16))
    return ORC_EBADARG;
  group = n_heads / n_kv_heads;
  qv = (double *)malloc(sizeof(double) * (size_t)head_dim);
  st = (double *)malloc(sizeof(double) * (size_t)tile);
  acc = (double *)malloc(sizeof(double) * (size_t)head_dim);
  if (!qv || !st || !acc) {
    free(qv); free(st); free(acc);
    return ORC_ENOMEM;
  }
  for (r = 0; r < rows; ++r) {
    int64_t n = context_lens[r];
    if (n < 0 || n > (int64_t)max_blocks_per_row * block_size) {
      free(qv); free(st); free(acc);
      return ORC_ERANGE;
    }
    for (h = 0; h < n_heads; ++h) {
      int32_t kvh = h / group;
      double m = -INFINITY, l = 0.0;
      int64_t widest = 0, start, t;
      double *o = out + ((size_t)r * n_heads + h) * head_dim;
      for (d = 0; d < head_dim; ++d) {
        qv[d] = widen(q, ((int64_t)r * n_heads + h) * head_dim + d, dtype);
        acc[d] = 0.0;
      }
      for (start = 0; start < n; start += tile) {
        int64_t w = n - start < tile ? n - start : tile;
        double mt = -INFINITY, m_new, alpha;
        if (w > widest) widest = w;
        for (t = 0; t < w; ++t) {
          int64_t pos = start + t;
          int64_t blk = block_table[(size_t)r * max_blocks_per_row + pos / block_size];
          int64_t base = ((blk * n_kv_heads + kvh) * block_size + pos % block_size) * head_dim;
          double dot = 0.0;
          if (blk < 0 || blk >= num_blocks) {
            free(qv); free(st); free(acc);
            return ORC_ERANGE;
          }
          for (d = 0; d < head_dim; ++d) dot += qv[d] * widen(k_pool, base + d, dtype);
          st[t] = scale * dot;
          if (st[t] > mt) mt = st[t];
        }
        m_new = m > mt ? m : mt;
        alpha = exp(m - m_new); /* exp(-inf) = 0 on the first tile */
        l *= alpha;
        for (d = 0; d < head_dim; ++d) acc[d] *= alpha;
        for (t = 0; t < w; ++t) {
          int64_t pos = start + t;
          int64_t blk = block_table[(size_t)r * max_blocks_per_row + pos / block_size];
          int64_t vrow = ((blk * n_kv_heads + kvh) * block_size + pos % block_size) * head_dim;
          double p = exp(st[t] - m_new);
          l += p;
          for (d = 0; d < head_dim; ++d) acc[d] += p * widen(v_pool, vrow + d, dtype);
        }
        m = m_new;
      }
      for (d = 0; d < head_dim; ++d) o[d] = n > 0 ? acc[d] / l : 0.0;
      held += widest;
    }
  }
  if (held_cells) *held_cells = held;
  free(qv); free(st); free(acc);
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Multi-query read (a chunk of query_len new positions per row over the    */
/* pool, as in chunked prefill): the chunk is the last query_len positions  */
/* of the row's context, already in the pool.  Query i of row r sits at     */
/* position p = n - query_len + i and attends causally to t <= p, i.e. to   */
/* the first p + 1 positions of the assembled history (Day 60 page, "What   */
/* I added today": the rectangle's query_len axis).  A query with p < 0 has */
/* no history and reads zeros (the empty-row reading).                      */
/* q and out are [rows][query_len][n_heads][head_dim].                      */
/* ------------------------------------------------------------------------ */
int oracle_paged_attention_multi(int32_t rows, int32_t query_len, int32_t n_heads,
                                 int32_t n_kv_heads, int32_t head_dim,
                                 int32_t block_size, int32_t max_blocks_per_row,
                                 int64_t num_blocks, int32_t dtype, const void *q,
                                 const void *k_pool, const void *v_pool,
                                 const int32_t *block_table,
                                 const int32_t *context_lens, double scale,
                                 double *out) {
  int32_t r, i, h, g, d;
  int32_t group;
  int64_t t, width;
  double *Kc, *Vc, *s, *qv;
  if (!q || !k_pool || !v_pool || !block_table || !context_lens || !out)
    return ORC_EBADARG;
  if (rows < 0 || query_len <= 0 || n_heads <= 0 || n_kv_heads <= 0 ||
      head_dim <= 0 || block_size <= 0 || num_blocks <= 0 ||
      max_blocks_per_row < 0 || n_heads % n_kv_heads != 0 ||
      (dtype != ORC_F32 && dtype != ORC_BF16))
    return ORC_EBADARG;
  group = n_heads / n_kv_heads;
  width = (int64_t)max_blocks_per_row * block_size;
  Kc = (double *)malloc(sizeof(double) * (size_t)(width > 0 ? width : 1) * n_kv_heads * head_dim);
  Vc = (double *)malloc(sizeof(double) * (size_t)(width > 0 ? width : 1) * n_kv_heads * head_dim);
  s = (double *)malloc(sizeof(double) * (size_t)(width > 0 ? width : 1));
  qv = (double *)malloc(sizeof(double) * (size_t)head_dim);
  if (!Kc || !Vc || !s || !qv) {
    free(Kc); free(Vc); free(s); free(qv);
    return ORC_ENOMEM;
  }
  for (r = 0; r < rows; ++r) {
    int64_t n = context_lens[r];
    if (n < 0 || n > width) {
      free(Kc); free(Vc); free(s); free(qv);
      return ORC_ERANGE;
    }
    /* The row's history by exact index through its block table. */
    for (t = 0; t < n; ++t) {
      int64_t blk = block_table[(size_t)r * max_blocks_per_row + t / block_size];
      int64_t off = t % block_size;
      if (blk < 0 || blk >= num_blocks) {
        free(Kc); free(Vc); free(s); free(qv);
        return ORC_ERANGE;
      }
      for (g = 0; g < n_kv_heads; ++g) {
        int64_t src = (((int64_t)blk * n_kv_heads + g) * block_size + off) * head_dim;
        for (d = 0; d < head_dim; ++d) {
          Kc[((size_t)t * n_kv_heads + g) * head_dim + d] = widen(k_pool, src + d, dtype);
          Vc[((size_t)t * n_kv_heads + g) * head_dim + d] = widen(v_pool, src + d, dtype);
        }
      }
    }
    for (i = 0; i < query_len; ++i) {
      int64_t visible = n - query_len + i + 1;  /* positions 0 .. p */
      for (h = 0; h < n_heads; ++h) {
        int64_t row = ((int64_t)r * query_len + i) * n_heads + h;
        if (visible <= 0) {
          for (d = 0; d < head_dim; ++d) out[row * head_dim + d] = 0.0;
          continue;
        }
        for (d = 0; d < head_dim; ++d) qv[d] = widen(q, row * head_dim + d, dtype);
        attend_one(qv, Kc + (size_t)(h / group) * head_dim, Vc + (size_t)(h / group) * head_dim,
                   visible, (int64_t)n_kv_heads * head_dim, head_dim, scale, s,
                   out + row * head_dim);
      }
    }
  }
  free(Kc); free(Vc); free(s); free(qv);
  return ORC_OK;
}
