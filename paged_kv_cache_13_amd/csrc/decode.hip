// Paged decode read for gfx950: split-context partitions + merge.
//
// What is computed (nanoserve "Day 25: the fused read dispatches to the kernel
// backend", sections "What I added today" and "Why it matters"; "Day 60: the
// read becomes a choice ...", section "What I added today"): each row's single
// query attends over the K/V its block table points at, with an online
// softmax streamed over the history, so the [rows, heads, 1, ctx] score
// rectangle is never built.  Query head h reads kv head h / group ("Day 25"
// page, "Diagram": the result feeds grouped-query attention).
//
// Work decomposition: one workgroup per (partition, kv head, row).  A
// partition is `partition_tokens` consecutive positions of one row.  The GQA
// group of query heads that share the kv head is handled by the same
// workgroup, so every K/V byte is read from HBM once and feeds `group` dot
// products.  Each of the 4 waves walks passes of the partition; a pass is
// kNI coalesced 16-byte loads per lane of K and of V.  Rows that fit one
// partition write `out` directly; longer rows write (max, sum, acc) per
// partition to the workspace and the merge kernel combines them.
//
// Lane layout of a 16-byte load: the (block, kv head) tile is one contiguous
// run of block_size * head_dim elements; LPT = head_dim * elem / 16 lanes
// cover one position's row, so a wave-wide load reads 64 * 16 bytes of whole
// consecutive rows.  Dot products are reduced across those LPT lanes with DPP
// row permutes.  Scores are kept in the log2 domain (scale * log2 e folded in)
// so the exponentials are v_exp_f32.
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kWave = 64;
constexpr int kWaves = 4;
constexpr int kThreads = kWave * kWaves;
constexpr int kNI = 4;  // 16-byte loads per lane per pass, for K and for V
constexpr float kLog2e = 1.4426950408889634f;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Value of the lane whose index differs in bit log2(D).  Exact for D = 1, 2
// and D >= 16; for D = 4, 8 it uses the row mirrors, which pair the right
// lane groups only when x is uniform across aligned groups of D lanes.
template <int D>
__device__ __forceinline__ float xchg_uniform(float x) {
  if constexpr (D == 1) return dpp_f<0xB1>(x);        // quad_perm [1,0,3,2]
  else if constexpr (D == 2) return dpp_f<0x4E>(x);   // quad_perm [2,3,0,1]
  else if constexpr (D == 4) return dpp_f<0x141>(x);  // row_half_mirror
  else if constexpr (D == 8) return dpp_f<0x140>(x);  // row_mirror
  else return __shfl_xor(x, D);
}

template <int D>
__device__ __forceinline__ float xchg_exact(float x) {
  if constexpr (D == 1) return dpp_f<0xB1>(x);
  else if constexpr (D == 2) return dpp_f<0x4E>(x);
  else return __shfl_xor(x, D);
}

// Sum over lane bits [log2 LO, log2 HI), inputs uniform below LO.
template <int LO, int HI>
__device__ __forceinline__ float sum_uniform(float x) {
  if constexpr (LO < HI) {
    x += xchg_uniform<LO>(x);
    return sum_uniform<LO * 2, HI>(x);
  } else {
    return x;
  }
}

template <int LO, int HI>
__device__ __forceinline__ float max_uniform(float x) {
  if constexpr (LO < HI) {
    x = fmaxf(x, xchg_uniform<LO>(x));
    return max_uniform<LO * 2, HI>(x);
  } else {
    return x;
  }
}

template <int LO, int HI>
__device__ __forceinline__ float sum_exact(float x) {
  if constexpr (LO < HI) {
    x += xchg_exact<LO>(x);
    return sum_exact<LO * 2, HI>(x);
  } else {
    return x;
  }
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// fp32 -> bf16, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
  uint32_t b = __builtin_bit_cast(uint32_t, x);
  if ((b & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((b >> 16) | 0x40u);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

__device__ __forceinline__ void store_out(void *out, int out_dtype, size_t idx, float v) {
  if (out_dtype == kF32)
    static_cast<float *>(out)[idx] = v;
  else
    static_cast<uint16_t *>(out)[idx] = f32_to_bf16_rne(v);
}

template <typename T>
struct Elem;
template <>
struct Elem<float> {
  // lane-local dot product of one 16-byte chunk with the query chunk
  __device__ static float dot(const uint4 &k, const uint4 &q, float acc) {
    acc = fmaf(__builtin_bit_cast(float, k.x), __builtin_bit_cast(float, q.x), acc);
    acc = fmaf(__builtin_bit_cast(float, k.y), __builtin_bit_cast(float, q.y), acc);
    acc = fmaf(__builtin_bit_cast(float, k.z), __builtin_bit_cast(float, q.z), acc);
    acc = fmaf(__builtin_bit_cast(float, k.w), __builtin_bit_cast(float, q.w), acc);
    return acc;
  }
  __device__ static void widen(const uint4 &v, float *f) {
    f[0] = __builtin_bit_cast(float, v.x);
    f[1] = __builtin_bit_cast(float, v.y);
    f[2] = __builtin_bit_cast(float, v.z);
    f[3] = __builtin_bit_cast(float, v.w);
  }
};
template <>
struct Elem<uint16_t> {  // bfloat16 storage
  __device__ static float dot2(uint32_t k, uint32_t q, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, k),
                                           __builtin_bit_cast(bf16x2_t, q), acc, false);
  }
  __device__ static float dot(const uint4 &k, const uint4 &q, float acc) {
    acc = dot2(k.x, q.x, acc);
    acc = dot2(k.y, q.y, acc);
    acc = dot2(k.z, q.z, acc);
    acc = dot2(k.w, q.w, acc);
    return acc;
  }
  __device__ static void widen(const uint4 &v, float *f) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __builtin_bit_cast(float, w[i] << 16);
      f[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xFFFF0000u);
    }
  }
};

__device__ __forceinline__ uint4 load16(const void *base, size_t byte_off) {
  return *reinterpret_cast<const uint4 *>(static_cast<const char *>(base) + byte_off);
}

// 16 bytes of one position's V row from a dimension-major tile: consecutive
// elements are `stride` elements apart starting at element index `first`.
template <typename T>
__device__ __forceinline__ uint4 gather_v(const void *base, size_t first, int stride);
template <>
__device__ __forceinline__ uint4 gather_v<float>(const void *base, size_t first, int stride) {
  const uint32_t *p = static_cast<const uint32_t *>(base) + first;
  return make_uint4(p[0], p[stride], p[2 * stride], p[3 * stride]);
}
template <>
__device__ __forceinline__ uint4 gather_v<uint16_t>(const void *base, size_t first, int stride) {
  const uint16_t *p = static_cast<const uint16_t *>(base) + first;
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    w[i] = (uint32_t)p[(2 * i) * stride] | ((uint32_t)p[(2 * i + 1) * stride] << 16);
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// Work item of this workgroup.  The grid is 1-D and ordered kv head fastest,
// then row, then partition.  Workgroups are handed to the 8 XCDs round-robin
// by linear id, so this order gives every XCD the same mix of full, partial
// and empty partitions (with the partition index fastest, XCD k would get
// only partition k of every row), and the mostly empty high partitions come
// last in dispatch order.
struct WorkItem {
  int p, g, r;
};
__device__ __forceinline__ WorkItem work_item(const DecodeArgs &a) {
  const unsigned id = blockIdx.x;
  const unsigned rest = id / (unsigned)a.n_kv_heads;
  WorkItem w;
  w.g = (int)(id - rest * (unsigned)a.n_kv_heads);
  w.p = (int)(rest / (unsigned)a.rows);
  w.r = (int)(rest - (unsigned)w.p * (unsigned)a.rows);
  return w;
}

template <typename T, int HD, int GP>
__global__ __launch_bounds__(kThreads) void decode_partition(DecodeArgs a) {
  constexpr int ES = sizeof(T);
  constexpr int EPL = 16 / ES;         // elements per lane per load
  constexpr int LPT = HD / EPL;        // lanes per position row
  constexpr int TPI = kWave / LPT;     // positions per wave-wide load
  constexpr int TPASS = kNI * TPI;     // positions per wave pass
  static_assert(LPT >= 1 && LPT <= kWave && (kWave % LPT) == 0, "row must tile a wave");

  __shared__ float s_m[kWaves][GP];
  __shared__ float s_l[kWaves][GP];
  __shared__ float s_acc[kWaves][GP][HD];
  extern __shared__ int32_t s_blk[];

  const WorkItem it = work_item(a);
  const int p = it.p, g = it.g, r = it.r;
  const int tid = threadIdx.x;
  const int cap = a.max_blocks_per_row * a.block_size;
  int n = a.context_lens[r];
  n = n < 0 ? 0 : (n > cap ? cap : n);
  const int P = a.partition_tokens;
  const int start = p * P;
  const int group = a.group;
  if (start >= n) {
    if (p == 0) {  // empty row: zeros
      for (int idx = tid; idx < group * HD; idx += kThreads) {
        const int j = idx / HD, d = idx % HD;
        store_out(a.out, a.out_dtype, ((size_t)r * a.n_heads + g * group + j) * HD + d, 0.f);
      }
    }
    return;
  }
  const int end = min(n, start + P);
  const bool single = n <= P;

  // This partition's block ids, clamped into the pool.
  const int nblk = (end - start + a.block_size - 1) >> a.log2_bs;
  const int first_blk = start >> a.log2_bs;
  const int32_t *table_row = a.block_table + (size_t)r * a.max_blocks_per_row + first_blk;
  for (int i = tid; i < nblk; i += kThreads) {
    int64_t b = table_row[i];
    b = b < 0 ? 0 : (b >= a.num_blocks ? a.num_blocks - 1 : b);
    s_blk[i] = (int32_t)b;
  }

  const int lane = tid % kWave;
  const int wave = tid / kWave;
  const int ts = lane / LPT;  // position slot inside a wave-wide load
  const int c = lane % LPT;   // 16-byte chunk of the row this lane holds

  // Query chunks of the GQA group, as raw 16-byte words (heads >= group are 0).
  uint4 qv[GP];
#pragma unroll
  for (int j = 0; j < GP; ++j) {
    if (j < group)
      qv[j] = load16(a.q, (((size_t)r * a.n_heads + g * group + j) * HD + c * EPL) * ES);
    else
      qv[j] = make_uint4(0, 0, 0, 0);
  }
  __syncthreads();

  const float sl2 = a.scale * kLog2e;
  float m[GP], l[GP], acc[GP][EPL];
#pragma unroll
  for (int j = 0; j < GP; ++j) {
    m[j] = -INFINITY;
    l[j] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[j][e] = 0.f;
  }

  const size_t tile_stride = (size_t)a.n_kv_heads;  // blocks -> (block, head) tiles
  const int bmask = a.block_size - 1;
  for (int base = start + wave * TPASS; base < end; base += kWaves * TPASS) {
    uint4 kr[kNI], vr[kNI];
    bool valid[kNI];
#pragma unroll
    for (int i = 0; i < kNI; ++i) {
      const int t = base + i * TPI + ts;
      valid[i] = t < end;
      kr[i] = make_uint4(0, 0, 0, 0);
      vr[i] = make_uint4(0, 0, 0, 0);
      if (valid[i]) {
        const int32_t blk = s_blk[(t - start) >> a.log2_bs];
        const size_t tile = (size_t)blk * tile_stride + g;
        const size_t row = (tile << a.log2_bs) + (t & bmask);
        kr[i] = load16(a.k_pool, (row * HD + c * EPL) * ES);
        // V tile is dimension-major: element d of position o at [d][o]
        vr[i] = gather_v<T>(a.v_pool, ((tile * HD + c * EPL) << a.log2_bs) + (t & bmask),
                            a.block_size);
      }
    }
    // scores
    float s[kNI][GP];
#pragma unroll
    for (int i = 0; i < kNI; ++i)
#pragma unroll
      for (int j = 0; j < GP; ++j) {
        float x = Elem<T>::dot(kr[i], qv[j], 0.f);
        x = sum_uniform<1, LPT>(x) * sl2;
        s[i][j] = valid[i] ? x : -INFINITY;
      }
    // online softmax update, one running max per head shared by the wave
#pragma unroll
    for (int j = 0; j < GP; ++j) {
      float mx = s[0][j];
#pragma unroll
      for (int i = 1; i < kNI; ++i) mx = fmaxf(mx, s[i][j]);
      mx = max_uniform<LPT, kWave>(mx);
      const float m_new = fmaxf(m[j], mx);
      const float alpha = (m[j] == m_new) ? 1.f : exp2_fast(m[j] - m_new);
      m[j] = m_new;
      float psum = 0.f;
      float pv[kNI];
#pragma unroll
      for (int i = 0; i < kNI; ++i) {
        pv[i] = valid[i] ? exp2_fast(s[i][j] - m_new) : 0.f;
        psum += pv[i];
      }
      l[j] = l[j] * alpha + psum;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[j][e] *= alpha;
#pragma unroll
      for (int i = 0; i < kNI; ++i) {
        float vf[EPL];
        Elem<T>::widen(vr[i], vf);
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[j][e] = fmaf(pv[i], vf[e], acc[j][e]);
      }
    }
  }

  // Combine the position slots of this wave, then the waves of the workgroup.
#pragma unroll
  for (int j = 0; j < GP; ++j) {
    l[j] = sum_uniform<LPT, kWave>(l[j]);
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[j][e] = sum_exact<LPT, kWave>(acc[j][e]);
  }
  if (ts == 0) {
#pragma unroll
    for (int j = 0; j < GP; ++j)
#pragma unroll
      for (int e = 0; e < EPL; ++e) s_acc[wave][j][c * EPL + e] = acc[j][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int j = 0; j < GP; ++j) {
      s_m[wave][j] = m[j];
      s_l[wave][j] = l[j];
    }
  }
  __syncthreads();

  const WsLayout ws = single ? WsLayout{} : ws_layout(a.rows, a.n_heads, a.max_parts, HD);
  for (int idx = tid; idx < group * HD; idx += kThreads) {
    const int j = idx / HD, d = idx % HD;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_m[w][j]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = s_m[w][j];
      const float wt = (mw == -INFINITY) ? 0.f : exp2_fast(mw - M);
      L = fmaf(s_l[w][j], wt, L);
      O = fmaf(s_acc[w][j][d], wt, O);
    }
    const int h = g * group + j;
    if (single) {
      store_out(a.out, a.out_dtype, ((size_t)r * a.n_heads + h) * HD + d, O / L);
    } else {
      const size_t slot = ((size_t)r * a.n_heads + h) * a.max_parts + p;
      a.ws[ws.acc_off + slot * HD + d] = O;
      if (d == 0) {
        a.ws[ws.m_off + slot] = M;
        a.ws[ws.l_off + slot] = L;
      }
    }
  }
}

// Merge of the partitions of rows that span more than one:
//   M = max_p m_p;  L = sum_p l_p 2^(m_p - M);  out = sum_p acc_p 2^(m_p - M) / L
// (m_p in the log2 domain).  Rows with one partition were written directly.
__global__ __launch_bounds__(128) void decode_merge(DecodeArgs a) {
  const int r = blockIdx.x / a.n_heads;
  const int h = blockIdx.x % a.n_heads;
  const int cap = a.max_blocks_per_row * a.block_size;
  int n = a.context_lens[r];
  n = n < 0 ? 0 : (n > cap ? cap : n);
  const int P = a.partition_tokens;
  const int nparts = (n + P - 1) / P;
  if (nparts <= 1) return;
  const WsLayout ws = ws_layout(a.rows, a.n_heads, a.max_parts, a.head_dim);
  const size_t base = ((size_t)r * a.n_heads + h) * a.max_parts;
  const float *mp = a.ws + ws.m_off + base;
  const float *lp = a.ws + ws.l_off + base;
  const float *ap = a.ws + ws.acc_off + base * a.head_dim;
  float M = -INFINITY;
  for (int p = 0; p < nparts; ++p) M = fmaxf(M, mp[p]);
  float L = 0.f;
  for (int p = 0; p < nparts; ++p) L = fmaf(lp[p], exp2_fast(mp[p] - M), L);
  const float inv = 1.f / L;
  for (int d = threadIdx.x; d < a.head_dim; d += blockDim.x) {
    float O = 0.f;
    for (int p = 0; p < nparts; ++p) O = fmaf(ap[(size_t)p * a.head_dim + d], exp2_fast(mp[p] - M), O);
    store_out(a.out, a.out_dtype, ((size_t)r * a.n_heads + h) * a.head_dim + d, O * inv);
  }
}

// ---------------------------------------------------------------------------
// bf16 path on the matrix cores.
//
// A wave takes 32 consecutive positions of its partition per iteration.  The
// GQA group (padded to 16 heads) is the N side of both contractions:
//   scores  S[t][h]  = sum_d K[t][d] Q[h][d]      v_mfma_f32_16x16x32_bf16,
//                      A = K rows (position-major tile), B = Q, two 16-row
//                      tiles per 32 positions, head_dim / 32 k-steps each;
//   output  O[d][h] += sum_t V[d][t] P[h][t]      same instruction, A = V
//                      (dimension-major tile), B = P, head_dim / 16 d-tiles.
// Row m of score tile tt is position 8*(m/4) + 4*tt + m%4 of the 32, so the
// 4 accumulator rows a lane receives from the two tiles are 8 consecutive
// positions 8*(lane/16) .. +7 for head lane%16 -- exactly the 8 k-values that
// lane must supply as the B operand of the P.V product.  Scores, softmax
// state and output rows of head h therefore all live in the lanes with
// lane%16 == h, and nothing crosses lanes except the max over positions.
// P is fed to the bf16 product as a hi + lo pair of bf16 values (16
// significant bits), so the weights carry fp32-grade precision into the
// fp32 accumulators.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// All-reduce over the four 16-lane rows (lane bits 4 and 5).  Written with
// ds_bpermute exchanges: this compiler folds the two results of a
// v_permlane{16,32}_swap whose operands are the same value into one, which
// breaks a swap-based all-reduce.
__device__ __forceinline__ float max_across_rows(float x) {
  x = fmaxf(x, __shfl_xor(x, 32));
  return fmaxf(x, __shfl_xor(x, 16));
}

__device__ __forceinline__ float sum_across_rows(float x) {
  x += __shfl_xor(x, 32);
  return x + __shfl_xor(x, 16);
}

__device__ __forceinline__ uint32_t bf16_bits_rne(float x) {  // finite x only
  const uint32_t b = __builtin_bit_cast(uint32_t, x);
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ bf16x8_t ld_bf16x8(const void *base, size_t byte_off) {
  return __builtin_bit_cast(bf16x8_t, load16(base, byte_off));
}

__device__ __forceinline__ bf16x8_t zero_bf16x8() { return __builtin_bit_cast(bf16x8_t, make_uint4(0, 0, 0, 0)); }

// Keep the first `nv` (0..8) of 8 packed bf16 values, zero the rest (NaN-safe).
__device__ __forceinline__ bf16x8_t keep_first(bf16x8_t v, int nv) {
  uint4 w = __builtin_bit_cast(uint4, v);
  uint32_t x[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = (2 * i < nv) ? 0x0000FFFFu : 0u;
    const uint32_t hi = (2 * i + 1 < nv) ? 0xFFFF0000u : 0u;
    x[i] &= (lo | hi);
  }
  return __builtin_bit_cast(bf16x8_t, make_uint4(x[0], x[1], x[2], x[3]));
}

template <int HD>
struct MfmaTiles {
  bf16x8_t k[2][HD / 32];  // score tiles x k-steps
  bf16x8_t v[HD / 16];     // output d-tiles
};

// Issue the loads of one 32-position group.  Branch-free: positions at or
// past `end` load from the partition's first position instead (always
// mapped), and are masked where they are used, so the loads of the next group
// can be in flight while this one is computed.
template <int HD, int BS>
__device__ __forceinline__ void mfma_load(MfmaTiles<HD> &T, const DecodeArgs &a, const int32_t *s_blk,
                                          int g, int start, int end, int gbase, int lr, int lg) {
  constexpr int KS = HD / 32, DT = HD / 16;
  constexpr int LOG2_BS = BS == 8 ? 3 : (BS == 16 ? 4 : 5);
  constexpr int bmask = BS - 1;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    int t = gbase + 8 * (lr >> 2) + 4 * tt + (lr & 3);
    t = t < end ? t : start;
    const int32_t blk = s_blk[(t - start) >> LOG2_BS];
    const size_t row = (((size_t)blk * a.n_kv_heads + g) << LOG2_BS) + (t & bmask);
    const char *kp = static_cast<const char *>(a.k_pool) + (row * HD + lg * 8) * 2;
#pragma unroll
    for (int i = 0; i < KS; ++i) T.k[tt][i] = ld_bf16x8(kp, i * 64);
  }
  int t0 = gbase + 8 * lg;
  t0 = t0 < end ? t0 : start;
  const int32_t blk = s_blk[(t0 - start) >> LOG2_BS];
  const size_t base = ((((size_t)blk * a.n_kv_heads + g) * HD + lr) << LOG2_BS) + (t0 & bmask);
  const char *vp = static_cast<const char *>(a.v_pool) + base * 2;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) T.v[dt] = ld_bf16x8(vp, dt * 16 * BS * 2);
}

// Online-softmax step over one loaded group (see the block comment above).
template <int HD>
__device__ __forceinline__ void mfma_compute(MfmaTiles<HD> &T, const bf16x8_t *qb, f32x4_t *acc, float &m,
                                             float &l, float c, int end, int gbase, int lg) {
  constexpr int KS = HD / 32, DT = HD / 16;
  f32x4_t sacc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int i = 0; i < KS; ++i)
      sacc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(T.k[tt][i], qb[i], sacc[tt], 0, 0, 0);

  // this lane: head lane%16, positions gbase + 8*lg + e with e = 4*tt + j
  const int tl = gbase + 8 * lg;
  float s[8];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int j = 0; j < 4; ++j) s[4 * tt + j] = (tl + 4 * tt + j < end) ? sacc[tt][j] * c : -INFINITY;
  float mx = fmaxf(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])), fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7])));
  mx = max_across_rows(mx);
  const float m_new = fmaxf(m, mx);
  const float alpha = (m == m_new) ? 1.f : exp2_fast(m - m_new);
  m = m_new;
  float pv[8], psum = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    pv[e] = exp2_fast(s[e] - m_new);
    psum += pv[e];
  }
  l = l * alpha + psum;
  if (__any(alpha != 1.f)) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[dt] *= alpha;
  }
  uint32_t hw[4], lw[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t h0 = bf16_bits_rne(pv[2 * i]), h1 = bf16_bits_rne(pv[2 * i + 1]);
    const float r0 = pv[2 * i] - __builtin_bit_cast(float, h0 << 16);
    const float r1 = pv[2 * i + 1] - __builtin_bit_cast(float, h1 << 16);
    hw[i] = h0 | (h1 << 16);
    lw[i] = bf16_bits_rne(r0) | (bf16_bits_rne(r1) << 16);
  }
  const bf16x8_t phi = __builtin_bit_cast(bf16x8_t, make_uint4(hw[0], hw[1], hw[2], hw[3]));
  const bf16x8_t plo = __builtin_bit_cast(bf16x8_t, make_uint4(lw[0], lw[1], lw[2], lw[3]));
  // The last group of a partition may hold positions past `end` (stale or
  // NaN pool slots): their weights are 0, but 0 * NaN is NaN, so the V values
  // themselves are zeroed.  Wave-uniform branch, taken once per partition.
  if (gbase + 32 > end) {
    int nv = end - tl;
    nv = nv < 0 ? 0 : (nv > 8 ? 8 : nv);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) T.v[dt] = keep_first(T.v[dt], nv);
  }
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(T.v[dt], phi, acc[dt], 0, 0, 0);
    acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(T.v[dt], plo, acc[dt], 0, 0, 0);
  }
}

template <int HD, int BS>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void decode_partition_mfma(DecodeArgs a) {
  constexpr int KS = HD / 32, DT = HD / 16, GT = 32;
  __shared__ float s_m[kWaves][16];
  __shared__ float s_l[kWaves][16];
  __shared__ float s_acc[kWaves][16][HD];
  extern __shared__ int32_t s_blk[];

  const WorkItem it = work_item(a);
  const int p = it.p, g = it.g, r = it.r;
  const int tid = threadIdx.x;
  const int cap = a.max_blocks_per_row * a.block_size;
  int n = a.context_lens[r];
  n = n < 0 ? 0 : (n > cap ? cap : n);
  const int P = a.partition_tokens;
  const int start = p * P;
  const int group = a.group;
  if (start >= n) {
    if (p == 0) {
      for (int idx = tid; idx < group * HD; idx += kThreads) {
        const int j = idx / HD, d = idx % HD;
        store_out(a.out, a.out_dtype, ((size_t)r * a.n_heads + g * group + j) * HD + d, 0.f);
      }
    }
    return;
  }
  const int end = min(n, start + P);
  const bool single = n <= P;
  const int nblk = (end - start + a.block_size - 1) >> a.log2_bs;
  const int32_t *table_row = a.block_table + (size_t)r * a.max_blocks_per_row + (start >> a.log2_bs);
  for (int i = tid; i < nblk; i += kThreads) {
    int64_t b = table_row[i];
    b = b < 0 ? 0 : (b >= a.num_blocks ? a.num_blocks - 1 : b);
    s_blk[i] = (int32_t)b;
  }

  const int lane = tid % kWave;
  const int wave = tid / kWave;
  const int lr = lane & 15;  // head of the group (N index)
  const int lg = lane >> 4;  // k-slot group

  bf16x8_t qb[KS];
#pragma unroll
  for (int i = 0; i < KS; ++i)
    qb[i] = lr < group
                ? ld_bf16x8(a.q, (((size_t)r * a.n_heads + g * group + lr) * HD + (4 * i + lg) * 8) * 2)
                : zero_bf16x8();
  __syncthreads();

  const float c = a.scale * kLog2e;
  float m = -INFINITY, l = 0.f;
  f32x4_t acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Two tile sets, alternating: while one group is computed the next one's
  // loads are in flight.  Uniform control flow only.
  constexpr int kStep = kWaves * GT;
  MfmaTiles<HD> A, B;
  int gb = start + wave * GT;
  if (gb < end) {
    mfma_load<HD, BS>(A, a, s_blk, g, start, end, gb, lr, lg);
    while (true) {
      if (gb + kStep >= end) {
        mfma_compute<HD>(A, qb, acc, m, l, c, end, gb, lg);
        break;
      }
      mfma_load<HD, BS>(B, a, s_blk, g, start, end, gb + kStep, lr, lg);
      mfma_compute<HD>(A, qb, acc, m, l, c, end, gb, lg);
      gb += kStep;
      if (gb + kStep >= end) {
        mfma_compute<HD>(B, qb, acc, m, l, c, end, gb, lg);
        break;
      }
      mfma_load<HD, BS>(A, a, s_blk, g, start, end, gb + kStep, lr, lg);
      mfma_compute<HD>(B, qb, acc, m, l, c, end, gb, lg);
      gb += kStep;
    }
  }

  // per-wave state -> LDS; lanes of head lr hold output dims 16*dt + 4*lg + j
  l = sum_across_rows(l);
  if (lr < group) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j) s_acc[wave][lr][16 * dt + 4 * lg + j] = acc[dt][j];
    if (lg == 0) {
      s_m[wave][lr] = m;
      s_l[wave][lr] = l;
    }
  }
  __syncthreads();

  const WsLayout ws = single ? WsLayout{} : ws_layout(a.rows, a.n_heads, a.max_parts, HD);
  for (int idx = tid; idx < group * HD; idx += kThreads) {
    const int j = idx / HD, d = idx % HD;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_m[w][j]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = s_m[w][j];
      const float wt = (mw == -INFINITY) ? 0.f : exp2_fast(mw - M);
      L = fmaf(s_l[w][j], wt, L);
      O = fmaf(s_acc[w][j][d], wt, O);
    }
    const int h = g * group + j;
    if (single) {
      store_out(a.out, a.out_dtype, ((size_t)r * a.n_heads + h) * HD + d, O / L);
    } else {
      const size_t slot = ((size_t)r * a.n_heads + h) * a.max_parts + p;
      a.ws[ws.acc_off + slot * HD + d] = O;
      if (d == 0) {
        a.ws[ws.m_off + slot] = M;
        a.ws[ws.l_off + slot] = L;
      }
    }
  }
}

template <int HD, int BS>
hipError_t launch_mfma(const DecodeArgs &a, hipStream_t stream) {
  const dim3 grid((unsigned)a.max_parts * a.n_kv_heads * a.rows);
  const size_t lds = (size_t)(a.partition_tokens >> a.log2_bs) * sizeof(int32_t);
  hipLaunchKernelGGL((decode_partition_mfma<HD, BS>), grid, dim3(kThreads), lds, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.max_parts <= 1) return e;
  hipLaunchKernelGGL(decode_merge, dim3((unsigned)a.rows * a.n_heads), dim3(128), 0, stream, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Balanced stream decomposition of the bf16 read.
//
// The unit of work is a group of 32 consecutive positions of one (kv head,
// row).  All groups, ordered by kv head, then row, then position, form one
// stream; a tiny plan kernel prefix-sums the groups per row on the device
// (no host sync) and cuts the stream into kStreamWaves equal contiguous
// slices.  Each persistent wave walks its slice with the next group's K/V
// and the group after next's block ids in flight, across row boundaries, so
// no wave waits on a partition start-up and every wave does the same work
// whatever the length mix.  A (kv head, row) covered by one wave is written
// to `out` directly; one cut into several slices gets one partial (max, sum,
// rescaled acc) per slice, and the wave that writes the last partial (a
// per-row counter, zeroed by the plan kernel on every call) merges them.
// ---------------------------------------------------------------------------
// Slice w of a stream of `total` groups cut into `waves` slices.
__device__ __forceinline__ long long slice_start(long long w, long long total, long long waves) {
  return w * total / waves;
}
// The slice holding group `pos`: the largest w with slice_start(w) <= pos.
__device__ __forceinline__ long long slice_of(long long pos, long long total, long long waves) {
  return ((pos + 1) * waves - 1) / total;
}

__global__ __launch_bounds__(1024) void decode_plan(DecodeArgs a) {
  __shared__ int32_t s_gpre[kPlanMaxRows + 1];
  __shared__ int32_t s_sum[1024];
  const int tid = threadIdx.x;
  const int rows = a.rows;
  const int cap = a.max_blocks_per_row * a.block_size;
  const StreamLayout L = stream_layout(rows, a.n_kv_heads, a.group, a.head_dim, a.max_parts);
  int32_t *wsi = reinterpret_cast<int32_t *>(a.ws);
  const int per = (rows + 1023) / 1024;
  const int r0 = min(rows, tid * per), r1 = min(rows, r0 + per);
  int local = 0;
  for (int r = r0; r < r1; ++r) {
    int n = a.context_lens[r];
    n = n < 0 ? 0 : (n > cap ? cap : n);
    s_gpre[r] = local;
    local += (n + kGroupPositions - 1) / kGroupPositions;
    if (n == 0) {  // an empty row reads zeros; no wave visits it
      for (int idx = 0; idx < a.n_heads * a.head_dim; ++idx)
        store_out(a.out, a.out_dtype, (size_t)r * a.n_heads * a.head_dim + idx, 0.f);
    }
  }
  s_sum[tid] = local;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {  // inclusive scan of the per-thread sums
    const int v = tid >= off ? s_sum[tid - off] : 0;
    __syncthreads();
    s_sum[tid] += v;
    __syncthreads();
  }
  const int base = tid ? s_sum[tid - 1] : 0;
  for (int r = r0; r < r1; ++r) s_gpre[r] += base;
  const int ngk = s_sum[1023];
  if (tid == 0) s_gpre[rows] = ngk;
  __syncthreads();
  // Waves used: every one gets at least cg_min groups.  Wave w's slice is
  // [floor(w * ng_all / waves), floor((w + 1) * ng_all / waves)), so slices
  // differ by at most one group.
  const long long ng_all = (long long)a.n_kv_heads * ngk;
  long long waves = ng_all / max(a.cg_min, 1);
  waves = waves < 1 ? 1 : (waves > kStreamWaves ? kStreamWaves : waves);
  if (ng_all == 0) waves = 0;
  if (tid == 0) {
    wsi[L.hdr] = ngk;
    wsi[L.hdr + 1] = (int)waves;
    wsi[L.hdr + 2] = 0;
    wsi[L.hdr + 3] = 0;
  }
  for (int r = tid; r <= rows; r += 1024) wsi[L.gpre + r] = s_gpre[r];
  const int pairs = a.n_kv_heads * rows;
  for (int qi = tid; qi < pairs; qi += 1024) {
    const int kvh = qi / rows, r = qi - kvh * rows;
    const int ng = s_gpre[r + 1] - s_gpre[r];
    if (ng == 0) continue;
    const long long S = (long long)kvh * ngk + s_gpre[r], E = S + ng;
    for (long long w = slice_of(S, ng_all, waves); w < waves; ++w) {  // waves whose slice starts here
      const long long st = slice_start(w, ng_all, waves);
      if (st >= E) break;
      if (st < S) continue;
      wsi[L.first_pos + 2 * w] = qi;
      wsi[L.first_pos + 2 * w + 1] = (int)(st - S);
    }
  }
}

// Position of one group of a (kv head, row) stream, plus what its segment
// end needs.  Wave-uniform.
struct Cursor {
  int kvh, r, j, n, ng, part, nparts, idx;
};

// Lengths and group prefixes of kWindowRows consecutive rows, staged in LDS
// so that moving a cursor to another row costs LDS reads only (lgkmcnt),
// never a global load the in-flight K/V loads would have to drain behind.
struct RowWindow {
  int r0;
  int32_t *ctx, *gpre;  // LDS, kWindowRows each
};

__device__ __forceinline__ void window_cover(RowWindow &win, const DecodeArgs &a, const int32_t *wsi,
                                             const StreamLayout &L, int r, int lane, int cap) {
  if (r < win.r0 || r >= win.r0 + kWindowRows) {  // rare: a wave crossing many rows
    win.r0 = r;
    for (int i = lane; i < kWindowRows; i += kWave) {
      const int rr = r + i;
      int n = rr < a.rows ? a.context_lens[rr] : 0;
      win.ctx[i] = n < 0 ? 0 : (n > cap ? cap : n);
      win.gpre[i] = rr <= a.rows ? wsi[L.gpre + rr] : 0;
    }
    __syncthreads();  // one wave per workgroup: orders the LDS writes before the reads
  }
}

// Fill the row fields of a cursor whose kv head, row and group are set.
// Slice numbers follow slice_of, so part/nparts name this piece of the row.
__device__ __forceinline__ void cursor_row(Cursor &c, RowWindow &win, int w, int ngk, long long ng_all,
                                           long long waves) {
  c.n = win.ctx[c.r - win.r0];
  c.ng = (c.n + kGroupPositions - 1) / kGroupPositions;
  const long long S = (long long)c.kvh * ngk + win.gpre[c.r - win.r0];
  const int first = (int)slice_of(S, ng_all, waves), last = (int)slice_of(S + c.ng - 1, ng_all, waves);
  c.part = w - first;
  c.nparts = last - first + 1;
}

// Next group of this wave's slice (only called while one remains).
__device__ __forceinline__ void cursor_next(Cursor &c, RowWindow &win, const DecodeArgs &a, const int32_t *wsi,
                                            const StreamLayout &L, int w, int ngk, long long ng_all,
                                            long long waves, int lane, int cap) {
  ++c.idx;
  if (c.j + 1 < c.ng) {
    ++c.j;
    return;
  }
  do {  // next row with positions (empty rows hold no group)
    if (++c.r == a.rows) {
      c.r = 0;
      ++c.kvh;
    }
    window_cover(win, a, wsi, L, c.r, lane, cap);
  } while (win.ctx[c.r - win.r0] == 0);
  c.j = 0;
  cursor_row(c, win, w, ngk, ng_all, waves);
}

// Inclusive prefix sum over the 64 lanes.
__device__ __forceinline__ int wave_inclusive_scan(int x, int lane) {
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  return x;
}

// In-kernel plan for batches of at most kWindowRows rows: every wave scans
// the (clamped) lengths itself -- lane l owns rows 4l..4l+3 -- into its LDS
// window, so no plan kernel runs and no plan is read back from memory.
// Returns the groups per kv head.
__device__ __forceinline__ int plan_in_wave(RowWindow &win, const DecodeArgs &a, int lane, int cap) {
  int ng[4], n[4], sum = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * lane + i;
    int x = r < a.rows ? a.context_lens[r] : 0;
    x = x < 0 ? 0 : (x > cap ? cap : x);
    n[i] = x;
    ng[i] = (x + kGroupPositions - 1) / kGroupPositions;
    sum += ng[i];
  }
  const int incl = wave_inclusive_scan(sum, lane);
  int run = incl - sum;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    win.ctx[4 * lane + i] = n[i];
    win.gpre[4 * lane + i] = run;
    run += ng[i];
  }
  win.r0 = 0;
  __syncthreads();  // one wave per workgroup: orders the LDS writes before the reads
  return __shfl(incl, kWave - 1);
}

// Row (and group in it) holding group `rem` of a kv head's stream, from the
// in-wave plan: lane l checks its rows 4l..4l+3.
__device__ __forceinline__ void plan_locate(const RowWindow &win, int rem, int lane, int &r, int &j) {
  int found = -1;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rr = 4 * lane + i;
    const int g0 = win.gpre[rr];
    const int ng = (win.ctx[rr] + kGroupPositions - 1) / kGroupPositions;
    if (ng > 0 && g0 <= rem && rem < g0 + ng) found = rr;
  }
  const unsigned long long hit = __ballot(found >= 0);
  const int src = (int)__builtin_ctzll(hit);
  r = __shfl(found, src);
  j = rem - win.gpre[r];
}

struct GroupIds {
  int32_t k0, k1, v;  // this lane's block ids: score tiles 0/1 rows, V chunk
};

template <int BS>
__device__ __forceinline__ GroupIds load_ids(const DecodeArgs &a, const Cursor &c, int lr, int lg) {
  constexpr int LOG2_BS = BS == 8 ? 3 : (BS == 16 ? 4 : 5);
  const int t0 = c.j * kGroupPositions, last = c.n - 1;
  const int tk0 = min(t0 + 8 * (lr >> 2) + (lr & 3), last);
  const int tk1 = min(t0 + 8 * (lr >> 2) + 4 + (lr & 3), last);
  const int tv = min(t0 + 8 * lg, last);
  const int32_t *row = a.block_table + (size_t)c.r * a.max_blocks_per_row;
  GroupIds ids;
  ids.k0 = row[tk0 >> LOG2_BS];
  ids.k1 = row[tk1 >> LOG2_BS];
  ids.v = row[tv >> LOG2_BS];
  return ids;
}

template <int HD, int BS>
__device__ __forceinline__ void load_group_k(bf16x8_t (&k)[2][HD / 32], const DecodeArgs &a, const Cursor &c,
                                             const GroupIds &ids, int lr, int lg) {
  constexpr int KS = HD / 32;
  constexpr int LOG2_BS = BS == 8 ? 3 : (BS == 16 ? 4 : 5);
  constexpr int bmask = BS - 1;
  const int t0 = c.j * kGroupPositions, last = c.n - 1;
  const int64_t nb1 = a.num_blocks - 1;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const int t = min(t0 + 8 * (lr >> 2) + 4 * tt + (lr & 3), last);
    int64_t blk = tt == 0 ? ids.k0 : ids.k1;
    blk = blk < 0 ? 0 : (blk > nb1 ? nb1 : blk);
    const size_t row = (((size_t)blk * a.n_kv_heads + c.kvh) << LOG2_BS) + (t & bmask);
    const char *kp = static_cast<const char *>(a.k_pool) + (row * HD + lg * 8) * 2;
#pragma unroll
    for (int i = 0; i < KS; ++i) k[tt][i] = ld_bf16x8(kp, i * 64);
  }
}

template <int HD, int BS>
__device__ __forceinline__ void load_group_v(bf16x8_t (&v)[HD / 16], const DecodeArgs &a, const Cursor &c,
                                             const GroupIds &ids, int lr, int lg) {
  constexpr int DT = HD / 16;
  constexpr int LOG2_BS = BS == 8 ? 3 : (BS == 16 ? 4 : 5);
  constexpr int bmask = BS - 1;
  const int t0 = c.j * kGroupPositions, last = c.n - 1;
  const int64_t nb1 = a.num_blocks - 1;
  const int tv = min(t0 + 8 * lg, last) & ~7;
  int64_t blk = ids.v;
  blk = blk < 0 ? 0 : (blk > nb1 ? nb1 : blk);
  const size_t base = ((((size_t)blk * a.n_kv_heads + c.kvh) * HD + lr) << LOG2_BS) + (tv & bmask);
  const char *vp = static_cast<const char *>(a.v_pool) + base * 2;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) v[dt] = ld_bf16x8(vp, dt * 16 * BS * 2);
}

// Scores of one group: two 16x16 tiles (see the P.V layout note above).
template <int HD>
__device__ __forceinline__ void group_scores(const bf16x8_t (&k)[2][HD / 32], const bf16x8_t *qb,
                                             f32x4_t (&sacc)[2]) {
  constexpr int KS = HD / 32;
  sacc[0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  sacc[1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int i = 0; i < KS; ++i) sacc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k[tt][i], qb[i], sacc[tt], 0, 0, 0);
}

// Online-softmax update and P.V of one group from its scores.
template <int HD>
__device__ __forceinline__ void group_softmax_pv(const f32x4_t (&sacc)[2], bf16x8_t (&v)[HD / 16], f32x4_t *acc,
                                                 float &m, float &l, float c, int end, int gbase, int lg) {
  constexpr int DT = HD / 16;
  const int tl = gbase + 8 * lg;
  float s[8];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int j = 0; j < 4; ++j) s[4 * tt + j] = (tl + 4 * tt + j < end) ? sacc[tt][j] * c : -INFINITY;
  float mx = fmaxf(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])), fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7])));
  mx = max_across_rows(mx);
  const float m_new = fmaxf(m, mx);
  const float alpha = (m == m_new) ? 1.f : exp2_fast(m - m_new);
  m = m_new;
  float pv[8], psum = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    pv[e] = exp2_fast(s[e] - m_new);
    psum += pv[e];
  }
  l = l * alpha + psum;
  if (__any(alpha != 1.f)) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[dt] *= alpha;
  }
  uint32_t hw[4], lw[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t h0 = bf16_bits_rne(pv[2 * i]), h1 = bf16_bits_rne(pv[2 * i + 1]);
    const float r0 = pv[2 * i] - __builtin_bit_cast(float, h0 << 16);
    const float r1 = pv[2 * i + 1] - __builtin_bit_cast(float, h1 << 16);
    hw[i] = h0 | (h1 << 16);
    lw[i] = bf16_bits_rne(r0) | (bf16_bits_rne(r1) << 16);
  }
  const bf16x8_t phi = __builtin_bit_cast(bf16x8_t, make_uint4(hw[0], hw[1], hw[2], hw[3]));
  const bf16x8_t plo = __builtin_bit_cast(bf16x8_t, make_uint4(lw[0], lw[1], lw[2], lw[3]));
  if (gbase + 32 > end) {  // positions past the row end: zero their (possibly NaN) V
    int nv = end - tl;
    nv = nv < 0 ? 0 : (nv > 8 ? 8 : nv);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) v[dt] = keep_first(v[dt], nv);
  }
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v[dt], phi, acc[dt], 0, 0, 0);
    acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v[dt], plo, acc[dt], 0, 0, 0);
  }
}

template <int HD>
__device__ __forceinline__ void write_out_rows(const DecodeArgs &a, const Cursor &c, const f32x4_t *o,
                                               float inv, int lr, int lg) {
  constexpr int DT = HD / 16;
  const size_t base = ((size_t)c.r * a.n_heads + c.kvh * a.group + lr) * HD + 4 * lg;
  if (a.out_dtype == kF32) {
    float *out = static_cast<float *>(a.out) + base;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      *reinterpret_cast<f32x4_t *>(out + 16 * dt) = o[dt] * inv;
  } else {
    uint16_t *out = static_cast<uint16_t *>(a.out) + base;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const uint32_t w0 = f32_to_bf16_rne(o[dt][0] * inv) | ((uint32_t)f32_to_bf16_rne(o[dt][1] * inv) << 16);
      const uint32_t w1 = f32_to_bf16_rne(o[dt][2] * inv) | ((uint32_t)f32_to_bf16_rne(o[dt][3] * inv) << 16);
      *reinterpret_cast<uint2 *>(out + 16 * dt) = make_uint2(w0, w1);
    }
  }
}

// End of one (kv head, row) slice: write the output, or, for a row cut
// into several slices, this slice's partial (max, sum, rescaled acc) for
// decode_stream_merge.  Plain stores: the merge runs as the next kernel.
template <int HD>
__device__ __forceinline__ void segment_end(const DecodeArgs &a, const StreamLayout &L, const Cursor &c,
                                            f32x4_t *acc, float &m, float &l, int lr, int lg) {
  constexpr int DT = HD / 16;
  const int G = a.group;
  const float lt = sum_across_rows(l);
  if (c.nparts == 1) {
    if (lr < G) write_out_rows<HD>(a, c, acc, 1.f / lt, lr, lg);
  } else if (lr < G) {
    const size_t pair = (size_t)c.kvh * a.rows + c.r;
    float *slot = a.ws + L.partials + (pair * a.max_parts + c.part) * L.slot_stride;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) *reinterpret_cast<f32x4_t *>(slot + lr * HD + 16 * dt + 4 * lg) = acc[dt];
    if (lg == 0) {
      slot[G * HD + lr] = m;
      slot[G * HD + G + lr] = lt;
    }
  }
  m = -INFINITY;
  l = 0.f;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
}

// Combine the partials of every (kv head, row) the stream cut into several
// slices: M = max_k m_k;  L = sum_k l_k 2^(m_k - M);
// out = sum_k acc_k 2^(m_k - M) / L.  One workgroup per (kv head, row);
// rows in one slice were written by the stream kernel already.  The maxima
// are read first (one independent load each), then the weighted sums.
constexpr int kMergeMaxParts = 8;
__global__ __launch_bounds__(256) void decode_stream_merge(DecodeArgs a) {
  const StreamLayout L = stream_layout(a.rows, a.n_kv_heads, a.group, a.head_dim, a.max_parts);
  const int32_t *wsi = reinterpret_cast<const int32_t *>(a.ws);
  const int pair = blockIdx.x;
  const int kvh = pair / a.rows, r = pair - kvh * a.rows;
  int ngk, g0, ng;
  long long waves;
  if (a.inplan) {
    // groups per kv head and before row r, by a block reduction over the
    // (at most 256) clamped lengths
    __shared__ int s_red[2][256 / kWave];
    const int cap = a.max_blocks_per_row * a.block_size;
    const int t = threadIdx.x;
    int x = t < a.rows ? a.context_lens[t] : 0;
    x = x < 0 ? 0 : (x > cap ? cap : x);
    const int gx = (x + kGroupPositions - 1) / kGroupPositions;
    int tot = gx, pre = t < r ? gx : 0;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      tot += __shfl_xor(tot, d);
      pre += __shfl_xor(pre, d);
    }
    if ((t & (kWave - 1)) == 0) {
      s_red[0][t / kWave] = tot;
      s_red[1][t / kWave] = pre;
    }
    __syncthreads();
    ngk = s_red[0][0] + s_red[0][1] + s_red[0][2] + s_red[0][3];
    g0 = s_red[1][0] + s_red[1][1] + s_red[1][2] + s_red[1][3];
    int xr = a.context_lens[r];
    xr = xr < 0 ? 0 : (xr > cap ? cap : xr);
    ng = (xr + kGroupPositions - 1) / kGroupPositions;
    const long long all = (long long)a.n_kv_heads * ngk;
    waves = all / max(a.cg_min, 1);
    waves = waves < 1 ? 1 : (waves > kStreamWaves ? kStreamWaves : waves);
  } else {
    ngk = wsi[L.hdr];
    waves = wsi[L.hdr + 1];
    g0 = wsi[L.gpre + r];
    ng = wsi[L.gpre + r + 1] - g0;
  }
  if (ng == 0) return;
  const long long ng_all = (long long)a.n_kv_heads * ngk;
  const long long S = (long long)kvh * ngk + g0;
  const int nparts = (int)(slice_of(S + ng - 1, ng_all, waves) - slice_of(S, ng_all, waves) + 1);
  if (nparts <= 1) return;
  const int G = a.group, HD = a.head_dim;
  const float *slots = a.ws + L.partials + (size_t)pair * a.max_parts * L.slot_stride;
  for (int idx = threadIdx.x; idx < G * HD; idx += blockDim.x) {
    const int j = idx / HD, d = idx - j * HD;
    float M = -INFINITY, Lm = 0.f, O = 0.f;
    for (int k0 = 0; k0 < nparts; k0 += kMergeMaxParts) {
      const int kn = min(nparts - k0, kMergeMaxParts);
      float mk[kMergeMaxParts], lk[kMergeMaxParts], ak[kMergeMaxParts];
#pragma unroll
      for (int k = 0; k < kMergeMaxParts; ++k) {
        if (k < kn) {
          const float *sk = slots + (size_t)(k0 + k) * L.slot_stride;
          mk[k] = sk[G * HD + j];
          lk[k] = sk[G * HD + G + j];
          ak[k] = sk[j * HD + d];
        }
      }
      float mn = M;
#pragma unroll
      for (int k = 0; k < kMergeMaxParts; ++k)
        if (k < kn) mn = fmaxf(mn, mk[k]);
      const float a0 = M == -INFINITY ? 0.f : exp2_fast(M - mn);
      Lm *= a0;
      O *= a0;
#pragma unroll
      for (int k = 0; k < kMergeMaxParts; ++k) {
        if (k < kn) {
          const float wk = exp2_fast(mk[k] - mn);
          Lm = fmaf(lk[k], wk, Lm);
          O = fmaf(ak[k], wk, O);
        }
      }
      M = mn;
    }
    store_out(a.out, a.out_dtype, ((size_t)r * a.n_heads + kvh * G + j) * HD + d, O / Lm);
  }
}

// Stage one group's K and V into this wave's LDS buffer with direct-to-LDS
// loads (no VGPRs): each 16-byte-per-lane load lands as one contiguous 1 KiB
// row of the buffer, lane l at offset 16*l -- the layout the matrix-core
// operands are read back in.
// Cache policy of the K/V loads: non-temporal.  Every K/V byte is read once
// per call, so keeping it in L2 / the Infinity Cache only evicts lines that
// are reused (block ids, q, partials); the streaming hint lifts the
// sustained read rate of 4 KiB tile gathers by about 14% on MI355X.
constexpr int kStreamingLoad = 2;  // the nt bit of the cache-policy operand

template <int HD, int BS>
__device__ __forceinline__ void stage_group(uint4 *s_k, uint4 *s_v, const DecodeArgs &a, const Cursor &c,
                                            const GroupIds &ids, int lane, int lr, int lg) {
  constexpr int KS = HD / 32, DT = HD / 16;
  constexpr int LOG2_BS = BS == 8 ? 3 : (BS == 16 ? 4 : 5);
  constexpr int bmask = BS - 1;
  const int t0 = c.j * kGroupPositions, last = c.n - 1;
  const int64_t nb1 = a.num_blocks - 1;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const int t = min(t0 + 8 * (lr >> 2) + 4 * tt + (lr & 3), last);
    int64_t blk = tt == 0 ? ids.k0 : ids.k1;
    blk = blk < 0 ? 0 : (blk > nb1 ? nb1 : blk);
    const size_t row = (((size_t)blk * a.n_kv_heads + c.kvh) << LOG2_BS) + (t & bmask);
    const char *kp = static_cast<const char *>(a.k_pool) + (row * HD + lg * 8) * 2;
#pragma unroll
    for (int i = 0; i < KS; ++i)
      __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1))) *)(kp + i * 64),
                                       (void __attribute__((address_space(3))) *)(s_k + (tt * KS + i) * kWave),
                                       16, 0, kStreamingLoad);
  }
  const int tv = min(t0 + 8 * lg, last) & ~7;
  int64_t blk = ids.v;
  blk = blk < 0 ? 0 : (blk > nb1 ? nb1 : blk);
  const size_t base = ((((size_t)blk * a.n_kv_heads + c.kvh) * HD + lr) << LOG2_BS) + (tv & bmask);
  const char *vp = static_cast<const char *>(a.v_pool) + base * 2;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
    __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1))) *)(vp + dt * 16 * BS * 2),
                                     (void __attribute__((address_space(3))) *)(s_v + dt * kWave), 16, 0, kStreamingLoad);
}

template <int HD, int BS>
__global__ __launch_bounds__(kWave) __attribute__((amdgpu_waves_per_eu(2))) void decode_stream(DecodeArgs a) {
  constexpr int KS = HD / 32, DT = HD / 16;
  __shared__ uint4 s_k[2 * KS * kWave];
  __shared__ uint4 s_v[DT * kWave];
  __shared__ int32_t s_wctx[kWindowRows], s_wgpre[kWindowRows];
  const StreamLayout L = stream_layout(a.rows, a.n_kv_heads, a.group, a.head_dim, a.max_parts);
  const int32_t *wsi = reinterpret_cast<const int32_t *>(a.ws);
  const int w = blockIdx.x;
  const int lane = threadIdx.x, lr = lane & 15, lg = lane >> 4;
  const int cap = a.max_blocks_per_row * a.block_size;
  // Start-up round trip 1: header, this wave's start and the first row window
  // (rows 0.. of the batch) are independent loads, issued together.
  RowWindow win;
  win.r0 = -(1 << 30);
  win.ctx = s_wctx;
  win.gpre = s_wgpre;
  int ngk;
  long long waves;
  Cursor c0;
  c0.idx = 0;
  if (a.inplan) {
    ngk = plan_in_wave(win, a, lane, cap);
    const long long ng_all0 = (long long)a.n_kv_heads * ngk;
    waves = ng_all0 / max(a.cg_min, 1);
    waves = waves < 1 ? 1 : (waves > kStreamWaves ? kStreamWaves : waves);
    if (w < a.rows && win.ctx[w] == 0) {  // an empty row reads zeros; no slice visits it
      for (int idx = lane; idx < a.n_heads * a.head_dim; idx += kWave)
        store_out(a.out, a.out_dtype, (size_t)w * a.n_heads * a.head_dim + idx, 0.f);
    }
    if (ng_all0 == 0 || w >= waves) return;
    const long long st = slice_start(w, ng_all0, waves);
    c0.kvh = (int)(st / ngk);
    plan_locate(win, (int)(st - (long long)c0.kvh * ngk), lane, c0.r, c0.j);
  } else {
    window_cover(win, a, wsi, L, 0, lane, cap);
    ngk = wsi[L.hdr];
    waves = wsi[L.hdr + 1];
    if (w >= waves) return;
    const int qi = wsi[L.first_pos + 2 * w];
    c0.kvh = qi / a.rows;
    c0.r = qi - c0.kvh * a.rows;
    c0.j = wsi[L.first_pos + 2 * w + 1];
    window_cover(win, a, wsi, L, c0.r, lane, cap);
  }
  const long long ng_all = (long long)a.n_kv_heads * ngk;
  const int total = (int)(slice_start(w + 1, ng_all, waves) - slice_start(w, ng_all, waves));
  cursor_row(c0, win, w, ngk, ng_all, waves);

  auto load_q = [&](const Cursor &c, bf16x8_t *qb) {
#pragma unroll
    for (int i = 0; i < KS; ++i)
      qb[i] = lr < a.group ? ld_bf16x8(a.q, (((size_t)c.r * a.n_heads + c.kvh * a.group + lr) * HD + (4 * i + lg) * 8) * 2)
                           : zero_bf16x8();
  };
  bf16x8_t qb[KS];
  load_q(c0, qb);
  const float cscale = a.scale * kLog2e;
  float m = -INFINITY, l = 0.f;
  f32x4_t acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  Cursor c1 = c0, c2;
  if (total > 1) cursor_next(c1, win, a, wsi, L, w, ngk, ng_all, waves, lane, cap);
  c2 = c1;
  if (total > 2) cursor_next(c2, win, a, wsi, L, w, ngk, ng_all, waves, lane, cap);

  GroupIds ids1;
  {
    const GroupIds ids0 = load_ids<BS>(a, c0, lr, lg);
    stage_group<HD, BS>(s_k, s_v, a, c0, ids0, lane, lr, lg);
  }
  ids1 = load_ids<BS>(a, c1, lr, lg);

  bf16x8_t kc[2][KS], vc[DT];
  while (true) {
    // The staged group (and the next group's block ids) must have landed.
    // The compiler does not order LDS reads after direct-to-LDS loads by
    // itself, so the wait is explicit and fenced against reordering.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    asm volatile("" ::: "memory");
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int i = 0; i < KS; ++i) kc[tt][i] = __builtin_bit_cast(bf16x8_t, s_k[(tt * KS + i) * kWave + lane]);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) vc[dt] = __builtin_bit_cast(bf16x8_t, s_v[dt * kWave + lane]);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the buffer may be refilled
    asm volatile("" ::: "memory");
    const bool last_group = c0.idx + 1 >= total;
    GroupIds ids2;
    if (!last_group) {
      ids2 = load_ids<BS>(a, c2, lr, lg);
      stage_group<HD, BS>(s_k, s_v, a, c1, ids1, lane, lr, lg);
    }
    f32x4_t sacc[2];
    group_scores<HD>(kc, qb, sacc);
    group_softmax_pv<HD>(sacc, vc, acc, m, l, cscale, c0.n, c0.j * kGroupPositions, lg);
    if (c0.j == c0.ng - 1 || last_group) segment_end<HD>(a, L, c0, acc, m, l, lr, lg);
    if (last_group) break;
    const bool new_row = c1.r != c0.r || c1.kvh != c0.kvh;
    c0 = c1;
    c1 = c2;
    if (c2.idx + 1 < total) cursor_next(c2, win, a, wsi, L, w, ngk, ng_all, waves, lane, cap);
    ids1 = ids2;
    if (new_row) load_q(c0, qb);
  }
}

template <int HD, int BS>
hipError_t launch_stream(const DecodeArgs &a, hipStream_t stream) {
  hipError_t e;
  if (!a.inplan) {
    hipLaunchKernelGGL(decode_plan, dim3(1), dim3(1024), 0, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((decode_stream<HD, BS>), dim3(kStreamWaves), dim3(kWave), 0, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_stream_merge, dim3((unsigned)a.n_kv_heads * a.rows), dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <typename T, int HD, int GP>
hipError_t launch_t(const DecodeArgs &a, hipStream_t stream) {
  const dim3 grid((unsigned)a.max_parts * a.n_kv_heads * a.rows);
  const size_t lds = (size_t)(a.partition_tokens >> a.log2_bs) * sizeof(int32_t);
  hipLaunchKernelGGL((decode_partition<T, HD, GP>), grid, dim3(kThreads), lds, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.max_parts <= 1) return e;
  hipLaunchKernelGGL(decode_merge, dim3((unsigned)a.rows * a.n_heads), dim3(128), 0, stream, a);
  return hipGetLastError();
}

template <typename T, int HD>
hipError_t launch_hd(const DecodeArgs &a, hipStream_t s) {
  const int g = a.group;
  if (g <= 1) return launch_t<T, HD, 1>(a, s);
  if (g <= 2) return launch_t<T, HD, 2>(a, s);
  if (g <= 4) return launch_t<T, HD, 4>(a, s);
  if (g <= 8) return launch_t<T, HD, 8>(a, s);
  return launch_t<T, HD, 16>(a, s);
}

template <typename T>
hipError_t launch_dt(const DecodeArgs &a, hipStream_t s) {
  switch (a.head_dim) {
    case 16: return launch_hd<T, 16>(a, s);
    case 64: return launch_hd<T, 64>(a, s);
    default: return launch_hd<T, 128>(a, s);
  }
}

// ---------------------------------------------------------------------------
// Multi-query read: each row brings a chunk of query_len queries, its last
// query_len positions (already in the pool), causal inside the chunk -- query
// i at position n - query_len + i sees positions 0 .. n - query_len + i.
//
// The 16 columns of the score tile S^T = K Q^T hold (query, head) pairs:
// 16 / group queries of one kv head's group per tile.  One wave per
// (position partition, query tile, kv head, row) walks its partition's
// 32-position groups -- only those some query of the tile can see -- with the
// same LDS-staged K/V and MFMA tiles as the one-query read, a per-column
// causal bound on the scores, and an online softmax that tolerates a column
// with nothing visible yet.  Rows of one partition are written directly;
// longer rows leave per-partition (max, sum, acc) for decode_multi_merge.
// ---------------------------------------------------------------------------
template <int HD>
__device__ __forceinline__ void group_softmax_pv_causal(const f32x4_t (&sacc)[2], bf16x8_t (&v)[HD / 16],
                                                        f32x4_t *acc, float &m, float &l, float c, int col_end,
                                                        int row_end, int gbase, int lg) {
  constexpr int DT = HD / 16;
  const int tl = gbase + 8 * lg;
  float s[8];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int j = 0; j < 4; ++j) s[4 * tt + j] = (tl + 4 * tt + j < col_end) ? sacc[tt][j] * c : -INFINITY;
  float mx = fmaxf(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])), fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7])));
  mx = max_across_rows(mx);
  const float m_new = fmaxf(m, mx);
  const float alpha = (m == m_new) ? 1.f : exp2_fast(m - m_new);
  m = m_new;
  float pv[8], psum = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    pv[e] = s[e] == -INFINITY ? 0.f : exp2_fast(s[e] - m_new);  // nothing visible yet: m_new is -inf too
    psum += pv[e];
  }
  l = l * alpha + psum;
  if (__any(alpha != 1.f)) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[dt] *= alpha;
  }
  uint32_t hw[4], lw[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t h0 = bf16_bits_rne(pv[2 * i]), h1 = bf16_bits_rne(pv[2 * i + 1]);
    const float r0 = pv[2 * i] - __builtin_bit_cast(float, h0 << 16);
    const float r1 = pv[2 * i + 1] - __builtin_bit_cast(float, h1 << 16);
    hw[i] = h0 | (h1 << 16);
    lw[i] = bf16_bits_rne(r0) | (bf16_bits_rne(r1) << 16);
  }
  const bf16x8_t phi = __builtin_bit_cast(bf16x8_t, make_uint4(hw[0], hw[1], hw[2], hw[3]));
  const bf16x8_t plo = __builtin_bit_cast(bf16x8_t, make_uint4(lw[0], lw[1], lw[2], lw[3]));
  if (gbase + 32 > row_end) {  // positions past the row end: zero their (possibly NaN) V
    int nv = row_end - tl;
    nv = nv < 0 ? 0 : (nv > 8 ? 8 : nv);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) v[dt] = keep_first(v[dt], nv);
  }
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v[dt], phi, acc[dt], 0, 0, 0);
    acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v[dt], plo, acc[dt], 0, 0, 0);
  }
}

template <int HD, int BS>
__global__ __launch_bounds__(kWave) void decode_multi(DecodeArgs a) {
  constexpr int KS = HD / 32, DT = HD / 16;
  __shared__ uint4 s_k[2 * KS * kWave];
  __shared__ uint4 s_v[DT * kWave];
  const int lane = threadIdx.x, lr = lane & 15, lg = lane >> 4;
  const int G = a.group, Q = a.query_len, QB = a.q_per_tile, P = a.partition_tokens;
  long long u = blockIdx.x;  // kv head fastest (spread over XCDs), then row, query tile, partition
  const int kvh = (int)(u % a.n_kv_heads);
  u /= a.n_kv_heads;
  const int r = (int)(u % a.rows);
  u /= a.rows;
  const int qt = (int)(u % a.q_tiles);
  const int part = (int)(u / a.q_tiles);
  const int cap = a.max_blocks_per_row * a.block_size;
  int n = a.context_lens[r];
  n = n < 0 ? 0 : (n > cap ? cap : n);
  const int nparts = n > 0 ? (n + P - 1) / P : 1;
  if (part >= nparts) return;
  // this lane's column: query qi, head kvh * G + hi
  const int qi = qt * QB + lr / G, hi = lr % G;
  const bool col = lr < QB * G && qi < Q;
  const int col_end = col ? max(n - Q + qi + 1, 0) : 0;  // positions this query sees
  const int q_last = min(Q - 1, qt * QB + QB - 1);
  const int pos0 = part * P;
  const int unit_end = max(min(pos0 + P, n - Q + q_last + 1), pos0);  // some query sees positions below
  bf16x8_t qb[KS];
#pragma unroll
  for (int i = 0; i < KS; ++i)
    qb[i] = col ? ld_bf16x8(a.q, ((((size_t)r * Q + qi) * a.n_heads + kvh * G + hi) * HD + (4 * i + lg) * 8) * 2)
                : zero_bf16x8();
  const float cscale = a.scale * kLog2e;
  float m = -INFINITY, l = 0.f;
  f32x4_t acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int g0 = pos0 / kGroupPositions, g1 = (unit_end + kGroupPositions - 1) / kGroupPositions;
  Cursor c;
  c.kvh = kvh;
  c.r = r;
  c.n = n;
  GroupIds ids1;
  if (g0 < g1) {
    c.j = g0;
    const GroupIds ids0 = load_ids<BS>(a, c, lr, lg);
    stage_group<HD, BS>(s_k, s_v, a, c, ids0, lane, lr, lg);
    if (g0 + 1 < g1) {
      c.j = g0 + 1;
      ids1 = load_ids<BS>(a, c, lr, lg);
    }
  }
  bf16x8_t kc[2][KS], vc[DT];
  for (int g = g0; g < g1; ++g) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the staged group has landed (LDS DMA is not ordered for us)
    asm volatile("" ::: "memory");
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int i = 0; i < KS; ++i) kc[tt][i] = __builtin_bit_cast(bf16x8_t, s_k[(tt * KS + i) * kWave + lane]);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) vc[dt] = __builtin_bit_cast(bf16x8_t, s_v[dt * kWave + lane]);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the buffer may be refilled
    asm volatile("" ::: "memory");
    if (g + 1 < g1) {
      c.j = g + 1;
      stage_group<HD, BS>(s_k, s_v, a, c, ids1, lane, lr, lg);
      if (g + 2 < g1) {
        c.j = g + 2;
        ids1 = load_ids<BS>(a, c, lr, lg);
      }
    }
    f32x4_t sacc[2];
    group_scores<HD>(kc, qb, sacc);
    group_softmax_pv_causal<HD>(sacc, vc, acc, m, l, cscale, col_end, n, g * kGroupPositions, lg);
  }
  const float lt = sum_across_rows(l);
  if (!col) return;
  const size_t vrow_head = ((size_t)r * Q + qi) * a.n_heads + kvh * G + hi;
  if (nparts == 1) {
    const float inv = lt > 0.f ? 1.f / lt : 0.f;  // a query before the history reads zeros
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int e = 0; e < 4; ++e) store_out(a.out, a.out_dtype, vrow_head * HD + 16 * dt + 4 * lg + e, acc[dt][e] * inv);
  } else {
    const WsLayout W = ws_layout(a.rows * Q, a.n_heads, a.max_parts, HD);
    const size_t slot = vrow_head * a.max_parts + part;
    float *accp = a.ws + W.acc_off + slot * HD;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) *reinterpret_cast<f32x4_t *>(accp + 16 * dt + 4 * lg) = acc[dt];
    if (lg == 0) {
      a.ws[W.m_off + slot] = m;
      a.ws[W.l_off + slot] = lt;
    }
  }
}

// Combine the partitions of one (row, query, head) of the multi-query read:
// M = max_k m_k over partitions that saw something; out = sum_k acc_k 2^(m_k - M)
// / sum_k l_k 2^(m_k - M), or zeros when no partition saw a position.
__global__ __launch_bounds__(128) void decode_multi_merge(DecodeArgs a) {
  const int Q = a.query_len, HD = a.head_dim;
  const size_t vh = blockIdx.x;  // ((row * Q + query) * n_heads + head)
  const int r = (int)(vh / ((size_t)Q * a.n_heads));
  const int cap = a.max_blocks_per_row * a.block_size;
  int n = a.context_lens[r];
  n = n < 0 ? 0 : (n > cap ? cap : n);
  const int nparts = n > 0 ? (n + a.partition_tokens - 1) / a.partition_tokens : 1;
  if (nparts <= 1) return;
  const WsLayout W = ws_layout(a.rows * Q, a.n_heads, a.max_parts, HD);
  const size_t s0 = vh * a.max_parts;
  float M = -INFINITY;
  for (int k = 0; k < nparts; ++k) M = fmaxf(M, a.ws[W.m_off + s0 + k]);
  for (int d = threadIdx.x; d < HD; d += blockDim.x) {
    float L = 0.f, O = 0.f;
    if (M != -INFINITY) {
      for (int k = 0; k < nparts; ++k) {
        const float mk = a.ws[W.m_off + s0 + k];
        if (mk == -INFINITY) continue;
        const float w = exp2_fast(mk - M);
        L = fmaf(a.ws[W.l_off + s0 + k], w, L);
        O = fmaf(a.ws[W.acc_off + (s0 + k) * HD + d], w, O);
      }
    }
    store_out(a.out, a.out_dtype, vh * HD + d, L > 0.f ? O / L : 0.f);
  }
}

template <int HD, int BS>
hipError_t launch_multi_t(const DecodeArgs &a, hipStream_t stream) {
  const long long units = (long long)a.max_parts * a.q_tiles * a.rows * a.n_kv_heads;
  hipLaunchKernelGGL((decode_multi<HD, BS>), dim3((unsigned)units), dim3(kWave), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.max_parts <= 1) return e;
  hipLaunchKernelGGL(decode_multi_merge, dim3((unsigned)((size_t)a.rows * a.query_len * a.n_heads)), dim3(128), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream) {
  if (a.dtype == kF32) return launch_dt<float>(a, stream);
  if (a.stream) {
    if (a.head_dim == 128) {
      if (a.block_size == 8) return launch_stream<128, 8>(a, stream);
      if (a.block_size == 16) return launch_stream<128, 16>(a, stream);
      return launch_stream<128, 32>(a, stream);
    }
    if (a.block_size == 8) return launch_stream<64, 8>(a, stream);
    if (a.block_size == 16) return launch_stream<64, 16>(a, stream);
    return launch_stream<64, 32>(a, stream);
  }
  if (a.head_dim == 128 || a.head_dim == 64) {
    if (a.head_dim == 128) {
      if (a.block_size == 8) return launch_mfma<128, 8>(a, stream);
      if (a.block_size == 16) return launch_mfma<128, 16>(a, stream);
      return launch_mfma<128, 32>(a, stream);
    }
    if (a.block_size == 8) return launch_mfma<64, 8>(a, stream);
    if (a.block_size == 16) return launch_mfma<64, 16>(a, stream);
    return launch_mfma<64, 32>(a, stream);
  }
  return launch_dt<uint16_t>(a, stream);
}

hipError_t launch_multi(const DecodeArgs &a, hipStream_t stream) {
  if (a.head_dim == 128) {
    if (a.block_size == 8) return launch_multi_t<128, 8>(a, stream);
    if (a.block_size == 16) return launch_multi_t<128, 16>(a, stream);
    return launch_multi_t<128, 32>(a, stream);
  }
  if (a.block_size == 8) return launch_multi_t<64, 8>(a, stream);
  if (a.block_size == 16) return launch_multi_t<64, 16>(a, stream);
  return launch_multi_t<64, 32>(a, stream);
}

}  // namespace pkv
