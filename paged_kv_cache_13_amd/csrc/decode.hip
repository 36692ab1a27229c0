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
#include <climits>

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

// Partition kernels: the partition's block ids, every entry up to the
// table's width whatever the row's length, loaded by thread tid (entries
// tid, tid + kThreads, ...) together with the row's length, so that the
// length and the ids cost one round trip, not two.  Entries past the row's
// blocks are loaded and never used.
constexpr int kIdsPerThread = kMaxPartitionBlocks / kThreads;
struct PartIds {
  int32_t v[kIdsPerThread];
};
__device__ __forceinline__ int part_ids_count(const DecodeArgs &a, int start) {
  const int cap = a.max_blocks_per_row * a.block_size;
  return (min(start + a.partition_tokens, cap) - start + a.block_size - 1) >> a.log2_bs;
}
__device__ __forceinline__ void part_ids_load(PartIds &ids, const DecodeArgs &a, int r, int start, int tid) {
  const int cnt = part_ids_count(a, start);
  const int32_t *row = a.block_table + (size_t)r * a.max_blocks_per_row + (start >> a.log2_bs);
#pragma unroll
  for (int x = 0; x < kIdsPerThread; ++x) {
    const int i = tid + x * kThreads;
    ids.v[x] = i < cnt ? row[i] : 0;
  }
}
// The ids, clamped into the pool, to LDS (the caller's barrier publishes them).
__device__ __forceinline__ void part_ids_store(const PartIds &ids, const DecodeArgs &a, int start, int tid,
                                               int32_t *s_blk) {
  const int cnt = part_ids_count(a, start);
#pragma unroll
  for (int x = 0; x < kIdsPerThread; ++x) {
    const int i = tid + x * kThreads;
    if (i < cnt) {
      const int64_t b = ids.v[x];
      s_blk[i] = (int32_t)(b < 0 ? 0 : (b >= a.num_blocks ? a.num_blocks - 1 : b));
    }
  }
}

// Partition kernels: one kv head's new token of row r, stored into its pool
// slot by threads t0, t0 + nthreads, ... (skipped like the scatter skips).
// E: the pool's element type, bit-copied.
template <typename E>
__device__ __forceinline__ void append_store_row(const DecodeArgs &a, int r, int kvh, int t0, int nthreads) {
  const int64_t s = a.slot_new[r];
  if (s < 0 || s >= a.num_blocks * a.block_size) return;
  const int64_t blk = s >> a.log2_bs, off = s & (a.block_size - 1);
  const size_t src = ((size_t)r * a.n_kv_heads + kvh) * a.head_dim;
  const E *kn = static_cast<const E *>(a.k_new) + src;
  const E *vn = static_cast<const E *>(a.v_new) + src;
  E *kp = static_cast<E *>(const_cast<void *>(a.k_pool)) +
          ((((size_t)blk * a.n_kv_heads + kvh) << a.log2_bs) + off) * a.head_dim;
  E *vp = static_cast<E *>(const_cast<void *>(a.v_pool)) +
          ((((size_t)blk * a.n_kv_heads + kvh) << a.log2_bs) + off) * a.head_dim;
  for (int d = t0; d < a.head_dim; d += nthreads) {
    kp[d] = kn[d];
    vp[d] = vn[d];
  }
}

// A row with no positions that still brings a token: appended whole (every
// kv head) by the threads that zero-fill the row, as the scatter would.
template <typename E>
__device__ __forceinline__ void append_empty_row(const DecodeArgs &a, int r, int t0, int nthreads) {
  for (int h = 0; h < a.n_kv_heads; ++h) append_store_row<E>(a, r, h, t0, nthreads);
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
  const int P = a.partition_tokens;
  const int start = p * P;
  int n = a.context_lens[r];
  PartIds pids;
  part_ids_load(pids, a, r, start, tid);
  n = n < 0 ? 0 : (n > cap ? cap : n);
  const int group = a.group;
  if (start >= n) {
    if (p == 0) {  // empty row: zeros
      for (int idx = tid; idx < group * HD; idx += kThreads) {
        const int j = idx / HD, d = idx % HD;
        store_out(a.out, a.out_dtype, ((size_t)r * a.n_heads + g * group + j) * HD + d, 0.f);
      }
      if (n == 0 && g == 0 && a.slot_new) append_empty_row<T>(a, r, tid, kThreads);
    }
    return;
  }
  const int end = min(n, start + P);
  const bool single = n <= P;

  part_ids_store(pids, a, start, tid, s_blk);  // this partition's block ids, clamped into the pool

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
  // A decode step's new token (position n - 1) in this partition: stored
  // into its pool slot before any K/V is loaded, as in the MFMA partition
  // kernel.
  if (a.slot_new != nullptr && n - 1 < end) {
    append_store_row<T>(a, r, g, tid, kThreads);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the stores have completed
  }
  __threadfence_block();
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
        vr[i] = load16(a.v_pool, (row * HD + c * EPL) * ES);
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
// One workgroup per (row, head), one output per thread (head_dim <= 128).
// The partials of up to kMergeBatch partitions are loaded together (one
// round trip per batch, not one per partition), then folded in order.  The
// first batch is loaded beside the row's length, before the partition count
// is known: slots below max_parts lie in the workspace whatever the length,
// and the slots past the row's last partition (which may hold anything)
// are then replaced by empty partials.
constexpr int kMergeBatch = 8;
__global__ __launch_bounds__(128) void decode_merge(DecodeArgs a) {
  const int r = blockIdx.x / a.n_heads;
  const int h = blockIdx.x % a.n_heads;
  const int cap = a.max_blocks_per_row * a.block_size;
  const int n_raw = a.context_lens[r];
  const int P = a.partition_tokens;
  const WsLayout ws = ws_layout(a.rows, a.n_heads, a.max_parts, a.head_dim);
  const size_t base = ((size_t)r * a.n_heads + h) * a.max_parts;
  const float *mp = a.ws + ws.m_off + base;
  const float *lp = a.ws + ws.l_off + base;
  const float *ap = a.ws + ws.acc_off + base * a.head_dim;
  const int d = (int)threadIdx.x;
  const bool live = d < a.head_dim;
  const int dl = live ? d : 0;
  const int kl = min(kMergeBatch, a.max_parts) - 1;  // the last slot every row has
  float mk[kMergeBatch], lk[kMergeBatch], ak[kMergeBatch];
#pragma unroll
  for (int k = 0; k < kMergeBatch; ++k) {
    const int sk = min(k, kl);
    mk[k] = mp[sk];
    lk[k] = lp[sk];
    ak[k] = ap[(size_t)sk * a.head_dim + dl];
  }
  // keep these loads ahead of the test below (in flight with the length's)
#pragma unroll
  for (int k = 0; k < kMergeBatch; ++k) asm volatile("" ::"v"(mk[k]), "v"(lk[k]), "v"(ak[k]));
  const int n = n_raw < 0 ? 0 : (n_raw > cap ? cap : n_raw);
  const int nparts = (n + P - 1) / P;
  if (nparts <= 1) return;
  float M = -INFINITY, L = 0.f, O = 0.f;
  for (int p0 = 0; p0 < nparts; p0 += kMergeBatch) {
    if (p0 == 0) {
#pragma unroll
      for (int k = 0; k < kMergeBatch; ++k)
        if (k >= nparts) {
          mk[k] = -INFINITY;
          lk[k] = 0.f;
          ak[k] = 0.f;
        }
    } else {
#pragma unroll
      for (int k = 0; k < kMergeBatch; ++k) {
        const bool in = p0 + k < nparts;
        mk[k] = in ? mp[p0 + k] : -INFINITY;
        lk[k] = in ? lp[p0 + k] : 0.f;
        ak[k] = in ? ap[(size_t)(p0 + k) * a.head_dim + dl] : 0.f;
      }
    }
    float mn = M;
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k) mn = fmaxf(mn, mk[k]);
    const float a0 = M == -INFINITY ? 0.f : exp2_fast(M - mn);
    L *= a0;
    O *= a0;
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k) {
      const float wk = mk[k] == -INFINITY ? 0.f : exp2_fast(mk[k] - mn);
      L = fmaf(lk[k], wk, L);
      O = fmaf(ak[k], wk, O);
    }
    M = mn;
  }
  if (live) store_out(a.out, a.out_dtype, ((size_t)r * a.n_heads + h) * a.head_dim + d, O / L);
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
//                      (read transposed out of a position-major LDS tile,
//                      see v_tile_frag), B = P, head_dim / 16 d-tiles.
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
typedef float f32x2_t __attribute__((ext_vector_type(2)));

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

// V comes out of the pool position-major, as K does: a 32-position group is
// 32 rows of head_dim bf16.  The P.V product needs, per lane, 8 consecutive
// positions of one dimension, so the group is staged in LDS as rows and read
// back with ds_read_b64_tr_b16: within each 16 lanes, lanes 4r .. 4r + 3
// name the four 8-byte pieces of row r of a 4 x 16 block (lane 4r + q:
// columns 4q .. 4q + 3) and lane i receives column i of rows 0 .. 3.
//
// Staged tile: row p (group position) at p * 2 head_dim bytes, its logical
// 16-byte chunk c at physical chunk c ^ vswz16(p).  The XOR keeps every
// transposed read free of bank conflicts (each 16-, 32- or 64-lane set of a
// read touches distinct banks) and leaves bit 2 of p alone, so the second
// read of a fragment (rows p + 4) is the first one's address plus 4 rows.
template <int HD>
__device__ __forceinline__ int vswz16(int p) {
  const int b0 = p & 1, b1 = (p >> 1) & 1, b3 = (p >> 3) & 1, b4 = (p >> 4) & 1;
  return HD == 128 ? 2 * ((b0 ^ b4) | (b1 << 1) | (b3 << 2)) : 2 * ((b0 ^ b3) | ((b1 ^ b4) << 1));
}

typedef short v4i16_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 lds_read_tr16(const void *lds, uint32_t byte_off) {
  auto *p = (__attribute__((address_space(3))) v4i16_t *)((__attribute__((address_space(3))) char *)lds + byte_off);
  return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(p));
}

// Byte offset, in a staged V tile, of this lane's first transposed read of
// d-tile 0 (rows 8 lg + lr / 4, dims 4 (lr % 4) .. + 3); d-tile dt is that
// offset XOR 32 dt, the second read 4 rows further.
template <int HD>
__device__ __forceinline__ uint32_t v_tile_lane(int lr, int lg) {
  const int p = 8 * lg + (lr >> 2), q = lr & 3;
  return (uint32_t)(p * 2 * HD + 16 * ((q >> 1) ^ vswz16<HD>(p)) + 8 * (q & 1));
}

// V fragment dt of lane (lr, lg): dim 16 dt + lr at positions 8 lg .. + 7.
template <int HD>
__device__ __forceinline__ bf16x8_t v_tile_frag(const void *tile, uint32_t lane_off, int dt) {
  const uint32_t o = lane_off ^ (uint32_t)(32 * dt);
  const uint2 lo = lds_read_tr16(tile, o), hi = lds_read_tr16(tile, o + 8 * HD);
  return __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
}

// Source of the 16 bytes that load i of a tile fill (LDS chunk 64 i + lane):
// group row p, logical chunk c.  A load covers 64 / (head_dim / 8) whole
// consecutive rows, which lie in one pool block.
template <int HD>
__device__ __forceinline__ void v_tile_src(int i, int lane, int &p, int &c) {
  constexpr int CPR = HD / 8, PPL = kWave / CPR;
  p = PPL * i + lane / CPR;
  c = (lane % CPR) ^ vswz16<HD>(p);
}

// s_waitcnt immediate for vmcnt(n) and lgkmcnt(0) (expcnt left alone).
__host__ __device__ constexpr int vmcnt_lgkm0(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0070; }

template <int HD>
struct MfmaTiles {
  bf16x8_t k[2][HD / 32];  // score tiles x k-steps
};

// Issue the loads of one 32-position group.  Branch-free: positions at or
// past `end` load from the partition's first position instead (always
// mapped), and are masked where they are used, so the loads of the next group
// can be in flight while this one is computed.
template <int HD, int BS>
__device__ __forceinline__ void mfma_load(MfmaTiles<HD> &T, uint4 *vtile, const DecodeArgs &a, const int32_t *s_blk,
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
  // V rows straight into the wave's LDS tile `vtile` (direct-to-LDS loads,
  // no registers).  Rows past `end` read row end - 1 instead.  A load's rows
  // are one aligned run of 64 / (head_dim / 8) positions, so they (clamped
  // or not) share the block of the run's first position, clamped the same way.
  constexpr int PPL = kWave / (HD / 8);
  const int lane = 16 * lg + lr;
#pragma unroll
  for (int i = 0; i < DT; ++i) {
    int p, col;
    v_tile_src<HD>(i, lane, p, col);
    const int t = min(gbase + p, end - 1);
    const int32_t blk =
        __builtin_amdgcn_readfirstlane(s_blk[(min(gbase + PPL * i, end - 1) - start) >> LOG2_BS]);
    const char *vb = static_cast<const char *>(a.v_pool) + ((((size_t)blk * a.n_kv_heads + g) << LOG2_BS) * HD) * 2 +
                     (uint32_t)(((t & bmask) * HD + 8 * col) * 2);
    __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1))) *)vb,
                                     (void __attribute__((address_space(3))) *)(vtile + i * kWave), 16, 0, 0);
  }
}

// Until only the next group's loads (issued after this group's) are in
// flight: this group's K registers and V tile have landed.  The compiler
// orders neither the V tile's LDS reads after its direct-to-LDS loads nor
// (by itself) the K registers' wait before them, so the wait is explicit.
template <int HD>
__device__ __forceinline__ void mfma_wait_group(bool next_in_flight) {
  constexpr int kNextLoads = 2 * (HD / 32) + HD / 16;  // K then V loads of one group
  asm volatile("" ::: "memory");
  if (next_in_flight)
    __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0(kNextLoads));
  else
    __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0(0));
  asm volatile("" ::: "memory");
}

// Online-softmax step over one loaded group (see the block comment above).
template <int HD>
__device__ __forceinline__ void mfma_compute(MfmaTiles<HD> &T, const bf16x8_t *qb, f32x4_t *acc, float &m,
                                             float &l, float c, int end, int gbase, int lg, const uint4 *s_vw,
                                             uint32_t v_lane) {
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
  bf16x8_t vf[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) vf[dt] = v_tile_frag<HD>(s_vw, v_lane, dt);
  // The last group of a partition may hold positions past `end` (stale or
  // NaN pool slots): their weights are 0, but 0 * NaN is NaN, so the V values
  // themselves are zeroed.  Wave-uniform branch, taken once per partition.
  if (gbase + 32 > end) {
    int nv = end - tl;
    nv = nv < 0 ? 0 : (nv > 8 ? 8 : nv);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) vf[dt] = keep_first(vf[dt], nv);
  }
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[dt], phi, acc[dt], 0, 0, 0);
    acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[dt], plo, acc[dt], 0, 0, 0);
  }
}

// The decode step's new token, appended inside the read.  Each (kv head,
// row) has one wave that reads the group holding the row's new token (its
// last position, n - 1); that wave loads the token's K and V row ahead of
// time, and once the group has been loaded it stores the token into its
// pool slot and over the loaded (stale) copy of that position, before the
// group is used.  No other wave reads the slot in this call, so the read
// sees exactly what a scatter followed by a read would.  Slots that are
// negative or past the pool are skipped, as the scatter skips them.
//
// Lane layout of a loaded group in the stream kernel's LDS: K tile tt, row
// 8 (lr / 4) + 4 tt + lr % 4, dims 32 i + 8 lg .. + 8 in K fragment (tt, i)
// of lane (lr, lg); V as a staged tile of rows (v_tile_frag).
template <int HD>
struct Append {
  bool pending;        // wave-uniform: the token's group is computed next
  int p;               // the token's position in its group
  int64_t slot;        // loaded by every lane, read after the wait
  bf16x8_t k[HD / 32]; // lanes lr == append_k_lane(p): K dims 32 i + 8 lg .. + 8
  uint4 v;             // lanes below head_dim / 8: V chunk `lane` of the row
};

__device__ __forceinline__ int append_k_lane(int p) { return ((p >> 3) << 2) | (p & 3); }

template <int HD>
__device__ __forceinline__ void append_fetch(Append<HD> &A, const DecodeArgs &a, int r, int kvh, int p, int lr,
                                             int lg) {
  constexpr int KS = HD / 32;
  A.p = p;
  A.slot = a.slot_new[r];
  const size_t base = ((size_t)r * a.n_kv_heads + kvh) * HD;
  if (lr == append_k_lane(p)) {
#pragma unroll
    for (int i = 0; i < KS; ++i) A.k[i] = ld_bf16x8(a.k_new, (base + i * 32 + lg * 8) * 2);
  }
  const int lane = 16 * lg + lr;
  if (lane < HD / 8) A.v = load16(a.v_new, (base + 8 * lane) * 2);
}

// The slot, once the fetch has landed; -1 when the token is skipped.
template <int BS>
__device__ __forceinline__ int64_t append_slot(int64_t slot, const DecodeArgs &a) {
  const int64_t s = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(slot >> 32)) << 32) |
                              (uint32_t)__builtin_amdgcn_readfirstlane((int)slot));
  return (s < 0 || s >= a.num_blocks * BS) ? -1 : s;
}

template <int HD, int BS>
__device__ __forceinline__ void append_store_pool(const Append<HD> &A, const DecodeArgs &a, int kvh, int64_t s, int lr,
                                                  int lg) {
  constexpr int KS = HD / 32;
  constexpr int LOG2_BS = BS == 8 ? 3 : (BS == 16 ? 4 : 5);
  const int64_t blk = s >> LOG2_BS;
  const int off = (int)(s & (BS - 1));
  if (lr == append_k_lane(A.p)) {
    uint16_t *kp = static_cast<uint16_t *>(const_cast<void *>(a.k_pool)) +
                   ((((size_t)blk * a.n_kv_heads + kvh) << LOG2_BS) + off) * HD + lg * 8;
#pragma unroll
    for (int i = 0; i < KS; ++i) *reinterpret_cast<uint4 *>(kp + i * 32) = __builtin_bit_cast(uint4, A.k[i]);
  }
  const int lane = 16 * lg + lr;
  if (lane < HD / 8) {
    uint16_t *vp = static_cast<uint16_t *>(const_cast<void *>(a.v_pool)) +
                   ((((size_t)blk * a.n_kv_heads + kvh) << LOG2_BS) + off) * HD + 8 * lane;
    *reinterpret_cast<uint4 *>(vp) = A.v;
  }
}

// One kv head's new token of a row in one wave's registers: lane l holds K
// and V dims l, l + 64, ... of the row (bf16), and the slot.
template <int HD>
struct TokenRow {
  int64_t slot;
  uint16_t k[(HD + kWave - 1) / kWave], v[(HD + kWave - 1) / kWave];
};

template <int HD>
__device__ __forceinline__ void token_fetch(TokenRow<HD> &t, const DecodeArgs &a, int r, int kvh, int lane) {
  constexpr int PER = (HD + kWave - 1) / kWave;
  t.slot = a.slot_new[r];
  const size_t src = ((size_t)r * a.n_kv_heads + kvh) * HD;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int d = lane + i * kWave;
    if (d < HD) {
      t.k[i] = static_cast<const uint16_t *>(a.k_new)[src + d];
      t.v[i] = static_cast<const uint16_t *>(a.v_new)[src + d];
    }
  }
}

// The stores, skipped for slots the scatter would skip.
template <int HD, int BS>
__device__ __forceinline__ void token_store(const TokenRow<HD> &t, const DecodeArgs &a, int kvh, int lane) {
  constexpr int PER = (HD + kWave - 1) / kWave;
  constexpr int LOG2_BS = BS == 8 ? 3 : (BS == 16 ? 4 : 5);
  const int64_t s = t.slot;
  if (s < 0 || s >= a.num_blocks * BS) return;
  const int64_t blk = s >> LOG2_BS;
  const int off = (int)(s & (BS - 1));
  uint16_t *kp = static_cast<uint16_t *>(const_cast<void *>(a.k_pool)) +
                 ((((size_t)blk * a.n_kv_heads + kvh) << LOG2_BS) + off) * HD;
  uint16_t *vp = static_cast<uint16_t *>(const_cast<void *>(a.v_pool)) +
                 ((((size_t)blk * a.n_kv_heads + kvh) << LOG2_BS) + off) * HD;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int d = lane + i * kWave;
    if (d < HD) {
      kp[d] = t.k[i];
      vp[d] = t.v[i];
    }
  }
}

template <int HD, int BS, int NWV>
__global__ __launch_bounds__(NWV * kWave) __attribute__((amdgpu_waves_per_eu(2))) void decode_partition_mfma(DecodeArgs a) {
  constexpr int kWaves = NWV;  // four, or eight for a grid of at most one workgroup per compute unit
  constexpr int kThreads = NWV * kWave;
  constexpr int KS = HD / 32, DT = HD / 16, GT = 32;
  __shared__ float s_m[kWaves][16];
  __shared__ float s_l[kWaves][16];
  // Wave w's two V tiles (32 rows of head_dim bf16 each): s_acc[w], which
  // holds 64 * head_dim bytes too, until the wave's last group has been
  // read, and s_vt[w].
  __shared__ float s_acc[kWaves][16][HD];
  __shared__ uint4 s_vt[kWaves][HD / 16 * kWave];
  static_assert(sizeof(s_acc[0]) == sizeof(s_vt[0]), "a wave's V tile fills its s_acc row");
  extern __shared__ int32_t s_blk[];

  const WorkItem it = work_item(a);
  const int p = it.p, g = it.g, r = it.r;
  const int tid = threadIdx.x;
  const int cap = a.max_blocks_per_row * a.block_size;
  const int P = a.partition_tokens;
  const int start = p * P;
  int n = a.context_lens[r];
  PartIds pids;
  part_ids_load(pids, a, r, start, tid);
  n = n < 0 ? 0 : (n > cap ? cap : n);
  const int group = a.group;
  if (start >= n) {
    if (p == 0) {
      for (int idx = tid; idx < group * HD; idx += kThreads) {
        const int j = idx / HD, d = idx % HD;
        store_out(a.out, a.out_dtype, ((size_t)r * a.n_heads + g * group + j) * HD + d, 0.f);
      }
      if (n == 0 && g == 0 && a.slot_new) append_empty_row<uint16_t>(a, r, tid, kThreads);
    }
    return;
  }
  const int end = min(n, start + P);
  const bool single = n <= P;
  const int lane = tid % kWave;
  const int wave = tid / kWave;
  const int lr = lane & 15;  // head of the group (N index)
  const int lg = lane >> 4;  // k-slot group

  // A decode step's new token (position n - 1) in this partition: the wave
  // that loads its 32-position group stores it into its pool slot first, so
  // its own later load of that group reads it back (one wave's accesses to
  // an address stay in order); no other wave reads the slot.  Its K and V
  // row come in with the block ids, and the stores add no wait.
  const bool tok_wave = a.slot_new != nullptr && n - 1 < end && ((n - 1 - start) / GT) % kWaves == wave;
  TokenRow<HD> tok;
  if (tok_wave) token_fetch<HD>(tok, a, r, g, lane);
  part_ids_store(pids, a, start, tid, s_blk);

  bf16x8_t qb[KS];
#pragma unroll
  for (int i = 0; i < KS; ++i)
    qb[i] = lr < group
                ? ld_bf16x8(a.q, (((size_t)r * a.n_heads + g * group + lr) * HD + (4 * i + lg) * 8) * 2)
                : zero_bf16x8();
  if (tok_wave) token_store<HD, BS>(tok, a, g, lane);
  __syncthreads();

  const float c = a.scale * kLog2e;
  float m = -INFINITY, l = 0.f;
  f32x4_t acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Two tile sets (K registers, V LDS tile), alternating: while one group is
  // computed the next one's loads are in flight.  A set's V tile is refilled
  // only after its previous group's reads of it have returned (their values
  // fed that group's products).  Uniform control flow only.
  constexpr int kStep = kWaves * GT;
  uint4 *va = reinterpret_cast<uint4 *>(&s_acc[wave][0][0]);
  uint4 *vb = s_vt[wave];
  const uint32_t v_lane = v_tile_lane<HD>(lr, lg);
  MfmaTiles<HD> A, B;
  int gb = start + wave * GT;
  if (gb < end) {
    mfma_load<HD, BS>(A, va, a, s_blk, g, start, end, gb, lr, lg);
    while (true) {
      if (gb + kStep >= end) {
        mfma_wait_group<HD>(false);
        mfma_compute<HD>(A, qb, acc, m, l, c, end, gb, lg, va, v_lane);
        break;
      }
      mfma_load<HD, BS>(B, vb, a, s_blk, g, start, end, gb + kStep, lr, lg);
      mfma_wait_group<HD>(true);
      mfma_compute<HD>(A, qb, acc, m, l, c, end, gb, lg, va, v_lane);
      gb += kStep;
      if (gb + kStep >= end) {
        mfma_wait_group<HD>(false);
        mfma_compute<HD>(B, qb, acc, m, l, c, end, gb, lg, vb, v_lane);
        break;
      }
      mfma_load<HD, BS>(A, va, a, s_blk, g, start, end, gb + kStep, lr, lg);
      mfma_wait_group<HD>(true);
      mfma_compute<HD>(B, qb, acc, m, l, c, end, gb, lg, vb, v_lane);
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
  if (mfma_partition_waves(a.max_parts, a.n_kv_heads, a.rows) == 8)
    hipLaunchKernelGGL((decode_partition_mfma<HD, BS, 8>), grid, dim3(8 * kWave), lds, stream, a);
  else
    hipLaunchKernelGGL((decode_partition_mfma<HD, BS, 4>), grid, dim3(kThreads), lds, stream, a);
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
// stream, prefix-summed per row on the device (no host sync: inside every
// wave for batches of at most kWindowRows rows, else by a plan kernel) and
// cut into kStreamWaves equal contiguous slices.  Each persistent wave walks its slice with the next group's K/V
// and the group after next's block ids in flight, across row boundaries, so
// no wave waits on a partition start-up and every wave does the same work
// whatever the length mix.  A (kv head, row) covered by one wave is written
// to `out` directly; one cut into several slices gets one partial (max, sum,
// rescaled acc) per slice, which decode_stream_merge, the next kernel on
// the stream, combines.
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
  const StreamLayout L = stream_layout(rows, a.cols, a.head_dim, a.stream_waves);
  int32_t *wsi = reinterpret_cast<int32_t *>(a.ws);
  const int per = (rows + 1023) / 1024;
  const int r0 = min(rows, tid * per), r1 = min(rows, r0 + per);
  int local = 0;
  for (int r = r0; r < r1; ++r) {
    int n = a.context_lens[r];
    n = n < 0 ? 0 : (n > cap ? cap : n);
    s_gpre[r] = local;
    local += (n + kGroupPositions - 1) / kGroupPositions;
    if (n == 0) {  // an empty row reads zeros (all its queries); no wave visits it
      const size_t per_row = (size_t)a.query_len * a.n_heads * a.head_dim;
      for (size_t idx = 0; idx < per_row; ++idx) store_out(a.out, a.out_dtype, (size_t)r * per_row + idx, 0.f);
      if (a.slot_new) append_empty_row<uint16_t>(a, r, 0, 1);
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
  waves = waves < 1 ? 1 : (waves > a.stream_waves ? a.stream_waves : waves);
  if (ng_all == 0) waves = 0;
  if (tid == 0) {
    wsi[L.hdr] = ngk;
    wsi[L.hdr + 1] = (int)waves;
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
  int32_t k0, k1;  // this lane's block ids: its rows of score tiles 0 and 1
  int32_t v;       // block of positions 8 lg .. of the group (V staging)
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

// Online-softmax update and P.V of one group from its scores.  `end` (per
// lane): positions this lane's column sees; `row_end`: the row's length,
// past which V is zeroed.  A column that has seen nothing yet keeps m = -inf
// and takes 0 as its exponent reference, so all its weights are 0.
template <int HD>
__device__ __forceinline__ void group_softmax_pv(const f32x4_t (&sacc)[2], bf16x8_t (&v)[HD / 16], f32x4_t *acc,
                                                 float &m, float &l, float c, int end, int row_end, int gbase,
                                                 int lg) {
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
  const float mref = m_new == -INFINITY ? 0.f : m_new;
  float pv[8], psum = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    pv[e] = exp2_fast(s[e] - mref);
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

// Output row of stream column `col` of (kv head, row): query col / group,
// head kv head * group + col % group.
__device__ __forceinline__ size_t stream_out_row(const DecodeArgs &a, int kvh, int r, int col) {
  if (a.query_len == 1) return (size_t)r * a.n_heads + kvh * a.group + col;  // no division on the one-query read
  return ((size_t)r * a.query_len + col / a.group) * a.n_heads + kvh * a.group + col % a.group;
}

template <int HD>
__device__ __forceinline__ void write_out_rows(const DecodeArgs &a, const Cursor &c, const f32x4_t *o,
                                               float inv, int lr, int lg) {
  constexpr int DT = HD / 16;
  const size_t base = stream_out_row(a, c.kvh, c.r, lr) * HD + 4 * lg;
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
__device__ __forceinline__ void segment_end(const DecodeArgs &a, const StreamLayout &L, const Cursor &c, int w,
                                            f32x4_t *acc, float &m, float &l, int lr, int lg) {
  constexpr int DT = HD / 16;
  const int C = a.cols;
  const float lt = sum_across_rows(l);
  if (c.nparts == 1) {
    if (lr < C) write_out_rows<HD>(a, c, acc, lt > 0.f ? 1.f / lt : 0.f, lr, lg);  // 0: a query before the history
  } else if (lr < C) {
    // piece c.part of the pair: 2w + 1 for its first piece, 2w for a later one
    float *slot = a.ws + L.partials + (size_t)(c.part == 0 ? 2 * w + 1 : 2 * w) * L.slot_stride;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) *reinterpret_cast<f32x4_t *>(slot + lr * HD + 16 * dt + 4 * lg) = acc[dt];
    if (lg == 0) {
      slot[C * HD + lr] = m;
      slot[C * HD + C + lr] = lt;
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
// rows in one slice were written by the stream kernel already.  Pieces are
// taken kMergeMaxParts at a time, the running sums moved to each batch's new
// maximum.  The stream paths have at most 16 columns (a GQA group of at most
// 16 heads, or a chunk of query_len * group <= 16 columns).
constexpr int kMergeMaxParts = 8;
__global__ __launch_bounds__(256) void decode_stream_merge(DecodeArgs a) {
  const StreamLayout L = stream_layout(a.rows, a.cols, a.head_dim, a.stream_waves);
  const int32_t *wsi = reinterpret_cast<const int32_t *>(a.ws);
  const int pair = blockIdx.x;
  const int kvh = pair / a.rows, r = pair - kvh * a.rows;
  int ngk, g0, ng;
  long long waves;
  if (a.inplan) {
    // groups per kv head and before row r, by a block reduction over the
    // (at most 256) clamped lengths
    __shared__ int s_red[2][256 / kWave];
    __shared__ int s_len;
    const int cap = a.max_blocks_per_row * a.block_size;
    const int t = threadIdx.x;
    int x = t < a.rows ? a.context_lens[t] : 0;
    x = x < 0 ? 0 : (x > cap ? cap : x);
    if (t == r) s_len = x;  // row r's length, across the barrier below (no second load)
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
    ng = (s_len + kGroupPositions - 1) / kGroupPositions;
    const long long all = (long long)a.n_kv_heads * ngk;
    waves = all / max(a.cg_min, 1);
    waves = waves < 1 ? 1 : (waves > a.stream_waves ? a.stream_waves : waves);
  } else {
    ngk = wsi[L.hdr];
    waves = wsi[L.hdr + 1];
    g0 = wsi[L.gpre + r];
    ng = wsi[L.gpre + r + 1] - g0;
  }
  if (ng == 0) return;
  const long long ng_all = (long long)a.n_kv_heads * ngk;
  const long long S = (long long)kvh * ngk + g0;
  const long long first = slice_of(S, ng_all, waves);
  const int nparts = (int)(slice_of(S + ng - 1, ng_all, waves) - first + 1);
  if (nparts <= 1) return;
  const int C = a.cols, HD = a.head_dim;
  const float *parts = a.ws + L.partials;
  // Each thread merges two adjacent outputs (one column, hd d and d + 1) at a
  // time: per piece one 8-byte load of their acc values, while threads
  // 0 .. C * kMergeMaxParts - 1 fetch the pieces' m and l of every column
  // into LDS.  Every load of a batch of pieces is issued before any output
  // is stored (a store in between would keep the next loads behind it: the
  // compiler cannot tell out from the workspace).  Terms are taken in slice
  // order.  The loop counts are uniform, so the barriers are too.
  __shared__ float s_ml[2][kMergeMaxParts][16];  // m and l of a batch of pieces, columns < 16
  const int iters = (C * HD + 2 * (int)blockDim.x - 1) / (2 * (int)blockDim.x);
  for (int it = 0; it < iters; ++it) {
    const int idx = 2 * ((int)threadIdx.x + it * (int)blockDim.x);
    const bool live = idx < C * HD;
    const int j = live ? idx / HD : 0, d = live ? idx - j * HD : 0;  // HD is even: idx, idx + 1 share column j
    float M = -INFINITY, Lm = 0.f;
    f32x2_t O = {0.f, 0.f};
    for (int k0 = 0; k0 < nparts; k0 += kMergeMaxParts) {
      const int kn = min(nparts - k0, kMergeMaxParts);
      if (it > 0 || k0 > 0) __syncthreads();  // every thread is done with the previous batch's m and l
      if ((int)threadIdx.x < C * kMergeMaxParts) {
        const int u = threadIdx.x / C, jj = threadIdx.x - u * C;
        const float *sk = parts + stream_piece_slot(first, k0 + min(u, kn - 1)) * L.slot_stride;
        s_ml[0][u][jj] = u < kn ? sk[C * HD + jj] : -INFINITY;
        s_ml[1][u][jj] = u < kn ? sk[C * HD + C + jj] : 0.f;
      }
      f32x2_t ak[kMergeMaxParts];
#pragma unroll
      for (int k = 0; k < kMergeMaxParts; ++k) {
        const float *sk = parts + stream_piece_slot(first, k0 + min(k, kn - 1)) * L.slot_stride;
        ak[k] = k < kn ? *reinterpret_cast<const f32x2_t *>(sk + j * HD + d) : f32x2_t{0.f, 0.f};
      }
      __syncthreads();  // m and l published
      float mn = M;
#pragma unroll
      for (int k = 0; k < kMergeMaxParts; ++k)
        if (k < kn) mn = fmaxf(mn, s_ml[0][k][j]);
      const float a0 = M == -INFINITY ? 0.f : exp2_fast(M - mn);
      Lm *= a0;
      O[0] *= a0;
      O[1] *= a0;
#pragma unroll
      for (int k = 0; k < kMergeMaxParts; ++k) {
        if (k < kn) {
          // a slice that saw nothing of this column (m = -inf) adds nothing
          const float mk = s_ml[0][k][j];
          const float wk = mk == -INFINITY ? 0.f : exp2_fast(mk - mn);
          Lm = fmaf(s_ml[1][k][j], wk, Lm);
          O[0] = fmaf(ak[k][0], wk, O[0]);
          O[1] = fmaf(ak[k][1], wk, O[1]);
        }
      }
      M = mn;
    }
    if (live) {
      const size_t o = stream_out_row(a, kvh, r, j) * HD + d;
      store_out(a.out, a.out_dtype, o, Lm > 0.f ? O[0] / Lm : 0.f);
      store_out(a.out, a.out_dtype, o + 1, Lm > 0.f ? O[1] / Lm : 0.f);
    }
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
// The multi-query read's staging loads take the default cache policy: a
// non-temporal hint measured slower there.
constexpr int kMultiLoadPolicy = 0;

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
  // V: load i fills LDS chunks 64 i .. of the row tile (v_tile_src); its rows
  // lie in the block of positions t0 + 8 q .., q = its first row / 8, whose id
  // lane 16 q holds.  Rows past `last` read row `last` (same block).
  constexpr int PPL = kWave / (HD / 8);
#pragma unroll
  for (int i = 0; i < DT; ++i) {
    int p, col;
    v_tile_src<HD>(i, lane, p, col);
    int64_t blk = __builtin_amdgcn_readlane(ids.v, 16 * ((PPL * i) >> 3));
    blk = blk < 0 ? 0 : (blk > nb1 ? nb1 : blk);
    const int t = min(t0 + p, last);
    const char *vp = static_cast<const char *>(a.v_pool) +
                     ((((size_t)blk * a.n_kv_heads + c.kvh) << LOG2_BS) * HD) * 2 +
                     (uint32_t)(((t & bmask) * HD + 8 * col) * 2);
    __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1))) *)vp,
                                     (void __attribute__((address_space(3))) *)(s_v + i * kWave), 16, 0, kStreamingLoad);
  }
}

// Stream kernel: fetch for cursor c when it is its row's last group.
template <int HD>
__device__ __forceinline__ void append_load(Append<HD> &A, const DecodeArgs &a, const Cursor &c, int lr, int lg) {
  A.pending = a.slot_new != nullptr && c.j == c.ng - 1;
  if (A.pending) append_fetch<HD>(A, a, c.r, c.kvh, c.n - 1 - c.j * kGroupPositions, lr, lg);
}

// Stream kernel: after the group's tile has landed in LDS, before it is read.
template <int HD, int BS>
__device__ __forceinline__ void append_apply(const Append<HD> &A, const DecodeArgs &a, const Cursor &c, uint4 *s_k,
                                             uint4 *s_v, int lane, int lr, int lg) {
  constexpr int KS = HD / 32;
  const int64_t s = append_slot<BS>(A.slot, a);
  if (s < 0) return;
  append_store_pool<HD, BS>(A, a, c.kvh, s, lr, lg);
  const int p = A.p;
  if (lr == append_k_lane(p)) {
    const int tt = (p >> 2) & 1;
#pragma unroll
    for (int i = 0; i < KS; ++i) s_k[(tt * KS + i) * kWave + lane] = __builtin_bit_cast(uint4, A.k[i]);
  }
  if (lane < HD / 8) s_v[p * (HD / 8) + (lane ^ vswz16<HD>(p))] = A.v;
}

template <int HD, int BS>
__global__ __launch_bounds__(kWave) __attribute__((amdgpu_waves_per_eu(2))) void decode_stream(DecodeArgs a) {
  constexpr int KS = HD / 32, DT = HD / 16;
  __shared__ uint4 s_k[2 * KS * kWave];
  __shared__ uint4 s_v[DT * kWave];
  __shared__ int32_t s_wctx[kWindowRows], s_wgpre[kWindowRows];
  const StreamLayout L = stream_layout(a.rows, a.cols, a.head_dim, a.stream_waves);
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
    waves = waves < 1 ? 1 : (waves > a.stream_waves ? a.stream_waves : waves);
    if (w < a.rows && win.ctx[w] == 0) {  // an empty row reads zeros (all its queries); no slice visits it
      const int per_row = a.query_len * a.n_heads * a.head_dim;
      for (int idx = lane; idx < per_row; idx += kWave)
        store_out(a.out, a.out_dtype, (size_t)w * per_row + idx, 0.f);
      if (a.slot_new) append_empty_row<uint16_t>(a, w, lane, kWave);
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

  // this lane's column: query lr / group of the row's chunk (the only one for
  // a one-query read), head kv head * group + lr % group
  const bool colv = lr < a.cols;
  const int qcol = colv ? lr / a.group : a.query_len - 1;
  auto load_q = [&](const Cursor &c, bf16x8_t *qb) {
#pragma unroll
    for (int i = 0; i < KS; ++i)
      qb[i] = colv ? ld_bf16x8(a.q, (stream_out_row(a, c.kvh, c.r, lr) * HD + (4 * i + lg) * 8) * 2) : zero_bf16x8();
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
  Append<HD> ap;
  append_load<HD>(ap, a, c0, lr, lg);

  bf16x8_t kc[2][KS], vc[DT];
  const uint32_t v_lane = v_tile_lane<HD>(lr, lg);
  while (true) {
    // The staged group (and the next group's block ids) must have landed.
    // The compiler does not order LDS reads after direct-to-LDS loads by
    // itself, so the wait is explicit and fenced against reordering.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    asm volatile("" ::: "memory");
    if (ap.pending) append_apply<HD, BS>(ap, a, c0, s_k, s_v, lane, lr, lg);
    asm volatile("" ::: "memory");
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int i = 0; i < KS; ++i) kc[tt][i] = __builtin_bit_cast(bf16x8_t, s_k[(tt * KS + i) * kWave + lane]);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) vc[dt] = v_tile_frag<HD>(s_v, v_lane, dt);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the buffer may be refilled
    asm volatile("" ::: "memory");
    const bool last_group = c0.idx + 1 >= total;
    GroupIds ids2;
    if (!last_group) {
      ids2 = load_ids<BS>(a, c2, lr, lg);
      stage_group<HD, BS>(s_k, s_v, a, c1, ids1, lane, lr, lg);
      append_load<HD>(ap, a, c1, lr, lg);
    }
    f32x4_t sacc[2];
    group_scores<HD>(kc, qb, sacc);
    // causal inside a chunk: query qcol sees positions below n - query_len + qcol + 1
    const int cend = max(c0.n - a.query_len + qcol + 1, 0);
    group_softmax_pv<HD>(sacc, vc, acc, m, l, cscale, cend, c0.n, c0.j * kGroupPositions, lg);
    if (c0.j == c0.ng - 1 || last_group) segment_end<HD>(a, L, c0, w, acc, m, l, lr, lg);
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
// Matrix-core layout (v_mfma_f32_32x32x16_bf16, which on gfx950 sustains
// twice the rate of the 16x16x32 shape):
//   scores  S^T[32 positions][32 columns] = K Q^T, hd in k-steps of 16;
//   output  O^T[32 hd][32 columns] += V^T P^T, positions in k-steps of 16.
// A column is a (query, head) pair: 32 / group queries of one kv head's group
// per tile.  Row m of the score tile holds position sigma(m) of the group,
// chosen so that the 16 scores a lane receives are, in register order, the
// 16 positions it must supply as its P operand (8 per k-step): lane half h
// gets positions 8h .. 8h+7 and 16+8h .. 16+8h+7.  The softmax therefore
// needs no data movement between the two products, and a column's max is
// one exchange between lanes l and l ^ 32.
//
// A workgroup of NW waves serves one (position partition, query block, kv
// head, row); wave w owns one 32-column tile, so a block covers NW * 32 /
// group queries and every K/V byte staged for the block feeds all of them.
// The 32-position groups of the partition (only those some query of the
// block can see) go through a ring of multi_ring(NW) LDS group buffers
// filled by direct-to-LDS loads, each wave loading its share of every group.
// Groups are consumed two per step: one barrier per step publishes the pair
// and frees the pair before it for refilling.  Rows of one partition are
// written directly; longer rows leave per-partition (max, sum, acc) for
// decode_multi_merge.
// ---------------------------------------------------------------------------
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// Position (0..31, within the group) of score-tile row m.
__device__ __forceinline__ int multi_row_pos(int m) {
  const int a = m >> 3, b = (m >> 2) & 1, c = m & 3;
  return 16 * (a >> 1) + 8 * b + 4 * (a & 1) + c;
}

// K of a staged group is kept as it lies in the pool: K slot s is the
// contiguous 1 KB of positions RPS s .. RPS s + RPS - 1 (RPS = 64 / CPR rows
// of CPR = head_dim / 8 16-byte chunks), so every load reads whole cache
// lines.  Within a slot, chunk `col` of row p (group-relative position) sits
// at chunk CPR (p % RPS) + (col ^ kswz(p)): the XOR spreads the 16 lanes of
// one fragment read over distinct LDS banks.
template <int HD>
__device__ __forceinline__ int kswz(int p) {
  return HD == 128 ? (p & 15) : ((p >> 1) & 7);
}

// V of a staged group is kept the same way, rows of positions in 1 KB slots
// after the K slots, with its own XOR vswz32(p): the P.V operand of lane
// (lr, h) is hd 32 dt + lr at positions 16 kk + 8 h .. + 8, read transposed
// (lds_read_tr16) from rows p and p + 4; the XOR spreads every such read
// over distinct banks and leaves bit 2 of p alone.
template <int HD>
__device__ __forceinline__ int vswz32(int p) {
  const int b0 = p & 1, b1 = (p >> 1) & 1, b3 = (p >> 3) & 1, b4 = (p >> 4) & 1;
  return HD == 128 ? (4 * (b0 ^ b3) | 10 * b1) : ((4 * b0) ^ (6 * b1) ^ (4 * b3) ^ (2 * b4));
}

// LDS uint4 index, within a staged group, of this lane's K fragment for
// k-step ks: position sigma(lane % 32), hd 16 ks + 8 (lane / 32) .. + 8.
template <int HD>
__device__ __forceinline__ int multi_kfrag(int ks, int lane) {
  constexpr int CPR = HD / 8, RPS = 64 / CPR;
  const int p = multi_row_pos(lane & 31), col = 2 * ks + (lane >> 5);
  return (p / RPS) * kWave + CPR * (p % RPS) + (col ^ kswz<HD>(p));
}

// Four entries of an LDS int table, read and waited for in one asm block.
// The compiler's wait insertion cannot tell these reads from the
// direct-to-LDS loads still in flight into the ring buffers, and would drain
// all of those first; the table is written once, before a barrier, and never
// by a direct-to-LDS load.
__device__ __forceinline__ void lds_read4(const int32_t *table, int i0, int i1, int i2, int i3, int32_t &x0,
                                          int32_t &x1, int32_t &x2, int32_t &x3) {
  const __attribute__((address_space(3))) int32_t *t = (const __attribute__((address_space(3))) int32_t *)table;
  const uint32_t a0 = (uint32_t)(uintptr_t)(t + i0), a1 = (uint32_t)(uintptr_t)(t + i1),
                 a2 = (uint32_t)(uintptr_t)(t + i2), a3 = (uint32_t)(uintptr_t)(t + i3);
  asm volatile(
      "ds_read_b32 %0, %4\n\t"
      "ds_read_b32 %1, %5\n\t"
      "ds_read_b32 %2, %6\n\t"
      "ds_read_b32 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(x0), "=&v"(x1), "=&v"(x2), "=&v"(x3)
      : "v"(a0), "v"(a1), "v"(a2), "v"(a3)
      : "memory");
}

// Block id of the j-th block a group touches (j < 32 / BS), by selects.
template <int BS>
__device__ __forceinline__ size_t group_block(int j, int32_t id0, int32_t id1, int32_t id2, int32_t id3) {
  int32_t b = id0;
  if constexpr (BS < 32) b = j >= 1 ? id1 : b;
  if constexpr (BS < 16) {
    b = j >= 2 ? id2 : b;
    b = j >= 3 ? id3 : b;
  }
  return (size_t)b;
}

// Stage one group: this wave's share of the NSLOT 1 KB slots.  K and V slots
// are contiguous runs of rows of the K and V tiles (see kswz, vswz32).
// Positions past `last` read position `last`.  id0 .. id3 are the block ids
// of the group's (up to four) blocks.
template <int HD, int BS, int NW>
__device__ __forceinline__ void stage_multi_ids(uint4 *st, const DecodeArgs &a, int32_t id0, int32_t id1, int32_t id2,
                                                int32_t id3, int kvh, int t0, int last, int wave, int lane) {
  constexpr int KS = HD / 16, NSLOT = HD / 8, SPW = NSLOT / NW, CPR = HD / 8, RPS = 64 / CPR;
  constexpr int LOG2_BS = BS == 8 ? 3 : (BS == 16 ? 4 : 5);
  constexpr int bmask = BS - 1;
  const int tb0 = t0 >> LOG2_BS;
#pragma unroll
  for (int x = 0; x < SPW; ++x) {
    const int s = wave + NW * x;  // wave-uniform slot
    const bool is_k = s < KS;
    const int p = RPS * (is_k ? s : s - KS) + lane / CPR, t = min(t0 + p, last);
    const int col = (lane % CPR) ^ (is_k ? kswz<HD>(p) : vswz32<HD>(p));
    const size_t bk = group_block<BS>((t >> LOG2_BS) - tb0, id0, id1, id2, id3);
    const char *src = static_cast<const char *>(is_k ? a.k_pool : a.v_pool) +
                      ((((bk * a.n_kv_heads + kvh) << LOG2_BS) + (t & bmask)) * HD + 8 * col) * 2;
    __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1))) *)src,
                                     (void __attribute__((address_space(3))) *)(st + s * kWave), 16, 0,
                                     kMultiLoadPolicy);
  }
}

// The same, reading the group's block ids from s_blk (entries from block
// blk0 on, nblk of them) first.
template <int HD, int BS, int NW>
__device__ __forceinline__ void stage_multi(uint4 *st, const DecodeArgs &a, const int32_t *s_blk, int blk0, int nblk,
                                            int kvh, int t0, int last, int wave, int lane) {
  constexpr int LOG2_BS = BS == 8 ? 3 : (BS == 16 ? 4 : 5);
  const int gb = (t0 >> LOG2_BS) - blk0;
  int32_t id0, id1, id2, id3;
  lds_read4(s_blk, gb, min(gb + 1, nblk - 1), min(gb + 2, nblk - 1), min(gb + 3, nblk - 1), id0, id1, id2, id3);
  stage_multi_ids<HD, BS, NW>(st, a, id0, id1, id2, id3, kvh, t0, last, wave, lane);
}

// Entries i0 .. i0 + N - 1 of an LDS int table (N = 4, 8 or 16), read in
// pairs and waited for in one asm block, like lds_read4.  The table must
// hold N - 1 entries past any i0 this is called with.
typedef int32_t i32x2_t __attribute__((ext_vector_type(2)));
template <int N>
__device__ __forceinline__ void lds_read_run(const int32_t *table, int i0, int32_t (&x)[N]) {
  static_assert(N == 4 || N == 8 || N == 16, "four groups of 32 positions in blocks of 32, 16 or 8");
  const uint32_t a0 = (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) int32_t *)table + i0);
  i32x2_t v[N / 2];
  if constexpr (N == 4) {
    asm volatile(
        "ds_read2_b32 %0, %2 offset0:0 offset1:1\n\t"
        "ds_read2_b32 %1, %2 offset0:2 offset1:3\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1])
        : "v"(a0)
        : "memory");
  } else if constexpr (N == 8) {
    asm volatile(
        "ds_read2_b32 %0, %4 offset0:0 offset1:1\n\t"
        "ds_read2_b32 %1, %4 offset0:2 offset1:3\n\t"
        "ds_read2_b32 %2, %4 offset0:4 offset1:5\n\t"
        "ds_read2_b32 %3, %4 offset0:6 offset1:7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
        : "v"(a0)
        : "memory");
  } else {
    asm volatile(
        "ds_read2_b32 %0, %8 offset0:0 offset1:1\n\t"
        "ds_read2_b32 %1, %8 offset0:2 offset1:3\n\t"
        "ds_read2_b32 %2, %8 offset0:4 offset1:5\n\t"
        "ds_read2_b32 %3, %8 offset0:6 offset1:7\n\t"
        "ds_read2_b32 %4, %8 offset0:8 offset1:9\n\t"
        "ds_read2_b32 %5, %8 offset0:10 offset1:11\n\t"
        "ds_read2_b32 %6, %8 offset0:12 offset1:13\n\t"
        "ds_read2_b32 %7, %8 offset0:14 offset1:15\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]), "=&v"(v[7])
        : "v"(a0)
        : "memory");
  }
#pragma unroll
  for (int i = 0; i < N / 2; ++i) {
    x[2 * i] = v[i][0];
    x[2 * i + 1] = v[i][1];
  }
}

// Block-id table entries past the last a segment can use: four groups' ids
// are read in one run from the first group's, whichever of them exist.
constexpr int kMultiBlkPad = 16;

// Per-lane parts of a group's staging addresses for one (kv head, row):
// for this wave's slot x, the byte address of its lane's 16 bytes in block
// 0 of the pool (`base`), and which of the group's blocks holds its
// position (`j`).  For a group that lies wholly before the row's end, the
// load address is then base + block id x the pool's block stride.
template <int HD, int NW>
struct MultiStageLane {
  uint64_t base[HD / 8 / NW];
  int j[HD / 8 / NW];
};

template <int HD, int BS, int NW>
__device__ __forceinline__ MultiStageLane<HD, NW> multi_stage_lane(const DecodeArgs &a, int kvh, int wave, int lane) {
  constexpr int KS = HD / 16, SPW = HD / 8 / NW, CPR = HD / 8, RPS = 64 / CPR;
  constexpr int LOG2_BS = BS == 8 ? 3 : (BS == 16 ? 4 : 5);
  MultiStageLane<HD, NW> L;
#pragma unroll
  for (int x = 0; x < SPW; ++x) {
    const int s = wave + NW * x;
    const bool is_k = s < KS;
    const int p = RPS * (is_k ? s : s - KS) + lane / CPR;
    const int col = (lane % CPR) ^ (is_k ? kswz<HD>(p) : vswz32<HD>(p));
    L.base[x] = (uint64_t)(uintptr_t)(is_k ? a.k_pool : a.v_pool) +
                ((((uint64_t)kvh << LOG2_BS) + (uint64_t)(p & (BS - 1))) * HD + 8 * col) * 2;
    L.j[x] = p >> LOG2_BS;
  }
  return L;
}

// stage_multi_ids for a group wholly before the row's end (no position is
// clamped), from the per-lane parts.
template <int HD, int BS, int NW>
__device__ __forceinline__ void stage_multi_fast(uint4 *st, const DecodeArgs &a, const MultiStageLane<HD, NW> &L,
                                                 int32_t id0, int32_t id1, int32_t id2, int32_t id3, int wave) {
  constexpr int SPW = HD / 8 / NW;
  const uint32_t stride = (uint32_t)a.n_kv_heads * (uint32_t)(BS * HD * 2);  // bytes per pool block
#pragma unroll
  for (int x = 0; x < SPW; ++x) {
    const int s = wave + NW * x;
    const uint32_t bk = (uint32_t)group_block<BS>(L.j[x], id0, id1, id2, id3);
    const char *src = (const char *)(uintptr_t)(L.base[x] + (uint64_t)bk * stride);
    __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1))) *)src,
                                     (void __attribute__((address_space(3))) *)(st + s * kWave), 16, 0,
                                     kMultiLoadPolicy);
  }
}

// Per-wave state of the multi-query read: this lane's column and its
// softmax state.  acc[dt] register j is output hd 32 dt + 8 (j / 4) +
// 4 (lane / 32) + j % 4 of the column.
template <int HD>
struct MultiState {
  bf16x8_t qb[HD / 16];  // q of the column, hd 16 ks + 8 (lane / 32) .. + 8
  int col_end;           // positions the column sees (INT_MAX: not a query)
  int min_end;           // wave-uniform: the least col_end of a query in the tile
  float m, l;            // reference max (log2 units) and this lane's part of the sum
  f32x16_t acc[HD / 32];
};

// Headroom, in log2 units, of the lazy rescaling: a column's reference max
// moves only when a group's max exceeds it by more than this, so its weights
// stay below 2^8 and the accumulators are rescaled for a few groups of a
// partition rather than for most of them.  The result is the same softmax:
// numerator and denominator share the reference.
constexpr float kLazyRescale = 8.f;

// 8 weights as RNE bf16 hi + lo pairs, packed for the B operand of the P.V
// product (hi + lo carries 16 significant bits).
__device__ __forceinline__ void split_bf16_hi_lo(const float *p, bf16x8_t &phi, bf16x8_t &plo) {
  uint32_t hw[4], lw[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f32x2_t v = {p[2 * i], p[2 * i + 1]};
    const uint32_t hb = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
    const f32x2_t r = {p[2 * i] - __builtin_bit_cast(float, hb << 16),
                       p[2 * i + 1] - __builtin_bit_cast(float, hb & 0xFFFF0000u)};
    hw[i] = hb;
    lw[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, bf16x2_t));
  }
  phi = __builtin_bit_cast(bf16x8_t, make_uint4(hw[0], hw[1], hw[2], hw[3]));
  plo = __builtin_bit_cast(bf16x8_t, make_uint4(lw[0], lw[1], lw[2], lw[3]));
}

// Raw scores of one group for the softmax statistics: register j holds
// position gbase + 16 (j / 8) + 8 h + j % 8.  Where the causal bound of some
// column falls in the group, positions the lane's column does not see become
// -inf; a group past the partition's last (`live` false) is all -inf.
template <int HD>
__device__ __forceinline__ void multi_raw(float (&raw)[16], const f32x16_t &sacc, const MultiState<HD> &S, int gbase,
                                          int h, bool live) {
#pragma unroll
  for (int j = 0; j < 16; ++j) raw[j] = sacc[j];
  if (!live || gbase + kGroupPositions > S.min_end) {
    const int lim = live ? S.col_end - gbase - 8 * h : 0;  // register j is seen iff 16 (j / 8) + j % 8 < lim
#pragma unroll
    for (int j = 0; j < 16; ++j) raw[j] = 16 * (j >> 3) + (j & 7) < lim ? raw[j] : -INFINITY;
  }
}

// V of one staged group, positions past the row end zeroed (they may hold
// NaN): vc[dt][kk] is hd rows 32 dt .., positions 16 kk + 8 h .. + 8.  In
// each 16 lanes, lanes 4r + q read row 16 kk + 8 h + r (then r + 4), hd
// 32 dt + 16 ((lane / 16) % 2) + 4 q .. + 3; lane i gets hd .. + i.
template <int HD>
__device__ __forceinline__ void multi_v(bf16x8_t (&vc)[HD / 32][2], const uint4 *buf, int gbase, int n, int lane) {
  constexpr int KS = HD / 16, DT = HD / 32;
  const void *vt = buf + KS * kWave;
  const int i16 = lane & 15, r = i16 >> 2, q = i16 & 3, h = lane >> 5, hs = (lane >> 4) & 1;
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const int p = 16 * kk + 8 * h + r;
    const uint32_t off = (uint32_t)(p * 2 * HD + 16 * ((2 * hs + (q >> 1)) ^ vswz32<HD>(p)) + 8 * (q & 1));
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const uint32_t o = off ^ (uint32_t)(64 * dt);
      const uint2 lo = lds_read_tr16(vt, o), hi = lds_read_tr16(vt, o + 8 * HD);
      vc[dt][kk] = __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
    }
  }
  if (gbase + kGroupPositions > n) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int nv = min(max(n - (gbase + 16 * kk + 8 * (lane >> 5)), 0), 8);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) vc[dt][kk] = keep_first(vc[dt][kk], nv);
    }
  }
}

template <int HD>
__device__ __forceinline__ void multi_pair_compute(MultiState<HD> &S, const uint4 *c0, const uint4 *c1,
                                                   const DecodeArgs &a, int g0, int k, int ng, int n, float cscale,
                                                   int lane);

// Groups k and k + 1 of the multi-query read (k even; k + 1 may lie past
// the partition's last group), from a ring of R = 4 group buffers.  Wait
// for both and publish them -- the barrier also says every wave is done
// with groups k - 2 and k - 1, whose buffers are then refilled with groups
// k + 2 and k + 3 -- then compute them (multi_pair_compute).  The ring's
// buffers are separate LDS arrays and each step names its four statically,
// so the compiler can tell the reads of these groups from the loads in
// flight into the others.
template <int HD, int BS, int NW, int R>
__device__ __forceinline__ void multi_pair(MultiState<HD> &S, const uint4 *c0, const uint4 *c1, uint4 *r0, uint4 *r1,
                                           const DecodeArgs &a, const int32_t *s_blk, int blk0, int nblk, int kvh, int g0,
                                           int k, int ng, int n, float cscale, bool active, int wave, int lane) {
  static_assert(R == 4, "the ring of eight steps by four groups (multi_quad)");
  // this wave's loads (groups k and k + 1: the ring holds no others) have landed
  __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0(0));
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  if (k + R - 2 < ng)
    stage_multi<HD, BS, NW>(r0, a, s_blk, blk0, nblk, kvh, (g0 + k + R - 2) * kGroupPositions, n - 1, wave, lane);
  if (k + R - 1 < ng)
    stage_multi<HD, BS, NW>(r1, a, s_blk, blk0, nblk, kvh, (g0 + k + R - 1) * kGroupPositions, n - 1, wave, lane);
  if (!active) return;
  multi_pair_compute<HD>(S, c0, c1, a, g0, k, ng, n, cscale, lane);
}

// Eight groups k .. k + 7 pass through a ring of R = 8 buffers four at a
// time: wait for all of this wave's loads (groups k .. k + 3, staged one
// step earlier) and publish them -- the barrier also says every wave is done
// with groups k - 4 .. k - 1 -- refill those four buffers with groups
// k + 4 .. k + 7, then compute groups k .. k + 3 as two pairs.  One wait and
// one barrier per four groups, and a step of computation to hide each load.
template <int HD, int BS, int NW>
__device__ __forceinline__ void multi_quad(MultiState<HD> &S, const uint4 *c0, const uint4 *c1, const uint4 *c2,
                                           const uint4 *c3, uint4 *r0, uint4 *r1, uint4 *r2, uint4 *r3,
                                           const DecodeArgs &a, const int32_t *s_blk, int blk0, int nblk, int kvh,
                                           int g0, int k, int ng, int n, float cscale, bool active, int wave,
                                           int lane, const MultiStageLane<HD, NW> &SL) {
  __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0(0));
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  uint4 *const r[4] = {r0, r1, r2, r3};
  if (k + 4 < ng) {
    // the four groups' block ids in one LDS round trip: IPG per group, from
    // the first group's first (entries of groups past the last are unused)
    constexpr int IPG = kGroupPositions / BS;
    constexpr int LOG2_BS = BS == 8 ? 3 : (BS == 16 ? 4 : 5);
    const int t4 = (g0 + k + 4) * kGroupPositions;
    int32_t ids[4 * IPG];
    lds_read_run<4 * IPG>(s_blk, (t4 >> LOG2_BS) - blk0, ids);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (k + 4 + i < ng) {
        const int j = IPG * i, t0 = t4 + i * kGroupPositions;
        const int32_t i0 = ids[j], i1 = ids[min(j + 1, 4 * IPG - 1)], i2 = ids[min(j + 2, 4 * IPG - 1)],
                      i3 = ids[min(j + 3, 4 * IPG - 1)];
        if (t0 + kGroupPositions <= n) stage_multi_fast<HD, BS, NW>(r[i], a, SL, i0, i1, i2, i3, wave);
        else stage_multi_ids<HD, BS, NW>(r[i], a, i0, i1, i2, i3, kvh, t0, n - 1, wave, lane);
      }
  }
  if (!active) return;
  multi_pair_compute<HD>(S, c0, c1, a, g0, k, ng, n, cscale, lane);
  if (k + 2 < ng) multi_pair_compute<HD>(S, c2, c3, a, g0, k + 2, ng, n, cscale, lane);
}

// Groups k and k + 1 from buffers c0 and c1, already published: the scores
// of both groups (two independent MFMA chains), one softmax update over
// their 64 positions (one max exchange, one rescale check) and the P.V
// products.
template <int HD>
__device__ __forceinline__ void multi_pair_compute(MultiState<HD> &S, const uint4 *c0, const uint4 *c1,
                                                   const DecodeArgs &a, int g0, int k, int ng, int n, float cscale,
                                                   int lane) {
  constexpr int KS = HD / 16, DT = HD / 32;
  const int h = lane >> 5;
  const bool two = k + 1 < ng;
  const int gb0 = (g0 + k) * kGroupPositions, gb1 = gb0 + kGroupPositions;
  // scores of both groups, k-step outermost: two independent chains (the
  // second group's is discarded when it does not exist)
  f32x16_t sc0, sc1;
#pragma unroll
  for (int j = 0; j < 16; ++j) sc0[j] = sc1[j] = 0.f;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int kf = multi_kfrag<HD>(ks, lane);
    sc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, c0[kf]), S.qb[ks], sc0, 0, 0, 0);
    sc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, c1[kf]), S.qb[ks], sc1, 0, 0, 0);
  }
  float raw0[16], raw1[16];
  multi_raw<HD>(raw0, sc0, S, gb0, h, true);
  multi_raw<HD>(raw1, sc1, S, gb1, h, two);
  // Does any score of this lane exceed its column's reference by more than
  // kLazyRescale?  With c > 0, raw > (m + kLazyRescale) / c is that test (up
  // to rounding at the threshold, which only lets a weight reach 2^8 times a
  // rounding error); it needs no data from other lanes.  The threshold is
  // -inf while the column has seen nothing.
  const float thr = (S.m + kLazyRescale) / cscale;
  bool over = false;
#pragma unroll
  for (int j = 0; j < 16; ++j) over |= (raw0[j] > thr) | (raw1[j] > thr);
  if (__any(over)) {  // rare after a partition's first pair
    // c > 0: the column max of the raw dot products, times c, is the max of
    // its scores; move the reference of the columns that outgrew it
    float mx = fmaxf(raw0[0], raw1[0]);
#pragma unroll
    for (int j = 1; j < 16; ++j) mx = fmaxf(mx, fmaxf(raw0[j], raw1[j]));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mxs = mx * cscale;  // -inf when the column sees nothing here
    const bool up = mxs > S.m + kLazyRescale;
    const float alpha = up ? exp2_fast(S.m - mxs) : 1.f;  // 0 from -inf
    S.m = up ? mxs : S.m;
    S.l *= alpha;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) S.acc[dt] *= alpha;
  }
  // Weights (below 2^kLazyRescale), this lane's part of the row sum, hi/lo
  // split, then the P.V products.  A -inf score gives weight 0; a column that
  // has seen nothing yet takes 0 as its reference.  For a bf16 output the lo
  // half is skipped: P rounded to bf16 moves the result by at most 2^-9
  // max|V|, below the output's own rounding for |V| ~ |out|, and saves a
  // third of the matrix-core work.  An fp32 output keeps both halves.
  const float mref = S.m == -INFINITY ? 0.f : S.m;
  float p0[16], p1[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    p0[j] = exp2_fast(fmaf(raw0[j], cscale, -mref));
    p1[j] = exp2_fast(fmaf(raw1[j], cscale, -mref));
  }
  float ps = 0.f;
#pragma unroll
  for (int j = 0; j < 16; j += 2) ps += (p0[j] + p0[j + 1]) + (p1[j] + p1[j + 1]);
  S.l += ps;
  bf16x8_t phi0[2], plo0[2], phi1[2], plo1[2];
  split_bf16_hi_lo(p0, phi0[0], plo0[0]);
  split_bf16_hi_lo(p0 + 8, phi0[1], plo0[1]);
  split_bf16_hi_lo(p1, phi1[0], plo1[0]);
  split_bf16_hi_lo(p1 + 8, phi1[1], plo1[1]);
  bf16x8_t vc[DT][2];
  multi_v<HD>(vc, c0, gb0, n, lane);
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      S.acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vc[dt][kk], phi0[kk], S.acc[dt], 0, 0, 0);
  const bool exact = a.out_dtype == kF32;
  if (exact) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        S.acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vc[dt][kk], plo0[kk], S.acc[dt], 0, 0, 0);
  }
  if (two) {
    multi_v<HD>(vc, c1, gb1, n, lane);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        S.acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vc[dt][kk], phi1[kk], S.acc[dt], 0, 0, 0);
    if (exact) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          S.acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vc[dt][kk], plo1[kk], S.acc[dt], 0, 0, 0);
    }
  }
}

// A column's output row (hd values at `orow`), from its accumulators scaled
// by inv: register j of acc[dt] is hd 32 dt + 8 (j / 4) + 4 h + j % 4, so
// each quad of registers is four consecutive hd values, stored as one
// 16-byte (fp32) or 8-byte (bf16, round to nearest even) store.
template <int HD>
__device__ __forceinline__ void multi_store_row(const DecodeArgs &a, size_t orow, const f32x16_t *acc, float inv,
                                                int h) {
#pragma unroll
  for (int dt = 0; dt < HD / 32; ++dt)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const size_t o = orow + 32 * dt + 8 * q4 + 4 * h;
      const float x0 = acc[dt][4 * q4] * inv, x1 = acc[dt][4 * q4 + 1] * inv;
      const float x2 = acc[dt][4 * q4 + 2] * inv, x3 = acc[dt][4 * q4 + 3] * inv;
      if (a.out_dtype == kF32) {
        *reinterpret_cast<f32x4_t *>(static_cast<float *>(a.out) + o) = f32x4_t{x0, x1, x2, x3};
      } else {
        const uint32_t w0 = f32_to_bf16_rne(x0) | ((uint32_t)f32_to_bf16_rne(x1) << 16);
        const uint32_t w1 = f32_to_bf16_rne(x2) | ((uint32_t)f32_to_bf16_rne(x3) << 16);
        *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(a.out) + o) = make_uint2(w0, w1);
      }
    }
}

// c > 0 for the statistics; a zero scale becomes 1e-30 (every weight still
// exp2(0) = 1) and a NaN scale stays NaN
__device__ __forceinline__ float multi_cscale(const DecodeArgs &a) {
  const float cs = fabsf(a.scale) * kLog2e;
  return cs < 1e-30f ? 1e-30f : cs;
}

// Groups g0 .. g0 + ng - 1 of (row, kv head) through the ring: the prologue
// stages the first four (a ring of eight) or two (a ring of four), then the
// steps (multi_quad or multi_pair).  s_blk holds the block ids from block
// blk0 on (nblk of them) and has been published; on return every staged
// load has been consumed, but other waves may still be reading the ring's
// last buffers.
template <int HD, int BS, int NW>
__device__ __forceinline__ void multi_run(MultiState<HD> &S, uint4 *s_b0, uint4 *s_b1, uint4 *s_b2, uint4 *s_b3,
                                          uint4 *s_b4, uint4 *s_b5, uint4 *s_b6, uint4 *s_b7, const DecodeArgs &a,
                                          const int32_t *s_blk, int blk0, int nblk, int kvh, int g0, int ng, int n,
                                          float cscale, bool active, int wave, int lane) {
  constexpr int R = multi_ring(NW);
  const int last = n - 1;
  auto stage = [&](uint4 *buf, int j) {
    if (j < ng) stage_multi<HD, BS, NW>(buf, a, s_blk, blk0, nblk, kvh, (g0 + j) * kGroupPositions, last, wave, lane);
  };
  stage(s_b0, 0);
  stage(s_b1, 1);
  if constexpr (R == 8) {
    stage(s_b2, 2);
    stage(s_b3, 3);
    const MultiStageLane<HD, NW> SL = multi_stage_lane<HD, BS, NW>(a, kvh, wave, lane);
    for (int k = 0; k < ng; k += 8) {
      multi_quad<HD, BS, NW>(S, s_b0, s_b1, s_b2, s_b3, s_b4, s_b5, s_b6, s_b7, a, s_blk, blk0, nblk, kvh, g0, k, ng,
                             n, cscale, active, wave, lane, SL);
      if (k + 4 >= ng) break;
      multi_quad<HD, BS, NW>(S, s_b4, s_b5, s_b6, s_b7, s_b0, s_b1, s_b2, s_b3, a, s_blk, blk0, nblk, kvh, g0, k + 4,
                             ng, n, cscale, active, wave, lane, SL);
    }
  } else {
    for (int k = 0; k < ng; k += 4) {
      multi_pair<HD, BS, NW, R>(S, s_b0, s_b1, s_b2, s_b3, a, s_blk, blk0, nblk, kvh, g0, k, ng, n, cscale, active, wave,
                                lane);
      if (k + 2 >= ng) break;
      multi_pair<HD, BS, NW, R>(S, s_b2, s_b3, s_b0, s_b1, a, s_blk, blk0, nblk, kvh, g0, k + 2, ng, n, cscale, active,
                                wave, lane);
    }
  }
}

template <int HD, int BS, int NW>
__global__ __launch_bounds__(NW * kWave) __attribute__((amdgpu_waves_per_eu(NW / 4 > 1 ? NW / 4 : 1, 2))) void
decode_multi(DecodeArgs a) {
  constexpr int KS = HD / 16, DT = HD / 32, NSLOT = HD / 8;
  static_assert(NSLOT % NW == 0, "every wave stages the same number of slots");
  constexpr int R = multi_ring(NW);  // group buffers in the ring
  constexpr int STAGE = NSLOT * kWave;  // uint4 per staged group
  constexpr int LOG2_BS = BS == 8 ? 3 : (BS == 16 ? 4 : 5);
  __shared__ uint4 s_b0[STAGE], s_b1[STAGE], s_b2[STAGE], s_b3[STAGE];
  __shared__ uint4 s_b4[R > 4 ? STAGE : 1], s_b5[R > 4 ? STAGE : 1], s_b6[R > 4 ? STAGE : 1], s_b7[R > 4 ? STAGE : 1];
  __shared__ int32_t s_blk[kMultiMaxPartition / 8 + kMultiBlkPad];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform, kept in a scalar
  const int lane = threadIdx.x & (kWave - 1), lr = lane & 31, h = lane >> 5;
  const int G = a.group, Q = a.query_len, QB = a.q_per_tile, P = a.partition_tokens;
  long long u = blockIdx.x;  // kv head fastest (spread over XCDs), then row, query block, partition
  const int kvh = (int)(u % a.n_kv_heads);
  u /= a.n_kv_heads;
  const int r = (int)(u % a.rows);
  u /= a.rows;
  const int qblk = (int)(u % a.q_blocks);
  const int part = (int)(u / a.q_blocks);
  const int cap = a.max_blocks_per_row * a.block_size;
  const int pos0 = part * P;  // < cap: part < max_parts
  const int blk0 = pos0 >> LOG2_BS;  // pos0 is a multiple of the block size
  // Start-up: the row length, the partition's slice of the block table (all
  // of it up to the table's width, whatever the length) and this lane's q
  // are independent loads, issued together.
  const int n_raw = a.context_lens[r];
  const int nblk_all = (min(pos0 + P, cap) - pos0) >> LOG2_BS;
  int32_t btab[kMultiMaxPartition / 8 / (NW * kWave) + 1];
#pragma unroll
  for (int x = 0; x * NW * kWave < kMultiMaxPartition / 8; ++x) {
    const int i = threadIdx.x + x * NW * kWave;
    btab[x] = i < nblk_all ? a.block_table[(size_t)r * a.max_blocks_per_row + blk0 + i] : 0;
  }
  // this lane's column: query q0 + lr / G, head kvh * G + lr % G of tile `wave`
  MultiState<HD> S;
  const int q_first = qblk * NW * QB;
  const int q0 = q_first + wave * QB;
  const int qi = q0 + lr / G, hi = lr % G;
  const bool colv = lr < QB * G && qi < Q;
  const uint32_t qsign = a.scale < 0.f ? 0x80008000u : 0u;  // fold a negative scale into q (exact)
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const bf16x8_t x = colv ? ld_bf16x8(a.q, ((((size_t)r * Q + qi) * a.n_heads + kvh * G + hi) * HD + 16 * ks + 8 * h) * 2)
                            : zero_bf16x8();
    uint4 w = __builtin_bit_cast(uint4, x);
    w.x ^= qsign;
    w.y ^= qsign;
    w.z ^= qsign;
    w.w ^= qsign;
    S.qb[ks] = __builtin_bit_cast(bf16x8_t, w);
  }
  const int n = n_raw < 0 ? 0 : (n_raw > cap ? cap : n_raw);
  const int nparts = n > 0 ? (n + P - 1) / P : 1;
  if (part >= nparts) return;  // the whole workgroup
  const int q_last = min(Q - 1, q_first + NW * QB - 1);
  const int unit_end = max(min(pos0 + P, n - Q + q_last + 1), pos0);  // some query of the block sees below
  const int g0 = pos0 / kGroupPositions, ng = (unit_end + kGroupPositions - 1) / kGroupPositions - g0;
  const int64_t nb1 = a.num_blocks - 1;
#pragma unroll
  for (int x = 0; x * NW * kWave < kMultiMaxPartition / 8; ++x) {
    const int i = threadIdx.x + x * NW * kWave;
    if (i < nblk_all) s_blk[i] = btab[x] < 0 ? 0 : (btab[x] > nb1 ? (int32_t)nb1 : btab[x]);
  }
  S.col_end = colv ? max(n - Q + qi + 1, 0) : INT_MAX;
  S.min_end = q0 < Q ? max(n - Q + q0 + 1, 0) : INT_MAX;
  S.m = -INFINITY;
  S.l = 0.f;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int j = 0; j < 16; ++j) S.acc[dt][j] = 0.f;
  const bool active = q0 < Q;  // some column of this wave is a query
  __syncthreads();  // s_blk is written
  multi_run<HD, BS, NW>(S, s_b0, s_b1, s_b2, s_b3, s_b4, s_b5, s_b6, s_b7, a, s_blk, blk0, nblk_all, kvh, g0, ng, n,
                        multi_cscale(a), active, wave, lane);
  const float lt = S.l + __shfl_xor(S.l, 32);
  if (!colv) return;
  const size_t vrow_head = ((size_t)r * Q + qi) * a.n_heads + kvh * G + hi;
  if (nparts == 1) {
    multi_store_row<HD>(a, vrow_head * HD, S.acc, lt > 0.f ? 1.f / lt : 0.f, h);  // 0: a query before the history
  } else {
    const WsLayout W = ws_layout(a.rows * Q, a.n_heads, a.max_parts, HD);
    const size_t slot = vrow_head * a.max_parts + part;
    float *accp = a.ws + W.acc_off + slot * HD;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *reinterpret_cast<f32x4_t *>(accp + 32 * dt + 8 * q4 + 4 * h) =
            f32x4_t{S.acc[dt][4 * q4], S.acc[dt][4 * q4 + 1], S.acc[dt][4 * q4 + 2], S.acc[dt][4 * q4 + 3]};
    if (h == 0) {
      a.ws[W.m_off + slot] = S.m;
      a.ws[W.l_off + slot] = lt;
    }
  }
}

// Combine the partials of one (row, query, head) of the multi-query read,
// 32 lanes: lane j reads partial j's (m, l) (m_at, l_at); M = max m_j over
// partials that saw something, w_j = 2^(m_j - M) (0 for those that did
// not), L = sum l_j w_j, and each lane sums w_j acc_j over its four hd
// values (acc_at(j): partial j's hd row), the loads of several partials in
// flight at once.  out = O / L, or zeros when nothing was visible.
template <typename MAt, typename LAt, typename AccAt>
__device__ __forceinline__ void merge_tuple(const DecodeArgs &a, int nparts, int sub, size_t out_base, MAt m_at,
                                            LAt l_at, AccAt acc_at) {
  const int HD = a.head_dim;
  float M = -INFINITY;  // the general path's maximum (more than four partials)
  for (int j0 = 0; j0 < nparts && nparts > 4; j0 += 32)
    if (j0 + sub < nparts) M = fmaxf(M, m_at(j0 + sub));
#pragma unroll
  for (int x = 16; x >= 1; x >>= 1) M = fmaxf(M, __shfl_xor(M, x, 32));
  const int d = 4 * sub;  // this lane's hd values d .. d + 3
  float L = 0.f;
  f32x4_t O = {0.f, 0.f, 0.f, 0.f};
  if (nparts <= 4) {
    // every load in one round trip: m and l of partial `sub`, and this
    // lane's acc values of all partials (none depends on the maximum);
    // then the same arithmetic, in the same order, as the general loop
    const bool own = sub < nparts;
    const float mj = own ? m_at(sub) : -INFINITY;
    const float lj = own ? l_at(sub) : 0.f;
    f32x4_t x[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      x[u] = u < nparts && d < HD ? *reinterpret_cast<const f32x4_t *>(acc_at(u) + d) : f32x4_t{0.f, 0.f, 0.f, 0.f};
    float M = mj;
#pragma unroll
    for (int x2 = 16; x2 >= 1; x2 >>= 1) M = fmaxf(M, __shfl_xor(M, x2, 32));
    float w = 0.f;
    if (own && M != -INFINITY) {
      w = mj == -INFINITY ? 0.f : exp2_fast(mj - M);
      L = fmaf(lj, w, L);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (u < nparts) O += __shfl(w, u, 32) * x[u];
  }
  for (int j0 = 0; j0 < nparts && nparts > 4; j0 += 32) {
    float w = 0.f;
    if (j0 + sub < nparts && M != -INFINITY) {
      const float mj = m_at(j0 + sub);
      w = mj == -INFINITY ? 0.f : exp2_fast(mj - M);
      L = fmaf(l_at(j0 + sub), w, L);
    }
    const int cnt = min(32, nparts - j0);
    int t = 0;
    for (; t + 4 <= cnt; t += 4) {  // four partials' loads in flight
      f32x4_t x[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        x[u] = d < HD ? *reinterpret_cast<const f32x4_t *>(acc_at(j0 + t + u) + d) : f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < 4; ++u) O += __shfl(w, t + u, 32) * x[u];
    }
    for (; t < cnt; ++t) {
      const f32x4_t x = d < HD ? *reinterpret_cast<const f32x4_t *>(acc_at(j0 + t) + d) : f32x4_t{0.f, 0.f, 0.f, 0.f};
      O += __shfl(w, t, 32) * x;
    }
  }
#pragma unroll
  for (int x = 16; x >= 1; x >>= 1) L += __shfl_xor(L, x, 32);
  if (d < HD) {  // four consecutive hd values: one 16-byte (fp32) or 8-byte (bf16) store
    const float inv = L > 0.f ? 1.f / L : 0.f;
    const float y0 = L > 0.f ? O[0] * inv : 0.f, y1 = L > 0.f ? O[1] * inv : 0.f;
    const float y2 = L > 0.f ? O[2] * inv : 0.f, y3 = L > 0.f ? O[3] * inv : 0.f;
    if (a.out_dtype == kF32) {
      *reinterpret_cast<f32x4_t *>(static_cast<float *>(a.out) + out_base + d) = f32x4_t{y0, y1, y2, y3};
    } else {
      const uint32_t w0 = f32_to_bf16_rne(y0) | ((uint32_t)f32_to_bf16_rne(y1) << 16);
      const uint32_t w1 = f32_to_bf16_rne(y2) | ((uint32_t)f32_to_bf16_rne(y3) << 16);
      *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(a.out) + out_base + d) = make_uint2(w0, w1);
    }
  }
}

// Combine the partitions of the multi-query read (merge_tuple over the
// partition workspace), kMultiMergeTuples (row, query, head) tuples per
// 256-thread workgroup.
constexpr int kMultiMergeTuples = 8;
__global__ __launch_bounds__(256) void decode_multi_merge(DecodeArgs a) {
  const int Q = a.query_len, HD = a.head_dim;
  const int sub = threadIdx.x & 31;
  const size_t vh = (size_t)blockIdx.x * kMultiMergeTuples + (threadIdx.x >> 5);  // (row * Q + query) * n_heads + head
  if (vh >= (size_t)a.rows * Q * a.n_heads) return;  // a whole 32-lane half
  const int r = (int)(vh / ((size_t)Q * a.n_heads));
  const int cap = a.max_blocks_per_row * a.block_size;
  int n = a.context_lens[r];
  n = n < 0 ? 0 : (n > cap ? cap : n);
  const int nparts = n > 0 ? (n + a.partition_tokens - 1) / a.partition_tokens : 1;
  if (nparts <= 1) return;  // written directly by decode_multi
  const WsLayout W = ws_layout(a.rows * Q, a.n_heads, a.max_parts, HD);
  const size_t s0 = vh * a.max_parts;
  merge_tuple(
      a, nparts, sub, vh * HD, [&](int j) { return a.ws[W.m_off + s0 + j]; },
      [&](int j) { return a.ws[W.l_off + s0 + j]; },
      [&](int j) { return (const float *)(a.ws + W.acc_off + (s0 + j) * HD); });
}

// ---------------------------------------------------------------------------
// Balanced multi-query read: one query block covers all the queries of a
// (row, kv head) and the batch has at most kWindowRows rows.  The groups of
// 32 positions of every (kv head, row), in that order -- the one-query
// read's stream -- are cut into at most a.stream_waves equal slices, one per
// persistent workgroup of NW waves, so that every workgroup does the same
// work whatever the length mix.  A workgroup walks the segments of its slice
// (runs of one (kv head, row)) through the ring of multi_run, restarting it
// between segments.  A (kv head, row) whole inside the slice is written to
// out; a piece of one cut by a slice boundary leaves its partial (m, l and
// acc for every column) in its slot (stream_piece_slot), which
// decode_multi_stream_merge combines.  A segment spans at most
// kMultiMaxPartition positions (the size of the block-id table); a longer
// run of one (kv head, row) is read in several and keeps its softmax state.
// ---------------------------------------------------------------------------
// Stream length of a (kv head, row) of n positions in the balanced multi-
// query read: its groups, behind kMultiSegmentCost groups of no work.
__device__ __forceinline__ int multi_stream_groups(int n) {
  return n > 0 ? (n + kGroupPositions - 1) / kGroupPositions + kMultiSegmentCost : 0;
}

template <int HD, int BS, int NW>
__global__ __launch_bounds__(NW * kWave) __attribute__((amdgpu_waves_per_eu(NW / 4 > 1 ? NW / 4 : 1, 2))) void
decode_multi_stream(DecodeArgs a) {
  constexpr int KS = HD / 16, DT = HD / 32, NSLOT = HD / 8;
  constexpr int R = multi_ring(NW);
  constexpr int STAGE = NSLOT * kWave;
  constexpr int LOG2_BS = BS == 8 ? 3 : (BS == 16 ? 4 : 5);
  constexpr int NT = NW * kWave;
  constexpr int RPT = (kWindowRows + NT - 1) / NT;  // rows per thread in the plan
  constexpr int kSegGroups = kMultiMaxPartition / kGroupPositions;
  __shared__ uint4 s_b0[STAGE], s_b1[STAGE], s_b2[STAGE], s_b3[STAGE];
  __shared__ uint4 s_b4[R > 4 ? STAGE : 1], s_b5[R > 4 ? STAGE : 1], s_b6[R > 4 ? STAGE : 1], s_b7[R > 4 ? STAGE : 1];
  __shared__ int32_t s_blk[kMultiMaxPartition / 8 + kMultiBlkPad];
  __shared__ int32_t s_ctx[kWindowRows], s_gpre[kWindowRows + 1];
  __shared__ int32_t s_sum[NW];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & (kWave - 1), lr = lane & 31, h = lane >> 5;
  const int G = a.group, Q = a.query_len, QB = a.q_per_tile, C = a.cols;
  const int rows = a.rows;
  const int cap = a.max_blocks_per_row * a.block_size;

  // Plan: clamped lengths and the exclusive prefix of groups per row.
  {
    int len[RPT], loc = 0;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int r = tid * RPT + i;
      int x = r < rows ? a.context_lens[r] : 0;
      len[i] = x < 0 ? 0 : (x > cap ? cap : x);
      loc += multi_stream_groups(len[i]);
    }
    const int incl = wave_inclusive_scan(loc, lane);
    if (lane == kWave - 1) s_sum[wave] = incl;
    __syncthreads();
    int run = incl - loc;
    for (int v = 0; v < wave; ++v) run += s_sum[v];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int r = tid * RPT + i;
      if (r < rows) {
        s_ctx[r] = len[i];
        s_gpre[r] = run;
      }
      run += multi_stream_groups(len[i]);
    }
    if (tid == 0) {
      int total = 0;
      for (int v = 0; v < NW; ++v) total += s_sum[v];
      s_gpre[rows] = total;
    }
    __syncthreads();
  }
  const int ngk = __builtin_amdgcn_readfirstlane(s_gpre[rows]);  // every LDS value below is uniform: kept scalar
  const long long ng_all = (long long)a.n_kv_heads * ngk;
  long long waves = ng_all / max(a.cg_min, 1);
  waves = waves < 1 ? 1 : (waves > a.stream_waves ? a.stream_waves : waves);
  const int w = blockIdx.x;
  if (w < rows && s_ctx[w] == 0) {  // an empty row reads zeros (all its queries); no slice visits it
    const size_t per_row = (size_t)Q * a.n_heads * HD;
    for (size_t idx = tid; idx < per_row; idx += NT) store_out(a.out, a.out_dtype, (size_t)w * per_row + idx, 0.f);
  }
  if (ng_all == 0 || w >= waves) return;  // the whole workgroup
  const long long s1 = slice_start(w + 1, ng_all, waves);

  // this lane's column: query q0 + lr / G, head kvh * G + lr % G of tile `wave`
  const int q0 = wave * QB;
  const int qi = q0 + lr / G, hi = lr % G;
  const bool colv = lr < QB * G && qi < Q;
  const bool active = q0 < Q;  // some column of this wave is a query
  const uint32_t qsign = a.scale < 0.f ? 0x80008000u : 0u;  // fold a negative scale into q (exact)
  const float cscale = multi_cscale(a);
  const StreamLayout L = stream_layout(rows, C, HD, a.stream_waves);
  MultiState<HD> S;
  int cur_kvh = -1, cur_r = -1, pair_j0 = 0;
  for (long long s = slice_start(w, ng_all, waves); s < s1;) {
    const int kvh = (int)(s / ngk);
    const int rem = (int)(s - (long long)kvh * ngk);
    int lo = 0, hr = rows - 1;  // the row holding group `rem`: the last r with s_gpre[r] <= rem
    while (lo < hr) {
      const int mid = (lo + hr + 1) >> 1;
      if (__builtin_amdgcn_readfirstlane(s_gpre[mid]) <= rem) lo = mid;
      else hr = mid - 1;
    }
    const int r = lo;
    const int jx = rem - __builtin_amdgcn_readfirstlane(s_gpre[r]);  // kMultiSegmentCost groups of no work, then the row's own
    s += min((long long)max(kMultiSegmentCost - jx, 0), s1 - s);  // skip what is left of those
    if (s == s1) break;
    const int j0 = max(jx - kMultiSegmentCost, 0);
    const int n = __builtin_amdgcn_readfirstlane(s_ctx[r]);
    const int ngp = (n + kGroupPositions - 1) / kGroupPositions;
    const int j1 = (int)min(min((long long)ngp, j0 + (s1 - s)), (long long)(j0 + kSegGroups));
    __syncthreads();  // every wave is done with the previous segment's ring buffers and block ids
    if (kvh != cur_kvh || r != cur_r) {  // a new (kv head, row): its queries and a fresh softmax state
      pair_j0 = j0;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8_t x =
            colv ? ld_bf16x8(a.q, ((((size_t)r * Q + qi) * a.n_heads + kvh * G + hi) * HD + 16 * ks + 8 * h) * 2)
                 : zero_bf16x8();
        uint4 u = __builtin_bit_cast(uint4, x);
        u.x ^= qsign;
        u.y ^= qsign;
        u.z ^= qsign;
        u.w ^= qsign;
        S.qb[ks] = __builtin_bit_cast(bf16x8_t, u);
      }
      S.col_end = colv ? max(n - Q + qi + 1, 0) : INT_MAX;
      S.min_end = active ? max(n - Q + q0 + 1, 0) : INT_MAX;
      S.m = -INFINITY;
      S.l = 0.f;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int j = 0; j < 16; ++j) S.acc[dt][j] = 0.f;
    }
    // the segment's block ids, clamped into the pool
    const int pos0 = j0 * kGroupPositions;
    const int blk0 = pos0 >> LOG2_BS;
    const int nblk = (min(j1 * kGroupPositions, n) - pos0 + BS - 1) >> LOG2_BS;
    const int32_t *trow = a.block_table + (size_t)r * a.max_blocks_per_row + blk0;
    for (int i = tid; i < nblk; i += NT) {
      const int64_t b = trow[i];
      s_blk[i] = (int32_t)(b < 0 ? 0 : (b >= a.num_blocks ? a.num_blocks - 1 : b));
    }
    __syncthreads();
    multi_run<HD, BS, NW>(S, s_b0, s_b1, s_b2, s_b3, s_b4, s_b5, s_b6, s_b7, a, s_blk, blk0, nblk, kvh, j0, j1 - j0, n,
                          cscale, active, wave, lane);
    s += j1 - j0;
    if (j1 == ngp || s == s1) {  // the (kv head, row) ends here, or the slice does
      const float lt = S.l + __shfl_xor(S.l, 32);
      if (colv) {
        if (pair_j0 == 0 && j1 == ngp) {  // whole inside this slice
          const size_t orow = (((size_t)r * Q + qi) * a.n_heads + kvh * G + hi) * HD;
          multi_store_row<HD>(a, orow, S.acc, lt > 0.f ? 1.f / lt : 0.f, h);  // 0: a query before the history
        } else {  // a piece: 2w + 1 if it starts the (kv head, row), else 2w
          float *slot = a.ws + L.partials + (size_t)(pair_j0 == 0 ? 2 * w + 1 : 2 * w) * L.slot_stride;
          // the stream column (query qi, head hi), formed here rather than held
          // in a register across the loop
          int cx = (int)threadIdx.x & 31;
          asm volatile("" : "+v"(cx));
          cx += q0 * G;
          float *accp = slot + (size_t)cx * HD;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4)
              *reinterpret_cast<f32x4_t *>(accp + 32 * dt + 8 * q4 + 4 * h) =
                  f32x4_t{S.acc[dt][4 * q4], S.acc[dt][4 * q4 + 1], S.acc[dt][4 * q4 + 2], S.acc[dt][4 * q4 + 3]};
          if (h == 0) {
            slot[(size_t)C * HD + cx] = S.m;
            slot[(size_t)C * HD + C + cx] = lt;
          }
        }
      }
      cur_kvh = -1;
    } else {
      cur_kvh = kvh;
      cur_r = r;
    }
  }
}

// Combine the pieces of the (kv head, row)s that the balanced multi-query
// read cut.  One 256-thread workgroup per (kv head, row, chunk of
// kStreamMergeCols columns), light enough (registers, LDS) that the whole
// grid is resident at once: the same plan as the read tells it whether its
// pair was cut and where the pieces lie (slots stream_piece_slot(first, k));
// a pair the read wrote whole leaves the workgroup nothing to do.  Four
// pieces at a time, threads 0 .. 63 fetch each piece's m and l of the chunk's
// columns into LDS while every thread fetches its acc values: wave w holds 8
// consecutive columns, whose acc rows are contiguous in every piece, and its
// load v (of head_dim / 32) reads 1 KiB of them, lane i the 16 bytes at
// (64 v + i) * 16, four hd values of column (256 v + 4 i) / head_dim.  Then
//   M = max_k m_k;  L = sum_k l_k 2^(m_k - M);  out = sum_k acc_k 2^(m_k - M) / L
// folded in slice order (the pieces past the first four rescale the running
// sums by 2^(M_old - M_new)), so the result does not depend on timing.
constexpr int kStreamMergeCols = 32;
template <int HD>
__global__ __launch_bounds__(256) void decode_multi_stream_merge(DecodeArgs a) {
  constexpr int F4 = HD / 32;  // 16-byte loads per lane per piece (1 KiB per wave each)
  constexpr int LPC = HD / 4;  // lanes per column in one load
  __shared__ int32_t s_gpre[kWindowRows + 1];
  __shared__ int32_t s_sum[256 / kWave];
  __shared__ float s_ml[2][4][kStreamMergeCols];  // m and l of four pieces, the chunk's columns
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
  const int rows = a.rows, Q = a.query_len, C = a.cols, G = a.group;
  const int cap = a.max_blocks_per_row * a.block_size;
  
  {
    int x = tid < rows ? a.context_lens[tid] : 0;
    x = x < 0 ? 0 : (x > cap ? cap : x);
    const int ng = multi_stream_groups(x);
    const int incl = wave_inclusive_scan(ng, lane);
    if (lane == kWave - 1) s_sum[wv] = incl;
    __syncthreads();
    int run = incl - ng;
    for (int v = 0; v < wv; ++v) run += s_sum[v];
    if (tid < rows) s_gpre[tid] = run;
    if (tid == 0) s_gpre[rows] = s_sum[0] + s_sum[1] + s_sum[2] + s_sum[3];
    __syncthreads();
  }
  
  const int nch = (C + kStreamMergeCols - 1) / kStreamMergeCols;
  const int pair = (int)blockIdx.x / nch, ch = (int)blockIdx.x - pair * nch;  // pair = kv head * rows + row
  const int kvh = pair / rows, r = pair - kvh * rows;
  const int ngk = s_gpre[rows], g0 = s_gpre[r], ng = s_gpre[r + 1] - g0 - kMultiSegmentCost;
  if (ng <= 0) return;  // zeros, written by the read (uniform: the whole workgroup)
  const long long ng_all = (long long)a.n_kv_heads * ngk;
  long long waves = ng_all / max(a.cg_min, 1);
  waves = waves < 1 ? 1 : (waves > a.stream_waves ? a.stream_waves : waves);
  const long long Sg = (long long)kvh * ngk + g0 + kMultiSegmentCost;  // the pair's first group of work
  const long long first = slice_of(Sg, ng_all, waves);
  const int nparts = (int)(slice_of(Sg + ng - 1, ng_all, waves) - first + 1);
  if (nparts <= 1) return;  // written by the read
  const int c0 = ch * kStreamMergeCols;
  const int d = 4 * (lane % LPC);
  const int cl0 = 8 * wv + lane / LPC;  // chunk column of load 0; load v adds (kWave / LPC) v
  const StreamLayout L = stream_layout(rows, C, HD, a.stream_waves);
  const float *parts = a.ws + L.partials;
  float M[F4], Lsum[F4];
  f32x4_t O[F4];
#pragma unroll
  for (int v = 0; v < F4; ++v) {
    M[v] = -INFINITY;
    Lsum[v] = 0.f;
    O[v] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  for (int k0 = 0; k0 < nparts; k0 += 4) {
    if (k0 > 0) __syncthreads();  // every thread is done with the previous four pieces' m and l
    if (tid < 2 * 4 * kStreamMergeCols / 2) {  // threads 0 .. 127: (piece u, column) m and l
      const int u = tid / kStreamMergeCols, cc = tid % kStreamMergeCols;
      const bool own = k0 + u < nparts && c0 + cc < C;
      const float *sk = parts + stream_piece_slot(first, own ? k0 + u : 0) * L.slot_stride;
      const int c = own ? c0 + cc : c0;
      s_ml[0][u][cc] = own ? sk[(size_t)C * HD + c] : -INFINITY;
      s_ml[1][u][cc] = own ? sk[(size_t)C * HD + C + c] : 0.f;
    }
    f32x4_t x[4][F4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const bool own = k0 + u < nparts;
      const float *sk = parts + stream_piece_slot(first, own ? k0 + u : 0) * L.slot_stride;
#pragma unroll
      for (int v = 0; v < F4; ++v) {
        const int c = min(c0 + cl0 + (kWave / LPC) * v, C - 1);
        x[u][v] = own ? *reinterpret_cast<const f32x4_t *>(sk + (size_t)c * HD + d) : f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
    }
    __syncthreads();  // m and l published
#pragma unroll
    for (int v = 0; v < F4; ++v) {
      const int cc = cl0 + (kWave / LPC) * v;
      const float m0 = s_ml[0][0][cc], m1 = s_ml[0][1][cc], m2 = s_ml[0][2][cc], m3 = s_ml[0][3][cc];
      const float Mn = fmaxf(M[v], fmaxf(fmaxf(m0, m1), fmaxf(m2, m3)));
      if (k0 > 0 && Mn != M[v]) {  // the running sums move to the new maximum
        const float al = exp2_fast(M[v] - Mn);  // M[v] = -inf: nothing accumulated yet, al = 0
        Lsum[v] *= al;
        O[v] *= al;
      }
      M[v] = Mn;
      const float mk[4] = {m0, m1, m2, m3};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float w = (mk[u] == -INFINITY) ? 0.f : exp2_fast(mk[u] - Mn);  // Mn = -inf only if every m_k is
        Lsum[v] = fmaf(s_ml[1][u][cc], w, Lsum[v]);
        O[v] += w * x[u][v];
      }
    }
  }
  
#pragma unroll
  for (int v = 0; v < F4; ++v) {
    const int c = c0 + cl0 + (kWave / LPC) * v;
    if (c >= C) continue;
    const float inv = Lsum[v] > 0.f ? 1.f / Lsum[v] : 0.f;  // 0: a query before the history
    const int query = c / G, hi = c - query * G;
    const size_t o = (((size_t)r * Q + query) * a.n_heads + kvh * G + hi) * HD + d;
    const float y0 = O[v][0] * inv, y1 = O[v][1] * inv, y2 = O[v][2] * inv, y3 = O[v][3] * inv;
    if (a.out_dtype == kF32) {
      *reinterpret_cast<f32x4_t *>(static_cast<float *>(a.out) + o) = f32x4_t{y0, y1, y2, y3};
    } else {
      const uint32_t w0 = f32_to_bf16_rne(y0) | ((uint32_t)f32_to_bf16_rne(y1) << 16);
      const uint32_t w1 = f32_to_bf16_rne(y2) | ((uint32_t)f32_to_bf16_rne(y3) << 16);
      *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(a.out) + o) = make_uint2(w0, w1);
    }
  }
}

template <int HD, int BS, int NW>
hipError_t launch_multi_t(const DecodeArgs &a, hipStream_t stream) {
  if (a.stream == 2) {
    hipLaunchKernelGGL((decode_multi_stream<HD, BS, NW>), dim3((unsigned)a.stream_waves), dim3(NW * kWave), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const unsigned pairs_chunks =
        (unsigned)((size_t)a.rows * a.n_kv_heads * ((a.cols + kStreamMergeCols - 1) / kStreamMergeCols));
    hipLaunchKernelGGL(decode_multi_stream_merge<HD>, dim3(pairs_chunks), dim3(256), 0, stream, a);
    return hipGetLastError();
  }
  const long long units = (long long)a.max_parts * a.q_blocks * a.rows * a.n_kv_heads;
  hipLaunchKernelGGL((decode_multi<HD, BS, NW>), dim3((unsigned)units), dim3(NW * kWave), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.max_parts <= 1) return e;
  const size_t tuples = (size_t)a.rows * a.query_len * a.n_heads;
  hipLaunchKernelGGL(decode_multi_merge, dim3((unsigned)((tuples + kMultiMergeTuples - 1) / kMultiMergeTuples)),
                     dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <int HD, int BS>
hipError_t launch_multi_shape(const DecodeArgs &a, hipStream_t stream) {
  const int32_t waves = multi_waves(a.q_tiles);
  if (waves == 8) return launch_multi_t<HD, BS, 8>(a, stream);
  if (waves == 4) return launch_multi_t<HD, BS, 4>(a, stream);
  return launch_multi_t<HD, BS, 2>(a, stream);
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
    if (a.block_size == 8) return launch_multi_shape<128, 8>(a, stream);
    if (a.block_size == 16) return launch_multi_shape<128, 16>(a, stream);
    return launch_multi_shape<128, 32>(a, stream);
  }
  if (a.block_size == 8) return launch_multi_shape<64, 8>(a, stream);
  if (a.block_size == 16) return launch_multi_shape<64, 16>(a, stream);
  return launch_multi_shape<64, 32>(a, stream);
}

}  // namespace pkv
