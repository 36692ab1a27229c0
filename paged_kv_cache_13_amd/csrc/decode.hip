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

  const int p = blockIdx.x;
  const int g = blockIdx.y;
  const int r = blockIdx.z;
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
        const size_t row = (((size_t)blk * tile_stride + g) << a.log2_bs) + (t & bmask);
        const size_t off = (row * HD + c * EPL) * ES;
        kr[i] = load16(a.k_pool, off);
        vr[i] = load16(a.v_pool, off);
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

template <typename T, int HD, int GP>
hipError_t launch_t(const DecodeArgs &a, hipStream_t stream) {
  dim3 grid(a.max_parts, a.n_kv_heads, a.rows);
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

}  // namespace

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream) {
  if (a.dtype == kF32) return launch_dt<float>(a, stream);
  return launch_dt<uint16_t>(a, stream);
}

}  // namespace pkv
