// Decode attention over a packed, variable-length per-head KV cache.
//
// The compressed cache exists to make later decoding cheaper: KVzip reports
// about 2x lower FlashAttention decode latency (abstract; atlas summary, Key
// results) and gives decode-attention latency against the kept ratio
// (paperhub rebuttal, computational analysis).  Here one decode token per
// query head attends over its KV head's kept rows:
//     out[h][g] = softmax(scale * q[h][g] . K_h^T) V_h,
// K_h, V_h = rows head_offsets[h] .. head_offsets[h+1] of the packed arrays.
// With head_offsets[h] = h * n_c over an uncompressed cache the same kernels
// give the full-cache baseline.
//
// The work is HBM-bound (every kept K and V row is read once; ~2 flops per
// byte for G = 4), so it runs on the VALU: d/8 lanes share a row, each lane
// holding 8 elements of q, K, V and of the output.  Each workgroup handles a
// segment of seg_rows rows of one head with an online softmax (one rescale
// per 4 rows), the segments are merged by decode_combine.
#include <math.h>

#include "common.h"

namespace kvz {

KVZ_DEBUG_WORD(debug_word_decode)

namespace {

constexpr int TPB = 256;
constexpr int GMAX = 8;  // query heads per KV head supported (instantiated as 4 or 8)
constexpr int RB = 4;    // rows per lane group between rescales (8: 232-256 VGPRs, slower)
// rows per workgroup segment: long segments stream best.  On the 128K cache
// (256 heads, d = 128) 1024, 2048, 4096 and 8192 rows read the full cache at
// 5.6, 5.8, 5.95 and 5.9 TB/s and a 30%-kept packed cache at 5.4, 5.7, 5.5
// and 5.3 TB/s (256 rows: 4.5); on one layer of it (8 heads) 2048-row
// segments (512 workgroups) take 0.13 ms, 256-row segments (4096
// workgroups) 0.19 ms
constexpr int SEG_ROWS = 2048;
constexpr float kNeg = -1e30f;

template <typename T>
struct Row8;
template <>
struct Row8<uint16_t> {  // 8 bf16 -> 8 fp32
  static __device__ __forceinline__ void load(const uint16_t* p, float (&o)[8]) {
    // every K and V row is read once: nontemporal loads (about 3-8% faster
    // than cached loads here)
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 u = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    const uint32_t w[4] = {u[0], u[1], u[2], u[3]};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = __uint_as_float(w[i] << 16);
      o[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
};
template <>
struct Row8<float> {
  static __device__ __forceinline__ void load(const float* p, float (&o)[8]) {
    const float4 a = reinterpret_cast<const float4*>(p)[0];
    const float4 b = reinterpret_cast<const float4*>(p)[1];
    o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
    o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
  }
};

// v moved across lanes by a DPP pattern (a modifier of the VALU instruction
// that consumes it: no LDS traffic, unlike a general lane shuffle)
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Sum of s over each aligned group of LPR lanes, in every lane of the group:
// pairs (quad_perm 1,0,3,2), quads (quad_perm 2,3,0,1), then the mirror
// images of the half row (lane i of 8 <- 7 - i) and of the row (lane i of 16
// <- 15 - i), each of which lands on the other, already summed, half; past
// 16 lanes one shuffle.
template <int LPR>
__device__ __forceinline__ float group_sum(float s) {
  s += dpp_f<0xB1>(s);
  s += dpp_f<0x4E>(s);
  if constexpr (LPR >= 8) s += dpp_f<0x141>(s);
  if constexpr (LPR >= 16) s += dpp_f<0x140>(s);
  if constexpr (LPR >= 32) s += __shfl_xor(s, 16);
  static_assert(LPR >= 4 && LPR <= 32, "lanes per row");
  return s;
}

// partial state per (head, segment, g): m (log2 domain), l, acc[D]
template <int D>
__device__ __forceinline__ size_t part_off(int64_t h, int seg, int n_seg, int g, int G) {
  return (size_t)(((h * n_seg + seg) * G) + g) * (D + 2);
}

template <int D, typename T, int GM>
__global__ __launch_bounds__(TPB) void decode_split(const T* __restrict__ q,
                                                    const T* __restrict__ k,
                                                    const T* __restrict__ v,
                                                    const int64_t* __restrict__ offs,
                                                    float cl2, float* __restrict__ part, int G,
                                                    int n_seg, int seg_rows) {
  constexpr int LPR = D / 8;          // lanes per row
  constexpr int RPW = 64 / LPR;       // rows per wave step
  constexpr int RPB = 4 * RPW;        // rows per block step
  __shared__ float red_m[4][GM], red_l[4][GM];
  __shared__ float red_acc[4][GM][D];

  const int64_t h = blockIdx.x / n_seg;
  const int seg = blockIdx.x - (int)h * n_seg;
  const int64_t a = offs[h], b = offs[h + 1];
  // offsets non-decreasing, no head longer than max_len (rows past it are not read)
  KVZ_DCHECK(b >= a && b - a <= (int64_t)n_seg * seg_rows, 1u);
  const int64_t r0 = a + (int64_t)seg * seg_rows;
  if (r0 >= b) return;  // segment past this head's rows (decode_combine skips it)
  const int64_t r1 = min(b, r0 + seg_rows);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int sub = lane / LPR, p8 = lane % LPR;

  float qv[GM][8];
#pragma unroll
  for (int g = 0; g < GM; ++g)
    if (g < G) Row8<T>::load(q + ((h * G + g) * D + p8 * 8), qv[g]);
  float m[GM], l[GM], acc[GM][8];
#pragma unroll
  for (int g = 0; g < GM; ++g) {
    m[g] = kNeg;
    l[g] = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[g][i] = 0.f;
  }

  // rows of this lane group: r0 + w*RPW + sub + RPB*t; RB of them per round
  for (int64_t base = r0 + w * RPW + sub; base < r1; base += (int64_t)RB * RPB) {
    float kf[RB][8], vf[RB][8];
    bool ok[RB];
#pragma unroll
    for (int j = 0; j < RB; ++j) {
      const int64_t row = base + (int64_t)j * RPB;
      ok[j] = row < r1;
      const int64_t rr = ok[j] ? row : base;  // stay in bounds; masked below
      Row8<T>::load(k + rr * D + p8 * 8, kf[j]);
      Row8<T>::load(v + rr * D + p8 * 8, vf[j]);
    }
#pragma unroll
    for (int g = 0; g < GM; ++g) {
      if (g >= G) continue;
      float x[RB];
#pragma unroll
      for (int j = 0; j < RB; ++j) {
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) s = fmaf(qv[g][i], kf[j][i], s);
        s = group_sum<LPR>(s);
        x[j] = ok[j] ? s * cl2 : -INFINITY;
      }
      float mn = m[g];
#pragma unroll
      for (int j = 0; j < RB; ++j) mn = fmaxf(mn, x[j]);
      const float c = fast_exp2(m[g] - mn);
      float ps[RB], psum = 0.f;
#pragma unroll
      for (int j = 0; j < RB; ++j) {
        ps[j] = fast_exp2(x[j] - mn);
        psum += ps[j];
      }
      l[g] = l[g] * c + psum;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float t = acc[g][i] * c;
#pragma unroll
        for (int j = 0; j < RB; ++j) t = fmaf(ps[j], vf[j][i], t);
        acc[g][i] = t;
      }
      m[g] = mn;
    }
  }

  // merge the RPW lane groups of the wave (lanes with the same p8)
#pragma unroll
  for (int g = 0; g < GM; ++g) {
    if (g >= G) continue;
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) {
      const float mo = __shfl_xor(m[g], off), lo = __shfl_xor(l[g], off);
      const float mn = fmaxf(m[g], mo);
      const float cs = fast_exp2(m[g] - mn), co = fast_exp2(mo - mn);
      l[g] = l[g] * cs + lo * co;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[g][i] = acc[g][i] * cs + __shfl_xor(acc[g][i], off) * co;
      m[g] = mn;
    }
    if (sub == 0) {
      if (p8 == 0) {
        red_m[w][g] = m[g];
        red_l[w][g] = l[g];
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) red_acc[w][g][p8 * 8 + i] = acc[g][i];
    }
  }
  __syncthreads();
  // merge the 4 waves and write this segment's partial
  for (int e = tid; e < G * D; e += TPB) {
    const int g = e / D, dd = e - g * D;
    float M = kNeg;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) M = fmaxf(M, red_m[ww][g]);
    float L = 0.f, A = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      const float f = fast_exp2(red_m[ww][g] - M);
      L += red_l[ww][g] * f;
      A += red_acc[ww][g][dd] * f;
    }
    float* pp = part + part_off<D>(h, seg, n_seg, g, G);
    pp[2 + dd] = A;
    if (dd == 0) {
      pp[0] = M;
      pp[1] = L;
    }
  }
}

// one workgroup per (head, g): merge the head's valid segments.  The max is
// a strided reduction over the segments; the weighted sums take the
// segments eight at a time so that their loads are in flight together.
template <int D>
__global__ __launch_bounds__(D) void decode_combine(const float* __restrict__ part,
                                                     const int64_t* __restrict__ offs,
                                                     float* __restrict__ out, int G, int n_seg,
                                                     int seg_rows) {
  constexpr int NWV = D / 64;  // waves per workgroup
  constexpr int U = 8;         // segments per batch
  __shared__ float red[NWV];
  const int64_t h = blockIdx.x / G;
  const int g = blockIdx.x - (int)h * G;
  const int dd = threadIdx.x;
  const int64_t len = offs[h + 1] - offs[h];
  const int nv = (int)min((int64_t)n_seg, (len + seg_rows - 1) / seg_rows);
  float M = kNeg;
  for (int s = dd; s < nv; s += D) M = fmaxf(M, part[part_off<D>(h, s, n_seg, g, G)]);
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  if ((dd & 63) == 0) red[dd >> 6] = M;
  __syncthreads();
  M = red[0];
#pragma unroll
  for (int w = 1; w < NWV; ++w) M = fmaxf(M, red[w]);
  // compensated sums over the segments (a long head has thousands, and one
  // of them may hold nearly all of the weight)
  float L = 0.f, A = 0.f, cL = 0.f, cA = 0.f;
  for (int s0 = 0; s0 < nv; s0 += U) {
    float m[U], l[U], a[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool ok = s0 + u < nv;
      const float* pp = part + part_off<D>(h, ok ? s0 + u : 0, n_seg, g, G);
      m[u] = ok ? pp[0] : kNeg;
      l[u] = ok ? pp[1] : 0.f;
      a[u] = ok ? pp[2 + dd] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float f = exp2f(m[u] - M);
      kahan_add(L, cL, l[u] * f);
      kahan_add(A, cA, a[u] * f);
    }
  }
  out[(h * G + g) * D + dd] = nv > 0 ? A / L : 0.f;
}

template <int D, typename T>
hipError_t launch(const DecodePlan& p, const void* q, const void* k, const void* v,
                  const int64_t* offs, float scale, float* out, void* ws, hipStream_t st) {
  float* part = reinterpret_cast<float*>(ws);
  const float cl2 = scale * 1.4426950408889634f;
  if (p.G <= 4)
    KVZ_LAUNCH("decode_split", (decode_split<D, T, 4>), (unsigned)(p.n_heads * p.n_seg), TPB, 0,
               st, (const T*)q, (const T*)k, (const T*)v, offs, cl2, part, p.G, p.n_seg,
               p.seg_rows);
  else
    KVZ_LAUNCH("decode_split", (decode_split<D, T, GMAX>), (unsigned)(p.n_heads * p.n_seg), TPB,
               0, st, (const T*)q, (const T*)k, (const T*)v, offs, cl2, part, p.G, p.n_seg,
               p.seg_rows);
  KVZ_LAUNCH("decode_combine", decode_combine<D>, (unsigned)(p.n_heads * p.G), D, 0, st, part,
             offs, out, p.G, p.n_seg, p.seg_rows);
  return hipGetLastError();
}

}  // namespace

DecodePlan decode_plan(int64_t n_heads, int G, int d, int max_len) {
  DecodePlan p{};
  p.n_heads = n_heads;
  p.G = G;
  p.d = d;
  p.seg_rows = SEG_ROWS;
  // 64-bit: max_len may be as large as INT_MAX
  p.n_seg = (int)(((int64_t)max_len + p.seg_rows - 1) / p.seg_rows);
  if (p.n_seg < 1) p.n_seg = 1;
  p.total_bytes = align256((size_t)n_heads * p.n_seg * G * (d + 2) * sizeof(float));
  return p;
}

hipError_t decode_launch(kvz_dtype dt, const DecodePlan& p, const void* q, const void* k,
                         const void* v, const int64_t* offs, float scale, float* out, void* ws,
                         hipStream_t st) {
  if (dt == KVZ_BF16) {
    switch (p.d) {
      case 64: return launch<64, uint16_t>(p, q, k, v, offs, scale, out, ws, st);
      case 128: return launch<128, uint16_t>(p, q, k, v, offs, scale, out, ws, st);
      case 256: return launch<256, uint16_t>(p, q, k, v, offs, scale, out, ws, st);
    }
  } else {
    switch (p.d) {
      case 64: return launch<64, float>(p, q, k, v, offs, scale, out, ws, st);
      case 128: return launch<128, float>(p, q, k, v, offs, scale, out, ws, st);
      case 256: return launch<256, float>(p, q, k, v, offs, scale, out, ws, st);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace kvz
