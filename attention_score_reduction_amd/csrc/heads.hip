// Head-level and token-level aggregates of the score tensor S[L*H][n_c], and
// the two structured evictions built on them.
//
// Head-level score (paperhub rebuttal, answer on head-level scores): the max
// of a head's scores along the sequence axis, used to rank whole heads for
// context-independent head eviction (KVzip blog post, section 5.4).
// Token-level score (blog section 4.3.3): one score per token, the max over
// every layer and head; sorting those decides which tokens every head keeps.
// Both aggregates read S once (HBM-bound) and are exact (max needs no
// rounding).
//
// Head eviction: the K_heads heads with the highest head scores keep every
// token; the others keep their first n_sink and last n_recent tokens (the
// streaming-head structure of DuoAttention, the head-level method the pages
// compare against; the pages do not say what an evicted head keeps).  Token
// eviction: the K_tokens positions with the highest token scores are kept in
// every head.  Both pick their heads or tokens with the radix select of
// kvz_select_threshold run on the aggregate (exact K, ties to the lower
// index), then expand that choice into the full per-(head, token) mask and
// the head offsets that kvz_compact consumes.
#include <math.h>

#include "common.h"

namespace kvz {

namespace {

constexpr int TPB = 256;

constexpr int HM_TPB = 1024;  // head_max: one workgroup of 16 waves per head

__device__ __forceinline__ float max4(float4 v) { return fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w)); }

// One workgroup per head: max over its n_c scores.  With n_c a multiple of 4
// every row is 16-byte aligned (S is), so each thread takes 16-byte loads,
// four in flight; otherwise 4-byte loads.  (One 256-thread workgroup with
// 4-byte loads read the 128K cache's scores at 2.8 TB/s.)
__global__ __launch_bounds__(HM_TPB) void head_max(const float* __restrict__ S, int n_c,
                                                   float* __restrict__ out) {
  __shared__ float red[HM_TPB / 64];
  const int64_t h = blockIdx.x;
  const float* row = S + h * (int64_t)n_c;
  const int t = threadIdx.x;
  float m = -INFINITY;
  if ((n_c & 3) == 0) {
    const float4* r4 = reinterpret_cast<const float4*>(row);
    const int n4 = n_c >> 2;
    int i = t;
    for (; i + 3 * HM_TPB < n4; i += 4 * HM_TPB) {
      const float4 a = r4[i], b = r4[i + HM_TPB], c = r4[i + 2 * HM_TPB], d = r4[i + 3 * HM_TPB];
      m = fmaxf(m, fmaxf(fmaxf(max4(a), max4(b)), fmaxf(max4(c), max4(d))));
    }
    for (; i < n4; i += HM_TPB) m = fmaxf(m, max4(r4[i]));
  } else {
    int j = t;
    for (; j + 3 * HM_TPB < n_c; j += 4 * HM_TPB)
      m = fmaxf(fmaxf(m, fmaxf(row[j], row[j + HM_TPB])),
                fmaxf(row[j + 2 * HM_TPB], row[j + 3 * HM_TPB]));
    for (; j < n_c; j += HM_TPB) m = fmaxf(m, row[j]);
  }
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if ((t & 63) == 0) red[t >> 6] = m;
  __syncthreads();
  if (t < 64) {
    float v = t < HM_TPB / 64 ? red[t] : -INFINITY;
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
    if (t == 0) out[h] = v;
  }
}

// Token maxima over all heads.  A workgroup covers 256 consecutive tokens,
// four per lane (one 16-byte load per head when n_c is a multiple of 4, so
// that rows stay 16-byte aligned); its four waves take every fourth head,
// eight loads in flight, and LDS merges the waves.  (One thread per token
// over all heads read the 128K cache's scores at 1.9 TB/s.)
constexpr int TM_U = 8;
__global__ __launch_bounds__(TPB) void token_max(const float* __restrict__ S, int64_t n_heads,
                                                 int n_c, float* __restrict__ out) {
  __shared__ float4 red[TPB / 64][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int j0 = blockIdx.x * 256 + lane * 4;
  float4 m = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
  if ((n_c & 3) == 0 && j0 < n_c) {  // j0 + 3 < n_c as well
    const float* col = S + j0;
    int64_t h = w;
    for (; h + 4 * (TM_U - 1) < n_heads; h += 4 * TM_U) {
      float4 v[TM_U];
#pragma unroll
      for (int u = 0; u < TM_U; ++u)
        v[u] = *reinterpret_cast<const float4*>(col + (h + 4 * u) * (int64_t)n_c);
#pragma unroll
      for (int u = 0; u < TM_U; ++u) {
        m.x = fmaxf(m.x, v[u].x);
        m.y = fmaxf(m.y, v[u].y);
        m.z = fmaxf(m.z, v[u].z);
        m.w = fmaxf(m.w, v[u].w);
      }
    }
    for (; h < n_heads; h += 4) {
      const float4 v = *reinterpret_cast<const float4*>(col + h * (int64_t)n_c);
      m.x = fmaxf(m.x, v.x);
      m.y = fmaxf(m.y, v.y);
      m.z = fmaxf(m.z, v.z);
      m.w = fmaxf(m.w, v.w);
    }
  } else if (j0 < n_c) {
    float r[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    for (int64_t h = w; h < n_heads; h += 4)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (j0 + c < n_c) r[c] = fmaxf(r[c], S[h * (int64_t)n_c + j0 + c]);
    m = make_float4(r[0], r[1], r[2], r[3]);
  }
  red[w][lane] = m;
  __syncthreads();
  if (w == 0 && j0 < n_c) {
    float4 v = red[0][lane];
#pragma unroll
    for (int ww = 1; ww < TPB / 64; ++ww) {
      const float4 o = red[ww][lane];
      v.x = fmaxf(v.x, o.x);
      v.y = fmaxf(v.y, o.y);
      v.z = fmaxf(v.z, o.z);
      v.w = fmaxf(v.w, o.w);
    }
    const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (j0 + c < n_c) out[j0 + c] = vv[c];
  }
}

// bytes f0 .. f0+15 of a flat mask of N bytes, packed little-endian in w:
// one 16-byte store (the mask is 16-byte aligned), byte stores at the tail
__device__ __forceinline__ void store_group(uint8_t* mask, int64_t f0, int64_t N,
                                            const uint32_t (&w)[4]) {
  if (f0 + 16 <= N) {
    *reinterpret_cast<uint4*>(mask + f0) = make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    for (int u = 0; f0 + u < N; ++u) mask[f0 + u] = (uint8_t)(w[u >> 2] >> (8 * (u & 3)));
  }
}

// keep mask of head eviction: byte f of the flat [n_heads][n_c] mask is 1 when
// its head is kept whole or its position lies in one of the two windows.
// Each thread writes 16 consecutive bytes with one 16-byte store.
__global__ __launch_bounds__(TPB) void head_window_mask(const uint8_t* __restrict__ keep,
                                                        int64_t n_heads, int n_c, int n_sink,
                                                        int n_recent, uint8_t* __restrict__ mask) {
  const int64_t N = n_heads * (int64_t)n_c;
  const int64_t groups = (N + 15) / 16;
  const int64_t stride = (int64_t)gridDim.x * TPB;
  for (int64_t g = (int64_t)blockIdx.x * TPB + threadIdx.x; g < groups; g += stride) {
    const int64_t f0 = g * 16;
    int64_t h = f0 / n_c;
    int j = (int)(f0 - h * n_c);
    uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const uint32_t bit = (h < n_heads && (keep[h] || j < n_sink || j >= n_c - n_recent)) ? 1 : 0;
      w[u >> 2] |= bit << (8 * (u & 3));
      if (++j == n_c) {
        j = 0;
        ++h;
      }
    }
    store_group(mask, f0, N, w);
  }
}

// head offsets of head eviction: exclusive scan of the kept count of every
// head (n_c when kept whole, else the size of the two windows), one
// workgroup looping over the heads 1024 at a time
__global__ __launch_bounds__(1024) void head_window_offsets(const uint8_t* __restrict__ keep,
                                                            int64_t n_heads, int n_c,
                                                            int64_t window,
                                                            int64_t* __restrict__ offs) {
  __shared__ int64_t wsum[16];
  __shared__ int64_t carry;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  if (t == 0) carry = 0;
  __syncthreads();
  for (int64_t base = 0; base < n_heads; base += 1024) {
    const int64_t h = base + t;
    const int64_t v = h < n_heads ? (keep[h] ? (int64_t)n_c : window) : 0;
    // inclusive scan within the wave
    int64_t x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int64_t y = __shfl_up(x, o);
      if (lane >= o) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    if (t == 0) {
      int64_t run = 0;
      for (int w = 0; w < 16; ++w) {
        const int64_t c = wsum[w];
        wsum[w] = run;
        run += c;
      }
    }
    __syncthreads();
    const int64_t excl = carry + wsum[wave] + x - v;
    if (h < n_heads) offs[h] = excl;
    __syncthreads();
    if (t == 1023) carry = excl + v;
    __syncthreads();
  }
  if (t == 0) offs[n_heads] = carry;
}

// keep mask of token eviction: row h of the flat mask is the token keep row
__global__ __launch_bounds__(TPB) void token_broadcast_mask(const uint8_t* __restrict__ tkeep,
                                                            int64_t n_heads, int n_c,
                                                            uint8_t* __restrict__ mask) {
  const int64_t N = n_heads * (int64_t)n_c;
  const int64_t groups = (N + 15) / 16;
  const int64_t stride = (int64_t)gridDim.x * TPB;
  for (int64_t g = (int64_t)blockIdx.x * TPB + threadIdx.x; g < groups; g += stride) {
    const int64_t f0 = g * 16;
    int j = (int)(f0 % n_c);
    uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      w[u >> 2] |= (uint32_t)tkeep[j] << (8 * (u & 3));
      if (++j == n_c) j = 0;
    }
    store_group(mask, f0, N, w);
  }
}

// The two mask writers when n_c is a multiple of 16 (and the keep array is
// 16-byte aligned): a 16-byte group g then lies in one head row, at offset
// 16 * (g % groups per row), and 32-bit index arithmetic suffices (N < 2^31).
// Token eviction: the group is the keep row's 16 bytes at that offset.
__global__ __launch_bounds__(TPB) void token_broadcast_mask16(const uint4* __restrict__ tkeep,
                                                              int gpr, int groups,
                                                              uint4* __restrict__ mask) {
  for (int g = blockIdx.x * TPB + threadIdx.x; g < groups; g += gridDim.x * TPB)
    mask[g] = tkeep[g % gpr];
}

// Head eviction: all ones when the group's head is kept whole, else byte u is
// 1 when position 16 * (g % gpr) + u lies in either window.
__global__ __launch_bounds__(TPB) void head_window_mask16(const uint8_t* __restrict__ keep,
                                                          int gpr, int groups, int n_c,
                                                          int n_sink, int n_recent,
                                                          uint4* __restrict__ mask) {
  for (int g = blockIdx.x * TPB + threadIdx.x; g < groups; g += gridDim.x * TPB) {
    const int h = g / gpr;
    const int j0 = (g - h * gpr) * 16;
    uint32_t w[4];
    if (keep[h]) {
      w[0] = w[1] = w[2] = w[3] = 0x01010101u;
    } else {
      w[0] = w[1] = w[2] = w[3] = 0u;
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int j = j0 + u;
        w[u >> 2] |= (uint32_t)(j < n_sink || j >= n_c - n_recent) << (8 * (u & 3));
      }
    }
    mask[g] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// head offsets of token eviction: every head keeps exactly K tokens
__global__ void token_offsets(int64_t n_heads, int64_t K, int64_t* __restrict__ offs) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t h = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; h <= n_heads; h += stride)
    offs[h] = h * K;
}

// grid of a grid-stride kernel over 16-byte groups: enough workgroups to
// fill the chip a few times, at most one group per thread
unsigned mask_grid(int64_t N) {
  const int64_t groups = (N + 15) / 16;
  int64_t b = (groups + TPB - 1) / TPB;
  if (b > 4096) b = 4096;
  return (unsigned)(b < 1 ? 1 : b);
}

// workspace of the structured selections: the aggregate scores, then the
// selection's own workspace, its two head offsets and its tau
struct AggWs {
  float* agg;
  int64_t* sel_offs;
  float* sel_tau;
  void* sel_ws;
};

AggWs carve_agg(int64_t n_agg, void* ws) {
  char* w = reinterpret_cast<char*>(ws);
  AggWs a;
  a.agg = reinterpret_cast<float*>(w);
  w += align256((size_t)n_agg * sizeof(float));
  a.sel_offs = reinterpret_cast<int64_t*>(w);
  w += 256;
  a.sel_tau = reinterpret_cast<float*>(w);
  w += 256;
  a.sel_ws = w;
  return a;
}

}  // namespace

size_t agg_select_workspace(int64_t n_agg) {
  return align256((size_t)n_agg * sizeof(float)) + 512 + select_plan(1, (int)n_agg).total_bytes;
}

hipError_t select_heads_launch(const float* S, int64_t n_heads, int n_c, int64_t K_heads,
                               int n_sink, int n_recent, uint8_t* mask, int64_t* head_offsets,
                               uint8_t* head_keep, void* ws, hipStream_t st) {
  const AggWs a = carve_agg(n_heads, ws);
  KVZ_LAUNCH("head_scores", head_max, (unsigned)n_heads, HM_TPB, 0, st, S, n_c, a.agg);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = select_launch(select_plan(1, (int)n_heads), a.agg, K_heads, head_keep, a.sel_offs,
                    a.sel_tau, a.sel_ws, st);
  if (e != hipSuccess) return e;
  const int64_t s = n_sink < n_c ? n_sink : n_c, r = n_recent < n_c ? n_recent : n_c;
  const int64_t window = s + r < n_c ? s + r : n_c;
  const int64_t N = n_heads * (int64_t)n_c;
  if (n_c % 16 == 0)
    KVZ_LAUNCH("evict_mask", head_window_mask16, mask_grid(N), TPB, 0, st, head_keep,
               n_c / 16, (int)(N / 16), n_c, n_sink, n_recent, reinterpret_cast<uint4*>(mask));
  else
    KVZ_LAUNCH("evict_mask", head_window_mask, mask_grid(N), TPB, 0, st, head_keep, n_heads, n_c,
               n_sink, n_recent, mask);
  KVZ_LAUNCH("evict_offsets", head_window_offsets, 1, 1024, 0, st, head_keep, n_heads, n_c,
             window, head_offsets);
  return hipGetLastError();
}

hipError_t select_tokens_launch(const float* S, int64_t n_heads, int n_c, int64_t K_tokens,
                                uint8_t* mask, int64_t* head_offsets, uint8_t* token_keep,
                                void* ws, hipStream_t st) {
  const AggWs a = carve_agg(n_c, ws);
  KVZ_LAUNCH("token_scores", token_max, (unsigned)(((int64_t)n_c + 255) / 256), TPB, 0, st, S,
             n_heads, n_c, a.agg);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = select_launch(select_plan(1, n_c), a.agg, K_tokens, token_keep, a.sel_offs, a.sel_tau,
                    a.sel_ws, st);
  if (e != hipSuccess) return e;
  const int64_t N = n_heads * (int64_t)n_c;
  if (n_c % 16 == 0 && (reinterpret_cast<uintptr_t>(token_keep) & 15u) == 0)
    KVZ_LAUNCH("evict_mask", token_broadcast_mask16, mask_grid(N), TPB, 0, st,
               reinterpret_cast<const uint4*>(token_keep), n_c / 16, (int)(N / 16),
               reinterpret_cast<uint4*>(mask));
  else
    KVZ_LAUNCH("evict_mask", token_broadcast_mask, mask_grid(N), TPB, 0, st, token_keep, n_heads,
               n_c, mask);
  int64_t ob = (n_heads + 1 + TPB - 1) / TPB;
  if (ob > 1024) ob = 1024;
  KVZ_LAUNCH("evict_offsets", token_offsets, (unsigned)ob, TPB, 0, st, n_heads, K_tokens,
             head_offsets);
  return hipGetLastError();
}

hipError_t head_scores_launch(const float* S, int64_t n_heads, int n_c, float* out,
                              hipStream_t st) {
  KVZ_LAUNCH("head_scores", head_max, (unsigned)n_heads, HM_TPB, 0, st, S, n_c, out);
  return hipGetLastError();
}

hipError_t token_scores_launch(const float* S, int64_t n_heads, int n_c, float* out,
                               hipStream_t st) {
  KVZ_LAUNCH("token_scores", token_max, (unsigned)(((int64_t)n_c + 255) / 256), TPB, 0, st, S, n_heads,
             n_c, out);
  return hipGetLastError();
}

}  // namespace kvz
