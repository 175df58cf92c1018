// Global keep-ratio selection over every (layer, head, token) score.
//
// KVzip sorts all KV pairs by importance and evicts the lowest (blog post,
// section 4.1 step 5), with one threshold over all heads so that head
// budgets come out non-uniform (atlas summary, "Measured effects").  Sorting
// 33-65M floats is not needed: the exact K-th largest score is found by a
// three-round radix select on the raw bits (scores are >= 0, so their IEEE
// bit patterns order like the values), then one tiled pass writes the mask:
// keep every score > tau and the first (K - #greater) scores == tau in flat
// index order, which makes exactly K.  All decisions stay on the device.
//
// Kernels, in launch order:
//   sel_init        zero the three histograms and the search state
//   sel_hist<r>     2048-bin histogram of radix digit r among candidates
//   sel_pick<r>     one workgroup: the digit where the running count from
//                   the top reaches the remaining K
//   sel_tile_count  per 4096-element tile of a head: #(> tau), #(== tau)
//   sel_scan        one workgroup: ties before each tile, per-head budgets,
//                   head offsets, tau
//   sel_mask        per tile: the mask, with tie ranks by wave ballots
#include <math.h>

#include "common.h"

namespace kvz {

namespace {

constexpr int BINS = 2048;
constexpr int TILE = 4096;        // elements per mask tile (within one head)
constexpr int TPB = 256;          // threads per block
constexpr int PER_T = TILE / TPB; // 16 elements per thread per tile

// radix digits: bits 31..21 (11), 20..10 (11), 9..0 (10)
__device__ __forceinline__ uint32_t digit(uint32_t key, int round) {
  return round == 0 ? (key >> 21) : round == 1 ? ((key >> 10) & 0x7FF) : (key & 0x3FF);
}
__device__ __forceinline__ bool prefix_ok(uint32_t key, int round, uint32_t prefix) {
  return round == 0 ? true : round == 1 ? (key >> 21) == prefix : (key >> 10) == prefix;
}
// canonical key of a non-negative float (-0 and +0 compare equal)
__device__ __forceinline__ uint32_t fkey(float f) { return __float_as_uint(f) & 0x7FFFFFFFu; }

struct SelState {
  uint32_t prefix[3];   // prefix after each round (digits so far)
  uint32_t pad;
  long long krem[4];    // remaining count to keep, before round r
};

__global__ void sel_init(uint32_t* hist, SelState* st, long long K) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t < 3 * BINS) hist[t] = 0;
  if (t == 0) {
    st->prefix[0] = st->prefix[1] = st->prefix[2] = 0;
    st->pad = 0;
    st->krem[0] = K;
    st->krem[1] = st->krem[2] = st->krem[3] = 0;
  }
}

template <int ROUND>
__global__ __launch_bounds__(TPB) void sel_hist(const float* __restrict__ S, long long N,
                                                uint32_t* __restrict__ hist,
                                                const SelState* __restrict__ st) {
  __shared__ uint32_t h[BINS];
  for (int b = threadIdx.x; b < BINS; b += TPB) h[b] = 0;
  __syncthreads();
  const uint32_t prefix = ROUND == 0 ? 0u : st->prefix[ROUND - 1];
  const long long n4 = N >> 2;
  const float4* S4 = reinterpret_cast<const float4*>(S);
  const long long stride = (long long)gridDim.x * TPB;
  for (long long i = (long long)blockIdx.x * TPB + threadIdx.x; i < n4; i += stride) {
    const float4 v = S4[i];
    const uint32_t k[4] = {fkey(v.x), fkey(v.y), fkey(v.z), fkey(v.w)};
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (prefix_ok(k[e], ROUND, prefix)) atomicAdd(&h[digit(k[e], ROUND)], 1u);
  }
  if (blockIdx.x == 0) {
    for (long long i = (n4 << 2) + threadIdx.x; i < N; i += TPB) {
      const uint32_t k = fkey(S[i]);
      if (prefix_ok(k, ROUND, prefix)) atomicAdd(&h[digit(k, ROUND)], 1u);
    }
  }
  __syncthreads();
  uint32_t* gh = hist + ROUND * BINS;
  for (int b = threadIdx.x; b < BINS; b += TPB)
    if (h[b]) atomicAdd(&gh[b], h[b]);
}

// One workgroup of 256 threads; thread t owns bins [8t, 8t+8).  Finds digit b
// with above(b) < krem <= above(b) + hist[b], above(b) = sum of bins > b.
template <int ROUND>
__global__ __launch_bounds__(TPB) void sel_pick(const uint32_t* __restrict__ hist,
                                                SelState* __restrict__ st) {
  __shared__ long long part[TPB];
  const uint32_t* gh = hist + ROUND * BINS;
  const int t = threadIdx.x;
  long long c[8], mine = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    c[e] = gh[8 * t + e];
    mine += c[e];
  }
  part[t] = mine;
  __syncthreads();
  // inclusive suffix sums: part[t] = sum of threads >= t
  for (int off = 1; off < TPB; off <<= 1) {
    long long add = (t + off < TPB) ? part[t + off] : 0;
    __syncthreads();
    part[t] += add;
    __syncthreads();
  }
  const long long krem = st->krem[ROUND];
  const long long above_thread = (t + 1 < TPB) ? part[t + 1] : 0;  // bins >= 8(t+1)
  if (above_thread < krem && krem <= part[t]) {
    long long above = above_thread;
    for (int e = 7; e >= 0; --e) {
      if (above < krem && krem <= above + c[e]) {
        const uint32_t prev = ROUND == 0 ? 0u : st->prefix[ROUND - 1];
        const int bits = ROUND == 2 ? 10 : 11;
        st->prefix[ROUND] = (prev << bits) | (uint32_t)(8 * t + e);
        st->krem[ROUND + 1] = krem - above;
        break;
      }
      above += c[e];
    }
  }
}

__device__ __forceinline__ long long tile_range(int64_t tile, int tiles_per_head, int n_c,
                                                int& len) {
  const int64_t head = tile / tiles_per_head;
  const int tt = (int)(tile - head * tiles_per_head);
  const int start = tt * TILE;
  len = min(TILE, n_c - start);
  return head * (long long)n_c + start;
}

__device__ __forceinline__ long long block_sum_ll(long long v, long long* red) {
  // wave reduction then across the 4 waves
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  const long long s = red[0] + red[1] + red[2] + red[3];
  __syncthreads();
  return s;
}

__global__ __launch_bounds__(TPB) void sel_tile_count(const float* __restrict__ S,
                                                      const SelState* __restrict__ st,
                                                      uint32_t* __restrict__ gtc,
                                                      uint32_t* __restrict__ eqc,
                                                      int tiles_per_head, int n_c) {
  __shared__ long long red[4];
  const int64_t tile = blockIdx.x;
  int len;
  const long long base = tile_range(tile, tiles_per_head, n_c, len);
  const uint32_t tau = st->prefix[2];
  long long gt = 0, eq = 0;
#pragma unroll
  for (int u = 0; u < PER_T; ++u) {
    const int e = u * TPB + threadIdx.x;
    if (e < len) {
      const uint32_t k = fkey(S[base + e]);
      gt += k > tau;
      eq += k == tau;
    }
  }
  gt = block_sum_ll(gt, red);
  eq = block_sum_ll(eq, red);
  if (threadIdx.x == 0) {
    gtc[tile] = (uint32_t)gt;
    eqc[tile] = (uint32_t)eq;
  }
}

// One workgroup of 1024 threads.  eqbase[tile] = ties in all earlier tiles;
// kept(tile) = gt + clamp(need_eq - eqbase, 0, eq); budgets summed per head,
// head_offsets = exclusive scan of budgets.
constexpr int SCAN_T = 1024;

__device__ long long block_exclusive_scan(long long v, long long* buf, long long* total) {
  const int t = threadIdx.x;
  buf[t] = v;
  __syncthreads();
  for (int off = 1; off < SCAN_T; off <<= 1) {
    long long add = t >= off ? buf[t - off] : 0;
    __syncthreads();
    buf[t] += add;
    __syncthreads();
  }
  const long long incl = buf[t];
  *total = buf[SCAN_T - 1];
  __syncthreads();
  return incl - v;
}

__global__ __launch_bounds__(SCAN_T) void sel_scan(const SelState* __restrict__ st,
                                                   const uint32_t* __restrict__ gtc,
                                                   const uint32_t* __restrict__ eqc,
                                                   uint32_t* __restrict__ keptc,
                                                   long long* __restrict__ eqbase,
                                                   int64_t* __restrict__ head_offsets,
                                                   float* __restrict__ tau_out, int64_t n_tiles,
                                                   int tiles_per_head, int64_t n_heads) {
  __shared__ long long buf[SCAN_T];
  const int t = threadIdx.x;
  const long long need_eq = st->krem[3];
  // pass A: ties before each tile, kept count per tile
  const int64_t per = (n_tiles + SCAN_T - 1) / SCAN_T;
  const int64_t b0 = (int64_t)t * per, b1 = min(n_tiles, b0 + per);
  long long mine = 0;
  for (int64_t i = b0; i < b1; ++i) mine += eqc[i];
  long long total;
  long long run = block_exclusive_scan(mine, buf, &total);
  for (int64_t i = b0; i < b1; ++i) {
    const long long e = eqc[i];
    eqbase[i] = run;
    long long take = need_eq - run;
    take = take < 0 ? 0 : (take > e ? e : take);
    keptc[i] = (uint32_t)(gtc[i] + take);
    run += e;
  }
  __syncthreads();
  // pass B: budgets per head and their exclusive scan
  const int64_t hper = (n_heads + SCAN_T - 1) / SCAN_T;
  const int64_t h0 = (int64_t)t * hper, h1 = min(n_heads, h0 + hper);
  long long hs = 0;
  for (int64_t h = h0; h < h1; ++h)
    for (int k = 0; k < tiles_per_head; ++k) hs += keptc[h * tiles_per_head + k];
  long long hrun = block_exclusive_scan(hs, buf, &total);
  for (int64_t h = h0; h < h1; ++h) {
    head_offsets[h] = hrun;
    for (int k = 0; k < tiles_per_head; ++k) hrun += keptc[h * tiles_per_head + k];
  }
  if (t == 0) {
    head_offsets[n_heads] = total;
    *tau_out = __uint_as_float(st->prefix[2]);
  }
}

// Local exclusive rank of `flag` over the tile in element order e = u*256 + t.
// flags[u] bit for this thread; returns per-u ranks through `rank_out`.
__global__ __launch_bounds__(TPB) void sel_mask(const float* __restrict__ S,
                                                const SelState* __restrict__ st,
                                                const long long* __restrict__ eqbase,
                                                uint8_t* __restrict__ mask, int tiles_per_head,
                                                int n_c) {
  __shared__ uint32_t wtot[PER_T][4];
  const int64_t tile = blockIdx.x;
  int len;
  const long long base = tile_range(tile, tiles_per_head, n_c, len);
  const uint32_t tau = st->prefix[2];
  const long long need_eq = st->krem[3];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  uint32_t kk[PER_T];
  bool eqf[PER_T];
#pragma unroll
  for (int u = 0; u < PER_T; ++u) {
    const int e = u * TPB + t;
    kk[u] = e < len ? fkey(S[base + e]) : 0u;
    eqf[u] = e < len && kk[u] == tau;
    const unsigned long long b = __ballot(eqf[u]);
    if (lane == 0) wtot[u][w] = (uint32_t)__popcll(b);
  }
  __syncthreads();
  const long long eb = eqbase[tile];
  long long run = 0;
#pragma unroll
  for (int u = 0; u < PER_T; ++u) {
    const int e = u * TPB + t;
    const unsigned long long b = __ballot(eqf[u]);
    long long before = run;
    for (int ww = 0; ww < w; ++ww) before += wtot[u][ww];
    before += __popcll(b & ((1ull << lane) - 1ull));
    if (e < len) {
      const bool keep = kk[u] > tau || (eqf[u] && eb + before < need_eq);
      mask[base + e] = keep ? 1 : 0;
    }
    run += wtot[u][0] + wtot[u][1] + wtot[u][2] + wtot[u][3];
  }
}

// K == 0: keep nothing
__global__ void sel_empty(uint8_t* mask, long long N, int64_t* head_offsets, int64_t n_heads,
                          float* tau_out) {
  const long long stride = (long long)gridDim.x * blockDim.x;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < N; i += stride)
    mask[i] = 0;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i <= n_heads; i += stride)
    head_offsets[i] = 0;
  if (blockIdx.x == 0 && threadIdx.x == 0) *tau_out = INFINITY;
}

}  // namespace

SelectPlan select_plan(int64_t n_heads, int n_c) {
  SelectPlan p{};
  p.n_heads = n_heads;
  p.n_c = n_c;
  p.N = n_heads * (int64_t)n_c;
  p.tiles_per_head = (n_c + TILE - 1) / TILE;
  p.n_tiles = n_heads * p.tiles_per_head;
  size_t b = 0;
  b += align256(3 * BINS * sizeof(uint32_t));        // histograms
  b += align256(sizeof(SelState));                    // state
  b += 3 * align256((size_t)p.n_tiles * sizeof(uint32_t));  // gtc, eqc, keptc
  b += align256((size_t)p.n_tiles * sizeof(long long));     // eqbase
  p.total_bytes = b;
  return p;
}

hipError_t select_launch(const SelectPlan& p, const float* S, int64_t K, uint8_t* mask,
                         int64_t* head_offsets, float* tau, void* ws, hipStream_t stream) {
  if (K == 0) {
    KVZ_LAUNCH("select_empty", sel_empty, 1024, 256, 0, stream, mask, (long long)p.N,
               head_offsets, p.n_heads, tau);
    return hipGetLastError();
  }
  char* w = reinterpret_cast<char*>(ws);
  uint32_t* hist = reinterpret_cast<uint32_t*>(w);
  w += align256(3 * BINS * sizeof(uint32_t));
  SelState* st = reinterpret_cast<SelState*>(w);
  w += align256(sizeof(SelState));
  uint32_t* gtc = reinterpret_cast<uint32_t*>(w);
  w += align256((size_t)p.n_tiles * sizeof(uint32_t));
  uint32_t* eqc = reinterpret_cast<uint32_t*>(w);
  w += align256((size_t)p.n_tiles * sizeof(uint32_t));
  uint32_t* keptc = reinterpret_cast<uint32_t*>(w);
  w += align256((size_t)p.n_tiles * sizeof(uint32_t));
  long long* eqbase = reinterpret_cast<long long*>(w);

  KVZ_LAUNCH("select_init", sel_init, (3 * BINS + 255) / 256, 256, 0, stream, hist, st,
             (long long)K);
  long long n4 = p.N / 4;
  int hb = (int)((n4 + TPB * 8 - 1) / (TPB * 8));
  if (hb < 1) hb = 1;
  if (hb > 2048) hb = 2048;
  KVZ_LAUNCH("select_hist", sel_hist<0>, hb, TPB, 0, stream, S, (long long)p.N, hist, st);
  KVZ_LAUNCH("select_pick", sel_pick<0>, 1, TPB, 0, stream, hist, st);
  KVZ_LAUNCH("select_hist", sel_hist<1>, hb, TPB, 0, stream, S, (long long)p.N, hist, st);
  KVZ_LAUNCH("select_pick", sel_pick<1>, 1, TPB, 0, stream, hist, st);
  KVZ_LAUNCH("select_hist", sel_hist<2>, hb, TPB, 0, stream, S, (long long)p.N, hist, st);
  KVZ_LAUNCH("select_pick", sel_pick<2>, 1, TPB, 0, stream, hist, st);
  KVZ_LAUNCH("select_tile_count", sel_tile_count, (unsigned)p.n_tiles, TPB, 0, stream, S, st,
             gtc, eqc, p.tiles_per_head, p.n_c);
  KVZ_LAUNCH("select_scan", sel_scan, 1, SCAN_T, 0, stream, st, gtc, eqc, keptc, eqbase,
             head_offsets, tau, p.n_tiles, p.tiles_per_head, p.n_heads);
  KVZ_LAUNCH("select_mask", sel_mask, (unsigned)p.n_tiles, TPB, 0, stream, S, st, eqbase, mask,
             p.tiles_per_head, p.n_c);
  return hipGetLastError();
}

}  // namespace kvz
