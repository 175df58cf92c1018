// Global keep-ratio selection over every (layer, head, token) score.
//
// KVzip sorts all KV pairs by importance and evicts the lowest (blog post,
// section 4.1 step 5), with one threshold over all heads so that head
// budgets come out non-uniform (atlas summary, "Measured effects").  Sorting
// 33-65M floats is not needed: each float maps to a 32-bit key that orders
// like the value (sign bit flipped for non-negative values, all bits flipped
// for negative ones, -0 folded onto +0), the exact K-th largest key tau is
// found by a radix select, then one tiled pass writes the mask: keep every score > tau
// and the first (K - #greater) scores == tau in flat index order, which makes
// exactly K.  Everything stays on the device (no host synchronisation) and
// every atomic is an integer add, so the result is deterministic.
//
// Passes over S (N floats): three, plus a re-read of the few tiles whose
// ties are kept when the K-th boundary splits a run of equal scores.
//   sel_init       zero the histograms and the search state
//   sel_hist0      full read: histogram of bits 31..20 (4096 bins)
//   sel_pick<0>    the top-level bin b0 holding the K-th largest
//   sel_hist12     full read: for scores in bin b0, a histogram of bits
//                  19..10 (1024 bins) and a joint histogram of bits 19..0
//                  (1M bins, global memory)
//   sel_pick<1>    bin b1 of bits 19..10
//   sel_pick2      bin b2 of bits 9..0 from the joint histogram row b1:
//                  tau, the number of ties to keep, and whether every
//                  score equal to tau is kept (the common case for
//                  continuous scores)
//   sel_mask       full read + mask write: keep > tau (>= tau when no tie
//                  is dropped); kept and tied counts per 4096-score tile
//   sel_eq_scan    only when ties are split: ties in all earlier tiles
//   sel_fixup      only when ties are split, and only tiles holding kept
//                  ties: re-read the tile, rank its ties in flat order (wave
//                  ballots), set their mask bytes, add them to its count
//   sel_heads      per-head budgets and their exclusive scan, tau
#include <math.h>

#include "common.h"

namespace kvz {

KVZ_DEBUG_WORD(debug_word_select)

namespace {

// radix digits of the 32-bit key: bits 31..20 (first pass), 19..10 and 9..0
constexpr int B0_SHIFT = 20;
constexpr int BINS0 = 1 << (32 - B0_SHIFT);  // 4096
constexpr int BINS1 = 1024;                  // bits 19..10
constexpr int JBINS = 1 << B0_SHIFT;         // joint histogram of bits 19..0
constexpr int TILE = 4096;        // scores per mask tile (within one head)
constexpr int TPB = 256;          // threads per block
constexpr int PER_T = TILE / TPB; // 16 scores per thread per tile
constexpr int HU = 8;             // float4 loads in flight per thread in the histograms
constexpr int HR = 4;             // lane-replicated copies of each LDS histogram bin
#ifndef KVZ_HB_MAX
#define KVZ_HB_MAX 512
#endif
constexpr int HB_MAX = KVZ_HB_MAX; // histogram workgroups per pass

// order-preserving key of a non-NaN float (-0 and +0 compare equal)
__device__ __forceinline__ uint32_t fkey(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_to_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

struct SelState {
  uint32_t b0, b1, tau, split_ties;  // digits found, tau bits, ties partially kept?
  long long krem[4];                 // count still to keep before digit r (krem[3]: ties)
};

__global__ void sel_init(uint32_t* __restrict__ hist, uint32_t* __restrict__ joint,
                         SelState* __restrict__ st, long long K) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  const int stride = gridDim.x * blockDim.x;
  for (int i = t; i < BINS0 + BINS1; i += stride) hist[i] = 0;
  for (int i = t; i < JBINS; i += stride) joint[i] = 0;
  if (t == 0) {
    st->b0 = st->b1 = st->tau = st->split_ties = 0;
    st->krem[0] = K;
    st->krem[1] = st->krem[2] = st->krem[3] = 0;
  }
}

// full read, histogram of the top 12 bits (bits 31..20)
__global__ __launch_bounds__(TPB) void sel_hist0(const float* __restrict__ S, long long N,
                                                 uint32_t* __restrict__ hist) {
  // HR copies of every bin in consecutive banks, copy = lane % HR: lanes of
  // a wave that hit the same bin (scores crowd into few bins) spread over HR
  // banks instead of serialising on one
  __shared__ uint32_t h[BINS0 * HR];
  for (int b = threadIdx.x; b < BINS0 * HR; b += TPB) h[b] = 0;
  __syncthreads();
  const uint32_t rep = threadIdx.x & (HR - 1);
  const long long n4 = N >> 2;
  const float4* S4 = reinterpret_cast<const float4*>(S);
  // HU independent 16-byte loads in flight per thread before any atomic
  const long long stride = (long long)gridDim.x * TPB * HU;
  for (long long i0 = (long long)blockIdx.x * TPB * HU + threadIdx.x; i0 < n4; i0 += stride) {
    float4 v[HU];
#pragma unroll
    for (int u = 0; u < HU; ++u) {
      const long long i = i0 + (long long)u * TPB;
      v[u] = i < n4 ? S4[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < HU; ++u) {
      if (i0 + (long long)u * TPB < n4) {
        KVZ_DCHECK(!isnan(v[u].x) && !isnan(v[u].y) && !isnan(v[u].z) && !isnan(v[u].w), 1u);
        atomicAdd(&h[(fkey(v[u].x) >> B0_SHIFT) * HR + rep], 1u);
        atomicAdd(&h[(fkey(v[u].y) >> B0_SHIFT) * HR + rep], 1u);
        atomicAdd(&h[(fkey(v[u].z) >> B0_SHIFT) * HR + rep], 1u);
        atomicAdd(&h[(fkey(v[u].w) >> B0_SHIFT) * HR + rep], 1u);
      }
    }
  }
  if (blockIdx.x == 0)
    for (long long i = (n4 << 2) + threadIdx.x; i < N; i += TPB) {
      KVZ_DCHECK(!isnan(S[i]), 1u);
      atomicAdd(&h[(fkey(S[i]) >> B0_SHIFT) * HR + rep], 1u);
    }
  __syncthreads();
  for (int b = threadIdx.x; b < BINS0; b += TPB) {
    uint32_t c = 0;
#pragma unroll
    for (int r = 0; r < HR; ++r) c += h[b * HR + r];
    if (c) atomicAdd(&hist[b], c);
  }
}

// full read, scores whose top 12 bits equal b0: LDS histogram of bits 19..10
// and global joint histogram of bits 19..0
__global__ __launch_bounds__(TPB) void sel_hist12(const float* __restrict__ S, long long N,
                                                  uint32_t* __restrict__ hist1,
                                                  uint32_t* __restrict__ joint,
                                                  const SelState* __restrict__ st) {
  __shared__ uint32_t h[BINS1 * HR];  // lane-replicated, as in sel_hist0
  for (int b = threadIdx.x; b < BINS1 * HR; b += TPB) h[b] = 0;
  __syncthreads();
  const uint32_t b0 = st->b0;
  const uint32_t rep = threadIdx.x & (HR - 1);
  auto add = [&](uint32_t k) {
    if ((k >> B0_SHIFT) == b0) {
      atomicAdd(&h[((k >> 10) & (BINS1 - 1)) * HR + rep], 1u);
      atomicAdd(&joint[k & (JBINS - 1)], 1u);
    }
  };
  const long long n4 = N >> 2;
  const float4* S4 = reinterpret_cast<const float4*>(S);
  const long long stride = (long long)gridDim.x * TPB * HU;
  for (long long i0 = (long long)blockIdx.x * TPB * HU + threadIdx.x; i0 < n4; i0 += stride) {
    float4 v[HU];
#pragma unroll
    for (int u = 0; u < HU; ++u) {
      const long long i = i0 + (long long)u * TPB;
      v[u] = i < n4 ? S4[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < HU; ++u) {
      if (i0 + (long long)u * TPB < n4) {
        add(fkey(v[u].x));
        add(fkey(v[u].y));
        add(fkey(v[u].z));
        add(fkey(v[u].w));
      }
    }
  }
  if (blockIdx.x == 0)
    for (long long i = (n4 << 2) + threadIdx.x; i < N; i += TPB) add(fkey(S[i]));
  __syncthreads();
  for (int b = threadIdx.x; b < BINS1; b += TPB) {
    uint32_t c = 0;
#pragma unroll
    for (int r = 0; r < HR; ++r) c += h[b * HR + r];
    if (c) atomicAdd(&hist1[b], c);
  }
}

// Suffix search over NB bins held by one 256-thread workgroup (NB/256 bins per
// thread): the bin d with above(d) < krem <= above(d) + bins[d], where
// above(d) = sum of bins > d.  Returns d and above(d) in *d_out, *above_out
// (written by the one thread that finds it).
template <int NB>
__device__ void suffix_pick(const uint32_t* __restrict__ bins, long long krem, long long* part,
                            int* d_out, long long* above_out) {
  constexpr int PT = NB / TPB;
  const int t = threadIdx.x;
  long long c[PT], mine = 0;
#pragma unroll
  for (int e = 0; e < PT; ++e) {
    c[e] = bins[PT * t + e];
    mine += c[e];
  }
  part[t] = mine;
  __syncthreads();
  for (int off = 1; off < TPB; off <<= 1) {  // inclusive suffix sums
    const long long add = (t + off < TPB) ? part[t + off] : 0;
    __syncthreads();
    part[t] += add;
    __syncthreads();
  }
  const long long above_thread = (t + 1 < TPB) ? part[t + 1] : 0;
  if (above_thread < krem && krem <= part[t]) {
    long long above = above_thread;
    for (int e = PT - 1; e >= 0; --e) {
      if (above < krem && krem <= above + c[e]) {
        *d_out = PT * t + e;
        *above_out = above;
        break;
      }
      above += c[e];
    }
  }
}

template <int ROUND>
__global__ __launch_bounds__(TPB) void sel_pick(const uint32_t* __restrict__ hist,
                                                SelState* __restrict__ st) {
  __shared__ long long part[TPB];
  __shared__ int d;
  __shared__ long long above;
  if (threadIdx.x == 0) d = -1;
  __syncthreads();
  const long long krem = st->krem[ROUND];
  if (ROUND == 0)
    suffix_pick<BINS0>(hist, krem, part, &d, &above);
  else
    suffix_pick<BINS1>(hist + BINS0, krem, part, &d, &above);
  __syncthreads();
  if (threadIdx.x == 0 && d >= 0) {
    if (ROUND == 0) st->b0 = (uint32_t)d; else st->b1 = (uint32_t)d;
    st->krem[ROUND + 1] = krem - above;
  }
}

// last digit from the joint histogram row of (b1); tau and the tie quota
__global__ __launch_bounds__(TPB) void sel_pick2(const uint32_t* __restrict__ joint,
                                                 SelState* __restrict__ st) {
  __shared__ long long part[TPB];
  __shared__ int d;
  __shared__ long long above;
  if (threadIdx.x == 0) d = -1;
  __syncthreads();
  const long long krem = st->krem[2];
  const uint32_t* row = joint + ((size_t)st->b1 << 10);
  suffix_pick<1024>(row, krem, part, &d, &above);
  __syncthreads();
  if (threadIdx.x == 0 && d >= 0) {
    const long long need = krem - above;  // ties to keep
    st->tau = (st->b0 << B0_SHIFT) | (st->b1 << 10) | (uint32_t)d;
    st->krem[3] = need;
    st->split_ties = need < (long long)row[d] ? 1u : 0u;
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

// Vector layout of a tile (n_c a multiple of 4, so every tile starts 16-byte
// aligned): in slab u (1024 scores) thread t owns scores u*1024 + 4t .. +3.
// Scores past the tile's length are flagged invalid.
constexpr int VSLABS = TILE / (4 * TPB);  // 4
__device__ __forceinline__ void load_keys4(const float* __restrict__ S, long long base, int e0,
                                           int len, uint32_t (&k)[4], bool (&ok)[4]) {
  if (e0 + 3 < len) {
    const float4 v = *reinterpret_cast<const float4*>(S + base + e0);
    k[0] = fkey(v.x);
    k[1] = fkey(v.y);
    k[2] = fkey(v.z);
    k[3] = fkey(v.w);
#pragma unroll
    for (int c = 0; c < 4; ++c) ok[c] = true;
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      ok[c] = e0 + c < len;
      k[c] = ok[c] ? fkey(S[base + e0 + c]) : 0u;
    }
  }
}
// mask bytes of 4 consecutive scores (one 32-bit store when all are valid)
__device__ __forceinline__ void store_mask4(uint8_t* __restrict__ mask, long long base, int e0,
                                            const bool (&keep)[4], const bool (&ok)[4]) {
  if (ok[3]) {
    const uint32_t w = (keep[0] ? 1u : 0u) | (keep[1] ? 1u << 8 : 0u) |
                       (keep[2] ? 1u << 16 : 0u) | (keep[3] ? 1u << 24 : 0u);
    *reinterpret_cast<uint32_t*>(mask + base + e0) = w;
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (ok[c]) mask[base + e0 + c] = keep[c] ? 1 : 0;
  }
}

__device__ __forceinline__ uint32_t block_sum_u32(uint32_t v, uint32_t* red) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  const uint32_t s = red[0] + red[1] + red[2] + red[3];
  __syncthreads();
  return s;
}

// one workgroup of 1024 threads: exclusive scans of block sums
constexpr int SCAN_T = 1024;
constexpr int SCAN_W = SCAN_T / 64;

// Exclusive scan of one value per thread over the workgroup: shuffle scans
// within each wave, then one wave scans the SCAN_W wave totals.  buf holds
// SCAN_W entries; *total gets the sum of all values.  32-bit: the callers
// scan per-tile counts whose sum is at most N < 2^31.
__device__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* buf, uint32_t* total) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  uint32_t x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) buf[w] = x;
  __syncthreads();
  if (w == 0) {
    uint32_t y = lane < SCAN_W ? buf[lane] : 0u;
#pragma unroll
    for (int off = 1; off < SCAN_W; off <<= 1) {
      const uint32_t z = __shfl_up(y, off);
      if (lane >= off) y += z;
    }
    if (lane < SCAN_W) buf[lane] = y;
  }
  __syncthreads();
  const uint32_t before = (w ? buf[w - 1] : 0u) + x - v;
  *total = buf[SCAN_W - 1];
  __syncthreads();  // buf may be reused at once
  return before;
}

// Exclusive scan of n per-tile counts by one SCAN_T workgroup, SPT
// consecutive tiles per thread per round; out(i, prefix) is called for every
// tile.  Returns the sum of all counts.
template <typename Out>
__device__ long long scan_tiles(const uint32_t* __restrict__ cnt, int64_t n, uint32_t* buf,
                                Out out) {
  constexpr int SPT = 8;
  const int t = threadIdx.x;
  uint32_t carry = 0;
  for (int64_t r0 = 0; r0 < n; r0 += (int64_t)SCAN_T * SPT) {
    const int64_t i0 = r0 + (int64_t)t * SPT;
    uint32_t v[SPT];
    uint32_t mine = 0;
#pragma unroll
    for (int e = 0; e < SPT; ++e) {
      v[e] = i0 + e < n ? cnt[i0 + e] : 0u;
      mine += v[e];
    }
    uint32_t total;
    uint32_t run = carry + block_exclusive_scan(mine, buf, &total);
#pragma unroll
    for (int e = 0; e < SPT; ++e) {
      if (i0 + e < n) out(i0 + e, (long long)run);
      run += v[e];
    }
    carry += total;
  }
  return carry;
}

// Mask of one tile: keep scores > tau, and == tau as well when every tie is
// kept.  When ties are split they are left out here and counted per tile;
// sel_fixup adds the first ones in flat order.
__global__ __launch_bounds__(TPB) void sel_mask(const float* __restrict__ S,
                                                const SelState* __restrict__ st,
                                                uint8_t* __restrict__ mask,
                                                uint32_t* __restrict__ keptc,
                                                uint32_t* __restrict__ eqc, int tiles_per_head,
                                                int n_c) {
  __shared__ uint32_t red[4];
  const int64_t tile = blockIdx.x;
  int len;
  const long long base = tile_range(tile, tiles_per_head, n_c, len);
  const uint32_t tau = st->tau;
  const bool all_eq = st->split_ties == 0;
  const int t = threadIdx.x;
  uint32_t kept = 0, eq = 0;
  if ((n_c & 3) == 0) {
#pragma unroll
    for (int u = 0; u < VSLABS; ++u) {
      const int e0 = u * 4 * TPB + 4 * t;
      uint32_t k[4];
      bool ok[4], keep[4];
      load_keys4(S, base, e0, len, k, ok);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const bool is_eq = ok[c] && k[c] == tau;
        keep[c] = ok[c] && (k[c] > tau || (all_eq && is_eq));
        kept += keep[c];
        eq += is_eq;
      }
      store_mask4(mask, base, e0, keep, ok);
    }
  } else {
#pragma unroll
    for (int u = 0; u < PER_T; ++u) {
      const int e = u * TPB + t;
      if (e < len) {
        const uint32_t k = fkey(S[base + e]);
        const bool keep = k > tau || (all_eq && k == tau);
        mask[base + e] = keep ? 1 : 0;
        kept += keep;
        eq += k == tau;
      }
    }
  }
  // both counts are at most TILE < 2^16: one sum of kept + 2^16 * eq
  const uint32_t both = block_sum_u32(kept | (eq << 16), red);
  if (t == 0) {
    keptc[tile] = both & 0xFFFFu;
    eqc[tile] = both >> 16;
  }
}

// only when ties are split: ties in all tiles before each tile
__global__ __launch_bounds__(SCAN_T) void sel_eq_scan(const SelState* __restrict__ st,
                                                      const uint32_t* __restrict__ eqc,
                                                      long long* __restrict__ eqbase,
                                                      int64_t n_tiles) {
  if (!st->split_ties) return;
  __shared__ uint32_t buf[SCAN_W];
  scan_tiles(eqc, n_tiles, buf, [&](int64_t i, long long before) { eqbase[i] = before; });
}

// Only when ties are split, and only in tiles that hold ties while the ties
// of all earlier tiles leave part of the quota (K - #greater): rank the
// tile's ties in flat order and set the mask bytes of the kept ones.
__global__ __launch_bounds__(TPB) void sel_fixup(const float* __restrict__ S,
                                                 const SelState* __restrict__ st,
                                                 const uint32_t* __restrict__ eqc,
                                                 const long long* __restrict__ eqbase,
                                                 uint8_t* __restrict__ mask,
                                                 uint32_t* __restrict__ keptc, int tiles_per_head,
                                                 int n_c) {
  if (!st->split_ties) return;
  const int64_t tile = blockIdx.x;
  if (eqc[tile] == 0) return;
  const long long need_eq = st->krem[3];
  const long long eb = eqbase[tile];
  if (eb >= need_eq) return;
  __shared__ uint32_t wtot[PER_T][4];
  __shared__ uint32_t red[4];
  int len;
  const long long base = tile_range(tile, tiles_per_head, n_c, len);
  const uint32_t tau = st->tau;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const unsigned long long lt = (1ull << lane) - 1ull;
  uint32_t added = 0;
  long long run = 0;  // ties in earlier slabs (rows) of this tile
  if ((n_c & 3) == 0) {
    // vector layout: earlier slabs, then earlier threads of the slab (a
    // ballot per bit of the per-thread tie count, 0..4), then earlier
    // scores of the thread
#pragma unroll
    for (int u = 0; u < VSLABS; ++u) {
      const int e0 = u * 4 * TPB + 4 * t;
      uint32_t k[4];
      bool ok[4], eq[4];
      load_keys4(S, base, e0, len, k, ok);
      uint32_t cnt = 0;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        eq[c] = ok[c] && k[c] == tau;
        cnt += eq[c];
      }
      uint32_t below = 0, wsum = 0;
#pragma unroll
      for (int bit = 0; bit < 3; ++bit) {
        const unsigned long long bb = __ballot((cnt >> bit) & 1u);
        below += (uint32_t)__popcll(bb & lt) << bit;
        wsum += (uint32_t)__popcll(bb) << bit;
      }
      if (lane == 0) wtot[u][w] = wsum;
      __syncthreads();
      long long before = eb + run + below;
      for (int ww = 0; ww < w; ++ww) before += wtot[u][ww];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if (eq[c]) {
          if (before < need_eq) {
            mask[base + e0 + c] = 1;
            ++added;
          }
          ++before;
        }
      }
      run += wtot[u][0] + wtot[u][1] + wtot[u][2] + wtot[u][3];
    }
  } else {
    // scalar layout: element e = u*256 + t
#pragma unroll
    for (int u = 0; u < PER_T; ++u) {
      const int e = u * TPB + t;
      const bool eq = e < len && fkey(S[base + e]) == tau;
      const unsigned long long bb = __ballot(eq);
      if (lane == 0) wtot[u][w] = (uint32_t)__popcll(bb);
      __syncthreads();
      long long before = eb + run + __popcll(bb & lt);
      for (int ww = 0; ww < w; ++ww) before += wtot[u][ww];
      if (eq && before < need_eq) {
        mask[base + e] = 1;
        ++added;
      }
      run += wtot[u][0] + wtot[u][1] + wtot[u][2] + wtot[u][3];
    }
  }
  added = block_sum_u32(added, red);
  if (t == 0) keptc[tile] += added;
}

// one workgroup: per-head budgets (each thread sums the tile counts of its
// heads) and their exclusive scan; tau
__global__ __launch_bounds__(SCAN_T) void sel_heads(const SelState* __restrict__ st,
                                                    const uint32_t* __restrict__ keptc,
                                                    int64_t* __restrict__ head_offsets,
                                                    float* __restrict__ tau_out,
                                                    int tiles_per_head, int64_t n_heads) {
  __shared__ uint32_t buf[SCAN_W];
  const int t = threadIdx.x;
  const int64_t hper = (n_heads + SCAN_T - 1) / SCAN_T;
  const int64_t h0 = (int64_t)t * hper, h1 = min(n_heads, h0 + hper);
  auto head_sum = [&](int64_t h) {
    const uint32_t* kp = keptc + h * tiles_per_head;
    uint32_t s = 0;
#pragma unroll 8
    for (int k = 0; k < tiles_per_head; ++k) s += kp[k];
    return s;
  };
  uint32_t hs = 0;
  for (int64_t h = h0; h < h1; ++h) hs += head_sum(h);
  uint32_t total;
  long long hrun = block_exclusive_scan(hs, buf, &total);
  for (int64_t h = h0; h < h1; ++h) {
    head_offsets[h] = hrun;
    hrun += head_sum(h);
  }
  if (t == 0) {
    KVZ_DCHECK((long long)total == st->krem[0], 2u);  // exactly K kept
    head_offsets[n_heads] = total;
    *tau_out = key_to_float(st->tau);
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

struct SelWs {
  uint32_t* hist;      // [BINS0 + BINS1]
  uint32_t* joint;     // [JBINS]
  SelState* st;
  uint32_t* eqc;       // [n_tiles]
  uint32_t* keptc;     // [n_tiles]
  long long* eqbase;   // [n_tiles]
};

SelWs carve(const SelectPlan& p, void* ws) {
  char* w = reinterpret_cast<char*>(ws);
  SelWs s;
  s.hist = reinterpret_cast<uint32_t*>(w);
  w += align256((BINS0 + BINS1) * sizeof(uint32_t));
  s.joint = reinterpret_cast<uint32_t*>(w);
  w += align256(JBINS * sizeof(uint32_t));
  s.st = reinterpret_cast<SelState*>(w);
  w += align256(sizeof(SelState));
  s.eqc = reinterpret_cast<uint32_t*>(w);
  w += align256((size_t)p.n_tiles * sizeof(uint32_t));
  s.keptc = reinterpret_cast<uint32_t*>(w);
  w += align256((size_t)p.n_tiles * sizeof(uint32_t));
  s.eqbase = reinterpret_cast<long long*>(w);
  return s;
}

}  // namespace

SelectPlan select_plan(int64_t n_heads, int n_c) {
  SelectPlan p{};
  p.n_heads = n_heads;
  p.n_c = n_c;
  p.N = n_heads * (int64_t)n_c;
  p.tiles_per_head = (int)(((int64_t)n_c + TILE - 1) / TILE);  // n_c may be INT_MAX
  p.n_tiles = n_heads * p.tiles_per_head;
  p.total_bytes = align256((BINS0 + BINS1) * sizeof(uint32_t)) + align256(JBINS * sizeof(uint32_t)) +
                  align256(sizeof(SelState)) + 2 * align256((size_t)p.n_tiles * sizeof(uint32_t)) +
                  align256((size_t)p.n_tiles * sizeof(long long));
  return p;
}

hipError_t select_launch(const SelectPlan& p, const float* S, int64_t K, uint8_t* mask,
                         int64_t* head_offsets, float* tau, void* ws, hipStream_t stream) {
  if (K == 0) {
    KVZ_LAUNCH("select_empty", sel_empty, 1024, 256, 0, stream, mask, (long long)p.N,
               head_offsets, p.n_heads, tau);
    return hipGetLastError();
  }
  const SelWs w = carve(p, ws);
  KVZ_LAUNCH("select_init", sel_init, 512, 256, 0, stream, w.hist, w.joint, w.st, (long long)K);
  const long long n4 = p.N / 4;
  // at most HB_MAX workgroups, each looping over its share: the LDS
  // histogram's clearing and flush are paid once per workgroup
  long long hbl = (n4 + TPB * HU - 1) / (TPB * HU);
  if (hbl > HB_MAX) hbl = HB_MAX;
  int hb = (int)hbl;
  if (hb < 1) hb = 1;
  if (hb > 2048) hb = 2048;
  KVZ_LAUNCH("select_hist", sel_hist0, hb, TPB, 0, stream, S, (long long)p.N, w.hist);
  KVZ_LAUNCH("select_pick", sel_pick<0>, 1, TPB, 0, stream, w.hist, w.st);
  KVZ_LAUNCH("select_hist", sel_hist12, hb, TPB, 0, stream, S, (long long)p.N, w.hist + BINS0,
             w.joint, w.st);
  KVZ_LAUNCH("select_pick", sel_pick<1>, 1, TPB, 0, stream, w.hist, w.st);
  KVZ_LAUNCH("select_pick", sel_pick2, 1, TPB, 0, stream, w.joint, w.st);
  KVZ_LAUNCH("select_mask", sel_mask, (unsigned)p.n_tiles, TPB, 0, stream, S, w.st, mask, w.keptc,
             w.eqc, p.tiles_per_head, p.n_c);
  KVZ_LAUNCH("select_scan", sel_eq_scan, 1, SCAN_T, 0, stream, w.st, w.eqc, w.eqbase, p.n_tiles);
  KVZ_LAUNCH("select_fixup", sel_fixup, (unsigned)p.n_tiles, TPB, 0, stream, S, w.st, w.eqc,
             w.eqbase, mask, w.keptc, p.tiles_per_head, p.n_c);
  KVZ_LAUNCH("select_scan", sel_heads, 1, SCAN_T, 0, stream, w.st, w.keptc, head_offsets, tau,
             p.tiles_per_head, p.n_heads);
  return hipGetLastError();
}

}  // namespace kvz
