// Compaction of the kept K/V rows into a packed per-head cache.
//
// After selection the surviving pairs form the reusable compressed cache
// (KVzip blog post, section 4.1 step 5; paperhub rebuttal: the compressed
// cache is built once and reused by later queries).  Heads are laid out one
// after another in flat (layer, head) order, each head's rows in ascending
// token position, with the position stored beside them (idx), so a
// variable-length per-head decode can address it with head_offsets.
//
// Kernels: cmp_count (kept rows per 4096-position tile), cmp_scan (one
// thread per head: output row of each tile), cmp_scatter (per tile: ranks by
// wave ballots, then the whole workgroup copies the kept rows with 16-byte
// loads and stores; the writes of a tile land in one contiguous range).
#include "common.h"

namespace kvz {

namespace {

constexpr int TILE = 4096;
constexpr int TPB = 256;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int PER_T = TILE / TPB;

__global__ __launch_bounds__(TPB) void cmp_count(const uint8_t* __restrict__ mask,
                                                 uint32_t* __restrict__ cnt, int64_t head_begin,
                                                 int tiles_per_head, int n_c) {
  __shared__ uint32_t red[4];
  const int64_t tile = blockIdx.x;
  const int64_t hh = tile / tiles_per_head;
  const int start = (int)(tile - hh * tiles_per_head) * TILE;
  const int len = min(TILE, n_c - start);
  const uint8_t* m = mask + (head_begin + hh) * (int64_t)n_c + start;
  uint32_t c = 0;
#pragma unroll
  for (int u = 0; u < PER_T; ++u) {
    const int e = u * TPB + threadIdx.x;
    if (e < len) c += m[e] != 0;
  }
  for (int off = 32; off > 0; off >>= 1) c += __shfl_xor(c, off);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = c;
  __syncthreads();
  if (threadIdx.x == 0) cnt[tile] = red[0] + red[1] + red[2] + red[3];
}

__global__ void cmp_scan(const uint32_t* __restrict__ cnt, const int64_t* __restrict__ head_offsets,
                         int64_t* __restrict__ base, int64_t head_begin, int64_t head_count,
                         int tiles_per_head) {
  const int64_t hh = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (hh >= head_count) return;
  int64_t run = head_offsets[head_begin + hh];
  for (int k = 0; k < tiles_per_head; ++k) {
    base[hh * tiles_per_head + k] = run;
    run += cnt[hh * tiles_per_head + k];
  }
}

// RC = 16-byte chunks per row (row bytes / 16), a compile-time constant so
// the (row, chunk) split of the copy index is a shift.
template <int RC>
__global__ __launch_bounds__(TPB) void cmp_scatter(
    const u32x4* __restrict__ kc, const u32x4* __restrict__ vc, const uint8_t* __restrict__ mask,
    const int64_t* __restrict__ head_offsets, const int64_t* __restrict__ base,
    u32x4* __restrict__ ko, u32x4* __restrict__ vo, int32_t* __restrict__ idx,
    int64_t head_begin, int tiles_per_head, int n_c) {
  constexpr int U = 4;  // copies in flight per thread and array
  __shared__ uint32_t wtot[PER_T][4];
  __shared__ int32_t list[TILE];
  const int64_t tile = blockIdx.x;
  const int64_t hh = tile / tiles_per_head;
  const int start = (int)(tile - hh * tiles_per_head) * TILE;
  const int len = min(TILE, n_c - start);
  const uint8_t* m = mask + (head_begin + hh) * (int64_t)n_c + start;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  bool f[PER_T];
#pragma unroll
  for (int u = 0; u < PER_T; ++u) {
    const int e = u * TPB + t;
    f[u] = e < len && m[e] != 0;
    const unsigned long long b = __ballot(f[u]);
    if (lane == 0) wtot[u][w] = (uint32_t)__popcll(b);
  }
  __syncthreads();
  int run = 0;
#pragma unroll
  for (int u = 0; u < PER_T; ++u) {
    const unsigned long long b = __ballot(f[u]);
    int before = run;
    for (int ww = 0; ww < w; ++ww) before += wtot[u][ww];
    before += __popcll(b & ((1ull << lane) - 1ull));
    if (f[u]) list[before] = start + u * TPB + t;
    run += wtot[u][0] + wtot[u][1] + wtot[u][2] + wtot[u][3];
  }
  __syncthreads();
  const int64_t o0 = base[tile];
  // never write past this head's range, whatever the offsets say
  const int64_t lim = head_offsets[head_begin + hh + 1];
  const int count = (int)max((int64_t)0, min((int64_t)run, lim - o0));
  const int64_t head_row0 = hh * (int64_t)n_c;  // k/v pointers start at head_begin
  for (int k = t; k < count; k += TPB) idx[o0 + k] = list[k];
  const int total = count * RC;
  const u32x4* ksrc = kc + head_row0 * RC;
  const u32x4* vsrc = vc + head_row0 * RC;
  u32x4* kdst = ko + o0 * RC;
  u32x4* vdst = vo + o0 * RC;
  // U independent 16-byte copies per array per thread per round: all loads
  // of a round are issued before its stores
  for (int x0 = t; x0 < total; x0 += U * TPB) {
    u32x4 kv[U], vv[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int x = x0 + j * TPB;
      if (x < total) {
        const int k = x / RC, c = x % RC;
        const int64_t src = (int64_t)list[k] * RC + c;
        // rows are read once: nontemporal loads keep them out of the caches
        kv[j] = __builtin_nontemporal_load(ksrc + src);
        vv[j] = __builtin_nontemporal_load(vsrc + src);
      }
    }
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int x = x0 + j * TPB;
      if (x < total) {
        __builtin_nontemporal_store(kv[j], kdst + x);
        __builtin_nontemporal_store(vv[j], vdst + x);
      }
    }
  }
}

}  // namespace

CompactPlan compact_plan(int64_t head_count, int n_c) {
  CompactPlan p{};
  p.head_count = head_count;
  p.n_c = n_c;
  p.tiles_per_head = (n_c + TILE - 1) / TILE;
  p.n_tiles = head_count * p.tiles_per_head;
  p.total_bytes = align256((size_t)p.n_tiles * sizeof(uint32_t)) +
                  align256((size_t)p.n_tiles * sizeof(int64_t));
  return p;
}

hipError_t compact_launch(const CompactPlan& p, int row_bytes, int64_t head_begin, const void* kc,
                          const void* vc, const uint8_t* mask, const int64_t* head_offsets,
                          void* ko, void* vo, int32_t* idx, void* ws, hipStream_t st) {
  char* w = reinterpret_cast<char*>(ws);
  uint32_t* cnt = reinterpret_cast<uint32_t*>(w);
  w += align256((size_t)p.n_tiles * sizeof(uint32_t));
  int64_t* base = reinterpret_cast<int64_t*>(w);
  KVZ_LAUNCH("compact_count", cmp_count, (unsigned)p.n_tiles, TPB, 0, st, mask, cnt, head_begin,
             p.tiles_per_head, p.n_c);
  KVZ_LAUNCH("compact_scan", cmp_scan, (unsigned)((p.head_count + 255) / 256), 256, 0, st, cnt,
             head_offsets, base, head_begin, p.head_count, p.tiles_per_head);
#define KVZ_SCATTER(RC)                                                                   \
  KVZ_LAUNCH("compact_scatter", cmp_scatter<RC>, (unsigned)p.n_tiles, TPB, 0, st,          \
             (const u32x4*)kc, (const u32x4*)vc, mask, head_offsets, base, (u32x4*)ko,      \
             (u32x4*)vo, idx, head_begin, p.tiles_per_head, p.n_c)
  switch (row_bytes / 16) {
    case 8: KVZ_SCATTER(8); break;
    case 16: KVZ_SCATTER(16); break;
    case 32: KVZ_SCATTER(32); break;
    case 64: KVZ_SCATTER(64); break;
    default: return hipErrorInvalidValue;
  }
#undef KVZ_SCATTER
  return hipGetLastError();
}

}  // namespace kvz
