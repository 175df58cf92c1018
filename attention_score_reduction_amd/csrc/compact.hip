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

__global__ __launch_bounds__(TPB) void cmp_scatter(
    const uint4* __restrict__ kc, const uint4* __restrict__ vc, const uint8_t* __restrict__ mask,
    const int64_t* __restrict__ head_offsets, const int64_t* __restrict__ base,
    uint4* __restrict__ ko, uint4* __restrict__ vo, int32_t* __restrict__ idx,
    int64_t head_begin, int tiles_per_head, int n_c, int row_chunks) {
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
  const int count = run;
  const int64_t o0 = base[tile];
  // never write past this head's range, whatever the offsets say
  const int64_t lim = head_offsets[head_begin + hh + 1];
  const int64_t head_row0 = hh * (int64_t)n_c;  // k/v pointers start at head_begin
  for (int k = t; k < count; k += TPB)
    if (o0 + k < lim) idx[o0 + k] = list[k];
  const int total = count * row_chunks;
  for (int x = t; x < total; x += TPB) {
    const int k = x / row_chunks, c = x - k * row_chunks;
    const int64_t o = o0 + k;
    if (o >= lim) continue;
    const int64_t src = (head_row0 + list[k]) * row_chunks + c;
    ko[o * row_chunks + c] = kc[src];
    vo[o * row_chunks + c] = vc[src];
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
  KVZ_LAUNCH("compact_scatter", cmp_scatter, (unsigned)p.n_tiles, TPB, 0, st,
             (const uint4*)kc, (const uint4*)vc, mask, head_offsets, base, (uint4*)ko,
             (uint4*)vo, idx, head_begin, p.tiles_per_head, p.n_c, row_bytes / 16);
  return hipGetLastError();
}

}  // namespace kvz
