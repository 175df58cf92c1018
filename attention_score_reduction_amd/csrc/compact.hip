// Compaction of the kept K/V rows into a packed per-head cache.
//
// After selection the surviving pairs form the reusable compressed cache
// (KVzip blog post, section 4.1 step 5; paperhub rebuttal: the compressed
// cache is built once and reused by later queries).  Heads are laid out one
// after another in flat (layer, head) order, each head's rows in ascending
// token position, with the position stored beside them (idx), so a
// variable-length per-head decode can address it with head_offsets.
//
// Kernels: cmp_offsets (one workgroup per head: kept rows per TILE-position
// tile and the first output row of each tile, by a block scan), cmp_scatter
// (per tile: ranks by wave ballots, then the whole workgroup copies the kept
// rows with 16-byte loads and stores; the writes of a tile land in one
// contiguous range).  Short tiles keep each workgroup's reads and writes in
// a few contiguous ranges and the workgroups short-lived, the pattern that
// streams fastest on this memory system.
#include "common.h"

namespace kvz {

KVZ_DEBUG_WORD(debug_word_compact)

namespace {

// Measured on the 30%-kept 128K cache (10.4 GB moved): tiles of 4096, 1024,
// 256, 128, 64 and 32 positions take 2.02, 1.95, 1.89, 1.85, 1.73 and
// 1.81 ms in the scatter; 64/128-thread workgroups, two copies in flight,
// plain stores, or K and V in separate workgroups are all slower.
constexpr int TILE = 64;   // positions per scatter workgroup
constexpr int TPB = 256;   // threads per workgroup (whole waves)
constexpr int U = 4;       // 16-byte copies in flight per thread and array
static_assert(TPB % 64 == 0, "whole waves");
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int PER_T = (TILE + TPB - 1) / TPB;  // mask bytes per thread in a tile

// nonzero bytes of a 16-byte vector (mask bytes are 0 or 1, but any nonzero
// byte counts as kept, as in cmp_scatter)
__device__ __forceinline__ uint32_t nonzero_bytes(u32x4 v) {
  uint32_t c = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w = v[i];
    c += __popc((((w & 0x7f7f7f7fu) + 0x7f7f7f7fu) | w) & 0x80808080u);
  }
  return c;
}

// kept rows in positions [lo, hi) of one head's mask row (VEC: 16-byte
// loads; lo and hi are multiples of 16 and the row is 16-byte aligned)
template <bool VEC>
__device__ __forceinline__ uint32_t count_kept(const uint8_t* __restrict__ m, int lo, int hi) {
  uint32_t c = 0;
  if constexpr (VEC) {
    const u32x4* v = reinterpret_cast<const u32x4*>(m);
    for (int i = lo / 16; i < hi / 16; i += 4) {
      u32x4 x[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) x[u] = i + u < hi / 16 ? v[i + u] : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int u = 0; u < 4; ++u) c += nonzero_bytes(x[u]);
    }
  } else {
    for (int i = lo; i < hi; ++i) c += m[i] != 0;
  }
  return c;
}

// One workgroup per head: thread t owns a contiguous run of tiles.  Sweep 1
// counts the run's kept rows, a block-wide exclusive scan gives the run's
// first output row, sweep 2 recounts each tile (from L2) and writes its first
// output row to base.
template <bool VEC>
__global__ __launch_bounds__(TPB) void cmp_offsets(const uint8_t* __restrict__ mask,
                                                   const int64_t* __restrict__ head_offsets,
                                                   int64_t* __restrict__ base, int64_t head_begin,
                                                   int tiles_per_head, int n_c) {
  __shared__ uint32_t wtot[TPB / 64];
  const int64_t hh = blockIdx.x;
  const uint8_t* m = mask + (head_begin + hh) * (int64_t)n_c;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int per = (tiles_per_head + TPB - 1) / TPB;
  const int k0 = min(tiles_per_head, t * per), k1 = min(tiles_per_head, k0 + per);
  const uint32_t mine = count_kept<VEC>(m, k0 * TILE, min(n_c, k1 * TILE));
  uint32_t incl = mine;  // inclusive scan over the wave
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == 63) wtot[w] = incl;
  __syncthreads();
#ifdef KVZ_DEBUG
  if (t == 0) {  // the head's kept rows must fill its range of the packed output
    uint32_t kept = 0;
    for (int ww = 0; ww < TPB / 64; ++ww) kept += wtot[ww];
    KVZ_DCHECK((int64_t)kept == head_offsets[head_begin + hh + 1] - head_offsets[head_begin + hh],
               1u);
  }
#endif
  uint32_t before = incl - mine;
  for (int ww = 0; ww < w; ++ww) before += wtot[ww];
  int64_t run = head_offsets[head_begin + hh] + before;
  for (int k = k0; k < k1; ++k) {
    base[hh * tiles_per_head + k] = run;
    run += count_kept<VEC>(m, k * TILE, min(n_c, (k + 1) * TILE));
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
  constexpr int NW = TPB / 64;  // waves per workgroup
  __shared__ uint32_t wtot[PER_T][NW];
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
    f[u] = e < TILE && e < len && m[e] != 0;
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
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) run += wtot[u][ww];
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

// 16-byte mask loads need every head's mask row 16-byte aligned
bool n_c_vec_ok(int n_c, const uint8_t* mask) {
  return n_c % 16 == 0 && (reinterpret_cast<uintptr_t>(mask) & 15u) == 0;
}

}  // namespace

CompactPlan compact_plan(int64_t head_count, int n_c) {
  CompactPlan p{};
  p.head_count = head_count;
  p.n_c = n_c;
  p.tiles_per_head = (int)(((int64_t)n_c + TILE - 1) / TILE);  // n_c may be INT_MAX
  p.n_tiles = head_count * p.tiles_per_head;
  p.total_bytes = align256((size_t)p.n_tiles * sizeof(int64_t));
  return p;
}

hipError_t compact_launch(const CompactPlan& p, int row_bytes, int64_t head_begin, const void* kc,
                          const void* vc, const uint8_t* mask, const int64_t* head_offsets,
                          void* ko, void* vo, int32_t* idx, void* ws, hipStream_t st) {
  int64_t* base = reinterpret_cast<int64_t*>(ws);
  const bool vec = n_c_vec_ok(p.n_c, mask);
  if (vec)
    KVZ_LAUNCH("compact_offsets", cmp_offsets<true>, (unsigned)p.head_count, TPB, 0, st, mask,
               head_offsets, base, head_begin, p.tiles_per_head, p.n_c);
  else
    KVZ_LAUNCH("compact_offsets", cmp_offsets<false>, (unsigned)p.head_count, TPB, 0, st, mask,
               head_offsets, base, head_begin, p.tiles_per_head, p.n_c);
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
