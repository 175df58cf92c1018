// Reconstruction-attention scoring of one chunk (all KV heads of one layer).
//
// What is computed (KVzip blog post, sections 4.3.1 and 4.3.2; paperhub
// rebuttal, answer on positional OOD): for every KV head h, query head g of
// its group and query row i of the chunk, p = softmax(scale * q . k) over all
// n_c context keys followed by the chunk's own keys 0..i; the score of
// context key j is the running max over chunks of max_{g,i} p[j].
//
// Two passes, neither of which materialises the (G*n_in) x (n_c + n_in)
// probability matrix (the blog's section 4.4 explains why a FlashAttention
// kernel that only returns P*V cannot give max_i softmax):
//   pass 1  per query row, lse = log2 sum_j 2^(x_j * scale * log2 e) over the
//           visible keys, by an online max/sum over 32-key tiles; the key
//           axis is split over workgroups and merged by score_combine;
//   pass 2  per context key, t_j = max over rows (x * scale * log2 e - lse),
//           then S_j = max(S_j, 2^t_j).  max_i 2^(y_i) = 2^(max_i y_i), so
//           pass 2 needs one exp per key, not per logit.
// Query rows are packed i-major (r = i*G + g) so that a tile of consecutive
// rows shares nearly the same causal limit.
//
// bf16 path: 32x32x16 bf16 MFMA with fp32 accumulation, K (pass 1) or Q
// (pass 2) tiles staged in LDS with an XOR swizzle of 16-byte chunks, the
// other operand held in registers for the whole key or row sweep.  Pass 1
// computes K*Q^T (keys on the MFMA row axis) so its reduction over keys is
// in-lane; pass 2 computes Q*K^T so its reduction over rows is in-lane.
// fp32 path: plain VALU kernels for small fp32 problems.
#include <math.h>

#include <type_traits>

#include "common.h"

namespace kvz {

KVZ_DEBUG_WORD(debug_word_score)

namespace {

constexpr int KT = 32;          // keys per pass-1 tile
constexpr float kNegBig = -1e30f;

#ifndef KVZ_P1_TARGET_WGS
#define KVZ_P1_TARGET_WGS 4096  // pass-1 workgroups aimed for per call (sets the key splits)
#endif

template <int D>
struct Geo {
  static constexpr int KS = D / 16;                 // MFMA k-steps over d
  static constexpr int CH = D / 8;                  // 16-byte chunks per row
  static constexpr int SWZ = (CH < 16 ? CH : 16) - 1;
};

template <int CH, int SWZ>
__device__ __forceinline__ int swz(int row, int ch) {
  return row * CH + (ch ^ (row & SWZ));
}

// Exact online max/sum of 16 logits (raw dot products) into (m, l), log2
// domain: raise m to the tile max, rescale l, add the tile's terms.
__device__ __forceinline__ void online_update(const f32x16& a, float& m, float& l, float cl2) {
  float mx = a[0];
#pragma unroll
  for (int v = 1; v < 16; ++v) mx = fmaxf(mx, a[v]);
  const float mn = fmaxf(m, mx * cl2);
  float s0 = fast_exp2(fmaf(a[0], cl2, -mn)), s1 = fast_exp2(fmaf(a[1], cl2, -mn));
  float s2 = fast_exp2(fmaf(a[2], cl2, -mn)), s3 = fast_exp2(fmaf(a[3], cl2, -mn));
#pragma unroll
  for (int v = 4; v < 16; v += 4) {
    s0 += fast_exp2(fmaf(a[v + 0], cl2, -mn));
    s1 += fast_exp2(fmaf(a[v + 1], cl2, -mn));
    s2 += fast_exp2(fmaf(a[v + 2], cl2, -mn));
    s3 += fast_exp2(fmaf(a[v + 3], cl2, -mn));
  }
  l = l * fast_exp2(m - mn) + ((s0 + s1) + (s2 + s3));
  m = mn;
}

// Sum of 2^(x*cl2 - m) over 16 logits against a fixed (possibly stale) m.
// Lazy rescaling: the running max only moves when a tile's sum exceeds
// kLazyLimit (or is inf/NaN-free but huge), which bounds every term by 2^30
// relative to m; the common tile then costs one fma, one exp and one add per
// logit instead of an extra max.  l stays below 2^30 * tiles, far from fp32
// overflow, and m - log2(l) is unchanged by the choice of m.
constexpr float kLazyLimit = 1073741824.f;  // 2^30

__device__ __forceinline__ float tile_sum(const f32x16& a, float m, float cl2) {
  float e[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) e[v] = fast_exp2(fmaf(a[v], cl2, -m));
  return (((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]))) +
         (((e[8] + e[9]) + (e[10] + e[11])) + ((e[12] + e[13]) + (e[14] + e[15])));
}

// Commit the tile sums of a lane's NQ query columns; one branch for all so
// that every sum is computed before it (and overlaps the MFMAs).
template <int NQ>
__device__ __forceinline__ void lazy_commit(const f32x16 (&a)[NQ], const float (&sm)[NQ],
                                            float (&m)[NQ], float (&l)[NQ], float cl2) {
  float big = sm[0];
#pragma unroll
  for (int t = 1; t < NQ; ++t) big = fmaxf(big, sm[t]);
  if (big <= kLazyLimit) {
#pragma unroll
    for (int t = 0; t < NQ; ++t) l[t] += sm[t];
  } else {
#pragma unroll
    for (int t = 0; t < NQ; ++t) {
      if (sm[t] <= kLazyLimit)
        l[t] += sm[t];
      else
        online_update(a[t], m[t], l[t], cl2);
    }
  }
}

// Pass-1 exp work of one tile, NE logits per lane, spread over the NCH MFMAs
// of the next tile: chunk c (the VALU work issued before MFMA c) takes logits
// [chunk_lo(c), chunk_lo(c+1)).  Chunk 0 takes a quarter of them, so the first
// MFMA's wait for its LDS operand is covered; the rest are spread evenly.
template <int NE, int NCH>
__device__ constexpr int chunk_lo(int c) {
  return c <= 0 ? 0 : NE / 4 + (c - 1) * (NE - NE / 4) / (NCH - 1);
}

// Row index (within a 32x32 MFMA output tile) held by accumulator v of a lane.
__device__ __forceinline__ int acc_row(int v, int half) {
  return 8 * (v >> 2) + 4 * half + (v & 3);
}

// ---------------------------------------------------------------------------
// pass 1, bf16: partial (max, sum) per query row and key split
// grid: H x splits x row tiles (XCD-remapped: head-major, row tile fastest)
//
// Each wave keeps NQ 32-row query tiles in registers (the B operand of
// K*Q^T) and sweeps 32-key tiles of K staged in LDS; every A operand read
// from LDS feeds NQ MFMAs.  Main loop (every tile but a ragged last one),
// software-pipelined: iteration t reads its first A operands of tile t+1,
// starts the global -> LDS copy of tile t+2 into the buffer tile t occupied
// (buffer loads with an LDS destination: no register staging), issues the
// NQ*KS MFMAs of tile t+1 into one accumulator set and, between them in a
// fixed order, the exp/sum work of tile t from the other set; then it waits
// for its copies and passes one barrier.  A operands are read AW k-steps
// ahead.  The online sum is lazy (tile_sum).  The causal chunk keys run the
// same loop with the mask in the accumulator start; the ragged last context
// tile takes a simple unpipelined path.
// ---------------------------------------------------------------------------
template <int D>
struct P1Shape {
  // query tiles per wave: two at d <= 128 (each LDS operand read feeds two
  // MFMAs); one at d=256, where two would need 300 VGPRs (occupancy 1) and
  // measured 10% slower
  static constexpr int NQ = D <= 128 ? 2 : 1;
  static constexpr int ROWS = 4 * 32 * NQ;                     // query rows per workgroup
};

// arguments of one pass-1 launch (one chunk, all heads)
struct P1Args {
  const uint16_t* q;     // [H][G][n_in][d]
  const uint16_t* kc;    // [H][n_c][d]
  const uint16_t* kin;   // [H][n_in][d]
  float2* part;          // [H][splits][R_pad] partial (max, sum), g-major rows
  int G, n_c, n_in, R, R_pad, n_rt, n_split_ctx, tiles_per_split;
  float cl2;
  int n_blocks;          // H * splits * n_rt
};

// key tiles of pass-1 item lb: [t_begin, t_clean) run the pipelined loop,
// [t_clean, t_end) the masked path (the ragged last context tile).  The
// context splits cover tiles_per_split 32-key tiles of the n_c context keys;
// the in-chunk split covers the causal chunk keys up to the last row of the
// item's row tile.
struct P1Range {
  int t_begin, t_end, t_clean;
};

template <int D>
__device__ __forceinline__ P1Range p1_range(const P1Args& a, int lb) {
  const int splits = a.n_split_ctx + 1;
  const int rt = lb % a.n_rt;
  const int s = (lb / a.n_rt) % splits;
  P1Range r;
  if (s != a.n_split_ctx) {
    const int n_tiles_ctx = (a.n_c + KT - 1) / KT;
    r.t_begin = s * a.tiles_per_split;
    r.t_end = min(n_tiles_ctx, r.t_begin + a.tiles_per_split);
    r.t_clean = (r.t_end == n_tiles_ctx && (a.n_c % KT) != 0) ? r.t_end - 1 : r.t_end;
  } else {
    const int rlast = min(a.R, (rt + 1) * P1Shape<D>::ROWS) - 1;
    r.t_begin = 0;
    r.t_end = (rlast / a.G) / KT + 1;
    r.t_clean = r.t_end;  // pipelined, causal mask in the accumulator start
  }
  return r;
}

// one pass-1 workgroup item lb (head, key split, row tile), run by 256
// threads whose local index is tid
template <int D>
__device__ __forceinline__ void p1_block(const P1Args& args, int lb, int tid) {
  constexpr int KS = Geo<D>::KS, CH = Geo<D>::CH, SWZ = Geo<D>::SWZ;
  constexpr int NQ = P1Shape<D>::NQ, ROWS = P1Shape<D>::ROWS;
  constexpr int LOADS = KT * CH / 256;
  constexpr int AW = KS <= 8 ? KS : 4;  // A-operand k-steps held at once
  __shared__ uint4 lds0[KT * CH], lds1[KT * CH];

  const uint16_t* __restrict__ q = args.q;
  const uint16_t* __restrict__ kc = args.kc;
  const uint16_t* __restrict__ kin = args.kin;
  float2* __restrict__ part = args.part;
  const int G = args.G, n_c = args.n_c, n_in = args.n_in, R = args.R, R_pad = args.R_pad;
  const int n_rt = args.n_rt, n_split_ctx = args.n_split_ctx;
  const int tiles_per_split = args.tiles_per_split;
  const float cl2 = args.cl2;
  const int splits = n_split_ctx + 1;
  const int rt = lb % n_rt;
  const int s = (lb / n_rt) % splits;
  const int h = lb / (n_rt * splits);

  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, half = lane >> 5;

  const bool inchunk = (s == n_split_ctx);
  const P1Range rg = p1_range<D>(args, lb);
  const int t_begin = rg.t_begin, t_end = rg.t_end, t_clean = rg.t_clean;
  const uint16_t* kbase = inchunk ? kin + (size_t)h * n_in * D : kc + (size_t)h * n_c * D;
  const int nkeys = inchunk ? n_in : n_c;

  // stationary query operand (B of K*Q^T): this lane's query column n of
  // each of the wave's NQ row tiles
  bf16x8 qr[NQ][KS];
  int irow[NQ], grow[NQ];
#pragma unroll
  for (int t = 0; t < NQ; ++t) {
    const int r = rt * ROWS + wave * (32 * NQ) + t * 32 + n;
    irow[t] = r / G;
    grow[t] = r - irow[t] * G;
    if (r < R) {
      const uint16_t* p = q + ((size_t)(h * G + grow[t]) * n_in + irow[t]) * D + half * 8;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qr[t][ks] = as_bf16x8(ld16(p + ks * 16));
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qr[t][ks] = as_bf16x8(make_uint4(0, 0, 0, 0));
    }
  }

  // a wave whose rows are all padding (only in the last row tile) still
  // copies its share of every K tile and passes the barriers, but skips the
  // MFMAs and exps, leaving its SIMD to the other resident waves
  const bool live = rt * ROWS + wave * (32 * NQ) < R;

  float m[NQ], l[NQ];
#pragma unroll
  for (int t = 0; t < NQ; ++t) {
    m[t] = kNegBig;
    l[t] = 0.f;
  }
  // LDS buffers of the K tiles, as two objects so that the copy into one
  // is never taken to alias the operand reads from the other
  auto ldsb = [&](int b) -> uint4* { return b ? lds1 : lds0; };
  uint4 reg[LOADS];
  auto load_tile = [&](int tile) {
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      const int c = tid + 256 * u, row = c / CH, ch = c % CH, key = tile * KT + row;
      reg[u] = key < nkeys ? ld16(kbase + (size_t)key * D + ch * 8) : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      const int c = tid + 256 * u, row = c / CH, ch = c % CH;
      ldsb(buf)[swz<CH, SWZ>(row, ch)] = reg[u];
    }
  };
  auto mfma_tile = [&](int buf, f32x16 (&c)[NQ]) {
    const f32x16 z = {};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 a = as_bf16x8(ldsb(buf)[swz<CH, SWZ>(n, ks * 2 + half)]);
#pragma unroll
      for (int t = 0; t < NQ; ++t)
        c[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qr[t][ks], ks == 0 ? z : c[t], 0, 0, 0);
    }
  };

  const int nclean = t_clean - t_begin;
  if (nclean > 0) {
    // Tile t (relative to t_begin) lives in LDS buffer t & 1.  Tiles of the
    // clean range go global -> LDS by buffer loads with an LDS destination:
    // one such load fills 64 consecutive 16-byte slots, one per lane, so each
    // lane fetches the (key, chunk) that the swizzled layout puts in its slot.
    // Indices past the range re-copy the last tile; those copies are never
    // consumed.
    constexpr int NCH = NQ * KS;      // one chunk of VALU work per MFMA
    constexpr int NE = 16 * NQ;       // logits per lane per tile
    f32x16 A[NQ], B[NQ];
    const int last = nclean - 1;
    const uint16_t* kseg = kbase + (size_t)t_begin * KT * D;
    const int seg_bytes = (nkeys - t_begin * KT) * D * 2;
    int koff[LOADS];
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      const int slot = (u * 4 + wave) * 64 + lane;
      const int row = slot / CH, ch = (slot % CH) ^ (row & SWZ);
      koff[u] = row * D * 2 + ch * 16;
    }
    auto copy_tile = [&](int rt_, int buf) {
#pragma unroll
      for (int u = 0; u < LOADS; ++u)
        copy16_to_lds(kseg, seg_bytes, koff[u] + rt_ * (KT * D * 2), ldsb(buf) + (u * 4 + wave) * 64);
    };
    // The causal in-chunk split runs the same loop with its mask in the
    // accumulator start: for query tile t, the MFMA over the first k-step
    // of a key tile starts at 0 on the keys its row sees and -inf on the
    // keys past it, so every logit consumer (exp/sum, lazy commit, exact
    // fallback) sees -inf there.  Instantiated twice (CAUSAL false/true) so
    // the context splits keep their zero start.
    auto run = [&](auto causal_c) {
      constexpr bool CAUSAL = decltype(causal_c)::value;
      auto mfma_first = [&](const bf16x8& a, const bf16x8& b, int tile, int t) -> f32x16 {
        if constexpr (CAUSAL) {
          // key row k of the tile is visible to this lane's row iff k <= lim
          const int lim = irow[t] - tile * KT - 4 * half;
          f32x16 zz;
#pragma unroll
          for (int v = 0; v < 16; ++v) zz[v] = 8 * (v >> 2) + (v & 3) > lim ? -INFINITY : 0.f;
          return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, zz, 0, 0, 0);
        } else {
          const f32x16 z = {};
          return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, z, 0, 0, 0);
        }
      };
      copy_tile(0, 0);
      copy_tile(min(1, last), 1);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 a = as_bf16x8(ldsb(0)[swz<CH, SWZ>(n, ks * 2 + half)]);
#pragma unroll
        for (int t = 0; t < NQ; ++t)
          A[t] = ks == 0 ? mfma_first(a, qr[t][0], t_begin, t)
                         : __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qr[t][ks], A[t], 0, 0, 0);
      }
      __syncthreads();  // every wave has read buffer 0 before it is refilled
      // iteration it (parity par = it & 1, a literal at each call): MFMAs of
      // tile it+1, exp/sum work of tile it, copy of tile it+2 into the buffer
      // tile it occupied
      auto body = [&](int it, f32x16 (&cur)[NQ], f32x16 (&nxt)[NQ], int par) {
        const int buf = par ^ 1;
        if (!live) {
          copy_tile(min(it + 2, last), par);
          __builtin_amdgcn_s_waitcnt(0);
          __syncthreads();
          return;
        }
        bf16x8 a[AW];
#pragma unroll
        for (int ks = 0; ks < AW; ++ks)
          a[ks] = as_bf16x8(ldsb(buf)[swz<CH, SWZ>(n, ks * 2 + half)]);
        copy_tile(min(it + 2, last), par);
        __builtin_amdgcn_sched_barrier(0);
        float sm[NQ][4], ex[NE];
        // three-stage VALU pipeline over the chunks: the fma of a logit is
        // issued one chunk (one MFMA) before its exp, and its add one chunk
        // after, so no VALU op waits on the result of the op just before it
        auto fma_chunk = [&](int c) {
#pragma unroll
          for (int e = chunk_lo<NE, NCH>(c); e < chunk_lo<NE, NCH>(c + 1); ++e) {
            const int col = e >> 4, v = e & 15;
            ex[e] = fmaf(cur[col][v], cl2, -m[col]);
          }
        };
        auto exp_chunk = [&](int c) {
#pragma unroll
          for (int e = chunk_lo<NE, NCH>(c); e < chunk_lo<NE, NCH>(c + 1); ++e)
            ex[e] = fast_exp2(ex[e]);
        };
        auto add_chunk = [&](int c) {
#pragma unroll
          for (int e = chunk_lo<NE, NCH>(c); e < chunk_lo<NE, NCH>(c + 1); ++e) {
            const int col = e >> 4, v = e & 15;
            if (v < 4) sm[col][v] = ex[e]; else sm[col][v & 3] += ex[e];
          }
        };
        fma_chunk(0);
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
          // logits [chunk_lo(c), chunk_lo(c+1)) of this lane's 16*NQ
          exp_chunk(c);
          if (c + 1 < NCH) fma_chunk(c + 1);
          if (c > 0) add_chunk(c - 1);
          __builtin_amdgcn_sched_barrier(0);
          const int ks = c / NQ, t = c % NQ;
          nxt[t] = ks == 0 ? mfma_first(a[0], qr[t][0], t_begin + it + 1, t)
                           : __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks % AW], qr[t][ks], nxt[t],
                                                                     0, 0, 0);
          if (t == NQ - 1 && ks + AW < KS)
            a[ks % AW] = as_bf16x8(ldsb(buf)[swz<CH, SWZ>(n, (ks + AW) * 2 + half)]);
          __builtin_amdgcn_sched_barrier(0);
        }
        add_chunk(NCH - 1);
        float tot[NQ];
#pragma unroll
        for (int t = 0; t < NQ; ++t) tot[t] = (sm[t][0] + sm[t][1]) + (sm[t][2] + sm[t][3]);
        lazy_commit<NQ>(cur, tot, m, l, cl2);
        __builtin_amdgcn_s_waitcnt(0);  // this wave's copy of tile it+2 has landed
        __syncthreads();
      };
      auto finish = [&](f32x16 (&cur)[NQ]) {
        float tot[NQ];
#pragma unroll
        for (int t = 0; t < NQ; ++t) tot[t] = tile_sum(cur[t], m[t], cl2);
        lazy_commit<NQ>(cur, tot, m, l, cl2);
      };
      int it = 0;
      for (; it + 2 < nclean; it += 2) {
        body(it, A, B, 0);
        body(it + 1, B, A, 1);
      }
      if (it + 1 < nclean) {
        body(it, A, B, 0);
        finish(B);
      } else {
        finish(A);
      }
    };
    if (inchunk)
      run(std::true_type{});
    else
      run(std::false_type{});
  }

  // masked tiles: the ragged context tail
  for (int tile = t_clean; tile < t_end; ++tile) {
    __syncthreads();
    load_tile(tile);
    store_tile(0);
    __syncthreads();
    if (!live) continue;
    f32x16 c[NQ];
    mfma_tile(0, c);
    const int key0 = tile * KT;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int key = key0 + acc_row(v, half);
#pragma unroll
      for (int t = 0; t < NQ; ++t)
        if (key >= n_c) c[t][v] = -INFINITY;
    }
#pragma unroll
    for (int t = 0; t < NQ; ++t) online_update(c[t], m[t], l[t], cl2);
  }

  // lanes n and n+32 hold the same query column, different key rows
#pragma unroll
  for (int t = 0; t < NQ; ++t) {
    const float mo = __shfl_xor(m[t], 32);
    const float lo = __shfl_xor(l[t], 32);
    const float M = fmaxf(m[t], mo);
    const float L = l[t] * fast_exp2(m[t] - M) + lo * fast_exp2(mo - M);
    const int r = rt * ROWS + wave * (32 * NQ) + t * 32 + n;
    if (half == 0 && r < R) {
      // partials and lse are stored in g-major row order (g * n_in + i)
      part[((size_t)h * splits + s) * R_pad + grow[t] * n_in + irow[t]] = make_float2(M, L);
    }
  }
}

template <int D>
__global__ __launch_bounds__(256) void score_pass1_bf16(P1Args args) {
  const int lb = xcd_logical_block();
  if (lb >= args.n_blocks) return;
  p1_block<D>(args, lb, threadIdx.x);
}

// merge the key splits: lse2 = M + log2(sum_s l_s 2^(m_s - M)), written
// times mul (1, or -1/(scale log2 e) when pass 2 takes it in raw dot-product
// units); padding rows get +inf * mul so that pass 2 ignores them.
__global__ __launch_bounds__(256) void score_combine(const float2* __restrict__ part,
                                                     float* __restrict__ lse2, int splits,
                                                     int R, int R_pad, int H, float mul) {
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= H * R_pad) return;
  const int h = idx / R_pad, r = idx - h * R_pad;
  if (r >= R) {
    lse2[idx] = INFINITY * mul;
    return;
  }
  const float2* p = part + (size_t)h * splits * R_pad + r;
  // unrolled so that the split loads are in flight together
  float M = kNegBig;
#pragma unroll 8
  for (int s = 0; s < splits; ++s) M = fmaxf(M, p[(size_t)s * R_pad].x);
  // compensated (Kahan) sum over the splits: with thousands of splits, one
  // of them can hold nearly all of the row's weight while the others each
  // add less than an ulp of it
  float L = 0.f, c = 0.f;
#pragma unroll 8
  for (int s = 0; s < splits; ++s) {
    const float2 v = p[(size_t)s * R_pad];
    kahan_add(L, c, v.y * exp2f(v.x - M));
  }
  KVZ_DCHECK(isfinite(M + log2f(L)), 1u);  // NaN or inf in q or the keys
  lse2[idx] = (M + log2f(L)) * mul;
}

// ---------------------------------------------------------------------------
// pass 2, bf16: column max over all query rows, running max into S
// grid: H x key blocks (XCD-remapped: head-major)
//
// Each wave keeps NT 32-key tiles of K in registers (128 keys for d <= 128)
// and sweeps 32-row query tiles staged in LDS (double buffer, one barrier per
// tile); every A operand read from LDS feeds NT MFMAs.  The epilogue of a key
// tile (fma with the row lse and a running max, or the sum / raw variants)
// overlaps the MFMAs of the following key tiles of the same query tile.
// Padding rows (r >= R) of the last row tile read as zero queries and carry
// lse = +inf (raw logits: a -inf accumulator start).
// MODE: 0 = max of probabilities (the method), 1 = sum of probabilities,
// 2 = max of raw logits scale * q . k (no softmax; lse2 unused)
// ---------------------------------------------------------------------------
template <int D>
struct P2Shape {
  static constexpr int NT = D <= 128 ? 4 : 2;    // key tiles per wave
  static constexpr int KEYS = 4 * 32 * NT;       // keys per workgroup
};

// arguments of one pass-2 launch (one chunk, all heads)
struct P2Args {
  const uint16_t* q;     // [H][G][n_in][d]
  const uint16_t* kc;    // [H][n_c][d]
  const float* lse2;     // [H][R_pad] row log-sum-exp (or its pass-2 form)
  float* S;              // [H][n_c]
  int G, n_c, n_in, R, R_pad, n_kt;
  float cl2, scale;
  int n_blocks;          // H * n_kt
};

// one pass-2 workgroup item lb (head, block of 4 * 32 * NT keys), run by 256
// threads whose local index is tid
template <int D, int MODE, int NT>
__device__ __forceinline__ void p2_block(const P2Args& args, int lb, int tid) {
  constexpr int KS = Geo<D>::KS, CH = Geo<D>::CH, SWZ = Geo<D>::SWZ;
  constexpr int RT = 32;                     // query rows per tile
  constexpr int LOADS = RT * CH / 256;       // 16-byte copies per thread per tile
  __shared__ uint4 ldq[2][RT * CH];
  // the tile's 32 row lse values (8 float4); 64 slots, one per lane of the
  // copying wave, although only 8 lanes copy
  __shared__ float4 ldl[2][64];

  const uint16_t* __restrict__ q = args.q;
  const uint16_t* __restrict__ kc = args.kc;
  const float* __restrict__ lse2 = args.lse2;
  float* __restrict__ S = args.S;
  const int n_c = args.n_c, R = args.R, R_pad = args.R_pad, n_kt = args.n_kt;
  const float cl2 = args.cl2, scale = args.scale;
  const int kt = lb % n_kt;
  const int h = lb / n_kt;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, half = lane >> 5;
  const int j0 = kt * (4 * 32 * NT) + wave * (32 * NT);

  // stationary key operand (B of Q*K^T): this lane's key column n of each
  // tile; keys past n_c re-read key n_c - 1 and are never written back
  bf16x8 kr[NT][KS];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int j = min(j0 + t * 32 + n, n_c - 1);
    const uint16_t* p = kc + ((size_t)h * n_c + j) * D + half * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kr[t][ks] = as_bf16x8(ld16(p + ks * 16));
  }

  // Query tiles go global -> LDS by buffer loads with an LDS destination (no
  // register staging).  One such load writes 64 consecutive 16-byte LDS slots,
  // one per lane, so each lane fetches the (row, chunk) that the swizzled
  // layout puts in its slot.  The buffer covers the R rows of head h: padding
  // rows (r >= R) fall outside it and read as zero (they carry lse = +inf).
  // row tiles holding real rows (the padding up to R_pad adds nothing)
  const int n_tiles = (R + RT - 1) / RT;
  const uint16_t* qh = q + (size_t)h * R * D;
  const float* lseh = lse2 + (size_t)h * R_pad;
  int qoff[LOADS];
#pragma unroll
  for (int u = 0; u < LOADS; ++u) {
    const int slot = (u * 4 + wave) * 64 + lane;
    const int row = slot / CH, ch = (slot % CH) ^ (row & SWZ);
    qoff[u] = row * D * 2 + ch * 16;
  }
  auto copy_tile = [&](int t, int buf) {
#pragma unroll
    for (int u = 0; u < LOADS; ++u)
      copy16_to_lds(qh, R * D * 2, qoff[u] + t * (RT * D * 2), &ldq[buf][(u * 4 + wave) * 64]);
    if (MODE != 2 && wave == 0 && lane < RT / 4)
      copy16_to_lds(lseh, R_pad * 4, (t * RT + 4 * lane) * 4, &ldl[buf][0]);
  };

  const float init = MODE == 1 ? 0.f : -INFINITY;
  // sum mode: a key's sum runs over every query row (up to 2^20); each key
  // tile's terms are summed on their own and folded into acc with Kahan
  // compensation (comp), so that small terms are not lost against the total
  float acc[NT], comp[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = init, comp[t] = 0.f;

  // epilogue of one key tile: elements 2p, 2p+1 for p in [p0, p1).  MODE 0
  // and 2 need only a running max: for MODE 0 the MFMA accumulator starts at
  // -lse2/(scale log2 e) of its row, so its output is already the row's
  // log-probability in dot-product units, and the scaling waits until after
  // the max (it is positive).
  // (sum mode: into the tile sum ts instead of acc)
  auto epilogue = [&](const f32x16& c, const float4 (&L)[4], float& ts, int t, int p0, int p1) {
#pragma unroll
    for (int pr = p0; pr < p1; ++pr) {
      const int v = 2 * pr;
      const float x0 = c[v], x1 = c[v + 1];
      if (MODE != 1) {
        acc[t] = fmaxf(fmaxf(acc[t], x0), x1);
      } else {
        const float4 L4 = L[v >> 2];
        const float l0 = (v & 3) == 0 ? L4.x : L4.z, l1 = (v & 3) == 0 ? L4.y : L4.w;
        ts += fast_exp2(fmaf(x0, cl2, -l0)) + fast_exp2(fmaf(x1, cl2, -l1));
      }
    }
  };
  auto fold = [&](float ts, int t) {
    if constexpr (MODE == 1) kahan_add(acc[t], comp[t], ts);
  };

  // one query tile: read this tile's operands from LDS, start the copy of the
  // next tile into the idle buffer, MFMAs and epilogues, then wait for this
  // wave's copies and pass the barrier.  The last tile re-copies itself into the idle buffer (never
  // read again): no branch in the body.
  auto body = [&](int it, int buf) {
    // lse of the 16 rows this lane holds in the MFMA output (rows 8*vg + 4*half + 0..3)
    float4 L[4];
    if (MODE != 2) {
#pragma unroll
      for (int vg = 0; vg < 4; ++vg) L[vg] = ldl[buf][2 * vg + half];
    }
    bf16x8 a[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) a[ks] = as_bf16x8(ldq[buf][swz<CH, SWZ>(n, ks * 2 + half)]);
    // issued after this tile's LDS reads, so that no read waits for the copy
    copy_tile(min(it + 1, n_tiles - 1), buf ^ 1);
    f32x16 c[NT], z;
    if (MODE == 0) {
      // accumulator start: -lse2/(scale log2 e) of the lane's 16 rows
#pragma unroll
      for (int v = 0; v < 16; ++v) z[v] = L[v >> 2][v & 3];
    } else if (MODE == 2) {
      // raw logits: padding rows (r >= R, zero queries) start at -inf so
      // that their zero logit never enters the max
      const int r0 = it * RT + 4 * half;
#pragma unroll
      for (int v = 0; v < 16; ++v) z[v] = r0 + 8 * (v >> 2) + (v & 3) < R ? 0.f : -INFINITY;
    } else {
      z = f32x16{};  // sum: padding rows carry lse = +inf and add 0
    }
    float ts[NT] = {};
    __builtin_amdgcn_sched_barrier(0);
    // MFMAs of key tile t, each followed by a share of key tile t-1's epilogue
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        c[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks], kr[t][ks], ks == 0 ? z : c[t], 0, 0,
                                                       0);
        if (t > 0) epilogue(c[t - 1], L, ts[t - 1], t - 1, ks * 8 / KS, (ks + 1) * 8 / KS);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (t > 0) fold(ts[t - 1], t - 1);
    }
    epilogue(c[NT - 1], L, ts[NT - 1], NT - 1, 0, 8);
    fold(ts[NT - 1], NT - 1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };

  copy_tile(0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int it = 0; it < n_tiles; ++it) body(it, it & 1);

#pragma unroll
  for (int t = 0; t < NT; ++t) {
    // lanes n and n+32 hold the same key column, different rows
    const float o = __shfl_xor(acc[t], 32);
    const float r = MODE == 1 ? acc[t] + o : fmaxf(acc[t], o);
    const int j = j0 + t * 32 + n;
    if (half == 0 && j < n_c) {
      float* sp = S + (size_t)h * n_c + j;
      if (MODE == 0)
        *sp = fmaxf(*sp, fminf(fast_exp2(r * cl2), 1.0f));
      else if (MODE == 1)
        *sp += r;
      else
        *sp = fmaxf(*sp, r * scale);
    }
  }
}

template <int D, int MODE>
__global__ __launch_bounds__(256) void score_pass2_bf16(P2Args args) {
  const int lb = xcd_logical_block();
  if (lb >= args.n_blocks) return;
  p2_block<D, MODE, P2Shape<D>::NT>(args, lb, threadIdx.x);
}

// ---------------------------------------------------------------------------
// fp32 path (VALU): one thread per query row (pass 1) / per context key (pass 2)
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(64) void score_pass1_f32(const float* __restrict__ q,
                                                      const float* __restrict__ kc,
                                                      const float* __restrict__ kin,
                                                      float* __restrict__ lse2, int G, int n_c,
                                                      int n_in, int R, int R_pad, float cl2) {
  __shared__ float ldq[D][64];
  __shared__ float ldk[KT][D + 1];
  const int h = blockIdx.y;
  const int tid = threadIdx.x;
  const int r = blockIdx.x * 64 + tid;
  const int i = r / G, g = r - (r / G) * G;
  for (int k = 0; k < D; ++k)
    ldq[k][tid] = (r < R) ? q[((size_t)(h * G + g) * n_in + i) * D + k] : 0.f;
  // one thread sums a row's terms over every key it sees (up to ~2^24):
  // compensated (Kahan) summation keeps the terms far below the running
  // sum, which a plain fp32 sum would drop, in the total
  float m = kNegBig, l = 0.f, c = 0.f;
  const int n_ctx_tiles = (n_c + KT - 1) / KT;
  const int imax = (min(R, (int)(blockIdx.x + 1) * 64) - 1) / G;
  const int n_tiles = n_ctx_tiles + imax / KT + 1;
  for (int tile = 0; tile < n_tiles; ++tile) {
    const bool ctx = tile < n_ctx_tiles;
    const int key0 = ctx ? tile * KT : (tile - n_ctx_tiles) * KT;
    const float* kb = ctx ? kc + (size_t)h * n_c * D : kin + (size_t)h * n_in * D;
    const int nk = ctx ? n_c : n_in;
    __syncthreads();
    for (int e = tid; e < KT * D; e += 64) {
      const int kk = e / D, dd = e - kk * D;
      ldk[kk][dd] = (key0 + kk < nk) ? kb[(size_t)(key0 + kk) * D + dd] : 0.f;
    }
    __syncthreads();
    for (int kk = 0; kk < KT; ++kk) {
      const int key = key0 + kk;
      const bool vis = ctx ? key < n_c : key <= i;
      if (!vis) continue;
      float dot = 0.f;
      for (int k = 0; k < D; ++k) dot = fmaf(ldq[k][tid], ldk[kk][k], dot);
      const float x = dot * cl2;
      const float mn = fmaxf(m, x);
      const float a = exp2f(m - mn);
      l *= a;
      c *= a;
      kahan_add(l, c, exp2f(x - mn));
      m = mn;
    }
  }
  KVZ_DCHECK(r >= R || isfinite(m + log2f(l)), 1u);  // NaN or inf in q or the keys
  if (r < R_pad) lse2[(size_t)h * R_pad + r] = (r < R) ? m + log2f(l) : INFINITY;
}

template <int D, int MODE>
__global__ __launch_bounds__(64) void score_pass2_f32(const float* __restrict__ q,
                                                      const float* __restrict__ kc,
                                                      const float* __restrict__ lse2,
                                                      float* __restrict__ S, int G, int n_c,
                                                      int n_in, int R, int R_pad, float cl2,
                                                      float scale) {
  __shared__ float ldk[D][64];
  __shared__ float ldq[32][D + 1];
  __shared__ float ldl[32];
  const int h = blockIdx.y;
  const int tid = threadIdx.x;
  const int j = blockIdx.x * 64 + tid;
  for (int k = 0; k < D; ++k)
    ldk[k][tid] = (j < n_c) ? kc[((size_t)h * n_c + j) * D + k] : 0.f;
  float mx = MODE == 1 ? 0.f : -INFINITY;
  float cmp = 0.f;  // sum mode: Kahan compensation of mx (up to 2^20 rows)
  for (int r0 = 0; r0 < R; r0 += 32) {
    __syncthreads();
    for (int e = tid; e < 32 * D; e += 64) {
      const int rr = e / D, dd = e - rr * D, r = r0 + rr;
      float v = 0.f;
      if (r < R) {
        const int i = r / G, g = r - i * G;
        v = q[((size_t)(h * G + g) * n_in + i) * D + dd];
      }
      ldq[rr][dd] = v;
    }
    if (tid < 32) ldl[tid] = lse2[(size_t)h * R_pad + r0 + tid];
    __syncthreads();
    for (int rr = 0; rr < 32 && r0 + rr < R; ++rr) {
      float dot = 0.f;
      for (int k = 0; k < D; ++k) dot = fmaf(ldq[rr][k], ldk[k][tid], dot);
      if (MODE == 0) mx = fmaxf(mx, dot * cl2 - ldl[rr]);
      else if (MODE == 1) kahan_add(mx, cmp, exp2f(dot * cl2 - ldl[rr]));
      else mx = fmaxf(mx, dot);
    }
  }
  if (j < n_c) {
    float* sp = S + (size_t)h * n_c + j;
    if (MODE == 0) *sp = fmaxf(*sp, fminf(exp2f(mx), 1.0f));
    else if (MODE == 1) *sp += mx;
    else *sp = fmaxf(*sp, mx * scale);
  }
}

template <int D, int MODE>
hipError_t launch_bf16(const ScorePlan& p, const void* q, const void* kc, const void* kin,
                       float scale, float* S, void* ws, hipStream_t st) {
  const float cl2 = scale * 1.4426950408889634f;
  float2* part = reinterpret_cast<float2*>(ws);
  float* lse2 = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + p.part_bytes);
  const int splits = p.n_split_ctx + 1;
  if (MODE != 2) {
    const int nb1 = p.H * splits * p.n_rt;
    const P1Args a1{(const uint16_t*)q, (const uint16_t*)kc, (const uint16_t*)kin, part, p.G,
                    p.n_c, p.n_in, p.R, p.R_pad, p.n_rt, p.n_split_ctx, p.tiles_per_split, cl2,
                    nb1};
    KVZ_LAUNCH("score_pass1", score_pass1_bf16<D>, xcd_padded_grid(nb1), 256, 0, st, a1);
    const int nc = p.H * p.R_pad;
    KVZ_LAUNCH("score_combine", score_combine, (nc + 255) / 256, 256, 0, st, part, lse2, splits,
               p.R, p.R_pad, p.H, MODE == 0 ? -1.0f / cl2 : 1.0f);
  }
  const int n_kt = (p.n_c + P2Shape<D>::KEYS - 1) / P2Shape<D>::KEYS;
  const int nb2 = p.H * n_kt;
  const P2Args a2{(const uint16_t*)q, (const uint16_t*)kc, lse2, S, p.G, p.n_c, p.n_in, p.R,
                  p.R_pad, n_kt, cl2, scale, nb2};
  KVZ_LAUNCH("score_pass2", (score_pass2_bf16<D, MODE>), xcd_padded_grid(nb2), 256, 0, st, a2);
  return hipGetLastError();
}

// the score update from per-split row (max, sum) partials formed elsewhere
// (the fused attention-output pass): split merge into the pass-2 row offsets,
// then pass 2
template <int D>
hipError_t launch_finish_bf16(const ScorePlan& p, const float2* part, int splits, const void* q,
                              const void* kc, float scale, float* S, void* ws, hipStream_t st) {
  const float cl2 = scale * 1.4426950408889634f;
  float* lse2 = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + p.part_bytes);
  const int nc = p.H * p.R_pad;
  KVZ_LAUNCH("score_combine", score_combine, (nc + 255) / 256, 256, 0, st, part, lse2, splits,
             p.R, p.R_pad, p.H, -1.0f / cl2);
  const int n_kt = (p.n_c + P2Shape<D>::KEYS - 1) / P2Shape<D>::KEYS;
  const int nb2 = p.H * n_kt;
  const P2Args a2{(const uint16_t*)q, (const uint16_t*)kc, lse2, S, p.G, p.n_c, p.n_in, p.R,
                  p.R_pad, n_kt, cl2, scale, nb2};
  KVZ_LAUNCH("score_pass2", (score_pass2_bf16<D, 0>), xcd_padded_grid(nb2), 256, 0, st, a2);
  return hipGetLastError();
}

template <int D, int MODE>
hipError_t launch_f32(const ScorePlan& p, const void* q, const void* kc, const void* kin,
                      float scale, float* S, void* ws, hipStream_t st) {
  const float cl2 = scale * 1.4426950408889634f;
  float* lse2 = reinterpret_cast<float*>(ws);
  if (MODE != 2) {
    dim3 g1((p.R + 63) / 64, p.H);
    KVZ_LAUNCH("score_pass1", score_pass1_f32<D>, g1, 64, 0, st, (const float*)q,
               (const float*)kc, (const float*)kin, lse2, p.G, p.n_c, p.n_in, p.R, p.R_pad, cl2);
  }
  dim3 g2((p.n_c + 63) / 64, p.H);
  KVZ_LAUNCH("score_pass2", (score_pass2_f32<D, MODE>), g2, 64, 0, st, (const float*)q,
             (const float*)kc, lse2, S, p.G, p.n_c, p.n_in, p.R, p.R_pad, cl2, scale);
  return hipGetLastError();
}

template <int MODE>
hipError_t launch_mode(kvz_dtype dt, const ScorePlan& p, const void* q, const void* kc,
                       const void* kin, float scale, float* S, void* ws, hipStream_t st) {
  if (dt == KVZ_BF16) {
    switch (p.d) {
      case 64: return launch_bf16<64, MODE>(p, q, kc, kin, scale, S, ws, st);
      case 128: return launch_bf16<128, MODE>(p, q, kc, kin, scale, S, ws, st);
      case 256: return launch_bf16<256, MODE>(p, q, kc, kin, scale, S, ws, st);
    }
  } else {
    switch (p.d) {
      case 64: return launch_f32<64, MODE>(p, q, kc, kin, scale, S, ws, st);
      case 128: return launch_f32<128, MODE>(p, q, kc, kin, scale, S, ws, st);
      case 256: return launch_f32<256, MODE>(p, q, kc, kin, scale, S, ws, st);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace

ScorePlan score_plan(kvz_dtype dt, int H, int G, int n_in, int d, int n_c) {
  ScorePlan p{};
  p.H = H;
  p.G = G;
  p.d = d;
  p.n_c = n_c;
  p.n_in = n_in;
  p.R = G * n_in;
  const int rows = d == 64 ? P1Shape<64>::ROWS : d == 128 ? P1Shape<128>::ROWS
                                                            : P1Shape<256>::ROWS;
  p.n_rt = (p.R + rows - 1) / rows;
  p.R_pad = p.n_rt * rows;  // a multiple of 32 (the pass-2 row tile)
  const int n_ctx_tiles = (n_c + KT - 1) / KT;
  if (dt == KVZ_BF16) {
    // enough workgroups to cover the chip a few times, at least 16 tiles each
    int want = (KVZ_P1_TARGET_WGS + H * p.n_rt - 1) / (H * p.n_rt);
    int maxs = n_ctx_tiles / 16;
    if (maxs < 1) maxs = 1;
    if (want > maxs) want = maxs;
    if (want < 1) want = 1;
    p.tiles_per_split = (n_ctx_tiles + want - 1) / want;
    p.n_split_ctx = (n_ctx_tiles + p.tiles_per_split - 1) / p.tiles_per_split;
    p.part_bytes = align256((size_t)H * (p.n_split_ctx + 1) * p.R_pad * sizeof(float2));
  } else {
    p.tiles_per_split = n_ctx_tiles;
    p.n_split_ctx = 1;
    p.part_bytes = 0;
  }
  p.lse_bytes = align256((size_t)H * p.R_pad * sizeof(float));
  p.total_bytes = p.part_bytes + p.lse_bytes;
  // row indices h * R_pad + r are int; the bf16 grids are XCD-padded
  const int keys2 = d == 64 ? P2Shape<64>::KEYS : d == 128 ? P2Shape<128>::KEYS
                                                           : P2Shape<256>::KEYS;
  const int64_t rows_all = (int64_t)H * p.R_pad;
  const int64_t nb1 = (int64_t)H * (p.n_split_ctx + 1) * p.n_rt;
  const int64_t nb2 = (int64_t)H * ((n_c + keys2 - 1) / keys2);
  p.fits = rows_all < (int64_t(1) << 31) && launch_fits((rows_all + 255) / 256, 256);
  if (dt == KVZ_BF16)
    p.fits = p.fits && launch_fits((nb1 + kNumXcd - 1) / kNumXcd * kNumXcd, 256) &&
             launch_fits((nb2 + kNumXcd - 1) / kNumXcd * kNumXcd, 256);
  return p;
}

hipError_t score_finish_launch(const ScorePlan& p, const float2* part, int splits, const void* q,
                               const void* kc, float scale, float* S, void* ws, hipStream_t st) {
  switch (p.d) {
    case 64: return launch_finish_bf16<64>(p, part, splits, q, kc, scale, S, ws, st);
    case 128: return launch_finish_bf16<128>(p, part, splits, q, kc, scale, S, ws, st);
    case 256: return launch_finish_bf16<256>(p, part, splits, q, kc, scale, S, ws, st);
  }
  return hipErrorInvalidValue;
}

hipError_t score_launch(kvz_dtype dt, kvz_aggregate agg, const ScorePlan& p, const void* q,
                        const void* kc, const void* kin, float scale, float* S, void* ws,
                        hipStream_t st) {
  switch (agg) {
    case KVZ_AGG_MAX: return launch_mode<0>(dt, p, q, kc, kin, scale, S, ws, st);
    case KVZ_AGG_SUM: return launch_mode<1>(dt, p, q, kc, kin, scale, S, ws, st);
    case KVZ_AGG_RAW_MAX: return launch_mode<2>(dt, p, q, kc, kin, scale, S, ws, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace kvz
