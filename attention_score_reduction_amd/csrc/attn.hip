// Reconstruction attention output of one chunk, beside its scores.
//
// The scoring stage is a full forward over [repeat prompt; chunk] (paperhub
// rebuttal, computational analysis: one MLP pass plus twice the prefill's
// attention work), so each layer's attention also produces the output the
// layer above consumes:
//     O[h][g][i] = sum over visible keys j of p_ij * v_j,
// v_j the rows of [V_c; V_in], p the same softmax rows the scores come from
// (KVzip blog post, section 4.4: a FlashAttention kernel returns exactly this
// product, and not the max over rows of p that the scores need).
//
// bf16 path, three kernels: (1) the output pass sweeps every visible key of
// each query row once, forming the row's unnormalised output and its running
// (max, sum) per key split, with a lazily moved max as in score pass 1;
// (2) the split merge of those (max, sum) pairs gives the row log-sum-exp and
// score pass 2 forms the scores from it (score.hip); (3) the output merge
// rescales each split's output by 2^(m_split - M) / L.  So the logits are
// formed twice per call (here and in score pass 2), not three times.
//
// Output pass: rows stationary, keys swept (the K*Q^T orientation of score
// pass 1); per 32-key tile one wave computes its 32 rows' logits on MFMA;
// p = 2^(scale log2 e * x - m) is rounded to bf16 and, still in the
// accumulator layout, is the B operand of O^T += V^T P.  The two lanes that
// hold the same query column share m, so their P values in one MFMA carry
// the same scale.  V tiles stay row-major in LDS; the A operand (keys
// contiguous per d index, in the key order that layout implies) comes from
// transposing LDS reads.  fp32 path: a plain VALU kernel for small fp32
// problems, after the fp32 score passes.
#include "common.h"

namespace kvz {

namespace {

constexpr int KT = 32;      // keys per tile
constexpr int ROWS3 = 128;  // query rows per workgroup (4 waves x 32)
constexpr float kNegBig3 = -1e30f;
// the running max of a row moves only when a tile's terms against it sum
// past 2^30 (every term then stays below 2^30 times the row's max term)
constexpr float kLazyLimit3 = 1073741824.f;

#ifndef KVZ_ATTN_TARGET_WGS
#define KVZ_ATTN_TARGET_WGS 4096  // workgroups aimed for per call (sets the key splits)
#endif

template <int D>
struct G3 {
  static constexpr int KS = D / 16, CH = D / 8, SWZ = (CH < 16 ? CH : 16) - 1, DT = D / 32;
  static constexpr int NB = D / 16;                  // 32-byte blocks per V row
  // V block swizzle of key k: block ^ vsw(k), vsw(k) = 2 (k & 3) (within the
  // row's NB blocks).  A 16-lane group of transposing reads takes one block
  // (2 dt + mh) of four keys k & 3 = 0..3: even XOR offsets keep those four
  // blocks distinct, and the two groups of a half-wave (mh = 0, 1) on even
  // and odd blocks, so 32 lanes read 64 distinct banks
  static constexpr int VSW = NB - 1;
};

__device__ __forceinline__ int acc_row3(int v, int half) {
  return 8 * (v >> 2) + 4 * half + (v & 3);
}

typedef short v4i16 __attribute__((ext_vector_type(4)));

// 4 x 16-bit transposed LDS read: within each group of 16 lanes, lane 4a+b
// receives element b of the 8-byte chunks addressed by lanes a, a+4, a+8
// and a+12 of its group.
__device__ __forceinline__ v4i16 lds_read_tr4(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16*)(const_cast<void*>(p)));
}

// grid: H x splits x row tiles (XCD-remapped, head-major); rows i-major
// (r = i*G + g).  opart: [splits][H][R_pad][D] fp32, rows i-major, each
// split's output unnormalised against its running max; mlpart:
// [H][splits][R_pad] (max, sum) of each (row, split), g-major rows, log2
// units of the scaled logits (the layout score pass 1 writes).
//
// K and V tiles (32 keys each) go global -> LDS by buffer loads with an LDS
// destination, row-major: K with 16-byte chunks XOR-swizzled by the key
// (conflict-free A-operand reads, as in score pass 1), V with 32-byte blocks
// XOR-swizzled by the key.  The A operand of O^T += V^T P (lane m: d index,
// eight keys) is read with transposing LDS reads: in a 16-lane group, lane
// j = a + 4c points at 4 d values (4a..4a+3 past the group's d base) of the
// group's key c, so lane 4a+b receives d = 4a+b of keys c = 0..3.  The keys
// follow the order the P accumulator layout gives the MFMA's k index (lane
// half h holds keys 8(v>>2) + 4h + (v&3)): k-slots 0..3 of half h are keys
// 4h + 0..3, slots 4..7 keys 8 + 4h + 0..3 (plus 16 for the second MFMA of
// the tile).  The block swizzle puts a group's four keys in four different
// 32-byte blocks of the bank space.
template <int D>
__global__ __launch_bounds__(256) void attn_flash_bf16(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ kin, const uint16_t* __restrict__ vc,
    const uint16_t* __restrict__ vin, float* __restrict__ opart, float2* __restrict__ mlpart,
    int H, int G, int n_c, int n_in, int R, int R_pad, int n_rt, int n_split_ctx,
    int tiles_per_split, float cl2, int n_blocks) {
  constexpr int KS = G3<D>::KS, CH = G3<D>::CH, SWZ = G3<D>::SWZ, DT = G3<D>::DT;
  constexpr int VSW = G3<D>::VSW;
  constexpr int LOADS = KT * CH / 256;
  // two stages, as separate objects so that a copy into one stage is never
  // taken to alias the reads of the other
  __shared__ uint4 ldk0[KT * CH], ldk1[KT * CH], ldv0[KT * CH], ldv1[KT * CH];

  const int lb = xcd_logical_block();
  if (lb >= n_blocks) return;
  const int splits = n_split_ctx + 1;
  const int rt = lb % n_rt;
  const int s = (lb / n_rt) % splits;
  const int h = lb / (n_rt * splits);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, half = lane >> 5;

  const bool inchunk = (s == n_split_ctx);
  const int n_tiles_ctx = (n_c + KT - 1) / KT;
  const uint16_t *kbase, *vbase;
  int nkeys, t_begin, t_end;
  if (!inchunk) {
    kbase = kc + (size_t)h * n_c * D;
    vbase = vc + (size_t)h * n_c * D;
    nkeys = n_c;
    t_begin = s * tiles_per_split;
    t_end = min(n_tiles_ctx, t_begin + tiles_per_split);
  } else {
    kbase = kin + (size_t)h * n_in * D;
    vbase = vin + (size_t)h * n_in * D;
    nkeys = n_in;
    const int rlast = min(R, (rt + 1) * ROWS3) - 1;
    t_begin = 0;
    t_end = (rlast / G) / KT + 1;
  }

  // this lane's query row (column n of the wave's 32-row tile)
  const int r = rt * ROWS3 + wave * 32 + n;
  const int irow = r / G, grow = r - irow * G;
  bf16x8 qr[KS];
  if (r < R) {
    const uint16_t* p = q + ((size_t)(h * G + grow) * n_in + irow) * D + half * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qr[ks] = as_bf16x8(ld16(p + ks * 16));
  } else {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qr[ks] = as_bf16x8(make_uint4(0, 0, 0, 0));
  }
  // running max of the row (log2 units, shared by the lanes n and n + 32 of
  // the query column) and this lane's share of the sum against it
  float m = kNegBig3, l = 0.f;

  f32x16 o[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) o[t] = f32x16{};

  // copies: slot p of a stage holds key p / CH; for K its 16-byte chunk
  // (p % CH) ^ (key & SWZ), for V its 32-byte block ((p % CH) / 2) ^ vsw(key)
  const int seg_bytes = nkeys * D * 2;
  int koff[LOADS], voff[LOADS];
#pragma unroll
  for (int u = 0; u < LOADS; ++u) {
    const int slot = (u * 4 + wave) * 64 + lane;
    const int row = slot / CH, cp = slot % CH;
    koff[u] = row * D * 2 + (cp ^ (row & SWZ)) * 16;
    voff[u] = row * D * 2 + ((((cp >> 1) ^ (((row & 3) << 1) & VSW)) << 1) | (cp & 1)) * 16;
  }
  auto copy_k = [&](int tile, int par) {
    uint4* dk = par ? ldk1 : ldk0;
#pragma unroll
    for (int u = 0; u < LOADS; ++u)
      copy16_to_lds(kbase, seg_bytes, koff[u] + tile * (KT * D * 2), dk + (u * 4 + wave) * 64);
  };
  auto copy_v = [&](int tile, int par) {
    uint4* dv = par ? ldv1 : ldv0;
#pragma unroll
    for (int u = 0; u < LOADS; ++u)
      copy16_to_lds(vbase, seg_bytes, voff[u] + tile * (KT * D * 2), dv + (u * 4 + wave) * 64);
  };
  // transposed-read byte offsets of this lane within a V stage, per d tile:
  // key 4*half + c (c = (lane & 15) >> 2), d = 32 dt + 16 mh + 4a
  const int tr_c = (lane & 15) >> 2, tr_a = lane & 3, tr_mh = (lane >> 4) & 1;
  const int tr_key = 4 * half + tr_c;
  int vrd[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
    vrd[dt] = tr_key * D * 2 + (((2 * dt + tr_mh) ^ (((tr_key & 3) << 1) & VSW)) * 32) + tr_a * 8;

  // accumulator start of a tile's logits: 0, or -inf on keys the row does
  // not see (only the ragged context tile and the chunk tiles)
  const f32x16 zero = {};
  auto init_of = [&](int tile) -> f32x16 {
    if (!inchunk && (tile + 1) * KT <= n_c) return zero;
    f32x16 z;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int key = tile * KT + acc_row3(v, half);
      const bool vis = inchunk ? key <= irow : key < n_c;
      z[v] = vis ? 0.f : -INFINITY;
    }
    return z;
  };

  // Software pipeline over tiles (relative index r, stage parity par = r & 1):
  // K runs one tile ahead of V.  Iteration r forms p of tile r from its
  // logits (computed one iteration earlier) between the MFMAs of tile r+1's
  // logits, then issues tile r's O^T MFMAs; it copies K of tile r+2 into K
  // stage par and V of tile r+1 into V stage par^1, both last read in
  // iteration r-1.  Past the range the copies repeat the last tile and the
  // extra logits are never used.
  const int last = t_end - 1;
  auto body = [&](int tile, int par, f32x16& cur, f32x16& nxt) {
    const uint4* skn = par ? ldk0 : ldk1;
    const char* sv = reinterpret_cast<const char*>(par ? ldv1 : ldv0);
    bf16x8 a[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) a[ks] = as_bf16x8(skn[n * CH + ((ks * 2 + half) ^ (n & SWZ))]);
    copy_k(min(tile + 2, last), par);
    copy_v(min(tile + 1, last), par ^ 1);
    const f32x16 init = init_of(min(tile + 1, last));
    float p[16];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int v = ks * 16 / KS; v < (ks + 1) * 16 / KS; ++v)
        p[v] = fast_exp2(fmaf(cur[v], cl2, -m));
      nxt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks], qr[ks], ks == 0 ? init : nxt, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    // lazy commit: the max of a query column moves only when one of its two
    // lanes sums this tile's terms past half the limit (so the column's sum
    // stays below the limit); then the whole wave (a uniform branch) raises
    // each column's max to its tile max, rescales the output and sum so far,
    // and forms the terms again (always on the first tile, whose max starts
    // at -1e30)
    float ts = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7])) +
               (((p[8] + p[9]) + (p[10] + p[11])) + ((p[12] + p[13]) + (p[14] + p[15])));
    if (__ballot(!(ts <= 0.5f * kLazyLimit3))) {
      float mx = cur[0];
#pragma unroll
      for (int v = 1; v < 16; ++v) mx = fmaxf(mx, cur[v]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mn = fmaxf(m, mx * cl2);
      const float alpha = fast_exp2(m - mn);
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[dt][v] *= alpha;
      m = mn;
#pragma unroll
      for (int v = 0; v < 16; ++v) p[v] = fast_exp2(fmaf(cur[v], cl2, -m));
      ts = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7])) +
           (((p[8] + p[9]) + (p[10] + p[11])) + ((p[12] + p[13]) + (p[14] + p[15])));
    }
    l += ts;
    bf16x8 pb[2];
#pragma unroll
    for (int qq = 0; qq < 2; ++qq)
#pragma unroll
      for (int i = 0; i < 8; ++i) pb[qq][i] = (__bf16)p[8 * qq + i];
    // O^T[d][query] += V^T[d][key] P[key][query]
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int qq = 0; qq < 2; ++qq) {
        const v4i16 lo = lds_read_tr4(sv + vrd[dt] + (16 * qq) * D * 2);
        const v4i16 hi = lds_read_tr4(sv + vrd[dt] + (16 * qq + 8) * D * 2);
        const v4i16 both[2] = {lo, hi};
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, both), pb[qq],
                                                        o[dt], 0, 0, 0);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's copies have landed
    __syncthreads();
  };

  if (t_begin < t_end) {
    copy_k(t_begin, 0);
    copy_k(min(t_begin + 1, last), 1);
    copy_v(t_begin, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    f32x16 A, B;
    {
      const f32x16 init = init_of(t_begin);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 a = as_bf16x8(ldk0[n * CH + ((ks * 2 + half) ^ (n & SWZ))]);
        A = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qr[ks], ks == 0 ? init : A, 0, 0, 0);
      }
    }
    __syncthreads();  // every wave has read K stage 0 before it is refilled
    int tile = t_begin;
    for (; tile + 1 < t_end; tile += 2) {
      body(tile, 0, A, B);
      body(tile + 1, 1, B, A);
    }
    if (tile < t_end) body(tile, 0, A, B);
  }

  // the two lanes of a query column share m: their sums add
  const float lcol = l + __shfl_xor(l, 32);
  if (half == 0 && r < R)
    mlpart[((size_t)h * splits + s) * R_pad + grow * n_in + irow] = make_float2(m, lcol);
  // lane (n, half) holds d = 32 dt + 8 vg + 4 half + 0..3 of query row r
  float* op = opart + (((size_t)s * H + h) * R_pad + r) * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int vg = 0; vg < 4; ++vg)
      *reinterpret_cast<float4*>(op + dt * 32 + 8 * vg + 4 * half) =
          make_float4(o[dt][4 * vg], o[dt][4 * vg + 1], o[dt][4 * vg + 2], o[dt][4 * vg + 3]);
}

// O[h][g][i][:] = sum over splits s of opart[s][h][i*G + g][:] * 2^(m_s - M) / L,
// M the max of the splits' maxima m_s and L = sum of l_s 2^(m_s - M)
template <int D>
__global__ __launch_bounds__(256) void attn_reduce(const float* __restrict__ opart,
                                                   const float2* __restrict__ mlpart,
                                                   float* __restrict__ O, int H, int G, int n_in,
                                                   int R_pad, int splits) {
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;  // one float4
  const long long total = (long long)H * G * n_in * (D / 4);
  if (idx >= total) return;
  const int c4 = (int)(idx % (D / 4));
  const long long row = idx / (D / 4);  // (h*G + g)*n_in + i
  const int i = (int)(row % n_in);
  const int hg = (int)(row / n_in);
  const int h = hg / G, g = hg - h * G;
  const int r = i * G + g;
  const float2* ml = mlpart + (size_t)h * splits * R_pad + g * n_in + i;
  float M = kNegBig3;
  for (int s = 0; s < splits; ++s) M = fmaxf(M, ml[(size_t)s * R_pad].x);
  // compensated (Kahan) sums over the splits, as in the score pass's merge
  float L = 0.f, cL = 0.f;
  float a[4] = {0.f, 0.f, 0.f, 0.f}, ca[4] = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < splits; ++s) {
    const float2 v2 = ml[(size_t)s * R_pad];
    const float w = fast_exp2(v2.x - M);
    kahan_add(L, cL, v2.y * w);
    const float4 v =
        *reinterpret_cast<const float4*>(opart + (((size_t)s * H + h) * R_pad + r) * D + 4 * c4);
    kahan_add(a[0], ca[0], w * v.x);
    kahan_add(a[1], ca[1], w * v.y);
    kahan_add(a[2], ca[2], w * v.z);
    kahan_add(a[3], ca[3], w * v.w);
  }
  const float4 acc = make_float4(a[0], a[1], a[2], a[3]);
  const float inv = 1.0f / L;
  *reinterpret_cast<float4*>(O + row * D + 4 * c4) =
      make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
}

// fp32: one workgroup of 64 threads per query row; 64 keys at a time, one
// thread per key forms p, then every thread accumulates its output columns.
// lse2: [H][R_pad] i-major, log2 units (the fp32 score pass 1).
template <int D>
__global__ __launch_bounds__(64) void attn_f32(const float* __restrict__ q,
                                               const float* __restrict__ kc,
                                               const float* __restrict__ kin,
                                               const float* __restrict__ vc,
                                               const float* __restrict__ vin,
                                               const float* __restrict__ lse2,
                                               float* __restrict__ O, int G, int n_c, int n_in,
                                               int R_pad, float cl2) {
  __shared__ float ldq[D];
  __shared__ float ldp[64];
  const int h = blockIdx.y;
  const int r = blockIdx.x;  // i-major row
  const int i = r / G, g = r - (r / G) * G;
  const int tid = threadIdx.x;
  const float* qrow = q + ((size_t)(h * G + g) * n_in + i) * D;
  for (int k = tid; k < D; k += 64) ldq[k] = qrow[k];
  const float l2 = lse2[(size_t)h * R_pad + r];
  constexpr int U = D / 64;
  float acc[U];
#pragma unroll
  for (int u = 0; u < U; ++u) acc[u] = 0.f;
  const int n_vis = n_c + i + 1;
  __syncthreads();
  for (int j0 = 0; j0 < n_vis; j0 += 64) {
    const int j = j0 + tid;
    float pj = 0.f;
    if (j < n_vis) {
      const float* krow = j < n_c ? kc + ((size_t)h * n_c + j) * D
                                  : kin + ((size_t)h * n_in + (j - n_c)) * D;
      float dot = 0.f;
      for (int k = 0; k < D; ++k) dot = fmaf(ldq[k], krow[k], dot);
      pj = exp2f(dot * cl2 - l2);
    }
    ldp[tid] = pj;
    __syncthreads();
    const int nk = min(64, n_vis - j0);
    for (int kk = 0; kk < nk; ++kk) {
      const int jj = j0 + kk;
      const float* vrow = jj < n_c ? vc + ((size_t)h * n_c + jj) * D
                                   : vin + ((size_t)h * n_in + (jj - n_c)) * D;
      const float pk = ldp[kk];
#pragma unroll
      for (int u = 0; u < U; ++u) acc[u] = fmaf(pk, vrow[tid + 64 * u], acc[u]);
    }
    __syncthreads();
  }
  float* orow = O + ((size_t)(h * G + g) * n_in + i) * D;
#pragma unroll
  for (int u = 0; u < U; ++u) orow[tid + 64 * u] = acc[u];
}

template <int D>
hipError_t launch3(kvz_dtype dt, const ScorePlan& p, const AttnPlan& a, const void* q,
                   const void* kc, const void* kin, const void* vc, const void* vin, float scale,
                   float* S, float* O, void* ws, hipStream_t st) {
  const float cl2 = scale * 1.4426950408889634f;
  if (dt == KVZ_BF16) {
    float* opart = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + p.total_bytes);
    float2* mlpart = reinterpret_cast<float2*>(reinterpret_cast<char*>(ws) + p.total_bytes +
                                               a.opart_bytes);
    const int splits = a.n_split_ctx + 1;
    const int nb = p.H * splits * a.n_rt;
    KVZ_LAUNCH("attn_flash", attn_flash_bf16<D>, xcd_padded_grid(nb), 256, 0, st,
               (const uint16_t*)q, (const uint16_t*)kc, (const uint16_t*)kin,
               (const uint16_t*)vc, (const uint16_t*)vin, opart, mlpart, p.H, p.G, p.n_c, p.n_in,
               p.R, p.R_pad, a.n_rt, a.n_split_ctx, a.tiles_per_split, cl2, nb);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = score_finish_launch(p, mlpart, splits, q, kc, scale, S, ws, st);
    if (e != hipSuccess) return e;
    const long long total = (long long)p.H * p.G * p.n_in * (D / 4);
    KVZ_LAUNCH("attn_reduce", attn_reduce<D>, (unsigned)((total + 255) / 256), 256, 0, st, opart,
               mlpart, O, p.H, p.G, p.n_in, p.R_pad, splits);
  } else {
    const float* lse2 = reinterpret_cast<const float*>(ws);
    dim3 grid(p.R, p.H);
    KVZ_LAUNCH("attn_flash", attn_f32<D>, grid, 64, 0, st, (const float*)q, (const float*)kc,
               (const float*)kin, (const float*)vc, (const float*)vin, lse2, O, p.G, p.n_c,
               p.n_in, p.R_pad, cl2);
  }
  return hipGetLastError();
}

}  // namespace

AttnPlan attn_plan(kvz_dtype dt, const ScorePlan& p) {
  AttnPlan a{};
  a.fits = true;
  if (dt != KVZ_BF16) return a;  // the fp32 kernel needs no workspace of its own
  a.n_rt = (p.R + ROWS3 - 1) / ROWS3;  // row tiles holding real rows (<= R_pad / ROWS3)
  const int n_ctx_tiles = (p.n_c + KT - 1) / KT;
  int want = (KVZ_ATTN_TARGET_WGS + p.H * a.n_rt - 1) / (p.H * a.n_rt);
  int maxs = n_ctx_tiles / 16;
  if (maxs < 1) maxs = 1;
  if (want > maxs) want = maxs;
  if (want < 1) want = 1;
  a.tiles_per_split = (n_ctx_tiles + want - 1) / want;
  a.n_split_ctx = (n_ctx_tiles + a.tiles_per_split - 1) / a.tiles_per_split;
  a.opart_bytes =
      align256((size_t)(a.n_split_ctx + 1) * p.H * p.R_pad * p.d * sizeof(float));
  a.part_bytes =
      a.opart_bytes + align256((size_t)(a.n_split_ctx + 1) * p.H * p.R_pad * sizeof(float2));
  const int64_t nb = (int64_t)p.H * (a.n_split_ctx + 1) * a.n_rt;
  const int64_t merge = (int64_t)p.H * p.G * p.n_in * (p.d / 4);  // one float4 per lane
  a.fits = launch_fits((nb + kNumXcd - 1) / kNumXcd * kNumXcd, 256) &&
           launch_fits((merge + 255) / 256, 256);
  return a;
}

hipError_t attn_launch(kvz_dtype dt, const ScorePlan& p, const AttnPlan& a, const void* q,
                       const void* kc, const void* kin, const void* vc, const void* vin,
                       float scale, float* S, float* O, void* ws, hipStream_t st) {
  switch (p.d) {
    case 64: return launch3<64>(dt, p, a, q, kc, kin, vc, vin, scale, S, O, ws, st);
    case 128: return launch3<128>(dt, p, a, q, kc, kin, vc, vin, scale, S, O, ws, st);
    case 256: return launch3<256>(dt, p, a, q, kc, kin, vc, vin, scale, S, O, ws, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace kvz
