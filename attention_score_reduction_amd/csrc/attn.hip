// Reconstruction attention output of one chunk, beside its scores.
//
// The scoring stage is a full forward over [repeat prompt; chunk] (paperhub
// rebuttal, computational analysis: one MLP pass plus twice the prefill's
// attention work), so each layer's attention also produces the output the
// layer above consumes:
//     O[h][g][i] = sum over visible keys j of p_ij * v_j,
// v_j the rows of [V_c; V_in], p the same softmax rows the scores come from
// (KVzip blog post, section 4.4: a FlashAttention kernel returns exactly this
// product).  It runs after the score passes of the same call and reuses their
// row log-sum-exp, so every p_ij is final when it is formed: no running
// rescale, and the key axis splits over workgroups whose partial outputs
// simply add.
//
// bf16 path: rows stationary, keys swept (the K*Q^T orientation of score
// pass 1); per 32-key tile one wave computes its 32 rows' logits on MFMA with
// the accumulator started at the row's -lse2/(scale log2 e), so
// p = 2^(scale log2 e * acc); p is rounded to bf16 and, still in the
// accumulator layout, is the B operand of O^T += V^T P.  V tiles are stored
// transposed in LDS (keys contiguous per d index) in the key order that
// layout implies.  fp32 path: a plain VALU kernel for small fp32 problems.
#include "common.h"

namespace kvz {

namespace {

constexpr int KT = 32;      // keys per tile
constexpr int ROWS3 = 128;  // query rows per workgroup (4 waves x 32)

#ifndef KVZ_ATTN_TARGET_WGS
#define KVZ_ATTN_TARGET_WGS 2048  // workgroups aimed for per call (sets the key splits)
#endif

template <int D>
struct G3 {
  static constexpr int KS = D / 16, CH = D / 8, SWZ = (CH < 16 ? CH : 16) - 1, DT = D / 32;
  static constexpr int VSTR = 40;  // V^T row stride in bf16: 32 keys + 8 pad (80 B)
};

// LDS slot of key kk (0..31) in a V^T row.  MFMA q (keys 16q..16q+15) takes
// k-slot s of lane half h as the key held by accumulator v = 8q + (s & 7) of
// that half: 16q + 8((s&7) >> 2) + 4h + (s & 3); this is its inverse.
__device__ __forceinline__ int vslot(int kk) {
  const int q = kk >> 4, kl = kk & 15;
  return q * 16 + ((kl >> 2) & 1) * 8 + 4 * (kl >> 3) + (kl & 3);
}

__device__ __forceinline__ int acc_row3(int v, int half) {
  return 8 * (v >> 2) + 4 * half + (v & 3);
}

// grid: H x splits x row tiles (XCD-remapped, head-major); rows i-major
// (r = i*G + g).  nlse: [H][R_pad] g-major, -lse2/(scale log2 e) (padding
// rows -inf).  opart: [splits][H][R_pad][D] fp32, rows i-major.
template <int D>
__global__ __launch_bounds__(256) void attn_pass3_bf16(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ kin, const uint16_t* __restrict__ vc,
    const uint16_t* __restrict__ vin, const float* __restrict__ nlse, float* __restrict__ opart,
    int H, int G, int n_c, int n_in, int R, int R_pad, int n_rt, int n_split_ctx,
    int tiles_per_split, float cl2, int n_blocks) {
  constexpr int KS = G3<D>::KS, CH = G3<D>::CH, SWZ = G3<D>::SWZ, DT = G3<D>::DT;
  constexpr int VSTR = G3<D>::VSTR;
  constexpr int LOADS = KT * CH / 256;
  // two LDS stages of K (row-major, swizzled) and V^T
  __shared__ uint4 ldk[2][KT * CH];
  __shared__ uint4 ldv4[2][D * VSTR / 8];

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
  float start = -INFINITY;
  if (r < R) {
    const uint16_t* p = q + ((size_t)(h * G + grow) * n_in + irow) * D + half * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qr[ks] = as_bf16x8(ld16(p + ks * 16));
    start = nlse[(size_t)h * R_pad + grow * n_in + irow];
  } else {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qr[ks] = as_bf16x8(make_uint4(0, 0, 0, 0));
  }

  f32x16 o[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) o[t] = f32x16{};

  // K copies: chunk-fastest (16-byte rows of one key per 16 lanes); V copies:
  // key-fastest, so the transposed 2-byte LDS writes of a wave land in
  // consecutive slots of one V^T row
  uint4 kreg[LOADS], vreg[LOADS];
  auto load = [&](int tile) {
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      const int c = tid + 256 * u;
      const int krow = c / CH, kch = c % CH, key = tile * KT + krow;
      kreg[u] = key < nkeys ? ld16(kbase + (size_t)key * D + kch * 8) : make_uint4(0, 0, 0, 0);
      const int vrow = c % KT, vch = c / KT, vkey = tile * KT + vrow;
      vreg[u] = vkey < nkeys ? ld16(vbase + (size_t)vkey * D + vch * 8) : make_uint4(0, 0, 0, 0);
    }
  };
  auto store = [&](int buf) {
    uint16_t* ldv = reinterpret_cast<uint16_t*>(ldv4[buf]);
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      const int c = tid + 256 * u;
      const int krow = c / CH, kch = c % CH;
      ldk[buf][krow * CH + (kch ^ (krow & SWZ))] = kreg[u];
      const int vrow = c % KT, vch = c / KT;
      const int sl = vslot(vrow);
      const uint32_t w[4] = {vreg[u].x, vreg[u].y, vreg[u].z, vreg[u].w};
#pragma unroll
      for (int e = 0; e < 8; ++e)
        ldv[(vch * 8 + e) * VSTR + sl] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
    }
  };

  if (t_begin < t_end) {
    load(t_begin);
    store(0);
  }
  __syncthreads();
  for (int tile = t_begin; tile < t_end; ++tile) {
    const int buf = (tile - t_begin) & 1;
    const bool more = tile + 1 < t_end;
    if (more) load(tile + 1);
    // logits of the lane's query column over the tile's 32 keys, offset by
    // the row's -lse2/(scale log2 e)
    f32x16 c;
#pragma unroll
    for (int v = 0; v < 16; ++v) c[v] = start;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 a = as_bf16x8(ldk[buf][n * CH + ((ks * 2 + half) ^ (n & SWZ))]);
      c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qr[ks], c, 0, 0, 0);
    }
    const int key0 = tile * KT;
    float p[16];
    if (!inchunk && key0 + KT <= n_c) {
#pragma unroll
      for (int v = 0; v < 16; ++v) p[v] = fast_exp2(c[v] * cl2);
    } else {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int key = key0 + acc_row3(v, half);
        const bool vis = inchunk ? key <= irow : key < n_c;
        p[v] = vis ? fast_exp2(c[v] * cl2) : 0.f;
      }
    }
    bf16x8 pb[2];
#pragma unroll
    for (int qq = 0; qq < 2; ++qq)
#pragma unroll
      for (int i = 0; i < 8; ++i) pb[qq][i] = (__bf16)p[8 * qq + i];
    // O^T[d][query] += V^T[d][key] P[key][query]
    const uint16_t* ldv = reinterpret_cast<const uint16_t*>(ldv4[buf]);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int qq = 0; qq < 2; ++qq) {
        const bf16x8 a = as_bf16x8(
            *reinterpret_cast<const uint4*>(ldv + (dt * 32 + n) * VSTR + qq * 16 + half * 8));
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[qq], o[dt], 0, 0, 0);
      }
    }
    // the other stage was last read one tile ago, before the last barrier
    if (more) store(buf ^ 1);
    __syncthreads();
  }

  // lane (n, half) holds d = 32 dt + 8 vg + 4 half + 0..3 of query row r
  float* op = opart + (((size_t)s * H + h) * R_pad + r) * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int vg = 0; vg < 4; ++vg)
      *reinterpret_cast<float4*>(op + dt * 32 + 8 * vg + 4 * half) =
          make_float4(o[dt][4 * vg], o[dt][4 * vg + 1], o[dt][4 * vg + 2], o[dt][4 * vg + 3]);
}

// O[h][g][i][:] = sum over splits of opart[s][h][i*G + g][:]
template <int D>
__global__ __launch_bounds__(256) void attn_reduce(const float* __restrict__ opart,
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
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s = 0; s < splits; ++s) {
    const float4 v =
        *reinterpret_cast<const float4*>(opart + (((size_t)s * H + h) * R_pad + r) * D + 4 * c4);
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
  }
  *reinterpret_cast<float4*>(O + row * D + 4 * c4) = acc;
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
                   float* O, void* ws, hipStream_t st) {
  const float cl2 = scale * 1.4426950408889634f;
  if (dt == KVZ_BF16) {
    const float* nlse = reinterpret_cast<const float*>(reinterpret_cast<char*>(ws) + p.part_bytes);
    float* opart = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + p.total_bytes);
    const int splits = a.n_split_ctx + 1;
    const int nb = p.H * splits * a.n_rt;
    KVZ_LAUNCH("attn_pass3", attn_pass3_bf16<D>, xcd_padded_grid(nb), 256, 0, st,
               (const uint16_t*)q, (const uint16_t*)kc, (const uint16_t*)kin,
               (const uint16_t*)vc, (const uint16_t*)vin, nlse, opart, p.H, p.G, p.n_c, p.n_in,
               p.R, p.R_pad, a.n_rt, a.n_split_ctx, a.tiles_per_split, cl2, nb);
    const long long total = (long long)p.H * p.G * p.n_in * (D / 4);
    KVZ_LAUNCH("attn_reduce", attn_reduce<D>, (unsigned)((total + 255) / 256), 256, 0, st, opart,
               O, p.H, p.G, p.n_in, p.R_pad, splits);
  } else {
    const float* lse2 = reinterpret_cast<const float*>(ws);
    dim3 grid(p.R, p.H);
    KVZ_LAUNCH("attn_pass3", attn_f32<D>, grid, 64, 0, st, (const float*)q, (const float*)kc,
               (const float*)kin, (const float*)vc, (const float*)vin, lse2, O, p.G, p.n_c,
               p.n_in, p.R_pad, cl2);
  }
  return hipGetLastError();
}

}  // namespace

AttnPlan attn_plan(kvz_dtype dt, const ScorePlan& p) {
  AttnPlan a{};
  if (dt != KVZ_BF16) return a;  // the fp32 kernel needs no workspace of its own
  a.n_rt = p.R_pad / ROWS3;
  const int n_ctx_tiles = (p.n_c + KT - 1) / KT;
  int want = (KVZ_ATTN_TARGET_WGS + p.H * a.n_rt - 1) / (p.H * a.n_rt);
  int maxs = n_ctx_tiles / 16;
  if (maxs < 1) maxs = 1;
  if (want > maxs) want = maxs;
  if (want < 1) want = 1;
  a.tiles_per_split = (n_ctx_tiles + want - 1) / want;
  a.n_split_ctx = (n_ctx_tiles + a.tiles_per_split - 1) / a.tiles_per_split;
  a.part_bytes =
      align256((size_t)(a.n_split_ctx + 1) * p.H * p.R_pad * p.d * sizeof(float));
  return a;
}

hipError_t attn_launch(kvz_dtype dt, const ScorePlan& p, const AttnPlan& a, const void* q,
                       const void* kc, const void* kin, const void* vc, const void* vin,
                       float scale, float* O, void* ws, hipStream_t st) {
  switch (p.d) {
    case 64: return launch3<64>(dt, p, a, q, kc, kin, vc, vin, scale, O, ws, st);
    case 128: return launch3<128>(dt, p, a, q, kc, kin, vc, vin, scale, O, ws, st);
    case 256: return launch3<256>(dt, p, a, q, kc, kin, vc, vin, scale, O, ws, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace kvz
