// Head-level and token-level aggregates of the score tensor S[L*H][n_c].
//
// Head-level score (paperhub rebuttal, answer on head-level scores): the max
// of a head's scores along the sequence axis, used to rank whole heads for
// context-independent head eviction.  Token-level score (KVzip blog post,
// section 4.3.3): one score per token, the max over every layer and head.
// Both read S once (HBM-bound) and are exact (max needs no rounding).
#include <math.h>

#include "common.h"

namespace kvz {

namespace {

constexpr int TPB = 256;

// one workgroup per head: max over n_c scores
__global__ __launch_bounds__(TPB) void head_max(const float* __restrict__ S, int n_c,
                                                float* __restrict__ out) {
  __shared__ float red[TPB / 64];
  const int64_t h = blockIdx.x;
  const float* row = S + h * (int64_t)n_c;
  float m = -INFINITY;
  int j = threadIdx.x;
  for (; j + 3 * TPB < n_c; j += 4 * TPB)
    m = fmaxf(fmaxf(m, fmaxf(row[j], row[j + TPB])), fmaxf(row[j + 2 * TPB], row[j + 3 * TPB]));
  for (; j < n_c; j += TPB) m = fmaxf(m, row[j]);
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) out[h] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// one thread per token: max over all heads (coalesced across threads)
__global__ __launch_bounds__(TPB) void token_max(const float* __restrict__ S, int64_t n_heads,
                                                 int n_c, float* __restrict__ out) {
  const int j = blockIdx.x * TPB + threadIdx.x;
  if (j >= n_c) return;
  float m = -INFINITY;
  for (int64_t h = 0; h < n_heads; ++h) m = fmaxf(m, S[h * (int64_t)n_c + j]);
  out[j] = m;
}

}  // namespace

hipError_t head_scores_launch(const float* S, int64_t n_heads, int n_c, float* out,
                              hipStream_t st) {
  KVZ_LAUNCH("head_scores", head_max, (unsigned)n_heads, TPB, 0, st, S, n_c, out);
  return hipGetLastError();
}

hipError_t token_scores_launch(const float* S, int64_t n_heads, int n_c, float* out,
                               hipStream_t st) {
  KVZ_LAUNCH("token_scores", token_max, (unsigned)((n_c + TPB - 1) / TPB), TPB, 0, st, S, n_heads,
             n_c, out);
  return hipGetLastError();
}

}  // namespace kvz
