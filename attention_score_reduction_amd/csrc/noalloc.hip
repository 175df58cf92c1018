// kvz_score_chunk_noalloc: the chunk-scoring call for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid allocation).  It runs the kernels of kvz_score_chunk
// with their workspace (per-split partial (max, sum) pairs and the row
// log-sum-exp) placed in a fixed file-scope device array instead of a
// caller-provided buffer.
//
// The array is a device symbol: in host code its name is only a stand-in,
// so its device address is looked up once per device with
// hipGetSymbolAddress (with that device current) and that address is what
// the kernels receive.  Every device the library runs on holds its own copy
// until the process ends.  Nothing in the array has to start at zero: pass 1
// writes every partial that the split merge reads, and the merge writes every
// row value that pass 2 reads.  Calls that overlap on one device share the
// array and race; callers serialise them (one stream, or events).
#include <math.h>

#include <mutex>

#include "common.h"

namespace kvz {
namespace {

constexpr size_t kScratchBytes = KVZ_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// device address of `scratch` on the current device (looked up once per
// device), or nullptr on a HIP error
void* scratch_on_current_device(hipError_t* err) {
  int dev = -1;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (*err != hipSuccess) return nullptr;
    g_scratch[dev] = p;
  }
  return g_scratch[dev];
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace
}  // namespace kvz

using namespace kvz;

extern "C" kvz_status kvz_score_chunk_noalloc(kvz_dtype dt, int H, int G, int d, int n_c,
                                              int n_prompt, int n_in, const void* q,
                                              const void* k_ctx, const void* k_in, float scale,
                                              float* S, void* stream) {
  if (dt != KVZ_BF16 && dt != KVZ_F32) return KVZ_ERR_UNSUPPORTED;
  if (d != 64 && d != 128 && d != 256) return KVZ_ERR_UNSUPPORTED;
  if (H < 1 || H > 4096 || G < 1 || n_in < 1 || n_c < 1 || n_prompt < 0 || n_prompt > n_in)
    return KVZ_ERR_INVALID_ARG;
  if ((long long)G * n_in > (1 << 20) || n_c > (1 << 24) ||
      (long long)n_c * d * 2 > 0x7fffffffLL)
    return KVZ_ERR_INVALID_ARG;
  if (!q || !k_ctx || !k_in || !S) return KVZ_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_ctx) || !aligned16(k_in) || !aligned16(S))
    return KVZ_ERR_INVALID_ARG;
  if (!(scale > 0.f) || !isfinite(scale)) return KVZ_ERR_INVALID_ARG;
  const ScorePlan p = score_plan(dt, H, G, n_in, d, n_c);
  if (!p.fits) return KVZ_ERR_INVALID_ARG;
  if (p.total_bytes > kScratchBytes) return KVZ_ERR_WORKSPACE;
  hipError_t e = hipSuccess;
  void* ws = scratch_on_current_device(&e);
  if (ws == nullptr) return KVZ_ERR_HIP;
  (void)hipGetLastError();
  e = score_launch(dt, KVZ_AGG_MAX, p, q, k_ctx, k_in, scale, S, ws,
                   reinterpret_cast<hipStream_t>(stream));
  return KVZ_RESULT(e, debug_word_score, reinterpret_cast<hipStream_t>(stream));
}
