// libkvz C ABI: argument validation, workspace sizing, launch dispatch and
// the optional kernel timer.  Every entry point validates all arguments
// before it launches anything; see include/kvz.h for the contract.
#include <math.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <string>
#include <vector>

#include "common.h"

namespace kvz {

// ---------------------------------------------------------------------------
// kernel timer
// ---------------------------------------------------------------------------
namespace {
struct ProfRec {
  std::string name;
  hipEvent_t a, b;
};
// All fields but `on` are guarded by mu; `on` lets a launch skip the lock
// while the timer is off.  Each thread keeps the index of its own open record
// (t_pending), so launches from several threads pair their events correctly.
struct Prof {
  std::atomic<bool> on{false};
  std::mutex mu;
  int max_launches = 0;
  uint64_t epoch = 0;  // bumped by every enable/disable: stale pending indexes are dropped
  std::vector<hipEvent_t> pool;
  std::vector<ProfRec> recs;
};
Prof& prof() {
  static Prof p;
  return p;
}
thread_local int t_pending = -1;
thread_local uint64_t t_epoch = 0;
}  // namespace

void prof_before(const char* name, hipStream_t s) {
  t_pending = -1;
  Prof& p = prof();
  if (!p.on.load(std::memory_order_acquire)) return;
  std::lock_guard<std::mutex> g(p.mu);
  if (!p.on.load(std::memory_order_relaxed) || (int)p.recs.size() >= p.max_launches) return;
  const size_t k = p.recs.size();
  ProfRec r{name, p.pool[2 * k], p.pool[2 * k + 1]};
  if (hipEventRecord(r.a, s) != hipSuccess) return;
  p.recs.push_back(r);
  t_pending = (int)k;
  t_epoch = p.epoch;
}

void prof_after(hipStream_t s) {
  if (t_pending < 0) return;
  Prof& p = prof();
  std::lock_guard<std::mutex> g(p.mu);
  if (t_epoch == p.epoch && t_pending < (int)p.recs.size())
    (void)hipEventRecord(p.recs[t_pending].b, s);
  t_pending = -1;
}

}  // namespace kvz

using namespace kvz;

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool head_dim_ok(int d) { return d == 64 || d == 128 || d == 256; }
// KV heads per scoring call: bounded so that every grid size and index
// product of the launch plans stays within 32 bits
constexpr int kMaxHeads = 4096;
bool heads_ok(int H) { return H >= 1 && H <= kMaxHeads; }
// one head's context keys (and values) must fit a buffer resource's 32-bit
// byte range: the score and output kernels copy them into LDS by buffer
// loads whose offsets and range are 32-bit
bool ctx_fits(int n_c, int d) {
  return n_c <= (1 << 24) && (long long)n_c * d * 2 <= 0x7fffffffLL;
}
void clear_error() { (void)hipGetLastError(); }

}  // namespace

#ifndef KVZ_BUILD_ID
#define KVZ_BUILD_ID "unknown"
#endif

extern "C" {

const char* kvz_build_id(void) { return KVZ_BUILD_ID; }

const char* kvz_status_string(kvz_status s) {
  switch (s) {
    case KVZ_OK: return "ok";
    case KVZ_ERR_INVALID_ARG: return "invalid argument";
    case KVZ_ERR_UNSUPPORTED: return "unsupported head_dim or dtype";
    case KVZ_ERR_WORKSPACE: return "workspace too small";
    case KVZ_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

size_t kvz_score_chunk_workspace(kvz_dtype dt, int H, int G, int n_in, int d, int n_c) {
  if (!heads_ok(H) || G < 1 || n_in < 1 || n_c < 1 || (dt != KVZ_BF16 && dt != KVZ_F32)) return 0;
  if ((long long)G * n_in > (1 << 20) || !ctx_fits(n_c, d)) return 0;
  const ScorePlan p = score_plan(dt, H, G, n_in, d, n_c);
  return p.fits ? p.total_bytes : 0;
}

kvz_status kvz_score_chunk_ex(kvz_dtype dt, kvz_aggregate agg, int H, int G, int d, int n_c,
                              int n_prompt, int n_in, const void* q, const void* k_ctx,
                              const void* k_in, float scale, float* S, void* ws, size_t ws_bytes,
                              void* stream) {
  if (dt != KVZ_BF16 && dt != KVZ_F32) return KVZ_ERR_UNSUPPORTED;
  if (agg != KVZ_AGG_MAX && agg != KVZ_AGG_SUM && agg != KVZ_AGG_RAW_MAX)
    return KVZ_ERR_UNSUPPORTED;
  if (!head_dim_ok(d)) return KVZ_ERR_UNSUPPORTED;
  if (!heads_ok(H) || G < 1 || n_in < 1 || n_c < 1 || n_prompt < 0 || n_prompt > n_in)
    return KVZ_ERR_INVALID_ARG;
  if ((long long)G * n_in > (1 << 20) || !ctx_fits(n_c, d)) return KVZ_ERR_INVALID_ARG;
  if (!q || !k_ctx || !k_in || !S || !ws) return KVZ_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_ctx) || !aligned16(k_in) || !aligned16(S))
    return KVZ_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return KVZ_ERR_INVALID_ARG;
  if (!(scale > 0.f) || !isfinite(scale)) return KVZ_ERR_INVALID_ARG;
  const ScorePlan p = score_plan(dt, H, G, n_in, d, n_c);
  if (!p.fits) return KVZ_ERR_INVALID_ARG;
  if (ws_bytes < p.total_bytes) return KVZ_ERR_WORKSPACE;
  clear_error();
  const hipError_t e = score_launch(dt, agg, p, q, k_ctx, k_in, scale, S, ws,
                                    reinterpret_cast<hipStream_t>(stream));
  return KVZ_RESULT(e, debug_word_score, reinterpret_cast<hipStream_t>(stream));
}

kvz_status kvz_score_chunk(kvz_dtype dt, int H, int G, int d, int n_c, int n_prompt, int n_in,
                           const void* q, const void* k_ctx, const void* k_in, float scale,
                           float* S, void* ws, size_t ws_bytes, void* stream) {
  return kvz_score_chunk_ex(dt, KVZ_AGG_MAX, H, G, d, n_c, n_prompt, n_in, q, k_ctx, k_in, scale,
                            S, ws, ws_bytes, stream);
}

size_t kvz_score_chunk_attn_workspace(kvz_dtype dt, int H, int G, int n_in, int d, int n_c) {
  if ((dt != KVZ_BF16 && dt != KVZ_F32) || !head_dim_ok(d) || !heads_ok(H) || G < 1 ||
      n_in < 1 || n_c < 1 || (long long)G * n_in > (1 << 20) || !ctx_fits(n_c, d))
    return 0;
  const ScorePlan p = score_plan(dt, H, G, n_in, d, n_c);
  const AttnPlan a = attn_plan(dt, p);
  return p.fits && a.fits ? p.total_bytes + a.part_bytes : 0;
}

kvz_status kvz_score_chunk_attn(kvz_dtype dt, int H, int G, int d, int n_c, int n_prompt,
                                int n_in, const void* q, const void* k_ctx, const void* k_in,
                                const void* v_ctx, const void* v_in, float scale, float* S,
                                float* O, void* ws, size_t ws_bytes, void* stream) {
  if (dt != KVZ_BF16 && dt != KVZ_F32) return KVZ_ERR_UNSUPPORTED;
  if (!head_dim_ok(d)) return KVZ_ERR_UNSUPPORTED;
  if (!heads_ok(H) || G < 1 || n_in < 1 || n_c < 1 || n_prompt < 0 || n_prompt > n_in)
    return KVZ_ERR_INVALID_ARG;
  if ((long long)G * n_in > (1 << 20) || !ctx_fits(n_c, d)) return KVZ_ERR_INVALID_ARG;
  if (!q || !k_ctx || !k_in || !v_ctx || !v_in || !S || !O || !ws) return KVZ_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_ctx) || !aligned16(k_in) || !aligned16(v_ctx) ||
      !aligned16(v_in) || !aligned16(S) || !aligned16(O))
    return KVZ_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return KVZ_ERR_INVALID_ARG;
  if (!(scale > 0.f) || !isfinite(scale)) return KVZ_ERR_INVALID_ARG;
  const ScorePlan p = score_plan(dt, H, G, n_in, d, n_c);
  const AttnPlan a = attn_plan(dt, p);
  if (!p.fits || !a.fits) return KVZ_ERR_INVALID_ARG;
  if (ws_bytes < p.total_bytes + a.part_bytes) return KVZ_ERR_WORKSPACE;
  clear_error();
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  // bf16: the output pass forms the rows' (max, sum) partials itself and the
  // score update runs from them; fp32: the score passes first, then the
  // output from their row log-sum-exp
  hipError_t e = hipSuccess;
  if (dt == KVZ_F32) e = score_launch(dt, KVZ_AGG_MAX, p, q, k_ctx, k_in, scale, S, ws, st);
  if (e == hipSuccess)
    e = attn_launch(dt, p, a, q, k_ctx, k_in, v_ctx, v_in, scale, S, O, ws, st);
  return KVZ_RESULT(e, debug_word_score, st);
}

// head maxima: one 1024-thread workgroup per head, so that the launch's
// work-item count stays 32-bit
constexpr int64_t kMaxHeadRows = int64_t(1) << 22;

kvz_status kvz_head_scores(const float* S, int64_t n_heads, int n_c, float* head_score,
                           void* stream) {
  if (n_heads < 1 || n_c < 1 || n_heads >= kMaxHeadRows) return KVZ_ERR_INVALID_ARG;
  if (!S || !head_score || !aligned16(S) || (reinterpret_cast<uintptr_t>(head_score) & 3u) != 0)
    return KVZ_ERR_INVALID_ARG;
  clear_error();
  const hipError_t e =
      head_scores_launch(S, n_heads, n_c, head_score, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? KVZ_OK : KVZ_ERR_HIP;
}

kvz_status kvz_token_scores(const float* S, int64_t n_heads, int n_c, float* token_score,
                            void* stream) {
  if (n_heads < 1 || n_c < 1) return KVZ_ERR_INVALID_ARG;
  if (!S || !token_score || !aligned16(S) || (reinterpret_cast<uintptr_t>(token_score) & 3u) != 0)
    return KVZ_ERR_INVALID_ARG;
  clear_error();
  const hipError_t e =
      token_scores_launch(S, n_heads, n_c, token_score, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? KVZ_OK : KVZ_ERR_HIP;
}

size_t kvz_select_heads_workspace(int64_t n_heads, int n_c) {
  if (n_heads < 1 || n_c < 1 || n_heads * (int64_t)n_c >= (int64_t(1) << 31)) return 0;
  if (n_heads >= kMaxHeadRows) return 0;
  return agg_select_workspace(n_heads);
}

kvz_status kvz_select_heads(const float* S, int64_t n_heads, int n_c, int64_t K_heads,
                            int n_sink, int n_recent, uint8_t* mask, int64_t* head_offsets,
                            uint8_t* head_keep, void* ws, size_t ws_bytes, void* stream) {
  if (n_heads < 1 || n_c < 1 || n_heads * (int64_t)n_c >= (int64_t(1) << 31) ||
      n_heads >= kMaxHeadRows)
    return KVZ_ERR_INVALID_ARG;
  if (K_heads < 0 || K_heads > n_heads || n_sink < 0 || n_recent < 0) return KVZ_ERR_INVALID_ARG;
  if (!S || !mask || !head_offsets || !head_keep || !ws) return KVZ_ERR_INVALID_ARG;
  if (!aligned16(S) || !aligned16(mask) || (reinterpret_cast<uintptr_t>(head_offsets) & 7u) != 0 ||
      (reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
    return KVZ_ERR_INVALID_ARG;
  if (ws_bytes < agg_select_workspace(n_heads)) return KVZ_ERR_WORKSPACE;
  clear_error();
  const hipError_t e = select_heads_launch(S, n_heads, n_c, K_heads, n_sink, n_recent, mask,
                                           head_offsets, head_keep, ws,
                                           reinterpret_cast<hipStream_t>(stream));
  return KVZ_RESULT(e, debug_word_select, reinterpret_cast<hipStream_t>(stream));
}

size_t kvz_select_tokens_workspace(int64_t n_heads, int n_c) {
  if (n_heads < 1 || n_c < 1 || n_heads * (int64_t)n_c >= (int64_t(1) << 31)) return 0;
  return agg_select_workspace(n_c);
}

kvz_status kvz_select_tokens(const float* S, int64_t n_heads, int n_c, int64_t K_tokens,
                             uint8_t* mask, int64_t* head_offsets, uint8_t* token_keep, void* ws,
                             size_t ws_bytes, void* stream) {
  if (n_heads < 1 || n_c < 1 || n_heads * (int64_t)n_c >= (int64_t(1) << 31))
    return KVZ_ERR_INVALID_ARG;
  if (K_tokens < 0 || K_tokens > n_c) return KVZ_ERR_INVALID_ARG;
  if (!S || !mask || !head_offsets || !token_keep || !ws) return KVZ_ERR_INVALID_ARG;
  if (!aligned16(S) || !aligned16(mask) || (reinterpret_cast<uintptr_t>(head_offsets) & 7u) != 0 ||
      (reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
    return KVZ_ERR_INVALID_ARG;
  if (ws_bytes < agg_select_workspace(n_c)) return KVZ_ERR_WORKSPACE;
  clear_error();
  const hipError_t e = select_tokens_launch(S, n_heads, n_c, K_tokens, mask, head_offsets,
                                            token_keep, ws, reinterpret_cast<hipStream_t>(stream));
  return KVZ_RESULT(e, debug_word_select, reinterpret_cast<hipStream_t>(stream));
}

int64_t kvz_keep_count(int64_t N, double r) {
  if (N <= 0 || !(r > 0.0)) return 0;
  if (r >= 1.0) return N;
  const double k = floor(r * (double)N + 0.5);
  if (k <= 0.0) return 0;
  if (k >= (double)N) return N;
  return (int64_t)k;
}

// the mask and fix-up passes launch one 256-thread workgroup per tile of a
// head's scores: fewer than 2^24 tiles keeps their work-item counts 32-bit
constexpr int64_t kMaxSelectTiles = int64_t(1) << 24;

size_t kvz_select_workspace(int64_t n_heads, int n_c) {
  if (n_heads < 1 || n_c < 1 || n_heads * (int64_t)n_c >= (int64_t(1) << 31)) return 0;
  const SelectPlan p = select_plan(n_heads, n_c);
  return p.n_tiles < kMaxSelectTiles ? p.total_bytes : 0;
}

kvz_status kvz_select_threshold(const float* S, int64_t n_heads, int n_c, int64_t K,
                                uint8_t* mask, int64_t* head_offsets, float* tau_out, void* ws,
                                size_t ws_bytes, void* stream) {
  if (n_heads < 1 || n_c < 1) return KVZ_ERR_INVALID_ARG;
  const int64_t N = n_heads * (int64_t)n_c;
  if (N >= (int64_t(1) << 31)) return KVZ_ERR_INVALID_ARG;
  if (K < 0 || K > N) return KVZ_ERR_INVALID_ARG;
  if (!S || !mask || !head_offsets || !tau_out || !ws) return KVZ_ERR_INVALID_ARG;
  if (!aligned16(S) || (reinterpret_cast<uintptr_t>(head_offsets) & 7u) != 0 ||
      (reinterpret_cast<uintptr_t>(tau_out) & 3u) != 0 ||
      (reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
    return KVZ_ERR_INVALID_ARG;
  const SelectPlan p = select_plan(n_heads, n_c);
  if (p.n_tiles >= kMaxSelectTiles) return KVZ_ERR_INVALID_ARG;
  if (ws_bytes < p.total_bytes) return KVZ_ERR_WORKSPACE;
  clear_error();
  const hipError_t e = select_launch(p, S, K, mask, head_offsets, tau_out, ws,
                                     reinterpret_cast<hipStream_t>(stream));
  return KVZ_RESULT(e, debug_word_select, reinterpret_cast<hipStream_t>(stream));
}

size_t kvz_compact_workspace(int64_t head_count, int n_c) {
  if (head_count < 1 || n_c < 1) return 0;
  return compact_plan(head_count, n_c).total_bytes;
}

kvz_status kvz_compact(kvz_dtype dt, int d, int n_c, int64_t head_begin, int64_t head_count,
                       const void* k_ctx, const void* v_ctx, const uint8_t* mask,
                       const int64_t* head_offsets, void* k_out, void* v_out, int32_t* idx_out,
                       void* ws, size_t ws_bytes, void* stream) {
  if (dt != KVZ_BF16 && dt != KVZ_F32) return KVZ_ERR_UNSUPPORTED;
  if (!head_dim_ok(d)) return KVZ_ERR_UNSUPPORTED;
  if (n_c < 1 || head_begin < 0 || head_count < 1) return KVZ_ERR_INVALID_ARG;
  if ((head_begin + head_count) * (int64_t)n_c >= (int64_t(1) << 31)) return KVZ_ERR_INVALID_ARG;
  if (!k_ctx || !v_ctx || !mask || !head_offsets || !k_out || !v_out || !idx_out || !ws)
    return KVZ_ERR_INVALID_ARG;
  if (!aligned16(k_ctx) || !aligned16(v_ctx) || !aligned16(k_out) || !aligned16(v_out) ||
      (reinterpret_cast<uintptr_t>(head_offsets) & 7u) != 0 ||
      (reinterpret_cast<uintptr_t>(idx_out) & 3u) != 0 ||
      (reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
    return KVZ_ERR_INVALID_ARG;
  const CompactPlan p = compact_plan(head_count, n_c);
  // one 256-thread scatter workgroup per 64 positions: the launch's
  // work-item count must fit in 32 bits
  if (p.n_tiles >= (int64_t(1) << 24)) return KVZ_ERR_INVALID_ARG;
  if (ws_bytes < p.total_bytes) return KVZ_ERR_WORKSPACE;
  const int row_bytes = d * (dt == KVZ_BF16 ? 2 : 4);
  clear_error();
  const hipError_t e = compact_launch(p, row_bytes, head_begin, k_ctx, v_ctx, mask, head_offsets,
                                      k_out, v_out, idx_out, ws,
                                      reinterpret_cast<hipStream_t>(stream));
  return KVZ_RESULT(e, debug_word_compact, reinterpret_cast<hipStream_t>(stream));
}

// Both decode launches stay below 2^32 work-items: one 256-thread workgroup
// per (head, 2048-row segment), then one d-thread workgroup per query head.
static bool decode_grid_ok(int64_t n_heads, int G, int d, int max_len) {
  const DecodePlan p = decode_plan(n_heads, G, d, max_len);
  return n_heads * (int64_t)p.n_seg < (int64_t(1) << 24) &&
         n_heads * G * (int64_t)d < (int64_t(1) << 32);
}

size_t kvz_decode_workspace(int64_t n_heads, int G, int d, int max_len) {
  if (n_heads < 1 || G < 1 || G > 8 || !head_dim_ok(d) || max_len < 1) return 0;
  if (!decode_grid_ok(n_heads, G, d, max_len)) return 0;
  return decode_plan(n_heads, G, d, max_len).total_bytes;
}

kvz_status kvz_decode_packed(kvz_dtype dt, int64_t n_heads, int G, int d, int max_len,
                             const void* q, const void* k_rows, const void* v_rows,
                             const int64_t* head_offsets, float scale, float* out, void* ws,
                             size_t ws_bytes, void* stream) {
  if (dt != KVZ_BF16 && dt != KVZ_F32) return KVZ_ERR_UNSUPPORTED;
  if (!head_dim_ok(d) || G < 1 || G > 8) return KVZ_ERR_UNSUPPORTED;
  if (n_heads < 1 || max_len < 1) return KVZ_ERR_INVALID_ARG;
  if (!decode_grid_ok(n_heads, G, d, max_len)) return KVZ_ERR_INVALID_ARG;
  const DecodePlan p = decode_plan(n_heads, G, d, max_len);
  if (!q || !k_rows || !v_rows || !head_offsets || !out || !ws) return KVZ_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_rows) || !aligned16(v_rows) ||
      (reinterpret_cast<uintptr_t>(head_offsets) & 7u) != 0 ||
      (reinterpret_cast<uintptr_t>(out) & 3u) != 0 ||
      (reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
    return KVZ_ERR_INVALID_ARG;
  if (!(scale > 0.f) || !isfinite(scale)) return KVZ_ERR_INVALID_ARG;
  if (ws_bytes < p.total_bytes) return KVZ_ERR_WORKSPACE;
  clear_error();
  const hipError_t e = decode_launch(dt, p, q, k_rows, v_rows, head_offsets, scale, out, ws,
                                     reinterpret_cast<hipStream_t>(stream));
  return KVZ_RESULT(e, debug_word_decode, reinterpret_cast<hipStream_t>(stream));
}

kvz_status kvz_prof_enable(int on, int max_launches) {
  if (on && max_launches < 1) return KVZ_ERR_INVALID_ARG;
  Prof& p = prof();
  std::lock_guard<std::mutex> g(p.mu);
  p.on.store(false, std::memory_order_release);
  ++p.epoch;
  for (hipEvent_t e : p.pool) (void)hipEventDestroy(e);
  p.pool.clear();
  p.recs.clear();
  if (!on) return KVZ_OK;
  p.pool.resize(2 * (size_t)max_launches);
  for (auto& e : p.pool)
    if (hipEventCreate(&e) != hipSuccess) return KVZ_ERR_HIP;
  p.max_launches = max_launches;
  p.recs.reserve(max_launches);
  p.on.store(true, std::memory_order_release);
  return KVZ_OK;
}

kvz_status kvz_prof_read(const char* name, int64_t* launches, double* total_ms) {
  if (!name || !launches || !total_ms) return KVZ_ERR_INVALID_ARG;
  Prof& p = prof();
  std::lock_guard<std::mutex> g(p.mu);
  int64_t n = 0;
  double ms = 0.0;
  bool known = false;
  static const char* kNames[] = {"score_pass1",     "score_combine",  "score_pass2",
                                 "select_empty",    "select_init",    "select_hist",
                                 "select_pick",     "select_fixup",   "select_scan",
                                 "select_mask",     "compact_offsets",
                                 "compact_scatter", "head_scores",    "token_scores",
                                 "decode_split",    "decode_combine", "attn_flash",
                                 "attn_reduce",     "evict_mask",     "evict_offsets"};
  for (const char* k : kNames) known |= strcmp(k, name) == 0;
  if (!known) return KVZ_ERR_INVALID_ARG;
  for (const ProfRec& r : p.recs) {
    if (r.name != name) continue;
    if (hipEventSynchronize(r.b) != hipSuccess) return KVZ_ERR_HIP;
    float t = 0.f;
    if (hipEventElapsedTime(&t, r.a, r.b) != hipSuccess) return KVZ_ERR_HIP;
    ms += t;
    ++n;
  }
  *launches = n;
  *total_ms = ms;
  return KVZ_OK;
}

}  // extern "C"
