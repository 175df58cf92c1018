// Host-side check of libkvz's C ABI under AddressSanitizer and
// UndefinedBehaviorSanitizer: every entry point is called with each kind of
// argument it must reject (null or misaligned pointers, out-of-range sizes,
// short workspaces), every workspace query with small, typical and
// overflowing sizes, and the host-only calls.  Nothing here reaches a kernel
// launch, so it runs without a GPU.  Exit status 0 = every expected status
// was returned and the sanitizers found nothing.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "kvz.h"

static int failures = 0;

static void expect(int got, int want, const char* what) {
  if (got != want) {
    fprintf(stderr, "FAIL %s: status %d, expected %d\n", what, got, want);
    ++failures;
  }
}

int main() {
  void* A = reinterpret_cast<void*>(uintptr_t(1) << 20);        // aligned, never dereferenced
  void* M = reinterpret_cast<void*>((uintptr_t(1) << 20) + 2);  // misaligned
  float* Af = static_cast<float*>(A);
  float* Mf = static_cast<float*>(M);
  const size_t big = size_t(1) << 40;
  const kvz_status INV = KVZ_ERR_INVALID_ARG, UNS = KVZ_ERR_UNSUPPORTED, WS = KVZ_ERR_WORKSPACE;

  // host-only calls
  for (int s = -1; s < 8; ++s) {
    const char* t = kvz_status_string(static_cast<kvz_status>(s));
    if (!t || !t[0]) { fprintf(stderr, "FAIL status string %d\n", s); ++failures; }
  }
  if (strlen(kvz_build_id()) == 0) { fprintf(stderr, "FAIL build id\n"); ++failures; }
  const double ratios[] = {-1.0, 0.0, 1e-300, 0.3, 0.5, 1.0, 2.0, NAN, INFINITY};
  const int64_t Ns[] = {-5, 0, 1, 7, 33554432, int64_t(1) << 62};
  for (int64_t N : Ns)
    for (double r : ratios) {
      const int64_t k = kvz_keep_count(N, r);
      if (k < 0 || (N > 0 && k > N) || (N <= 0 && k != 0)) {
        fprintf(stderr, "FAIL keep_count(%lld, %g) = %lld\n", (long long)N, r, (long long)k);
        ++failures;
      }
    }

  // workspace queries: zero for bad sizes, no overflow for huge ones
  const int sizes[] = {-1, 0, 1, 64, 128, 256, 2064, 131072, 1 << 24, 1 << 30, 2147483647};
  for (int H : sizes)
    for (int n : sizes) {
      (void)kvz_score_chunk_workspace(KVZ_BF16, H, 4, n, 128, n);
      (void)kvz_score_chunk_attn_workspace(KVZ_BF16, H, 4, n, 128, n);
      (void)kvz_select_workspace(H, n);
      (void)kvz_compact_workspace(H, n);
      (void)kvz_select_heads_workspace(H, n);
      (void)kvz_select_tokens_workspace(H, n);
      (void)kvz_decode_workspace(H, 4, 128, n);
    }

  // scoring
  expect(kvz_score_chunk(KVZ_BF16, 2, 4, 96, 100, 4, 20, A, A, A, 0.1f, Af, A, big, nullptr), UNS, "score d");
  expect(kvz_score_chunk(KVZ_BF16, 0, 4, 128, 100, 4, 20, A, A, A, 0.1f, Af, A, big, nullptr), INV, "score H");
  expect(kvz_score_chunk(KVZ_BF16, 4097, 4, 128, 100, 4, 20, A, A, A, 0.1f, Af, A, big, nullptr), INV, "score H max");
  expect(kvz_score_chunk(static_cast<kvz_dtype>(-3), 2, 4, 128, 100, 4, 20, A, A, A, 0.1f, Af, A, big, nullptr), UNS, "score dtype");
  expect(kvz_score_chunk(KVZ_BF16, 2, 4, 128, 100, 21, 20, A, A, A, 0.1f, Af, A, big, nullptr), INV, "score n_prompt");
  expect(kvz_score_chunk(KVZ_BF16, 2, 4, 128, 100, 4, 20, nullptr, A, A, 0.1f, Af, A, big, nullptr), INV, "score q");
  expect(kvz_score_chunk(KVZ_BF16, 2, 4, 128, 100, 4, 20, A, M, A, 0.1f, Af, A, big, nullptr), INV, "score k_ctx align");
  expect(kvz_score_chunk(KVZ_BF16, 2, 4, 128, 100, 4, 20, A, A, A, NAN, Af, A, big, nullptr), INV, "score scale");
  expect(kvz_score_chunk(KVZ_BF16, 2, 4, 128, 100, 4, 20, A, A, A, 0.1f, Af, A, 16, nullptr), WS, "score ws");
  expect(kvz_score_chunk(KVZ_BF16, 2, 1 << 11, 128, 100, 4, 1 << 10, A, A, A, 0.1f, Af, A, big, nullptr), INV, "score G*n_in");
  expect(kvz_score_chunk(KVZ_BF16, 2, 4, 256, 4194304, 4, 20, A, A, A, 0.1f, Af, A, big, nullptr), INV, "score 2 GiB keys");
  expect(kvz_score_chunk_ex(KVZ_BF16, static_cast<kvz_aggregate>(9), 2, 4, 128, 100, 4, 20, A, A, A, 0.1f, Af, A, big, nullptr), UNS, "score_ex agg");
  expect(kvz_score_chunk_noalloc(KVZ_BF16, 4, 64, 128, 1000, 16, 8192, A, A, A, 0.1f, Af, nullptr), WS, "noalloc too big");
  expect(kvz_score_chunk_noalloc(KVZ_BF16, 2, 4, 128, 100, 4, 20, A, A, A, 0.1f, Mf, nullptr), INV, "noalloc S align");
  expect(kvz_score_chunk_attn(KVZ_BF16, 2, 4, 128, 100, 4, 20, A, A, A, A, nullptr, 0.1f, Af, Af, A, big, nullptr), INV, "attn v_in");
  expect(kvz_score_chunk_attn(KVZ_BF16, 2, 4, 128, 100, 4, 20, A, A, A, A, A, 0.1f, Af, Mf, A, big, nullptr), INV, "attn O align");
  expect(kvz_score_chunk_attn(KVZ_BF16, 2, 4, 128, 100, 4, 20, A, A, A, A, A, 0.1f, Af, Af, A, 16, nullptr), WS, "attn ws");

  // selection and the structured evictions
  uint8_t* Am = static_cast<uint8_t*>(A);
  int64_t* Ao = static_cast<int64_t*>(A);
  expect(kvz_select_threshold(Af, 4, 10, 41, Am, Ao, Af, A, big, nullptr), INV, "select K");
  expect(kvz_select_threshold(Af, 1 << 20, 1 << 12, 5, Am, Ao, Af, A, big, nullptr), INV, "select N");
  expect(kvz_select_threshold(Mf, 4, 10, 5, Am, Ao, Af, A, big, nullptr), INV, "select S align");
  expect(kvz_select_threshold(Af, 4, 10, 5, Am, Ao, Af, A, 8, nullptr), WS, "select ws");
  expect(kvz_select_heads(Af, 4, 10, 5, 1, 1, Am, Ao, Am, A, big, nullptr), INV, "heads K");
  expect(kvz_select_heads(Af, 4, 10, 2, -1, 1, Am, Ao, Am, A, big, nullptr), INV, "heads sink");
  expect(kvz_select_heads(Af, 4, 10, 2, 1, 1, static_cast<uint8_t*>(M), Ao, Am, A, big, nullptr), INV, "heads mask align");
  expect(kvz_select_heads(Af, 4, 10, 2, 1, 1, Am, Ao, Am, A, 8, nullptr), WS, "heads ws");
  expect(kvz_select_tokens(Af, 4, 10, 11, Am, Ao, Am, A, big, nullptr), INV, "tokens K");
  expect(kvz_select_tokens(Af, 4, 10, 3, Am, Ao, nullptr, A, big, nullptr), INV, "tokens keep");
  expect(kvz_select_tokens(Af, 4, 10, 3, Am, Ao, Am, A, 8, nullptr), WS, "tokens ws");
  expect(kvz_head_scores(nullptr, 4, 10, Af, nullptr), INV, "head_scores S");
  expect(kvz_token_scores(Af, 4, 0, Af, nullptr), INV, "token_scores n_c");

  // launch-size limits (32-bit work-item counts, int row indices)
  expect(kvz_score_chunk(KVZ_BF16, 4096, 1, 128, 64, 0, 1 << 20, A, A, A, 0.1f, Af, A, big, nullptr), INV, "score rows limit");
  expect(kvz_score_chunk(KVZ_BF16, 4096, 1, 64, 1 << 24, 0, 16, A, A, A, 0.1f, Af, A, big, nullptr), INV, "score pass-2 grid");
  expect(kvz_score_chunk_attn(KVZ_BF16, 4096, 1, 256, 64, 0, 1 << 17, A, A, A, A, A, 0.1f, Af, Af, A, big, nullptr), INV, "attn merge grid");
  expect(kvz_score_chunk_noalloc(KVZ_BF16, 4096, 1, 128, 64, 0, 1 << 20, A, A, A, 0.1f, Af, nullptr), INV, "noalloc rows limit");
  expect(kvz_select_threshold(Af, int64_t(1) << 24, 64, 5, Am, Ao, Af, A, big, nullptr), INV, "select tiles");
  expect(kvz_head_scores(Af, int64_t(1) << 22, 1, Af, nullptr), INV, "head_scores heads");
  expect(kvz_select_heads(Af, int64_t(1) << 22, 1, 1, 0, 0, Am, Ao, Am, A, big, nullptr), INV, "heads count");
  expect(kvz_decode_packed(KVZ_BF16, 16, 1, 64, 2147483647, A, A, A, Ao, 0.1f, Af, A, big, nullptr), INV, "decode segments");
  expect(kvz_decode_packed(KVZ_BF16, 15, 1, 64, 2147483647, A, A, A, Ao, 0.1f, Af, A, 8, nullptr), WS, "decode max_len INT_MAX");
  expect(kvz_decode_packed(KVZ_BF16, int64_t(1) << 21, 8, 256, 1, A, A, A, Ao, 0.1f, Af, A, big, nullptr), INV, "decode merge grid");

  // compaction and decode
  int32_t* Ai = static_cast<int32_t*>(A);
  expect(kvz_compact(KVZ_BF16, 100, 10, 0, 2, A, A, Am, Ao, A, A, Ai, A, big, nullptr), UNS, "compact d");
  expect(kvz_compact(KVZ_BF16, 128, 10, -1, 2, A, A, Am, Ao, A, A, Ai, A, big, nullptr), INV, "compact head_begin");
  expect(kvz_compact(KVZ_BF16, 128, 10, 0, 2, A, M, Am, Ao, A, A, Ai, A, big, nullptr), INV, "compact v align");
  expect(kvz_compact(KVZ_BF16, 128, 10, 0, 2, A, A, Am, Ao, A, A, Ai, A, 8, nullptr), WS, "compact ws");
  expect(kvz_decode_packed(KVZ_BF16, 4, 9, 128, 100, A, A, A, Ao, 0.1f, Af, A, big, nullptr), UNS, "decode G");
  expect(kvz_decode_packed(KVZ_BF16, 4, 4, 128, 0, A, A, A, Ao, 0.1f, Af, A, big, nullptr), INV, "decode max_len");
  expect(kvz_decode_packed(KVZ_BF16, 4, 4, 128, 100, A, A, A, Ao, -1.0f, Af, A, big, nullptr), INV, "decode scale");
  expect(kvz_decode_packed(KVZ_BF16, 4, 4, 128, 100, A, A, A, Ao, 0.1f, Af, A, 8, nullptr), WS, "decode ws");

  // the timer's host paths
  int64_t n = -1;
  double ms = -1;
  expect(kvz_prof_read("no such kernel", &n, &ms), INV, "prof name");
  expect(kvz_prof_read(nullptr, &n, &ms), INV, "prof null");
  expect(kvz_prof_read("score_pass1", &n, &ms), KVZ_OK, "prof read");
  if (n != 0) { fprintf(stderr, "FAIL prof launches %lld\n", (long long)n); ++failures; }
  expect(kvz_prof_enable(1, 0), INV, "prof enable 0 launches");

  printf("%s: %d failure(s)\n", failures ? "FAILED" : "ok", failures);
  return failures ? 1 : 0;
}
