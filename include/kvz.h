/*
 * kvz.h -- C ABI of libkvz: KVzip reconstruction-attention scoring, global
 * keep-ratio selection and compaction of a KV cache on AMD Instinct MI355X
 * (gfx950).
 *
 * The method (sources are named by page title and section):
 *   - "KVzip: Query-Agnostic KV Cache Compression with Context
 *     Reconstruction" (jjl357 blog post), section 4.1: prefill the context,
 *     run a teacher-forced reconstruction (repeat prompt + context), score
 *     every cached KV pair, sort by score and evict;
 *     section 4.3.1: the reconstruction attention is a softmax over the
 *     query-key products of each layer l and KV head h;
 *     section 4.3.2: the importance of context token j is the maximum, over
 *     the G query heads of the group and all query rows i, of the normalised
 *     probability it receives;
 *     section 4.5.1: the reconstruction runs chunk by chunk and per-chunk
 *     scores are merged (here: a running max).
 *   - paperhub.cn OpenReview rebuttals by the authors, answer on positional
 *     OOD: each chunk's positions continue after the whole prefilled context,
 *     i.e. every chunk attends to all n_c cached keys; answer on head-level
 *     scores: the score tensor has shape L x H x n_c.
 *   - atlas.scime.ai summary, "Approach": the lowest-scoring pairs are
 *     evicted once per context; "Measured effects": non-uniform KV-head
 *     budgets.
 *
 * Conventions shared by every call
 *   - Buffers are caller-owned, contiguous, row-major.  Pointers named
 *     "device" point to device memory on the current HIP device; "host"
 *     pointers to host memory.  The library allocates no memory: scratch is
 *     the caller's workspace, sized by the matching *_workspace() query.
 *   - Every launching call is asynchronous on `stream` (a hipStream_t; NULL
 *     is the null stream).  Arguments are validated before any launch; on a
 *     validation error nothing is launched and nothing is written.  Faults of
 *     launched kernels surface at the caller's next synchronisation.
 *   - bf16 tensors are raw 16-bit bfloat16 patterns; their pointers must be
 *     16-byte aligned.  fp32 tensors must be 16-byte aligned as well.
 *   - The library keeps no state between calls except the optional profiler
 *     below; calls on different streams may run concurrently if their
 *     buffers and workspaces are disjoint.
 *   - libkvz_debug.so, the same sources built with KVZ_DEBUG, exports the
 *     same calls.  Its kernels also check conditions the documentation puts
 *     on device-side data (no NaN or inf in scores, queries and keys; head
 *     offsets that match the mask they come with; no packed head longer
 *     than max_len) and invariants of their own results (exactly K kept).
 *     Where the release library returns a silent result for such input, the
 *     debug library synchronises the stream after the call and returns
 *     KVZ_ERR_INVALID_ARG.  Its checks share one flag per device: use it
 *     from one thread.
 */
#ifndef KVZ_H_
#define KVZ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVZ_API __attribute__((visibility("default")))

/* The enums are int-sized in C.  In C++ they get a fixed int underlying type,
 * so that any int a caller passes (an out-of-range value included, which the
 * calls reject) is a valid value of the enum type: the ABI is the same. */
#ifdef __cplusplus
#define KVZ_ENUM enum : int
#else
#define KVZ_ENUM enum
#endif

typedef KVZ_ENUM {
  KVZ_OK = 0,
  KVZ_ERR_INVALID_ARG = 1,     /* null pointer, bad size, misalignment      */
  KVZ_ERR_UNSUPPORTED = 2,     /* head_dim not in {64,128,256}, bad dtype   */
  KVZ_ERR_WORKSPACE = 3,       /* workspace smaller than the query returns  */
  KVZ_ERR_HIP = 4              /* a HIP launch or runtime call failed       */
} kvz_status;

typedef KVZ_ENUM {
  KVZ_BF16 = 0,                /* bfloat16 inputs, fp32 accumulation        */
  KVZ_F32 = 1                  /* fp32 inputs, fp32 arithmetic              */
} kvz_dtype;

/* How a context key's per-row attention is aggregated into its score. */
typedef KVZ_ENUM {
  KVZ_AGG_MAX = 0,     /* max over g, i of the softmax probability (the method,
                          blog 4.3.2); S starts at 0                          */
  KVZ_AGG_SUM = 1,     /* sum over g, i (and chunks) of the probability: the
                          aggregation the rebuttal compares against (sum and
                          mean rank keys identically); S starts at 0           */
  KVZ_AGG_RAW_MAX = 2  /* max over g, i of the raw logit scale*q.k, no softmax
                          (blog 5.5.5 ablation); S starts at -inf            */
} kvz_aggregate;

/* Human-readable name of a status code (static string, never NULL). */
KVZ_API const char* kvz_status_string(kvz_status s);

/* Build id of this library: the sha256 (hex) of the sources, this header and
 * the compiler flags it was built from, or "unknown" when built without one.
 * Callers compare it with the digest of their checkout to refuse a stale
 * binary.  Static string, never NULL. */
KVZ_API const char* kvz_build_id(void);

/* ------------------------------------------------------------------------
 * Scoring of one reconstruction chunk for all KV heads of one layer
 * (blog 4.3.1, 4.3.2, 4.5.1; rebuttal, positional OOD).
 *
 * Shapes (all device, row-major):
 *   q      [H][G][n_in][d]   query rows of the chunk: rows 0..n_prompt-1 are
 *                            the repeat prompt, rows n_prompt..n_in-1 the
 *                            copied context tokens.
 *   k_ctx  [H][n_c][d]       the layer's cached context keys.
 *   k_in   [H][n_in][d]      keys of the chunk's own tokens (prompt + copy).
 *   S      [H][n_c] fp32     running scores, read and written in place.
 *
 * For every head h, query head g and row i, the visible keys are all n_c
 * context keys followed by in-chunk keys 0..i (one causal mask over the
 * n_in chunk tokens).  With p = softmax(scale * q . k) over those keys,
 *     S[h][j] <- max(S[h][j], max over g, i of p[j])   for 0 <= j < n_c.
 * The caller zero-fills S once before the first chunk of a context; the
 * result does not depend on the order in which chunks are scored.
 * `scale` (normally 1/sqrt(d)) multiplies the fp32 dot product; it must be
 * finite and > 0.  n_prompt is validated (0 <= n_prompt <= n_in) and only
 * documents the row split: every row is a query and is masked the same way.
 *
 * Limits: d in {64, 128, 256}; 1 <= n_in, 1 <= n_c <= 2^24 with one head's
 * keys under 2 GiB (n_c * d * 2 <= 2^31 - 1, i.e. n_c <= 4,194,303 at d=256
 * and 8,388,607 at d=128), 1 <= H <= 4096, 1 <= G,
 * G * n_in <= 2^20.  A problem too large for the launches' 32-bit
 * work-item counts returns KVZ_ERR_INVALID_ARG (and a workspace size of 0);
 * every problem with H * G * n_in <= 2^29 and H * n_c <= 2^31 fits.  Workspace:
 * kvz_score_chunk_workspace() bytes, 256-byte aligned, device memory.
 * ---------------------------------------------------------------------- */
KVZ_API size_t kvz_score_chunk_workspace(kvz_dtype dt, int H, int G, int n_in, int d, int n_c);

KVZ_API kvz_status kvz_score_chunk(kvz_dtype dt, int H, int G, int d, int n_c, int n_prompt,
                           int n_in, const void* q, const void* k_ctx, const void* k_in,
                           float scale, float* S, void* ws, size_t ws_bytes, void* stream);

/* kvz_score_chunk with a chosen aggregation (kvz_score_chunk == KVZ_AGG_MAX).
 * KVZ_AGG_SUM: S[h][j] += sum over g, i of p[j] (running sum over chunks).
 * KVZ_AGG_RAW_MAX: S[h][j] <- max(S[h][j], max over g, i of scale*q.k_j); no
 * softmax is formed, so the in-chunk keys play no role.  Same arguments,
 * workspace and errors as kvz_score_chunk; agg outside the enum ->
 * KVZ_ERR_UNSUPPORTED. */
KVZ_API kvz_status kvz_score_chunk_ex(kvz_dtype dt, kvz_aggregate agg, int H, int G, int d,
                                      int n_c, int n_prompt, int n_in, const void* q,
                                      const void* k_ctx, const void* k_in, float scale, float* S,
                                      void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * kvz_score_chunk for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 * Same arguments, S update, limits and errors as kvz_score_chunk, without
 * the workspace: the library keeps a fixed scratch array of
 * KVZ_NOALLOC_SCRATCH_BYTES in device memory (one per device it runs on,
 * held until the process ends) and this call allocates nothing.  A problem
 * whose workspace (kvz_score_chunk_workspace) exceeds that size is rejected
 * with KVZ_ERR_WORKSPACE before anything is launched; every workload up to
 * 8 KV heads, G = 5 and 2K-token chunks of a 170K context fits.  Calls that
 * overlap on one device share the scratch array and race: serialise them
 * (one stream, or events).  Nothing carries over between calls.
 * ---------------------------------------------------------------------- */
#define KVZ_NOALLOC_SCRATCH_BYTES (16u << 20)

KVZ_API kvz_status kvz_score_chunk_noalloc(kvz_dtype dt, int H, int G, int d, int n_c,
                                           int n_prompt, int n_in, const void* q,
                                           const void* k_ctx, const void* k_in, float scale,
                                           float* S, void* stream);

/* ------------------------------------------------------------------------
 * Scoring of one chunk together with the chunk's attention output: the
 * fused reconstruction attention (rebuttal, computational analysis: the
 * scoring stage is a full forward over [repeat prompt; chunk], one MLP pass
 * and twice the prefill's attention work, so each layer's attention also
 * feeds the layer above; blog 4.4: this product is what a FlashAttention
 * kernel returns).
 *
 * Same S update, arguments, limits and errors as kvz_score_chunk, plus
 *   v_ctx  [H][n_c][d]       the layer's cached context values (dtype dt),
 *   v_in   [H][n_in][d]      values of the chunk's own tokens (dtype dt),
 *   O      [H][G][n_in][d]   fp32, written (not accumulated):
 *     O[h][g][i] = sum over the visible keys j of p[j] * v_j,
 * with v_j the rows of [v_ctx[h]; v_in[h]] and p the softmax row of query
 * (h, g, i) that the scores are taken from.  bf16 inputs: p is rounded to
 * bf16 for the matrix product, sums in fp32.  All pointers device, 16-byte
 * aligned; NULL or misaligned -> KVZ_ERR_INVALID_ARG.  The output merge's
 * launch adds to the score limits: every problem with also
 * H * G * n_in * d <= 2^33 fits.  Workspace:
 * kvz_score_chunk_attn_workspace() bytes (it includes the score workspace),
 * 256-byte aligned; too small -> KVZ_ERR_WORKSPACE.
 * ---------------------------------------------------------------------- */
KVZ_API size_t kvz_score_chunk_attn_workspace(kvz_dtype dt, int H, int G, int n_in, int d,
                                              int n_c);
KVZ_API kvz_status kvz_score_chunk_attn(kvz_dtype dt, int H, int G, int d, int n_c, int n_prompt,
                                        int n_in, const void* q, const void* k_ctx,
                                        const void* k_in, const void* v_ctx, const void* v_in,
                                        float scale, float* S, float* O, void* ws,
                                        size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Head-level score (rebuttal, answer on head-level scores: the max of S along
 * the sequence axis, used for context-independent head eviction):
 *   head_score[h] = max over j of S[h][j]        (device fp32 [n_heads])
 * Token-level score (blog 4.3.3: one score per token, max over layers and
 * heads):
 *   token_score[j] = max over h of S[h][j]       (device fp32 [n_c])
 * S: device fp32 [n_heads][n_c], 16-byte aligned.  No workspace.
 * Limits: n_heads < 2^22 for the head maxima.
 * ---------------------------------------------------------------------- */
KVZ_API kvz_status kvz_head_scores(const float* S, int64_t n_heads, int n_c, float* head_score,
                                   void* stream);
KVZ_API kvz_status kvz_token_scores(const float* S, int64_t n_heads, int n_c, float* token_score,
                                    void* stream);

/* ------------------------------------------------------------------------
 * Structured evictions on the same scores, each producing the mask and head
 * offsets that kvz_compact consumes (same layout as kvz_select_threshold's).
 *
 * kvz_select_heads -- context-independent head-level eviction (rebuttal,
 * answer on how head-level scores were computed: a head's score is the max
 * of S along the sequence axis; blog 5.4: KVzip's scores drive head-level
 * eviction in place of DuoAttention's).  The K_heads heads with the highest
 * head scores keep every token (exactly K_heads; ties to the lower flat head
 * index); every other head keeps its first n_sink and its last n_recent
 * tokens (the streaming-head structure of DuoAttention: the pages do not say
 * what an evicted head keeps).
 *   S            device fp32 [n_heads][n_c], 16-byte aligned, no NaN.
 *   mask         device uint8 [n_heads * n_c], 16-byte aligned, out.
 *   head_offsets device int64 [n_heads + 1], out (exclusive scan of the
 *                per-head kept counts).
 *   head_keep    device uint8 [n_heads], out: 1 = head kept whole.
 * 0 <= K_heads <= n_heads < 2^22, n_sink >= 0, n_recent >= 0,
 * n_heads * n_c < 2^31.
 * Workspace: kvz_select_heads_workspace() bytes, 256-byte aligned.
 *
 * kvz_select_tokens -- token-level eviction (blog 4.3.3: one score per
 * token, the max over all layers and heads; sorting those decides which
 * tokens stay).  The K_tokens positions with the highest token scores
 * (exactly K_tokens; ties to the lower position) are kept in every head, so
 * head_offsets[h] = h * K_tokens.
 *   token_keep   device uint8 [n_c], out: 1 = position kept.
 * 0 <= K_tokens <= n_c; the other arguments as for kvz_select_heads.
 * Workspace: kvz_select_tokens_workspace() bytes, 256-byte aligned.
 * ---------------------------------------------------------------------- */
KVZ_API size_t kvz_select_heads_workspace(int64_t n_heads, int n_c);
KVZ_API kvz_status kvz_select_heads(const float* S, int64_t n_heads, int n_c, int64_t K_heads,
                                    int n_sink, int n_recent, uint8_t* mask,
                                    int64_t* head_offsets, uint8_t* head_keep, void* ws,
                                    size_t ws_bytes, void* stream);
KVZ_API size_t kvz_select_tokens_workspace(int64_t n_heads, int n_c);
KVZ_API kvz_status kvz_select_tokens(const float* S, int64_t n_heads, int n_c, int64_t K_tokens,
                                     uint8_t* mask, int64_t* head_offsets, uint8_t* token_keep,
                                     void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Keep count K = r * N rounded half up, clamped to [0, N] (host only).
 * ---------------------------------------------------------------------- */
KVZ_API int64_t kvz_keep_count(int64_t N, double r);

/* ------------------------------------------------------------------------
 * Global selection over every (layer, head, token) score (blog 4.1 step 5;
 * atlas, Approach and Measured effects).
 *
 *   S            device fp32 [n_heads][n_c], n_heads = L*H in flat (l, h)
 *                order; any values except NaN (raw-logit scores may be
 *                negative); -0.0 ranks as +0.0.
 *   K            number of entries to keep, 0 <= K <= n_heads * n_c.
 *   mask         device uint8 [n_heads * n_c], out: 1 = kept.
 *   head_offsets device int64 [n_heads + 1], out: head_offsets[0] = 0 and
 *                head_offsets[h+1] - head_offsets[h] = kept count of head h.
 *   tau_out      device fp32 [1], out: the K-th largest score (+inf if K=0).
 *
 * Exactly K entries are kept: every score > tau, then the scores equal to tau
 * in ascending flat index (l*H + h)*n_c + j until K is reached.  No
 * device-to-host synchronisation happens.
 * Limits: n_heads * n_c < 2^31 and n_heads * ceil(n_c / 4096) < 2^24 (else
 * KVZ_ERR_INVALID_ARG and a workspace size of 0).  Workspace:
 * kvz_select_workspace() bytes.
 * ---------------------------------------------------------------------- */
KVZ_API size_t kvz_select_workspace(int64_t n_heads, int n_c);

KVZ_API kvz_status kvz_select_threshold(const float* S, int64_t n_heads, int n_c, int64_t K,
                                uint8_t* mask, int64_t* head_offsets, float* tau_out,
                                void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Compaction of the kept rows into a packed per-head cache (blog 4.1 step 5;
 * rebuttal, the compressed cache is built once and reused by many queries).
 *
 * Packs heads [head_begin, head_begin + head_count) so that a whole cache
 * can be packed in one call or one layer at a time.
 *   k_ctx, v_ctx  device [head_count][n_c][d] rows of those heads (pointer to
 *                 head head_begin), element type dt.
 *   mask          device uint8 [n_heads * n_c], the full mask from
 *                 kvz_select_threshold (indexed by absolute head).
 *   head_offsets  device int64 [n_heads + 1] from kvz_select_threshold.
 *   k_out, v_out  device [K][d] packed outputs, idx_out device int32 [K]:
 *                 for absolute head h, the r-th kept j (ascending) goes to
 *                 row head_offsets[h] + r, with idx_out = j.
 * Rows are copied bit-exactly.  Workspace: kvz_compact_workspace() bytes.
 * Limits: d in {64, 128, 256}; (head_begin + head_count) * n_c < 2^31;
 * head_count * ceil(n_c / 64) < 2^24 (about 2^30 positions per call).
 * KVZ_ERR_INVALID_ARG otherwise, before anything is launched.
 * ---------------------------------------------------------------------- */
KVZ_API size_t kvz_compact_workspace(int64_t head_count, int n_c);

KVZ_API kvz_status kvz_compact(kvz_dtype dt, int d, int n_c, int64_t head_begin, int64_t head_count,
                       const void* k_ctx, const void* v_ctx, const uint8_t* mask,
                       const int64_t* head_offsets, void* k_out, void* v_out,
                       int32_t* idx_out, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Decode attention over the packed per-head cache (abstract and atlas Key
 * results: the compressed cache cuts FlashAttention decode latency about 2x;
 * rebuttal, computational analysis: decode attention latency vs kept ratio).
 * One decode token per query head:
 *   out[h][g] = softmax(scale * q[h][g] . K_h^T) V_h      (zeros if K_h empty)
 * with K_h, V_h = rows head_offsets[h] .. head_offsets[h+1]-1 of k_rows,
 * v_rows.  Passing an uncompressed cache [n_heads][n_c][d] with
 * head_offsets[h] = h * n_c gives full-cache decoding.
 *   q             device [n_heads][G][d], element type dt, 16-byte aligned
 *   k_rows,v_rows device [rows][d], element type dt, 16-byte aligned
 *   head_offsets  device int64 [n_heads + 1], non-decreasing
 *   max_len       host upper bound on every head's row count (rows of a head
 *                 beyond it are not read)
 *   out           device fp32 [n_heads][G][d]
 * Limits: d in {64, 128, 256}, 1 <= G <= 8, n_heads * ceil(max_len / 2048)
 * < 2^24, n_heads * G * d < 2^32 (else KVZ_ERR_INVALID_ARG, and a workspace
 * size of 0).  Workspace: kvz_decode_workspace() bytes (per-segment partial
 * results).
 * ---------------------------------------------------------------------- */
KVZ_API size_t kvz_decode_workspace(int64_t n_heads, int G, int d, int max_len);

KVZ_API kvz_status kvz_decode_packed(kvz_dtype dt, int64_t n_heads, int G, int d, int max_len,
                                     const void* q, const void* k_rows, const void* v_rows,
                                     const int64_t* head_offsets, float scale, float* out,
                                     void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Optional kernel timer (measurement only).
 * The timer is the library's one piece of process-wide state; it is guarded
 * by a lock and safe to use from several threads.  Disabled (the default), it
 * costs one atomic load per launch; enabled, one lock per launch.  A call
 * that launches while another thread enables or disables the timer may leave
 * its launch untimed.
 * While enabled, every kernel the library launches is bracketed by a pair of
 * HIP events on its stream.  kvz_prof_read() synchronises those events and
 * returns, for the kernel named `name` ("score_pass1", "score_combine",
 * "score_pass2", "attn_flash", "attn_reduce", "select_*", "compact_*",
 * "head_scores", "token_scores", "evict_mask", "evict_offsets",
 * "decode_split", "decode_combine"), the
 * number of launches and the
 * summed duration in milliseconds since the last enable.  Returns KVZ_OK, or
 * KVZ_ERR_INVALID_ARG for an unknown name.  max_launches bounds the event
 * pool; launches beyond it are not timed.
 * ---------------------------------------------------------------------- */
KVZ_API kvz_status kvz_prof_enable(int on, int max_launches);
KVZ_API kvz_status kvz_prof_read(const char* name, int64_t* launches, double* total_ms);

#ifdef __cplusplus
}
#endif

#endif /* KVZ_H_ */
