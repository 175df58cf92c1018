// Shared device helpers and host-side launch plumbing for libkvz (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvz.h"

namespace kvz {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr int kNumXcd = 8;  // MI355X: 8 XCDs, workgroups dealt round-robin

// Workgroup index remap so that consecutive logical indices share an XCD.
// The hardware hands workgroup b to XCD (b % 8); the grid is padded to a
// multiple of 8 and logical index = xcd * (grid / 8) + b / 8.  Logical
// indices >= the real count must return immediately.
__device__ __forceinline__ int xcd_logical_block() {
  const int nb = gridDim.x;
  const int per = nb / kNumXcd;
  const int b = blockIdx.x;
  return (b % kNumXcd) * per + b / kNumXcd;
}

inline int xcd_padded_grid(int n) { return (n + kNumXcd - 1) / kNumXcd * kNumXcd; }

// A 1-D launch of `blocks` workgroups of `threads` lanes: its work-item count
// is a 32-bit dispatch field.
inline bool launch_fits(int64_t blocks, int threads) {
  return blocks >= 1 && blocks * threads <= int64_t(0xffffffff);
}

__device__ __forceinline__ uint4 ld16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) {
  return __builtin_bit_cast(bf16x8, u);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Debug builds (-DKVZ_DEBUG, libkvz_debug.so).  Kernels check conditions
// their inputs must meet and invariants of their own results; a failed check
// sets a bit in a device word of its source file (KVZ_DCHECK) instead of
// trapping, and never changes what a kernel reads or writes.  The call that
// launched the kernels synchronises its stream, takes and clears the word
// (debug_word_<file>), and returns KVZ_ERR_INVALID_ARG when a bit was set.
// Release builds compile every check away.  The words are per device and
// shared by all calls on it: debug builds are meant for one caller thread.
#ifdef KVZ_DEBUG
#define KVZ_DEBUG_WORD(fn)                                                            \
  static __device__ unsigned int kvz_dbg_word;                                        \
  unsigned int fn(hipStream_t st) {                                                   \
    unsigned int v = 0, z = 0;                                                        \
    if (hipStreamSynchronize(st) != hipSuccess) return ~0u;                           \
    if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(kvz_dbg_word), sizeof v) != hipSuccess)    \
      return ~0u;                                                                     \
    if (v && hipMemcpyToSymbol(HIP_SYMBOL(kvz_dbg_word), &z, sizeof z) != hipSuccess) \
      return ~0u;                                                                     \
    return v;                                                                         \
  }
#define KVZ_DCHECK(cond, bit)                          \
  do {                                                 \
    if (!(cond)) atomicOr(&kvz_dbg_word, (bit));       \
  } while (0)
unsigned int debug_word_score(hipStream_t st);
unsigned int debug_word_select(hipStream_t st);
unsigned int debug_word_compact(hipStream_t st);
unsigned int debug_word_decode(hipStream_t st);
#define KVZ_RESULT(e, word, st) \
  ((e) != hipSuccess ? KVZ_ERR_HIP : ((word)(st) != 0u ? KVZ_ERR_INVALID_ARG : KVZ_OK))
#else
#define KVZ_RESULT(e, word, st) ((e) == hipSuccess ? KVZ_OK : KVZ_ERR_HIP)
#define KVZ_DEBUG_WORD(fn)
#define KVZ_DCHECK(cond, bit) \
  do {                        \
  } while (0)
#endif

// Compensated (Kahan) accumulation: sum += term, with the rounding error of
// each step carried in comp, so that terms far below the running sum still
// count.  Contraction is off: every step must round on its own.
__device__ __forceinline__ void kahan_add(float& sum, float& comp, float term) {
#pragma clang fp contract(off)
  const float y = term - comp;
  const float t = sum + y;
  comp = (t - sum) - y;
  sum = t;
}
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Word 3 of a raw buffer resource on gfx9-family parts: 32-bit data format
// (a zero format makes buffer loads return zero), no swizzle, no index
// stride.  With stride 0 the hardware range check is offset < num_records
// bytes; loads outside return zero and touch no memory.
constexpr int kBufferFlags = 0x00020000;

// LDS address-space view of a __shared__ object (the LDS destination of a
// buffer load with the lds flag is a wave-uniform base in M0; lane i writes
// base + 16*i for a 16-byte load).
__device__ __forceinline__ __attribute__((address_space(3))) void* lds_ptr(void* p) {
  return (__attribute__((address_space(3))) void*)(p);
}

// Each lane of the wave copies the 16 bytes at base + voff into LDS at
// dst + 16*lane (dst wave-uniform).  base..base+nbytes is the buffer's range:
// offsets outside it read as zero.  The copy is counted by vmcnt.
__device__ __forceinline__ void copy16_to_lds(const void* base, int nbytes, int voff, void* dst) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, nbytes, kBufferFlags);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_ptr(dst), 16, voff, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// host side: launch timing hooks (see kvz_prof_enable in kvz.h)
// ---------------------------------------------------------------------------
void prof_before(const char* name, hipStream_t s);
void prof_after(hipStream_t s);

#define KVZ_LAUNCH(name, kern, grid, block, shmem, stream, ...)                     \
  do {                                                                             \
    ::kvz::prof_before(name, stream);                                              \
    hipLaunchKernelGGL(kern, dim3(grid), dim3(block), shmem, stream, __VA_ARGS__); \
    ::kvz::prof_after(stream);                                                     \
  } while (0)

// ---------------------------------------------------------------------------
// internal launchers (argument validation happens in api.hip)
// ---------------------------------------------------------------------------
struct ScorePlan {
  int H, G, d, n_c, n_in, R, R_pad;
  int n_rt;             // pass-1 row tiles per head
  int n_split_ctx;      // pass-1 splits of the context keys (+1 in-chunk split)
  int tiles_per_split;  // 32-key tiles per context split
  size_t part_bytes, lse_bytes, total_bytes;
  bool fits;  // every launch within 32-bit work-item counts and int row indices
};
ScorePlan score_plan(kvz_dtype dt, int H, int G, int n_in, int d, int n_c);
hipError_t score_launch(kvz_dtype dt, kvz_aggregate agg, const ScorePlan& p, const void* q,
                        const void* kc, const void* kin, float scale, float* S, void* ws,
                        hipStream_t st);
// bf16 score update from per-split row (max, sum) partials part[H][splits][R_pad]
// (g-major rows, log2 units of the scaled logits): split merge into the
// score workspace's row offsets, then pass 2 into S
hipError_t score_finish_launch(const ScorePlan& p, const float2* part, int splits, const void* q,
                               const void* kc, float scale, float* S, void* ws, hipStream_t st);


// reconstruction attention output (after the score passes of the same call,
// reusing their row log-sum-exp from the score workspace)
struct AttnPlan {
  int n_rt;             // row tiles of 128 rows per head
  int n_split_ctx;      // splits of the context keys (+1 in-chunk split)
  int tiles_per_split;  // 32-key tiles per context split
  size_t part_bytes;    // partial outputs and row (max, sum) partials, after the
                        // score workspace
  size_t opart_bytes;   // the partial outputs' share of part_bytes
  bool fits;            // every launch within 32-bit work-item counts
};
AttnPlan attn_plan(kvz_dtype dt, const ScorePlan& p);
// bf16: the whole fused call (output pass forming the row (max, sum) partials
// and O, the score update from those partials, the output merge); fp32: the
// output after a kvz_score_chunk-style score update of the same call
hipError_t attn_launch(kvz_dtype dt, const ScorePlan& p, const AttnPlan& a, const void* q,
                       const void* kc, const void* kin, const void* vc, const void* vin,
                       float scale, float* S, float* O, void* ws, hipStream_t st);

hipError_t head_scores_launch(const float* S, int64_t n_heads, int n_c, float* out,
                              hipStream_t st);
hipError_t token_scores_launch(const float* S, int64_t n_heads, int n_c, float* out,
                               hipStream_t st);

// structured selections on the head-level / token-level aggregates of S
size_t agg_select_workspace(int64_t n_agg);
hipError_t select_heads_launch(const float* S, int64_t n_heads, int n_c, int64_t K_heads,
                               int n_sink, int n_recent, uint8_t* mask, int64_t* head_offsets,
                               uint8_t* head_keep, void* ws, hipStream_t st);
hipError_t select_tokens_launch(const float* S, int64_t n_heads, int n_c, int64_t K_tokens,
                                uint8_t* mask, int64_t* head_offsets, uint8_t* token_keep,
                                void* ws, hipStream_t st);

struct SelectPlan {
  int64_t N, n_heads;
  int n_c, tiles_per_head;
  int64_t n_tiles;
  size_t total_bytes;
};
SelectPlan select_plan(int64_t n_heads, int n_c);
hipError_t select_launch(const SelectPlan& p, const float* S, int64_t K, uint8_t* mask,
                         int64_t* head_offsets, float* tau, void* ws, hipStream_t st);

struct CompactPlan {
  int64_t head_count;
  int n_c, tiles_per_head;
  int64_t n_tiles;
  size_t total_bytes;
};
CompactPlan compact_plan(int64_t head_count, int n_c);
hipError_t compact_launch(const CompactPlan& p, int row_bytes, int64_t head_begin,
                          const void* kc, const void* vc, const uint8_t* mask,
                          const int64_t* head_offsets, void* ko, void* vo, int32_t* idx,
                          void* ws, hipStream_t st);

struct DecodePlan {
  int64_t n_heads;
  int G, d, seg_rows, n_seg;
  size_t total_bytes;
};
DecodePlan decode_plan(int64_t n_heads, int G, int d, int max_len);
hipError_t decode_launch(kvz_dtype dt, const DecodePlan& p, const void* q, const void* k,
                         const void* v, const int64_t* offs, float scale, float* out, void* ws,
                         hipStream_t st);

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace kvz
