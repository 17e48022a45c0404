// tg_common.hpp -- helpers shared by the HIP kernels and their host entry
// points (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tokengate.h"

namespace tg {

// ---- host side -----------------------------------------------------------

// Records a thread-local message and returns `s`.
tg_status fail(tg_status s, const char* fmt, ...)
    __attribute__((format(printf, 2, 3)));

// Clears the thread-local message (successful calls).
void clear_error();

// TG_ERR_LAUNCH if the runtime reports a launch error, else TG_OK.
tg_status check_launch(const char* what);

inline bool aligned(const void* p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// Compute units of the current device, read from the runtime once per
// device and cached (256 on MI355X); 256 if the query fails.
int device_cu_count();

constexpr int64_t kMaxTokens = 2147483647LL;  // token counts fit in int32

// The entry points with run-time lengths, for the chain captured once per
// padded length.  Arguments as the C entry points of the same name; then
//   t_dyn  (gate, select) NULL, or a device int32 read by the kernels: the
//          prompt's length; T is the capacity the launches are sized for and
//          tokens at or past the length are not scored, kept or counted;
//   n_dyn  (gathers, attention) NULL, or a device int32 read by the kernels:
//          the kept count (the select's n_kept); N is the capacity, and kept
//          rows at or past the count are padding: zero rows, position -1,
//          score 0, attention output 0 with lse -inf, keys masked.
tg_status gate_score_call(const char* fn, tg_dtype dt, int64_t T, int64_t d, int64_t h,
                          const void* resid, int64_t resid_row_stride, const uint8_t* prunable,
                          const float* rms_weight, float eps, const void* w1, bool packed,
                          const float* b1, const float* w2, float b2, float* scores,
                          void* stream, const int32_t* t_dyn);
tg_status topk_select_call(int64_t T, const float* scores, const uint8_t* prunable, int64_t K,
                           int32_t* kept_idx, int64_t kept_capacity, int32_t* n_kept,
                           void* workspace, size_t workspace_bytes, void* stream,
                           const int32_t* t_dyn);
tg_status compact_gather_call(tg_dtype dt, int64_t T, int64_t N, int64_t d, const void* resid,
                              int64_t resid_row_stride, const float* scores,
                              const int32_t* kept_idx, void* resid_kept,
                              int64_t kept_row_stride, int32_t* pos_kept, float* score_kept,
                              void* stream, const int32_t* n_dyn);
tg_status kv_gather_call(tg_dtype dt, int64_t L, int64_t T, int64_t N, int64_t Hkv, int64_t D,
                         const void* k_cache, const void* v_cache, const int32_t* kept_idx,
                         void* k_kept, void* v_kept, void* stream, const int32_t* n_dyn);
tg_status bias_attn_call(tg_dtype dt, int64_t N, int64_t Hq, int64_t Hkv, int64_t D,
                         const void* q, const void* k, const void* v, const float* key_score,
                         const float* gain, const float* q_scale, float softmax_scale,
                         int causal, void* out, float* lse, void* workspace,
                         size_t workspace_bytes, void* stream, const int32_t* n_dyn);

// ---- device side ---------------------------------------------------------

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Device-scope (L2-coherent) relaxed atomic load / store.
template <typename T>
__device__ __forceinline__ T ld_agent(const T* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ void st_agent(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace tg
