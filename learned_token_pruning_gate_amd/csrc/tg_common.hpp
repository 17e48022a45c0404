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

// ---- device side ---------------------------------------------------------

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
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
