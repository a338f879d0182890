// Shared device/host helpers of libgptq (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <stddef.h>
#include <stdint.h>

#include "gptq.h"

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef double doublex4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

#define GPTQ_TRY_HIP(expr)                      \
  do {                                          \
    if ((expr) != hipSuccess) return GPTQ_ERR_HIP; \
  } while (0)

#define GPTQ_TRY_LAUNCH()                                   \
  do {                                                      \
    if (hipGetLastError() != hipSuccess) return GPTQ_ERR_HIP; \
  } while (0)

namespace gptq {

// Number of XCDs on MI355X; workgroups are dispatched round-robin over them.
constexpr int kXcds = 8;

// Maps a linear workgroup id to a work-item id so that each XCD receives a
// contiguous range of work items (neighbouring items share operands, which
// then stay in that XCD's L2).  `launched` is a multiple of kXcds; returns
// an index in [0, launched).
__device__ inline int64_t xcd_contiguous(int64_t wg, int64_t launched) {
  const int64_t per = launched / kXcds;
  return (wg % kXcds) * per + wg / kXcds;
}

inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }
inline int64_t ceil_div(int64_t x, int64_t m) { return (x + m - 1) / m; }

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

inline int elem_bytes(int dtype) { return dtype == GPTQ_F32 ? 4 : 2; }

inline bool valid_dtype(int dtype) {
  return dtype == GPTQ_F32 || dtype == GPTQ_F16 || dtype == GPTQ_BF16;
}

// Converts one stored element to float32 (bf16 and fp16 widen exactly).
template <int DT> __device__ inline float load_as_f32(const void* p, int64_t i);
template <> __device__ inline float load_as_f32<GPTQ_F32>(const void* p, int64_t i) {
  return static_cast<const float*>(p)[i];
}
template <> __device__ inline float load_as_f32<GPTQ_F16>(const void* p, int64_t i) {
  return static_cast<float>(static_cast<const _Float16*>(p)[i]);
}
template <> __device__ inline float load_as_f32<GPTQ_BF16>(const void* p, int64_t i) {
  const uint32_t b = static_cast<const uint16_t*>(p)[i];
  return __uint_as_float(b << 16);
}

}  // namespace gptq
