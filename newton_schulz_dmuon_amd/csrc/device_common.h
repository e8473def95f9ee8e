// Device helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace dmuon {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// fp32 -> bf16, round to nearest even (gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Every buffer the kernels read or write element by element is device
// (global) memory.  Accesses go through address-space-1 pointers: a generic
// pointer compiles to flat instructions, which the compiler must assume may
// alias LDS and which also count on the LDS wait counter, so each LDS access
// after one would wait for it.
typedef __attribute__((address_space(1))) uint16_t g_u16;
typedef __attribute__((address_space(1))) float g_f32;

// Element access by run-time dtype code for caller buffers.
__device__ __forceinline__ float load_elem(const void *p, int32_t dt, int64_t i) {
  return dt == kBF16 ? bf16_bits_to_f32(((const g_u16 *)p)[i]) : ((const g_f32 *)p)[i];
}

__device__ __forceinline__ void store_elem(void *p, int32_t dt, int64_t i, float v) {
  if (dt == kBF16)
    ((g_u16 *)p)[i] = f32_to_bf16_bits(v);
  else
    ((g_f32 *)p)[i] = v;
}

// Workspace element type: bf16 (stored as raw bits) or fp32.
template <typename T> struct WsType;
template <> struct WsType<uint16_t> {
  static __device__ __forceinline__ float ld(const uint16_t *p, int64_t i) {
    return bf16_bits_to_f32(((const g_u16 *)p)[i]);
  }
  static __device__ __forceinline__ void st(uint16_t *p, int64_t i, float v) {
    ((g_u16 *)p)[i] = f32_to_bf16_bits(v);
  }
};
template <> struct WsType<float> {
  static __device__ __forceinline__ float ld(const float *p, int64_t i) { return ((const g_f32 *)p)[i]; }
  static __device__ __forceinline__ void st(float *p, int64_t i, float v) { ((g_f32 *)p)[i] = v; }
};

// Index of the entry whose [first, next first) range holds `w`, for a
// table sorted by `first` (binary search; tables hold at most a few hundred
// entries).
template <typename F>
__device__ __forceinline__ int32_t find_range(int32_t n, int64_t w, F first) {
  int32_t lo = 0, hi = n - 1;
  while (lo < hi) {
    const int32_t mid = (lo + hi + 1) >> 1;
    if (first(mid) <= w) lo = mid; else hi = mid - 1;
  }
  return lo;
}

}  // namespace dmuon
