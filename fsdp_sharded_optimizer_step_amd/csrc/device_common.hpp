// Device helpers shared by the kernels of the library (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#pragma clang fp contract(off)

namespace zs {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Streaming accesses: every byte is touched exactly once per call.  NT
// selects the non-temporal cache hint.  Measured on MI355X, it pays only
// where each cache line is fetched by a single instruction of a wave; where
// a lane reads two halves of a line with two instructions the line is
// fetched twice.  It is chosen per kernel and per stream.
template <bool NT, class T>
__device__ __forceinline__ T ld_stream(const T* p) {
  if constexpr (NT)
    return __builtin_nontemporal_load(p);
  else
    return *p;
}
template <bool NT, class T>
__device__ __forceinline__ void st_stream(T* p, T v) {
  if constexpr (NT)
    __builtin_nontemporal_store(v, p);
  else
    *p = v;
}

// bf16 -> binary32 is exact: the bf16 pattern is the upper half.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_one(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// binary32 -> bf16, round to nearest, ties to even.  Adding 0x7fff plus the
// lowest kept bit to the pattern carries into the kept half exactly when the
// discarded half is above the midpoint, or at it with an odd kept half;
// a carry out of the significand moves to the next binade or to infinity,
// which is the correct rounding.  NaN keeps sign and top payload, quiet bit
// forced on.
__device__ __forceinline__ uint32_t bf16_round(float x) {
  const uint32_t b = __float_as_uint(x);
  if ((b & 0x7fffffffu) > 0x7f800000u) return (b >> 16) | 0x0040u;
  return (b + 0x7fffu + ((b >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ uint32_t bf16_pack2(float lo, float hi) {
  return bf16_round(lo) | (bf16_round(hi) << 16);
}

// Host side: a HIP error already pending on the calling thread, left by an
// earlier unrelated call, would be read back by the launch check of an entry
// point as if its own launch had failed, after part of its work was enqueued.
// Entry points test for one before enqueuing anything and return ZERO_EHIP
// without touching it, so the caller still reads it with hipGetLastError.
inline bool hip_error_pending() { return hipPeekAtLastError() != hipSuccess; }

}  // namespace zs
