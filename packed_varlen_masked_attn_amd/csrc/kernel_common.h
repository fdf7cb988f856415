// Device helpers shared by the gfx950 attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pva_internal.h"

namespace pva {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

#define PVA_LDS __attribute__((address_space(3)))

// Softmax scores are kept in log2 units; the running max is only raised when
// a tile's max exceeds it by more than this many units, so probabilities stay
// below 2^kLazyRescale and O/l are rescaled rarely. Exact up to rounding: O
// and l always share the same reference max.
constexpr float kLazyRescale = 8.0f;

// LDS layout of a streamed K or V tile: row r (a key), 16-byte chunk c of the
// head dimension. Chunks are XOR-permuted per row so that the MFMA operand
// reads hit distinct banks:
//  * K is read 16 bytes per lane, 16 consecutive rows per LDS cycle: the
//    swizzle maps the same chunk of those 16 rows onto 16 different chunks;
//  * V is read with ds_read_b64_tr_b16, 4 rows x 64 bytes per half-wave: the
//    swizzle moves each of 4 consecutive rows to a different 64-byte quarter.
template <int C>  // C = 16-byte chunks per row (D / 8)
__device__ __forceinline__ int swz_k(int r) {
  return ((r * C) / 16) % C;
}
template <int C>
__device__ __forceinline__ int swz_v(int r) {
  return 4 * (((r * C) / 16) % (C / 4));
}

// Maximum over the two 32-lane halves of a wave: permlane32_swap(x, x) hands
// each lane its own value and its partner's (lane ^ 32) in some order.
__device__ __forceinline__ float half_swap_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_swap_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace pva
