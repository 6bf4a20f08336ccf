// Device helpers shared by the quantise and decode kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace tq {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
  _Float16 h = (_Float16)x;  // v_cvt_f16_f32, round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float f16_bits_to_f32(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }

// Round-to-nearest-even fp32 -> bf16 bits (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Sum over groups of `width` consecutive lanes (width a power of two <= 64).
template <int width>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
  for (int m = 1; m < width; m <<= 1) x += __shfl_xor(x, m, 64);
  return x;
}

template <int width>
__device__ __forceinline__ float group_max(float x) {
#pragma unroll
  for (int m = 1; m < width; m <<= 1) x = fmaxf(x, __shfl_xor(x, m, 64));
  return x;
}

// Walsh-Hadamard butterfly between lanes l and l ^ M (M a power of two up to
// 32) on the VALU: the lower lane of each pair gets x + y, the upper y - x
// (y = the partner's x), computed as y + sg * x with sg = -1 on upper lanes
// (one rounding: identical to the add / subtract).  M = 1, 2: quad_perm DPP;
// M = 4: row_half_mirror (l ^ 7) then quad_perm [3,2,1,0] (l ^ 3); M = 8:
// row_ror:8; M = 16 / 32: v_permlane16_swap / v_permlane32_swap, which hand
// every lane the pair's lower value in [0] and upper value in [1].
template <int M>
__device__ __forceinline__ float wht_xlane(float x, float sg) {
  static_assert(M == 1 || M == 2 || M == 4 || M == 8 || M == 16 || M == 32, "lane stride");
  if constexpr (M <= 8) {
    int y;
    if constexpr (M == 1) {
      y = __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false);
    } else if constexpr (M == 2) {
      y = __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false);
    } else if constexpr (M == 4) {
      const int t = __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false);
      y = __builtin_amdgcn_update_dpp(0, t, 0x1B, 0xF, 0xF, false);
    } else {
      y = __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false);
    }
    return __builtin_fmaf(sg, x, __int_as_float(y));
  } else {
    auto r = M == 16 ? __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false)
                     : __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __builtin_fmaf(sg, __uint_as_float(r[1]), __uint_as_float(r[0]));
  }
}
// +1 on lanes with bit M clear, -1 where it is set.
template <int M>
__device__ __forceinline__ float lane_sign(int lane) {
  return (lane & M) ? -1.f : 1.f;
}

// Reduction over aligned groups of W lanes (W = 2, 4, 8 or 16), result in
// every lane of the group, by DPP (xor 1, xor 2 within quads; the 8-lane
// half-row mirror; the 16-lane row rotation by 8).  op must be associative,
// commutative and idempotent-safe for the combination order (min, max, or).
template <int W, class Op>
__device__ __forceinline__ uint32_t group_reduce_xl(uint32_t x, Op op) {
  static_assert(W == 2 || W == 4 || W == 8 || W == 16, "group width");
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xF, 0xF, false));
  if constexpr (W >= 4) x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xF, 0xF, false));
  if constexpr (W >= 8) x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x141, 0xF, 0xF, false));
  if constexpr (W >= 16) x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x128, 0xF, 0xF, false));
  return x;
}

// Sum over each quad of lanes, in every lane of the quad: (x0 + x1) + (x2 + x3)
// as the xor-1 / xor-2 shuffle tree forms it.
__device__ __forceinline__ float quad_sum_xl(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
  return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
}

// Sum / max over the whole wave, in every lane: 16-lane rows by DPP
// rotations, then the rows by the permlane swaps.
__device__ __forceinline__ float wave_sum_xl(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x122, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x121, 0xF, 0xF, false));
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}
__device__ __forceinline__ float wave_max_xl(float x) {
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xF, 0xF, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x122, 0xF, 0xF, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x121, 0xF, 0xF, false)));
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}

}  // namespace tq
