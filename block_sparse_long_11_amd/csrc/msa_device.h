// Device-side helpers shared by the MSA kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "msa.h"

namespace msa {

constexpr int kBlk = MSA_BLOCK_SIZE;   // tokens per KV block
constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16 bits, round to nearest even (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// 2-wide bf16 dot product accumulated in fp32 (v_dot2c_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c, false);
}

// Reductions over aligned groups of W consecutive lanes (W a power of two up to 64),
// without LDS round trips: DPP moves inside rows of 16 lanes (quad permutations,
// then the half-row and row mirrors, which pair the already reduced quads and
// halves), then the row swaps of v_permlane16_swap / v_permlane32_swap.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}

template <int W, typename Op>
__device__ __forceinline__ float group_reduce(float v, Op op) {
  static_assert(W >= 1 && W <= 64 && (W & (W - 1)) == 0, "group width");
  if constexpr (W >= 2) v = op(v, dpp_move<0xB1>(v));    // quad_perm [1,0,3,2]
  if constexpr (W >= 4) v = op(v, dpp_move<0x4E>(v));    // quad_perm [2,3,0,1]
  if constexpr (W >= 8) v = op(v, dpp_move<0x141>(v));   // row_half_mirror
  if constexpr (W >= 16) v = op(v, dpp_move<0x140>(v));  // row_mirror
  if constexpr (W >= 32) {
    const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v),
                                                     false, false);
    v = op(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
  }
  if constexpr (W >= 64) {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                     false, false);
    v = op(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
  }
  return v;
}

template <int W>
__device__ __forceinline__ float group_sum(float v) {
  return group_reduce<W>(v, [](float x, float y) { return x + y; });
}

template <int W>
__device__ __forceinline__ float group_max(float v) {
  return group_reduce<W>(v, [](float x, float y) { return fmaxf(x, y); });
}

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }
__device__ __forceinline__ float pos_inf() { return __builtin_inff(); }

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// 16-byte streaming load (data read once: non-temporal hint).
__device__ __forceinline__ uint4 load_stream16(const void *p) {
  const u32x4 v = __builtin_nontemporal_load(static_cast<const u32x4 *>(p));
  return uint4{v.x, v.y, v.z, v.w};
}

// 16 bytes of a row as an MFMA bf16x8 operand.
__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

}  // namespace msa
