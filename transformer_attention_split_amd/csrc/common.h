// Device helpers shared by the gfx950 kernels (wave64, CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_inff();

// ---------------------------------------------------------------------------
// bf16 <-> fp32. A bf16 value is the upper half of the fp32 bit pattern, so
// widening is a shift; narrowing uses the hardware's round-to-nearest-even
// pack instruction (v_cvt_pk_bf16_f32 on gfx950).
// ---------------------------------------------------------------------------
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16lo(uint32_t w) {
  return __uint_as_float(w << 16);
}
__device__ __forceinline__ float bf16hi(uint32_t w) {
  return __uint_as_float(w & 0xffff0000u);
}
// Pack two fp32 values (a -> low half, b -> high half) as RNE bf16.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2_t x = {a, b};
  bf16x2_t r = __builtin_convertvector(x, bf16x2_t);
  return __builtin_bit_cast(uint32_t, r);
}

// exp2 on the transcendental unit (v_exp_f32); exp2(-inf) == 0.
__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);
}

// ---------------------------------------------------------------------------
// DPP cross-lane moves inside a 16-lane row (gfx9 encodings).
// ---------------------------------------------------------------------------
enum : int {
  kDppQuadXor1 = 0xB1,      // quad_perm [1,0,3,2]
  kDppQuadXor2 = 0x4E,      // quad_perm [2,3,0,1]
  kDppRowHalfMirror = 0x141, // lane i <-> 7-i inside each 8-lane half row
  kDppRowMirror = 0x140,     // lane i <-> 15-i inside each 16-lane row
};

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF,
                                                 0xF, true));
}

// Sum over groups of N consecutive lanes (N in {1,2,4,8,16,32,64}); every
// lane of the group receives the group total. Groups up to 16 lanes use DPP
// row operations; wider groups add cross-row swizzles.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (N >= 2) v += dpp_mov<kDppQuadXor1>(v);
  if constexpr (N >= 4) v += dpp_mov<kDppQuadXor2>(v);
  if constexpr (N >= 8) v += dpp_mov<kDppRowHalfMirror>(v);
  if constexpr (N >= 16) v += dpp_mov<kDppRowMirror>(v);
  if constexpr (N >= 32) v += __shfl_xor(v, 16);
  if constexpr (N >= 64) v += __shfl_xor(v, 32);
  return v;
}

// Inclusive prefix sum over the 64 lanes: DPP row shifts inside each
// 16-lane row (out-of-row sources contribute 0), then the totals of the
// earlier rows read with readlane.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t x, int lane) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, false);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, false);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, false);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, false);
  const uint32_t t0 = __builtin_amdgcn_readlane(x, 15);
  const uint32_t t1 = __builtin_amdgcn_readlane(x, 31);
  const uint32_t t2 = __builtin_amdgcn_readlane(x, 47);
  return x + (lane >= 16 ? t0 : 0u) + (lane >= 32 ? t1 : 0u) + (lane >= 48 ? t2 : 0u);
}

}  // namespace attn
