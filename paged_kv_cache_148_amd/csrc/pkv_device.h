// pkv_device.h -- device-side helpers shared by the libpkv kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr float kNegInf = -__builtin_inff();

// 16-byte global load / store (global_load_dwordx4 / global_store_dwordx4).
__device__ __forceinline__ u32x4 ld16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }
__device__ __forceinline__ void st16(void *p, u32x4 v) { *reinterpret_cast<u32x4 *>(p) = v; }
// 16-byte load with the non-temporal hint, for data read exactly once (the K/V stream):
// it keeps the caches for data with reuse and streams markedly faster on gfx950.
__device__ __forceinline__ u32x4 ld16_stream(const void *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}

// bf16 is the high half of an fp32 word: widening is a shift (low element) or a mask
// (high element) of a packed pair.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16, round to nearest even; NaN stays NaN (quiet).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Two fp32 -> packed bf16 pair (lo in bits 0..15), round to nearest even
// (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = __builtin_convertvector((float __attribute__((ext_vector_type(2)))){lo, hi}, bf16x2);
  return __builtin_bit_cast(uint32_t, v);
}

// Raw hardware 2^x (v_exp_f32): exp2(-inf) = 0, exp2(0) = 1 exactly.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// DPP lane exchange inside a 16-lane row (fused into the consuming VALU op).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppRor4 = 0x124;       // row_ror:4
constexpr int kDppRor8 = 0x128;       // row_ror:8
constexpr int kDppHalfMirror = 0x141; // row_half_mirror

// Sum over aligned groups of N lanes (N = 8, 16 or 32); every lane of a group gets the sum.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 8 || N == 16 || N == 32, "group size");
  x += dpp<kDppXor1>(x);
  x += dpp<kDppXor2>(x);
  if constexpr (N == 8) {
    x += dpp<kDppHalfMirror>(x);
  } else {
    x += dpp<kDppRor4>(x);
    x += dpp<kDppRor8>(x);
    if constexpr (N == 32) x += __shfl_xor(x, 16);
  }
  return x;
}

// Maximum over aligned groups of 16 lanes; every lane of a group gets it.
__device__ __forceinline__ float group_max16(float x) {
  x = fmaxf(x, dpp<kDppXor1>(x));
  x = fmaxf(x, dpp<kDppXor2>(x));
  x = fmaxf(x, dpp<kDppRor4>(x));
  x = fmaxf(x, dpp<kDppRor8>(x));
  return x;
}

}  // namespace pkv
