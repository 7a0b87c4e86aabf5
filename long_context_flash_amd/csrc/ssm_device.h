// ssm_device.h -- gfx950 device helpers shared by the Skip Softmax kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

// Two fp32 -> packed bf16 pair (round to nearest even; v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// 2^x on the transcendental unit (v_exp_f32): exact 0 for -inf.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

// Value held by lane (lane ^ 32): the two halves of a wave swap.
__device__ __forceinline__ float swap_halves(float x) { return __shfl_xor(x, 32, 64); }

__device__ __forceinline__ uint64_t wave_ballot(bool p) { return __ballot(p); }

__device__ __forceinline__ u32x4 ld_global_16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ u32x2 ld_global_8(const void* p) { return *reinterpret_cast<const u32x2*>(p); }

}  // namespace ssm
