// ssm_device.h -- gfx950 device helpers shared by the Skip Softmax kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm {

struct true_type { static constexpr bool value = true; };
struct false_type { static constexpr bool value = false; };

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
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

// max(a, b) as one v_max_f32.  For operands that are never NaN (scores, -inf for masked keys): written as
// fmaxf, the compiler first quiets each operand it cannot prove canonical with a v_max_f32 of the operand with
// itself, three instructions instead of one.
__device__ __forceinline__ float max_nonan(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
// v_permlane32_swap with both operands equal to x: lanes < 32 get {x[l], x[l+32]}, lanes >= 32 get
// {x[l-32], x[l]}, so each lane sees the value of lane ^ 32 without LDS.  The maximum of the two (for operands
// that are never NaN) and their sum:
__device__ __forceinline__ float pair_max_nonan(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max_nonan(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// (lo16(a), lo16(b)) and (hi16(a), hi16(b)) as one dword each: one v_perm_b32.  v_perm_b32 numbers the
// bytes of {src0, src1} with src1 as bytes 0-3 and src0 as bytes 4-7.
__device__ __forceinline__ uint32_t pack_lo16(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x05040100u); }
__device__ __forceinline__ uint32_t pack_hi16(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x07060302u); }

// Rowmax-PoT weight pair: 2^rint(s*c2 - kref) for two scores (kref an integer), with no transcendental, and
// their sum added to `acc`.  Adding 1.5*2^23 to the clamped log weight rounds it to an integer k (ties to even)
// held in the low mantissa bits; (bits << 23) + bits(1.0), modulo 2^32, is then the fp32 pattern of 2^k (0 for
// k = -127), whose high half is the bf16 pattern.  The row sum adds the two fp32 powers of two (two plain adds
// draw less energy than a bf16 dot product of the packed pair, and give the same sums here).  A score of -inf,
// or one whose log weight rounds to -127 or less, gives +0; the log weight must stay below 128 (the callers keep
// it at most 9).
__device__ __forceinline__ uint32_t pot_pack_sum_bf16x2(float s0, float s1, float c2, float kref, float& acc) {
  constexpr float kRound = 12582912.f;  // 1.5 * 2^23: its low 16 bits are zero
  const float t0 = fmaxf(fmaf(s0, c2, -kref), -127.f) + kRound;
  const float t1 = fmaxf(fmaf(s1, c2, -kref), -127.f) + kRound;
  const uint32_t w0 = (__float_as_uint(t0) << 23) + 0x3F800000u;
  const uint32_t w1 = (__float_as_uint(t1) << 23) + 0x3F800000u;
  acc += __uint_as_float(w0) + __uint_as_float(w1);
  return pack_hi16(w0, w1);
}

__device__ __forceinline__ float fmax3(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }

// acc + lo(pk) + hi(pk) for a packed bf16 pair (v_dot2c_f32_bf16 against (1, 1)).
__device__ __forceinline__ float dot2_bf16_sum(uint32_t pk, float acc) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk), one, acc, false);
}

// Wave-uniform read of p[i] from memory the kernel never writes (page tables, sequence lengths), through
// the constant address space: the compiler emits a scalar load, counted apart from the vector loads, so
// the read does not wait for the tile loads already in flight (a vector load would need vmcnt(0)).
__device__ __forceinline__ int load_uniform_i32(const int32_t* p, int64_t i) {
  typedef const __attribute__((address_space(4))) int32_t* cptr;
  return ((cptr)p)[i];
}

// Two OCP fp8 e4m3 codes (bytes 0-1, or 2-3 when hi, of w) as two packed bf16, with gfx950's
// v_cvt_scalef32_pk_bf16_fp8 at scale 1: exact, since every e4m3 value has at most four significant bits
// and an exponent inside bf16's range.
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w, bool hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t r = hi ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true)
                        : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  return __builtin_bit_cast(uint32_t, r);
}
// Eight e4m3 codes (bytes 0..7 of x) as eight bf16
__device__ __forceinline__ u32x4 fp8x8_to_bf16x8(u32x2 x) {
  return u32x4{fp8x2_to_bf16x2(x[0], false), fp8x2_to_bf16x2(x[0], true), fp8x2_to_bf16x2(x[1], false),
               fp8x2_to_bf16x2(x[1], true)};
}

// ---- buffer loads: a resource covers [base, base + num_bytes); dwords outside read as 0.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;  // gfx9 buffer descriptor word 3 (32-bit data format)

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t num_bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)num_bytes, kRsrcWord3);
}
// bytes spanned by rows [0, n) of a [n, ...] slice with row stride `stride` elements and d contiguous bf16
__device__ __forceinline__ uint32_t rows_bytes(int n, int64_t stride, int d) {
  return n <= 0 ? 0u : (uint32_t)((int64_t)(n - 1) * stride * 2 + d * 2);
}
__device__ __forceinline__ u32x4 buffer_load_16(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
__device__ __forceinline__ u32x2 buffer_load_8(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
}
// The same loads with the non-temporal cache policy (the `nt` bit): for data read once whose lines should not
// displace lines that are still to be read again from L2.
constexpr int kCachePolicyNT = 2;
__device__ __forceinline__ u32x4 buffer_load_16_nt(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCachePolicyNT);
}
__device__ __forceinline__ u32x2 buffer_load_8_nt(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kCachePolicyNT);
}

__device__ __forceinline__ uint64_t wave_ballot(bool p) { return __ballot(p); }

// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their maxima): all vector memory loads of this wave done.
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0f70); }


}  // namespace ssm
