// mfma_ceiling.hip -- the rate at which this GPU sustains v_mfma_f32_32x32x16_bf16 (the matrix instruction
// of the prefill kernel), once with operands that are all zero and once with random bf16 operands.  The
// chip's clock depends on its power draw, which depends on the operand bits, so the second figure is the
// practical ceiling for a kernel that multiplies real data; the first approaches the published peak.
//
// Standalone measurement program (not part of libssm.so).  Prints one JSON line.  It also times the VALU
// rate of v_fma_f32 and of v_exp_f32 (the exponential of the softmax step) followed by an add, and reports
// how many fma issue slots one exponential with its add takes.
//   mfma_ceiling [iterations]
//   mfma_ceiling [iterations] sustain SECONDS
// The second form holds each phase for SECONDS, launching its loop back to back, and prints for each its
// CLOCK_MONOTONIC interval and its rate, so that a sampler of the board's power reading running beside it can
// attribute its samples: the GPU idle, the MFMA loop on zero and on random operands, and the random-operand
// loop with, per 16 MFMAs of a wave, the other kinds of work an attention kernel adds (an idle phase before
// each): the A operand of every MFMA read from LDS (16 ds_read_b128, 16 KB, as the prefill reads its K and V
// operands); 16 v_exp_f32 with 16 adds and 48 fmas that do not depend on the MFMAs (about the prefill's VALU
// work per 16 MFMAs); two 1 KB direct-to-LDS buffer loads from a 4 MB buffer that stays in L2 (the prefill's
// tile loads per 16 MFMAs); the LDS operand reads done as transposing reads (as the prefill reads V); one
// workgroup barrier; about 48 scalar instructions; conversions to bf16 and bf16 dot products in place of the
// exponentials and adds; the first three together; and the loop's FLOP issued as v_mfma_f32_16x16x32_bf16
// instead. A last phase runs the loop alone on normally distributed operands.
//
// Each of 512 workgroups (two per compute unit, four waves each, i.e. two waves per SIMD, the occupancy
// of the prefill kernel) reads its 16 operand registers per lane once and then issues only MFMAs on four
// independent accumulator chains; the accumulators are written out so that nothing is optimised away.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <cmath>
#include <ctime>
#include <unistd.h>
#include <vector>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

namespace {

constexpr int kGrid = 512, kThreads = 256, kOps = 16;  // u32x4 operand registers per lane (8 A, 8 B)
constexpr int kValuGrid = 2048;  // workgroups of the VALU timing loops (256 threads, one output word each)
constexpr int kMfmaPerIter = 16;
constexpr double kFlopPerMfma = 2.0 * 32 * 32 * 16;

__global__ __launch_bounds__(kThreads, 2) void mfma_loop(const u32x4* __restrict__ src, float* __restrict__ out, int iters) {
  const int tid = blockIdx.x * kThreads + threadIdx.x;
  u32x4 a[8], b[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = src[(size_t)tid * kOps + i];
    b[i] = src[(size_t)tid * kOps + 8 + i];
  }
  f32x16 acc[4] = {f32x16{}, f32x16{}, f32x16{}, f32x16{}};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      acc[(2 * j) & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[j]), __builtin_bit_cast(bf16x8, b[j]),
                                                                 acc[(2 * j) & 3], 0, 0, 0);
      acc[(2 * j + 1) & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[(j + 3) & 7]),
                                                                     __builtin_bit_cast(bf16x8, b[j]), acc[(2 * j + 1) & 3], 0, 0, 0);
    }
  }
  float r = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) r += acc[c][i];
  out[tid] = r;
}

// The sustained form's loop: the MFMA stream of mfma_loop (random operands) plus, per 16 MFMAs, the work that
// MIX selects: bit 0 the A operand of every MFMA from LDS (random operand data staged there at the start, 64 KB
// per workgroup), bit 1 independent VALU work (16 v_exp_f32 + 16 v_add_f32 + 48 v_fma_f32), bit 2 two 1 KB
// direct-to-LDS buffer loads per wave from the first kL2Bytes of `l2src` (a range that stays in the L2
// caches), waited for two iterations later, bit 3 (with bit 0) the same LDS bytes through two transposing
// 8-byte reads (ds_read_b64_tr_b16) per operand instead of one ds_read_b128, bit 4 one workgroup barrier,
// bit 5 24 scalar multiplies (s_mul_i32, which leaves the condition code alone) with the scalar adds that form
// their operands, about 48 scalar instructions, bit 6 the prefill's other VALU kinds in place of bit 1's
// exponentials and adds: 16 v_cvt_pk_bf16_f32 and 16 v_dot2c_f32_bf16 (as the weights are packed and summed)
// with the same 48 fmas, bit 7 the MFMA FLOP issued as v_mfma_f32_16x16x32_bf16 (twice as many instructions).
constexpr int kLdsOps = 4096;            // u32x4 of operand data in LDS
constexpr uint32_t kL2Bytes = 4u << 20;  // bytes of l2src the loads sweep
static_assert((size_t)kGrid * kLdsOps <= (size_t)kGrid * kThreads * kOps, "LDS staging reads stay inside src");
static_assert((size_t)kL2Bytes <= (size_t)kGrid * kThreads * kOps * 16, "the loads stay inside l2src");
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u32x4 tr_read16(const char* p) {
  const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4*)p);
  const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4*)(p + 8));
  return __builtin_bit_cast(u32x4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

template <int MIX>
__global__ __launch_bounds__(kThreads, 2) void mfma_mix(const u32x4* __restrict__ src, const uint8_t* __restrict__ l2src,
                                                        float* __restrict__ out, int iters) {
  __shared__ u32x4 lds[kLdsOps];
  __shared__ u32x4 dma_dst[kThreads / 64][2][64];
  const int tid = blockIdx.x * kThreads + threadIdx.x, lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if constexpr ((MIX & 1) != 0) {
    // kGrid * kLdsOps <= kGrid * kThreads * kOps: every workgroup's slice lies inside src
    for (int i = threadIdx.x; i < kLdsOps; i += kThreads) lds[i] = src[(size_t)blockIdx.x * kLdsOps + i];
    __syncthreads();
  }
  u32x4 a[8], b[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = src[(size_t)tid * kOps + i];
    b[i] = src[(size_t)tid * kOps + 8 + i];
  }
  float va[8], vb[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) va[i] = vb[i] = (float)(lane + i) * 1e-6f - 1.0f;
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)l2src, (short)0, (int)kL2Bytes, 0x00020000);
  const uint32_t gw = (uint32_t)(blockIdx.x * (kThreads / 64) + w);
  f32x16 acc[4] = {f32x16{}, f32x16{}, f32x16{}, f32x16{}};
  f32x4 acc4[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc4[c] = f32x4{};
  uint32_t salu = (uint32_t)blockIdx.x;
  for (int it = 0; it < iters; ++it) {
    if constexpr ((MIX & 4) != 0) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        // a 1 KB-aligned slot below kL2Bytes; lane l writes its 16 bytes at slot + 16 l
        const uint32_t off = (((uint32_t)(it * 2 + i) * (kGrid * kThreads / 64) + gw) * 1024u) & (kL2Bytes - 1);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)&dma_dst[w][i][0], 16, off + lane * 16, 0, 0, 0);
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      u32x4 a1 = a[j], a2 = a[(j + 3) & 7];
      const int i1 = ((it * 16 + 2 * j) * 64 + w * 1024 + lane) & (kLdsOps - 1);
      const int i2 = ((it * 16 + 2 * j + 1) * 64 + w * 1024 + lane) & (kLdsOps - 1);
      if constexpr ((MIX & 9) == 1) {
        a1 = lds[i1];
        a2 = lds[i2];
      } else if constexpr ((MIX & 9) == 9) {
        // the 16 bytes of lds[i] in two transposing 8-byte reads (the bytes each lane receives differ from
        // lds[i]'s, the bytes read per operand do not); every address stays inside lds
        a1 = tr_read16(reinterpret_cast<const char*>(lds) + i1 * 16);
        a2 = tr_read16(reinterpret_cast<const char*>(lds) + i2 * 16);
      }
      if constexpr ((MIX & 128) != 0) {
        // the same FLOP as four v_mfma_f32_16x16x32_bf16 (16 x 16 outputs, 32-deep), each A operand feeding two
        // of them as one 32x32 product's A operand would feed both of its 16-row halves
        acc4[(4 * j) & 7] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a1), __builtin_bit_cast(bf16x8, b[j]),
                                                                    acc4[(4 * j) & 7], 0, 0, 0);
        acc4[(4 * j + 1) & 7] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a1),
                                                                        __builtin_bit_cast(bf16x8, b[(j + 1) & 7]), acc4[(4 * j + 1) & 7], 0, 0, 0);
        acc4[(4 * j + 2) & 7] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a2), __builtin_bit_cast(bf16x8, b[j]),
                                                                        acc4[(4 * j + 2) & 7], 0, 0, 0);
        acc4[(4 * j + 3) & 7] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a2),
                                                                        __builtin_bit_cast(bf16x8, b[(j + 1) & 7]), acc4[(4 * j + 3) & 7], 0, 0, 0);
      } else {
        acc[(2 * j) & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a1), __builtin_bit_cast(bf16x8, b[j]),
                                                                   acc[(2 * j) & 3], 0, 0, 0);
        acc[(2 * j + 1) & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a2), __builtin_bit_cast(bf16x8, b[j]),
                                                                       acc[(2 * j + 1) & 3], 0, 0, 0);
      }
      if constexpr ((MIX & 64) != 0) {
        const bf16x2 p0 = {(__bf16)va[j], (__bf16)va[(j + 1) & 7]};
        const bf16x2 p1 = {(__bf16)va[(j + 2) & 7], (__bf16)va[(j + 3) & 7]};
        const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
        vb[j] = __builtin_amdgcn_fdot2_f32_bf16(p0, one, vb[j], false);
        vb[(j + 4) & 7] = __builtin_amdgcn_fdot2_f32_bf16(p1, one, vb[(j + 4) & 7], false);
#pragma unroll
        for (int u = 0; u < 6; ++u) va[(j + u) & 7] = __builtin_fmaf(va[(j + u) & 7], 0.999f, -0.001f);
      }
      if constexpr ((MIX & 2) != 0) {
        va[j] = __builtin_amdgcn_exp2f(va[j]) - 1.5f;
        va[(j + 4) & 7] = __builtin_amdgcn_exp2f(va[(j + 4) & 7]) - 1.5f;
#pragma unroll
        for (int u = 0; u < 6; ++u) vb[(j + u) & 7] = __builtin_fmaf(vb[(j + u) & 7], 0.999f, -0.001f);
      }
    }
    if constexpr ((MIX & 4) != 0) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    // every wave of the workgroup runs the same iterations, so each barrier is met by all four
    if constexpr ((MIX & 16) != 0) asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if constexpr ((MIX & 32) != 0) {
#pragma unroll
      for (int u = 0; u < 24; ++u) asm volatile("s_mul_i32 %0, %0, %1" : "+s"(salu) : "s"(2 * (u + it) + 1));
    }
  }
  if constexpr ((MIX & 4) != 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  float sum = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) sum += acc[c][i];
#pragma unroll
  for (int i = 0; i < 8; ++i) sum += va[i] + vb[i];
#pragma unroll
  for (int c = 0; c < 8; ++c) sum += acc4[c][0] + acc4[c][1] + acc4[c][2] + acc4[c][3];
  if constexpr ((MIX & 4) != 0) sum += __builtin_bit_cast(float, dma_dst[w][1][lane][0]) * 0.f;
  if constexpr ((MIX & 32) != 0) sum += (float)(salu & 1u) * 0.f;
  out[tid] = sum;
}

// the same with v_mfma_f32_32x32x64_f8f6f4 on OCP e4m3 operands (32 bytes per lane and operand): four A and
// four B operands from the same 16 registers, 8 MFMAs per iteration on four chains
constexpr double kFlopPerMfmaF8 = 2.0 * 32 * 32 * 64;
__global__ __launch_bounds__(kThreads, 2) void mfma_loop_f8(const u32x4* __restrict__ src, float* __restrict__ out,
                                                            int iters) {
  const int tid = blockIdx.x * kThreads + threadIdx.x;
  i32x8 a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u32x4 lo = src[(size_t)tid * kOps + 2 * i], hi = src[(size_t)tid * kOps + 2 * i + 1];
    const u32x4 lo2 = src[(size_t)tid * kOps + 8 + 2 * i], hi2 = src[(size_t)tid * kOps + 9 + 2 * i];
    a[i] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    b[i] = i32x8{(int)lo2[0], (int)lo2[1], (int)lo2[2], (int)lo2[3], (int)hi2[0], (int)hi2[1], (int)hi2[2], (int)hi2[3]};
  }
  f32x16 acc[4] = {f32x16{}, f32x16{}, f32x16{}, f32x16{}};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      acc[j & 3] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[j & 3], b[(j + (j >> 2)) & 3], acc[j & 3], 0, 0, 0, 0,
                                                                   0, 0);
  }
  float r = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) r += acc[c][i];
  out[tid] = r;
}

// VALU issue rate of one instruction kind: 8 independent chains per lane, OP 0 = v_fma_f32, 1 = v_exp_f32
// (each exponential followed by one v_add_f32 that keeps its argument in range)
template <int OP>
__global__ __launch_bounds__(256) void valu_loop(float* __restrict__ out, int iters) {
  float a[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = (float)(threadIdx.x + i) * 1e-6f - 1.0f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = OP == 0 ? __builtin_fmaf(a[i], 0.999f, -0.001f) : __builtin_amdgcn_exp2f(a[i]) - 1.5f;
  }
  float r = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) r += a[i];
  out[blockIdx.x * 256 + threadIdx.x] = r;
}

// Softmax weights of 8 scores per lane per iteration, packed to bf16 pairs as the attention kernels pack P:
// OP 0 = exponential weights 2^t (v_exp_f32, then a bf16 pack); OP 1 = power-of-two weights 2^round(t) built
// in the bf16 exponent field (clamp at the smallest normal exponent, round to an integer, shift, pack), the
// coarse logarithmic weights of the Rowmax-PoT idea, in the fewest full-rate instructions found.  Both share the scaling fma that produces t (a chain per
// element, so nothing is loop-invariant) and one xor per pair that keeps the result live.
template <int OP>
__global__ __launch_bounds__(256) void weight_loop(uint32_t* __restrict__ out, int iters) {
  float a[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = (float)(threadIdx.x + i) * 1e-6f - 1.0f;
  uint32_t acc = 0;
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      const float t0 = __builtin_fmaf(a[i], 0.999f, -0.001f), t1 = __builtin_fmaf(a[i + 1], 0.999f, -0.001f);
      uint32_t w;
      if constexpr (OP == 0) {
        const bf16x2 v = {(__bf16)__builtin_amdgcn_exp2f(t0), (__bf16)__builtin_amdgcn_exp2f(t1)};
        w = __builtin_bit_cast(uint32_t, v);
      } else {
        // k = t rounded to the nearest integer (ties to even) appears in the low mantissa bits of
        // t + 1.5 * 2^23 (0x4B400000 + k); the bf16 bits of 2^k are (k + 127) << 7, clamped at k = -126
        const uint32_t u0 = __builtin_bit_cast(uint32_t, __builtin_fmaxf(t0, -126.f) + 12582912.0f);
        const uint32_t u1 = __builtin_bit_cast(uint32_t, __builtin_fmaxf(t1, -126.f) + 12582912.0f);
        w = (((u0 << 7) + ((127u - 0x4B400000u) << 7)) & 0xffffu) | ((u1 << 23) + ((127u - 0x4B400000u) << 23));
      }
      acc ^= w;
      a[i] = t0;
      a[i + 1] = t1;
    }
  }
  out[blockIdx.x * 256 + threadIdx.x] = acc;
}

#define CHECK(x)                                                                        \
  do {                                                                                  \
    const hipError_t e_ = (x);                                                          \
    if (e_ != hipSuccess) {                                                             \
      std::fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));               \
      std::exit(1);                                                                     \
    }                                                                                   \
  } while (0)

// TFLOP/s of one timed launch (after one short warm-up launch) over the operands at `src`; f8: the fp8 loop
double rate(const u32x4* src, float* out, int iters, bool f8 = false) {
  auto launch = [&](int n) {
    if (f8) hipLaunchKernelGGL(mfma_loop_f8, dim3(kGrid), dim3(kThreads), 0, 0, src, out, n);
    else hipLaunchKernelGGL(mfma_loop, dim3(kGrid), dim3(kThreads), 0, 0, src, out, n);
  };
  launch(64);
  CHECK(hipGetLastError());
  CHECK(hipDeviceSynchronize());
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  CHECK(hipEventRecord(e0, 0));
  launch(iters);
  CHECK(hipGetLastError());
  CHECK(hipEventRecord(e1, 0));
  CHECK(hipEventSynchronize(e1));
  float ms = 0.f;
  CHECK(hipEventElapsedTime(&ms, e0, e1));
  CHECK(hipEventDestroy(e0));
  CHECK(hipEventDestroy(e1));
  const double waves = (double)kGrid * kThreads / 64;
  return f8 ? waves * iters * 8 * kFlopPerMfmaF8 / (ms * 1e-3) / 1e12
            : waves * iters * kMfmaPerIter * kFlopPerMfma / (ms * 1e-3) / 1e12;
}

// weights per second per SIMD (one per lane and score) of weight_loop<OP>
template <int OP>
double weight_rate(uint32_t* out, int num_simds) {
  const int grid = kValuGrid, iters = 4096;
  hipLaunchKernelGGL(weight_loop<OP>, dim3(grid), dim3(256), 0, 0, out, 16);
  CHECK(hipGetLastError());
  CHECK(hipDeviceSynchronize());
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  float best = 1e30f;
  for (int rep = 0; rep < 3; ++rep) {
    CHECK(hipEventRecord(e0, 0));
    hipLaunchKernelGGL(weight_loop<OP>, dim3(grid), dim3(256), 0, 0, out, iters);
    CHECK(hipGetLastError());
    CHECK(hipEventRecord(e1, 0));
    CHECK(hipEventSynchronize(e1));
    float ms = 0.f;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    best = ms < best ? ms : best;
  }
  CHECK(hipEventDestroy(e0));
  CHECK(hipEventDestroy(e1));
  return (double)grid * 256 * iters * 8 / num_simds / (best * 1e-3);
}

// wave instructions per second per SIMD of valu_loop<OP> (OP 1 counts the exponential and its add as two)
template <int OP>
double valu_rate(float* out, int num_simds) {
  const int grid = kValuGrid, iters = 4096;
  hipLaunchKernelGGL(valu_loop<OP>, dim3(grid), dim3(256), 0, 0, out, 16);
  CHECK(hipGetLastError());
  CHECK(hipDeviceSynchronize());
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  CHECK(hipEventRecord(e0, 0));
  hipLaunchKernelGGL(valu_loop<OP>, dim3(grid), dim3(256), 0, 0, out, iters);
  CHECK(hipGetLastError());
  CHECK(hipEventRecord(e1, 0));
  CHECK(hipEventSynchronize(e1));
  float ms = 0.f;
  CHECK(hipEventElapsedTime(&ms, e0, e1));
  CHECK(hipEventDestroy(e0));
  CHECK(hipEventDestroy(e1));
  const double insts = (double)grid * 4 * iters * 8 * (OP == 0 ? 1 : 2);
  return insts / num_simds / (ms * 1e-3);
}

// SplitMix64 (Steele, Lea, Flood 2014), used here only to fill operand registers with varied bits
uint64_t splitmix64(uint64_t& s) {
  uint64_t z = (s += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

}  // namespace

double now_monotonic() {
  timespec ts;
  clock_gettime(CLOCK_MONOTONIC, &ts);
  return (double)ts.tv_sec + 1e-9 * (double)ts.tv_nsec;
}

typedef void (*mix_fn)(const u32x4*, const uint8_t*, float*, int);
mix_fn mix_kernel(int mix) {
  switch (mix) {
    case 0: return mfma_mix<0>;
    case 1: return mfma_mix<1>;
    case 2: return mfma_mix<2>;
    case 4: return mfma_mix<4>;
    case 9: return mfma_mix<9>;
    case 16: return mfma_mix<16>;
    case 32: return mfma_mix<32>;
    case 64: return mfma_mix<64>;
    case 128: return mfma_mix<128>;
    default: return mfma_mix<7>;
  }
}

// one phase of the sustained form: mfma_mix<mix> over `src` launched back to back for `seconds` (src null: the
// GPU left idle); prints the phase's interval, its rate and its wave-iterations (16 MFMAs each) per second
void sustain_phase(const char* name, const u32x4* src, const uint8_t* l2src, float* out, int iters, int mix,
                   double seconds, bool first) {
  CHECK(hipDeviceSynchronize());
  const mix_fn f = mix_kernel(mix);
  if (src != nullptr) {
    hipLaunchKernelGGL(f, dim3(kGrid), dim3(kThreads), 0, 0, src, l2src, out, 64);
    CHECK(hipGetLastError());
    CHECK(hipDeviceSynchronize());
  }
  const double t0 = now_monotonic();
  double wave_iters = 0.0;
  if (src == nullptr) {
    usleep((useconds_t)(seconds * 1e6));
  } else {
    while (now_monotonic() - t0 < seconds) {
      for (int i = 0; i < 4; ++i) hipLaunchKernelGGL(f, dim3(kGrid), dim3(kThreads), 0, 0, src, l2src, out, iters);
      CHECK(hipGetLastError());
      CHECK(hipDeviceSynchronize());
      wave_iters += 4.0 * kGrid * (kThreads / 64) * iters;
    }
  }
  const double t1 = now_monotonic();
  std::printf("%s{\"phase\": \"%s\", \"mix\": %d, \"t0\": %.4f, \"t1\": %.4f, \"tflops\": %.1f, "
              "\"wave_iters_per_s\": %.5e}", first ? "" : ", ", name, src ? mix : -1, t0, t1,
              wave_iters * kMfmaPerIter * kFlopPerMfma / (t1 - t0) / 1e12, wave_iters / (t1 - t0));
}

int main(int argc, char** argv) {
  const int iters = argc > 1 ? std::atoi(argv[1]) : 20000;
  const bool sustain = argc > 3 && std::strcmp(argv[2], "sustain") == 0;
  const double seconds = sustain ? std::atof(argv[3]) : 0.0;
  if (iters <= 0 || (argc > 2 && !(sustain && seconds > 0.0 && seconds <= 60.0))) {
    std::fprintf(stderr, "usage: mfma_ceiling [iterations > 0] [sustain SECONDS (0, 60]]\n");
    return 2;
  }
  const size_t n = (size_t)kGrid * kThreads * kOps;  // u32x4 elements
  // random operands: bf16 of values uniform in [-2, 2)
  std::vector<uint32_t> host(n * 4);
  uint64_t state = 2026;
  for (size_t i = 0; i < host.size(); ++i) {
    uint32_t w = 0;
    for (int h = 0; h < 2; ++h) {
      const float f = (float)((double)(splitmix64(state) >> 11) * 0x1.0p-53 * 4.0 - 2.0);
      uint32_t u;
      std::memcpy(&u, &f, 4);
      w |= (u >> 16) << (16 * h);
    }
    host[i] = w;
  }
  // random OCP e4m3 codes for the fp8 loop (the two NaN codes replaced by the largest finite ones)
  std::vector<uint32_t> host8(n * 4);
  for (size_t i = 0; i < host8.size(); ++i) {
    uint32_t w = 0;
    for (int h = 0; h < 4; ++h) {
      uint32_t c = (uint32_t)(splitmix64(state) >> 56);
      if ((c & 0x7F) == 0x7F) c -= 1;
      w |= c << (8 * h);
    }
    host8[i] = w;
  }
  u32x4 *zero = nullptr, *rnd = nullptr, *rnd8 = nullptr;
  float* out = nullptr;
  CHECK(hipMalloc(&zero, n * sizeof(u32x4)));
  CHECK(hipMalloc(&rnd, n * sizeof(u32x4)));
  CHECK(hipMalloc(&rnd8, n * sizeof(u32x4)));
  CHECK(hipMemcpy(rnd8, host8.data(), n * sizeof(u32x4), hipMemcpyHostToDevice));
  // one word per thread of the largest grid that writes it (the VALU loops' kValuGrid x 256)
  CHECK(hipMalloc(&out, (size_t)(kGrid > kValuGrid ? kGrid : kValuGrid) * kThreads * sizeof(float)));
  CHECK(hipMemset(zero, 0, n * sizeof(u32x4)));
  CHECK(hipMemcpy(rnd, host.data(), n * sizeof(u32x4), hipMemcpyHostToDevice));
  if (sustain) {
    std::printf("{\"instruction\": \"v_mfma_f32_32x32x16_bf16\", \"mode\": \"sustain\", \"iterations\": %d, "
                "\"seconds\": %.1f, \"clock\": \"CLOCK_MONOTONIC\", \"phases\": [", iters, seconds);
    // the loads of the mixed phases sweep the first 4 MB of the random fp8 codes (n u32x4 = 32 MB)
    const uint8_t* l2src = reinterpret_cast<const uint8_t*>(rnd8);
    sustain_phase("idle", nullptr, nullptr, out, iters, 0, seconds, true);
    sustain_phase("zero", zero, l2src, out, iters, 0, seconds, false);
    const struct { const char* name; int mix; } mixed[] = {
        {"random", 0}, {"random+lds_operands", 1}, {"random+lds_operands_transposing", 9}, {"random+valu", 2},
        {"random+valu_convert_dot", 64}, {"random+tile_loads", 4}, {"random+barrier", 16}, {"random+scalar", 32},
        {"random+all", 7}, {"random_16x16x32", 128}};
    for (const auto& m : mixed) {
      sustain_phase("idle", nullptr, nullptr, out, iters, 0, seconds / 2, false);
      sustain_phase(m.name, rnd, l2src, out, iters, m.mix, seconds, false);
    }
    // the MFMA loop alone on normal operands (bf16 of N(0, 1) values, as the attention inputs are drawn) in
    // place of uniform ones, over the zero buffer, which is no longer needed
    std::vector<uint32_t> gauss(n * 4);
    for (size_t i = 0; i < gauss.size(); ++i) {
      uint32_t w = 0;
      for (int h = 0; h < 2; ++h) {
        // Box-Muller on two 53-bit uniforms, the first in (0, 1]
        const double u1 = (double)((splitmix64(state) >> 11) + 1) * 0x1.0p-53;
        const double u2 = (double)(splitmix64(state) >> 11) * 0x1.0p-53;
        const float f = (float)(std::sqrt(-2.0 * std::log(u1)) * std::cos(6.283185307179586 * u2));
        uint32_t u;
        std::memcpy(&u, &f, 4);
        w |= (u >> 16) << (16 * h);
      }
      gauss[i] = w;
    }
    CHECK(hipMemcpy(zero, gauss.data(), n * sizeof(u32x4), hipMemcpyHostToDevice));
    sustain_phase("idle", nullptr, nullptr, out, iters, 0, seconds / 2, false);
    sustain_phase("normal", zero, l2src, out, iters, 0, seconds, false);
    std::printf("]}\n");
    CHECK(hipFree(zero));
    CHECK(hipFree(rnd));
    CHECK(hipFree(rnd8));
    CHECK(hipFree(out));
    return 0;
  }
  double z = 0, r = 0, z8 = 0, r8 = 0;
  for (int rep = 0; rep < 2; ++rep) {  // the better of two runs each
    const double rz = rate(zero, out, iters), rr = rate(rnd, out, iters);
    const double rz8 = rate(zero, out, iters, true), rr8 = rate(rnd8, out, iters, true);
    z = rz > z ? rz : z;
    r = rr > r ? rr : r;
    z8 = rz8 > z8 ? rz8 : z8;
    r8 = rr8 > r8 ? rr8 : r8;
  }
  // VALU: the exponential's cost relative to an fma follows from the two rates (the clock is the same)
  int dev = 0, num_cus = 0;
  CHECK(hipGetDevice(&dev));
  CHECK(hipDeviceGetAttribute(&num_cus, hipDeviceAttributeMultiprocessorCount, dev));
  const double fma_rate = valu_rate<0>(out, num_cus * 4), pair_rate = valu_rate<1>(out, num_cus * 4) / 2.0;
  uint32_t* out32 = reinterpret_cast<uint32_t*>(out);
  const double exp_w = weight_rate<0>(out32, num_cus * 4), pot_w = weight_rate<1>(out32, num_cus * 4);
  std::printf("{\"instruction\": \"v_mfma_f32_32x32x16_bf16\", \"zero_operands_tflops\": %.1f, "
              "\"random_operands_tflops\": %.1f, \"published_peak_tflops\": 2500.0, \"workgroups\": %d, "
              "\"waves_per_simd\": 2, \"iterations\": %d, \"valu_fma_f32_per_us_per_simd\": %.1f, "
              "\"valu_exp_f32_plus_add_per_us_per_simd\": %.1f, \"exp_plus_add_in_fma_times\": %.2f, "
              "\"weights\": {\"exp2_bf16_per_us_per_simd\": %.1f, \"pow2_bf16_per_us_per_simd\": %.1f, "
              "\"pow2_time_over_exp2_time\": %.3f}, "
              "\"fp8\": {\"instruction\": \"v_mfma_f32_32x32x64_f8f6f4\", \"zero_operands_tflops\": %.1f, "
              "\"random_operands_tflops\": %.1f, \"published_peak_tflops\": 5000.0}}\n",
              z, r, kGrid, iters, fma_rate * 1e-6, pair_rate * 1e-6, fma_rate / pair_rate, exp_w * 1e-6, pot_w * 1e-6,
              exp_w / pot_w, z8, r8);
  CHECK(hipFree(zero));
  CHECK(hipFree(rnd));
  CHECK(hipFree(rnd8));
  CHECK(hipFree(out));
  return 0;
}
