// mfma_ceiling.hip -- the rate at which this GPU sustains v_mfma_f32_32x32x16_bf16 (the matrix instruction
// of the prefill kernel), once with operands that are all zero and once with random bf16 operands.  The
// chip's clock depends on its power draw, which depends on the operand bits, so the second figure is the
// practical ceiling for a kernel that multiplies real data; the first approaches the published peak.
//
// Standalone measurement program (not part of libssm.so).  Prints one JSON line.  It also times the VALU
// rate of v_fma_f32 and of v_exp_f32 (the exponential of the softmax step) followed by an add, and reports
// how many fma issue slots one exponential with its add takes.
//   mfma_ceiling [iterations]
//
// Each of 512 workgroups (two per compute unit, four waves each, i.e. two waves per SIMD, the occupancy
// of the prefill kernel) reads its 16 operand registers per lane once and then issues only MFMAs on four
// independent accumulator chains; the accumulators are written out so that nothing is optimised away.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

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

int main(int argc, char** argv) {
  const int iters = argc > 1 ? std::atoi(argv[1]) : 20000;
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
