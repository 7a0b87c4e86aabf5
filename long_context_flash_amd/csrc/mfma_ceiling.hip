// mfma_ceiling.hip -- the rate at which this GPU sustains v_mfma_f32_32x32x16_bf16 (the matrix instruction
// of the prefill kernel), once with operands that are all zero and once with random bf16 operands.  The
// chip's clock depends on its power draw, which depends on the operand bits, so the second figure is the
// practical ceiling for a kernel that multiplies real data; the first approaches the published peak.
//
// Standalone measurement program (not part of libssm.so).  Prints one JSON line.
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

namespace {

constexpr int kGrid = 512, kThreads = 256, kOps = 16;  // u32x4 operand registers per lane (8 A, 8 B)
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

#define CHECK(x)                                                                        \
  do {                                                                                  \
    const hipError_t e_ = (x);                                                          \
    if (e_ != hipSuccess) {                                                             \
      std::fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));               \
      std::exit(1);                                                                     \
    }                                                                                   \
  } while (0)

// TFLOP/s of one timed launch (after one short warm-up launch) over the operands at `src`
double rate(const u32x4* src, float* out, int iters) {
  hipLaunchKernelGGL(mfma_loop, dim3(kGrid), dim3(kThreads), 0, 0, src, out, 64);
  CHECK(hipGetLastError());
  CHECK(hipDeviceSynchronize());
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  CHECK(hipEventRecord(e0, 0));
  hipLaunchKernelGGL(mfma_loop, dim3(kGrid), dim3(kThreads), 0, 0, src, out, iters);
  CHECK(hipGetLastError());
  CHECK(hipEventRecord(e1, 0));
  CHECK(hipEventSynchronize(e1));
  float ms = 0.f;
  CHECK(hipEventElapsedTime(&ms, e0, e1));
  CHECK(hipEventDestroy(e0));
  CHECK(hipEventDestroy(e1));
  const double waves = (double)kGrid * kThreads / 64;
  return waves * iters * kMfmaPerIter * kFlopPerMfma / (ms * 1e-3) / 1e12;
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
  u32x4 *zero = nullptr, *rnd = nullptr;
  float* out = nullptr;
  CHECK(hipMalloc(&zero, n * sizeof(u32x4)));
  CHECK(hipMalloc(&rnd, n * sizeof(u32x4)));
  CHECK(hipMalloc(&out, (size_t)kGrid * kThreads * sizeof(float)));
  CHECK(hipMemset(zero, 0, n * sizeof(u32x4)));
  CHECK(hipMemcpy(rnd, host.data(), n * sizeof(u32x4), hipMemcpyHostToDevice));
  double z = 0, r = 0;
  for (int rep = 0; rep < 2; ++rep) {  // the better of two runs each
    const double rz = rate(zero, out, iters), rr = rate(rnd, out, iters);
    z = rz > z ? rz : z;
    r = rr > r ? rr : r;
  }
  std::printf("{\"instruction\": \"v_mfma_f32_32x32x16_bf16\", \"zero_operands_tflops\": %.1f, "
              "\"random_operands_tflops\": %.1f, \"published_peak_tflops\": 2500.0, \"workgroups\": %d, "
              "\"waves_per_simd\": 2, \"iterations\": %d}\n",
              z, r, kGrid, iters);
  CHECK(hipFree(zero));
  CHECK(hipFree(rnd));
  CHECK(hipFree(out));
  return 0;
}
