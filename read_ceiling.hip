// read_ceiling.hip -- the rate at which this GPU streams reads from HBM in the decode kernel's load shapes,
// with no compute.  Every tile of a 4 GiB buffer is read exactly once (the last-level cache holds 256 MiB,
// so nothing is re-read from it).  Prints one JSON line.
//   read_ceiling
//
// Shapes (per load instruction of one wave, 16 bytes per lane unless noted):
//   k_bf16    16 key rows x 64 B of 256-byte rows (the bf16 K tile of 64 rows, 16 KB, in 16 instructions)
//   rows_256  4 rows x 256 B (row-contiguous reads of the same 16 KB tile)
//   k_fp8     16 key rows x 64 B of 128-byte rows (the fp8 K tile, 8 KB, in 8 instructions)
//   k_fp8_b64 16 key rows x 32 B of 128-byte rows, 8 bytes per lane (8 KB in 16 instructions)
// each at 2 workgroups of 4 waves per CU with one or two tiles in flight per wave, and at 4 workgroups with
// one; the bf16 shapes also with the non-temporal cache policy (the `nt` bit, `_nt`).  Tile i of wave w is tile
// (i * waves + w) of the buffer, so the grid sweeps the buffer front to back.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

namespace {

enum Shape { kKBf16 = 0, kRows256 = 1, kKFp8 = 2, kKFp8B64 = 3 };

constexpr int kNT = 2;  // cache policy bits of the buffer loads: non-temporal

constexpr uint32_t tile_bytes(int shape) { return shape <= kRows256 ? 16384u : 8192u; }

// byte offset of load i of a tile for this lane; every offset + access width stays inside the tile
__device__ __forceinline__ uint32_t load_offset(int shape, int i, int lane) {
  const int r = lane % 16, c = lane / 16;
  switch (shape) {
    case kKBf16: return (uint32_t)(((i / 4) * 16 + r) * 256 + c * 16 + (i % 4) * 64);
    case kRows256: return (uint32_t)((i * 4 + lane / 16) * 256 + (lane % 16) * 16);
    case kKFp8: return (uint32_t)(((i / 2) * 16 + r) * 128 + c * 16 + (i % 2) * 64);
    default: return (uint32_t)(((i / 4) * 16 + r) * 128 + c * 8 + (i % 4) * 32);
  }
}

template <int SHAPE, int DEPTH, int OCC, int POLICY>
__global__ __launch_bounds__(256, OCC) void stream(const uint8_t* __restrict__ src, uint64_t nbytes,
                                                   uint32_t* __restrict__ out, int tiles_per_wave) {
  constexpr uint32_t TB = tile_bytes(SHAPE);
  constexpr int NL = SHAPE == kKFp8 ? 8 : 16;  // load instructions per tile
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * 4 + (threadIdx.x >> 6), nw = gridDim.x * 4;
  u32x4 acc = {};
  for (int t = 0; t < tiles_per_wave; t += DEPTH) {
    u32x4 x[DEPTH][NL];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      const uint64_t base = ((uint64_t)(t + d) * nw + gw) * TB;
      // a tile past the end gets an empty resource (its loads read zero); the host sizes the sweep so that
      // none is
      const bool ok = base + TB <= nbytes;
      const __amdgpu_buffer_rsrc_t r =
          __builtin_amdgcn_make_buffer_rsrc((void*)(src + (ok ? base : 0)), (short)0, ok ? (int)TB : 0, 0x00020000);
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const uint32_t off = load_offset(SHAPE, i, lane);
        if constexpr (SHAPE == kKFp8B64) {
          const u32x2 y = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, POLICY);
          x[d][i] = u32x4{y[0], y[1], 0u, 0u};
        } else {
          x[d][i] = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, POLICY);
        }
      }
    }
#pragma unroll
    for (int d = 0; d < DEPTH; ++d)
#pragma unroll
      for (int i = 0; i < NL; ++i) acc ^= x[d][i];
  }
  out[blockIdx.x * 256 + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

#define CHECK(x)                                                                        \
  do {                                                                                  \
    const hipError_t e_ = (x);                                                          \
    if (e_ != hipSuccess) {                                                             \
      std::fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));               \
      std::exit(1);                                                                     \
    }                                                                                   \
  } while (0)

// GB/s of the best of three sweeps
template <int SHAPE, int DEPTH, int OCC, int POLICY = 0>
double rate(const uint8_t* src, uint64_t nbytes, uint32_t* out, int num_cus) {
  const int grid = num_cus * OCC;
  const uint32_t TB = tile_bytes(SHAPE);
  const int tpw = (int)(nbytes / TB / ((uint64_t)grid * 4)) / DEPTH * DEPTH;
  hipLaunchKernelGGL((stream<SHAPE, DEPTH, OCC, POLICY>), dim3(grid), dim3(256), 0, 0, src, nbytes, out, DEPTH);
  CHECK(hipGetLastError());
  CHECK(hipDeviceSynchronize());
  float best = 1e30f;
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  for (int rep = 0; rep < 3; ++rep) {
    CHECK(hipEventRecord(e0, 0));
    hipLaunchKernelGGL((stream<SHAPE, DEPTH, OCC, POLICY>), dim3(grid), dim3(256), 0, 0, src, nbytes, out, tpw);
    CHECK(hipGetLastError());
    CHECK(hipEventRecord(e1, 0));
    CHECK(hipEventSynchronize(e1));
    float ms = 0.f;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    best = ms < best ? ms : best;
  }
  CHECK(hipEventDestroy(e0));
  CHECK(hipEventDestroy(e1));
  return (double)grid * 4 * tpw * TB / (best * 1e-3) / 1e9;
}

}  // namespace

int main() {
  const uint64_t nbytes = 4ull << 30;
  int dev = 0, num_cus = 0;
  CHECK(hipGetDevice(&dev));
  CHECK(hipDeviceGetAttribute(&num_cus, hipDeviceAttributeMultiprocessorCount, dev));
  uint8_t* src = nullptr;
  uint32_t* out = nullptr;
  CHECK(hipMalloc(&src, nbytes));
  CHECK(hipMalloc(&out, (size_t)num_cus * 4 * 256 * sizeof(uint32_t)));
  CHECK(hipMemset(src, 1, nbytes));
  CHECK(hipDeviceSynchronize());
  struct R { const char* name; double gbps; } res[] = {
      {"k_bf16_depth1_2wg", rate<kKBf16, 1, 2>(src, nbytes, out, num_cus)},
      {"k_bf16_depth2_2wg", rate<kKBf16, 2, 2>(src, nbytes, out, num_cus)},
      {"k_bf16_depth1_4wg", rate<kKBf16, 1, 4>(src, nbytes, out, num_cus)},
      {"rows_256_depth1_2wg", rate<kRows256, 1, 2>(src, nbytes, out, num_cus)},
      {"rows_256_depth1_4wg", rate<kRows256, 1, 4>(src, nbytes, out, num_cus)},
      {"rows_256_depth2_2wg", rate<kRows256, 2, 2>(src, nbytes, out, num_cus)},
      {"k_fp8_depth1_2wg", rate<kKFp8, 1, 2>(src, nbytes, out, num_cus)},
      {"k_fp8_depth2_2wg", rate<kKFp8, 2, 2>(src, nbytes, out, num_cus)},
      {"k_fp8_b64_depth1_2wg", rate<kKFp8B64, 1, 2>(src, nbytes, out, num_cus)},
      {"k_fp8_b64_depth2_2wg", rate<kKFp8B64, 2, 2>(src, nbytes, out, num_cus)},
      {"k_bf16_depth2_2wg_nt", rate<kKBf16, 2, 2, kNT>(src, nbytes, out, num_cus)},
      {"rows_256_depth1_2wg_nt", rate<kRows256, 1, 2, kNT>(src, nbytes, out, num_cus)},
      {"rows_256_depth2_2wg_nt", rate<kRows256, 2, 2, kNT>(src, nbytes, out, num_cus)},
      {"rows_256_depth1_4wg_nt", rate<kRows256, 1, 4, kNT>(src, nbytes, out, num_cus)},
  };
  double best = 0;
  std::printf("{\"buffer_bytes\": %llu, \"compute_units\": %d, \"gbps\": {", (unsigned long long)nbytes, num_cus);
  for (size_t i = 0; i < sizeof(res) / sizeof(res[0]); ++i) {
    std::printf("%s\"%s\": %.1f", i ? ", " : "", res[i].name, res[i].gbps);
    best = res[i].gbps > best ? res[i].gbps : best;
  }
  std::printf("}, \"best_gbps\": %.1f, \"published_peak_gbps\": 8000.0}\n", best);
  CHECK(hipFree(src));
  CHECK(hipFree(out));
  return 0;
}
