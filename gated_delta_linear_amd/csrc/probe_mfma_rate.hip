// Sustained dense bf16 MFMA rate of the chip: a measurement aid for the roofline, not part of the
// layer.  Each work-group (8 waves, two per SIMD, 96 KB of LDS so that one work-group holds a CU)
// runs independent chains of 32x32x16 bf16 MFMAs with fp32 accumulation, 8 per wave and
// iteration, and nothing else.  For a grid of G work-groups the program prints, as one JSON line
// per grid: the achieved rate (FLOPs over the kernel's wall time from HIP events) and the shader
// clock the waves saw (their s_memtime cycle count over the same wall time).  Grids: 156 (one
// work-group per 128-query tile of a 12-head, 1560-token pass) and 256 (every CU).
//
// Usage: probe_mfma_rate [iterations]
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <vector>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWaves = 8;
constexpr int kChains = 8;                      // independent accumulators per wave
constexpr double kFlopPerMfma = 2.0 * 32 * 32 * 16;

__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(2, 2))) void mfma_rate_kernel(
    unsigned long long* __restrict__ cycles, float* __restrict__ sink, int iters) {
  __shared__ unsigned char hold[96 * 1024];  // one work-group per CU
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (iters < 0) hold[tid] = 0;  // never taken: keeps the allocation
  bf16x8 a[kChains];
#pragma unroll
  for (int j = 0; j < kChains; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) a[j][e] = (__bf16)(1e-3f * (float)(lane + e + 3 * j));
  f32x16 acc[kChains];
#pragma unroll
  for (int j = 0; j < kChains; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
  __syncthreads();
  const unsigned long long t0 = __builtin_readcyclecounter();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kChains; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j], a[(j + 1) % kChains], acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kChains; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[j][e];
  const unsigned long long t1 = __builtin_readcyclecounter();
  sink[blockIdx.x * blockDim.x + tid] = s;  // keeps the chains live
  if (lane == 0) cycles[blockIdx.x * kWaves + wave] = t1 - t0;
}

bool ok(hipError_t e, const char* what) {
  if (e != hipSuccess) {
    std::fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
    return false;
  }
  return true;
}

bool run(int grid, int iters) {
  unsigned long long* cyc = nullptr;
  float* sink = nullptr;
  if (!ok(hipMalloc(&cyc, sizeof(unsigned long long) * grid * kWaves), "hipMalloc") ||
      !ok(hipMalloc(&sink, sizeof(float) * grid * 64 * kWaves), "hipMalloc"))
    return false;
  hipEvent_t e0, e1;
  if (!ok(hipEventCreate(&e0), "hipEventCreate") || !ok(hipEventCreate(&e1), "hipEventCreate")) return false;
  // warm-up launches (clock ramp), then one timed launch
  for (int w = 0; w < 3; ++w) hipLaunchKernelGGL(mfma_rate_kernel, dim3(grid), dim3(64 * kWaves), 0, 0, cyc, sink, iters);
  if (!ok(hipEventRecord(e0, 0), "hipEventRecord")) return false;
  hipLaunchKernelGGL(mfma_rate_kernel, dim3(grid), dim3(64 * kWaves), 0, 0, cyc, sink, iters);
  if (!ok(hipGetLastError(), "launch") || !ok(hipEventRecord(e1, 0), "hipEventRecord") ||
      !ok(hipEventSynchronize(e1), "hipEventSynchronize"))
    return false;
  float ms = 0.f;
  if (!ok(hipEventElapsedTime(&ms, e0, e1), "hipEventElapsedTime")) return false;
  std::vector<unsigned long long> h((size_t)grid * kWaves);
  if (!ok(hipMemcpy(h.data(), cyc, h.size() * sizeof(h[0]), hipMemcpyDeviceToHost), "hipMemcpy")) return false;
  std::sort(h.begin(), h.end());
  const double med_cycles = (double)h[h.size() / 2];
  const double flops = kFlopPerMfma * kChains * (double)iters * kWaves * grid;
  const double tflops = flops / (ms * 1e-3) / 1e12;
  const double ghz = med_cycles / (ms * 1e-3) / 1e9;
  // cycles per MFMA per SIMD (two waves share a SIMD): 32 at the full rate
  const double cyc_per_mfma = med_cycles / ((double)iters * kChains * 2);
  std::printf("{\"work_groups\": %d, \"waves_per_simd\": 2, \"iterations\": %d, \"ms\": %.4f, \"tflops\": %.1f, "
              "\"clock_ghz\": %.3f, \"cycles_per_mfma_per_simd\": %.2f, \"frac_of_2500\": %.4f}\n",
              grid, iters, ms, tflops, ghz, cyc_per_mfma, tflops / 2500.0);
  (void)hipFree(cyc);
  (void)hipFree(sink);
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  return true;
}

}  // namespace

int main(int argc, char** argv) {
  const int iters = argc > 1 ? std::atoi(argv[1]) : 40000;
  if (iters <= 0 || iters > 10000000) {
    std::fprintf(stderr, "iterations must be in (0, 1e7]\n");
    return 2;
  }
  for (int grid : {156, 256})
    if (!run(grid, iters)) return 1;
  return 0;
}
