// fp32 -> bf16 input staging of the ARL2 layer (io_dtype ARL2_F32): the caller's fp32 q, k, v
// (and, at creation, phi_q, phi_k, phi_v) are rounded to nearest even into bf16 copies that the
// bf16 kernels then read, so an fp32 caller gets exactly the bf16 path on the rounded values.
#include "arl2_device.h"
#include "arl2_kernels.h"

namespace arl2 {
namespace {

// Tensor blockIdx.y of the job: 8 values per thread, grid-stride over n8 groups of 8.
__global__ __launch_bounds__(256) void arl2_cvt_bf16_kernel(const CvtJobs jobs, int64_t n8) {
  const float* __restrict__ src = jobs.src[blockIdx.y];
  bf16* __restrict__ dst = static_cast<bf16*>(jobs.dst[blockIdx.y]);
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n8; i += (int64_t)gridDim.x * blockDim.x) {
    const f32x4 a = reinterpret_cast<const f32x4*>(src)[2 * i];
    const f32x4 b = reinterpret_cast<const f32x4*>(src)[2 * i + 1];
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      o[e] = (bf16)a[e];  // round to nearest even
      o[4 + e] = (bf16)b[e];
    }
    reinterpret_cast<bf16x8*>(dst)[i] = o;
  }
}

}  // namespace

hipError_t launch_cvt_bf16(const CvtJobs& jobs, int n_jobs, int64_t n, hipStream_t stream) {
  if (n_jobs < 1 || n_jobs > 3 || n % 8) return hipErrorInvalidValue;
  if (n == 0) return hipSuccess;
  const int64_t n8 = n / 8;
  const int64_t want = (n8 + 255) / 256;
  const int blocks = (int)(want < 2048 ? want : 2048);
  hipLaunchKernelGGL(arl2_cvt_bf16_kernel, dim3(blocks, n_jobs), dim3(256), 0, stream, jobs, n8);
  return hipGetLastError();
}

}  // namespace arl2
