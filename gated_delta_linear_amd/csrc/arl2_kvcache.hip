// K/V cache of the retained softmax layers ("Attend Locally, Remember Linearly",
// gist.science technical summary, section 1: the cache grows by one block of keys and values
// per generated frame): copy one frame's k and v, [B][T][H][d] bf16, into rows
// [row0, row0 + T) of the caches [B][rows][H][d].  Per stream both sides are contiguous, so
// the copy runs in 16-byte units, grid-stride.
#include "arl2_device.h"
#include "arl2_kernels.h"

namespace arl2 {
namespace {

__global__ __launch_bounds__(256) void arl2_kv_append_kernel(const uint4* __restrict__ k, const uint4* __restrict__ v,
                                                             uint4* __restrict__ kc, uint4* __restrict__ vc,
                                                             int64_t n16, int64_t dst0, int64_t slice16, int64_t total) {
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < total; e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t b = e / n16, i = e - b * n16;
    const int64_t o = b * slice16 + dst0 + i;
    kc[o] = k[e];
    vc[o] = v[e];
  }
}

}  // namespace

hipError_t launch_kv_append(const KvAppendArgs& a, hipStream_t stream) {
  const int64_t n16 = (int64_t)a.T * a.H * a.d / 8;  // 16-byte units of one stream's frame
  const int64_t total = n16 * a.B;
  const int64_t blocks = (total + 255) / 256 < 2048 ? (total + 255) / 256 : 2048;
  hipLaunchKernelGGL(arl2_kv_append_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     static_cast<const uint4*>(a.k), static_cast<const uint4*>(a.v), static_cast<uint4*>(a.kc),
                     static_cast<uint4*>(a.vc), n16, (int64_t)a.row0 * a.H * a.d / 8,
                     (int64_t)a.rows * a.H * a.d / 8, total);
  return hipGetLastError();
}

}  // namespace arl2
