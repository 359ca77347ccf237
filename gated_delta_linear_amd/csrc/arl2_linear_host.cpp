// Host side of the linear projections (include/arl2_linear.h): argument checks and the launch.
#include <hip/hip_runtime.h>

#include "../../include/arl2_linear.h"
#include "arl2_host_util.h"
#include "arl2_kernels.h"

using arl2host::aligned16;
using arl2host::fail;

extern "C" arl2_status arl2_linear(const void* x, const void* w_t, int32_t m, int32_t n, int32_t k, int32_t parts,
                                   void* const* y, int32_t y_dtype, void* stream_) {
  if (m < 0 || n < 0 || k < 0) return fail(ARL2_E_INVALID_ARG, "m, n and k must be >= 0");
  if (k % 64) return fail(ARL2_E_UNSUPPORTED, "k must be a multiple of 64 (got %d)", k);
  if (k > (1 << 20)) return fail(ARL2_E_UNSUPPORTED, "k must be at most 2^20 (got %d)", k);
  if (n % 8) return fail(ARL2_E_UNSUPPORTED, "n must be a multiple of 8 (got %d)", n);
  if (parts < 1 || parts > arl2::kLinearMaxParts) return fail(ARL2_E_INVALID_ARG, "parts must be in [1, 4]");
  if (n % parts || (n / parts) % 4) return fail(ARL2_E_INVALID_ARG, "n / parts must be a whole multiple of 4");
  if (y_dtype != ARL2_F32 && y_dtype != ARL2_BF16) return fail(ARL2_E_INVALID_ARG, "bad y_dtype");
  if (!y) return fail(ARL2_E_INVALID_ARG, "y is NULL");
  const void* need[2] = {x, w_t};
  const char* names[2] = {"x", "w_t"};
  for (int i = 0; i < 2; ++i) {
    if (!need[i]) return fail(ARL2_E_INVALID_ARG, "%s is NULL", names[i]);
    if (!aligned16(need[i])) return fail(ARL2_E_INVALID_ARG, "%s is not 16-byte aligned", names[i]);
  }
  arl2::LinearArgs a;
  for (int p = 0; p < arl2::kLinearMaxParts; ++p) a.y.ptr[p] = nullptr;
  for (int p = 0; p < parts; ++p) {
    if (!y[p]) return fail(ARL2_E_INVALID_ARG, "y[%d] is NULL", p);
    if (!aligned16(y[p])) return fail(ARL2_E_INVALID_ARG, "y[%d] is not 16-byte aligned", p);
    a.y.ptr[p] = y[p];
  }
  a.y.parts = parts;
  a.x = x;
  a.wt = w_t;
  a.M = m;
  a.N = n;
  a.K = k;
  a.out_bf16 = y_dtype == ARL2_BF16;
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  hipError_t e = arl2::launch_linear(a, stream);
  if (e == hipSuccess && arl2host::debug_sync()) {
    e = hipStreamSynchronize(stream);
    if (e == hipSuccess) e = hipGetLastError();
  }
  if (e != hipSuccess) return fail(ARL2_E_HIP, "linear projection launch: %s", hipGetErrorString(e));
  return ARL2_OK;
}
