// Allocation-free clean pass (arl2_commit_frame_noalloc, include/arl2.h): the same kernels as a
// layer's arl2_commit_frame, with every buffer the layer would own (the maps' working layouts,
// the derived forms of S, the state write's per-chunk partial sums) carved out of one
// file-scope device array instead of a hipMalloc'd slab, and the state in a buffer the caller
// owns.  For callers that cannot allocate device memory.
//
// The array is a symbol of this code object: every GPU the library runs on holds its own copy
// until the process ends.  Its device address is looked up once per device with
// hipGetSymbolAddress (in host code the array's name is not a device address).  Every call on a
// device reuses that device's copy, so calls that overlap on one GPU (other streams, other
// threads) race on it.
#include <hip/hip_runtime.h>

#include <cmath>
#include <mutex>

#include "../../include/arl2.h"
#include "arl2_host_util.h"
#include "arl2_kernels.h"

namespace {

__device__ __align__(256) unsigned char scratch[ARL2_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};  // device address of `scratch` per device (null: not set up yet)

size_t align_up(size_t x) { return (x + 255) & ~size_t(255); }

// Once per device, with the device current: check that it is a gfx950 and look up the device
// address of its copy of `scratch`.
arl2_status scratch_for_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    int n = 0;
    if (hipGetDeviceCount(&n) != hipSuccess || n < 1) {
      (void)hipGetLastError();
      return arl2host::fail(ARL2_E_NO_DEVICE, "no HIP device");
    }
    return arl2host::fail(ARL2_E_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  }
  if (dev < 0 || dev >= kMaxDevices) return arl2host::fail(ARL2_E_UNSUPPORTED, "device index %d too large", dev);
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    int cur = 0;
    arl2_status st = arl2host::current_gfx950(&cur);
    if (st) return st;
    void* p = nullptr;
    if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess || !p) {
      (void)hipGetLastError();
      return arl2host::fail(ARL2_E_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    }
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return ARL2_OK;
}

arl2_status launched(hipError_t e, hipStream_t stream, const char* what) {
  if (e == hipSuccess && arl2host::debug_sync()) {
    e = hipStreamSynchronize(stream);
    if (e == hipSuccess) e = hipGetLastError();
  }
  return e == hipSuccess ? ARL2_OK : arl2host::fail(ARL2_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned_or_null(const void* p) { return !p || arl2host::aligned16(p); }

// Bytes of `scratch` one call uses (0 for a configuration the call rejects anyway).
size_t noalloc_scratch_bytes(const arl2_config* cfg) {
  if (!cfg || cfg->batch < 1 || cfg->heads < 1 || cfg->tokens_per_frame < 1 ||
      (cfg->head_dim != 16 && cfg->head_dim != 64 && cfg->head_dim != 128))
    return 0;
  const size_t H = (size_t)cfg->heads, BH = (size_t)cfg->batch * H, d = (size_t)cfg->head_dim;
  const size_t dp = (size_t)arl2::padded_dim(cfg->head_dim), chunks = (size_t)arl2::commit_chunks(cfg->tokens_per_frame);
  return align_up(H * dp * d * 2) + 3 * align_up(H * dp * dp * 2)  // pq; pkt, pvt, pqt
         + 2 * align_up(BH * dp * dp * 2)                            // -S hi / lo fragments
         + 2 * align_up(BH * dp * d * 2)                             // W^T hi / lo
         + align_up(BH * chunks * dp * dp * 4);                      // per-chunk partial sums
}

}  // namespace

extern "C" arl2_status arl2_commit_frame_noalloc(const arl2_config* cfg, const void* phi_q, const void* phi_k,
                                                 const void* phi_v, float* state, const void* q, const void* k,
                                                 const void* v, const float* beta, const float* alpha, void* out,
                                                 void* stream_) {
  using arl2host::fail;
  if (!cfg) return fail(ARL2_E_INVALID_ARG, "config is NULL");
  const arl2_config c = *cfg;
  arl2_status st;
  if ((st = arl2host::check_config(c))) return st;
  if (c.io_dtype != ARL2_BF16) return fail(ARL2_E_UNSUPPORTED, "the allocation-free clean pass takes bf16 inputs");
  if (c.access != ARL2_ACCESS_FRAME) return fail(ARL2_E_UNSUPPORTED, "the allocation-free clean pass is frame-level");
  const void* need[] = {phi_q, phi_k, phi_v, state, k, v, beta, alpha};
  const char* names[] = {"phi_q", "phi_k", "phi_v", "state", "k", "v", "beta", "alpha"};
  for (int i = 0; i < 8; ++i) {
    if (!need[i]) return fail(ARL2_E_INVALID_ARG, "%s is NULL", names[i]);
    if (!arl2host::aligned16(need[i])) return fail(ARL2_E_INVALID_ARG, "%s is not 16-byte aligned", names[i]);
  }
  if (out && !q) return fail(ARL2_E_INVALID_ARG, "q is NULL");
  if (!aligned_or_null(q) || !aligned_or_null(out)) return fail(ARL2_E_INVALID_ARG, "q or out is not 16-byte aligned");
  const size_t want = noalloc_scratch_bytes(&c);
  if (want > (size_t)ARL2_NOALLOC_SCRATCH_BYTES)
    return fail(ARL2_E_UNSUPPORTED, "the frame needs %zu bytes of scratch; the allocation-free clean pass has %zu",
                want, (size_t)ARL2_NOALLOC_SCRATCH_BYTES);
  void* base = nullptr;
  if ((st = scratch_for_current_device(&base))) return st;

  const int d = c.head_dim, dp = arl2::padded_dim(d), chunks = arl2::commit_chunks(c.tokens_per_frame);
  const size_t H = (size_t)c.heads, BH = (size_t)c.batch * H;
  char* p = static_cast<char*>(base);
  auto take = [&](size_t bytes) {
    void* r = p;
    p += align_up(bytes);
    return r;
  };
  void* pq = take(H * dp * d * 2);
  void* pkt = take(H * dp * dp * 2);
  void* pvt = take(H * dp * dp * 2);
  void* pqt = take(H * dp * dp * 2);
  void* sneg_hi = take(BH * dp * dp * 2);
  void* sneg_lo = take(BH * dp * dp * 2);
  void* wt_hi = take(BH * dp * d * 2);
  void* wt_lo = take(BH * dp * d * 2);
  float* partial = static_cast<float*>(take(BH * (size_t)chunks * dp * dp * 4));
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  const float scale = c.softmax_scale > 0.f ? c.softmax_scale : 1.f / std::sqrt((float)d);

  // 1. the maps' working layouts (every element written, padding included)
  arl2::PrepMapsArgs pm{phi_q, phi_k, phi_v, pq, pkt, pvt, pqt, c.heads};
  if ((st = launched(arl2::launch_prep_maps(d, pm, stream), stream, "map preparation launch"))) return st;
  // 2. the forms of S_{N-1} the clean pass reads (-S fragments, W^T), from the caller's state,
  //    which the reduce rewrites unchanged (alpha = 1, no partials)
  arl2::CommitReduceArgs r;
  r.s_prev = state;
  r.alpha = nullptr;
  r.partial = partial;
  r.chunks = 0;
  r.pq = pq;
  r.s_new = state;
  r.sneg_hi = sneg_hi;
  r.sneg_lo = sneg_lo;
  r.wt_hi = wt_hi;
  r.wt_lo = wt_lo;
  r.B = c.batch;
  r.H = c.heads;
  if ((st = launched(arl2::launch_commit_reduce(d, r, stream), stream, "state preparation launch"))) return st;
  // 3. the clean pass's output (if wanted) and the state write's per-chunk partial sums
  arl2::WritePartialArgs w;
  w.k = k;
  w.v = v;
  w.beta = beta;
  w.pkt = pkt;
  w.pvt = pvt;
  w.sneg_hi = sneg_hi;
  w.sneg_lo = sneg_lo;
  w.partial = partial;
  w.knorm_eps = c.knorm_eps > 0.f ? c.knorm_eps : 1e-6f;
  arl2::FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.wt_hi = wt_hi;
  a.wt_lo = wt_lo;
  a.out = out;
  a.B = c.batch;
  a.H = c.heads;
  a.T = c.tokens_per_frame;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.out_bf16 = c.out_dtype == ARL2_BF16;
  if ((st = launched(arl2::launch_fwd(d, a, &w, stream), stream, "clean pass and state write launch"))) return st;
  // 4. S_N = alpha S_{N-1} + sum of the partials, into the caller's state (in place)
  r.alpha = alpha;
  r.chunks = chunks;
  return launched(arl2::launch_commit_reduce(d, r, stream), stream, "state reduce kernel launch");
}
