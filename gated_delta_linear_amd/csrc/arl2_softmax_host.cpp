// Host runtime of the retained softmax layers: the C interface declared in
// include/arl2_softmax.h.  Frame N's passes attend over the cached clean K/V of frames
// 0..N-1 and their own k, v ("Attend Locally, Remember Linearly", gist.science technical
// summary, section 1: the cache grows by one block per generated frame): every pass copies
// its k, v into cache slot N and runs the pass kernel as plain attention over keys
// [0, (N + 1) T); the clean pass's k, v stay in slot N and the frame index advances.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>

#include "../../include/arl2_softmax.h"
#include "arl2_host_util.h"
#include "arl2_kernels.h"

using arl2host::aligned16;
using arl2host::debug_sync;
using arl2host::fail;

struct arl2_softmax_layer {
  arl2_softmax_config cfg;
  float scale_log2 = 0.f;
  void* slab = nullptr;  // the K cache, then the V cache, bf16 [B][max_frames * T][H][d] each
  size_t bytes = 0;
  void* kc = nullptr;
  void* vc = nullptr;
  int64_t frame = 0;
  bool poisoned = false;
  hipStream_t last_stream = nullptr;
  bool have_last_stream = false;
  hipEvent_t handoff = nullptr;
};

namespace {

arl2_status hip_fail(arl2_softmax_layer* L, hipError_t e, const char* what) {
  if (L) L->poisoned = true;
  return fail(ARL2_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

arl2_status use_stream(arl2_softmax_layer* L, hipStream_t stream) {
  if (L->have_last_stream && L->last_stream != stream) {
    hipError_t e = hipEventRecord(L->handoff, L->last_stream);
    if (e == hipSuccess) e = hipStreamWaitEvent(stream, L->handoff, 0);
    if (e != hipSuccess) return hip_fail(L, e, "stream handoff");
  }
  L->last_stream = stream;
  L->have_last_stream = true;
  return ARL2_OK;
}

arl2_status after_launch(arl2_softmax_layer* L, hipError_t e, hipStream_t stream, const char* what) {
  if (e != hipSuccess) return hip_fail(L, e, what);
  if (debug_sync()) {
    e = hipStreamSynchronize(stream);
    if (e == hipSuccess) e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(L, e, what);
  }
  return ARL2_OK;
}

arl2_status check_ptr(const void* p, const char* name) {
  if (!p) return fail(ARL2_E_INVALID_ARG, "%s is NULL", name);
  if (!aligned16(p)) return fail(ARL2_E_INVALID_ARG, "%s is not 16-byte aligned", name);
  return ARL2_OK;
}

// Checks shared by the pass and the commit; then k, v into slot N and, if out, the attention.
arl2_status run_pass(arl2_softmax_layer* L, const void* q, const void* k, const void* v, void* out,
                     void* stream_, const char* who) {
  if (!L) return fail(ARL2_E_INVALID_ARG, "%s: layer is NULL", who);
  if (L->poisoned) return fail(ARL2_E_PROTOCOL, "%s: layer is poisoned by an earlier failure; reset it", who);
  arl2_status st;
  if ((st = check_ptr(k, "k")) || (st = check_ptr(v, "v"))) return st;
  if (out && ((st = check_ptr(q, "q")) || (st = check_ptr(out, "out")))) return st;
  const arl2_softmax_config& c = L->cfg;
  if (L->frame >= c.max_frames)
    return fail(ARL2_E_PROTOCOL, "%s: the K/V cache is full (%d frames)", who, c.max_frames);
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  if ((st = use_stream(L, stream))) return st;
  const int64_t rows = (int64_t)c.max_frames * c.tokens_per_frame;
  arl2::KvAppendArgs ap{k, v, L->kc, L->vc, c.batch, c.heads, c.head_dim, c.tokens_per_frame,
                        L->frame * c.tokens_per_frame, rows};
  if ((st = after_launch(L, arl2::launch_kv_append(ap, stream), stream, "K/V cache append launch"))) return st;
  if (!out) return ARL2_OK;
  arl2::FwdArgs a;
  a.q = q;
  a.k = L->kc;
  a.v = L->vc;
  a.wt_hi = nullptr;
  a.wt_lo = nullptr;
  a.out = out;
  a.B = c.batch;
  a.H = c.heads;
  a.T = c.tokens_per_frame;
  a.scale_log2 = L->scale_log2;
  a.out_bf16 = c.out_dtype == ARL2_BF16;
  a.Tk = (int)((L->frame + 1) * c.tokens_per_frame);
  a.kv_rows = (int)rows;
  return after_launch(L, arl2::launch_fwd(c.head_dim, a, nullptr, stream), stream, "attention launch");
}

}  // namespace

extern "C" {

arl2_status arl2_softmax_layer_create(const arl2_softmax_config* cfg, void* stream_, arl2_softmax_layer** out_layer) {
  if (!out_layer) return fail(ARL2_E_INVALID_ARG, "out_layer is NULL");
  *out_layer = nullptr;
  if (!cfg) return fail(ARL2_E_INVALID_ARG, "config is NULL");
  const arl2_softmax_config c = *cfg;
  if (c.batch < 1 || c.heads < 1 || c.batch > 65535 || c.heads > 65535)
    return fail(ARL2_E_INVALID_ARG, "batch and heads must be in [1, 65535]");
  if (c.tokens_per_frame < 1 || c.tokens_per_frame > ARL2_MAX_TOKENS)
    return fail(ARL2_E_INVALID_ARG, "tokens_per_frame must be in [1, %d]", ARL2_MAX_TOKENS);
  if (c.max_frames < 1) return fail(ARL2_E_INVALID_ARG, "max_frames must be >= 1");
  if (c.head_dim != 16 && c.head_dim != 64 && c.head_dim != 128)
    return fail(ARL2_E_UNSUPPORTED, "head_dim %d not supported (16, 64, 128)", c.head_dim);
  if (c.out_dtype != ARL2_F32 && c.out_dtype != ARL2_BF16) return fail(ARL2_E_INVALID_ARG, "bad out_dtype");
  if (!(c.softmax_scale >= 0.f) || !std::isfinite(c.softmax_scale))
    return fail(ARL2_E_INVALID_ARG, "softmax_scale must be finite and >= 0");
  // the attention kernel addresses one stream's cache [rows][H][d] with 32-bit byte offsets
  const int64_t rows = (int64_t)c.max_frames * c.tokens_per_frame;
  if ((rows + 256) * c.heads * c.head_dim * 2 >= (int64_t(1) << 31))
    return fail(ARL2_E_UNSUPPORTED, "one stream's K/V cache (max_frames x T x H x d bf16) must stay below 2 GiB");
  if ((((int64_t)c.tokens_per_frame + 127) / 128) * c.batch * c.heads + 7 > (int64_t(1) << 24))
    return fail(ARL2_E_UNSUPPORTED, "B x H x T too large for one launch");

  int ndev = 0;
  hipError_t e = hipGetDeviceCount(&ndev);
  if (e != hipSuccess || ndev < 1) {
    (void)hipGetLastError();
    return fail(ARL2_E_NO_DEVICE, "no HIP device (%s)", hipGetErrorString(e));
  }
  int dev = 0;
  if ((e = hipGetDevice(&dev)) != hipSuccess) return fail(ARL2_E_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  hipDeviceProp_t prop;
  if ((e = hipGetDeviceProperties(&prop, dev)) != hipSuccess)
    return fail(ARL2_E_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(ARL2_E_UNSUPPORTED, "device %d is %s; this library is built for gfx950 only", dev, prop.gcnArchName);

  arl2_softmax_layer* L = new arl2_softmax_layer();
  L->cfg = c;
  const float scale = c.softmax_scale > 0.f ? c.softmax_scale : 1.f / std::sqrt((float)c.head_dim);
  L->scale_log2 = scale * 1.4426950408889634f;
  const size_t cache_bytes = (size_t)c.batch * rows * c.heads * c.head_dim * 2;
  L->bytes = 2 * cache_bytes;
  if ((e = hipMalloc(&L->slab, L->bytes)) != hipSuccess) {
    (void)hipGetLastError();
    const size_t want = L->bytes;
    delete L;
    return fail(ARL2_E_OUT_OF_MEMORY, "hipMalloc(%zu bytes): %s", want, hipGetErrorString(e));
  }
  L->kc = L->slab;
  L->vc = static_cast<char*>(L->slab) + cache_bytes;
  if ((e = hipEventCreateWithFlags(&L->handoff, hipEventDisableTiming)) != hipSuccess) {
    (void)hipFree(L->slab);
    delete L;
    return fail(ARL2_E_HIP, "hipEventCreate: %s", hipGetErrorString(e));
  }
  L->last_stream = static_cast<hipStream_t>(stream_);
  L->have_last_stream = true;
  *out_layer = L;
  return ARL2_OK;
}

arl2_status arl2_softmax_pass(arl2_softmax_layer* L, const void* q, const void* k, const void* v, void* out,
                              void* stream) {
  if (L && !out) return fail(ARL2_E_INVALID_ARG, "out is NULL");
  if (L && !q) return fail(ARL2_E_INVALID_ARG, "q is NULL");
  return run_pass(L, q, k, v, out, stream, "arl2_softmax_pass");
}

arl2_status arl2_softmax_commit(arl2_softmax_layer* L, const void* q, const void* k, const void* v, void* out,
                                void* stream) {
  arl2_status st = run_pass(L, q, k, v, out, stream, "arl2_softmax_commit");
  if (st) return st;
  L->frame += 1;
  return ARL2_OK;
}

arl2_status arl2_softmax_reset(arl2_softmax_layer* L) {
  if (!L) return fail(ARL2_E_INVALID_ARG, "layer is NULL");
  L->frame = 0;
  L->poisoned = false;
  return ARL2_OK;
}

arl2_status arl2_softmax_destroy(arl2_softmax_layer* L) {
  if (!L) return ARL2_OK;
  hipError_t e = hipSuccess;
  if (L->have_last_stream) e = hipStreamSynchronize(L->last_stream);
  hipError_t e2 = L->slab ? hipFree(L->slab) : hipSuccess;
  if (L->handoff) (void)hipEventDestroy(L->handoff);
  delete L;
  if (e != hipSuccess) return fail(ARL2_E_HIP, "destroy: synchronise: %s", hipGetErrorString(e));
  if (e2 != hipSuccess) return fail(ARL2_E_HIP, "destroy: hipFree: %s", hipGetErrorString(e2));
  return ARL2_OK;
}

int64_t arl2_softmax_frame_index(const arl2_softmax_layer* L) { return L ? L->frame : -1; }

size_t arl2_softmax_device_bytes(const arl2_softmax_layer* L) { return L ? L->bytes : 0; }

}  // extern "C"
