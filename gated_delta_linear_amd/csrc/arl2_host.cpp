// Host runtime of the ARL2 layer library: the C interface declared in include/arl2.h.
//
// It owns the protocol of "Attend Locally, Remember Linearly" (gist.science technical
// summary, section 2.2): passes of a frame only read the state, the clean pass writes it
// once, and every pass of frame N reads S_{N-1}.  S lives in one buffer that the write updates
// in place (every element of S_N is written by the thread that read the same element of
// S_{N-1}, after the pass kernels that read S's derived forms), so the device addresses every
// call uses are fixed: a captured graph of any number of frames replays the protocol.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>

#include "../../include/arl2.h"
#include "arl2_host_util.h"
#include "arl2_kernels.h"

namespace arl2host {

thread_local std::string g_last_error;

arl2_status fail(arl2_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool debug_sync() {
  static const bool on = [] {
    const char* e = std::getenv("ARL2_DEBUG_SYNC");
    return e && e[0] && e[0] != '0';
  }();
  return on;
}

const char* last_error() { return g_last_error.c_str(); }

arl2_status check_config(const arl2_config& c) {
  if (c.batch < 1 || c.heads < 1 || c.batch > 65535 || c.heads > 65535)
    return fail(ARL2_E_INVALID_ARG, "batch and heads must be in [1, 65535]");
  if (c.tokens_per_frame < 1 || c.tokens_per_frame > ARL2_MAX_TOKENS)
    return fail(ARL2_E_INVALID_ARG, "tokens_per_frame must be in [1, %d]", ARL2_MAX_TOKENS);
  if (c.head_dim != 16 && c.head_dim != 64 && c.head_dim != 128)
    return fail(ARL2_E_UNSUPPORTED, "head_dim %d not supported (16, 64, 128)", c.head_dim);
  if (c.io_dtype != ARL2_BF16 && c.io_dtype != ARL2_F32) return fail(ARL2_E_INVALID_ARG, "bad io_dtype");
  if (c.access != ARL2_ACCESS_FRAME && c.access != ARL2_ACCESS_TOKEN) return fail(ARL2_E_INVALID_ARG, "bad access");
  if (c.access == ARL2_ACCESS_TOKEN && c.head_dim == 16)
    return fail(ARL2_E_UNSUPPORTED, "token-level access supports head_dim 64 and 128");
  // token-level access addresses one stream's fp32 inter-frame reads [T][H][d] with 32-bit byte offsets
  if (c.access == ARL2_ACCESS_TOKEN && ((int64_t)c.tokens_per_frame + 64) * c.heads * c.head_dim * 4 >= (int64_t(1) << 31))
    return fail(ARL2_E_UNSUPPORTED, "token-level access: one stream's frame (T x H x d fp32) must stay below 2 GiB");
  if (c.out_dtype != ARL2_F32 && c.out_dtype != ARL2_BF16) return fail(ARL2_E_INVALID_ARG, "bad out_dtype");
  if (!(c.softmax_scale >= 0.f) || !std::isfinite(c.softmax_scale))
    return fail(ARL2_E_INVALID_ARG, "softmax_scale must be finite and >= 0");
  if (!(c.knorm_eps >= 0.f) || !std::isfinite(c.knorm_eps))
    return fail(ARL2_E_INVALID_ARG, "knorm_eps must be finite and >= 0");
  // the kernels address one stream's frame slice [T][H][d] with 32-bit byte offsets
  const int64_t slice_bytes = ((int64_t)c.tokens_per_frame + 256) * c.heads * c.head_dim * 2;
  if (slice_bytes >= (int64_t(1) << 31))
    return fail(ARL2_E_UNSUPPORTED, "one stream's frame (T x H x d bf16) must stay below 2 GiB");
  // the clean pass's launch runs ceil(T / 128) x B x H work-groups for the pass and as many for
  // the state write (each rounded up to 8) in one grid dimension
  const int64_t pass_wgs = 2 * ((((int64_t)c.tokens_per_frame + 127) / 128) * c.batch * c.heads + 7);
  if (pass_wgs > (int64_t(1) << 24))
    return fail(ARL2_E_UNSUPPORTED, "B x H x T too large for one launch (%lld work-groups)", (long long)pass_wgs);
  return ARL2_OK;
}

arl2_status current_gfx950(int* dev) {
  int ndev = 0;
  hipError_t e = hipGetDeviceCount(&ndev);
  if (e != hipSuccess || ndev < 1) {
    (void)hipGetLastError();
    return fail(ARL2_E_NO_DEVICE, "no HIP device (%s)", hipGetErrorString(e));
  }
  if ((e = hipGetDevice(dev)) != hipSuccess) return fail(ARL2_E_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  hipDeviceProp_t prop;
  if ((e = hipGetDeviceProperties(&prop, *dev)) != hipSuccess)
    return fail(ARL2_E_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(ARL2_E_UNSUPPORTED, "device %d is %s; this library is built for gfx950 only", *dev, prop.gcnArchName);
  return ARL2_OK;
}


}  // namespace arl2host

using arl2host::aligned16;
using arl2host::debug_sync;
using arl2host::fail;

struct arl2_layer {
  arl2_config cfg;
  int device = 0;
  int d = 0, dp = 0, chunks = 0;
  float scale_log2 = 0.f, eps = 0.f;
  // one device slab, carved into the regions below
  void* slab = nullptr;
  size_t bytes = 0;
  float* s = nullptr;                // S, fp32 [B][H][d][d], updated in place by the write
  float* partial = nullptr;          // [B][H][chunks][dp][dp]
  void* sneg_hi = nullptr;           // -S as B fragments, bf16 [B][H][dp/32][dp/16][64][8]
  void* sneg_lo = nullptr;
  void* wt_hi = nullptr;             // (phi_q S)^T, bf16 [B][H][d/16][dp][16] (k-step planes)
  void* wt_lo = nullptr;
  void* pq = nullptr;                // maps' working layouts, bf16 [H][dp][d]
  void* pkt = nullptr;
  void* pvt = nullptr;
  void* pqt = nullptr;               // phi_q^T, bf16 [H][dp][dp]
  void* seq_ws = nullptr;            // token-level access: chunk operands of the scan
  float* o_inter = nullptr;          // token-level access: inter-frame reads, fp32 [B][T][H][d]
  float* gate_beta = nullptr;        // beta from the gate projection, fp32 [B][T][H]
  float* gate_alpha = nullptr;       // alpha logit sums per 32-token block, fp32 [B][gate_blocks(T)][H]
  void* stage[3] = {nullptr, nullptr, nullptr};  // io_dtype F32: q, k, v rounded to bf16 [B][T][H][d]
  int64_t frame_elems = 0;                        // B T H d
  int n_ablk = 0;
  int64_t frame = 0;
  bool poisoned = false;
  hipStream_t last_stream = nullptr;
  bool have_last_stream = false;
  hipEvent_t handoff = nullptr;
};

namespace {

arl2_status hip_fail(arl2_layer* L, hipError_t e, const char* what) {
  if (L) L->poisoned = true;
  return fail(ARL2_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Make `stream` the layer's stream, ordering it after the previous one when it differs.
arl2_status use_stream(arl2_layer* L, hipStream_t stream) {
  if (L->have_last_stream && L->last_stream != stream) {
    hipError_t e = hipEventRecord(L->handoff, L->last_stream);
    if (e == hipSuccess) e = hipStreamWaitEvent(stream, L->handoff, 0);
    if (e != hipSuccess) return hip_fail(L, e, "stream handoff");
  }
  L->last_stream = stream;
  L->have_last_stream = true;
  return ARL2_OK;
}

arl2_status after_launch(arl2_layer* L, hipError_t e, hipStream_t stream, const char* what) {
  if (e != hipSuccess) return hip_fail(L, e, what);
  if (debug_sync()) {
    e = hipStreamSynchronize(stream);
    if (e == hipSuccess) e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(L, e, what);
  }
  return ARL2_OK;
}

arl2_status check_layer(arl2_layer* L) {
  if (!L) return fail(ARL2_E_INVALID_ARG, "layer is NULL");
  if (L->poisoned) return fail(ARL2_E_PROTOCOL, "layer is poisoned by an earlier failure; restore a state first");
  return ARL2_OK;
}

arl2_status check_access(arl2_layer* L, int access) {
  if (L->cfg.access == access) return ARL2_OK;
  return fail(ARL2_E_INVALID_ARG, access == ARL2_ACCESS_FRAME
                                      ? "the layer uses token-level access: call the *_seq entry points"
                                      : "the layer uses frame-level access: the *_seq entry points do not apply");
}

arl2_status check_ptr(const void* p, const char* name) {
  if (!p) return fail(ARL2_E_INVALID_ARG, "%s is NULL", name);
  if (!aligned16(p)) return fail(ARL2_E_INVALID_ARG, "%s is not 16-byte aligned", name);
  return ARL2_OK;
}

// The pass kernel's launch: the pass (when out is not null) and the state write's per-chunk
// partial sums (when w is not null).
arl2_status launch_pass(arl2_layer* L, const void* q, const void* k, const void* v, void* out,
                        const arl2::WritePartialArgs* w, hipStream_t stream) {
  arl2::FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.wt_hi = L->wt_hi;
  a.wt_lo = L->wt_lo;
  a.out = out;
  a.B = L->cfg.batch;
  a.H = L->cfg.heads;
  a.T = L->cfg.tokens_per_frame;
  a.scale_log2 = L->scale_log2;
  a.out_bf16 = L->cfg.out_dtype == ARL2_BF16;
  return after_launch(L, arl2::launch_fwd(L->d, a, w, stream), stream,
                      w ? "clean pass and state write launch" : "pass kernel launch");
}

// Derive S_N = alpha S_prev + partials (chunks may be 0) into the layer's S (s_prev may be S
// itself: the reduce updates it in place), plus its derived forms; alpha from the gate
// projection's partial sums when alpha_bias is not null.
arl2_status launch_reduce(arl2_layer* L, const float* s_prev, const float* alpha, int chunks, hipStream_t stream,
                          const float* alpha_bias = nullptr) {
  arl2::CommitReduceArgs r;
  r.s_prev = s_prev;
  r.alpha = alpha;
  if (alpha_bias) {
    r.alpha_part = L->gate_alpha;
    r.alpha_bias = alpha_bias;
    r.n_ablk = L->n_ablk;
    r.T = L->cfg.tokens_per_frame;
  }
  r.partial = L->partial;
  r.chunks = chunks;
  r.pq = L->pq;
  r.s_new = L->s;
  r.sneg_hi = L->sneg_hi;
  r.sneg_lo = L->sneg_lo;
  r.wt_hi = L->wt_hi;
  r.wt_lo = L->wt_lo;
  r.B = L->cfg.batch;
  r.H = L->cfg.heads;
  return after_launch(L, arl2::launch_commit_reduce(L->d, r, stream), stream, "state reduce kernel launch");
}

size_t align_up(size_t x) { return (x + 255) & ~size_t(255); }

// The clean pass's launch (output, if wanted, and the state write's per-chunk sums with beta),
// then the reduce with alpha, or with alpha from the gate projection when alpha_bias is given.
arl2_status commit(arl2_layer* L, const void* q, const void* k, const void* v, const float* beta,
                   const float* alpha, const float* alpha_bias, void* out, hipStream_t stream) {
  // One launch: the clean pass's output (when wanted) and the state write's per-chunk partial
  // sums, the latter in work-groups that the dispatcher places after the pass's, on the CUs
  // the pass leaves idle (as a second kernel, beside the pass on another stream or after it,
  // the write either took CUs the pass needed or added its whole time to the frame).  Then the
  // reduce, in stream order.
  arl2::WritePartialArgs w;
  w.k = k;
  w.v = v;
  w.beta = beta;
  w.pkt = L->pkt;
  w.pvt = L->pvt;
  w.sneg_hi = L->sneg_hi;
  w.sneg_lo = L->sneg_lo;
  w.partial = L->partial;
  w.knorm_eps = L->eps;
  arl2_status st;
  if ((st = launch_pass(L, q, k, v, out, &w, stream))) return st;
  if ((st = launch_reduce(L, L->s, alpha, L->chunks, stream, alpha_bias))) return st;
  L->frame += 1;
  return ARL2_OK;
}

// io_dtype F32: round the caller's fp32 q, k, v (those not null) to bf16 into the layer's staging
// copies and point the call at them; io_dtype BF16: nothing to do.
arl2_status stage_inputs(arl2_layer* L, const void*& q, const void*& k, const void*& v, hipStream_t stream) {
  if (L->cfg.io_dtype != ARL2_F32) return ARL2_OK;
  arl2::CvtJobs j{};
  int n = 0;
  const void** ptr[3] = {&q, &k, &v};
  for (int i = 0; i < 3; ++i) {
    if (!*ptr[i]) continue;
    j.src[n] = static_cast<const float*>(*ptr[i]);
    j.dst[n] = L->stage[i];
    *ptr[i] = L->stage[i];
    ++n;
  }
  if (n == 0) return ARL2_OK;
  return after_launch(L, arl2::launch_cvt_bf16(j, n, L->frame_elems, stream), stream, "fp32 input conversion launch");
}

}  // namespace

extern "C" {

const char* arl2_status_string(arl2_status st) {
  switch (st) {
    case ARL2_OK: return "ok";
    case ARL2_E_INVALID_ARG: return "invalid argument";
    case ARL2_E_UNSUPPORTED: return "unsupported configuration or device";
    case ARL2_E_NO_DEVICE: return "no HIP device";
    case ARL2_E_OUT_OF_MEMORY: return "out of device memory";
    case ARL2_E_HIP: return "HIP runtime error";
    case ARL2_E_PROTOCOL: return "protocol error (layer poisoned)";
  }
  return "unknown status";
}

const char* arl2_last_error(void) { return arl2host::last_error(); }

arl2_status arl2_layer_create(const arl2_config* cfg, const void* phi_q, const void* phi_k, const void* phi_v,
                              void* stream_, arl2_layer** out_layer) {
  if (!out_layer) return fail(ARL2_E_INVALID_ARG, "out_layer is NULL");
  *out_layer = nullptr;
  if (!cfg) return fail(ARL2_E_INVALID_ARG, "config is NULL");
  const arl2_config c = *cfg;
  arl2_status st;
  if ((st = arl2host::check_config(c))) return st;
  if ((st = check_ptr(phi_q, "phi_q")) || (st = check_ptr(phi_k, "phi_k")) || (st = check_ptr(phi_v, "phi_v")))
    return st;

  int dev = 0;
  if ((st = arl2host::current_gfx950(&dev))) return st;
  hipError_t e;

  arl2_layer* L = new arl2_layer();
  L->cfg = c;
  L->device = dev;
  L->d = c.head_dim;
  L->dp = arl2::padded_dim(c.head_dim);
  L->chunks = arl2::commit_chunks(c.tokens_per_frame);
  const float scale = c.softmax_scale > 0.f ? c.softmax_scale : 1.f / std::sqrt((float)c.head_dim);
  L->scale_log2 = scale * 1.4426950408889634f;
  L->eps = c.knorm_eps > 0.f ? c.knorm_eps : 1e-6f;

  const size_t BH = (size_t)c.batch * c.heads, d = L->d, dp = L->dp;
  const size_t s_bytes = align_up(BH * d * d * sizeof(float));
  const size_t part_bytes = align_up(BH * L->chunks * dp * dp * sizeof(float));
  const size_t frag_bytes = align_up(BH * dp * dp * 2);  // [B][H][dp/32][dp/16][64][8] bf16
  const size_t wt_bytes = align_up(BH * dp * d * 2);
  const size_t pq_bytes = align_up((size_t)c.heads * dp * d * 2);
  const size_t map_bytes = align_up((size_t)c.heads * dp * dp * 2);
  L->n_ablk = arl2::gate_blocks(c.tokens_per_frame);
  const size_t gbeta_bytes = align_up((size_t)c.batch * c.tokens_per_frame * c.heads * sizeof(float));
  const size_t galpha_bytes = align_up((size_t)c.batch * L->n_ablk * c.heads * sizeof(float));
  const bool seq = c.access == ARL2_ACCESS_TOKEN;
  const size_t seqws_bytes = seq ? align_up(arl2::seq_workspace_bytes(L->d, c.batch, c.heads, c.tokens_per_frame)) : 0;
  const size_t oint_bytes = seq ? align_up((size_t)c.batch * c.tokens_per_frame * c.heads * d * sizeof(float)) : 0;
  const bool f32 = c.io_dtype == ARL2_F32;
  L->frame_elems = (int64_t)c.batch * c.tokens_per_frame * c.heads * c.head_dim;
  const size_t stage_bytes = f32 ? align_up((size_t)L->frame_elems * 2) : 0;
  const size_t phi_stage_bytes = f32 ? align_up((size_t)c.heads * d * d * 2) : 0;
  L->bytes = s_bytes + part_bytes + 2 * frag_bytes + 2 * wt_bytes + gbeta_bytes + galpha_bytes + seqws_bytes +
             oint_bytes + 3 * stage_bytes + 3 * phi_stage_bytes + pq_bytes + 3 * map_bytes;
  if ((e = hipMalloc(&L->slab, L->bytes)) != hipSuccess) {
    (void)hipGetLastError();
    const size_t want = L->bytes;
    delete L;
    return fail(ARL2_E_OUT_OF_MEMORY, "hipMalloc(%zu bytes): %s", want, hipGetErrorString(e));
  }
  char* p = static_cast<char*>(L->slab);
  L->s = reinterpret_cast<float*>(p); p += s_bytes;
  L->partial = reinterpret_cast<float*>(p); p += part_bytes;
  L->sneg_hi = p; p += frag_bytes;
  L->sneg_lo = p; p += frag_bytes;
  L->wt_hi = p; p += wt_bytes;
  L->wt_lo = p; p += wt_bytes;
  L->gate_beta = reinterpret_cast<float*>(p); p += gbeta_bytes;
  L->gate_alpha = reinterpret_cast<float*>(p); p += galpha_bytes;
  if (seq) {
    L->seq_ws = p; p += seqws_bytes;
    L->o_inter = reinterpret_cast<float*>(p); p += oint_bytes;
  }
  void* phi_stage[3] = {nullptr, nullptr, nullptr};
  for (int i = 0; i < 3 && f32; ++i) {
    L->stage[i] = p; p += stage_bytes;
  }
  for (int i = 0; i < 3 && f32; ++i) {
    phi_stage[i] = p; p += phi_stage_bytes;
  }
  L->pq = p; p += pq_bytes;
  L->pkt = p; p += map_bytes;
  L->pvt = p; p += map_bytes;
  L->pqt = p; p += map_bytes;

  hipStream_t stream = static_cast<hipStream_t>(stream_);
  auto bail = [&](hipError_t err, const char* what) {
    (void)hipStreamSynchronize(stream);
    (void)hipFree(L->slab);
    if (L->handoff) (void)hipEventDestroy(L->handoff);
    delete L;
    return fail(ARL2_E_HIP, "%s: %s", what, hipGetErrorString(err));
  };
  if ((e = hipEventCreateWithFlags(&L->handoff, hipEventDisableTiming)) != hipSuccess) return bail(e, "hipEventCreate");
  // S_0 = 0 and everything derived from it is 0 as well.
  if ((e = hipMemsetAsync(L->slab, 0, L->bytes - pq_bytes - 3 * map_bytes, stream)) != hipSuccess)
    return bail(e, "hipMemsetAsync");
  if (f32) {  // the maps arrive in fp32: round them to bf16 first
    arl2::CvtJobs j{{static_cast<const float*>(phi_q), static_cast<const float*>(phi_k),
                     static_cast<const float*>(phi_v)},
                    {phi_stage[0], phi_stage[1], phi_stage[2]}};
    if ((e = arl2::launch_cvt_bf16(j, 3, (int64_t)c.heads * d * d, stream)) != hipSuccess)
      return bail(e, "fp32 map conversion launch");
    phi_q = phi_stage[0];
    phi_k = phi_stage[1];
    phi_v = phi_stage[2];
  }
  arl2::PrepMapsArgs pm{phi_q, phi_k, phi_v, L->pq, L->pkt, L->pvt, L->pqt, c.heads};
  if ((e = arl2::launch_prep_maps(L->d, pm, stream)) != hipSuccess) return bail(e, "map preparation launch");
  if (debug_sync() && (e = hipStreamSynchronize(stream)) != hipSuccess) return bail(e, "map preparation");
  L->last_stream = stream;
  L->have_last_stream = true;
  *out_layer = L;
  return ARL2_OK;
}

arl2_status arl2_denoise_step(arl2_layer* L, const void* q, const void* k, const void* v, void* out, void* stream_) {
  arl2_status st;
  if ((st = check_layer(L)) || (st = check_access(L, ARL2_ACCESS_FRAME))) return st;
  if ((st = check_ptr(q, "q")) || (st = check_ptr(k, "k")) || (st = check_ptr(v, "v")) || (st = check_ptr(out, "out")))
    return st;
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  if ((st = use_stream(L, stream)) || (st = stage_inputs(L, q, k, v, stream))) return st;
  return launch_pass(L, q, k, v, out, nullptr, stream);
}

// Token-level access: the chunked recurrence (inter-frame reads into o_inter, and S_N into the
// other state buffer when alpha is given), then, if out, the softmax branch plus o_inter.
static arl2_status seq_pass(arl2_layer* L, const void* q, const void* k, const void* v, const float* beta,
                            const float* alpha, void* out, hipStream_t stream) {
  arl2_status st;
  arl2::SeqArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.beta = beta;
  a.pqt = L->pqt;
  a.pkt = L->pkt;
  a.pvt = L->pvt;
  a.ws = L->seq_ws;
  a.s_prev = L->s;
  a.alpha = alpha;
  a.s_new = alpha ? L->s : nullptr;  // in place: each wave reads its columns of S first, writes them last
  a.o_inter = L->o_inter;
  a.B = L->cfg.batch;
  a.H = L->cfg.heads;
  a.T = L->cfg.tokens_per_frame;
  a.eps = L->eps;
  // (q is read by the recurrence for Q'; with no output the clean pass still needs it)
  if ((st = after_launch(L, arl2::launch_seq(L->d, a, stream), stream, "token-level recurrence launch"))) return st;
  if (!out) return ARL2_OK;
  arl2::FwdArgs f;
  f.q = q;
  f.k = k;
  f.v = v;
  f.wt_hi = nullptr;
  f.wt_lo = nullptr;
  f.out = out;
  f.B = L->cfg.batch;
  f.H = L->cfg.heads;
  f.T = L->cfg.tokens_per_frame;
  f.scale_log2 = L->scale_log2;
  f.out_bf16 = L->cfg.out_dtype == ARL2_BF16;
  f.Tk = f.T;
  f.kv_rows = f.T;
  f.add = L->o_inter;
  return after_launch(L, arl2::launch_fwd(L->d, f, nullptr, stream), stream, "pass kernel launch");
}

arl2_status arl2_denoise_step_seq(arl2_layer* L, const void* q, const void* k, const void* v, const float* beta,
                                  void* out, void* stream_) {
  arl2_status st;
  if ((st = check_layer(L)) || (st = check_access(L, ARL2_ACCESS_TOKEN))) return st;
  if ((st = check_ptr(q, "q")) || (st = check_ptr(k, "k")) || (st = check_ptr(v, "v")) ||
      (st = check_ptr(beta, "beta")) || (st = check_ptr(out, "out")))
    return st;
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  if ((st = use_stream(L, stream)) || (st = stage_inputs(L, q, k, v, stream))) return st;
  return seq_pass(L, q, k, v, beta, nullptr, out, stream);
}

arl2_status arl2_commit_frame_seq(arl2_layer* L, const void* q, const void* k, const void* v, const float* beta,
                                  const float* alpha, void* out, void* stream_) {
  arl2_status st;
  if ((st = check_layer(L)) || (st = check_access(L, ARL2_ACCESS_TOKEN))) return st;
  if ((st = check_ptr(q, "q")) || (st = check_ptr(k, "k")) || (st = check_ptr(v, "v")) ||
      (st = check_ptr(beta, "beta")) || (st = check_ptr(alpha, "alpha")))
    return st;
  if (out && !aligned16(out)) return fail(ARL2_E_INVALID_ARG, "out is not 16-byte aligned");
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  if ((st = use_stream(L, stream)) || (st = stage_inputs(L, q, k, v, stream))) return st;
  if ((st = seq_pass(L, q, k, v, beta, alpha, out, stream))) return st;
  // (the derived forms of S_N are only read by frame-level passes)
  L->frame += 1;
  return ARL2_OK;
}

arl2_status arl2_commit_frame(arl2_layer* L, const void* q, const void* k, const void* v, const float* beta,
                              const float* alpha, void* out, void* stream_) {
  arl2_status st;
  if ((st = check_layer(L)) || (st = check_access(L, ARL2_ACCESS_FRAME))) return st;
  if ((st = check_ptr(k, "k")) || (st = check_ptr(v, "v")) || (st = check_ptr(beta, "beta")) ||
      (st = check_ptr(alpha, "alpha")))
    return st;
  if (out && (st = check_ptr(q, "q"))) return st;
  if (out && !aligned16(out)) return fail(ARL2_E_INVALID_ARG, "out is not 16-byte aligned");
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  if (!out) q = nullptr;  // not read without an output
  if ((st = use_stream(L, stream)) || (st = stage_inputs(L, q, k, v, stream))) return st;
  return commit(L, q, k, v, beta, alpha, nullptr, out, stream);
}

arl2_status arl2_commit_frame_gated(arl2_layer* L, const void* q, const void* k, const void* v, const void* x,
                                    const void* w_gates, const float* b_gates, float beta_scale, void* out,
                                    void* stream_) {
  arl2_status st;
  if ((st = check_layer(L)) || (st = check_access(L, ARL2_ACCESS_FRAME))) return st;
  if ((st = check_ptr(k, "k")) || (st = check_ptr(v, "v")) || (st = check_ptr(x, "x")) ||
      (st = check_ptr(w_gates, "w_gates")))
    return st;
  if (!b_gates) return fail(ARL2_E_INVALID_ARG, "b_gates is NULL");
  if (!(beta_scale >= 0.f) || !std::isfinite(beta_scale))
    return fail(ARL2_E_INVALID_ARG, "beta_scale must be finite and >= 0");
  if (out && (st = check_ptr(q, "q"))) return st;
  if (out && !aligned16(out)) return fail(ARL2_E_INVALID_ARG, "out is not 16-byte aligned");
  // the gate kernel addresses the weights [2H][H d] with 32-bit byte offsets
  if ((int64_t)2 * L->cfg.heads * L->cfg.heads * L->d * 2 >= (int64_t(1) << 31))
    return fail(ARL2_E_UNSUPPORTED, "gate weights (2H x H d bf16) must stay below 2 GiB");
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  if (!out) q = nullptr;  // not read without an output
  if ((st = use_stream(L, stream)) || (st = stage_inputs(L, q, k, v, stream))) return st;
  arl2::GateArgs g{x, w_gates, b_gates, beta_scale, L->gate_beta, L->gate_alpha,
                   L->cfg.batch, L->cfg.heads, L->d, L->cfg.tokens_per_frame};
  if ((st = after_launch(L, arl2::launch_gates(g, stream), stream, "gate projection launch"))) return st;
  return commit(L, q, k, v, L->gate_beta, nullptr, b_gates + L->cfg.heads, out, stream);
}

arl2_status arl2_destroy(arl2_layer* L) {
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

arl2_status arl2_state_read(arl2_layer* L, float* dst, void* stream_) {
  arl2_status st;
  if ((st = check_layer(L))) return st;
  if ((st = check_ptr(dst, "dst"))) return st;
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  if ((st = use_stream(L, stream))) return st;
  const size_t n = (size_t)L->cfg.batch * L->cfg.heads * L->d * L->d * sizeof(float);
  hipError_t e = hipMemcpyAsync(dst, L->s, n, hipMemcpyDeviceToDevice, stream);
  return after_launch(L, e, stream, "state read copy");
}

arl2_status arl2_state_write(arl2_layer* L, const float* src, int64_t frame_index, void* stream_) {
  if (!L) return fail(ARL2_E_INVALID_ARG, "layer is NULL");
  arl2_status st;
  if ((st = check_ptr(src, "src"))) return st;
  if (frame_index < 0) return fail(ARL2_E_INVALID_ARG, "frame_index must be >= 0");
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  L->poisoned = false;
  if ((st = use_stream(L, stream))) return st;
  // S = 1 * src with no partials, and the derived forms the next passes read.
  if ((st = launch_reduce(L, src, nullptr, 0, stream))) {
    L->poisoned = true;
    return st;
  }
  L->frame = frame_index;
  return ARL2_OK;
}

int64_t arl2_frame_index(const arl2_layer* L) { return L ? L->frame : -1; }

size_t arl2_device_bytes(const arl2_layer* L) { return L ? L->bytes : 0; }

}  // extern "C"
