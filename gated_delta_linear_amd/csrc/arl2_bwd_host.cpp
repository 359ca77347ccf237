// Host runtime of the ARL2 layer's backward: the C interface declared in include/arl2_bwd.h.
//
// The object walks the frames of a stream in reverse ("Attend Locally, Remember Linearly",
// gist.science technical summary, sections 2.1-2.3: the forward reads S_{N-1} in every pass and
// writes S_N once per frame, so dL/dS flows from frame N back to frame N-1 through the write and
// through every pass's read).  It holds dL/dS of the frame it stands at (double-buffered: a
// commit reads one buffer and fills the other), the frame's sum of the passes' Q^T dO, and the
// dphi sums; per call it recomputes what the backward needs from the forward's inputs.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>

#include "../../include/arl2_bwd.h"
#include "arl2_host_util.h"
#include "arl2_kernels.h"

using arl2host::aligned16;
using arl2host::debug_sync;
using arl2host::fail;

struct arl2_bwd {
  arl2_config cfg;
  int d = 0, nch = 0;
  float scale = 0.f, scale_log2 = 0.f, eps = 0.f;
  void* slab = nullptr;
  size_t bytes = 0;
  float* o_sm = nullptr;       // recomputed softmax-branch output of a pass, fp32 [B][T][H][d]
  float* lse = nullptr;        // its rows' log-sum-exp, [B][H][T]
  float* dvec = nullptr;       // dO . O per row, [B][H][T]
  float* dq_read = nullptr;    // a pass's inter-frame read part of dq, [B][T][H][d]
  void* do_h = nullptr;        // d_out in fp16
  void* v16 = nullptr;         // the pass's v in fp16, [B][T][H][d]; k^T, q^T, dO^T in fp16, [B][H][d][tp]
  void* kt16 = nullptr;
  void* qt16 = nullptr;
  void* dot16 = nullptr;
  float* ds[2] = {nullptr, nullptr};  // dL/dS, [B][H][d][d], ping-pong
  int cur = 0;
  float* gr = nullptr;         // sum over the frame's passes of Q^T dO
  bool gr_valid = false;
  float* read_part = nullptr;  // [B][H][nch][d][d]
  float* write_part = nullptr; // [B][H][nch][3][d][d]
  void* mf[8] = {};            // S, S^T, G, G^T (hi, lo) fragments, [B][H][d][d] bf16 each
  void* phi_q = nullptr;       // bf16 [H][d][d]
  void* phif[5] = {};          // phi_k, phi_v, phi_k^T, phi_v^T, phi_q^T fragments, [H][d][d] bf16
  float* dphi[3] = {};         // dphi_q, dphi_k, dphi_v, fp32 [H][d][d]
  bool poisoned = false;
  hipStream_t last_stream = nullptr;
  bool have_last_stream = false;
  hipEvent_t handoff = nullptr;
  // A second stream of the object's own (default priority, not blocking with the null stream):
  // a pass's inter-frame read runs there, beside the softmax recompute on the caller's stream,
  // on the CUs that one leaves idle.  Forked from and joined back into the caller's stream
  // within each call.
  hipStream_t side = nullptr;
  hipEvent_t ev_fork = nullptr, ev_join = nullptr;
};

namespace {

size_t align_up(size_t x) { return (x + 255) & ~size_t(255); }

void release_sync_objects(arl2_bwd* g) {
  if (g->side) (void)hipStreamDestroy(g->side);
  for (hipEvent_t ev : {g->handoff, g->ev_fork, g->ev_join})
    if (ev) (void)hipEventDestroy(ev);
  g->side = nullptr;
  g->handoff = g->ev_fork = g->ev_join = nullptr;
}

// `waiter` waits for what `signaller` has enqueued so far
hipError_t order_after(hipEvent_t ev, hipStream_t signaller, hipStream_t waiter) {
  hipError_t e = hipEventRecord(ev, signaller);
  if (e == hipSuccess) e = hipStreamWaitEvent(waiter, ev, 0);
  return e;
}

arl2_status hip_fail(arl2_bwd* g, hipError_t e, const char* what) {
  if (g) g->poisoned = true;
  return fail(ARL2_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

arl2_status after_launch(arl2_bwd* g, hipError_t e, hipStream_t stream, const char* what) {
  if (e != hipSuccess) return hip_fail(g, e, what);
  if (debug_sync()) {
    e = hipStreamSynchronize(stream);
    if (e == hipSuccess) e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(g, e, what);
  }
  return ARL2_OK;
}

arl2_status use_stream(arl2_bwd* g, hipStream_t stream) {
  if (g->have_last_stream && g->last_stream != stream) {
    hipError_t e = hipEventRecord(g->handoff, g->last_stream);
    if (e == hipSuccess) e = hipStreamWaitEvent(stream, g->handoff, 0);
    if (e != hipSuccess) return hip_fail(g, e, "stream handoff");
  }
  g->last_stream = stream;
  g->have_last_stream = true;
  return ARL2_OK;
}

arl2_status check_obj(arl2_bwd* g) {
  if (!g) return fail(ARL2_E_INVALID_ARG, "backward object is NULL");
  if (g->poisoned) return fail(ARL2_E_PROTOCOL, "backward object is poisoned by an earlier failure; call arl2_bwd_begin");
  return ARL2_OK;
}

arl2_status check_ptr(const void* p, const char* name, bool need16 = true) {
  if (!p) return fail(ARL2_E_INVALID_ARG, "%s is NULL", name);
  if (need16 && !aligned16(p)) return fail(ARL2_E_INVALID_ARG, "%s is not 16-byte aligned", name);
  if (!need16 && (reinterpret_cast<uintptr_t>(p) & 3u)) return fail(ARL2_E_INVALID_ARG, "%s is not 4-byte aligned", name);
  return ARL2_OK;
}

size_t bh_dd(const arl2_bwd* g) { return (size_t)g->cfg.batch * g->cfg.heads * g->d * g->d; }

// Fragment-order copies of S_{N-1} (and S^T), and of G = dL/dS_N (and G^T) when with_g.
arl2_status frags(arl2_bwd* g, const float* s_prev, bool with_g, hipStream_t stream) {
  arl2::BwdFragJobs j{};
  j.job[0] = {s_prev, g->mf[0], g->mf[1], 0};
  j.job[1] = {s_prev, g->mf[2], g->mf[3], 1};
  j.job[2] = {g->ds[g->cur], g->mf[4], g->mf[5], 0};
  j.job[3] = {g->ds[g->cur], g->mf[6], g->mf[7], 1};
  return after_launch(g, arl2::launch_bwd_frags(g->d, j, g->cfg.batch * g->cfg.heads, with_g ? 4 : 2, stream), stream,
                      "fragment copies");
}

arl2::BwdTokArgs tok_args(arl2_bwd* g) {
  arl2::BwdTokArgs t{};
  t.s_hi = g->mf[0];
  t.s_lo = g->mf[1];
  t.st_hi = g->mf[2];
  t.st_lo = g->mf[3];
  t.g_hi = g->mf[4];
  t.g_lo = g->mf[5];
  t.gt_hi = g->mf[6];
  t.gt_lo = g->mf[7];
  t.phik = g->phif[0];
  t.phiv = g->phif[1];
  t.phikt = g->phif[2];
  t.phivt = g->phif[3];
  t.pqt = g->phif[4];
  t.B = g->cfg.batch;
  t.H = g->cfg.heads;
  t.T = g->cfg.tokens_per_frame;
  t.knorm_eps = g->eps;
  return t;
}

}  // namespace

extern "C" {

arl2_status arl2_bwd_create(const arl2_config* cfg, const void* phi_q, const void* phi_k, const void* phi_v,
                            void* stream_, arl2_bwd** out) {
  if (!out) return fail(ARL2_E_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (!cfg) return fail(ARL2_E_INVALID_ARG, "cfg is NULL");
  const arl2_config c = *cfg;
  if (c.batch < 1 || c.batch > 65535 || c.heads < 1 || c.heads > 65535)
    return fail(ARL2_E_INVALID_ARG, "batch and heads must be in [1, 65535]");
  if (c.tokens_per_frame < 1 || c.tokens_per_frame > ARL2_MAX_TOKENS)
    return fail(ARL2_E_INVALID_ARG, "tokens_per_frame must be in [1, %d]", ARL2_MAX_TOKENS);
  if (c.head_dim != 64 && c.head_dim != 128) return fail(ARL2_E_UNSUPPORTED, "the backward supports head_dim 64 and 128");
  if (c.io_dtype != ARL2_BF16) return fail(ARL2_E_UNSUPPORTED, "io_dtype must be ARL2_BF16");
  if (c.access != ARL2_ACCESS_FRAME) return fail(ARL2_E_UNSUPPORTED, "the backward covers frame-level access");
  if (!(c.softmax_scale >= 0.f) || !std::isfinite(c.softmax_scale))
    return fail(ARL2_E_INVALID_ARG, "softmax_scale must be finite and >= 0");
  if (!(c.knorm_eps >= 0.f) || !std::isfinite(c.knorm_eps))
    return fail(ARL2_E_INVALID_ARG, "knorm_eps must be finite and >= 0");
  const int64_t slice_bytes = ((int64_t)c.tokens_per_frame + 256) * c.heads * c.head_dim * 4;
  if (slice_bytes >= (int64_t(1) << 31))
    return fail(ARL2_E_UNSUPPORTED, "one stream's frame (T x H x d fp32) must stay below 2 GiB");
  if ((int64_t)arl2::bwd_chunks(c.tokens_per_frame) * c.batch * c.heads >= (int64_t(1) << 31))
    return fail(ARL2_E_UNSUPPORTED, "B x H x T too large for one launch");
  arl2_status st;
  if ((st = check_ptr(phi_q, "phi_q")) || (st = check_ptr(phi_k, "phi_k")) || (st = check_ptr(phi_v, "phi_v")))
    return st;
  int ndev = 0;
  hipError_t e = hipGetDeviceCount(&ndev);
  if (e != hipSuccess || ndev < 1) {
    (void)hipGetLastError();
    return fail(ARL2_E_NO_DEVICE, "no HIP device (%s)", hipGetErrorString(e));
  }
  int dev = 0;
  hipDeviceProp_t prop;
  if ((e = hipGetDevice(&dev)) != hipSuccess || (e = hipGetDeviceProperties(&prop, dev)) != hipSuccess)
    return fail(ARL2_E_HIP, "device query: %s", hipGetErrorString(e));
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(ARL2_E_UNSUPPORTED, "device %d is %s; this library is built for gfx950 only", dev, prop.gcnArchName);

  arl2_bwd* g = new arl2_bwd();
  g->cfg = c;
  g->d = c.head_dim;
  g->nch = arl2::bwd_chunks(c.tokens_per_frame);
  g->scale = c.softmax_scale > 0.f ? c.softmax_scale : 1.f / std::sqrt((float)c.head_dim);
  g->scale_log2 = g->scale * 1.4426950408889634f;
  g->eps = c.knorm_eps > 0.f ? c.knorm_eps : 1e-6f;
  const size_t B = c.batch, H = c.heads, T = c.tokens_per_frame, d = g->d, BH = B * H;
  const size_t tok_f32 = align_up(B * T * H * d * 4), tok_bf = align_up(B * T * H * d * 2);
  const size_t row_f32 = align_up(BH * T * 4), mat = align_up(BH * d * d * 4), matbf = align_up(BH * d * d * 2);
  const size_t hmat = align_up(H * d * d * 4), hmatbf = align_up(H * d * d * 2);
  const size_t rpart = align_up(BH * g->nch * d * d * 4), wpart = align_up(BH * g->nch * 3 * d * d * 4);
  const size_t kt_bf = align_up(BH * d * (size_t)arl2::bwd_key_pitch(c.tokens_per_frame) * 2);
  g->bytes = 2 * tok_f32 + 2 * row_f32 + 2 * tok_bf + 3 * kt_bf + 3 * mat + rpart + wpart + 8 * matbf + 6 * hmatbf + 3 * hmat;
  if ((e = hipMalloc(&g->slab, g->bytes)) != hipSuccess) {
    (void)hipGetLastError();
    const size_t want = g->bytes;
    delete g;
    return fail(ARL2_E_OUT_OF_MEMORY, "hipMalloc(%zu bytes): %s", want, hipGetErrorString(e));
  }
  char* p = static_cast<char*>(g->slab);
  g->o_sm = reinterpret_cast<float*>(p); p += tok_f32;
  g->dq_read = reinterpret_cast<float*>(p); p += tok_f32;
  g->lse = reinterpret_cast<float*>(p); p += row_f32;
  g->dvec = reinterpret_cast<float*>(p); p += row_f32;
  g->do_h = p; p += tok_bf;
  g->v16 = p; p += tok_bf;
  g->kt16 = p; p += kt_bf;
  g->qt16 = p; p += kt_bf;
  g->dot16 = p; p += kt_bf;
  g->ds[0] = reinterpret_cast<float*>(p); p += mat;
  g->ds[1] = reinterpret_cast<float*>(p); p += mat;
  g->gr = reinterpret_cast<float*>(p); p += mat;
  g->read_part = reinterpret_cast<float*>(p); p += rpart;
  g->write_part = reinterpret_cast<float*>(p); p += wpart;
  for (auto& m : g->mf) { m = p; p += matbf; }
  g->phi_q = p; p += hmatbf;
  for (auto& m : g->phif) { m = p; p += hmatbf; }
  for (auto& m : g->dphi) { m = reinterpret_cast<float*>(p); p += hmat; }

  hipStream_t stream = static_cast<hipStream_t>(stream_);
  auto bail = [&](hipError_t err, const char* what) {
    (void)hipStreamSynchronize(stream);
    if (g->side) (void)hipStreamSynchronize(g->side);
    (void)hipFree(g->slab);
    release_sync_objects(g);
    delete g;
    return fail(ARL2_E_HIP, "%s: %s", what, hipGetErrorString(err));
  };
  for (hipEvent_t* ev : {&g->handoff, &g->ev_fork, &g->ev_join})
    if ((e = hipEventCreateWithFlags(ev, hipEventDisableTiming)) != hipSuccess) return bail(e, "hipEventCreate");
  if ((e = hipStreamCreateWithFlags(&g->side, hipStreamNonBlocking)) != hipSuccess) return bail(e, "hipStreamCreate");
  if ((e = hipMemcpyAsync(g->phi_q, phi_q, H * d * d * 2, hipMemcpyDeviceToDevice, stream)) != hipSuccess)
    return bail(e, "phi_q copy");
  const void* src[5] = {phi_k, phi_v, phi_k, phi_v, phi_q};
  for (int i = 0; i < 5; ++i)
    if ((e = arl2::launch_bwd_phi_frags(g->d, src[i], g->phif[i], c.heads, i >= 2, stream)) != hipSuccess)
      return bail(e, "map fragments");
  g->last_stream = stream;
  g->have_last_stream = true;
  if ((st = arl2_bwd_begin(g, nullptr, stream_)) != ARL2_OK) {
    (void)hipStreamSynchronize(stream);
    (void)hipFree(g->slab);
    release_sync_objects(g);
    delete g;
    return st;
  }
  *out = g;
  return ARL2_OK;
}

arl2_status arl2_bwd_begin(arl2_bwd* g, const float* ds_last, void* stream_) {
  if (!g) return fail(ARL2_E_INVALID_ARG, "backward object is NULL");
  if (ds_last && !aligned16(ds_last)) return fail(ARL2_E_INVALID_ARG, "ds_last is not 16-byte aligned");
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  g->poisoned = false;
  arl2_status st;
  if ((st = use_stream(g, stream))) return st;
  g->cur = 0;
  g->gr_valid = false;
  if ((st = after_launch(g, arl2::launch_bwd_fill(g->ds[0], ds_last, bh_dd(g), stream), stream, "dS init"))) return st;
  const size_t hdd = (size_t)g->cfg.heads * g->d * g->d;
  for (float* m : g->dphi)
    if ((st = after_launch(g, arl2::launch_bwd_fill(m, nullptr, hdd, stream), stream, "dphi init"))) return st;
  return ARL2_OK;
}

arl2_status arl2_bwd_pass(arl2_bwd* g, const void* q, const void* k, const void* v, const float* s_prev,
                          const float* d_out, float* dq, float* dk, float* dv, void* stream_) {
  arl2_status st;
  if ((st = check_obj(g))) return st;
  if ((st = check_ptr(q, "q")) || (st = check_ptr(k, "k")) || (st = check_ptr(v, "v")) ||
      (st = check_ptr(s_prev, "s_prev")) || (st = check_ptr(d_out, "d_out")) || (st = check_ptr(dq, "dq")) ||
      (st = check_ptr(dk, "dk")) || (st = check_ptr(dv, "dv")))
    return st;
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  if ((st = use_stream(g, stream))) return st;
  // the softmax branch's output and log-sum-exp, recomputed with the pass kernel
  arl2::FwdArgs f;
  f.q = q;
  f.k = k;
  f.v = v;
  f.wt_hi = f.wt_lo = nullptr;
  f.out = g->o_sm;
  f.B = g->cfg.batch;
  f.H = g->cfg.heads;
  f.T = g->cfg.tokens_per_frame;
  f.scale_log2 = g->scale_log2;
  f.out_bf16 = false;
  f.Tk = f.T;
  f.kv_rows = f.T;
  f.lse = g->lse;
  arl2::BwdPassArgs a;
  a.tok = tok_args(g);
  a.tok.q = q;
  a.tok.k = k;
  a.tok.v = v;
  a.tok.d_out = d_out;
  a.tok.dq = dq;
  a.tok.dk = dk;
  a.tok.dv = dv;
  a.tok.part = g->read_part;
  a.d_out = d_out;
  a.o_sm = g->o_sm;
  a.lse = g->lse;
  a.do_h = g->do_h;
  a.v16 = g->v16;
  a.kt16 = g->kt16;
  a.qt16 = g->qt16;
  a.dot16 = g->dot16;
  a.tp = arl2::bwd_key_pitch(g->cfg.tokens_per_frame);
  a.dvec = g->dvec;
  a.gr = g->gr;
  a.gr_first = !g->gr_valid;
  a.B = g->cfg.batch;
  a.H = g->cfg.heads;
  a.T = g->cfg.tokens_per_frame;
  a.scale = g->scale;
  a.scale_log2 = g->scale_log2;
  a.dq_read = g->dq_read;
  // Caller's stream: recompute | prep | dK, dV, dQ | (join) gr sums, dq += read's part
  // side stream:     (fork) S fragments | read (dq_read, chunk partials of Q^T dO) |
  // Only the read takes the S fragments, so they stay off the caller's stream; the fragment
  // buffers are next written by a later call's work, which the join or the next fork orders
  // after the read.  Each wait is enqueued after the record it waits for.
  using arl2::BwdStage;
  hipError_t e;
  if ((e = order_after(g->ev_fork, stream, g->side)) != hipSuccess) return hip_fail(g, e, "stream fork");
  if ((st = frags(g, s_prev, false, g->side))) return st;
  if ((st = after_launch(g, arl2::launch_bwd_stage(g->d, BwdStage::kRead, a, g->side), g->side, "inter-frame read backward")))
    return st;
  if ((st = after_launch(g, arl2::launch_fwd(g->d, f, nullptr, stream), stream, "softmax recompute"))) return st;
  if ((st = after_launch(g, arl2::launch_bwd_stage(g->d, BwdStage::kPrep, a, stream), stream, "attention backward prep")))
    return st;
  if ((st = after_launch(g, arl2::launch_bwd_stage(g->d, BwdStage::kAttn, a, stream), stream, "attention backward")))
    return st;
  if ((e = order_after(g->ev_join, g->side, stream)) != hipSuccess) return hip_fail(g, e, "stream join");
  if ((st = after_launch(g, arl2::launch_bwd_stage(g->d, BwdStage::kFinish, a, stream), stream, "pass backward sums")))
    return st;
  g->gr_valid = true;
  return ARL2_OK;
}

arl2_status arl2_bwd_commit(arl2_bwd* g, const void* k, const void* v, const float* beta, const float* alpha,
                            const float* s_prev, float* dk, float* dv, float* dbeta, float* dalpha, void* stream_) {
  arl2_status st;
  if ((st = check_obj(g))) return st;
  if ((st = check_ptr(k, "k")) || (st = check_ptr(v, "v")) || (st = check_ptr(beta, "beta", false)) ||
      (st = check_ptr(alpha, "alpha", false)) || (st = check_ptr(s_prev, "s_prev")) || (st = check_ptr(dk, "dk")) ||
      (st = check_ptr(dv, "dv")) || (st = check_ptr(dbeta, "dbeta", false)) || (st = check_ptr(dalpha, "dalpha", false)))
    return st;
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  if ((st = use_stream(g, stream))) return st;
  if ((st = frags(g, s_prev, true, stream))) return st;
  arl2::BwdTokArgs t = tok_args(g);
  t.k = k;
  t.v = v;
  t.beta = beta;
  t.dk = dk;
  t.dv = dv;
  t.dbeta = dbeta;
  t.part = g->write_part;
  arl2::BwdFrameArgs f;
  f.g = g->ds[g->cur];
  f.s_prev = s_prev;
  f.alpha = alpha;
  f.gr = g->gr_valid ? g->gr : nullptr;
  f.part = g->write_part;
  f.phi_q = g->phi_q;
  f.ds_prev = g->ds[g->cur ^ 1];
  f.dalpha = dalpha;
  f.dphi_q = g->dphi[0];
  f.dphi_k = g->dphi[1];
  f.dphi_v = g->dphi[2];
  f.B = g->cfg.batch;
  f.H = g->cfg.heads;
  f.chunks = g->nch;
  if ((st = after_launch(g, arl2::launch_bwd_commit(g->d, t, f, stream), stream, "state write backward"))) return st;
  g->cur ^= 1;
  g->gr_valid = false;
  return ARL2_OK;
}

arl2_status arl2_bwd_read(arl2_bwd* g, float* ds, float* dphi_q, float* dphi_k, float* dphi_v, void* stream_) {
  arl2_status st;
  if ((st = check_obj(g))) return st;
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  if ((st = use_stream(g, stream))) return st;
  const size_t hdd = (size_t)g->cfg.heads * g->d * g->d * 4;
  struct {
    void* dst;
    const void* src;
    size_t n;
  } cp[4] = {{ds, g->ds[g->cur], bh_dd(g) * 4}, {dphi_q, g->dphi[0], hdd}, {dphi_k, g->dphi[1], hdd}, {dphi_v, g->dphi[2], hdd}};
  for (auto& c : cp) {
    if (!c.dst) continue;
    const hipError_t e = hipMemcpyAsync(c.dst, c.src, c.n, hipMemcpyDefault, stream);
    if (e != hipSuccess) return hip_fail(g, e, "gradient copy");
  }
  return ARL2_OK;
}

arl2_status arl2_bwd_destroy(arl2_bwd* g) {
  if (!g) return ARL2_OK;
  hipError_t e = g->have_last_stream ? hipStreamSynchronize(g->last_stream) : hipSuccess;
  if (e == hipSuccess && g->side) e = hipStreamSynchronize(g->side);
  const hipError_t e2 = hipFree(g->slab);
  release_sync_objects(g);
  delete g;
  if (e == hipSuccess) e = e2;
  return e == hipSuccess ? ARL2_OK : fail(ARL2_E_HIP, "destroy: %s", hipGetErrorString(e));
}

size_t arl2_bwd_device_bytes(const arl2_bwd* g) { return g ? g->bytes : 0; }

}  // extern "C"
