/*
 * arl2_bwd.h - C interface of the ARL2 layer's backward, for AMD Instinct MI355X (gfx950), in
 * the same library as arl2.h.
 *
 * Source: "Attend Locally, Remember Linearly: Linear Attention as Cross-Frame Memory for
 * Autoregressive Video Diffusion" - the technical summary on gist.science: sections 2.1 and 2.2
 * define the layer's forward (arl2.h); section 2.3 converts a pretrained model by distillation,
 * the second stage fine-tuning the whole hybrid model end to end, through every replaced layer,
 * with the per-head maps (and gates) as the trainable parameters.  The gradients here are the
 * chain rule of that forward; the pages print no backward.
 *
 * Forward whose gradients are taken (per stream b, head h, frame N; arl2.h's conventions):
 *   pass p:   out_p = softmax(Q_p K_p^T * scale) V_p + (Q_p phi_q) S_{N-1}
 *   commit:   S_N = alpha S_{N-1} + K'^T diag(beta) (V' - K' S_{N-1}),
 *             K' = rows of K phi_k / max(norm, knorm_eps), V' = V phi_v   (K, V of the clean pass)
 * The backward sweeps the frames in reverse.  For each frame N = F-1 .. 0: any number of
 * arl2_bwd_pass calls (one per pass whose output enters the loss, with that output's gradient),
 * then one arl2_bwd_commit (the frame's state write).  The object carries dL/dS across frames
 * and accumulates dL/dphi_q, dL/dphi_k, dL/dphi_v; arl2_bwd_read copies them and dL/dS_0 out.
 * The caller keeps the forward's S_{N-1} of every frame (arl2_state_read after frame N-1's
 * commit), and alpha, beta as given to the forward: their gradients are returned as such (gate
 * projections that produce them are the caller's).
 *
 * Tensors (device memory, contiguous, row-major, 16-byte aligned unless noted, owned by the
 * caller and valid until the enqueued work has finished):
 *   q, k, v           bf16 [B][T][H][d]   inputs of the pass (of the clean pass for commit)
 *   d_out             fp32 [B][T][H][d]   dL/d out of the pass
 *   s_prev            fp32 [B][H][d][d]   S_{N-1} (row = key feature, column = value feature)
 *   beta, alpha       fp32 [B][T][H], [B][H]  (4-byte aligned)
 *   dq, dk, dv        fp32 [B][T][H][d]   arl2_bwd_pass writes them; arl2_bwd_commit adds the
 *                                         state write's share to dk, dv (pass the clean pass's
 *                                         buffers after its arl2_bwd_pass, or zeroed buffers)
 *   dbeta, dalpha     fp32 [B][T][H], [B][H] (4-byte aligned), written by arl2_bwd_commit
 *   ds_last, ds0      fp32 [B][H][d][d]   dL/dS after the last frame (in), dL/dS_0 (out)
 *   dphi_q/k/v        fp32 [H][d][d]      accumulated over the frames since arl2_bwd_begin
 * Precision: the softmax branch's backward forms the scores Q K^T from the bf16 inputs as given
 * and multiplies fp16 operands elsewhere, all with fp32 accumulation (q, k, v converted from
 * bf16, exact for 2^-14 <= |x| <= 65504; P, dS and dO rounded to fp16); the inter-frame read and
 * the state write use split-bf16 products (about fp32 accuracy).  Results are bitwise
 * reproducible (no atomics).
 * Status codes, arl2_last_error() and the stream rule (a call on a different stream than the
 * previous one waits for it) are those of arl2.h.  A failed launch poisons the object
 * (ARL2_E_PROTOCOL) until arl2_bwd_begin.
 * Streams: arl2_bwd_pass also runs part of its work on a second stream that the object creates
 * (default priority, not synchronising with the null stream), forked from and joined back into
 * the caller's stream inside the call: work the caller enqueues afterwards on its stream sees
 * every result of the call.
 * Graph capture: unlike the forward's calls, these are meant for eager launch.  Each
 * arl2_bwd_commit reads dL/dS from one of two device buffers and writes the other, chosen on the
 * host, so a captured commit would replay with the buffers it was captured with.
 */
#ifndef ARL2_BWD_H
#define ARL2_BWD_H

#include <stddef.h>
#include <stdint.h>

#include "arl2.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct arl2_bwd arl2_bwd; /* opaque, owned by the library */

/* Create a backward object on the current HIP device for a layer of configuration cfg (frame-
 * level access, head_dim 64 or 128, else ARL2_E_UNSUPPORTED) and maps phi_q, phi_k, phi_v
 * (device pointers, bf16 [H][d][d], copied).  It allocates all the device memory it will use
 * (arl2_bwd_device_bytes) and starts as after arl2_bwd_begin(ds_last = NULL). */
arl2_status arl2_bwd_create(const arl2_config* cfg, const void* phi_q, const void* phi_k, const void* phi_v,
                            void* stream, arl2_bwd** out);

/* Start a backward sweep: dL/dS after the last frame = ds_last (zero if NULL); the dphi sums are
 * zeroed; clears the poisoned condition. */
arl2_status arl2_bwd_begin(arl2_bwd* g, const float* ds_last, void* stream);

/* Backward of one pass of the current frame (the frame before the last one committed in this
 * sweep): writes dq, dk, dv for its q, k, v and adds its share to dL/dS_{N-1} and dphi_q. */
arl2_status arl2_bwd_pass(arl2_bwd* g, const void* q, const void* k, const void* v, const float* s_prev,
                          const float* d_out, float* dq, float* dk, float* dv, void* stream);

/* Backward of the current frame's state write, with the clean pass's k, v and the frame's beta,
 * alpha and S_{N-1}: adds to dk, dv, writes dbeta, dalpha, adds to dphi_k, dphi_v, and forms
 * dL/dS_{N-1} (with the passes' shares); the sweep moves to the previous frame. */
arl2_status arl2_bwd_commit(arl2_bwd* g, const void* k, const void* v, const float* beta, const float* alpha,
                            const float* s_prev, float* dk, float* dv, float* dbeta, float* dalpha, void* stream);

/* Copy out dL/dS of the frame the sweep stands at (dL/dS_0 after the first frame's commit) and
 * the dphi sums; any pointer may be NULL. */
arl2_status arl2_bwd_read(arl2_bwd* g, float* ds, float* dphi_q, float* dphi_k, float* dphi_v, void* stream);

arl2_status arl2_bwd_destroy(arl2_bwd* g);

/* Device memory held by the object, in bytes. */
size_t arl2_bwd_device_bytes(const arl2_bwd* g);

#ifdef __cplusplus
}
#endif

#endif /* ARL2_BWD_H */
