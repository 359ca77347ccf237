/*
 * arl2.h - C interface of the ARL2 hybrid attention layer (forward hot path) for AMD
 * Instinct MI355X (gfx950).
 *
 * Source of the operations: "Attend Locally, Remember Linearly: Linear Attention as
 * Cross-Frame Memory for Autoregressive Video Diffusion" - the technical summary on
 * gist.science (section 2.1, hybrid attention decomposition; section 2.2, memory state
 * management) and the authors' abstract (fugumt.com page of the same title).
 *
 * One layer object holds, for B independent streams and H heads, a fixed-size recurrent
 * state S[b][h] (d x d, fp32) and three per-head d x d maps phi_q, phi_k, phi_v.  For every
 * latent frame N of T tokens the caller runs any number of denoising passes and then one
 * clean pass:
 *
 *   every pass:  O = softmax(Q K^T * scale) V  +  (Q phi_q) S_{N-1}
 *                (softmax over the frame's own tokens, bidirectional: section 2.1, intra-frame
 *                branch; the second term is the inter-frame read, section 2.1 "output", with
 *                the same S_{N-1} for every token: section 2.2, frame-level access)
 *   clean pass:  afterwards S_N = alpha S_{N-1} + K'^T diag(beta) (V' - K' S_{N-1}),
 *                K' = rows of K phi_k scaled to unit length, V' = V phi_v
 *                (section 2.1, state update; written once per frame and never during
 *                denoising: section 2.2, clean-pass updates)
 *
 * Conventions that the pages leave open and this library fixes:
 *   - maps act on row vectors: x'[j] = sum_i x[i] * phi[i][j]; no bias, no activation;
 *   - the first K' of the update is transposed (shapes), alpha scales S_{N-1} only;
 *   - alpha is one value per (stream, head) and frame, beta one per (stream, token, head);
 *   - the two branches are added; scale defaults to 1/sqrt(d); K' rows are divided by
 *     max(norm, knorm_eps); S_0 = 0.
 *
 * Tensors (all device memory, contiguous, row-major, 16-byte aligned, owned by the caller
 * and required to stay valid until the work enqueued on the stream has finished):
 *   q, k, v     bf16  [B][T][H][d]        token-major, as a fused QKV projection emits them
 *                                         (fp32 with io_dtype ARL2_F32)
 *   out         fp32 or bf16 (config) [B][T][H][d]
 *   beta        fp32  [B][T][H]
 *   alpha       fp32  [B][H]
 *   phi_q/k/v   bf16  [H][d][d]           phi[h][i][j], read once by arl2_layer_create
 *                                         (fp32 with io_dtype ARL2_F32)
 *   state       fp32  [B][H][d][d]        S[b][h][i][j]: i = key feature, j = value feature
 *
 * Arithmetic: Q K^T and the inter-frame read use bf16 products with fp32 accumulation (the
 * read as Q (phi_q S_{N-1}), its d x d factor split into two bf16 terms); the softmax runs in
 * fp32; P V multiplies P rounded to fp16 by V converted to fp16, which is exact for
 * 2^-14 <= |v| <= 65504 (smaller |v| round to fp16 subnormals, larger ones become infinite);
 * the state write uses split-bf16 products (about fp32 accuracy) and keeps S in fp32.
 * With io_dtype ARL2_F32 the fp32 q, k, v and maps are rounded to bf16 (nearest even) on the
 * device first, into copies the layer owns; the result is the bf16 path's on those values.
 *
 * Graph capture: every call's device addresses are fixed (S is one buffer that the clean pass
 * updates in place), so calls captured into a HIP graph replay the protocol frame after frame.
 * The frame index is host state: it counts calls, not replays of captured calls.
 *
 * Streams: every call enqueues its work on `stream` (a hipStream_t; NULL = the null
 * stream) and returns without waiting.  If a call uses a different stream from the
 * previous call on the same layer, the library makes the new stream wait for the old one.
 *
 * Errors: functions return arl2_status.  Argument errors are detected before any work is
 * enqueued and leave the layer unchanged.  A failed launch returns ARL2_E_HIP and poisons
 * the layer: later calls return ARL2_E_PROTOCOL until arl2_state_write succeeds.  Faults
 * inside kernels surface at the caller's next synchronisation, as usual in HIP.
 * arl2_last_error() returns a human-readable detail of the calling thread's last failure.
 *
 * Threading: a layer is not thread-safe; distinct layers are independent.
 */
#ifndef ARL2_H
#define ARL2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct arl2_layer arl2_layer; /* opaque, owned by the library */

typedef enum {
  ARL2_OK = 0,
  ARL2_E_INVALID_ARG = 1,   /* null / misaligned pointer, bad size or shape */
  ARL2_E_UNSUPPORTED = 2,   /* head_dim, dtype or device not supported */
  ARL2_E_NO_DEVICE = 3,     /* no HIP device visible */
  ARL2_E_OUT_OF_MEMORY = 4, /* device allocation failed at create */
  ARL2_E_HIP = 5,           /* a HIP runtime call or launch failed */
  ARL2_E_PROTOCOL = 6       /* layer poisoned by an earlier failure, or destroyed */
} arl2_status;

typedef enum { ARL2_BF16 = 0, ARL2_F32 = 1 } arl2_dtype;

typedef struct {
  int32_t batch;            /* B, 1 <= B <= 65535 independent streams */
  int32_t heads;            /* H, 1 <= H <= 65535 */
  int32_t head_dim;         /* d: 16, 64 or 128 */
  int32_t tokens_per_frame; /* T, 1 <= T <= ARL2_MAX_TOKENS (a chunk of frames counts as one frame);
                               (T + 256) * H * d * 2 bytes must stay below 2 GiB, and
                               ceil(T / 128) * B * H below 2^24 (ARL2_E_UNSUPPORTED) */
  int32_t io_dtype;         /* dtype of q, k, v and phi: ARL2_BF16, or ARL2_F32 (rounded to bf16,
                               nearest even, on the device; the gated call's x stays bf16) */
  int32_t out_dtype;        /* ARL2_F32 (recommended) or ARL2_BF16 (round to nearest even) */
  float softmax_scale;      /* 0 selects 1/sqrt(d) */
  float knorm_eps;          /* 0 selects 1e-6 */
  int32_t access;           /* ARL2_ACCESS_FRAME (the method) or ARL2_ACCESS_TOKEN (the sequential
                               variant the pages reject, for A/B; head_dim 64 or 128) */
} arl2_config;

/* Frame-level access: every token of a frame reads S_{N-1} and the write takes every token's
 * residual against it (section 2.2).  Token-level access: token t reads, and takes its residual
 * against, the state updated by the frame's earlier tokens,
 *   o_t = softmax branch_t + (q_t phi_q) S^(t-1),  S^(0) = S_{N-1},
 *   S^(t) = S^(t-1) + beta_t k'_t^T (v'_t - k'_t S^(t-1)),  clean pass: S_N = S^(T) - (1 - alpha) S_{N-1};
 * every pass needs beta, so such a layer runs arl2_denoise_step_seq / arl2_commit_frame_seq
 * instead of arl2_denoise_step / arl2_commit_frame (ARL2_E_INVALID_ARG either way round). */
enum { ARL2_ACCESS_FRAME = 0, ARL2_ACCESS_TOKEN = 1 };

#define ARL2_MAX_TOKENS (1 << 20)

/* Create a layer on the current HIP device (section 2.1: per-head maps phi_q, phi_k, phi_v and
 * a d x d state per stream and head; S_0 = 0): allocates all device memory the layer will ever
 * use (S, derived forms of S, per-chunk partial sums of the write, the maps' working layouts,
 * and with io_dtype ARL2_F32 bf16 copies of a frame's q, k, v), copies phi_q, phi_k, phi_v
 * (device pointers, [H][d][d] of io_dtype) into it with work enqueued on `stream`, and sets
 * S_0 = 0 and the frame index to 0.  No call after create allocates.  On failure *out_layer is
 * set to NULL. */
arl2_status arl2_layer_create(const arl2_config* cfg, const void* phi_q, const void* phi_k,
                              const void* phi_v, void* stream, arl2_layer** out_layer);

/* One denoising pass of the current frame (section 2.1: the intra-frame softmax branch plus the
 * inter-frame read Q' S_{N-1}; section 2.2: frame-level access, and no state write during
 * denoising): out = softmax branch + inter-frame read of S_{N-1}.  q, k, v [B][T][H][d] of
 * io_dtype, out [B][T][H][d] of out_dtype.  Reads S, never writes it; the frame index does not
 * change. */
arl2_status arl2_denoise_step(arl2_layer* layer, const void* q, const void* k, const void* v,
                              void* out, void* stream);

/* The clean pass of the current frame (section 2.2: the state is written once per frame, after
 * the final clean pass; section 2.1: the gated update S_N = alpha S_{N-1} + K'^T diag(beta)
 * (V' - K' S_{N-1})).  If `out` is not NULL it first computes the pass's output exactly as
 * arl2_denoise_step does (with S_{N-1}; `q` may be NULL when `out` is NULL).  It then writes
 * S_N from k, v, beta [B][T][H] and alpha [B][H] and advances the frame index by one. */
arl2_status arl2_commit_frame(arl2_layer* layer, const void* q, const void* k, const void* v,
                              const float* beta, const float* alpha, void* out, void* stream);

/* The clean pass with alpha and beta from the layer's gate projections (section 2.1: the
 * forget gate alpha and the learning rate beta are learned projections of the tokens; section
 * 4, ablations: head-wise gates), computed on the device from the frame's hidden states x, bf16
 * [B][T][H d] (the input of the QKV projection), and the caller's gate weights w_gates, bf16
 * [2H][H d] (row h: beta of head h; row H + h: alpha of head h), and biases b_gates, fp32 [2H]:
 *   beta[b][t][h] = beta_scale * sigmoid(x[b][t] . w_gates[h] + b_gates[h])
 *   alpha[b][h]   = sigmoid(mean over the frame's tokens t of x[b][t] . w_gates[H + h]
 *                           + b_gates[H + h])
 * (one decay per stream, head and frame, as the frame-level write applies it).  Otherwise as
 * arl2_commit_frame.  ARL2_E_UNSUPPORTED if 2H x H d x 2 bytes of weights reach 2 GiB. */
arl2_status arl2_commit_frame_gated(arl2_layer* layer, const void* q, const void* k, const void* v,
                                    const void* x, const void* w_gates, const float* b_gates,
                                    float beta_scale, void* out, void* stream);

/* Token-level access layers: a denoising pass (beta [B][T][H] of the pass's tokens; the state is
 * not written) and the clean pass (writes S_N with beta and alpha [B][H], then advances the frame
 * index; `out` may be NULL; q is always read, by the recurrence). */
arl2_status arl2_denoise_step_seq(arl2_layer* layer, const void* q, const void* k, const void* v,
                                  const float* beta, void* out, void* stream);
arl2_status arl2_commit_frame_seq(arl2_layer* layer, const void* q, const void* k, const void* v,
                                  const float* beta, const float* alpha, void* out, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): the clean pass of one frame without a layer object.
 * It computes exactly what arl2_commit_frame does on a layer created with cfg, phi_q, phi_k,
 * phi_v whose state equals `state`: `out` (if not NULL) = the pass's output with S_{N-1} =
 * state, then state <- S_N, in place.  state: fp32 [B][H][d][d] device memory owned by the
 * caller (S_0 = 0 is the caller's zero buffer); the other arguments as arl2_layer_create and
 * arl2_commit_frame (bf16 inputs, frame-level access only: ARL2_E_UNSUPPORTED otherwise).
 * It allocates nothing: the maps' working layouts, the derived forms of S and the state
 * write's per-chunk partial sums live in a device array of ARL2_NOALLOC_SCRATCH_BYTES that the
 * library holds on every GPU it runs on until the process ends; a frame needing more is
 * refused with ARL2_E_UNSUPPORTED (about 13 MB for 12 heads x 1560 tokens x d = 128).  Every
 * call on a GPU reuses that GPU's array: calls that overlap on one GPU (on different streams,
 * or from different threads) race and give wrong results; calls on one stream are ordered. */
#define ARL2_NOALLOC_SCRATCH_BYTES (32u << 20)
arl2_status arl2_commit_frame_noalloc(const arl2_config* cfg, const void* phi_q, const void* phi_k,
                                      const void* phi_v, float* state, const void* q, const void* k,
                                      const void* v, const float* beta, const float* alpha, void* out,
                                      void* stream);

/* Synchronise the last stream the layer used and free everything.  NULL is accepted. */
arl2_status arl2_destroy(arl2_layer* layer);

/* Copy the current state S (fp32 [B][H][d][d], device memory) to dst, enqueued on stream. */
arl2_status arl2_state_read(arl2_layer* layer, float* dst, void* stream);

/* Replace the state with src (fp32 [B][H][d][d], device memory) and set the frame index:
 * restores a checkpoint taken with arl2_state_read + arl2_frame_index.  Also clears the
 * poisoned condition. */
arl2_status arl2_state_write(arl2_layer* layer, const float* src, int64_t frame_index, void* stream);

/* Number of frames committed so far (N after committing frame N); -1 for NULL. */
int64_t arl2_frame_index(const arl2_layer* layer);

/* Device bytes held by the layer; fixed at create. 0 for NULL. */
size_t arl2_device_bytes(const arl2_layer* layer);

/* Static description of a status code. */
const char* arl2_status_string(arl2_status status);

/* Detail of the calling thread's most recent failure ("" if none). */
const char* arl2_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ARL2_H */
