/*
 * arl2_softmax.h - C interface of the retained softmax attention layer that an ARL2 model
 * keeps beside its ARL2 layers, for AMD Instinct MI355X (gfx950), in the same library.
 *
 * Source: "Attend Locally, Remember Linearly: Linear Attention as Cross-Frame Memory for
 * Autoregressive Video Diffusion" - the technical summary on gist.science (section 1, the
 * problem: autoregressive video DiTs attend over a key-value cache that grows by one block
 * per generated frame; section 2, the two-stage conversion in which the layers not replaced
 * keep softmax attention; section 4, the memory and speed comparison against that baseline)
 * and the authors' abstract (fugumt.com page of the same title).
 *
 * One layer object holds, for B independent streams and H heads, a cache of the clean keys
 * and values of up to max_frames frames of T tokens.  For every latent frame N (0-based)
 * the caller runs any number of denoising passes and then one clean pass, with the frame's
 * q, k, v:
 *
 *   every pass:  out = softmax(Q [K_0; ...; K_{N-1}; K]^T * scale) [V_0; ...; V_{N-1}; V]
 *                (block-causal: the frame's queries see every earlier frame's clean keys
 *                and all of their own frame's keys)
 *   clean pass:  afterwards K, V become frame N's cached K_N, V_N and N advances.
 *
 * Readings this library fixes: keys and values of denoising passes are never cached;
 * scale defaults to 1/sqrt(d); no projection, position encoding or mask beyond the block-
 * causal one (the caller supplies q, k, v as its projections emit them).
 *
 * Tensors (device memory, contiguous, row-major, 16-byte aligned, owned by the caller and
 * valid until the enqueued work has finished):
 *   q, k, v   bf16  [B][T][H][d]
 *   out       fp32 or bf16 (config) [B][T][H][d]
 * Arithmetic: that of arl2.h's softmax branch (bf16 Q K^T, fp32 softmax, fp16 P and V in P V).
 * Status codes, the stream rule (a call on a different stream than the previous one waits
 * for it) and arl2_last_error() are those of arl2.h.  A failed launch poisons the layer
 * (later calls return ARL2_E_PROTOCOL) until arl2_softmax_reset.
 * Graph capture: the number of cached frames is host state, and every call's launch is shaped
 * by it (keys attended, the cache slot a commit writes), so a captured call replays as the call
 * it was: capture the passes of one frame and replay them only while that frame is current.
 */
#ifndef ARL2_SOFTMAX_H
#define ARL2_SOFTMAX_H

#include <stddef.h>
#include <stdint.h>

#include "arl2.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct arl2_softmax_layer arl2_softmax_layer; /* opaque, owned by the library */

typedef struct {
  int32_t batch;            /* B, 1 <= B <= 65535 */
  int32_t heads;            /* H, 1 <= H <= 65535 */
  int32_t head_dim;         /* d: 16, 64 or 128 */
  int32_t tokens_per_frame; /* T, 1 <= T <= ARL2_MAX_TOKENS */
  int32_t max_frames;       /* frames the cache holds, >= 1; max_frames * T * H * d * 2 bytes
                               (one stream's cache of K or V) must stay below 2 GiB, and
                               ceil(T / 128) * B * H below 2^24 (ARL2_E_UNSUPPORTED) */
  int32_t out_dtype;        /* ARL2_F32 or ARL2_BF16 (round to nearest even) */
  float softmax_scale;      /* 0 selects 1/sqrt(d) */
} arl2_softmax_config;

/* Create a layer on the current HIP device: allocates the K and V caches (bf16
 * [B][max_frames * T][H][d] each), the only device memory it will use; frame index 0.
 * `stream` is the layer's first stream.  On failure *out_layer is set to NULL. */
arl2_status arl2_softmax_layer_create(const arl2_softmax_config* cfg, void* stream,
                                      arl2_softmax_layer** out_layer);

/* One denoising pass of frame N: out over the cached frames 0..N-1 and this pass's k, v.
 * The cache keeps frames 0..N-1 unchanged (this pass's k, v go to slot N, which the clean
 * pass overwrites); the frame index does not change.  ARL2_E_PROTOCOL if N == max_frames. */
arl2_status arl2_softmax_pass(arl2_softmax_layer* layer, const void* q, const void* k, const void* v,
                              void* out, void* stream);

/* The clean pass of frame N: if `out` is not NULL, the output as arl2_softmax_pass computes it
 * (`q` may be NULL when `out` is NULL); k, v become cached frame N; the frame index advances.
 * ARL2_E_PROTOCOL if N == max_frames. */
arl2_status arl2_softmax_commit(arl2_softmax_layer* layer, const void* q, const void* k, const void* v,
                                void* out, void* stream);

/* Empty the cache (frame index 0) and clear the poisoned condition; enqueues nothing. */
arl2_status arl2_softmax_reset(arl2_softmax_layer* layer);

/* Synchronise the last stream the layer used and free everything.  NULL is accepted. */
arl2_status arl2_softmax_destroy(arl2_softmax_layer* layer);

/* Frames cached so far (N); -1 for NULL. */
int64_t arl2_softmax_frame_index(const arl2_softmax_layer* layer);

/* Device bytes held by the layer (the two caches); fixed at create.  0 for NULL. */
size_t arl2_softmax_device_bytes(const arl2_softmax_layer* layer);

#ifdef __cplusplus
}
#endif

#endif /* ARL2_SOFTMAX_H */
