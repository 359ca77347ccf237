/*
 * arl2_linear.h - the linear projections around the attention layers of an ARL2 model (the fused
 * Q, K, V projection in front of each layer and its output projection), for AMD Instinct MI355X
 * (gfx950), in the same library.
 *
 * Source: "Attend Locally, Remember Linearly: Linear Attention as Cross-Frame Memory for
 * Autoregressive Video Diffusion" - the technical summary on gist.science (section 2.1: the
 * intra-frame branch reuses the pretrained layer's frozen projections, and the ARL2 layer reads
 * the same Q, K, V through its per-head maps; section 1 and section 4: the attention stack of
 * the 1.3B video DiT whose layers the conversion keeps or replaces).
 *
 *   y = x W        x bf16 [M][K] (the M = B T tokens of a frame, K = H d features),
 *                  W given transposed: w_t bf16 [N][K] (row n holds output feature n's weights),
 *                  y [M][N] in y_dtype (ARL2_F32 or ARL2_BF16, rounded to nearest even).
 *
 * With parts > 1 the N output features are dealt to `parts` outputs y[0..parts-1], each a
 * row-major [M][N / parts] tensor: output p holds features p N / parts .. (p + 1) N / parts - 1.
 * A Q, K, V projection with parts = 3 and N = 3 H d writes the three bf16 [B][T][H][d] tensors
 * that arl2_denoise_step / arl2_commit_frame and the softmax layers read.
 *
 * Arithmetic: bf16 products, fp32 accumulation over K (no split-K: every output is one fixed-order
 * sum, so results repeat bitwise), then the output rounding of y_dtype.
 *
 * Limits: M, N, K >= 0; K a multiple of 64 and at most 2^20; N a multiple of 8; 1 <= parts <= 4
 * with N / parts a multiple of 4; all pointers device memory, 16-byte aligned, owned by the
 * caller and valid until the enqueued work has finished.  Outputs must not overlap x or w_t.
 * Errors: ARL2_E_INVALID_ARG for null / misaligned pointers or bad sizes, ARL2_E_UNSUPPORTED for
 * sizes beyond the limits, ARL2_E_HIP if the launch fails; nothing is enqueued on an error.
 * The work is enqueued on `stream` (a hipStream_t; NULL = the null stream).
 */
#ifndef ARL2_LINEAR_H
#define ARL2_LINEAR_H

#include <stdint.h>

#include "arl2.h"

#ifdef __cplusplus
extern "C" {
#endif

arl2_status arl2_linear(const void* x, const void* w_t, int32_t m, int32_t n, int32_t k, int32_t parts,
                        void* const* y, int32_t y_dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ARL2_LINEAR_H */
