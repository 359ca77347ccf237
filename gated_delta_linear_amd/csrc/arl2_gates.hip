// Gate projections of the ARL2 state write ("Attend Locally, Remember Linearly", gist.science
// technical summary, section 2.1: alpha, the forget gate, and beta, the learning rate, are
// learned projections of the tokens; section 4, ablations: head-wise gates):
//   beta[b][t][h] = beta_scale * sigmoid(x[b][t] . w[h] + bias[h])
//   alpha logit partial[b][blk][h] = sum over tokens t of block blk of x[b][t] . w[H + h]
// from the layer's input hidden states x [B][T][H d] bf16 and the gate weights w [2H][H d]
// bf16 (rows 0..H-1: beta, rows H..2H-1: alpha), bias [2H] fp32.  The reduce kernel turns the
// partials into alpha[b][h] = sigmoid(mean over the frame's tokens + bias[H + h]), one decay
// per (stream, head) and frame, as the frame-level write applies it; the state write's
// per-chunk work-groups read beta.
//
// One work-group of 4 waves per (16-token block, 64 gate columns, stream).  The waves split
// the H d features in four: wave w forms, with 16x16x32 bf16 MFMAs, the 16 x 64 logits over its
// quarter (A = token rows of x, B = weight rows, both straight from memory, 16 bytes per lane
// per k-step, a batch of k-steps' loads in flight at a time); the quarters are then added
// through LDS in a fixed order (bitwise reproducible) by the wave that finishes each 16-column
// block.  At 1560 tokens and 12 heads: 98 work-groups, one latency round per batch.
#include "arl2_device.h"
#include "arl2_kernels.h"

namespace arl2 {
namespace {

constexpr int kGateTokens = 16;  // tokens per work-group
constexpr int kGateCols = 64;    // gate columns per work-group (four 16-column blocks)
constexpr int kGateBatch = 12;   // k-steps whose loads are in flight together

__device__ __forceinline__ __amdgpu_buffer_rsrc_t gate_rsrc(const void* p, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

__global__ __launch_bounds__(256) void arl2_gates_kernel(const bf16* __restrict__ x, const bf16* __restrict__ w,
                                                         const float* __restrict__ bias, float beta_scale,
                                                         float* __restrict__ beta, float* __restrict__ alpha_part,
                                                         int T, int H, int Dm) {
  __shared__ f32x4 red[4][4][64];  // [feature quarter][column block][lane]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, g4 = lane >> 4;
  const int blk = blockIdx.x, b = blockIdx.z;
  const int t0 = blk * kGateTokens;
  const int c0 = blockIdx.y * kGateCols;                 // first gate column of the work-group
  const int nblk = min(4, (2 * H - c0 + 15) / 16);       // 16-column blocks with gates
  // x rows of this stream past the frame, and weight rows past 2H, read as zeros
  const __amdgpu_buffer_rsrc_t rx = gate_rsrc(x + (int64_t)b * T * Dm, (int64_t)T * Dm * 2);
  const __amdgpu_buffer_rsrc_t rw = gate_rsrc(w, (int64_t)2 * H * Dm * 2);
  const int ks_n = (Dm + 31) / 32, kq = (ks_n + 3) / 4;
  const int ks0 = wave * kq, ks1 = min(ks_n, ks0 + kq);  // this wave's k-steps
  f32x4 acc[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  // lane l: token row t0 + l % 16 of x, weight rows c0 + 16 n + l % 16; features 32 ks + 8 (l / 16) ..
  const int xo = (t0 + r16) * Dm * 2;
  int wo[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) wo[n] = (c0 + 16 * n + r16) * Dm * 2;
  for (int kb = ks0; kb < ks1; kb += kGateBatch) {
    bf16x8 a[kGateBatch], bw[kGateBatch][4];
#pragma unroll
    for (int j = 0; j < kGateBatch; ++j) {
      const int f = 32 * (kb + j) + 8 * g4;
      const bool in = kb + j < ks1 && f < Dm;  // (H d is a multiple of 16: a lane's 8 features are all in or out)
      const int fo = 2 * (in ? f : 0);
      a[j] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rx, xo + fo, 0, 0));
#pragma unroll
      for (int n = 0; n < 4; ++n)
        bw[j][n] = n < nblk ? __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rw, wo[n] + fo, 0, 0))
                            : zero_bf16x8();
      if (!in) a[j] = zero_bf16x8();
    }
#pragma unroll
    for (int j = 0; j < kGateBatch; ++j)
#pragma unroll
      for (int n = 0; n < 4; ++n) acc[n] = mfma16(a[j], bw[j][n], acc[n]);
  }
#pragma unroll
  for (int n = 0; n < 4; ++n) red[wave][n][lane] = acc[n];
  __syncthreads();
  if (wave >= nblk) return;
  // wave n finishes column block n: lane l, register i = token t0 + 4 (l / 16) + i, column g
  const f32x4 z4 = red[0][wave][lane] + red[1][wave][lane] + red[2][wave][lane] + red[3][wave][lane];
  const int g = c0 + 16 * wave + r16;
  float asum = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + 4 * g4 + i;
    if (t >= T) continue;
    if (g < H) beta[((int64_t)b * T + t) * H + g] = beta_scale / (1.f + expf(-(z4[i] + bias[g])));
    else asum += z4[i];
  }
  // the alpha partial of column g: the sum over the lanes l, l ^ 16, l ^ 32, l ^ 48
  asum += __shfl_xor(asum, 16);
  asum += __shfl_xor(asum, 32);
  if (g >= H && g < 2 * H && lane < 16) alpha_part[((int64_t)b * gridDim.x + blk) * H + (g - H)] = asum;
}

}  // namespace

int gate_blocks(int T) { return (T + kGateTokens - 1) / kGateTokens; }

hipError_t launch_gates(const GateArgs& a, hipStream_t stream) {
  const int Dm = a.H * a.d;
  dim3 grid(gate_blocks(a.T), (2 * a.H + kGateCols - 1) / kGateCols, a.B);
  hipLaunchKernelGGL(arl2_gates_kernel, grid, dim3(256), 0, stream, static_cast<const bf16*>(a.x),
                     static_cast<const bf16*>(a.w), a.bias, a.beta_scale, a.beta, a.alpha_part, a.T, a.H, Dm);
  return hipGetLastError();
}

}  // namespace arl2
