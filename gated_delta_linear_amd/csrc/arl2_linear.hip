// Linear projections of an attention layer in the stack (include/arl2_linear.h):
//   y = x W,   x bf16 [M][K],  W given transposed (W^T bf16 [N][K]),  y bf16 or fp32 [M][N],
// the N output features optionally dealt to `parts` separate row-major outputs of N / parts
// features each (a fused Q, K, V projection writing the three [B][T][H][d] tensors the attention
// layers read).  "Attend Locally, Remember Linearly", gist.science technical summary, section
// 2.1: the intra-frame branch reuses the pretrained layer's frozen projections; section 1 / 4:
// the softmax baseline whose key-value cache the hybrid replaces.
//
// Kernel.  One work-group of 4 waves (one per SIMD, two work-groups per CU) per 128 x BN tile of
// y, BN = 128 or 64, over K in steps of 64.  The tile is computed transposed, y^T = W^T x^T, with
// 32x32x16 bf16 MFMAs (fp32 accumulation): W^T rows are the A operand and x rows the B operand,
// both read as 16-byte row segments, so that each lane of a finished block holds four
// consecutive output features of one row (16-byte fp32 / 8-byte bf16 stores).  Wave w owns rows
// 64 (w / 2) .. + 63 and features (BN / 2) (w % 2) .. of the tile.  Operand tiles come into LDS
// with direct-to-LDS buffer loads, double-buffered (one work-group barrier per 64-deep step);
// the 16-byte granules of row r are permuted (granule g holds chunk g ^ (r % 8)) so that every
// load brings whole rows and the fragment reads of 32 rows hit distinct banks.  Rows past M or N
// lie outside the buffer descriptors and load as zeros; their outputs are not stored.
#include "arl2_device.h"
#include "arl2_kernels.h"

namespace arl2 {
namespace {

constexpr int kBM = 128;    // rows of y per work-group
constexpr int kBK = 64;     // contraction depth per step
constexpr int kThreadsL = 256;
typedef __attribute__((address_space(3))) void lds_void_l;

__device__ __forceinline__ void dma16l(__amdgpu_buffer_rsrc_t r, void* lds, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_l*)lds, 16, voff, soff, 0, 0);
}

// Buffer resource over rows [row0, rows) of a row-major bf16 matrix with `k` columns.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t mat_rsrc(const bf16* base, int64_t row0, int64_t rows, int k) {
  const int64_t left = rows - row0;
  const bool any = left > 0;
  const int64_t bytes = any ? left * k * 2 : 0;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16*>(any ? base + row0 * k : base), (short)0,
                                           (int)(bytes < 0x7FFFFFFF ? bytes : 0x7FFFFFFF), 0x00020000);
}

template <int BN, bool OUT_BF16>
__global__ __launch_bounds__(kThreadsL) __attribute__((amdgpu_waves_per_eu(2, 2))) void arl2_linear_kernel(
    const bf16* __restrict__ x, const bf16* __restrict__ wt, LinearOut y, int M, int N, int K, int n_tiles_n) {
  constexpr int WN = BN / 2;       // features per wave
  constexpr int NB = WN / 32;      // 32-feature blocks per wave (A operand)
  constexpr int MB = 2;            // 32-row blocks per wave (B operand)
  constexpr int A_BYTES = BN * kBK * 2, X_BYTES = kBM * kBK * 2;
  __shared__ __attribute__((aligned(16))) unsigned char wl0[A_BYTES], wl1[A_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char xl0[X_BYTES], xl1[X_BYTES];

  // XCD-aware order: work-group i runs on XCD i % 8; each XCD takes a contiguous run of tiles in
  // feature-major order, so the row tiles that share a block of W^T run on one L2.
  const int n_tiles = n_tiles_n * ((M + kBM - 1) / kBM), per_xcd = (n_tiles + 7) / 8;
  const int tile = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (tile >= n_tiles) return;
  const int tn = tile % n_tiles_n, tm = tile / n_tiles_n;
  const int n0 = tn * BN, m0 = tm * kBM;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave >> 1, wc = wave & 1;

  const __amdgpu_buffer_rsrc_t rw = mat_rsrc(wt, n0, N, K);
  const __amdgpu_buffer_rsrc_t rx = mat_rsrc(x, m0, M, K);
  // Loads: 1 KB per wave instruction = 8 rows of 128 bytes; lane l brings granule (l % 8) ^ (row % 8)
  // of row l / 8 (rows 8 i .. 8 i + 7 of instruction i), stored at granule l % 8 of its row.
  const int lrow = lane >> 3;
  const int g_vo = lrow * K * 2 + 16 * ((lane & 7) ^ (lrow & 7));  // (row % 8 == lrow for rows 8 i + lrow)
  constexpr int W_LD = A_BYTES / 1024, X_LD = X_BYTES / 1024;       // 1-KB loads per tile
  auto load_step = [&](int kb, unsigned char* wdst, unsigned char* xdst) {
    const int kofs = kb * kBK * 2;
#pragma unroll
    for (int i = wave; i < W_LD; i += 4) dma16l(rw, wdst + i * 1024, g_vo, i * 8 * K * 2 + kofs);
#pragma unroll
    for (int i = wave; i < X_LD; i += 4) dma16l(rx, xdst + i * 1024, g_vo, i * 8 * K * 2 + kofs);
  };
  // Fragment of 32 rows starting at row r0 of a staged tile, k-step s (16 deep): lane l reads row
  // r0 + l % 32, chunk 2 s + l / 32, at granule chunk ^ (row % 8).
  auto frag = [&](const unsigned char* t, int r0, int s) {
    const int row = r0 + (lane & 31);
    const int ch = 2 * s + (lane >> 5);
    return *reinterpret_cast<const bf16x8*>(t + row * (kBK * 2) + 16 * (ch ^ (row & 7)));
  };

  f32x16 acc[NB][MB];
#pragma unroll
  for (int a = 0; a < NB; ++a)
#pragma unroll
    for (int b = 0; b < MB; ++b) acc[a][b] = zero16();

  const int steps = K / kBK;
  load_step(0, wl0, xl0);
  auto compute = [&](const unsigned char* wt_l, const unsigned char* x_l) {
#pragma unroll
    for (int s = 0; s < kBK / 16; ++s) {
      bf16x8 af[NB], bf[MB];
#pragma unroll
      for (int a = 0; a < NB; ++a) af[a] = frag(wt_l, wc * WN + 32 * a, s);
#pragma unroll
      for (int b = 0; b < MB; ++b) bf[b] = frag(x_l, wr * 64 + 32 * b, s);
#pragma unroll
      for (int a = 0; a < NB; ++a)
#pragma unroll
        for (int b = 0; b < MB; ++b) acc[a][b] = mfma32(af[a], bf[b], acc[a][b]);
    }
  };
  for (int kb = 0; kb < steps; kb += 2) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // this wave's loads into buffer 0 have landed
    __syncthreads();                     // everyone's have; buffer 1 is free again
    if (kb + 1 < steps) load_step(kb + 1, wl1, xl1);
    compute(wl0, xl0);
    if (kb + 1 >= steps) break;
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    if (kb + 2 < steps) load_step(kb + 2, wl0, xl0);
    compute(wl1, xl1);
  }

  // Block (a, b): lane l, register i holds y[m0 + 64 wr + 32 b + l % 32][n0 + WN wc + 32 a +
  // 8 (i / 4) + 4 (l / 32) + i % 4]: registers 4 g .. 4 g + 3 are four consecutive features
  // (the C layout of the 32x32 product, whose rows are features and columns rows of x).
  const int part_n = N / y.parts;
#pragma unroll
  for (int b = 0; b < MB; ++b) {
    const int m = m0 + 64 * wr + 32 * b + (lane & 31);
    if (m >= M) continue;
#pragma unroll
    for (int a = 0; a < NB; ++a)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + WN * wc + 32 * a + 8 * g + 4 * (lane >> 5);
        if (n >= N) continue;
        const int p = n / part_n, c = n - p * part_n;
        const int64_t o = (int64_t)m * part_n + c;
        const f32x4 v = f32x4{acc[a][b][4 * g], acc[a][b][4 * g + 1], acc[a][b][4 * g + 2], acc[a][b][4 * g + 3]};
        if (OUT_BF16) {
          bf16x4 h;
#pragma unroll
          for (int e = 0; e < 4; ++e) h[e] = (bf16)v[e];
          *reinterpret_cast<bf16x4*>(static_cast<bf16*>(y.ptr[p]) + o) = h;
        } else {
          *reinterpret_cast<f32x4*>(static_cast<float*>(y.ptr[p]) + o) = v;
        }
      }
  }
}

template <int BN>
hipError_t launch_linear_bn(const LinearArgs& a, hipStream_t stream) {
  const int ntn = (a.N + BN - 1) / BN, ntm = (a.M + kBM - 1) / kBM;
  dim3 grid(8 * ((ntn * ntm + 7) / 8));
  const bf16* x = static_cast<const bf16*>(a.x);
  const bf16* w = static_cast<const bf16*>(a.wt);
  if (a.out_bf16)
    hipLaunchKernelGGL((arl2_linear_kernel<BN, true>), grid, dim3(kThreadsL), 0, stream, x, w, a.y, a.M, a.N, a.K, ntn);
  else
    hipLaunchKernelGGL((arl2_linear_kernel<BN, false>), grid, dim3(kThreadsL), 0, stream, x, w, a.y, a.M, a.N, a.K, ntn);
  return hipGetLastError();
}

}  // namespace

int linear_tile_n(int M, int N) {
  // the wider tile when it alone fills the chip's two work-group slots per CU
  const int64_t wide = (int64_t)((M + kBM - 1) / kBM) * ((N + 127) / 128);
  return wide >= 384 ? 128 : 64;
}

hipError_t launch_linear(const LinearArgs& a, hipStream_t stream) {
  const int parts = a.y.parts;
  if (a.K % kBK || a.N % 8 || parts < 1 || parts > kLinearMaxParts || a.N % parts || (a.N / parts) % 4)
    return hipErrorInvalidValue;
  if (a.M == 0 || a.N == 0) return hipSuccess;
  return linear_tile_n(a.M, a.N) == 128 ? launch_linear_bn<128>(a, stream) : launch_linear_bn<64>(a, stream);
}

}  // namespace arl2
