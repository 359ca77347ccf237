// State write of the ARL2 layer, once per frame after the clean pass:
//   S_N = alpha S_{N-1} + K'^T diag(beta) (V' - K' S_{N-1}),
//   K' = rows of K phi_k scaled to unit length,  V' = V phi_v
// ("Attend Locally, Remember Linearly", gist.science technical summary, section 2.1: the
// gated update and the per-head 1x1 maps; section 2.2: one write per frame, after the clean
// pass, with every token's residual taken against the same S_{N-1}).
//
// The per-chunk partial sums P_c = K'_c^T diag(beta_c) (V'_c - K'_c S_{N-1}) run as extra
// work-groups of the clean pass's launch (arl2_write_partial.h).  arl2_commit_reduce: one
// work-group per (stream, head, 16 value columns) adds alpha S_{N-1} and the partials in a
// fixed order (bitwise reproducible), stores S_N, and prepares what the next frame reads:
// -S_N as MFMA B fragments (for the next write's K' S product) and (phi_q S_N)^T (for the
// passes' inter read).
//
// Precision: K', S and the residual enter MFMAs as bf16 hi + lo pairs (x = hi + lo to about
// 16 mantissa bits; products hi*hi + hi*lo + lo*hi), because a single bf16 rounding of any of
// them costs more than the state tolerance over a long stream.  K, V and the maps are exact
// in bf16 and need no split.
#include "arl2_device.h"
#include "arl2_kernels.h"

namespace arl2 {
namespace {

template <int D>
struct CommitShape {
  static constexpr int DP = D < 32 ? 32 : D;
  static constexpr int NB = DP / 16;    // 16-column stripes of S (one work-group each)
  static constexpr int FB = DP / 16;    // 16-blocks of the state write's partials and -S fragments
  static constexpr int KS32 = DP / 32;  // 32-deep k-steps (the -S fragments, and W = phi_q S)
};

constexpr int kReduceThreads = 512;

// s_prev and s_new may be the same buffer (the layer updates S in place): each element of S_new is
// stored by the thread that loaded the same element of s_prev, and no other thread reads it.
//
// One work-group per (stream, head, 16 value columns): a 16-column stripe keeps the chunk sum
// spread over DP / 16 work-groups per head (the partials are read once, and one CU's load path
// is what bounds each work-group), and it is one 16x16 MFMA block wide for W.
template <int D>
__global__ __launch_bounds__(kReduceThreads) void arl2_commit_reduce_kernel(
    const float* s_prev, const float* __restrict__ alpha, const float* __restrict__ alpha_part,
    const float* __restrict__ alpha_bias, int n_ablk, int T, const float* __restrict__ partial,
    int chunks, const bf16* __restrict__ pq, float* s_new, bf16* __restrict__ sneg_hi,
    bf16* __restrict__ sneg_lo, bf16* __restrict__ wt_hi, bf16* __restrict__ wt_lo, int H) {
  using S = CommitShape<D>;
  constexpr int DP = S::DP, FB = S::FB, KS32 = S::KS32;
  constexpr int V4 = DP * 4;  // float4 groups of the 16-column stripe
  static_assert(V4 <= kReduceThreads, "one float4 group per thread");
  static_assert(FB <= kReduceThreads / 64, "one W block per wave");
  constexpr int kUnroll = 16;  // chunk loads in flight per thread (a 2048-token frame in one round)
  __shared__ float tile[DP][17];  // S_new[:, 16 nb .. 16 nb + 15], padded against bank conflicts

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nb = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int64_t bh = (int64_t)b * H + h;
  // phi_q rows of this wave's 16-row W block (A fragments of 16x16x32 MFMAs: lane l holds row
  // l % 16, k 32 st + 8 (l / 16) .. + 7), loaded first: they depend on nothing.
  const bf16* pqh = pq + (int64_t)h * DP * D;
  bf16x8 af[KS32];
  if (wave < FB) {
#pragma unroll
    for (int st = 0; st < KS32; ++st) {
      const int k0 = 32 * st + 8 * (lane >> 4);
      af[st] = k0 < D ? ld_bf16x8(pqh + (16 * wave + (lane & 15)) * D + k0) : bf16x8{};
    }
  }
  float a = alpha ? alpha[bh] : 1.f;
  if (alpha_part) {  // the per-frame decay from the gate projection: sigmoid(mean logit + bias)
    // every wave adds the block partials the same way: lane l the blocks l, l + 64, .. in
    // order, then a fixed butterfly over the lanes (bitwise the same result in every wave)
    float z = 0.f;
    for (int j = lane; j < n_ablk; j += 64) z += alpha_part[((int64_t)b * n_ablk + j) * H + h];
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) z += __shfl_xor(z, m);
    a = 1.f / (1.f + expf(-(z / (float)T + alpha_bias[h])));
  }
  constexpr int kStride = DP * DP / 4;  // float4 between consecutive chunks

  // S_new = alpha S_prev + sum_c P_c, chunks added in a fixed order.  The partials are stored
  // as 16 x 16 blocks in 16x16 MFMA C-register order ([row block][column block][register i]
  // [lane l] = P[16 rb + 4 (l / 16) + i][16 cb + l % 16]); thread e < V4 owns row block e / 64,
  // register (e / 16) % 4 and lanes 4 (e % 16) .. + 3 of column block nb: 4 adjacent columns.
  const int e = tid;
  const int rb = e >> 6, ri = (e >> 4) & 3, q = e & 15;
  const int row = 16 * rb + 4 * (q >> 2) + ri, c4 = 4 * (q & 3), col = 16 * nb + c4;
  const bool ok = e < V4 && row < D && col < D;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  const f32x4* pp = reinterpret_cast<const f32x4*>(partial + bh * chunks * DP * DP + ((rb * FB + nb) * 4 + ri) * 64 + 4 * q);
  if (ok) acc = a * *reinterpret_cast<const f32x4*>(s_prev + (bh * D + row) * D + col);
  for (int c = 0; c < chunks; c += kUnroll) {
    f32x4 x[kUnroll];
#pragma unroll
    for (int w = 0; w < kUnroll; ++w)
      x[w] = (ok && c + w < chunks) ? pp[(int64_t)(c + w) * kStride] : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kUnroll; ++w)
      if (c + w < chunks) acc += x[w];
  }
  if (e < V4) {
    if (ok) *reinterpret_cast<f32x4*>(s_new + (bh * D + row) * D + col) = acc;
#pragma unroll
    for (int c = 0; c < 4; ++c) tile[row][c4 + c] = acc[c];  // zeros outside d x d
  }
  __syncthreads();

  // -S_new as 16x16x32 B fragments for the next write's K' S: fragment (k-step ks, value block
  // nb), lane l, element j <-> -S[32 ks + 16 (j / 4) + 4 (l / 16) + j % 4][16 nb + l % 16] (the
  // row order of two stacked 16x16 C blocks, in which K' enters as the A operand).
  if (tid < KS32 * 64) {
    const int ks = tid >> 6;
    bf16x8 hi, lo;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const Bf16Pair sp = split_bf16(-tile[32 * ks + 16 * (j >> 2) + 4 * (lane >> 4) + (j & 3)][lane & 15]);
      hi[j] = sp.hi;
      lo[j] = sp.lo;
    }
    const int64_t fo = ((bh * KS32 + ks) * FB + nb) * 64 + lane;
    reinterpret_cast<bf16x8*>(sneg_hi)[fo] = hi;
    reinterpret_cast<bf16x8*>(sneg_lo)[fo] = lo;
  }

  // W = phi_q S_new on this column stripe, wave w the rows 16 w .. 16 w + 15 (16x16x32 MFMAs;
  // B lane l holds S rows 32 st + 8 (l / 16) .. + 7 of column l % 16, split hi + lo).  Stored
  // transposed and split, W^T[j][i], as the pass kernel stages it: k-step planes
  // [i / 16][j][i % 16], so that every kilobyte it loads is contiguous.
  if (wave < FB) {
    f32x4 w = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < KS32; ++st) {
      bf16x8 bhi, blo;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const Bf16Pair sp = split_bf16(tile[32 * st + 8 * (lane >> 4) + j][lane & 15]);
        bhi[j] = sp.hi;
        blo[j] = sp.lo;
      }
      w = mfma16(af[st], bhi, w);
      w = mfma16(af[st], blo, w);
    }
    const int i0 = 16 * wave + 4 * (lane >> 4);  // C lane l, register r: W[i0 + r][16 nb + l % 16]
    if (i0 < D) {
      bf16x4 hi, lo;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const Bf16Pair sp = split_bf16(w[r]);
        hi[r] = sp.hi;
        lo[r] = sp.lo;
      }
      const int64_t o = bh * DP * D + ((int64_t)(i0 >> 4) * DP + 16 * nb + (lane & 15)) * 16 + (i0 & 15);
      *reinterpret_cast<bf16x4*>(wt_hi + o) = hi;
      *reinterpret_cast<bf16x4*>(wt_lo + o) = lo;
    }
  }
}

template <int D>
__global__ void arl2_prep_maps_kernel(const bf16* __restrict__ phi_q, const bf16* __restrict__ phi_k,
                                      const bf16* __restrict__ phi_v, bf16* __restrict__ pq, bf16* __restrict__ pkt,
                                      bf16* __restrict__ pvt, bf16* __restrict__ pqt, int H) {
  constexpr int DP = CommitShape<D>::DP;
  // pq [H][DP][D]: phi_q with zero rows past d
  const int64_t nq = (int64_t)H * DP * D;
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < nq; e += (int64_t)gridDim.x * blockDim.x) {
    const int col = e % D, row = (e / D) % DP;
    const int64_t hh = e / ((int64_t)DP * D);
    pq[e] = row < D ? phi_q[(hh * D + row) * D + col] : (bf16)0.f;
  }
  // pkt, pvt [H][DP][DP]: phi^T with zero rows and columns past d
  const int64_t nt = (int64_t)H * DP * DP;
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < nt; e += (int64_t)gridDim.x * blockDim.x) {
    const int col = e % DP, row = (e / DP) % DP;
    const int64_t hh = e / ((int64_t)DP * DP);
    const bool ok = row < D && col < D;
    const int64_t srt = (hh * D + col) * D + row;  // phi[h][col][row]
    pkt[e] = ok ? phi_k[srt] : (bf16)0.f;
    pvt[e] = ok ? phi_v[srt] : (bf16)0.f;
    pqt[e] = ok ? phi_q[srt] : (bf16)0.f;
  }
}

template <int D>
hipError_t launch_reduce_d(const CommitReduceArgs& a, hipStream_t stream) {
  dim3 grid(CommitShape<D>::NB, a.H, a.B);
  hipLaunchKernelGGL((arl2_commit_reduce_kernel<D>), grid, dim3(kReduceThreads), 0, stream, a.s_prev, a.alpha,
                     a.alpha_part, a.alpha_bias, a.n_ablk, a.T, a.partial, a.chunks, static_cast<const bf16*>(a.pq), a.s_new, static_cast<bf16*>(a.sneg_hi),
                     static_cast<bf16*>(a.sneg_lo), static_cast<bf16*>(a.wt_hi), static_cast<bf16*>(a.wt_lo),
                     a.H);
  return hipGetLastError();
}

template <int D>
hipError_t launch_prep_d(const PrepMapsArgs& a, hipStream_t stream) {
  const int64_t n = (int64_t)a.H * CommitShape<D>::DP * CommitShape<D>::DP;
  const int blocks = (int)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096);
  hipLaunchKernelGGL((arl2_prep_maps_kernel<D>), dim3(blocks), dim3(256), 0, stream,
                     static_cast<const bf16*>(a.phi_q), static_cast<const bf16*>(a.phi_k),
                     static_cast<const bf16*>(a.phi_v), static_cast<bf16*>(a.pq), static_cast<bf16*>(a.pkt),
                     static_cast<bf16*>(a.pvt), static_cast<bf16*>(a.pqt), a.H);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_commit_reduce(int d, const CommitReduceArgs& a, hipStream_t stream) {
  switch (d) {
    case 16: return launch_reduce_d<16>(a, stream);
    case 64: return launch_reduce_d<64>(a, stream);
    case 128: return launch_reduce_d<128>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_prep_maps(int d, const PrepMapsArgs& a, hipStream_t stream) {
  switch (d) {
    case 16: return launch_prep_d<16>(a, stream);
    case 64: return launch_prep_d<64>(a, stream);
    case 128: return launch_prep_d<128>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace arl2
