// State write of the ARL2 layer, once per frame after the clean pass:
//   S_N = alpha S_{N-1} + K'^T diag(beta) (V' - K' S_{N-1}),
//   K' = rows of K phi_k scaled to unit length,  V' = V phi_v
// ("Attend Locally, Remember Linearly", gist.science technical summary, section 2.1: the
// gated update and the per-head 1x1 maps; section 2.2: one write per frame, after the clean
// pass, with every token's residual taken against the same S_{N-1}).
//
// Two launches.  arl2_commit_partial: one work-group per (stream, head, 128-token chunk)
// forms the chunk's K', V' and residual in registers and reduces K'^T diag(beta) R over the
// chunk into a d x d partial.  arl2_commit_reduce: one work-group per (stream, head, 32
// value columns) adds alpha S_{N-1} and the partials in a fixed order (bitwise
// reproducible), stores S_N, and prepares what the next frame reads: -S_N as MFMA B
// fragments (for the next write's K' S product) and (phi_q S_N)^T (for the passes' inter
// read).
//
// Precision: K', S and the residual enter MFMAs as bf16 hi + lo pairs (x = hi + lo to about
// 16 mantissa bits; products hi*hi + hi*lo + lo*hi), because a single bf16 rounding of any of
// them costs more than the state tolerance over a long stream.  K, V and the maps are exact
// in bf16 and need no split.
#include "arl2_device.h"
#include "arl2_kernels.h"

namespace arl2 {
namespace {

constexpr int kThreads = 256;

template <int D>
struct CommitShape {
  static constexpr int DP = D < 32 ? 32 : D;
  static constexpr int KS = D / 16;   // k-steps over input features
  static constexpr int MB = DP / 32;  // 32-blocks over key features (rows of S)
  static constexpr int NB = DP / 32;  // 32-blocks over value features (columns of S)
};

typedef __attribute__((address_space(3))) void lds_void;

// LDS of the partial kernel.  Phase 1 reads the operands shared by all waves as MFMA
// fragments (1 KB per fragment, 16 bytes per lane): phi_k^T and phi_v^T [block][k-step] and
// -S hi/lo [k-step][block].  Phase 2 reuses the space for the fragments whose contraction runs
// over tokens: [wave][block][k-step of 16 tokens][hi/lo][lane].
template <int D>
struct PartialSmem {
  static constexpr int MB = CommitShape<D>::MB, KS = CommitShape<D>::KS;
  union {
    struct {
      bf16x8 pk[MB][KS][64];
      bf16x8 pv[MB][KS][64];
      bf16x8 shi[KS][MB][64];
      bf16x8 slo[KS][MB][64];
    } op;
    struct {
      bf16x8 kfrag[4][MB][2][2][64];
      bf16x8 rfrag[4][MB][2][2][64];
    } fr;
  };
  float beta[kCommitChunk];
  float inv_norm[kCommitChunk];
};

// Wait until at most N of this wave's vector memory loads are in flight (N < 64; loads complete
// in issue order).  The count's low 4 bits and high 2 bits sit apart in the instruction.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// 16 bytes per lane from the buffer straight into LDS at lds + 16 * lane (lds wave-uniform).
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, void* lds, int off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, off, 0, 0, 0);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, bytes, 0x00020000);
}

template <int D>
__global__ __launch_bounds__(kThreads) void arl2_commit_partial_kernel(
    const bf16* __restrict__ k, const bf16* __restrict__ v, const float* __restrict__ beta,
    const bf16* __restrict__ pkt, const bf16* __restrict__ pvt, const bf16* __restrict__ sneg_hi,
    const bf16* __restrict__ sneg_lo, float* __restrict__ partial, int T, int H, float eps) {
  using S = CommitShape<D>;
  constexpr int DP = S::DP, KS = S::KS, MB = S::MB, NB = S::NB;
  __shared__ PartialSmem<D> sm;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int chunk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int chunks = gridDim.x;
  const int64_t rs = (int64_t)H * D;
  const int64_t base = ((int64_t)b * T * H + h) * D;
  const int t0 = chunk * kCommitChunk;

  if (tid < kCommitChunk) {
    const int t = t0 + tid;
    sm.beta[tid] = t < T ? beta[((int64_t)b * T + t) * H + h] : 0.f;
  }

  // This lane's token for the A/B fragments of K and V (row-major, 8 features per lane).
  const int tok = t0 + 32 * wave + (lane & 31);
  const int64_t sb = ((int64_t)b * H + h) * (KS * NB * 64);  // fragment index base

  // Loads in the order the products need them, each group waited for just before its first
  // use (when the operand fragments deal evenly over the 4 waves; otherwise all at once):
  // phi_k^T fragments and this lane's row of K; phi_v^T and the row of V; -S hi / lo.
  // Operands go straight into LDS (4 * MB * KS fragments of 1 KB); K and V come through
  // buffer loads, so rows past the frame read as zeros and every wave issues the same loads.
  constexpr int NFRAG = MB * KS;
  constexpr bool EVEN = NFRAG % 4 == 0;
  constexpr int NF = NFRAG / 4;  // fragments per wave and operand when EVEN
  const __amdgpu_buffer_rsrc_t rk = rsrc(pkt + (int64_t)h * DP * D, DP * D * 2);
  const __amdgpu_buffer_rsrc_t rv = rsrc(pvt + (int64_t)h * DP * D, DP * D * 2);
  const __amdgpu_buffer_rsrc_t rh = rsrc(sneg_hi + sb * 8, KS * NB * 1024);
  const __amdgpu_buffer_rsrc_t rl = rsrc(sneg_lo + sb * 8, KS * NB * 1024);
  const int slice_bytes = (int)(((int64_t)(T - 1) * rs + D) * 2);
  const __amdgpu_buffer_rsrc_t rkin = rsrc(k + base, slice_bytes);
  const __amdgpu_buffer_rsrc_t rvin = rsrc(v + base, slice_bytes);
  const int map_lane = ((lane & 31) * D + 8 * (lane >> 5)) * 2;  // row l % 32, features 8 (l / 32) ..
  const int row_lane = (int)(tok * rs * 2) + 16 * (lane >> 5);      // this lane's token row, 8 features
  bf16x8 kf[KS], vf[KS];
  for (int f = wave; f < NFRAG; f += 4)
    dma16(rk, &sm.op.pk[f / KS][f % KS][0], map_lane + (32 * (f / KS) * D + 16 * (f % KS)) * 2);
#pragma unroll
  for (int st = 0; st < KS; ++st)
    kf[st] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rkin, row_lane + 32 * st, 0, 0));
  for (int f = wave; f < NFRAG; f += 4)
    dma16(rv, &sm.op.pv[f / KS][f % KS][0], map_lane + (32 * (f / KS) * D + 16 * (f % KS)) * 2);
#pragma unroll
  for (int st = 0; st < KS; ++st)
    vf[st] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rvin, row_lane + 32 * st, 0, 0));
  for (int f = wave; f < NFRAG; f += 4) {
    dma16(rh, &sm.op.shi[0][0][0] + 64 * f, f * 1024 + lane * 16);
    dma16(rl, &sm.op.slo[0][0][0] + 64 * f, f * 1024 + lane * 16);
  }
  wait_vmcnt<EVEN ? 3 * NF + KS : 0>();  // phi_k^T (every wave's share, after the barrier) and K
  __syncthreads();

  // K'^T = phi_k^T K^T: rows = key features, lane column = token.
  f32x16 kt[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    kt[mb] = zero16();
#pragma unroll
    for (int st = 0; st < KS; ++st) kt[mb] = mfma32(sm.op.pk[mb][st][lane], kf[st], kt[mb]);
  }

  // Unit rows: this lane holds half of its token's features; the other half is in lane ^ 32.
  float ss = 0.f;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) ss = fmaf(kt[mb][i], kt[mb][i], ss);
  ss += other_half(ss, lane);
  const float inv = 1.f / fmaxf(sqrtf(ss), eps);
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) kt[mb][i] *= inv;
  if (lane < 32) sm.inv_norm[32 * wave + lane] = inv;

  // R = V' - K' S: first V phi_v, then K' (-S) with split operands accumulated on top.
  // A fragment of K' for k-step st: register 8 (st % 2) + j of block st / 2.
  f32x16 r[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) r[nb] = zero16();
  wait_vmcnt<EVEN ? 2 * NF : 0>();  // phi_v^T and V
  __syncthreads();
#pragma unroll
  for (int st = 0; st < KS; ++st)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) r[nb] = mfma32(vf[st], sm.op.pv[nb][st][lane], r[nb]);
  wait_vmcnt<0>();  // -S hi / lo
  __syncthreads();
#pragma unroll
  for (int st = 0; st < KS; ++st) {
    bf16x8 khi, klo;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const Bf16Pair sp = split_bf16(kt[st >> 1][8 * (st & 1) + j]);
      khi[j] = sp.hi;
      klo[j] = sp.lo;
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const bf16x8 shi = sm.op.shi[st][nb][lane], slo = sm.op.slo[st][nb][lane];
      r[nb] = mfma32(khi, shi, r[nb]);
      r[nb] = mfma32(khi, slo, r[nb]);
      r[nb] = mfma32(klo, shi, r[nb]);
    }
  }

  // K' = K phi_k (rows = tokens, lane column = key feature): the operands of K'^T in swapped
  // MFMA slots; it is the A operand of the token contraction below.
  f32x16 kk[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    kk[mb] = zero16();
#pragma unroll
    for (int st = 0; st < KS; ++st) kk[mb] = mfma32(kf[st], sm.op.pk[mb][st][lane], kk[mb]);
  }
  __syncthreads();  // beta and inverse norms of all waves are in LDS; the operands are no longer read

  // beta R and K' (rows = tokens) carry a token per register; scale and store both as
  // fragments whose contraction runs over the wave's 32 tokens.
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int tl = 32 * wave + c_row(i, lane);
    const float bt = sm.beta[tl], in = sm.inv_norm[tl];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) r[nb][i] *= bt;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) kk[mb][i] *= in;
  }
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int ts = 0; ts < 2; ++ts) {
      bf16x8 hi, lo;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const Bf16Pair sp = split_bf16(kk[mb][8 * ts + j]);
        hi[j] = sp.hi;
        lo[j] = sp.lo;
      }
      sm.fr.kfrag[wave][mb][ts][0][lane] = hi;
      sm.fr.kfrag[wave][mb][ts][1][lane] = lo;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const Bf16Pair sp = split_bf16(r[mb][8 * ts + j]);
        hi[j] = sp.hi;
        lo[j] = sp.lo;
      }
      sm.fr.rfrag[wave][mb][ts][0][lane] = hi;
      sm.fr.rfrag[wave][mb][ts][1][lane] = lo;
    }
  __syncthreads();

  // P_chunk = sum over the chunk's tokens of K'^T (beta R): wave w owns key-feature blocks
  // w, w + 4, ...; token blocks are summed in a fixed order.
  const int nsrc = min(4, (T - t0 + 31) / 32);
  for (int mb = wave; mb < MB; mb += 4) {
    f32x16 p[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) p[nb] = zero16();
    for (int src = 0; src < nsrc; ++src)
#pragma unroll
      for (int ts = 0; ts < 2; ++ts) {
        const bf16x8 ah = sm.fr.kfrag[src][mb][ts][0][lane], al = sm.fr.kfrag[src][mb][ts][1][lane];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const bf16x8 bh = sm.fr.rfrag[src][nb][ts][0][lane], bl = sm.fr.rfrag[src][nb][ts][1][lane];
          p[nb] = mfma32(ah, bh, p[nb]);
          p[nb] = mfma32(ah, bl, p[nb]);
          p[nb] = mfma32(al, bh, p[nb]);
        }
      }
    float* pb = partial + (((int64_t)b * H + h) * chunks + chunk) * DP * DP;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) pb[(32 * mb + c_row(i, lane)) * DP + 32 * nb + (lane & 31)] = p[nb][i];
  }
}

constexpr int kReduceThreads = 512;

template <int D>
__global__ __launch_bounds__(kReduceThreads) void arl2_commit_reduce_kernel(
    const float* __restrict__ s_prev, const float* __restrict__ alpha, const float* __restrict__ partial,
    int chunks, const bf16* __restrict__ pq, float* __restrict__ s_new, bf16* __restrict__ sneg_hi,
    bf16* __restrict__ sneg_lo, bf16* __restrict__ wt_hi, bf16* __restrict__ wt_lo, int H) {
  using S = CommitShape<D>;
  constexpr int DP = S::DP, KS = S::KS, MB = S::MB, NB = S::NB;
  constexpr int V4 = DP * 8;  // float4 groups of the 32-column block
  constexpr int PER = (V4 + kReduceThreads - 1) / kReduceThreads;
  constexpr int kUnroll = 8;  // chunk loads in flight per group
  __shared__ float tile[DP][33];  // S_new[:, 32 nb .. 32 nb + 31], padded against bank conflicts

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nb = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int64_t bh = (int64_t)b * H + h;
  const float a = alpha ? alpha[bh] : 1.f;
  constexpr int kStride = DP * DP / 4;  // float4 between consecutive chunks

  // S_new = alpha S_prev + sum_c P_c, chunks added in a fixed order.  Each thread owns PER
  // float4 groups (4 adjacent columns of a row) and keeps all their loads of a round in flight.
  f32x4 acc[PER];
  bool ok[PER];
  const f32x4* pp[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int e = tid + kReduceThreads * u;
    const int row = e >> 3, col = 32 * nb + (e & 7) * 4;
    ok[u] = e < V4 && row < D && col < D;
    acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    pp[u] = reinterpret_cast<const f32x4*>(partial + bh * chunks * DP * DP + row * DP + col);
    if (ok[u]) acc[u] = a * *reinterpret_cast<const f32x4*>(s_prev + (bh * D + row) * D + col);
  }
  for (int c = 0; c < chunks; c += kUnroll) {
    f32x4 x[PER][kUnroll];
#pragma unroll
    for (int u = 0; u < PER; ++u)
#pragma unroll
      for (int w = 0; w < kUnroll; ++w)
        x[u][w] = (ok[u] && c + w < chunks) ? pp[u][(int64_t)(c + w) * kStride] : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < PER; ++u)
#pragma unroll
      for (int w = 0; w < kUnroll; ++w)
        if (c + w < chunks) acc[u] += x[u][w];
  }
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int e = tid + kReduceThreads * u;
    if (e >= V4) continue;
    const int row = e >> 3, c4 = (e & 7) * 4, col = 32 * nb + c4;
    if (ok[u]) *reinterpret_cast<f32x4*>(s_new + (bh * D + row) * D + col) = acc[u];
#pragma unroll
    for (int q = 0; q < 4; ++q) tile[row][c4 + q] = acc[u][q];
  }
  __syncthreads();

  // -S_new as B fragments for the next write: k-step st, element j <-> key feature
  // 16 st + 8 (j / 4) + 4 (l / 32) + j % 4 (the row order of a C block), lane column = value feature.
  for (int e = tid; e < KS * 64; e += kReduceThreads) {
    const int st = e >> 6, l = e & 63;
    bf16x8 hi, lo;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const Bf16Pair sp = split_bf16(-tile[16 * st + 8 * (j >> 2) + 4 * (l >> 5) + (j & 3)][l & 31]);
      hi[j] = sp.hi;
      lo[j] = sp.lo;
    }
    const int64_t fo = ((bh * KS + st) * NB + nb) * 64 + l;
    reinterpret_cast<bf16x8*>(sneg_hi)[fo] = hi;
    reinterpret_cast<bf16x8*>(sneg_lo)[fo] = lo;
  }

  // W = phi_q S_new on this column block; stored transposed and split, W^T[j][i], as the pass
  // kernel stages it: k-step planes [i / 16][j][i % 16], so that every kilobyte it loads is
  // contiguous.
  const bf16* pqh = pq + (int64_t)h * DP * D;
  for (int mb = wave; mb < MB; mb += kReduceThreads / 64) {
    f32x16 w = zero16();
#pragma unroll
    for (int st = 0; st < KS; ++st) {
      const bf16x8 af = ld_bf16x8(pqh + (32 * mb + (lane & 31)) * D + 16 * st + 8 * (lane >> 5));
      bf16x8 bhi, blo;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const Bf16Pair sp = split_bf16(tile[16 * st + 8 * (lane >> 5) + j][lane & 31]);
        bhi[j] = sp.hi;
        blo[j] = sp.lo;
      }
      w = mfma32(af, bhi, w);
      w = mfma32(af, blo, w);
    }
    const int col = 32 * nb + (lane & 31);  // value feature j = row of W^T
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int i0 = 32 * mb + 8 * g + 4 * (lane >> 5);
      if (i0 < D) {
        bf16x4 hi, lo;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const Bf16Pair sp = split_bf16(w[4 * g + e]);
          hi[e] = sp.hi;
          lo[e] = sp.lo;
        }
        const int64_t o = bh * DP * D + ((int64_t)(i0 >> 4) * DP + col) * 16 + (i0 & 15);
        *reinterpret_cast<bf16x4*>(wt_hi + o) = hi;
        *reinterpret_cast<bf16x4*>(wt_lo + o) = lo;
      }
    }
  }
}

template <int D>
__global__ void arl2_prep_maps_kernel(const bf16* __restrict__ phi_q, const bf16* __restrict__ phi_k,
                                      const bf16* __restrict__ phi_v, bf16* __restrict__ pq, bf16* __restrict__ pkt,
                                      bf16* __restrict__ pvt, int H) {
  constexpr int DP = CommitShape<D>::DP;
  const int64_t n = (int64_t)H * DP * D;
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < n; e += (int64_t)gridDim.x * blockDim.x) {
    const int col = e % D, row = (e / D) % DP;
    const int64_t hh = e / ((int64_t)DP * D);
    const bool ok = row < D;
    const int64_t src = (hh * D + row) * D + col;   // phi[h][row][col]
    const int64_t srt = (hh * D + col) * D + row;   // phi[h][col][row]
    pq[e] = ok ? phi_q[src] : (bf16)0.f;
    pkt[e] = ok ? phi_k[srt] : (bf16)0.f;
    pvt[e] = ok ? phi_v[srt] : (bf16)0.f;
  }
}

template <int D>
hipError_t launch_partial_d(const CommitPartialArgs& a, hipStream_t stream) {
  dim3 grid(commit_chunks(a.T), a.H, a.B);
  hipLaunchKernelGGL((arl2_commit_partial_kernel<D>), grid, dim3(kThreads), 0, stream,
                     static_cast<const bf16*>(a.k), static_cast<const bf16*>(a.v), a.beta,
                     static_cast<const bf16*>(a.pkt), static_cast<const bf16*>(a.pvt),
                     static_cast<const bf16*>(a.sneg_hi), static_cast<const bf16*>(a.sneg_lo), a.partial, a.T,
                     a.H, a.knorm_eps);
  return hipGetLastError();
}

template <int D>
hipError_t launch_reduce_d(const CommitReduceArgs& a, hipStream_t stream) {
  dim3 grid(CommitShape<D>::NB, a.H, a.B);
  hipLaunchKernelGGL((arl2_commit_reduce_kernel<D>), grid, dim3(kReduceThreads), 0, stream, a.s_prev, a.alpha,
                     a.partial, a.chunks, static_cast<const bf16*>(a.pq), a.s_new, static_cast<bf16*>(a.sneg_hi),
                     static_cast<bf16*>(a.sneg_lo), static_cast<bf16*>(a.wt_hi), static_cast<bf16*>(a.wt_lo),
                     a.H);
  return hipGetLastError();
}

template <int D>
hipError_t launch_prep_d(const PrepMapsArgs& a, hipStream_t stream) {
  const int64_t n = (int64_t)a.H * CommitShape<D>::DP * D;
  const int blocks = (int)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096);
  hipLaunchKernelGGL((arl2_prep_maps_kernel<D>), dim3(blocks), dim3(256), 0, stream,
                     static_cast<const bf16*>(a.phi_q), static_cast<const bf16*>(a.phi_k),
                     static_cast<const bf16*>(a.phi_v), static_cast<bf16*>(a.pq), static_cast<bf16*>(a.pkt),
                     static_cast<bf16*>(a.pvt), a.H);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_commit_partial(int d, const CommitPartialArgs& a, hipStream_t stream) {
  switch (d) {
    case 16: return launch_partial_d<16>(a, stream);
    case 64: return launch_partial_d<64>(a, stream);
    case 128: return launch_partial_d<128>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

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
