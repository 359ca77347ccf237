// Fused per-pass kernel of the ARL2 layer:
//   out = softmax(Q K^T * scale) V + Q W,   W = phi_q S_{N-1}
// ("Attend Locally, Remember Linearly", gist.science technical summary, section 2.1:
// intra-frame softmax branch and inter-frame output Q' S_{N-1} with Q' = Q phi_q; section
// 2.2: every token of the frame reads the same pre-update state).  Q' S = Q (phi_q S) by
// associativity; W is formed once per frame by the state-write kernels, so a pass only
// adds a Q x W product to the attention accumulator.
//
// Work decomposition: one work-group of 4 waves per (stream, head, 128-query tile); wave w
// owns 32 query rows.  Scores are computed transposed, S^T = K Q^T, so that every lane holds
// one query row and 32 of the tile's keys: the softmax max needs one cross-lane exchange
// (lanes l and l ^ 32), the sums none until the end.  The output is accumulated transposed,
// O^T += V^T P^T, again one query row per lane, so the online-softmax rescale is a per-lane
// multiply.  K and V tiles of 64 keys are double-buffered in LDS; V stays row-major and its
// transposed operand comes from ds_read_b64_tr_b16.
#include "arl2_device.h"
#include "arl2_kernels.h"

namespace arl2 {
namespace {

constexpr int kQTile = 128;   // query rows per work-group
constexpr int kKV = 64;       // keys per LDS tile
constexpr int kThreads = 256;

template <int D>
struct FwdShape {
  static constexpr int DP = D < 32 ? 32 : D;  // padded feature rows of the O^T blocks
  static constexpr int KS = D / 16;          // 16-wide k-steps over features
  static constexpr int MB = DP / 32;         // 32-row blocks over output features
  static constexpr int LDW = DP + 8;         // LDS row stride in bf16 (16 bytes of padding)
  static constexpr int CPR = D / 8;          // 16-byte chunks per token row
  static constexpr int NCH = (kKV * CPR + kThreads - 1) / kThreads;  // chunks per thread
};

template <int D, bool OUT_BF16>
__global__ __launch_bounds__(kThreads, 2) void arl2_fwd_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ wt_hi, const bf16* __restrict__ wt_lo, void* __restrict__ out,
    int T, int H, float scale_log2) {
  using S = FwdShape<D>;
  constexpr int DP = S::DP, KS = S::KS, MB = S::MB, LDW = S::LDW, CPR = S::CPR, NCH = S::NCH;

  __shared__ __attribute__((aligned(16))) bf16 ks[2][kKV * LDW];
  __shared__ __attribute__((aligned(16))) bf16 vs[2][kKV * LDW];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int h = blockIdx.y, b = blockIdx.z;
  const int64_t rs = (int64_t)H * D;  // elements between consecutive tokens
  const int64_t base = ((int64_t)b * T * H + h) * D;
  const bf16* qb = q + base;
  const bf16* kb = k + base;
  const bf16* vb = v + base;

  if (D < DP) {  // padded feature columns are read as zeros and never written again
    for (int i = tid; i < 2 * kKV * LDW; i += kThreads) {
      (&ks[0][0])[i] = (bf16)0.f;
      (&vs[0][0])[i] = (bf16)0.f;
    }
    __syncthreads();
  }

  // This lane's query row, as B fragments of Q^T (k-step st covers features 16 st .. 16 st + 15).
  const int qrow = blockIdx.x * kQTile + wave * 32 + (lane & 31);
  bf16x8 qf[KS];
#pragma unroll
  for (int st = 0; st < KS; ++st)
    qf[st] = qrow < T ? ld_bf16x8(qb + qrow * rs + 16 * st + 8 * (lane >> 5)) : zero_bf16x8();

  uint4 kreg[NCH], vreg[NCH];
  auto load_tile = [&](int tile) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int chunk = tid + c * kThreads;
      const int key = tile * kKV + chunk / CPR;
      const int col = (chunk % CPR) * 8;
      const bool ok = (chunk < kKV * CPR) && key < T;
      kreg[c] = ok ? *reinterpret_cast<const uint4*>(kb + key * rs + col) : make_uint4(0, 0, 0, 0);
      vreg[c] = ok ? *reinterpret_cast<const uint4*>(vb + key * rs + col) : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int chunk = tid + c * kThreads;
      if (chunk < kKV * CPR) {
        const int off = (chunk / CPR) * LDW + (chunk % CPR) * 8;
        *reinterpret_cast<uint4*>(&ks[buf][off]) = kreg[c];
        *reinterpret_cast<uint4*>(&vs[buf][off]) = vreg[c];
      }
    }
  };

  f32x16 acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = zero16();
  float m_run = -INFINITY;  // running row max (raw score units), same in lanes l and l ^ 32
  float l_run = 0.f;        // this lane's share of the running row sum

  const int ntiles = (T + kKV - 1) / kKV;
  load_tile(0);
  store_tile(0);
  __syncthreads();

  // Transposed-read addressing for V^T fragments (see lds_tr_pair).
  const int tr_src = lane & 15, tr_grp = lane >> 4;
  const int tr_row = 4 * (tr_grp >> 1) + (tr_src >> 2);
  const int tr_col = 16 * (tr_grp & 1) + 4 * (tr_src & 3);

  for (int tile = 0; tile < ntiles; ++tile) {
    const int buf = tile & 1;
    if (tile + 1 < ntiles) load_tile(tile + 1);

    // S^T for the tile's two 32-key blocks: rows = keys, this lane's column = its query row.
    f32x16 s[2];
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
      s[kb2] = zero16();
      const bf16* krow = &ks[buf][(32 * kb2 + (lane & 31)) * LDW + 8 * (lane >> 5)];
#pragma unroll
      for (int st = 0; st < KS; ++st) {
        bf16x8 a = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(krow + 16 * st));
        s[kb2] = mfma32(a, qf[st], s[kb2]);
      }
    }
    if ((tile + 1) * kKV > T) {  // ragged last tile: keys beyond the frame do not exist
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (tile * kKV + 32 * kb2 + c_row(i, lane) >= T) s[kb2][i] = -INFINITY;
    }

    float mx = s[0][0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[0][i]);
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[1][i]);
    mx = fmaxf(mx, other_half(mx, lane));
    const float m_new = fmaxf(m_run, mx);
    const float corr = __builtin_amdgcn_exp2f((m_run - m_new) * scale_log2);
    const float mc = m_new * scale_log2;
    m_run = m_new;

    // P^T as B fragments: k-step ks4 = 16 keys, element j <-> register 8 (ks4 % 2) + j of block ks4 / 2.
    bf16x8 pf[4];
    float rsum = 0.f;
#pragma unroll
    for (int ks4 = 0; ks4 < 4; ++ks4)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[ks4 >> 1][8 * (ks4 & 1) + j], scale_log2, -mc));
        rsum += p;
        pf[ks4][j] = (bf16)p;
      }
    l_run = l_run * corr + rsum;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mb][i] *= corr;

    // O^T += V^T P^T: A fragment (feature row, 8 keys in the P^T row order) from two
    // transposed reads of the row-major V tile.
#pragma unroll
    for (int ks4 = 0; ks4 < 4; ++ks4) {
      const bf16* p0 = &vs[buf][(16 * ks4 + tr_row) * LDW + tr_col];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        bf16x8 a = lds_tr_pair(p0 + 32 * mb, p0 + 8 * LDW + 32 * mb);
        acc[mb] = mfma32(a, pf[ks4], acc[mb]);
      }
    }

    if (tile + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // Normalise the softmax branch, then add Q W = Q (phi_q S) with W^T split in two bf16 terms.
  const float inv = 1.f / (l_run + other_half(l_run, lane));
  const int64_t wbase = ((int64_t)b * H + h) * DP * D;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[mb][i] *= inv;
    const int64_t off = wbase + (32 * mb + (lane & 31)) * D + 8 * (lane >> 5);
#pragma unroll
    for (int st = 0; st < KS; ++st) {
      acc[mb] = mfma32(ld_bf16x8(wt_hi + off + 16 * st), qf[st], acc[mb]);
      acc[mb] = mfma32(ld_bf16x8(wt_lo + off + 16 * st), qf[st], acc[mb]);
    }
  }

  if (qrow < T) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * mb + 8 * g + 4 * (lane >> 5);
        if (d < D) {
          const int64_t o = base + qrow * rs + d;
          if (OUT_BF16) {
            bf16x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = (bf16)acc[mb][4 * g + e];
            *reinterpret_cast<bf16x4*>(reinterpret_cast<bf16*>(out) + o) = w;
          } else {
            f32x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = acc[mb][4 * g + e];
            *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + o) = w;
          }
        }
      }
  }
}

template <int D>
hipError_t launch_fwd_d(const FwdArgs& a, hipStream_t stream) {
  dim3 grid((a.T + kQTile - 1) / kQTile, a.H, a.B);
  const bf16* q = static_cast<const bf16*>(a.q);
  const bf16* k = static_cast<const bf16*>(a.k);
  const bf16* v = static_cast<const bf16*>(a.v);
  const bf16* wh = static_cast<const bf16*>(a.wt_hi);
  const bf16* wl = static_cast<const bf16*>(a.wt_lo);
  if (a.out_bf16)
    hipLaunchKernelGGL((arl2_fwd_kernel<D, true>), grid, dim3(kThreads), 0, stream, q, k, v, wh, wl, a.out,
                       a.T, a.H, a.scale_log2);
  else
    hipLaunchKernelGGL((arl2_fwd_kernel<D, false>), grid, dim3(kThreads), 0, stream, q, k, v, wh, wl, a.out,
                       a.T, a.H, a.scale_log2);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd(int d, const FwdArgs& a, hipStream_t stream) {
  switch (d) {
    case 16: return launch_fwd_d<16>(a, stream);
    case 64: return launch_fwd_d<64>(a, stream);
    case 128: return launch_fwd_d<128>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace arl2
