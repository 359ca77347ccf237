// Backward of the ARL2 layer: gradients through a pass (softmax branch and inter-frame read),
// through the frame's state write, and across frames through S.  "Attend Locally, Remember
// Linearly", gist.science technical summary: sections 2.1-2.2 define the forward, section 2.3
// fine-tunes the converted model end to end by distillation, through every replaced layer, with
// the per-head maps as trainable parameters.  The formulas are the chain rule of the forward:
//
//   softmax branch  P = softmax rows of scale Q K^T (recomputed: the pass kernel's plain-attention
//                   instance returns O and the rows' log-sum-exp), Dv_t = dO_t . O_t,
//                   dS = P o (dO V^T - Dv), dQ = scale dS K, dK = scale dS^T Q, dV = P^T dO
//   inter read      out += Q phi_q S:  dQ += (dO S^T) phi_q^T,  Gr = Q^T dO (summed over passes),
//                   dS_{N-1} += phi_q^T Gr,  dphi_q += Gr S^T
//   state write     S_N = alpha S + K'^T diag(beta) R, R = V' - K' S, G = dL/dS_N:
//                   X = K' G, dR = diag(beta) X, dbeta_t = x_t . r_t, dalpha = <G, S>,
//                   dK' = diag(beta) R G^T - dR S^T, dS_{N-1} += alpha G - K'^T dR,
//                   dV += dR phi_v^T, dphi_v += V^T dR; K' = U / max(|U|, eps), U = K phi_k:
//                   dU_t = (dK'_t - k'_t (k'_t . dK'_t)) / |u_t| (or dK'_t / eps), dK += dU phi_k^T,
//                   dphi_k += K^T dU
//
// Kernels.  The attention backward runs as two MFMA kernels with no atomics (bitwise
// reproducible): dK, dV per 64-key block (the keys' fragments stay in registers, query blocks
// stream through LDS) and dQ per 64-query block (key blocks stream through LDS); the scores
// are recomputed in each.  Their products run in fp16 with fp32 accumulation: the bf16 inputs
// convert exactly, and P, dS and dO round with a relative step of 2^-11.  The
// token kernels (inter read, state write) work per 128-token chunk with 16x16x32 MFMAs on
// split-bf16 operands (hi + lo, three products per term), so that their d x d products keep
// about fp32 accuracy as the forward's state write does; their sums over tokens leave the chunk
// as partials that a per-head kernel adds in a fixed order.
#include <algorithm>

#include "arl2_device.h"
#include "arl2_kernels.h"

namespace arl2 {
namespace {

constexpr int kAttnBlock = 64;  // queries or keys per work-group of the attention backward
constexpr int kTokChunk = 128;  // tokens per work-group of the token kernels (8 waves x 16)

template <int D>
struct BwdShape {
  static constexpr int KS = D / 32;          // 32-deep k-steps over features
  static constexpr int NB = D / 16;          // 16-wide blocks over features
  static constexpr int LR = D + 8;           // bf16 row pitch of staged row-major tiles
  static constexpr int LT = kAttnBlock + 8;  // bf16 row pitch of staged transposed tiles
  static constexpr int LF = D + 4;           // fp32 row pitch of the token kernels' row buffers
  static constexpr int BPW = NB * NB / 8;    // 16x16 blocks of a d x d sum per wave (8 waves)
};

// B fragment (s, nb) of a d x d matrix kept in fragment order [s][nb][lane][8]: lane l holds
// M[32 s + 8 (l / 16) + j][16 nb + l % 16].
template <int D>
__device__ __forceinline__ bf16x8 frag(const bf16* f, int s, int nb, int lane) {
  return ld_bf16x8(f + ((s * BwdShape<D>::NB + nb) * 64 + lane) * 8);
}

__device__ __forceinline__ void split8(const float (&x)[8], bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const Bf16Pair p = split_bf16(x[j]);
    hi[j] = p.hi;
    lo[j] = p.lo;
  }
}

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16h(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// 8 bf16 inputs as fp16 (exact for magnitudes in [2^-14, 65504]; smaller ones keep an absolute
// accuracy of 2^-25, larger ones become infinite and show up)
__device__ __forceinline__ f16x8 to_f16(bf16x8 x) {
  f16x8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = (f16)(float)x[j];
  return r;
}

__device__ __forceinline__ f16x8 ld_f16x8(const f16* p) {
  return __builtin_bit_cast(f16x8, *reinterpret_cast<const uint4*>(p));
}

// a b with both operands split: hi hi + hi lo + lo hi
__device__ __forceinline__ f32x4 mfma3(f32x4 c, bf16x8 ah, bf16x8 al, bf16x8 bh, bf16x8 bl) {
  c = mfma16(ah, bh, c);
  c = mfma16(ah, bl, c);
  return mfma16(al, bh, c);
}

// Keeps the scheduler from hoisting the next block's fragment loads above this point (hoisted
// loads of every block at once would need more registers than a wave has).
#define ARL2_BLOCK_FENCE() __builtin_amdgcn_sched_barrier(0)

// --- recompute helpers ----------------------------------------------------------------------

// Dv[b][h][t] = dO . O over the row's features with dO rounded to fp16 (the attention backward's
// MFMA operand, also written out), so that dS = P (dP - Dv) is the gradient of one consistent dO.
// rows = B T H rows of d values.
template <int D>
__global__ __launch_bounds__(256) void arl2_bwd_rowdot_kernel(const float* __restrict__ d_out,
                                                              const float* __restrict__ o_sm, f16* __restrict__ do_h,
                                                              float* __restrict__ dvec, int rows, int T, int H) {
  constexpr int TPR = D / 4, RPB = 256 / TPR;
  const int row = blockIdx.x * RPB + (int)threadIdx.x / TPR, li = threadIdx.x % TPR;
  float s = 0.f;
  if (row < rows) {
    const int64_t o = (int64_t)row * D + 4 * li;
    const f32x4 x = *reinterpret_cast<const f32x4*>(d_out + o);
    const f32x4 y = *reinterpret_cast<const f32x4*>(o_sm + o);
    f16x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      w[e] = (f16)x[e];
      s += (float)w[e] * y[e];  // the rounded dO, as dP = dO V^T sees it
    }
    *reinterpret_cast<f16x4*>(do_h + o) = w;
  }
#pragma unroll
  for (int m = 1; m < TPR; m <<= 1) s += __shfl_xor(s, m);
  if (row < rows && li == 0) {
    const int h = row % H, t = (row / H) % T, b = row / (H * T);
    dvec[((int64_t)b * H + h) * T + t] = s;
  }
}

// --- attention backward ---------------------------------------------------------------------
// All products in fp16 with fp32 accumulation (P, dS and dO round with a relative step of 2^-11,
// four times finer than bf16; the bf16 inputs convert exactly), at the bf16 MFMA rate.

template <typename T>
__device__ __forceinline__ f16x8 load_f16x8(const T* p) {
  if constexpr (sizeof(T) == 2 && __is_same(T, f16)) return ld_f16x8(p);
  else return to_f16(ld_bf16x8(p));
}

// One 4-row x 8-feature block of a 64-row tile of a [.][T][H][D] bf16 or fp16 tensor, staged
// through registers into LDS as fp16: row-major (pitch LR) and, when tr is not null, transposed
// (pitch LT: tr[f][r]).  Rows past T are zeros.  Block i of a tile is (row group i % 16, feature
// chunk i / 16): the 16 lanes of a group take the 16 row groups of one feature chunk, so that every
// transposed write instruction fills whole 128-byte rows of the tile.
template <int D>
struct TileBlock {
  uint4 raw[4];  // the rows' bits as loaded (bf16 or fp16): converted only when stored, so that a
                 // load issued before the current block's products is not waited for until then
  int rg, cc;
  bool on, from_bf16;
  __device__ __forceinline__ void init(int i, bool bf) {
    on = i >= 0 && i < 16 * (D / 8);
    rg = i % 16;
    cc = i / 16;
    from_bf16 = bf;
  }
  __device__ __forceinline__ void load(const void* __restrict__ src, int64_t base, int64_t rs, int r0, int T) {
    const uint16_t* p = static_cast<const uint16_t*>(src);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = r0 + 4 * rg + e;
      raw[e] = on && r < T ? *reinterpret_cast<const uint4*>(p + base + (int64_t)r * rs + 8 * cc) : make_uint4(0, 0, 0, 0);
    }
  }
  __device__ __forceinline__ void store(f16* rowm, f16* tr) const {
    if (!on) return;
    using Sh = BwdShape<D>;
    f16x8 x[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[e] = from_bf16 ? to_f16(__builtin_bit_cast(bf16x8, raw[e])) : __builtin_bit_cast(f16x8, raw[e]);
      *reinterpret_cast<f16x8*>(rowm + (4 * rg + e) * Sh::LR + 8 * cc) = x[e];
    }
    if (tr) {
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        f16x4 t;
#pragma unroll
        for (int e = 0; e < 4; ++e) t[e] = x[e][c];
        *reinterpret_cast<f16x4*>(tr + (8 * cc + c) * Sh::LT + 4 * rg) = t;
      }
    }
  }
};

// A fragment of a contraction over 32 staged rows (k-step s2 of a 64-row block) from a transposed
// tile, in the row order of two stacked 16x16 C blocks: element j <-> row 32 s2 + 16 (j / 4) +
// 4 g + j % 4, feature row f of the tile.
template <int D>
__device__ __forceinline__ f16x8 tr_frag(const f16* tr, int f, int s2, int g) {
  const f16* p = tr + f * BwdShape<D>::LT + 32 * s2 + 4 * g;
  const f16x4 a = *reinterpret_cast<const f16x4*>(p), b = *reinterpret_cast<const f16x4*>(p + 16);
  return f16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// exp2 on the transcendental unit (arguments are at most about 0 here: lse bounds every score)
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// dK, dV of 16 NW keys of one (stream, head).  NW waves, wave w owning keys 16 w .. 16 w + 15; every
// key block reads the head's whole Q and dO, so wider work-groups cut that stream (and the staging
// per wave) in proportion.  Per query block: S = Q K^T and dP = dO V^T (16x16 C blocks: lane l,
// register i <-> query 16 m + 4 (l / 16) + i, key l % 16), P = exp2(S scale log2 e - lse), dS =
// P (dP - Dv); then dV^T += dO^T P and dK^T += Q^T dS with P, dS as the B operands straight from
// the C registers.  The next block's Q and dO rows are loaded into registers while the current
// block is multiplied: with 64 NW >= 2 x the tile's blocks each thread moves one block of one
// tile, otherwise one block of each.
template <int D, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2))) void arl2_bwd_dkdv_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v, const f16* __restrict__ doh,
    const float* __restrict__ lse, const float* __restrict__ dvec, float* __restrict__ dk, float* __restrict__ dv,
    int T, int H, float scale, float scale_log2) {
  using Sh = BwdShape<D>;
  constexpr int KS = Sh::KS, NB = Sh::NB, LR = Sh::LR;
  constexpr int TILE = kAttnBlock * LR + D * Sh::LT;  // f16 elements of one staged tile (rows + transposed)
  constexpr int NBLK = 16 * (D / 8);                  // 4-row x 8-feature blocks of one tile
  constexpr bool SPLIT = 64 * NW >= 2 * NBLK;         // one block of one tile per thread
  __shared__ __align__(16) f16 lds[2 * TILE];
  __shared__ __align__(16) float lse_s[kAttnBlock], dv_s[kAttnBlock];
  f16 *qr = lds, *qtr = lds + kAttnBlock * LR, *dor = lds + TILE, *dotr = lds + TILE + kAttnBlock * LR;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l16 = lane & 15, g = lane >> 4;
  const int bh = blockIdx.y, b = bh / H, h = bh % H;
  const int64_t rs = (int64_t)H * D, base = ((int64_t)b * T * H + h) * D;
  const int key = blockIdx.x * (16 * NW) + 16 * wave + l16;
  f16x8 kf[KS], vf[KS];  // B operands: K^T, V^T columns of this wave's keys
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    kf[s] = key < T ? load_f16x8(k + base + (int64_t)key * rs + 32 * s + 8 * g) : f16x8{};
    vf[s] = key < T ? load_f16x8(v + base + (int64_t)key * rs + 32 * s + 8 * g) : f16x8{};
  }
  f32x4 dkt[NB], dvt[NB];
#pragma unroll
  for (int n = 0; n < NB; ++n) dkt[n] = dvt[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  // SPLIT: threads [0, NBLK) move Q blocks and [NBLK, 2 NBLK) dO blocks (whole waves either way),
  // through one register block; otherwise every thread moves block tid of both tiles.
  const bool mover_q = !SPLIT || tid < NBLK;
  TileBlock<D> tq, to;
  if constexpr (SPLIT) {
    tq.init(mover_q ? tid : tid - NBLK, mover_q);
  } else {
    tq.init(tid, true);
    to.init(tid, false);
  }
  float lse_r = 0.f, dv_r = 0.f;
  auto load_block = [&](int r0) {
    if constexpr (SPLIT) {
      if (mover_q) tq.load(q, base, rs, r0, T);
      else tq.load(doh, base, rs, r0, T);
    } else {
      tq.load(q, base, rs, r0, T);
      to.load(doh, base, rs, r0, T);
    }
    if (tid < kAttnBlock) {
      const int r = r0 + tid;
      lse_r = r < T ? lse[(int64_t)bh * T + r] : INFINITY;  // rows past T get P = 0
      dv_r = r < T ? dvec[(int64_t)bh * T + r] : 0.f;
    }
  };
  const int nqb = (T + kAttnBlock - 1) / kAttnBlock;
  load_block(0);
  for (int qb = 0; qb < nqb; ++qb) {
    __syncthreads();  // the previous block's LDS reads are done
    if constexpr (SPLIT) {
      if (mover_q) tq.store(qr, qtr);
      else tq.store(dor, dotr);
    } else {
      tq.store(qr, qtr);
      to.store(dor, dotr);
    }
    if (tid < kAttnBlock) {
      lse_s[tid] = lse_r;
      dv_s[tid] = dv_r;
    }
    __syncthreads();
    if (qb + 1 < nqb) load_block((qb + 1) * kAttnBlock);
    // per 32-query half s2: S and dP of its two 16-query blocks, then its share of dV^T, dK^T
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      f16x8 pb, dsb;
#pragma unroll
      for (int mm = 0; mm < 2; ++mm) {
        const int m = 2 * s2 + mm;
        f32x4 sc = {0.f, 0.f, 0.f, 0.f}, dp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const f16x8 aq = *reinterpret_cast<const f16x8*>(qr + (16 * m + l16) * LR + 32 * s + 8 * g);
          const f16x8 ao = *reinterpret_cast<const f16x8*>(dor + (16 * m + l16) * LR + 32 * s + 8 * g);
          sc = mfma16h(aq, kf[s], sc);
          dp = mfma16h(ao, vf[s], dp);
        }
        const f32x4 L = *reinterpret_cast<const f32x4*>(lse_s + 16 * m + 4 * g);
        const f32x4 Dd = *reinterpret_cast<const f32x4*>(dv_s + 16 * m + 4 * g);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = fast_exp2(sc[i] * scale_log2 - L[i]);
          pb[4 * mm + i] = (f16)p;
          dsb[4 * mm + i] = (f16)(p * (dp[i] - Dd[i]));
        }
      }
#pragma unroll
      for (int mb = 0; mb < NB; ++mb) {
        dvt[mb] = mfma16h(tr_frag<D>(dotr, 16 * mb + l16, s2, g), pb, dvt[mb]);
        dkt[mb] = mfma16h(tr_frag<D>(qtr, 16 * mb + l16, s2, g), dsb, dkt[mb]);
      }
    }
  }
  // lane l, register i: feature 16 mb + 4 (l / 16) + i of key 16 w + l % 16
  if (key < T) {
#pragma unroll
    for (int mb = 0; mb < NB; ++mb) {
      const int64_t o = base + (int64_t)key * rs + 16 * mb + 4 * g;
      *reinterpret_cast<f32x4*>(dk + o) = dkt[mb] * scale;
      *reinterpret_cast<f32x4*>(dv + o) = dvt[mb];
    }
  }
}

// dQ of 32 NQG queries of one (stream, head), with 32x32x16 MFMAs.  2 NQG waves: wave w owns
// queries 32 (w % NQG) .. +31 and the key half w / NQG of every 64-key block; the halves are added
// at the end.  Every query block reads the head's whole K and V, so wider work-groups cut that
// stream (and the staging per wave) in proportion.  Per key block: S^T = K Q^T and dP^T = V dO^T (32x32 C blocks: lane l, register i <-> key
// 8 (i / 4) + 4 (l / 32) + i % 4 of the wave's 32, query l % 32: every lane holds one query, so
// its lse and Dv are one value each), dS^T = P^T (dP^T - Dv), then dQ^T += K^T dS^T with dS^T as
// the B operand straight from the C registers (k-step h: registers 8 h .. 8 h + 7).  A 32x32x16
// product reads one 1 KB operand from LDS per 32 K multiply-adds, twice the 16x16x32 ratio.  The
// next block's K and V rows are loaded into registers while the current block is multiplied.
template <int D, int NQG>
__global__ __launch_bounds__(128 * NQG) __attribute__((amdgpu_waves_per_eu(2, 2))) void arl2_bwd_dq_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v, const f16* __restrict__ doh,
    const float* __restrict__ lse, const float* __restrict__ dvec, float* __restrict__ dq, int T, int H, float scale,
    float scale_log2) {
  using Sh = BwdShape<D>;
  constexpr int K16 = D / 16, FB = D / 32, LR = Sh::LR, LT = Sh::LT;
  constexpr int STAGE = 2 * kAttnBlock * LR + D * LT;  // f16: K rows, V rows, K transposed
  constexpr int XCH = NQG * FB * 64 * 32;              // f16: the key halves' exchange (f32x16 per lane)
  constexpr int NBLK = 16 * (D / 8);                   // 4-row x 8-feature blocks of one tile
  constexpr bool SPLIT = 128 * NQG >= 2 * NBLK;        // one block of one tile per thread
  __shared__ __align__(16) f16 lds[STAGE > XCH ? STAGE : XCH];
  f16 *kr = lds, *vr = lds + kAttnBlock * LR, *ktr = lds + 2 * kAttnBlock * LR;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, hi = lane >> 5;
  const int qh = wave % NQG, kh = wave / NQG;
  const int bh = blockIdx.y, b = bh / H, h = bh % H;
  const int64_t rs = (int64_t)H * D, base = ((int64_t)b * T * H + h) * D;
  const int qi = blockIdx.x * (32 * NQG) + 32 * qh + l32;
  f16x8 qf[K16], df[K16];  // B operands: lane l holds Q (dO) of query qi, features 16 s + 8 (l / 32) ..
#pragma unroll
  for (int s = 0; s < K16; ++s) {
    qf[s] = qi < T ? load_f16x8(q + base + (int64_t)qi * rs + 16 * s + 8 * hi) : f16x8{};
    df[s] = qi < T ? load_f16x8(doh + base + (int64_t)qi * rs + 16 * s + 8 * hi) : f16x8{};
  }
  const float L = qi < T ? lse[(int64_t)bh * T + qi] : 0.f;
  const float Dd = qi < T ? dvec[(int64_t)bh * T + qi] : 0.f;
  f32x16 dqt[FB];
#pragma unroll
  for (int n = 0; n < FB; ++n) dqt[n] = zero16();
  // SPLIT: threads [0, NBLK) move K blocks (with the transpose), [NBLK, 2 NBLK) V blocks, through
  // one register block (whole waves either way); otherwise every thread moves block tid of both.
  const bool mover_k = !SPLIT || tid < NBLK;
  TileBlock<D> tk, tv;
  if constexpr (SPLIT) {
    tk.init(mover_k ? tid : tid - NBLK, true);
  } else {
    tk.init(tid, true);
    tv.init(tid, true);
  }
  auto load_block = [&](int r0) {
    if constexpr (SPLIT) {
      tk.load(mover_k ? k : v, base, rs, r0, T);
    } else {
      tk.load(k, base, rs, r0, T);
      tv.load(v, base, rs, r0, T);
    }
  };
  const int nkb = (T + kAttnBlock - 1) / kAttnBlock;
  load_block(0);
  for (int kb = 0; kb < nkb; ++kb) {
    const int r0 = kb * kAttnBlock;
    __syncthreads();
    if constexpr (SPLIT) {
      if (mover_k) tk.store(kr, ktr);
      else tk.store(vr, nullptr);
    } else {
      tk.store(kr, ktr);
      tv.store(vr, nullptr);
    }
    __syncthreads();
    if (kb + 1 < nkb) load_block(r0 + kAttnBlock);
    f32x16 sc = zero16(), dp = zero16();
#pragma unroll
    for (int s = 0; s < K16; ++s) {
      const f16x8 ak = *reinterpret_cast<const f16x8*>(kr + (32 * kh + l32) * LR + 16 * s + 8 * hi);
      const f16x8 av = *reinterpret_cast<const f16x8*>(vr + (32 * kh + l32) * LR + 16 * s + 8 * hi);
      sc = mfma32(ak, qf[s], sc);
      dp = mfma32(av, df[s], dp);
    }
    f16x8 dsb[2];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = r0 + 32 * kh + 8 * (i / 4) + 4 * hi + i % 4;
      const float p = key < T ? fast_exp2(sc[i] * scale_log2 - L) : 0.f;
      dsb[i / 8][i % 8] = (f16)(p * (dp[i] - Dd));
    }
#pragma unroll
    for (int fb = 0; fb < FB; ++fb)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        // A: K^T rows 32 fb + l % 32, keys 32 kh + 16 hh + 8 (j / 4) + 4 (l / 32) + j % 4
        const f16* pa = ktr + (32 * fb + l32) * LT + 32 * kh + 16 * hh + 4 * hi;
        const f16x4 a0 = *reinterpret_cast<const f16x4*>(pa), a1 = *reinterpret_cast<const f16x4*>(pa + 8);
        dqt[fb] = mfma32(f16x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]}, dsb[hh], dqt[fb]);
      }
  }
  __syncthreads();
  f32x16* xs = reinterpret_cast<f32x16*>(lds) + (size_t)qh * FB * 64;
  static_assert(NQG * FB * 64 * 64 <= (int)sizeof(lds), "the exchange must fit in the staging tiles");
  if (kh) {
#pragma unroll
    for (int fb = 0; fb < FB; ++fb) xs[fb * 64 + lane] = dqt[fb];
  }
  __syncthreads();
  // lane l, register i: feature 32 fb + 8 (i / 4) + 4 (l / 32) + i % 4 of query qi
  if (!kh && qi < T) {
#pragma unroll
    for (int fb = 0; fb < FB; ++fb) {
      const f32x16 x = dqt[fb] + xs[fb * 64 + lane];
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        *reinterpret_cast<f32x4*>(dq + base + (int64_t)qi * rs + 32 * fb + 8 * g4 + 4 * hi) =
            f32x4{x[4 * g4], x[4 * g4 + 1], x[4 * g4 + 2], x[4 * g4 + 3]} * scale;
    }
  }
}

// --- fragment-order copies of d x d matrices ----------------------------------------------------

// Up to four d x d fp32 matrices per (stream, head) as split-bf16 B fragments (M or M^T).
template <int D>
__global__ __launch_bounds__(256) void arl2_bwd_frags_kernel(const BwdFragJobs jobs) {
  using Sh = BwdShape<D>;
  const BwdFragJobs::Job& jb = jobs.job[blockIdx.z];
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= Sh::KS * Sh::NB * 64) return;
  const int lane = idx & 63, nb = (idx >> 6) % Sh::NB, s = (idx >> 6) / Sh::NB;
  const int col = 16 * nb + (lane & 15), row0 = 32 * s + 8 * (lane >> 4);
  const int64_t mat = (int64_t)blockIdx.y * D * D;
  float x[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = jb.transpose ? jb.src[mat + (int64_t)col * D + row0 + j] : jb.src[mat + (int64_t)(row0 + j) * D + col];
  bf16x8 hi, lo;
  split8(x, hi, lo);
  const int64_t o = mat + (int64_t)idx * 8;
  *reinterpret_cast<bf16x8*>(static_cast<bf16*>(jb.hi) + o) = hi;
  *reinterpret_cast<bf16x8*>(static_cast<bf16*>(jb.lo) + o) = lo;
}

// The per-head maps (bf16 [H][d][d]) in fragment order: phi or phi^T (exact in bf16).
template <int D>
__global__ __launch_bounds__(256) void arl2_bwd_phi_frags_kernel(const bf16* __restrict__ phi, bf16* __restrict__ dst,
                                                                 int transpose) {
  using Sh = BwdShape<D>;
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= Sh::KS * Sh::NB * 64) return;
  const int lane = idx & 63, nb = (idx >> 6) % Sh::NB, s = (idx >> 6) / Sh::NB;
  const int col = 16 * nb + (lane & 15), row0 = 32 * s + 8 * (lane >> 4);
  const int64_t mat = (int64_t)blockIdx.y * D * D;
  bf16x8 x;
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = transpose ? phi[mat + (int64_t)col * D + row0 + j] : phi[mat + (int64_t)(row0 + j) * D + col];
  *reinterpret_cast<bf16x8*>(dst + mat + (int64_t)idx * 8) = x;
}

// --- token kernels ----------------------------------------------------------------------------

// Eight consecutive fp32 values of a row buffer as a split A fragment.
template <int D>
__device__ __forceinline__ void row_frag(const float* buf, int row, int col, bf16x8& hi, bf16x8& lo) {
  const float* p = buf + row * BwdShape<D>::LF + col;
  const f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 4);
  const float x[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  split8(x, hi, lo);
}

// A fragment over 32 rows (k-step s of a 128-row chunk) of one 16-column block of a row buffer:
// lane l holds rows 32 s + 8 (l / 16) + j of column col (a contraction over rows).
template <int D>
__device__ __forceinline__ void col_frag(const float* buf, int s, int col, int g, bf16x8& hi, bf16x8& lo) {
  float x[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = buf[(32 * s + 8 * g + j) * BwdShape<D>::LF + col];
  split8(x, hi, lo);
}

// The same over rows of a bf16 [.][T][H][D] tensor in global memory (rows past T read as zero).
__device__ __forceinline__ bf16x8 col_frag_global(const bf16* __restrict__ x, int64_t base, int64_t rs, int t0,
                                                  int T, int col) {
  bf16x8 a;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int t = t0 + j;
    a[j] = t < T ? x[base + (int64_t)t * rs + col] : (bf16)0.f;
  }
  return a;
}

__device__ __forceinline__ void store_rows(float* buf, int ld, int r0, int g, int col, const f32x4& c) {
#pragma unroll
  for (int i = 0; i < 4; ++i) buf[(r0 + 4 * g + i) * ld + col] = c[i];
}

// Sum over the 16 lanes of a lane group (the 16 columns of a C block row).
__device__ __forceinline__ float group16_sum(float x) {
  x += __shfl_xor(x, 1);
  x += __shfl_xor(x, 2);
  x += __shfl_xor(x, 4);
  x += __shfl_xor(x, 8);
  return x;
}

// Inter-frame read of one pass, per (stream, head, 128-token chunk); wave w owns tokens 16 w ..
// 16 w + 15 of the chunk.  dq += (dO S^T) phi_q^T, and the chunk's partial of Gr = Q^T dO.
template <int D>
__global__ __launch_bounds__(512) void arl2_bwd_read_kernel(const BwdTokArgs a) {
  using Sh = BwdShape<D>;
  constexpr int KS = Sh::KS, NB = Sh::NB, LF = Sh::LF, BPW = Sh::BPW;
  __shared__ __align__(16) float ybuf[kTokChunk * LF];  // Y = dO S^T rows (each wave its own)
  __shared__ __align__(16) float dbuf[kTokChunk * LF];  // the chunk's dO rows
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, l16 = lane & 15, g = lane >> 4;
  const int T = a.T, H = a.H, nch = (T + kTokChunk - 1) / kTokChunk;
  const int chunk = blockIdx.x % nch, bh = blockIdx.x / nch, b = bh / H, h = bh % H;
  const int64_t rs = (int64_t)H * D, base = ((int64_t)b * T * H + h) * D, mat = (int64_t)bh * D * D;
  const int t0 = chunk * kTokChunk, r0 = 16 * wave, ta = t0 + r0 + l16;
  const bf16* st_hi = static_cast<const bf16*>(a.st_hi) + mat;
  const bf16* st_lo = static_cast<const bf16*>(a.st_lo) + mat;
  const bf16* pqt = static_cast<const bf16*>(a.pqt) + (int64_t)h * D * D;

  bf16x8 xh[KS], xl[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    f32x4 u = {0.f, 0.f, 0.f, 0.f}, w = {0.f, 0.f, 0.f, 0.f};
    if (ta < T) {
      const float* p = a.d_out + base + (int64_t)ta * rs + 32 * s + 8 * g;
      u = *reinterpret_cast<const f32x4*>(p);
      w = *reinterpret_cast<const f32x4*>(p + 4);
    }
    float* dst = dbuf + (r0 + l16) * LF + 32 * s + 8 * g;
    *reinterpret_cast<f32x4*>(dst) = u;
    *reinterpret_cast<f32x4*>(dst + 4) = w;
    const float x[8] = {u[0], u[1], u[2], u[3], w[0], w[1], w[2], w[3]};
    split8(x, xh[s], xl[s]);
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) y = mfma3(y, xh[s], xl[s], frag<D>(st_hi, s, nb, lane), frag<D>(st_lo, s, nb, lane));
    store_rows(ybuf, LF, r0, g, 16 * nb + l16, y);
    if (nb & 1) ARL2_BLOCK_FENCE();  // two blocks' loads in flight
  }
  __syncthreads();
#pragma unroll
  for (int s = 0; s < KS; ++s) row_frag<D>(ybuf, r0 + l16, 32 * s + 8 * g, xh[s], xl[s]);
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const bf16x8 f = frag<D>(pqt, s, nb, lane);
      c = mfma16(xh[s], f, c);
      c = mfma16(xl[s], f, c);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + r0 + 4 * g + i;
      if (t < T) a.dq[base + (int64_t)t * rs + 16 * nb + l16] += c[i];
    }
    if (nb & 1) ARL2_BLOCK_FENCE();  // two blocks' loads in flight
  }
  // Gr partial: wave w owns the 16x16 blocks (mb, nb0 .. nb0 + BPW - 1) of Q^T dO
  const int mb = wave * BPW / NB, nb0 = wave * BPW % NB;
  f32x4 p[BPW];
#pragma unroll
  for (int n = 0; n < BPW; ++n) p[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  const bf16* qg = static_cast<const bf16*>(a.q);
#pragma unroll
  for (int s = 0; s < kTokChunk / 32; ++s) {
    const bf16x8 aq = col_frag_global(qg, base, rs, t0 + 32 * s + 8 * g, T, 16 * mb + l16);
#pragma unroll
    for (int n = 0; n < BPW; ++n) {
      bf16x8 bh_, bl_;
      col_frag<D>(dbuf, s, 16 * (nb0 + n) + l16, g, bh_, bl_);
      p[n] = mfma16(aq, bh_, p[n]);
      p[n] = mfma16(aq, bl_, p[n]);
    }
    ARL2_BLOCK_FENCE();
  }
  float* part = a.part + ((int64_t)bh * nch + chunk) * D * D;
#pragma unroll
  for (int n = 0; n < BPW; ++n)
#pragma unroll
    for (int i = 0; i < 4; ++i) part[(16 * mb + 4 * g + i) * D + 16 * (nb0 + n) + l16] = p[n][i];
}

// State write of one frame, per (stream, head, 128-token chunk); wave w owns tokens 16 w ..
// 16 w + 15.  Per token: U = k phi_k, K' = U / max(|U|, eps), V' = v phi_v, R = V' - K' S,
// X3 = R G^T, X = K' G, dbeta = x . r, dR = beta X, dK' = beta X3 - dR S^T, dU; dv += dR phi_v^T,
// dk += dU phi_k^T.  Chunk partials (in this order): K'^T dR, V^T dR, K^T dU.
template <int D>
__global__ __launch_bounds__(512) void arl2_bwd_write_kernel(const BwdTokArgs a) {
  using Sh = BwdShape<D>;
  constexpr int KS = Sh::KS, NB = Sh::NB, LF = Sh::LF, BPW = Sh::BPW;
  __shared__ __align__(16) float abuf[kTokChunk * LF];  // K' rows, later dU rows
  __shared__ __align__(16) float bbuf[kTokChunk * LF];  // R rows, later dR rows
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, l16 = lane & 15, g = lane >> 4;
  const int T = a.T, H = a.H, nch = (T + kTokChunk - 1) / kTokChunk;
  const int chunk = blockIdx.x % nch, bh = blockIdx.x / nch, b = bh / H, h = bh % H;
  const int64_t rs = (int64_t)H * D, base = ((int64_t)b * T * H + h) * D, mat = (int64_t)bh * D * D;
  const int64_t hmat = (int64_t)h * D * D;
  const int t0 = chunk * kTokChunk, r0 = 16 * wave, ta = t0 + r0 + l16;
  const bf16* kg = static_cast<const bf16*>(a.k);
  const bf16* vg = static_cast<const bf16*>(a.v);
  auto M = [&](const void* p, int64_t off) { return static_cast<const bf16*>(p) + off; };
  const bf16 *s_hi = M(a.s_hi, mat), *s_lo = M(a.s_lo, mat), *st_hi = M(a.st_hi, mat), *st_lo = M(a.st_lo, mat);
  const bf16 *g_hi = M(a.g_hi, mat), *g_lo = M(a.g_lo, mat), *gt_hi = M(a.gt_hi, mat), *gt_lo = M(a.gt_lo, mat);
  const bf16 *phik = M(a.phik, hmat), *phiv = M(a.phiv, hmat), *phikt = M(a.phikt, hmat), *phivt = M(a.phivt, hmat);

  // this wave's token rows as A operands (bf16 inputs: exact)
  bf16x8 ka[KS], va[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    ka[s] = ta < T ? ld_bf16x8(kg + base + (int64_t)ta * rs + 32 * s + 8 * g) : zero_bf16x8();
    va[s] = ta < T ? ld_bf16x8(vg + base + (int64_t)ta * rs + 32 * s + 8 * g) : zero_bf16x8();
  }
  // C registers: lane l, register i <-> token r0 + 4 (l / 16) + i, feature 16 nb + l % 16
  f32x4 kp[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    f32x4 u = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) u = mfma16(ka[s], frag<D>(phik, s, nb, lane), u);
    kp[nb] = u;
    if (nb & 1) ARL2_BLOCK_FENCE();  // two blocks' loads in flight
  }
  float nrm[4], inv[4], bet[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float ss = 0.f;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) ss += kp[nb][i] * kp[nb][i];
    nrm[i] = sqrtf(group16_sum(ss));
    inv[i] = 1.f / fmaxf(nrm[i], a.knorm_eps);
    const int t = t0 + r0 + 4 * g + i;
    bet[i] = t < T ? a.beta[((int64_t)b * T + t) * H + h] : 0.f;
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) kp[nb][i] *= inv[i];
    store_rows(abuf, LF, r0, g, 16 * nb + l16, kp[nb]);
    if (nb & 1) ARL2_BLOCK_FENCE();  // two blocks' loads in flight
  }
  __syncthreads();
  bf16x8 kh[KS], kl[KS];  // K' as split A fragments
#pragma unroll
  for (int s = 0; s < KS; ++s) row_frag<D>(abuf, r0 + l16, 32 * s + 8 * g, kh[s], kl[s]);
  // R = V' - K' S with V' = v phi_v, into bbuf
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    f32x4 c = {0.f, 0.f, 0.f, 0.f}, w = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      w = mfma16(va[s], frag<D>(phiv, s, nb, lane), w);
      c = mfma3(c, kh[s], kl[s], frag<D>(s_hi, s, nb, lane), frag<D>(s_lo, s, nb, lane));
    }
    store_rows(bbuf, LF, r0, g, 16 * nb + l16, w - c);
    if (nb & 1) ARL2_BLOCK_FENCE();  // two blocks' loads in flight
  }
  __syncthreads();
  // X3 = R G^T (becomes dK')
  f32x4 dkp[NB];
  {
    bf16x8 rh[KS], rl[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) row_frag<D>(bbuf, r0 + l16, 32 * s + 8 * g, rh[s], rl[s]);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) c = mfma3(c, rh[s], rl[s], frag<D>(gt_hi, s, nb, lane), frag<D>(gt_lo, s, nb, lane));
      dkp[nb] = c;
      if (nb & 1) ARL2_BLOCK_FENCE();  // two blocks' loads in flight
    }
  }
  // X = K' G; dbeta = x . r; dR = beta X
  f32x4 dr[NB];
  float db[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) c = mfma3(c, kh[s], kl[s], frag<D>(g_hi, s, nb, lane), frag<D>(g_lo, s, nb, lane));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      db[i] += c[i] * bbuf[(r0 + 4 * g + i) * LF + 16 * nb + l16];  // x . r
      dr[nb][i] = bet[i] * c[i];
    }
    if (nb & 1) ARL2_BLOCK_FENCE();  // two blocks' loads in flight
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float s = group16_sum(db[i]);
    const int t = t0 + r0 + 4 * g + i;
    if (l16 == 0 && t < T) a.dbeta[((int64_t)b * T + t) * H + h] = s;
  }
  __syncthreads();  // every wave has read its R fragments before dR replaces R
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) store_rows(bbuf, LF, r0, g, 16 * nb + l16, dr[nb]);
  __syncthreads();
  bf16x8 dh[KS], dl[KS];  // dR as split A fragments
#pragma unroll
  for (int s = 0; s < KS; ++s) row_frag<D>(bbuf, r0 + l16, 32 * s + 8 * g, dh[s], dl[s]);
  // dK' = beta X3 - dR S^T; dU; dv += dR phi_v^T
  float cdot[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) c = mfma3(c, dh[s], dl[s], frag<D>(st_hi, s, nb, lane), frag<D>(st_lo, s, nb, lane));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      dkp[nb][i] = bet[i] * dkp[nb][i] - c[i];
      cdot[i] += abuf[(r0 + 4 * g + i) * LF + 16 * nb + l16] * dkp[nb][i];  // k' . dK'
    }
    if (nb & 1) ARL2_BLOCK_FENCE();  // two blocks' loads in flight
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float c = group16_sum(cdot[i]);  // (every lane shuffles; the branch only selects)
    cdot[i] = nrm[i] > a.knorm_eps ? c : 0.f;
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      dkp[nb][i] = (dkp[nb][i] - abuf[(r0 + 4 * g + i) * LF + 16 * nb + l16] * cdot[i]) * inv[i];  // dU
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const bf16x8 f = frag<D>(phivt, s, nb, lane);
      c = mfma16(dh[s], f, c);
      c = mfma16(dl[s], f, c);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + r0 + 4 * g + i;
      if (t < T) a.dv[base + (int64_t)t * rs + 16 * nb + l16] += c[i];
    }
    if (nb & 1) ARL2_BLOCK_FENCE();  // two blocks' loads in flight
  }
  // chunk sums K'^T dR and V^T dR: wave w owns the 16x16 blocks (mb, nb0 .. nb0 + BPW - 1)
  const int mb = wave * BPW / NB, nb0 = wave * BPW % NB;
  // partial sum p of 16-column block nb at [bh][p][nb][chunk][row][16]: each (p, nb) strip of all
  // chunks is contiguous for the per-head kernel that adds them
  auto pidx = [&](int p, int nb, int row) -> int64_t {
    return ((((int64_t)bh * 3 + p) * NB + nb) * nch + chunk) * D * 16 + row * 16 + l16;
  };
  {
    f32x4 p[BPW];
#pragma unroll
    for (int n = 0; n < BPW; ++n) p[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < kTokChunk / 32; ++s) {
      bf16x8 ah, al;
      col_frag<D>(abuf, s, 16 * mb + l16, g, ah, al);
#pragma unroll
      for (int n = 0; n < BPW; ++n) {
        bf16x8 bh_, bl_;
        col_frag<D>(bbuf, s, 16 * (nb0 + n) + l16, g, bh_, bl_);
        p[n] = mfma3(p[n], ah, al, bh_, bl_);
        ARL2_BLOCK_FENCE();
      }
    }
#pragma unroll
    for (int n = 0; n < BPW; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) a.part[pidx(0, nb0 + n, 16 * mb + 4 * g + i)] = p[n][i];
#pragma unroll
    for (int n = 0; n < BPW; ++n) p[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < kTokChunk / 32; ++s) {
      const bf16x8 av = col_frag_global(vg, base, rs, t0 + 32 * s + 8 * g, T, 16 * mb + l16);
#pragma unroll
      for (int n = 0; n < BPW; ++n) {
        bf16x8 bh_, bl_;
        col_frag<D>(bbuf, s, 16 * (nb0 + n) + l16, g, bh_, bl_);
        p[n] = mfma16(av, bh_, p[n]);
        p[n] = mfma16(av, bl_, p[n]);
        ARL2_BLOCK_FENCE();
      }
    }
#pragma unroll
    for (int n = 0; n < BPW; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) a.part[pidx(1, nb0 + n, 16 * mb + 4 * g + i)] = p[n][i];
  }
  __syncthreads();  // K' is no longer read: dU replaces it
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) store_rows(abuf, LF, r0, g, 16 * nb + l16, dkp[nb]);
  __syncthreads();
  // dk += dU phi_k^T
#pragma unroll
  for (int s = 0; s < KS; ++s) row_frag<D>(abuf, r0 + l16, 32 * s + 8 * g, dh[s], dl[s]);
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const bf16x8 f = frag<D>(phikt, s, nb, lane);
      c = mfma16(dh[s], f, c);
      c = mfma16(dl[s], f, c);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + r0 + 4 * g + i;
      if (t < T) a.dk[base + (int64_t)t * rs + 16 * nb + l16] += c[i];
    }
    if (nb & 1) ARL2_BLOCK_FENCE();  // two blocks' loads in flight
  }
  // chunk sum K^T dU
  {
    f32x4 p3[BPW];
#pragma unroll
    for (int n = 0; n < BPW; ++n) p3[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < kTokChunk / 32; ++s) {
      const bf16x8 ak = col_frag_global(kg, base, rs, t0 + 32 * s + 8 * g, T, 16 * mb + l16);
#pragma unroll
      for (int n = 0; n < BPW; ++n) {
        bf16x8 bh_, bl_;
        col_frag<D>(abuf, s, 16 * (nb0 + n) + l16, g, bh_, bl_);
        p3[n] = mfma16(ak, bh_, p3[n]);
        p3[n] = mfma16(ak, bl_, p3[n]);
      }
      ARL2_BLOCK_FENCE();
    }
#pragma unroll
    for (int n = 0; n < BPW; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) a.part[pidx(2, nb0 + n, 16 * mb + 4 * g + i)] = p3[n][i];
  }
}

// --- sums over chunks, frames' end ---------------------------------------------------------------

// gr[bh] (+)= sum over chunks of the read partials, in chunk order.
__global__ __launch_bounds__(256) void arl2_bwd_gsum_kernel(const float* __restrict__ part, float* __restrict__ gr,
                                                            int dd, int nch, int first) {
  const int bh = blockIdx.y, i4 = blockIdx.x * 256 + threadIdx.x;
  if (4 * i4 >= dd) return;
  const f32x4* p = reinterpret_cast<const f32x4*>(part + (int64_t)bh * nch * dd) + i4;
  f32x4 s = first ? f32x4{0.f, 0.f, 0.f, 0.f} : reinterpret_cast<const f32x4*>(gr + (int64_t)bh * dd)[i4];
  for (int c = 0; c < nch; ++c) s += p[(int64_t)c * (dd / 4)];
  reinterpret_cast<f32x4*>(gr + (int64_t)bh * dd)[i4] = s;
}

// End of a frame's backward, per (head, 16 x 16 output tile), streams in order:
//   dS_{N-1} = alpha G - sum_chunks K'^T dR + phi_q^T Gr,   dalpha = <G, S_{N-1}>,
//   dphi_q += Gr S^T,  dphi_k += sum_chunks K^T dU,  dphi_v += sum_chunks V^T dR.
// Thread t owns element (t / 16, t % 16) of the tile; the strips of Gr, S and phi_q that the
// d-long dot products read come through LDS.
template <int D>
__global__ __launch_bounds__(256) void arl2_bwd_frame_kernel(const BwdFrameArgs a) {
  constexpr int NB = D / 16, CP = 17, RP = D + 4;
  __shared__ float gcol[D * CP];  // Gr[k][16 ct + c]
  __shared__ float phc[D * CP];   // phi_q[k][16 rt + r]
  __shared__ __align__(16) float grow[16 * RP];  // Gr[16 rt + r][k]
  __shared__ __align__(16) float srow[16 * RP];  // S[16 ct + c][k]
  __shared__ float red[256];
  const int ct = blockIdx.x, rt = blockIdx.y, h = blockIdx.z, tid = threadIdx.x;
  const int r = tid / 16, c = tid % 16, row = 16 * rt + r, col = 16 * ct + c;
  const int64_t dd = (int64_t)D * D;
  if (a.gr) {
    const bf16* ph = static_cast<const bf16*>(a.phi_q) + h * dd;
    for (int i = tid; i < 16 * D; i += 256) phc[(i / 16) * CP + i % 16] = (float)ph[(i / 16) * D + 16 * rt + i % 16];
  }
  float aq = 0.f, ak = 0.f, av = 0.f;
  for (int b = 0; b < a.B; ++b) {
    const int64_t bh = (int64_t)b * a.H + h;
    const float* G = a.g + bh * dd;
    const float* S = a.s_prev + bh * dd;
    // the 16-column strips of the three sums, chunk after chunk ([bh][sum][strip][chunk][row][16])
    const float* part = a.part + ((bh * 3) * NB + ct) * a.chunks * D * 16 + row * 16 + c;
    const int64_t pstride = (int64_t)NB * a.chunks * D * 16;  // from one sum to the next
    float ds = a.alpha[bh] * G[row * D + col];
#pragma unroll 8
    for (int ch = 0; ch < a.chunks; ++ch) {
      const float* p = part + (int64_t)ch * D * 16;
      ds -= p[0];
      av += p[pstride];
      ak += p[2 * pstride];
    }
    if (a.gr) {
      const float* gr = a.gr + bh * dd;
      __syncthreads();  // the previous stream's strips are no longer read
#pragma unroll
      for (int it = 0; it < 16 * D / 256; ++it) {
        const int i = tid + 256 * it;
        gcol[(i / 16) * CP + i % 16] = gr[(i / 16) * D + 16 * ct + i % 16];
        grow[(i / D) * RP + i % D] = gr[(16 * rt + i / D) * D + i % D];
        srow[(i / D) * RP + i % D] = S[(16 * ct + i / D) * D + i % D];
      }
      __syncthreads();
#pragma unroll 8
      for (int k = 0; k < D; ++k) {
        ds += phc[k * CP + r] * gcol[k * CP + c];   // (phi_q^T Gr)[row][col]
        aq += grow[r * RP + k] * srow[c * RP + k];  // (Gr S^T)[row][col]
      }
    }
    a.ds_prev[bh * dd + row * D + col] = ds;
    if (ct == 0 && rt == 0) {  // dalpha over the whole matrix (all loads of a thread in flight at once)
      float s = 0.f;
#pragma unroll
      for (int it = 0; it < D * D / 1024; ++it) {
        const int i = tid + 256 * it;
        const f32x4 x = reinterpret_cast<const f32x4*>(G)[i], y = reinterpret_cast<const f32x4*>(S)[i];
        s += x[0] * y[0] + x[1] * y[1] + x[2] * y[2] + x[3] * y[3];
      }
      red[tid] = s;
      __syncthreads();
      for (int w = 128; w > 0; w >>= 1) {
        if (tid < w) red[tid] += red[tid + w];
        __syncthreads();
      }
      if (tid == 0) a.dalpha[bh] = red[0];
    }
  }
  const int64_t o = (int64_t)h * dd + row * D + col;
  a.dphi_q[o] += aq;
  a.dphi_k[o] += ak;
  a.dphi_v[o] += av;
}

// dst[i] = src ? src[i] : 0 (n4 float4 elements); a kernel rather than a memset node, so that the
// calls stay correct inside a captured graph.
__global__ __launch_bounds__(256) void arl2_bwd_fill_kernel(float* __restrict__ dst, const float* __restrict__ src,
                                                            int64_t n4) {
  for (int64_t i = blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256)
    reinterpret_cast<f32x4*>(dst)[i] = src ? reinterpret_cast<const f32x4*>(src)[i] : f32x4{0.f, 0.f, 0.f, 0.f};
}

template <int D>
hipError_t launch_bwd_pass_d(const BwdPassArgs& a, hipStream_t stream) {
  const int BH = a.B * a.H;
  const int rows = a.B * a.T * a.H, rpb = 256 / (D / 4);
  hipLaunchKernelGGL(arl2_bwd_rowdot_kernel<D>, dim3((rows + rpb - 1) / rpb), dim3(256), 0, stream, a.d_out, a.o_sm,
                     static_cast<f16*>(a.do_h), a.dvec, rows, a.T, a.H);
  const bf16* q = static_cast<const bf16*>(a.tok.q);
  const bf16* k = static_cast<const bf16*>(a.tok.k);
  const bf16* v = static_cast<const bf16*>(a.tok.v);
  const f16* doh = static_cast<const f16*>(a.do_h);
  constexpr int kDkdvWaves = 8;
  const int nkb = (a.T + 16 * kDkdvWaves - 1) / (16 * kDkdvWaves);
  hipLaunchKernelGGL((arl2_bwd_dkdv_kernel<D, kDkdvWaves>), dim3(nkb, BH), dim3(64 * kDkdvWaves), 0, stream, q, k, v,
                     doh, a.lse, a.dvec, a.tok.dk, a.tok.dv, a.T, a.H, a.scale, a.scale_log2);
  constexpr int kDqGroups = 4;  // 32-query groups per work-group (times two key halves: 8 waves)
  const int nqb = (a.T + 32 * kDqGroups - 1) / (32 * kDqGroups);
  hipLaunchKernelGGL((arl2_bwd_dq_kernel<D, kDqGroups>), dim3(nqb, BH), dim3(128 * kDqGroups), 0, stream, q, k, v, doh,
                     a.lse, a.dvec, a.tok.dq, a.T, a.H, a.scale, a.scale_log2);
  const int nch = (a.T + kTokChunk - 1) / kTokChunk;
  hipLaunchKernelGGL(arl2_bwd_read_kernel<D>, dim3(nch * BH), dim3(512), 0, stream, a.tok);
  hipLaunchKernelGGL(arl2_bwd_gsum_kernel, dim3((D * D / 4 + 255) / 256, BH), dim3(256), 0, stream, a.tok.part, a.gr,
                     D * D, nch, a.gr_first ? 1 : 0);
  return hipGetLastError();
}

template <int D>
hipError_t launch_bwd_frags_d(const BwdFragJobs& j, int BH, int n_jobs, hipStream_t stream) {
  hipLaunchKernelGGL(arl2_bwd_frags_kernel<D>, dim3((D * D / 8 + 255) / 256, BH, n_jobs), dim3(256), 0, stream, j);
  return hipGetLastError();
}

template <int D>
hipError_t launch_bwd_commit_d(const BwdTokArgs& t, const BwdFrameArgs& f, hipStream_t stream) {
  const int nch = (t.T + kTokChunk - 1) / kTokChunk;
  hipLaunchKernelGGL(arl2_bwd_write_kernel<D>, dim3(nch * t.B * t.H), dim3(512), 0, stream, t);
  hipLaunchKernelGGL(arl2_bwd_frame_kernel<D>, dim3(D / 16, D / 16, t.H), dim3(256), 0, stream, f);
  return hipGetLastError();
}

template <int D>
hipError_t launch_bwd_phi_d(const bf16* phi, bf16* dst, int H, bool transpose, hipStream_t stream) {
  hipLaunchKernelGGL(arl2_bwd_phi_frags_kernel<D>, dim3((D * D / 8 + 255) / 256, H), dim3(256), 0, stream, phi, dst,
                     transpose ? 1 : 0);
  return hipGetLastError();
}

}  // namespace

int bwd_chunks(int T) { return (T + kTokChunk - 1) / kTokChunk; }

hipError_t launch_bwd_fill(float* dst, const float* src, size_t n, hipStream_t stream) {
  if (n % 4) return hipErrorInvalidValue;
  const int64_t n4 = (int64_t)(n / 4);
  const int blocks = (int)std::min<int64_t>((n4 + 255) / 256, 2048);
  if (blocks > 0) hipLaunchKernelGGL(arl2_bwd_fill_kernel, dim3(blocks), dim3(256), 0, stream, dst, src, n4);
  return hipGetLastError();
}

hipError_t launch_bwd_pass(int d, const BwdPassArgs& a, hipStream_t stream) {
  switch (d) {
    case 64: return launch_bwd_pass_d<64>(a, stream);
    case 128: return launch_bwd_pass_d<128>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bwd_frags(int d, const BwdFragJobs& j, int BH, int n_jobs, hipStream_t stream) {
  if (n_jobs < 1 || n_jobs > 4) return hipErrorInvalidValue;
  switch (d) {
    case 64: return launch_bwd_frags_d<64>(j, BH, n_jobs, stream);
    case 128: return launch_bwd_frags_d<128>(j, BH, n_jobs, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bwd_commit(int d, const BwdTokArgs& t, const BwdFrameArgs& f, hipStream_t stream) {
  switch (d) {
    case 64: return launch_bwd_commit_d<64>(t, f, stream);
    case 128: return launch_bwd_commit_d<128>(t, f, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bwd_phi_frags(int d, const void* phi, void* dst, int H, bool transpose, hipStream_t stream) {
  switch (d) {
    case 64: return launch_bwd_phi_d<64>(static_cast<const bf16*>(phi), static_cast<bf16*>(dst), H, transpose, stream);
    case 128: return launch_bwd_phi_d<128>(static_cast<const bf16*>(phi), static_cast<bf16*>(dst), H, transpose, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace arl2
