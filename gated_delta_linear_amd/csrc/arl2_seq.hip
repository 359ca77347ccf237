// Token-level (sequential) access variant of the ARL2 layer: the alternative to frame-level
// access that the pages reject ("Attend Locally, Remember Linearly", gist.science technical
// summary, section 2.2: every token of a frame reads the same pre-update state; section 4:
// ablations), built as an A/B.  Per (stream, head) and frame, with Q' = Q phi_q,
// K' = unit_rows(K phi_k), V' = V phi_v and the frame's tokens in order:
//   o_t = softmax branch_t + q'_t S^(t-1),   S^(0) = S_{N-1},
//   S^(t) = S^(t-1) + beta_t k'_t^T (v'_t - k'_t S^(t-1)),   clean pass: S_N = S^(T) - (1 - alpha) S_{N-1}.
//
// Computed in chunks of 64 tokens in the WY form of the delta rule: with A = I +
// strictly_lower(diag(beta) K' K'^T) and T = A^-1, per chunk U = T diag(beta) V', W = T diag(beta) K',
//   U_hat = U - W S,   O = Q' S + strictly_lower(Q' K'^T) U_hat,   S <- S + K'^T U_hat.
// Two kernels:
//   arl2_seq_prep: one work-group per (stream, head, chunk), all chunks in parallel: the maps, row
//     norms, L, the triangular solve for T (one wave, forward substitution in fp32), U, -W, the
//     masked Q' K'^T, and the operands the scan needs, written to a workspace as MFMA fragments.
//   arl2_seq_scan: one work-group per (stream, head, 64 value columns), the chunks in order: each
//     wave keeps a 16-column slice of S in registers (the value columns of the recurrence are
//     independent) and runs the three products per chunk; the chunk operands shared by the slices
//     are staged in LDS, the next chunk's while the current one computes.  Writes O_inter and, for
//     the clean pass, S_N.  The pass kernel then adds the softmax branch.
// All products use 16x16x32 bf16 MFMAs with both operands as hi + lo pairs (three products), as
// the frame-level write does; the C blocks of one product are the operands of the next in the
// stacked-row order (element j <-> row 16 (j / 4) + 4 (l / 16) + j % 4 of a 32-deep step).
#include "arl2_device.h"
#include "arl2_kernels.h"

namespace arl2 {
namespace {

constexpr int kSeqChunk = 64;  // tokens per chunk
typedef __attribute__((address_space(3))) void seq_lds_void;

template <int D>
struct SeqShape {
  static constexpr int KS = D / 32;        // 32-deep k-steps over features
  static constexpr int FB = D / 16;        // 16-wide blocks over features
  static constexpr int LD = D + 4;         // fp32 row stride of the token-row tiles in LDS
  static constexpr int LT = kSeqChunk + 4; // fp32 row stride of the 64 x 64 tiles
  // workspace of one chunk, in 1-KB units (one MFMA fragment, or one fp32 C block)
  static constexpr int NW_KB = 4 * KS * 2;  // -W A-fragments [token block][feature k-step][hi, lo]
  static constexpr int QF_KB = 4 * KS * 2;  // Q' A-fragments, same layout
  static constexpr int MF_KB = 4 * 2 * 2;   // M = strictly_lower(Q' K'^T) A-fragments [token block][token k-step][hi, lo]
  static constexpr int KT_KB = FB * 2 * 2;  // K'^T A-fragments [feature block][token k-step][hi, lo]
  static constexpr int UC_KB = 4 * FB;      // U C blocks [token block][feature block] fp32
  static constexpr int NW_O = 0, QF_O = NW_KB, MF_O = QF_O + QF_KB, KT_O = MF_O + MF_KB, UC_O = KT_O + KT_KB;
  static constexpr int CHUNK_KB = UC_O + UC_KB;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t seq_rsrc(const void* p, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ f32x4 z4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }
__device__ __forceinline__ bf16x8 ldg16(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }

// 8 fp32 values as hi + lo bf16 operands.
__device__ __forceinline__ void split8(const float (&x)[8], bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const Bf16Pair p = split_bf16(x[j]);
    hi[j] = p.hi;
    lo[j] = p.lo;
  }
}
__device__ __forceinline__ f32x4 mfma3(const bf16x8& ah, const bf16x8& al, const bf16x8& bh, const bf16x8& bl,
                                       f32x4 c) {
  c = mfma16(ah, bh, c);
  c = mfma16(ah, bl, c);
  return mfma16(al, bh, c);
}

template <int D>
__global__ __launch_bounds__(256) void arl2_seq_prep_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                                                            const bf16* __restrict__ v, const float* __restrict__ beta,
                                                            const bf16* __restrict__ pqt, const bf16* __restrict__ pkt,
                                                            const bf16* __restrict__ pvt, unsigned char* __restrict__ ws,
                                                            int T, int H, int n_chunks, float eps) {
  using S = SeqShape<D>;
  constexpr int KS = S::KS, FB = S::FB, LD = S::LD, LT = S::LT;
  __shared__ __attribute__((aligned(16))) float Kl[kSeqChunk * LD];  // K' rows
  __shared__ __attribute__((aligned(16))) float Vl[kSeqChunk * LD];  // V' rows
  __shared__ __attribute__((aligned(16))) float Ql[kSeqChunk * LD];  // Q' rows
  __shared__ __attribute__((aligned(16))) float Lt[kSeqChunk * LT];  // L, then T
  __shared__ float bl[kSeqChunk];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, g4 = lane >> 4;
  const int item = blockIdx.x, chunk = item % n_chunks, bh = item / n_chunks;
  const int h = bh % H, b = bh / H;
  const int tw = chunk * kSeqChunk + 16 * wave;  // this wave's first token
  const int64_t rs = (int64_t)H * D;
  const int64_t base = ((int64_t)b * T * H + h) * D;
  const int64_t slice_bytes = ((int64_t)(T - 1) * rs + D) * 2;
  unsigned char* cw = ws + (int64_t)item * S::CHUNK_KB * 1024;

  if (lane < 16) bl[16 * wave + lane] = tw + lane < T ? beta[((int64_t)b * T + tw + lane) * H + h] : 0.f;

  // This lane's token row (tw + l % 16), features 32 ks + 8 (l / 16) ..: the A operand of
  // K phi_k and V phi_v, the B operand of phi_q^T Q^T.  Rows past the frame read as zeros.
  bf16x8 qr[KS], kr[KS], vr[KS];
  {
    const __amdgpu_buffer_rsrc_t rq = seq_rsrc(q + base, slice_bytes), rk = seq_rsrc(k + base, slice_bytes),
                                 rv = seq_rsrc(v + base, slice_bytes);
    const int ro = (int)((int64_t)(tw + r16) * rs * 2) + 16 * g4;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qr[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rq, ro + 64 * ks, 0, 0));
      kr[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rk, ro + 64 * ks, 0, 0));
      vr[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rv, ro + 64 * ks, 0, 0));
    }
  }
  const bf16* mq = pqt + (int64_t)h * D * D;
  const bf16* mk = pkt + (int64_t)h * D * D;
  const bf16* mv = pvt + (int64_t)h * D * D;
  auto map_frag = [&](const bf16* m, int blk, int ks) { return ldg16(m + (16 * blk + r16) * D + 32 * ks + 8 * g4); };

  // Q'^T = phi_q^T Q^T: block mb holds Q'[token tw + l % 16][feature 16 mb + 4 (l / 16) + i].
  {
    f32x4 qt[FB];
#pragma unroll
    for (int mb = 0; mb < FB; ++mb) {
      qt[mb] = z4();
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qt[mb] = mfma16(map_frag(mq, mb, ks), qr[ks], qt[mb]);
#pragma unroll
      for (int i = 0; i < 4; ++i) Ql[(16 * wave + r16) * LD + 16 * mb + 4 * g4 + i] = qt[mb][i];
    }
    // Q' A-fragments of the scan (token block = this wave, feature k-step ks)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      float x[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = qt[2 * ks + (j >> 2)][j & 3];
      bf16x8 hi, lo;
      split8(x, hi, lo);
      unsigned char* f = cw + (S::QF_O + (wave * KS + ks) * 2) * 1024 + 16 * lane;
      *reinterpret_cast<bf16x8*>(f) = hi;
      *reinterpret_cast<bf16x8*>(f + 1024) = lo;
    }
  }
  // K' = unit_rows(K phi_k): block fb holds K'[token tw + 4 (l / 16) + i][feature 16 fb + l % 16].
  {
    f32x4 kc[FB];
#pragma unroll
    for (int fb = 0; fb < FB; ++fb) {
      kc[fb] = z4();
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kc[fb] = mfma16(kr[ks], map_frag(mk, fb, ks), kc[fb]);
    }
    float ss[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ss[i] = 0.f;
#pragma unroll
      for (int fb = 0; fb < FB; ++fb) ss[i] = fmaf(kc[fb][i], kc[fb][i], ss[i]);
#pragma unroll
      for (int m = 1; m < 16; m <<= 1) ss[i] += __shfl_xor(ss[i], m);  // the row's other 15 lanes
      ss[i] = 1.f / fmaxf(sqrtf(ss[i]), eps);
    }
#pragma unroll
    for (int fb = 0; fb < FB; ++fb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        kc[fb][i] *= ss[i];
        Kl[(16 * wave + 4 * g4 + i) * LD + 16 * fb + r16] = kc[fb][i];
      }
      // K'^T A-fragments of the scan: this wave's 16 tokens are half (wave % 2) of token k-step wave / 2
      bf16x4 hi, lo;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const Bf16Pair p = split_bf16(kc[fb][i]);
        hi[i] = p.hi;
        lo[i] = p.lo;
      }
      unsigned char* f = cw + (S::KT_O + (fb * 2 + (wave >> 1)) * 2) * 1024 + 16 * lane + 8 * (wave & 1);
      *reinterpret_cast<bf16x4*>(f) = hi;
      *reinterpret_cast<bf16x4*>(f + 1024) = lo;
    }
  }
  // V' = V phi_v rows
#pragma unroll
  for (int fb = 0; fb < FB; ++fb) {
    f32x4 vc = z4();
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) vc = mfma16(vr[ks], map_frag(mv, fb, ks), vc);
#pragma unroll
    for (int i = 0; i < 4; ++i) Vl[(16 * wave + 4 * g4 + i) * LD + 16 * fb + r16] = vc[i];
  }
  __syncthreads();

  // 8 consecutive fp32 of a row of an LDS tile (16-byte aligned), or 8 rows of one column.
  auto row8 = [&](const float* t, int ld, int row, int col, bf16x8& hi, bf16x8& lo) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(t + row * ld + col);
    const f32x4 c = *reinterpret_cast<const f32x4*>(t + row * ld + col + 4);
    const float x[8] = {a[0], a[1], a[2], a[3], c[0], c[1], c[2], c[3]};
    split8(x, hi, lo);
  };
  auto col8_beta = [&](const float* t, int row0, int col, bf16x8& hi, bf16x8& lo) {  // beta_row * t[row][col]
    float x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = bl[row0 + j] * t[(row0 + j) * LD + col];
    split8(x, hi, lo);
  };

  // L = strictly_lower(diag(beta) K' K'^T): blocks (t1 block = this wave, t2 block <= it).
  // M^T = K' Q'^T masked to t2 < t1: blocks (t2 block <= this wave, t1 block = this wave), whose
  // C blocks are the A-fragments of M (rows t1, 32-deep token steps of t2).
  {
    f32x4 mt[4];
#pragma unroll
    for (int m2 = 0; m2 < 4; ++m2) {
      mt[m2] = z4();
      if (m2 > wave) continue;
      f32x4 g = z4();
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        bf16x8 ah, al, bh, bq, bql, bhl;
        row8(Kl, LD, 16 * wave + r16, 32 * ks + 8 * g4, ah, al);   // K' rows t1
        row8(Kl, LD, 16 * m2 + r16, 32 * ks + 8 * g4, bh, bhl);    // K' rows t2
        row8(Ql, LD, 16 * wave + r16, 32 * ks + 8 * g4, bq, bql);  // Q' rows t1
        g = mfma3(ah, al, bh, bhl, g);
        mt[m2] = mfma3(bh, bhl, bq, bql, mt[m2]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t1 = 16 * wave + 4 * g4 + i, t2 = 16 * m2 + r16;
        Lt[t1 * LT + t2] = t2 < t1 ? bl[t1] * g[i] : 0.f;
        const int u2 = 16 * m2 + 4 * g4 + i, u1 = 16 * wave + r16;  // M^T element (t2 = u2, t1 = u1)
        if (!(u2 < u1)) mt[m2][i] = 0.f;
      }
    }
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2) {
      float x[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = mt[2 * ks2 + (j >> 2)][j & 3];
      bf16x8 hi, lo;
      split8(x, hi, lo);
      unsigned char* f = cw + (S::MF_O + (wave * 2 + ks2) * 2) * 1024 + 16 * lane;
      *reinterpret_cast<bf16x8*>(f) = hi;
      *reinterpret_cast<bf16x8*>(f + 1024) = lo;
    }
  }
  __syncthreads();

  // T = (I + L)^-1 by forward substitution, one wave: lane c keeps column c.  Row i of L is
  // read whole before its products (one LDS round trip per row), and the products go to four
  // partial sums (independent FMA chains), added in a fixed order.
  if (wave == 0) {
    float tc[kSeqChunk];
#pragma unroll
    for (int i = 0; i < kSeqChunk; ++i) {
      f32x4 lr[(kSeqChunk + 3) / 4];
#pragma unroll
      for (int j = 0; j < i; j += 4) lr[j / 4] = *reinterpret_cast<const f32x4*>(Lt + i * LT + j);
      float acc[4] = {i == lane ? 1.f : 0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < i; j += 4)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (j + e < i) acc[e] = fmaf(-lr[j / 4][e], tc[j + e], acc[e]);
      tc[i] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
    }
#pragma unroll
    for (int i = 0; i < kSeqChunk; ++i) Lt[i * LT + lane] = tc[i];
  }
  __syncthreads();

  // U = T diag(beta) V' (C blocks [t1 block = this wave][feature block]) and
  // W^T = K'^T diag(beta) T^T (C blocks [feature block][t1 block = this wave]), negated and
  // regrouped into the A-fragments of -W.
  {
    bf16x8 th[2], tl[2];  // T rows t1 (this wave), 32-deep steps of t2: A of U, B of W^T
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2) row8(Lt, LT, 16 * wave + r16, 32 * ks2 + 8 * g4, th[ks2], tl[ks2]);
    f32x4 wt[FB];
#pragma unroll
    for (int fb = 0; fb < FB; ++fb) {
      f32x4 u = z4();
      wt[fb] = z4();
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2) {
        bf16x8 vh, vl, kh, kl;
        col8_beta(Vl, 32 * ks2 + 8 * g4, 16 * fb + r16, vh, vl);
        col8_beta(Kl, 32 * ks2 + 8 * g4, 16 * fb + r16, kh, kl);
        u = mfma3(th[ks2], tl[ks2], vh, vl, u);
        wt[fb] = mfma3(kh, kl, th[ks2], tl[ks2], wt[fb]);
      }
      *reinterpret_cast<f32x4*>(cw + (S::UC_O + wave * FB + fb) * 1024 + 16 * lane) = u;
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      float x[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = -wt[2 * ks + (j >> 2)][j & 3];
      bf16x8 hi, lo;
      split8(x, hi, lo);
      unsigned char* f = cw + (S::NW_O + (wave * KS + ks) * 2) * 1024 + 16 * lane;
      *reinterpret_cast<bf16x8*>(f) = hi;
      *reinterpret_cast<bf16x8*>(f + 1024) = lo;
    }
  }
}

template <int D>
__global__ __launch_bounds__(256) void arl2_seq_scan_kernel(const unsigned char* __restrict__ ws,
                                                            const float* s_prev,
                                                            const float* __restrict__ alpha,
                                                            float* s_new, float* __restrict__ o_inter,
                                                            int T, int H, int n_chunks) {
  using S = SeqShape<D>;
  constexpr int KS = S::KS, FB = S::FB;
  constexpr int SHARED_KB = S::QF_KB + S::MF_KB + S::KT_KB;
  __shared__ __attribute__((aligned(16))) unsigned char nw_lds[2][S::NW_KB * 1024];  // -W, double-buffered
  __shared__ __attribute__((aligned(16))) unsigned char sh_lds[SHARED_KB * 1024];    // Q', M, K'^T

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, g4 = lane >> 4;
  const int groups = (FB + 3) / 4;  // 64-column groups
  const int grp = blockIdx.x % groups, bh = blockIdx.x / groups;
  const int h = bh % H, b = bh / H;
  const int slice = 4 * grp + wave;  // this wave's 16 value columns
  const bool active = slice < FB;    // (d = 64: one group of four slices)
  const unsigned char* wsh = ws + (int64_t)bh * n_chunks * S::CHUNK_KB * 1024;

  auto dma = [&](unsigned char* lds, const unsigned char* src, int kb) {
    // kb kilobytes, dealt over the 4 waves
    const __amdgpu_buffer_rsrc_t r = seq_rsrc(src, (int64_t)kb * 1024);
    for (int i = wave; i < kb; i += 4)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (seq_lds_void*)(lds + i * 1024), 16, 16 * lane + i * 1024, 0, 0, 0);
  };
  auto chunk_ws = [&](int c) { return wsh + (int64_t)c * S::CHUNK_KB * 1024; };
  auto frag = [&](const unsigned char* base, int f) {
    return *reinterpret_cast<const bf16x8*>(base + f * 1024 + 16 * lane);
  };

  // The slice of S (C blocks [key-feature block fb]: S[16 fb + 4 (l / 16) + i][16 slice + l % 16]).
  // Only this wave reads or writes these columns, so s_new may be s_prev (S updated in place).
  const float* sp = s_prev + (int64_t)bh * D * D;
  f32x4 s[FB], s0[FB];
#pragma unroll
  for (int fb = 0; fb < FB; ++fb)
#pragma unroll
    for (int i = 0; i < 4; ++i) s[fb][i] = active ? sp[(16 * fb + 4 * g4 + i) * D + 16 * slice + r16] : 0.f;
#pragma unroll
  for (int fb = 0; fb < FB; ++fb) s0[fb] = s[fb];

  // U of this slice (C blocks [token block]), one chunk ahead
  auto load_u = [&](int c, f32x4 (&u)[4]) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
      u[mt] = active ? *reinterpret_cast<const f32x4*>(chunk_ws(c) + (S::UC_O + mt * FB + slice) * 1024 + 16 * lane)
                     : z4();
  };
  f32x4 u_next[4];
  f32x4 o_prev[4];  // the previous chunk's output, stored one chunk late (its stores then complete
                    // while this chunk computes instead of holding up the next wait)
  auto store_o = [&](int c, const f32x4 (&o)[4]) {
    if (!active) return;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = c * kSeqChunk + 16 * mt + 4 * g4 + i;
        if (t < T) o_inter[(((int64_t)b * T + t) * H + h) * D + 16 * slice + r16] = o[mt][i];
      }
  };
  dma(nw_lds[0], chunk_ws(0) + S::NW_O * 1024, S::NW_KB);
  dma(sh_lds, chunk_ws(0) + S::QF_O * 1024, SHARED_KB);  // Q', M, K'^T are contiguous in the workspace
  load_u(0, u_next);
  for (int c = 0; c < n_chunks; ++c) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // this wave's loads (into LDS, and U) have landed
    __syncthreads();
    if (c > 0) store_o(c - 1, o_prev);
    f32x4 u[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) u[mt] = u_next[mt];
    if (c + 1 < n_chunks) {
      dma(nw_lds[(c + 1) & 1], chunk_ws(c + 1) + S::NW_O * 1024, S::NW_KB);
      load_u(c + 1, u_next);
    }
    const unsigned char* nw = nw_lds[c & 1];
    const unsigned char* qf = sh_lds;
    const unsigned char* mf = sh_lds + S::QF_KB * 1024;
    const unsigned char* kt = sh_lds + (S::QF_KB + S::MF_KB) * 1024;

    // S as B operands (32-deep key-feature steps), hi + lo
    bf16x8 sh[KS], sl[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      float x[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = s[2 * ks + (j >> 2)][j & 3];
      split8(x, sh[ks], sl[ks]);
    }
    // U_hat = U - W S;  O = Q' S (+ M U_hat below)
    f32x4 o[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      o[mt] = z4();
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int f = (mt * KS + ks) * 2;
        u[mt] = mfma3(frag(nw, f), frag(nw, f + 1), sh[ks], sl[ks], u[mt]);
        o[mt] = mfma3(frag(qf, f), frag(qf, f + 1), sh[ks], sl[ks], o[mt]);
      }
    }
    // U_hat as B operands (32-deep token steps), hi + lo
    bf16x8 uh[2], ul[2];
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2) {
      float x[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = u[2 * ks2 + (j >> 2)][j & 3];
      split8(x, uh[ks2], ul[ks2]);
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2) {
        const int f = (mt * 2 + ks2) * 2;
        o[mt] = mfma3(frag(mf, f), frag(mf, f + 1), uh[ks2], ul[ks2], o[mt]);
      }
    // S += K'^T U_hat
#pragma unroll
    for (int fb = 0; fb < FB; ++fb)
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2) {
        const int f = (fb * 2 + ks2) * 2;
        s[fb] = mfma3(frag(kt, f), frag(kt, f + 1), uh[ks2], ul[ks2], s[fb]);
      }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) o_prev[mt] = o[mt];
    __syncthreads();  // every wave is done with this chunk's Q', M, K'^T
    if (c + 1 < n_chunks) dma(sh_lds, chunk_ws(c + 1) + S::QF_O * 1024, SHARED_KB);
  }
  store_o(n_chunks - 1, o_prev);
  // clean pass: S_N = S^(T) - (1 - alpha) S_{N-1}
  if (s_new && active) {
    const float a1 = 1.f - alpha[bh];
    float* sn = s_new + (int64_t)bh * D * D;
#pragma unroll
    for (int fb = 0; fb < FB; ++fb)
#pragma unroll
      for (int i = 0; i < 4; ++i) sn[(16 * fb + 4 * g4 + i) * D + 16 * slice + r16] = s[fb][i] - a1 * s0[fb][i];
  }
}

template <int D>
hipError_t launch_seq_d(const SeqArgs& a, hipStream_t stream) {
  using S = SeqShape<D>;
  const int n_chunks = seq_chunks(a.T);
  hipLaunchKernelGGL((arl2_seq_prep_kernel<D>), dim3(a.B * a.H * n_chunks), dim3(256), 0, stream,
                     static_cast<const bf16*>(a.q), static_cast<const bf16*>(a.k), static_cast<const bf16*>(a.v),
                     a.beta, static_cast<const bf16*>(a.pqt), static_cast<const bf16*>(a.pkt),
                     static_cast<const bf16*>(a.pvt), static_cast<unsigned char*>(a.ws), a.T, a.H, n_chunks, a.eps);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((arl2_seq_scan_kernel<D>), dim3(a.B * a.H * ((S::FB + 3) / 4)), dim3(256), 0, stream,
                     static_cast<const unsigned char*>(a.ws), a.s_prev, a.alpha, a.s_new, a.o_inter, a.T, a.H,
                     n_chunks);
  return hipGetLastError();
}

}  // namespace

int seq_chunks(int T) { return (T + kSeqChunk - 1) / kSeqChunk; }

size_t seq_workspace_bytes(int d, int B, int H, int T) {
  const size_t per = d == 128 ? SeqShape<128>::CHUNK_KB : SeqShape<64>::CHUNK_KB;
  return (size_t)B * H * seq_chunks(T) * per * 1024;
}

hipError_t launch_seq(int d, const SeqArgs& a, hipStream_t stream) {
  switch (d) {
    case 64: return launch_seq_d<64>(a, stream);
    case 128: return launch_seq_d<128>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace arl2
