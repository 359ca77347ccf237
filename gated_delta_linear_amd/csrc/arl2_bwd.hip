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
// Kernels.  The attention backward runs as one MFMA launch with no atomics (bitwise
// reproducible), 8 waves per work-group, 32x32x16 MFMAs: dK, dV work-groups per 128-key block,
// four 32-key groups in two wave roles each (scores, P and dV beside dP, dS and dK; P handed over
// through LDS), then dQ work-groups per 128-query block, four 32-query groups times two key
// halves; 64-row blocks of the other side stream through LDS and the scores are recomputed in
// each.  Every streamed tile reaches LDS by direct-to-LDS buffer loads, two stages deep (block
// b + 1 is in flight while block b is multiplied, one barrier per block), with rows
// chunk-swizzled so that the fragment reads hit distinct banks; no thread converts or transposes
// anything on the way.  The operands those loads need in another type or layout (dO, V in fp16,
// and K^T, Q^T, dO^T in fp16, stored in the order in which an MFMA lane takes its k-values) are
// written once per pass by a conversion kernel, which also forms dO . O per row.  The score
// products S = Q K^T run in bf16 on the inputs as given; the others (dP = dO V^T, dV, dK, dQ) in
// fp16, where P, dS and dO round with a relative step of 2^-11; all accumulate in fp32.  The
// token kernels (inter read, state write) work per 128-token chunk with 16x16x32 MFMAs on
// split-bf16 operands (hi + lo, three products per term), so that their d x d products keep
// about fp32 accuracy as the forward's state write does, each product's B fragments read from L2
// one 16-column block ahead; their sums over tokens leave the chunk as partials that per-head
// kernels add in a fixed order.
#include <algorithm>
#include <type_traits>

#include "arl2_device.h"
#include "arl2_kernels.h"

namespace arl2 {
namespace {

constexpr int kAttnBlock = 64;  // queries or keys per work-group of the attention backward
constexpr int kTokChunk = 128;  // tokens per work-group of the token kernels (8 waves x 16)

// XCD-aware order of a 1-D grid of 8 ceil(n / 8) work-groups over n items (blocks of rows of
// one (stream, head) after another): the hardware deals work-group i to XCD i % 8, and item
// x ceil(n / 8) + j goes to work-group 8 j + x, so each XCD takes a contiguous run of items, one
// or two heads, and a head's operands fill one or two L2 caches instead of all eight.  Returns
// -1 for the padding work-groups.
__device__ __forceinline__ int xcd_item_at(int wg, int n) {
  const int per = (n + 7) / 8, item = (wg & 7) * per + (wg >> 3);
  return item < n ? item : -1;
}
__device__ __forceinline__ int xcd_item(int n) { return xcd_item_at((int)blockIdx.x, n); }
__host__ __device__ inline int xcd_grid(int n) { return 8 * ((n + 7) / 8); }

template <int D>
struct BwdShape {
  static constexpr int KS = D / 32;          // 32-deep k-steps over features
  static constexpr int NB = D / 16;          // 16-wide blocks over features
  static constexpr int LF = D + 4;           // fp32 row pitch of the token kernels' row buffers
};

// B fragment (s, nb) of a d x d matrix kept in fragment order [s][nb][lane][8]: lane l holds
// M[32 s + 8 (l / 16) + j][16 nb + l % 16].
template <int D>
__device__ __forceinline__ bf16x8 frag(const bf16* f, int s, int nb, int lane) {
  return ld_bf16x8(f + ((s * BwdShape<D>::NB + nb) * 64 + lane) * 8);
}

// 8 fp32 values as bf16 hi + lo (split_bf16's rounding), two at a time so that each rounding
// of a pair is one packed conversion
__device__ __forceinline__ void split8(const float (&x)[8], bf16x8& hi, bf16x8& lo) {
  typedef float f32x2v __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
#pragma unroll
  for (int j = 0; j < 8; j += 2) {
    const f32x2v v = {x[j], x[j + 1]};
    const bf16x2v h = __builtin_convertvector(v, bf16x2v);
    const f32x2v hf = __builtin_convertvector(h, f32x2v);
    const f32x2v r = {v[0] - hf[0], v[1] - hf[1]};
    const bf16x2v l = __builtin_convertvector(r, bf16x2v);
    hi[j] = h[0];
    hi[j + 1] = h[1];
    lo[j] = l[0];
    lo[j + 1] = l[1];
  }
}

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

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

// --- attention backward ---------------------------------------------------------------------
// S = Q K^T in bf16 on the inputs as given; every other product in fp16 (P, dS and dO round with
// a relative step of 2^-11, four times finer than bf16; the bf16 inputs convert exactly when
// they lie in fp16's normal range); all with fp32 accumulation, at the bf16 MFMA rate.

template <typename T>
__device__ __forceinline__ f16x8 load_f16x8(const T* p) {
  if constexpr (sizeof(T) == 2 && __is_same(T, f16)) return ld_f16x8(p);
  else return to_f16(ld_bf16x8(p));
}

// exp2 on the transcendental unit (arguments are at most about 0 here: lse bounds every score)
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

typedef __attribute__((address_space(3))) void lds_void_b;

// 16 bytes per lane from the buffer straight into LDS at lds + 16 * lane (lds wave-uniform).
__device__ __forceinline__ void dma16b(__amdgpu_buffer_rsrc_t r, void* lds, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_b*)lds, 16, voff, soff, 0, 0);
}

// Buffer resource over rows [first_row, T) of one (stream, head) slice of a [B][T][H][d] fp16
// tensor: rows past the frame lie outside num_records and load as zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc16(const f16* base, int T, int64_t rs, int d,
                                                              int first_row) {
  const int64_t start = (int64_t)first_row * rs;
  const int64_t left = (int64_t)(T - 1) * rs + d - start;
  const bool any = left > 0;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<f16*>(any ? base + start : base), (short)0,
                                           any ? (int)(left * 2) : 0, 0x00020000);
}

// dK, dV of 32 NKG keys of one (stream, head), with 32x32x16 MFMAs.  2 NKG waves in two roles
// that share each 32-key group kg: wave kg (role P) forms S = Q K^T and P = exp2(S scale log2 e
// - lse) and accumulates dV^T += dO^T P; wave NKG + kg (role dS) forms dP = dO V^T, takes P
// from role P through LDS, dS = P (dP - Dv), and accumulates dK^T += Q^T dS.  Per 64-query block
// and 32-query half, C blocks of S and dP hold lane l, register i <-> query
// 8 (i / 4) + 4 (l / 32) + i % 4, key l % 32: every lane holds one key, so P and dS go straight
// from the C registers into the B operands of the dV, dK products (k-step h: registers
// 8 h .. 8 h + 7), and the P handed over is the producer lane's registers as they are.  A block
// runs in two phases split by a barrier: role P's scores and exponentials beside role dS's dP
// products, then role P's dV products beside role dS's dS and dK products; the two waves of a
// key group share a SIMD, so one's vector work overlaps the other's MFMAs.  Each 32x32x16
// product reads one 1 KB operand from LDS.  Every key block reads the head's whole Q and dO.
// Staging: each 64-query block's Q rows (bf16, as given: S = Q K^T runs on the bf16 inputs), dO
// rows (the fp16 dO) and the transposed fp16 copies Q^T and dO^T (64 queries per feature row)
// come straight into LDS with direct-to-LDS loads, in two stages: block qb + 1's loads fly while
// block qb is multiplied.  Row tiles keep 16-byte chunk c of query row r at c ^ (r mod d/8), the
// transposed tiles stored chunk c of feature row f at c ^ (f mod 8): every load brings whole
// rows, and every fragment read (one 16-byte chunk per lane) hits distinct banks.
// Operands of the attention backward launch (dK/dV and dQ work-groups in one grid).
struct BwdAttnArgs {
  const bf16 *q, *k, *v;
  const f16 *doh, *v16, *kt16, *qt16, *dot16;
  const float *lse, *dvec;
  float *dk, *dv, *dq;
  int T, H, BH, tp;
  float scale, scale_log2;
};

template <int D, int NKG, int TILE>
__device__ __forceinline__ void dkdv_body(const BwdAttnArgs& A, int item, unsigned char (&qr0)[TILE],
                                          unsigned char (&qr1)[TILE], unsigned char (&or0)[TILE],
                                          unsigned char (&or1)[TILE], unsigned char (&qt0)[TILE],
                                          unsigned char (&qt1)[TILE], unsigned char (&ot0)[TILE],
                                          unsigned char (&ot1)[TILE], float (&lse_s)[2][kAttnBlock],
                                          float (&dv_s)[2][kAttnBlock], f16x8 (&p_x)[NKG][2][2][64]) {
  const bf16* __restrict__ q = A.q;
  const bf16* __restrict__ k = A.k;
  const bf16* __restrict__ v = A.v;
  const f16* __restrict__ doh = A.doh;
  const f16* __restrict__ qt16 = A.qt16;
  const f16* __restrict__ dot16 = A.dot16;
  const float* __restrict__ lse = A.lse;
  const float* __restrict__ dvec = A.dvec;
  float* __restrict__ dk = A.dk;
  float* __restrict__ dv = A.dv;
  const int T = A.T, H = A.H, tp = A.tp;
  const float scale = A.scale, scale_log2 = A.scale_log2;
  constexpr int K16 = D / 16, FB = D / 32, NW = 2 * NKG;
  constexpr int RB = 2 * D, CPR = D / 8, RPI = 1024 / RB;  // bytes per query row, 16-byte chunks per row, rows per 1-KB load
  static_assert(TILE == kAttnBlock * RB, "a 64-row tile; a transposed tile (d rows of 128 bytes) too");
  constexpr int LD = TILE / 1024, LPT = LD / NW;           // 1-KB loads per tile, of them per wave
  static_assert(LD % NW == 0, "every wave issues the same number of loads per tile");
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kg = wave % NKG, role = wave / NKG;
  const int nkb = (T + 32 * NKG - 1) / (32 * NKG);
  const int bh = item / nkb, b = bh / H, h = bh % H;
  const int64_t rs = (int64_t)H * D, base = ((int64_t)b * T * H + h) * D;
  const int key = (item % nkb) * (32 * NKG) + 32 * kg + l32;

  // Loads of block qb (a wave's loads i = wave + NW m of each tile; see the dQ kernel's).
  auto issue = [&](int qb, unsigned char* qd, unsigned char* od, unsigned char* qtd, unsigned char* otd) {
    const int r0 = qb * kAttnBlock;
    const __amdgpu_buffer_rsrc_t rq = rows_rsrc16(reinterpret_cast<const f16*>(q) + base, T, rs, D, r0);  // bf16 bits
    const __amdgpu_buffer_rsrc_t ro = rows_rsrc16(doh + base, T, rs, D, r0);
    const int64_t toff = (int64_t)bh * D * tp + r0;
    const uint64_t qa = reinterpret_cast<uint64_t>(qt16 + toff), oa = reinterpret_cast<uint64_t>(dot16 + toff);
    const int tbytes = __builtin_amdgcn_readfirstlane(D * tp * 2 - r0 * 2);
    auto uni = [](uint64_t a) {  // wave-uniform address, so that the descriptor lives in scalar registers
      const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a), hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
      return reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
    };
    const __amdgpu_buffer_rsrc_t rqt = __builtin_amdgcn_make_buffer_rsrc(uni(qa), (short)0, tbytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rot = __builtin_amdgcn_make_buffer_rsrc(uni(oa), (short)0, tbytes, 0x00020000);
#pragma unroll
    for (int m = 0; m < LPT; ++m) {
      const int i = wave + NW * m, row = RPI * i + lane / CPR;
      const int vo = (lane / CPR) * (int)(rs * 2) + 16 * ((lane % CPR) ^ (row % CPR));
      dma16b(rq, qd + i * 1024, vo, RPI * i * (int)(rs * 2));
      dma16b(ro, od + i * 1024, vo, RPI * i * (int)(rs * 2));
    }
#pragma unroll
    for (int m = 0; m < LPT; ++m) {
      const int i = wave + NW * m, row = 8 * i + lane / 8;
      const int vo = (lane / 8) * tp * 2 + 16 * ((lane % 8) ^ (row & 7));
      dma16b(rqt, qtd + i * 1024, vo, 8 * i * tp * 2);
      dma16b(rot, otd + i * 1024, vo, 8 * i * tp * 2);
    }
  };
  // lse and Dv of a block's rows: loaded into registers (threads < 64) one block ahead of their
  // store into LDS, and before that block's tile loads, so that waiting for them waits for nothing
  // else
  float lse_r = 0.f, dv_r = 0.f;
  auto load_ld = [&](int qb) {
    if (tid < kAttnBlock) {
      const int r = qb * kAttnBlock + tid;
      lse_r = r < T ? lse[(int64_t)bh * T + r] : INFINITY;  // rows past T get P = 0
      dv_r = r < T ? dvec[(int64_t)bh * T + r] : 0.f;
    }
  };
  auto store_ld = [&](int buf) {
    if (tid < kAttnBlock) {
      lse_s[buf][tid] = lse_r;
      dv_s[buf][tid] = dv_r;
    }
  };
  // A fragment of a transposed tile: feature row 32 fb + l % 32, queries 32 h2 + 16 hh +
  // 8 (j / 4) + 4 (l / 32) + j % 4 (the stacked-C row order of P and dS), which the quad order of
  // the copies puts in stored chunk 4 h2 + 2 hh + l / 32
  auto tfrag = [&](const unsigned char* t, int fb, int h2, int hh) {
    const int f = 32 * fb + l32;
    return *reinterpret_cast<const f16x8*>(t + f * 128 + 16 * ((4 * h2 + 2 * hh + hi) ^ (f & 7)));
  };
  // A fragment of a row tile: query row 32 h2 + l % 32, features 16 s + 8 (l / 32) ..
  auto rfrag_off = [&](int h2, int s) {
    const int r = 32 * h2 + l32;
    return r * RB + 16 * ((2 * s + hi) ^ (r % CPR));
  };
  // the phase barrier: role P's stores of P are done (lgkmcnt(0)); the block's tile loads stay in
  // flight (no vmcnt wait), and the compiler keeps LDS accesses on their side of it
  auto phase_barrier = [] { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };
  const int nqb = (T + kAttnBlock - 1) / kAttnBlock;
  // block qb (odd_c: qb % 2): this wave's loads of it have landed and its reads of block qb - 1
  // are done; after the barrier everyone's are, so block qb + 1 goes into the other stage while
  // block qb is multiplied
  auto begin_block = [&](int qb, auto odd_c) {
    constexpr int odd = decltype(odd_c)::value;
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
    __syncthreads();
    if (qb + 1 < nqb) {
      store_ld(1 - odd);
      if (qb + 2 < nqb) load_ld(qb + 2);
      if constexpr (odd) issue(qb + 1, qr0, or0, qt0, ot0);
      else issue(qb + 1, qr1, or1, qt1, ot1);
    }
  };
  load_ld(0);
  store_ld(0);
  if (nqb > 1) load_ld(1);
  issue(0, qr0, or0, qt0, ot0);

  if (role == 0) {
    // role P: B operands K^T (lane l: key, features 16 s + 8 (l / 32) ..; bf16, as given)
    bf16x8 kf[K16];
#pragma unroll
    for (int s = 0; s < K16; ++s)
      kf[s] = key < T ? ld_bf16x8(k + base + (int64_t)key * rs + 16 * s + 8 * hi) : zero_bf16x8();
    f32x16 dvt[FB];
#pragma unroll
    for (int n = 0; n < FB; ++n) dvt[n] = zero16();
    auto qblock = [&](int qb, auto odd_c) {
      constexpr int odd = decltype(odd_c)::value;
      const unsigned char* qc = odd ? qr1 : qr0;
      const unsigned char* otc = odd ? ot1 : ot0;
      const float* lse_c = lse_s[odd];
      begin_block(qb, odd_c);
      // every fragment of a product group is read before its MFMAs, and the dV operands before
      // the exponentials, so that LDS latency hides behind MFMA and vector work
      bf16x8 fa[2][K16];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int s = 0; s < K16; ++s) fa[h2][s] = *reinterpret_cast<const bf16x8*>(qc + rfrag_off(h2, s));
      __builtin_amdgcn_sched_barrier(0);
      f32x16 sc[2] = {zero16(), zero16()};
#pragma unroll
      for (int s = 0; s < K16; ++s)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) sc[h2] = mfma32(fa[h2][s], kf[s], sc[h2]);
      __builtin_amdgcn_sched_barrier(0);
      f16x8 ta[FB][2];  // dO^T operands of the first 32-query half
#pragma unroll
      for (int fb = 0; fb < FB; ++fb)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) ta[fb][hh] = tfrag(otc, fb, 0, hh);
      __builtin_amdgcn_sched_barrier(0);
      f16x8 pb[2][2];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x4 L = *reinterpret_cast<const f32x4*>(lse_c + 32 * h2 + 8 * j + 4 * hi);
#pragma unroll
          for (int e = 0; e < 4; ++e) pb[h2][j / 2][4 * (j % 2) + e] = (f16)fast_exp2(sc[h2][4 * j + e] * scale_log2 - L[e]);
        }
        p_x[kg][h2][0][lane] = pb[h2][0];
        p_x[kg][h2][1][lane] = pb[h2][1];
      }
      phase_barrier();
      f16x8 tb[FB][2];  // the second half's, read while the first half's products run
#pragma unroll
      for (int fb = 0; fb < FB; ++fb)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) tb[fb][hh] = tfrag(otc, fb, 1, hh);
#pragma unroll
      for (int fb = 0; fb < FB; ++fb)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) dvt[fb] = mfma32(ta[fb][hh], pb[0][hh], dvt[fb]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int fb = 0; fb < FB; ++fb)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) dvt[fb] = mfma32(tb[fb][hh], pb[1][hh], dvt[fb]);
    };
    int qb = 0;
    for (; qb + 1 < nqb; qb += 2) {
      qblock(qb, std::integral_constant<int, 0>());
      qblock(qb + 1, std::integral_constant<int, 1>());
    }
    if (qb < nqb) qblock(qb, std::integral_constant<int, 0>());
    // lane l, register i: feature 32 fb + 8 (i / 4) + 4 (l / 32) + i % 4 of key l % 32
    if (key < T) {
#pragma unroll
      for (int fb = 0; fb < FB; ++fb)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4)
          *reinterpret_cast<f32x4*>(dv + base + (int64_t)key * rs + 32 * fb + 8 * g4 + 4 * hi) =
              f32x4{dvt[fb][4 * g4], dvt[fb][4 * g4 + 1], dvt[fb][4 * g4 + 2], dvt[fb][4 * g4 + 3]};
    }
  } else {
    // role dS: B operands V^T in fp16 (lane l: key, features 16 s + 8 (l / 32) ..)
    f16x8 vf[K16];
#pragma unroll
    for (int s = 0; s < K16; ++s)
      vf[s] = key < T ? load_f16x8(v + base + (int64_t)key * rs + 16 * s + 8 * hi) : f16x8{};
    f32x16 dkt[FB];
#pragma unroll
    for (int n = 0; n < FB; ++n) dkt[n] = zero16();
    auto qblock = [&](int qb, auto odd_c) {
      constexpr int odd = decltype(odd_c)::value;
      const unsigned char* oc = odd ? or1 : or0;
      const unsigned char* qtc = odd ? qt1 : qt0;
      const float* dv_c = dv_s[odd];
      begin_block(qb, odd_c);
      // as in role P: fragment reads ahead of their MFMAs, the dK operands before the barrier
      f16x8 fa[2][K16];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int s = 0; s < K16; ++s) fa[h2][s] = *reinterpret_cast<const f16x8*>(oc + rfrag_off(h2, s));
      __builtin_amdgcn_sched_barrier(0);
      f32x16 dp[2] = {zero16(), zero16()};
#pragma unroll
      for (int s = 0; s < K16; ++s)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) dp[h2] = mfma32(fa[h2][s], vf[s], dp[h2]);
      __builtin_amdgcn_sched_barrier(0);
      f16x8 ta[FB][2];  // Q^T operands of the first 32-query half
#pragma unroll
      for (int fb = 0; fb < FB; ++fb)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) ta[fb][hh] = tfrag(qtc, fb, 0, hh);
      phase_barrier();
      // dS of a 32-query half from role P's P (this lane's registers there) and dP
      auto ds_half = [&](int h2, f16x8 (&dsb)[2]) {
        const f16x8 p0 = p_x[kg][h2][0][lane], p1 = p_x[kg][h2][1][lane];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x4 Dd = *reinterpret_cast<const f32x4*>(dv_c + 32 * h2 + 8 * j + 4 * hi);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = 4 * j + e;
            const float p = (float)(i < 8 ? p0[i] : p1[i - 8]);
            dsb[i / 8][i % 8] = (f16)(p * (dp[h2][i] - Dd[e]));
          }
        }
      };
      f16x8 d0[2], d1[2];
      ds_half(0, d0);
      __builtin_amdgcn_sched_barrier(0);
      f16x8 tb[FB][2];  // the second half's, read while the first half's products run
#pragma unroll
      for (int fb = 0; fb < FB; ++fb)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) tb[fb][hh] = tfrag(qtc, fb, 1, hh);
#pragma unroll
      for (int fb = 0; fb < FB; ++fb)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) dkt[fb] = mfma32(ta[fb][hh], d0[hh], dkt[fb]);
      ds_half(1, d1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int fb = 0; fb < FB; ++fb)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) dkt[fb] = mfma32(tb[fb][hh], d1[hh], dkt[fb]);
    };
    int qb = 0;
    for (; qb + 1 < nqb; qb += 2) {
      qblock(qb, std::integral_constant<int, 0>());
      qblock(qb + 1, std::integral_constant<int, 1>());
    }
    if (qb < nqb) qblock(qb, std::integral_constant<int, 0>());
    if (key < T) {
#pragma unroll
      for (int fb = 0; fb < FB; ++fb)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4)
          *reinterpret_cast<f32x4*>(dk + base + (int64_t)key * rs + 32 * fb + 8 * g4 + 4 * hi) =
              f32x4{dkt[fb][4 * g4], dkt[fb][4 * g4 + 1], dkt[fb][4 * g4 + 2], dkt[fb][4 * g4 + 3]} * scale;
    }
  }
}

// A pass's operands in fp16 for the attention backward's direct-to-LDS staging: v16 in the
// [B][T][H][d] layout of v (rows past T not written), and the transposes kt16, qt16, dot16
// [B][H][d][tp] of k, q and the fp16 dO: each head's features as rows of its tokens, 64-token
// blocks (tokens past T zero), each 16-token group stored as its 4-token quads 0, 2, 1, 3 (the
// order in which a 32x32x16 MFMA lane takes its 8 k-values when P or dS come straight from C
// registers, so that a lane's A fragment is one 16-byte chunk).  The same pass also rounds dO to
// fp16 (do_h, the attention backward's MFMA operand) and forms Dv[b][h][t] = dO . O over each
// row's features with that rounded dO, so that dS = P (dP - Dv) is the gradient of one
// consistent dO.  One work-group per (stream, head, 64-token block); thread j moves rows
// 4 (j % 16) .. + 3 of 8-feature chunk j / 16, transposing through LDS; a row's dot product is
// summed over its chunks in chunk order.
template <int D>
__global__ __launch_bounds__(256) void arl2_bwd_cvt16_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                                                           const bf16* __restrict__ v, const float* __restrict__ d_out,
                                                           const float* __restrict__ o_sm, f16* __restrict__ doh,
                                                           float* __restrict__ dvec, f16* __restrict__ v16,
                                                           f16* __restrict__ kt16, f16* __restrict__ qt16,
                                                           f16* __restrict__ dot16, int T, int H, int tp) {
  constexpr int CPR = D / 8, TPITCH = kAttnBlock + 8;  // chunks per row; transposing tiles' pitch (f16)
  __shared__ __align__(16) f16 tr[3][D * TPITCH];     // K^T, Q^T, dO^T of the block
  __shared__ float dpart[kAttnBlock][CPR + 1];        // dO . O per row and chunk
  const int tid = threadIdx.x, bh = blockIdx.y, b = bh / H, h = bh % H, k0 = blockIdx.x * kAttnBlock;
  const int64_t rs = (int64_t)H * D, base = ((int64_t)b * T * H + h) * D;
  for (int j = tid; j < 16 * CPR; j += 256) {
    const int rg = j % 16, cc = j / 16;
    f16x8 x[3][4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = k0 + 4 * rg + e;
      x[0][e] = x[1][e] = x[2][e] = f16x8{};
      float dot = 0.f;
      if (t < T) {
        const int64_t o = base + (int64_t)t * rs + 8 * cc;
        x[0][e] = to_f16(ld_bf16x8(k + o));
        x[1][e] = to_f16(ld_bf16x8(q + o));
        const f32x4 g0 = *reinterpret_cast<const f32x4*>(d_out + o), g1 = *reinterpret_cast<const f32x4*>(d_out + o + 4);
        const f32x4 y0 = *reinterpret_cast<const f32x4*>(o_sm + o), y1 = *reinterpret_cast<const f32x4*>(o_sm + o + 4);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          x[2][e][c] = (f16)g0[c];
          x[2][e][4 + c] = (f16)g1[c];
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) dot += (float)x[2][e][c] * y0[c];  // the rounded dO, as dP = dO V^T sees it
#pragma unroll
        for (int c = 0; c < 4; ++c) dot += (float)x[2][e][4 + c] * y1[c];
        *reinterpret_cast<f16x8*>(doh + o) = x[2][e];
        *reinterpret_cast<f16x8*>(v16 + o) = to_f16(ld_bf16x8(v + o));
      }
      dpart[4 * rg + e][cc] = dot;
    }
#pragma unroll
    for (int m = 0; m < 3; ++m)
#pragma unroll
      for (int c = 0; c < 8; ++c)
        *reinterpret_cast<f16x4*>(tr[m] + (8 * cc + c) * TPITCH + 4 * rg) =
            f16x4{x[m][0][c], x[m][1][c], x[m][2][c], x[m][3][c]};
  }
  __syncthreads();
  if (tid < kAttnBlock && k0 + tid < T) {
    float dot = 0.f;
#pragma unroll
    for (int cc = 0; cc < CPR; ++cc) dot += dpart[tid][cc];
    dvec[(int64_t)bh * T + k0 + tid] = dot;
  }
  f16* const dst[3] = {kt16, qt16, dot16};
  for (int j = tid; j < 3 * D * (kAttnBlock / 8); j += 256) {
    const int m = j / (D * (kAttnBlock / 8)), jj = j % (D * (kAttnBlock / 8));
    const int f = jj / (kAttnBlock / 8), c = jj % (kAttnBlock / 8);
    // stored chunk c = 2 g + e of a row: tokens 16 g + 4 e .. + 3, then 16 g + 8 + 4 e .. + 3
    const f16* src = tr[m] + f * TPITCH + 16 * (c / 2) + 4 * (c % 2);
    const f16x4 lo = *reinterpret_cast<const f16x4*>(src), hi = *reinterpret_cast<const f16x4*>(src + 8);
    *reinterpret_cast<f16x8*>(dst[m] + ((int64_t)bh * D + f) * tp + k0 + 8 * c) =
        f16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
}

// dQ of 32 NQG queries of one (stream, head), with 32x32x16 MFMAs.  2 NQG waves: wave w owns
// queries 32 (w % NQG) .. +31 and the key half w / NQG of every 64-key block; the halves are added
// at the end.  Every query block reads the head's whole K and V, so wider work-groups cut that
// stream in proportion.  Per key block: S^T = K Q^T and dP^T = V dO^T (32x32 C blocks: lane l,
// register i <-> key 8 (i / 4) + 4 (l / 32) + i % 4 of the wave's 32, query l % 32: every lane
// holds one query, so its lse and Dv are one value each), dS^T = P^T (dP^T - Dv), then
// dQ^T += K^T dS^T with dS^T as the B operand straight from the C registers (k-step h: registers
// 8 h .. 8 h + 7).  A 32x32x16 product reads one 1 KB operand from LDS per 32 K multiply-adds,
// twice the 16x16x32 ratio.
// Staging: each block's K rows (bf16, as given), V rows (the fp16 copy v16) and K^T (kt16, 64
// keys per feature row, fp16) come straight into LDS with direct-to-LDS loads, in two stages: block kb + 1's
// loads fly while block kb is multiplied, and no thread converts or transposes anything.  A row
// tile keeps 16-byte chunk c of key row r at chunk c ^ (r mod d/8), the K^T tile stored chunk c
// of feature row f at c ^ (f mod 8): every load brings whole rows, and every fragment read (one
// 16-byte chunk per lane) hits distinct banks.
template <int D, int NQG, int TILE>
__device__ __forceinline__ void dq_body(const BwdAttnArgs& A, int item, unsigned char (&kr0)[TILE],
                                        unsigned char (&kr1)[TILE], unsigned char (&vr0)[TILE],
                                        unsigned char (&vr1)[TILE], unsigned char (&kt0)[TILE],
                                        unsigned char (&kt1)[TILE]) {
  const bf16* __restrict__ q = A.q;
  const bf16* __restrict__ k = A.k;
  const f16* __restrict__ v16 = A.v16;
  const f16* __restrict__ kt16 = A.kt16;
  const f16* __restrict__ doh = A.doh;
  const float* __restrict__ lse = A.lse;
  const float* __restrict__ dvec = A.dvec;
  float* __restrict__ dq = A.dq;
  const int T = A.T, H = A.H, tp = A.tp;
  const float scale = A.scale, scale_log2 = A.scale_log2;
  constexpr int K16 = D / 16, FB = D / 32, NW = 2 * NQG;
  constexpr int RB = 2 * D, CPR = D / 8, RPI = 1024 / RB;  // bytes per key row, 16-byte chunks per row, rows per 1-KB load
  static_assert(TILE == kAttnBlock * RB, "a 64-row tile; the K^T tile (d rows of 128 bytes) too");
  constexpr int LD = TILE / 1024;                          // 1-KB loads per tile
  constexpr int LPT = LD / NW;                             // of them per wave
  static_assert(LD % NW == 0, "every wave issues the same number of loads per tile");
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qh = wave % NQG, kh = wave / NQG;
  const int nqb = (T + 32 * NQG - 1) / (32 * NQG);
  const int bh = item / nqb, b = bh / H, h = bh % H;
  const int64_t rs = (int64_t)H * D, base = ((int64_t)b * T * H + h) * D;
  const int qi = (item % nqb) * (32 * NQG) + 32 * qh + l32;
  // B operands: lane l holds Q (bf16, as given: S^T = K Q^T runs on the bf16 inputs) and dO (fp16)
  // of query qi, features 16 s + 8 (l / 32) ..
  bf16x8 qf[K16];
  f16x8 df[K16];
#pragma unroll
  for (int s = 0; s < K16; ++s) {
    qf[s] = qi < T ? ld_bf16x8(q + base + (int64_t)qi * rs + 16 * s + 8 * hi) : zero_bf16x8();
    df[s] = qi < T ? load_f16x8(doh + base + (int64_t)qi * rs + 16 * s + 8 * hi) : f16x8{};
  }
  const float L = qi < T ? lse[(int64_t)bh * T + qi] : 0.f;
  const float Dd = qi < T ? dvec[(int64_t)bh * T + qi] : 0.f;
  f32x16 dqt[FB];
#pragma unroll
  for (int n = 0; n < FB; ++n) dqt[n] = zero16();

  // Loads of block kb: a wave's loads i = wave + NW m of each tile (row tiles: rows RPI i ..,
  // lane l row RPI i + l / CPR, chunk (l % CPR) ^ (row % CPR); K^T: feature rows 8 i .., lane l row
  // 8 i + l / 8, key chunk (l % 8) ^ (row % 8)).
  auto issue = [&](int kb, unsigned char* kd, unsigned char* vd, unsigned char* td) {
    const int r0 = kb * kAttnBlock;
    const __amdgpu_buffer_rsrc_t rk = rows_rsrc16(reinterpret_cast<const f16*>(k) + base, T, rs, D, r0);  // bf16 bits
    const __amdgpu_buffer_rsrc_t rv = rows_rsrc16(v16 + base, T, rs, D, r0);
    // (base and size made explicitly wave-uniform, so that the descriptor lives in scalar registers)
    const uint64_t kt_addr = reinterpret_cast<uint64_t>(kt16 + ((int64_t)bh * D * tp + r0));
    const uint32_t kt_lo = __builtin_amdgcn_readfirstlane((uint32_t)kt_addr);
    const uint32_t kt_hi = __builtin_amdgcn_readfirstlane((uint32_t)(kt_addr >> 32));
    const __amdgpu_buffer_rsrc_t rkt = __builtin_amdgcn_make_buffer_rsrc(
        reinterpret_cast<void*>(((uint64_t)kt_hi << 32) | kt_lo), (short)0,
        __builtin_amdgcn_readfirstlane(D * tp * 2 - r0 * 2), 0x00020000);
#pragma unroll
    for (int m = 0; m < LPT; ++m) {
      const int i = wave + NW * m, row = RPI * i + lane / CPR;
      const int vo = (lane / CPR) * (int)(rs * 2) + 16 * ((lane % CPR) ^ (row % CPR));
      dma16b(rk, kd + i * 1024, vo, RPI * i * (int)(rs * 2));
      dma16b(rv, vd + i * 1024, vo, RPI * i * (int)(rs * 2));
    }
#pragma unroll
    for (int m = 0; m < LPT; ++m) {
      const int i = wave + NW * m, row = 8 * i + lane / 8;
      dma16b(rkt, td + i * 1024, (lane / 8) * tp * 2 + 16 * ((lane % 8) ^ (row & 7)), 8 * i * tp * 2);
    }
  };
  const int nkb = (T + kAttnBlock - 1) / kAttnBlock;
  issue(0, kr0, vr0, kt0);
  // block kb (odd_c: kb % 2): this wave's loads of it have landed and its reads of block kb - 1
  // are done; after the barrier everyone's are, so block kb + 1 goes into the other stage while
  // block kb is multiplied
  auto kblock = [&](int kb, auto odd_c) {
    constexpr int odd = decltype(odd_c)::value;
    const unsigned char* kc = odd ? kr1 : kr0;
    const unsigned char* vc = odd ? vr1 : vr0;
    const unsigned char* tc = odd ? kt1 : kt0;
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
    __syncthreads();
    if (kb + 1 < nkb) {
      if constexpr (odd) issue(kb + 1, kr0, vr0, kt0);
      else issue(kb + 1, kr1, vr1, kt1);
    }
    // every row fragment is read before the score and dP products, and the K^T fragments
    // before dS^T is formed, so that LDS latency hides behind MFMA and vector work
    bf16x8 ak[K16];
    f16x8 av[K16];
#pragma unroll
    for (int s = 0; s < K16; ++s) {
      const int r = 32 * kh + l32;
      const int ro = r * RB + 16 * ((2 * s + hi) ^ (r % CPR));
      ak[s] = *reinterpret_cast<const bf16x8*>(kc + ro);
      av[s] = *reinterpret_cast<const f16x8*>(vc + ro);
    }
    __builtin_amdgcn_sched_barrier(0);
    f32x16 sc = zero16(), dp = zero16();
#pragma unroll
    for (int s = 0; s < K16; ++s) {
      sc = mfma32(ak[s], qf[s], sc);
      dp = mfma32(av[s], df[s], dp);
    }
    __builtin_amdgcn_sched_barrier(0);
    // A: K^T rows 32 fb + l % 32, keys 32 kh + 16 hh + 8 (j / 4) + 4 (l / 32) + j % 4: stored
    // chunk 4 kh + 2 hh + l / 32 of the row (the copies' quad order)
    f16x8 at[FB][2];
#pragma unroll
    for (int fb = 0; fb < FB; ++fb)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int f = 32 * fb + l32;
        at[fb][hh] = *reinterpret_cast<const f16x8*>(tc + f * 128 + 16 * ((4 * kh + 2 * hh + hi) ^ (f & 7)));
      }
    f16x8 dsb[2];
    // Keys past T need no mask: their K^T columns are zero in the copy, so their dS adds nothing,
    // provided it is finite; the exponent is clamped at 0 (a key of the frame has S scale log2 e
    // <= lse up to rounding, so P <= 1), which keeps every P finite.
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = fast_exp2(fminf(sc[i] * scale_log2 - L, 0.f));
      dsb[i / 8][i % 8] = (f16)(p * (dp[i] - Dd));
    }
#pragma unroll
    for (int fb = 0; fb < FB; ++fb)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) dqt[fb] = mfma32(at[fb][hh], dsb[hh], dqt[fb]);
  };
  int kb = 0;
  for (; kb + 1 < nkb; kb += 2) {
    kblock(kb, std::integral_constant<int, 0>());
    kblock(kb + 1, std::integral_constant<int, 1>());
  }
  if (kb < nkb) kblock(kb, std::integral_constant<int, 0>());
  // the key halves' exchange, in the row tiles (4 KB per wave and feature block)
  constexpr int PER = TILE / 4096;
  static_assert(NQG * FB <= 4 * PER, "the exchange must fit in the row tiles");
  auto xslot = [&](int i) -> f32x16* {
    const int a = i / PER;
    unsigned char* p = a == 0 ? kr0 : a == 1 ? kr1 : a == 2 ? vr0 : vr1;
    return reinterpret_cast<f32x16*>(p + (i % PER) * 4096);
  };
  // lane l, register i: feature 32 fb + 8 (i / 4) + 4 (l / 32) + i % 4 of query qi
  const bool out = !kh && qi < T;
  __syncthreads();
  if (kh) {
#pragma unroll
    for (int fb = 0; fb < FB; ++fb) xslot(qh * FB + fb)[lane] = dqt[fb];
  }
  __syncthreads();
  if (out) {
#pragma unroll
    for (int fb = 0; fb < FB; ++fb) {
      const f32x16 x = dqt[fb] + xslot(qh * FB + fb)[lane];
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        *reinterpret_cast<f32x4*>(dq + base + (int64_t)qi * rs + 32 * fb + 8 * g4 + 4 * hi) =
            f32x4{x[4 * g4], x[4 * g4 + 1], x[4 * g4 + 2], x[4 * g4 + 3]} * scale;
    }
  }
}

// The attention backward in one launch: work-groups [0, G) take dK/dV key blocks, the rest dQ
// query blocks (G = the dK/dV grid rounded up to a multiple of 8, so that both ranges keep the
// XCD-aware order).  dK/dV comes first: its work-groups run longest, and dQ's fill the CUs it
// leaves idle.  The two share one set of LDS arrays (dQ uses six of the eight tiles).
template <int D>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void arl2_bwd_attn_kernel(
    const BwdAttnArgs A) {
  constexpr int TILE = kAttnBlock * 2 * D, NG = 4;
  __shared__ __align__(16) unsigned char t0[TILE], t1[TILE], t2[TILE], t3[TILE], t4[TILE], t5[TILE], t6[TILE],
      t7[TILE];
  __shared__ __align__(16) float lse_s[2][kAttnBlock], dv_s[2][kAttnBlock];
  __shared__ __align__(16) f16x8 p_x[NG][2][2][64];
  const int nkb = (A.T + 32 * NG - 1) / (32 * NG), nqb = (A.T + 32 * NG - 1) / (32 * NG);
  const int g1 = xcd_grid(nkb * A.BH), wg = (int)blockIdx.x;
  if (wg < g1) {
    const int item = xcd_item_at(wg, nkb * A.BH);
    if (item >= 0) dkdv_body<D, NG, TILE>(A, item, t0, t1, t2, t3, t4, t5, t6, t7, lse_s, dv_s, p_x);
  } else {
    const int item = xcd_item_at(wg - g1, nqb * A.BH);
    if (item >= 0) dq_body<D, NG, TILE>(A, item, t0, t1, t2, t3, t4, t5);
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

// The same over rows of a bf16 [.][T][H][D] tensor in global memory: r is a buffer resource
// over one (stream, head) slice, rows [0, T) (rows past T lie outside it and read as zero), voff
// the byte offset of the lane's first row and column, rs2 the row pitch in bytes; the row step
// goes in the scalar offset, so that no load needs address arithmetic of its own.
__device__ __forceinline__ bf16x8 col_frag_global(__amdgpu_buffer_rsrc_t r, int voff, int rs2) {
  bf16x8 a;
#pragma unroll
  for (int j = 0; j < 8; ++j)
    a[j] = __builtin_bit_cast(bf16, __builtin_amdgcn_raw_buffer_load_b16(r, voff, j * rs2, 0));
  return a;
}

// Buffer resource over rows [0, T) of one (stream, head) slice of a bf16 [B][T][H][D] tensor.
template <int D>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t slice_rsrc(const void* x, int64_t base, int T, int64_t rs) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16*>(static_cast<const bf16*>(x) + base), (short)0,
                                           (int)(((int64_t)(T - 1) * rs + D) * 2), 0x00020000);
}

// Output blocks of a d x d chunk sum per wave: an MBW x NBW group, so that each column
// fragment a wave splits from LDS feeds several blocks.
template <int D>
struct SumGroup {
  static constexpr int NB = D / 16;
  static constexpr int MBW = NB >= 8 ? 2 : 1, NBW = NB * NB / 8 / MBW;
  static_assert((NB / MBW) * (NB / NBW) == 8, "one group per wave");
};

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

// B fragments of one 16-column block of NO d x d operands kept in fragment order, every k-step.
template <int D, int NO>
struct FragSet {
  bf16x8 f[NO][BwdShape<D>::KS];
};

// body(nb, fragments of block nb) for nb = 0 .. d/16 - 1, with block nb + 1's fragment loads
// issued before block nb's products (two register sets), so that each block's L2 latency hides
// behind the previous block's MFMAs instead of every MFMA waiting for its own load.
template <int D, int NO, class Body>
__device__ __forceinline__ void pipelined_blocks(const bf16* const (&ops)[NO], int lane, Body&& body) {
  constexpr int KS = BwdShape<D>::KS, NB = BwdShape<D>::NB;
  FragSet<D, NO> fs[2];
  auto load = [&](int nb, FragSet<D, NO>& f) {
#pragma unroll
    for (int o = 0; o < NO; ++o)
#pragma unroll
      for (int s = 0; s < KS; ++s) f.f[o][s] = frag<D>(ops[o], s, nb, lane);
  };
  load(0, fs[0]);
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    if (nb + 1 < NB) load(nb + 1, fs[(nb + 1) & 1]);
    __builtin_amdgcn_sched_barrier(0);
    body(nb, fs[nb & 1]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Inter-frame read of one pass, per (stream, head, 128-token chunk); wave w owns tokens 16 w ..
// 16 w + 15 of the chunk.  dq = (dO S^T) phi_q^T (the dQ kernel adds the softmax branch's part
// later), and the chunk's partial of Gr = Q^T dO.
template <int D>
__global__ __launch_bounds__(512) void arl2_bwd_read_kernel(const BwdTokArgs a) {
  using Sh = BwdShape<D>;
  constexpr int KS = Sh::KS, NB = Sh::NB, LF = Sh::LF;
  __shared__ __align__(16) float ybuf[kTokChunk * LF];  // Y = dO S^T rows (each wave its own)
  __shared__ __align__(16) float dbuf[kTokChunk * LF];  // the chunk's dO rows
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, l16 = lane & 15, g = lane >> 4;
  const int T = a.T, H = a.H, nch = (T + kTokChunk - 1) / kTokChunk;
  const int item = xcd_item(nch * a.B * H);
  if (item < 0) return;
  const int chunk = item % nch, bh = item / nch, b = bh / H, h = bh % H;
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
  {
    const bf16* const ops[2] = {st_hi, st_lo};
    pipelined_blocks<D, 2>(ops, lane, [&](int nb, const FragSet<D, 2>& f) {
      f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) y = mfma3(y, xh[s], xl[s], f.f[0][s], f.f[1][s]);
      store_rows(ybuf, LF, r0, g, 16 * nb + l16, y);
    });
  }
  __syncthreads();
#pragma unroll
  for (int s = 0; s < KS; ++s) row_frag<D>(ybuf, r0 + l16, 32 * s + 8 * g, xh[s], xl[s]);
  {
    const bf16* const ops[1] = {pqt};
    pipelined_blocks<D, 1>(ops, lane, [&](int nb, const FragSet<D, 1>& f) {
      f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        c = mfma16(xh[s], f.f[0][s], c);
        c = mfma16(xl[s], f.f[0][s], c);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t0 + r0 + 4 * g + i;
        if (t < T) a.dq[base + (int64_t)t * rs + 16 * nb + l16] = c[i];
      }
    });
  }
  // Gr partial: wave w owns an MBW x NBW group of the 16x16 blocks of Q^T dO
  using SG = SumGroup<D>;
  constexpr int MBW = SG::MBW, NBW = SG::NBW;
  const int mb0 = MBW * (wave % (NB / MBW)), nb0 = NBW * (wave / (NB / MBW));
  f32x4 p[MBW][NBW];
#pragma unroll
  for (int i = 0; i < MBW; ++i)
#pragma unroll
    for (int j = 0; j < NBW; ++j) p[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const __amdgpu_buffer_rsrc_t rq = slice_rsrc<D>(a.q, base, T, rs);
  const int rs2 = (int)(rs * 2);
#pragma unroll
  for (int s = 0; s < kTokChunk / 32; ++s) {
    bf16x8 aq[MBW];
#pragma unroll
    for (int i = 0; i < MBW; ++i) aq[i] = col_frag_global(rq, (t0 + 32 * s + 8 * g) * rs2 + 2 * (16 * (mb0 + i) + l16), rs2);
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
      bf16x8 bh_, bl_;
      col_frag<D>(dbuf, s, 16 * (nb0 + j) + l16, g, bh_, bl_);
#pragma unroll
      for (int i = 0; i < MBW; ++i) {
        p[i][j] = mfma16(aq[i], bh_, p[i][j]);
        p[i][j] = mfma16(aq[i], bl_, p[i][j]);
      }
    }
    ARL2_BLOCK_FENCE();
  }
  float* part = a.part + ((int64_t)bh * nch + chunk) * D * D;
#pragma unroll
  for (int i = 0; i < MBW; ++i)
#pragma unroll
    for (int j = 0; j < NBW; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) part[(16 * (mb0 + i) + 4 * g + e) * D + 16 * (nb0 + j) + l16] = p[i][j][e];
}

// State write of one frame, per (stream, head, 128-token chunk); wave w owns tokens 16 w ..
// 16 w + 15.  Per token: U = k phi_k, K' = U / max(|U|, eps), V' = v phi_v, R = V' - K' S,
// X3 = R G^T, X = K' G, dbeta = x . r, dR = beta X, dK' = beta X3 - dR S^T, dU; dv += dR phi_v^T,
// dk += dU phi_k^T.  Chunk partials (in this order): K'^T dR, V^T dR, K^T dU.
template <int D>
__global__ __launch_bounds__(512) void arl2_bwd_write_kernel(const BwdTokArgs a) {
  using Sh = BwdShape<D>;
  constexpr int KS = Sh::KS, NB = Sh::NB, LF = Sh::LF;
  __shared__ __align__(16) float abuf[kTokChunk * LF];  // K' rows, later dU rows
  __shared__ __align__(16) float bbuf[kTokChunk * LF];  // R rows, later dR rows
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, l16 = lane & 15, g = lane >> 4;
  const int T = a.T, H = a.H, nch = (T + kTokChunk - 1) / kTokChunk;
  const int item = xcd_item(nch * a.B * H);
  if (item < 0) return;
  const int chunk = item % nch, bh = item / nch, b = bh / H, h = bh % H;
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
  {
    const bf16* const ops[1] = {phik};
    pipelined_blocks<D, 1>(ops, lane, [&](int nb, const FragSet<D, 1>& f) {
      f32x4 u = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) u = mfma16(ka[s], f.f[0][s], u);
      kp[nb] = u;
    });
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
  }
  __syncthreads();
  bf16x8 kh[KS], kl[KS];  // K' as split A fragments
#pragma unroll
  for (int s = 0; s < KS; ++s) row_frag<D>(abuf, r0 + l16, 32 * s + 8 * g, kh[s], kl[s]);
  // R = V' - K' S with V' = v phi_v, into bbuf
  {
    const bf16* const ops[3] = {phiv, s_hi, s_lo};
    pipelined_blocks<D, 3>(ops, lane, [&](int nb, const FragSet<D, 3>& f) {
      f32x4 c = {0.f, 0.f, 0.f, 0.f}, w = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        w = mfma16(va[s], f.f[0][s], w);
        c = mfma3(c, kh[s], kl[s], f.f[1][s], f.f[2][s]);
      }
      store_rows(bbuf, LF, r0, g, 16 * nb + l16, w - c);
    });
  }
  __syncthreads();
  // X3 = R G^T (becomes dK')
  f32x4 dkp[NB];
  {
    bf16x8 rh[KS], rl[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) row_frag<D>(bbuf, r0 + l16, 32 * s + 8 * g, rh[s], rl[s]);
    const bf16* const ops[2] = {gt_hi, gt_lo};
    pipelined_blocks<D, 2>(ops, lane, [&](int nb, const FragSet<D, 2>& f) {
      f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) c = mfma3(c, rh[s], rl[s], f.f[0][s], f.f[1][s]);
      dkp[nb] = c;
    });
  }
  // X = K' G; dbeta = x . r; dR = beta X
  f32x4 dr[NB];
  float db[4] = {0.f, 0.f, 0.f, 0.f};
  {
    const bf16* const ops[2] = {g_hi, g_lo};
    pipelined_blocks<D, 2>(ops, lane, [&](int nb, const FragSet<D, 2>& f) {
      f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) c = mfma3(c, kh[s], kl[s], f.f[0][s], f.f[1][s]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        db[i] += c[i] * bbuf[(r0 + 4 * g + i) * LF + 16 * nb + l16];  // x . r
        dr[nb][i] = bet[i] * c[i];
      }
    });
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
  {
    const bf16* const ops[2] = {st_hi, st_lo};
    pipelined_blocks<D, 2>(ops, lane, [&](int nb, const FragSet<D, 2>& f) {
      f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) c = mfma3(c, dh[s], dl[s], f.f[0][s], f.f[1][s]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        dkp[nb][i] = bet[i] * dkp[nb][i] - c[i];
        cdot[i] += abuf[(r0 + 4 * g + i) * LF + 16 * nb + l16] * dkp[nb][i];  // k' . dK'
      }
    });
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
  {
    // dv before this kernel's share, loaded ahead of the products rather than one element at a
    // time after each
    float prior[NB][4];
    float* rowp[4];  // the lane's column in rows t0 + r0 + 4 (l / 16) + i
#pragma unroll
    for (int i = 0; i < 4; ++i) rowp[i] = a.dv + base + (int64_t)(t0 + r0 + 4 * g + i) * rs + l16;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) prior[nb][i] = t0 + r0 + 4 * g + i < T ? rowp[i][16 * nb] : 0.f;
    const bf16* const ops[1] = {phivt};
    pipelined_blocks<D, 1>(ops, lane, [&](int nb, const FragSet<D, 1>& f) {
      f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        c = mfma16(dh[s], f.f[0][s], c);
        c = mfma16(dl[s], f.f[0][s], c);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t0 + r0 + 4 * g + i;
        if (t < T) rowp[i][16 * nb] = prior[nb][i] + c[i];
      }
    });
  }
  // chunk sums K'^T dR and V^T dR: wave w owns an MBW x NBW group of the 16x16 blocks
  using SG = SumGroup<D>;
  constexpr int MBW = SG::MBW, NBW = SG::NBW;
  const int mb0 = MBW * (wave % (NB / MBW)), nb0 = NBW * (wave / (NB / MBW));
  // partial sum p of 16-column block nb at [bh][p][nb][chunk][row][16]: each (p, nb) strip of all
  // chunks is contiguous for the per-head kernel that adds them
  float* const pbase = a.part + (((int64_t)bh * 3 * NB) * nch + chunk) * D * 16 + l16;
  auto pstore = [&](int p, const f32x4 (&acc)[MBW][NBW]) {
#pragma unroll
    for (int i = 0; i < MBW; ++i)
#pragma unroll
      for (int j = 0; j < NBW; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          pbase[((p * NB + nb0 + j) * nch) * D * 16 + (16 * (mb0 + i) + 4 * g + e) * 16] = acc[i][j][e];
  };
  const int rs2 = (int)(rs * 2);
  const __amdgpu_buffer_rsrc_t rkg = slice_rsrc<D>(a.k, base, T, rs), rvg = slice_rsrc<D>(a.v, base, T, rs);
  // A fragments of the K or V columns of the wave's row blocks for 32-token step s (from global)
  auto gcols = [&](__amdgpu_buffer_rsrc_t r, int s, bf16x8 (&out)[MBW]) {
#pragma unroll
    for (int i = 0; i < MBW; ++i) out[i] = col_frag_global(r, (t0 + 32 * s + 8 * g) * rs2 + 2 * (16 * (mb0 + i) + l16), rs2);
  };
  {
    f32x4 p[MBW][NBW];
#pragma unroll
    for (int i = 0; i < MBW; ++i)
#pragma unroll
      for (int j = 0; j < NBW; ++j) p[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < kTokChunk / 32; ++s) {
      bf16x8 ah[MBW], al[MBW];
#pragma unroll
      for (int i = 0; i < MBW; ++i) col_frag<D>(abuf, s, 16 * (mb0 + i) + l16, g, ah[i], al[i]);
#pragma unroll
      for (int j = 0; j < NBW; ++j) {
        bf16x8 bh_, bl_;
        col_frag<D>(bbuf, s, 16 * (nb0 + j) + l16, g, bh_, bl_);
#pragma unroll
        for (int i = 0; i < MBW; ++i) p[i][j] = mfma3(p[i][j], ah[i], al[i], bh_, bl_);
        ARL2_BLOCK_FENCE();
      }
    }
    pstore(0, p);
#pragma unroll
    for (int i = 0; i < MBW; ++i)
#pragma unroll
      for (int j = 0; j < NBW; ++j) p[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < kTokChunk / 32; ++s) {
      bf16x8 av[MBW];
      gcols(rvg, s, av);
#pragma unroll
      for (int j = 0; j < NBW; ++j) {
        bf16x8 bh_, bl_;
        col_frag<D>(bbuf, s, 16 * (nb0 + j) + l16, g, bh_, bl_);
#pragma unroll
        for (int i = 0; i < MBW; ++i) {
          p[i][j] = mfma16(av[i], bh_, p[i][j]);
          p[i][j] = mfma16(av[i], bl_, p[i][j]);
        }
        ARL2_BLOCK_FENCE();
      }
    }
    pstore(1, p);
  }
  __syncthreads();  // K' is no longer read: dU replaces it
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) store_rows(abuf, LF, r0, g, 16 * nb + l16, dkp[nb]);
  __syncthreads();
  // dk += dU phi_k^T
#pragma unroll
  for (int s = 0; s < KS; ++s) row_frag<D>(abuf, r0 + l16, 32 * s + 8 * g, dh[s], dl[s]);
  {
    // dk before this kernel's share, loaded ahead of the products rather than one element at a
    // time after each
    float prior[NB][4];
    float* rowp[4];  // the lane's column in rows t0 + r0 + 4 (l / 16) + i
#pragma unroll
    for (int i = 0; i < 4; ++i) rowp[i] = a.dk + base + (int64_t)(t0 + r0 + 4 * g + i) * rs + l16;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) prior[nb][i] = t0 + r0 + 4 * g + i < T ? rowp[i][16 * nb] : 0.f;
    const bf16* const ops[1] = {phikt};
    pipelined_blocks<D, 1>(ops, lane, [&](int nb, const FragSet<D, 1>& f) {
      f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        c = mfma16(dh[s], f.f[0][s], c);
        c = mfma16(dl[s], f.f[0][s], c);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t0 + r0 + 4 * g + i;
        if (t < T) rowp[i][16 * nb] = prior[nb][i] + c[i];
      }
    });
  }
  // chunk sum K^T dU
  {
    f32x4 p3[MBW][NBW];
#pragma unroll
    for (int i = 0; i < MBW; ++i)
#pragma unroll
      for (int j = 0; j < NBW; ++j) p3[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < kTokChunk / 32; ++s) {
      bf16x8 ak[MBW];
      gcols(rkg, s, ak);
#pragma unroll
      for (int j = 0; j < NBW; ++j) {
        bf16x8 bh_, bl_;
        col_frag<D>(abuf, s, 16 * (nb0 + j) + l16, g, bh_, bl_);
#pragma unroll
        for (int i = 0; i < MBW; ++i) {
          p3[i][j] = mfma16(ak[i], bh_, p3[i][j]);
          p3[i][j] = mfma16(ak[i], bl_, p3[i][j]);
        }
      }
      ARL2_BLOCK_FENCE();
    }
    pstore(2, p3);
  }
}

// --- sums over chunks, frames' end ---------------------------------------------------------------

// The pass backward's last step: work-groups [0, n_gsum) sum the chunk partials of Q^T dO into
// gr (per (stream, head), blockIdx.x % gsum_x picks the float4s); the rest add the inter-frame
// read's part of dq (dq_read) to the softmax branch's (dq), n4 float4 elements.
__global__ __launch_bounds__(256) void arl2_bwd_finish_kernel(const float* __restrict__ part, float* __restrict__ gr,
                                                              int dd, int nch, int first, int gsum_x, int n_gsum,
                                                              float* __restrict__ dq,
                                                              const float* __restrict__ dq_read, int64_t n4) {
  if ((int)blockIdx.x < n_gsum) {
    const int bh = blockIdx.x / gsum_x, i4 = (blockIdx.x % gsum_x) * 256 + threadIdx.x;
    if (4 * i4 >= dd) return;
    const f32x4* p = reinterpret_cast<const f32x4*>(part + (int64_t)bh * nch * dd) + i4;
    f32x4 s = first ? f32x4{0.f, 0.f, 0.f, 0.f} : reinterpret_cast<const f32x4*>(gr + (int64_t)bh * dd)[i4];
    for (int c = 0; c < nch; ++c) s += p[(int64_t)c * (dd / 4)];
    reinterpret_cast<f32x4*>(gr + (int64_t)bh * dd)[i4] = s;
    return;
  }
  const int64_t stride = (int64_t)(gridDim.x - n_gsum) * 256;
  for (int64_t i = (int64_t)(blockIdx.x - n_gsum) * 256 + threadIdx.x; i < n4; i += stride)
    reinterpret_cast<f32x4*>(dq)[i] += reinterpret_cast<const f32x4*>(dq_read)[i];
}

// End of a frame's backward, per (head, strip of RW = 2048 / d rows of the d x d outputs), streams
// in order:
//   dS_{N-1} = alpha G - sum_chunks K'^T dR + phi_q^T Gr,   dalpha = <G, S_{N-1}> (strip 0),
//   dphi_q += Gr S^T,  dphi_k += sum_chunks K^T dU,  dphi_v += sum_chunks V^T dR.
// 512 threads (two waves per SIMD); thread t owns row RW strip + t / (d / 4) and the 4 columns
// 4 (t mod d / 4) ..: the chunk partials come as float4s, and the d-long dot products read
// phi_q's column strip, Gr and S^T from LDS (per k: two scalars and two float4 for 8
// multiply-adds).
template <int D>
__global__ __launch_bounds__(512) void arl2_bwd_frame_kernel(const BwdFrameArgs a) {
  constexpr int NT = 512, NB = D / 16, NC = D / 4, RW = NT / NC, GP = D + 4;  // threads per row; rows; LDS pitch
  __shared__ __align__(16) float phc[D * RW];  // phi_q[k][RW rt + r]
  __shared__ __align__(16) float grf[D * GP];  // Gr[i][j]
  __shared__ __align__(16) float stf[D * GP];  // S^T[k][j] = S[j][k]
  __shared__ float red[NT];
  const int rt = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int r = tid / NC, c0 = 4 * (tid % NC), row = RW * rt + r;
  const int64_t dd = (int64_t)D * D;
  if (a.gr) {
    const bf16* ph = static_cast<const bf16*>(a.phi_q) + h * dd;
    for (int i = tid; i < D * RW; i += NT) phc[i] = (float)ph[(i / RW) * D + RW * rt + i % RW];
  }
  f32x4 aq = {0.f, 0.f, 0.f, 0.f}, ak = aq, av = aq;
  for (int b = 0; b < a.B; ++b) {
    const int64_t bh = (int64_t)b * a.H + h;
    const float* G = a.g + bh * dd;
    const float* S = a.s_prev + bh * dd;
    // the three sums' partials, [bh][sum][16-column strip][chunk][row][16]: this thread's 4
    // columns sit in strip c0 / 16 at offset c0 % 16
    const float* part = a.part + ((bh * 3) * NB + c0 / 16) * a.chunks * D * 16 + row * 16 + c0 % 16;
    const int64_t pstride = (int64_t)NB * a.chunks * D * 16;  // from one sum to the next
    f32x4 ds = a.alpha[bh] * *reinterpret_cast<const f32x4*>(G + row * D + c0);
#pragma unroll 4
    for (int ch = 0; ch < a.chunks; ++ch) {
      const float* p = part + (int64_t)ch * D * 16;
      ds -= *reinterpret_cast<const f32x4*>(p);
      av += *reinterpret_cast<const f32x4*>(p + pstride);
      ak += *reinterpret_cast<const f32x4*>(p + 2 * pstride);
    }
    if (a.gr) {
      const float* gr = a.gr + bh * dd;
      __syncthreads();  // the previous stream's Gr and S^T are no longer read
      for (int i = tid; i < D * D / 4; i += NT) {
        const int rr = i / (D / 4), cc = 4 * (i % (D / 4));
        *reinterpret_cast<f32x4*>(grf + rr * GP + cc) = *reinterpret_cast<const f32x4*>(gr + rr * D + cc);
        // S^T: consecutive threads take consecutive rows of S, so that the transposed stores of
        // a wave hit consecutive banks
        const int sr = i % D, sc = 4 * (i / D);
        const f32x4 sv = *reinterpret_cast<const f32x4*>(S + sr * D + sc);
#pragma unroll
        for (int e = 0; e < 4; ++e) stf[(sc + e) * GP + sr] = sv[e];
      }
      __syncthreads();
#pragma unroll 8
      for (int k = 0; k < D; ++k) {
        const float pq = phc[k * RW + r], gq = grf[row * GP + k];
        ds += pq * *reinterpret_cast<const f32x4*>(grf + k * GP + c0);  // (phi_q^T Gr)[row][col]
        aq += gq * *reinterpret_cast<const f32x4*>(stf + k * GP + c0);  // (Gr S^T)[row][col]
      }
    }
    *reinterpret_cast<f32x4*>(a.ds_prev + bh * dd + row * D + c0) = ds;
    if (rt == 0) {  // dalpha over the whole matrix (all loads of a thread in flight at once)
      float sum = 0.f;
#pragma unroll
      for (int it = 0; it < D * D / (4 * NT); ++it) {
        const int i = tid + NT * it;
        const f32x4 x = reinterpret_cast<const f32x4*>(G)[i], y = reinterpret_cast<const f32x4*>(S)[i];
        sum += x[0] * y[0] + x[1] * y[1] + x[2] * y[2] + x[3] * y[3];
      }
      red[tid] = sum;
      __syncthreads();
      for (int w = NT / 2; w > 0; w >>= 1) {
        if (tid < w) red[tid] += red[tid + w];
        __syncthreads();
      }
      if (tid == 0) a.dalpha[bh] = red[0];
    }
  }
  const int64_t o = (int64_t)h * dd + row * D + c0;
  *reinterpret_cast<f32x4*>(a.dphi_q + o) += aq;
  *reinterpret_cast<f32x4*>(a.dphi_k + o) += ak;
  *reinterpret_cast<f32x4*>(a.dphi_v + o) += av;
}

// dst[i] = src ? src[i] : 0 (n4 float4 elements); a kernel rather than a memset node, so that the
// calls stay correct inside a captured graph.
__global__ __launch_bounds__(256) void arl2_bwd_fill_kernel(float* __restrict__ dst, const float* __restrict__ src,
                                                            int64_t n4) {
  for (int64_t i = blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256)
    reinterpret_cast<f32x4*>(dst)[i] = src ? reinterpret_cast<const f32x4*>(src)[i] : f32x4{0.f, 0.f, 0.f, 0.f};
}

template <int D>
hipError_t launch_bwd_stage_d(BwdStage stage, const BwdPassArgs& a, hipStream_t stream) {
  const int BH = a.B * a.H;
  const bf16* q = static_cast<const bf16*>(a.tok.q);
  const bf16* k = static_cast<const bf16*>(a.tok.k);
  const bf16* v = static_cast<const bf16*>(a.tok.v);
  const f16* doh = static_cast<const f16*>(a.do_h);
  const int nch = (a.T + kTokChunk - 1) / kTokChunk;
  switch (stage) {
    case BwdStage::kRead: {
      BwdTokArgs t = a.tok;
      t.dq = a.dq_read;
      hipLaunchKernelGGL(arl2_bwd_read_kernel<D>, dim3(xcd_grid(nch * BH)), dim3(512), 0, stream, t);
      break;
    }
    case BwdStage::kPrep:
      hipLaunchKernelGGL(arl2_bwd_cvt16_kernel<D>, dim3(a.tp / kAttnBlock, BH), dim3(256), 0, stream, q, k, v, a.d_out,
                         a.o_sm, static_cast<f16*>(a.do_h), a.dvec, static_cast<f16*>(a.v16),
                         static_cast<f16*>(a.kt16), static_cast<f16*>(a.qt16), static_cast<f16*>(a.dot16), a.T, a.H,
                         a.tp);
      break;
    case BwdStage::kAttn: {
      BwdAttnArgs A;
      A.q = q;
      A.k = k;
      A.v = v;
      A.doh = doh;
      A.v16 = static_cast<const f16*>(a.v16);
      A.kt16 = static_cast<const f16*>(a.kt16);
      A.qt16 = static_cast<const f16*>(a.qt16);
      A.dot16 = static_cast<const f16*>(a.dot16);
      A.lse = a.lse;
      A.dvec = a.dvec;
      A.dk = a.tok.dk;
      A.dv = a.tok.dv;
      A.dq = a.tok.dq;
      A.T = a.T;
      A.H = a.H;
      A.BH = BH;
      A.tp = a.tp;
      A.scale = a.scale;
      A.scale_log2 = a.scale_log2;
      const int nb = (a.T + 127) / 128;  // 128-key (dK/dV) and 128-query (dQ) blocks per head
      hipLaunchKernelGGL(arl2_bwd_attn_kernel<D>, dim3(2 * xcd_grid(nb * BH)), dim3(512), 0, stream, A);
      break;
    }
    case BwdStage::kFinish: {
      const int gsum_x = (D * D / 4 + 255) / 256, n_gsum = gsum_x * BH;
      const int64_t n4 = (int64_t)a.B * a.T * a.H * D / 4;
      const int n_add = (int)std::min<int64_t>((n4 + 255) / 256, 1024);
      hipLaunchKernelGGL(arl2_bwd_finish_kernel, dim3(n_gsum + n_add), dim3(256), 0, stream, a.tok.part, a.gr, D * D,
                         nch, a.gr_first ? 1 : 0, gsum_x, n_gsum, a.tok.dq, a.dq_read, n4);
      break;
    }
    default:
      return hipErrorInvalidValue;
  }
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
  hipLaunchKernelGGL(arl2_bwd_write_kernel<D>, dim3(xcd_grid(nch * t.B * t.H)), dim3(512), 0, stream, t);
  hipLaunchKernelGGL(arl2_bwd_frame_kernel<D>, dim3(D / (2048 / D), t.H), dim3(512), 0, stream, f);
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

int bwd_key_pitch(int T) { return (T + kAttnBlock - 1) / kAttnBlock * kAttnBlock; }

hipError_t launch_bwd_stage(int d, BwdStage stage, const BwdPassArgs& a, hipStream_t stream) {
  switch (d) {
    case 64: return launch_bwd_stage_d<64>(stage, a, stream);
    case 128: return launch_bwd_stage_d<128>(stage, a, stream);
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
