// State write of the ARL2 layer, per-chunk part, run as extra work-groups of the pass kernel
// in the clean pass's launch:
//   P_c = K'_c^T diag(beta_c) (V'_c - K'_c S_{N-1}),
//   K' = rows of K phi_k scaled to unit length,  V' = V phi_v,
// over the chunk's 128 tokens; the reduce kernel then forms S_N = alpha S_{N-1} + sum_c P_c.
// ("Attend Locally, Remember Linearly", gist.science technical summary, section 2.1: the
// gated update and the per-head 1x1 maps; section 2.2: one write per frame, after the clean
// pass, with every token's residual taken against the same S_{N-1}.)
//
// Why in the pass's grid.  The pass runs one 128-query work-group per CU and, at the frame
// sizes of a video DiT layer, fewer work-groups than the chip has CUs.  The write only reads
// S_{N-1}, so it does not depend on the pass; its work-groups come after the pass's in the
// same grid, so the dispatcher places them on the CUs the pass leaves idle (a pass
// work-group's LDS leaves no room for a second work-group on its CU), and no pass
// work-group ever waits for a CU.  They use the pass kernel's block size, register budget
// (8 waves, at most 256 registers each) and LDS arrays.
//
// One work-group per (stream, head, 128-token chunk).  Wave w owns tokens 16 w .. 16 w + 15
// of the chunk and forms on its own, with 16x16x32 MFMAs: K'^T (key features x tokens; the
// row norms, and the A operand of K' S), R = V' - K' S (tokens x value features), and K'
// (tokens x key features).  The token contraction P_c = sum over the chunk of K'^T (beta R)
// then reads the K' and beta R fragments of all waves from LDS, each wave owning a group of
// output blocks.
//
// Precision: K', S and beta R enter the MFMAs as bf16 hi + lo pairs (x = hi + lo to about 16
// mantissa bits; products hi*hi + hi*lo + lo*hi), because a single bf16 rounding of any of
// them costs more than the state tolerance over a long stream.  K, V and the maps are exact
// in bf16 and need no split.
#pragma once

#include "arl2_device.h"
#include "arl2_kernels.h"

// Lambdas here are always inlined (with their captures in registers, not on the stack).
#define ARL2_WRITE_INLINE __attribute__((always_inline))

namespace arl2 {

template <int D>
struct WriteShape {
  static constexpr int DP = D < 32 ? 32 : D;  // padded features (input, key and value)
  static constexpr int KS = DP / 32;         // 32-deep k-steps over features
  static constexpr int FB = DP / 16;         // 16-wide blocks over features
  // LDS in 1-KB fragment slots (16 bytes per lane).  Region A: phi_k^T fragments [block][k-step],
  // then phi_v^T; after the per-wave products, K' over tokens [32-token step][key block][hi, lo].
  // Region B: -S hi fragments [k-step][value block], then lo; after the per-wave products,
  // beta R over tokens [32-token step][value block][hi, lo].
  static constexpr int NMF = FB * KS;  // fragments of one map, and of one term of -S
  static constexpr int TOK_SLOTS = 4 * FB * 2;
  static constexpr int A_SLOTS = 2 * NMF > TOK_SLOTS ? 2 * NMF : TOK_SLOTS;
  static constexpr int B_SLOTS = 2 * NMF > TOK_SLOTS ? 2 * NMF : TOK_SLOTS;
};

namespace write_detail {

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, bytes, 0x00020000);
}
// 16 bytes per lane from the buffer straight into LDS at lds + 16 * lane (lds wave-uniform).
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, unsigned char* lds, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, voff, 0, 0, 0);
}
// Wait until at most N of this wave's vector memory loads are in flight (N < 64; loads complete
// in issue order).  The count's low 4 bits and high 2 bits sit apart in the instruction.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}
__device__ __forceinline__ bf16x8 frag(const unsigned char* slot, int lane) {
  return *reinterpret_cast<const bf16x8*>(slot + 16 * lane);
}
__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

}  // namespace write_detail

// Work-group item = (stream b, head h, chunk c) as (b H + h) chunks + c.  slot_a(i) / slot_b(i)
// give the LDS address of 1-KB slot i of regions A and B (at least WriteShape<D>::A_SLOTS and
// B_SLOTS slots).  Every wave of the work-group calls this; it contains work-group barriers.
template <int D, class SlotA, class SlotB>
__device__ __attribute__((always_inline)) inline void write_partial(const WritePartialArgs& a, int T, int H,
                                                                   int item, SlotA&& slot_a, SlotB&& slot_b) {
  using namespace write_detail;
  using W = WriteShape<D>;
  constexpr int DP = W::DP, KS = W::KS, FB = W::FB, NMF = W::NMF;
  const int n_chunks = commit_chunks(T);
  const int chunk = item % n_chunks, bh = item / n_chunks;
  const int h = bh % H, b = bh / H;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, g4 = lane >> 4;
  const int64_t rs = (int64_t)H * D;
  const int t0 = chunk * kCommitChunk;
  const int tw = t0 + 16 * wave;  // this wave's first token

  // The lane's column token (tw + r16): its beta (zero past the frame).
  const float beta_l = tw + r16 < T ? a.beta[((int64_t)b * T + tw + r16) * H + h] : 0.f;

  // Loads, in the order the products need them: phi_k^T fragments (into LDS, dealt over the
  // waves) and the lane's K row, phi_v^T and the V row, then -S hi / lo.  K and V come through
  // buffer loads over the (stream, head) slice, so rows past the frame read as zeros.
  const int64_t base = ((int64_t)b * T * H + h) * D;
  const int slice_bytes = (int)(((int64_t)(T - 1) * rs + D) * 2);
  const __amdgpu_buffer_rsrc_t rk = rsrc(static_cast<const bf16*>(a.k) + base, slice_bytes);
  const __amdgpu_buffer_rsrc_t rv = rsrc(static_cast<const bf16*>(a.v) + base, slice_bytes);
  const __amdgpu_buffer_rsrc_t rpk = rsrc(static_cast<const bf16*>(a.pkt) + (int64_t)h * DP * DP, DP * DP * 2);
  const __amdgpu_buffer_rsrc_t rpv = rsrc(static_cast<const bf16*>(a.pvt) + (int64_t)h * DP * DP, DP * DP * 2);
  const __amdgpu_buffer_rsrc_t rsh = rsrc(static_cast<const bf16*>(a.sneg_hi) + (int64_t)bh * NMF * 512, NMF * 1024);
  const __amdgpu_buffer_rsrc_t rsl = rsrc(static_cast<const bf16*>(a.sneg_lo) + (int64_t)bh * NMF * 512, NMF * 1024);
  // map fragment f = (block f / KS, k-step f % KS): lane l reads row 16 (f / KS) + l % 16,
  // features 32 (f % KS) + 8 (l / 16) ..
  auto map_off = [&](int f) ARL2_WRITE_INLINE { return ((16 * (f / KS) + r16) * DP + 32 * (f % KS) + 8 * g4) * 2; };
  // token row tw + l % 16, features 32 st + 8 (l / 16) ..; features past d (d < 32) read as zero
  const int row_off = (int)((int64_t)(tw + r16) * rs * 2) + 16 * g4;
  auto row_load = [&](__amdgpu_buffer_rsrc_t r, int st) ARL2_WRITE_INLINE {
    const bf16x8 x = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, row_off + 64 * st, 0, 0));
    return (D >= 32 || 32 * st + 8 * g4 < D) ? x : zero_bf16x8();
  };
  constexpr bool EVEN = NMF % 8 == 0;  // every wave issues the same number of fragment loads
  constexpr int NW = NMF / 8;          // fragment loads per wave and operand when EVEN
  bf16x8 kf[KS], vf[KS];
  asm volatile("" ::: "memory");  // the counted loads below keep their order
  for (int f = wave; f < NMF; f += 8) dma16(rpk, slot_a(f), map_off(f));
#pragma unroll
  for (int st = 0; st < KS; ++st) kf[st] = row_load(rk, st);
  for (int f = wave; f < NMF; f += 8) dma16(rpv, slot_a(NMF + f), map_off(f));
#pragma unroll
  for (int st = 0; st < KS; ++st) vf[st] = row_load(rv, st);
  for (int f = wave; f < NMF; f += 8) {
    dma16(rsh, slot_b(f), 1024 * f + 16 * lane);
    dma16(rsl, slot_b(NMF + f), 1024 * f + 16 * lane);
  }
  asm volatile("" ::: "memory");
  wait_vmcnt<EVEN ? 3 * NW + KS : 0>();  // phi_k^T (this wave's share) and the K row
  __syncthreads();

  // K'^T = phi_k^T K^T before the row scaling: rows = key features, lane column = token.
  f32x4 kt[FB];
#pragma unroll
  for (int mb = 0; mb < FB; ++mb) {
    kt[mb] = zero4();
#pragma unroll
    for (int st = 0; st < KS; ++st) kt[mb] = mfma16(frag(slot_a(mb * KS + st), lane), kf[st], kt[mb]);
  }
  // Row norms: a lane holds 4 of its token's key features per block; the rest sit in lanes
  // l ^ 16, l ^ 32 and l ^ 48.
  float ss = 0.f;
#pragma unroll
  for (int mb = 0; mb < FB; ++mb)
#pragma unroll
    for (int i = 0; i < 4; ++i) ss = fmaf(kt[mb][i], kt[mb][i], ss);
  ss += __shfl_xor(ss, 16);
  ss += __shfl_xor(ss, 32);
  const float inv = 1.f / fmaxf(sqrtf(ss), a.knorm_eps);
  // K' as the A operand of K' S: k-step ks = key features 32 ks .. 32 ks + 31 from blocks 2 ks and
  // 2 ks + 1, split into hi and lo.
  bf16x8 khi[KS], klo[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const Bf16Pair sp = split_bf16(kt[2 * ks + (j >> 2)][j & 3] * inv);
      khi[ks][j] = sp.hi;
      klo[ks][j] = sp.lo;
    }

  wait_vmcnt<0>();  // phi_v^T, the V row and -S
  __syncthreads();
  // R = V phi_v + K' (-S): rows = tokens, lane column = value feature.
  f32x4 r[FB];
#pragma unroll
  for (int nb = 0; nb < FB; ++nb) {
    r[nb] = zero4();
#pragma unroll
    for (int st = 0; st < KS; ++st) r[nb] = mfma16(vf[st], frag(slot_a(NMF + nb * KS + st), lane), r[nb]);
  }
  // (per k-step, each of the three products over all value blocks in turn, so that consecutive
  // MFMAs go to different accumulators)
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    bf16x8 sh[FB], sl[FB];
#pragma unroll
    for (int nb = 0; nb < FB; ++nb) {
      sh[nb] = frag(slot_b(ks * FB + nb), lane);
      sl[nb] = frag(slot_b(NMF + ks * FB + nb), lane);
    }
#pragma unroll
    for (int nb = 0; nb < FB; ++nb) r[nb] = mfma16(khi[ks], sh[nb], r[nb]);
#pragma unroll
    for (int nb = 0; nb < FB; ++nb) r[nb] = mfma16(khi[ks], sl[nb], r[nb]);
#pragma unroll
    for (int nb = 0; nb < FB; ++nb) r[nb] = mfma16(klo[ks], sh[nb], r[nb]);
  }
  // K' = K phi_k (rows = tokens, lane column = key feature): the operands of K'^T swapped.
  f32x4 kk[FB];
#pragma unroll
  for (int mb = 0; mb < FB; ++mb) {
    kk[mb] = zero4();
#pragma unroll
    for (int st = 0; st < KS; ++st) kk[mb] = mfma16(kf[st], frag(slot_a(mb * KS + st), lane), kk[mb]);
  }
  // Row i of the lane's blocks is token tw + 4 (l / 16) + i: its inverse norm and beta come
  // from the lane that holds that token as its column.
  float inv_i[4], beta_i[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    inv_i[i] = __shfl(inv, 4 * g4 + i);
    beta_i[i] = __shfl(beta_l, 4 * g4 + i);
  }
  __syncthreads();  // every wave is done with the maps and -S

  // K' and beta R over tokens: this wave's 16 tokens are half hf of 32-token step ts, i.e.
  // elements 4 hf .. 4 hf + 3 of each lane's 16 bytes in the fragments of step ts.
  const int ts = wave >> 1, hf = wave & 1;
  auto put = [&](unsigned char* hi_slot, unsigned char* lo_slot, const f32x4& x, const float (&s)[4])
                 ARL2_WRITE_INLINE {
    bf16x4 hi, lo;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const Bf16Pair sp = split_bf16(x[i] * s[i]);
      hi[i] = sp.hi;
      lo[i] = sp.lo;
    }
    *reinterpret_cast<bf16x4*>(hi_slot + 16 * lane + 8 * hf) = hi;
    *reinterpret_cast<bf16x4*>(lo_slot + 16 * lane + 8 * hf) = lo;
  };
#pragma unroll
  for (int mb = 0; mb < FB; ++mb) put(slot_a((ts * FB + mb) * 2), slot_a((ts * FB + mb) * 2 + 1), kk[mb], inv_i);
#pragma unroll
  for (int nb = 0; nb < FB; ++nb) put(slot_b((ts * FB + nb) * 2), slot_b((ts * FB + nb) * 2 + 1), r[nb], beta_i);
  __syncthreads();

  // P_c block (mb, nb) = sum over the chunk's 32-token steps of K'^T (beta R); steps wholly past
  // the frame hold zeros and are skipped.  Wave w owns an MBW x NBW group of output blocks, so
  // that each fragment it reads from LDS feeds NBW or MBW blocks.
  constexpr int MBW = FB >= 8 ? 2 : 1, NBW = FB >= 8 ? 4 : FB >= 4 ? 2 : 1;
  constexpr int GROUPS = (FB / MBW) * (FB / NBW);
  static_assert(GROUPS <= 8, "one block group per wave");
  const int nts = min(4, (T - t0 + 31) / 32);
  float* pout = a.partial + (int64_t)item * DP * DP;
  if (wave < GROUPS) {
    const int mb0 = MBW * (wave % (FB / MBW)), nb0 = NBW * (wave / (FB / MBW));
    f32x4 p[MBW][NBW];
#pragma unroll
    for (int i = 0; i < MBW; ++i)
#pragma unroll
      for (int j = 0; j < NBW; ++j) p[i][j] = zero4();
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (t < nts) {
        bf16x8 ah[MBW], al[MBW], bh[NBW], bl[NBW];
#pragma unroll
        for (int i = 0; i < MBW; ++i) {
          ah[i] = frag(slot_a((t * FB + mb0 + i) * 2), lane);
          al[i] = frag(slot_a((t * FB + mb0 + i) * 2 + 1), lane);
        }
#pragma unroll
        for (int j = 0; j < NBW; ++j) {
          bh[j] = frag(slot_b((t * FB + nb0 + j) * 2), lane);
          bl[j] = frag(slot_b((t * FB + nb0 + j) * 2 + 1), lane);
        }
#pragma unroll
        for (int i = 0; i < MBW; ++i)
#pragma unroll
          for (int j = 0; j < NBW; ++j) p[i][j] = mfma16(ah[i], bh[j], p[i][j]);
#pragma unroll
        for (int i = 0; i < MBW; ++i)
#pragma unroll
          for (int j = 0; j < NBW; ++j) p[i][j] = mfma16(ah[i], bl[j], p[i][j]);
#pragma unroll
        for (int i = 0; i < MBW; ++i)
#pragma unroll
          for (int j = 0; j < NBW; ++j) p[i][j] = mfma16(al[i], bh[j], p[i][j]);
      }
    }
#pragma unroll
    for (int i = 0; i < MBW; ++i)
#pragma unroll
      for (int j = 0; j < NBW; ++j) {
        const int blk = (mb0 + i) * FB + nb0 + j;
#pragma unroll
        for (int e = 0; e < 4; ++e) pout[(blk * 4 + e) * 64 + lane] = p[i][j][e];
      }
  }
}

}  // namespace arl2
