// Fused per-pass kernel of the ARL2 layer:
//   out = softmax(Q K^T * scale) V + Q W,   W = phi_q S_{N-1}
// ("Attend Locally, Remember Linearly", gist.science technical summary, section 2.1:
// intra-frame softmax branch and inter-frame output Q' S_{N-1} with Q' = Q phi_q; section
// 2.2: every token of the frame reads the same pre-update state).  Q' S = Q (phi_q S) by
// associativity; W is formed once per frame by the state-write kernels, so a pass only
// adds a Q x W product to the attention accumulator.
//
// Work decomposition.  One work-group of 8 waves, two per SIMD, per (stream, head, 128-query
// tile).  Wave w owns the 32 query rows w % 4 of the tile and one half of the frame's keys
// (w / 4); the two halves of a row block are merged through LDS at the end (max / sum
// rescaling), so no partial result leaves the chip.  The two waves on a SIMD work on
// different key halves with no ordering between them inside an iteration, so the matrix
// cores run one wave's MFMAs while the vector ALU runs the other's softmax: the overlap
// that one wave cannot get from its own in-order instruction stream.  Every K or V fragment
// a wave reads from LDS feeds one MFMA; at the full MFMA rate the CU reads 128 bytes per
// clock, half of what gfx950's LDS delivers.  The four waves of a key half share its staging.
//
// Pipeline.  A wave walks its keys in units of 32.  Step u overlaps the score MFMAs of unit
// u+1 (S^T = K Q^T) with the VALU softmax of unit u (phase A), then the O^T += V^T P^T MFMAs
// of unit u with the row max of unit u+1 (phase B); each phase is a few short stages closed
// by scheduling barriers, and LDS fragments are read two stages ahead of their MFMAs.  Keys
// are staged per 64-key iteration (two units, one work-group barrier): K as 32-key
// half-tiles in a ring of four LDS slots per key half (direct-to-LDS buffer loads), since
// an iteration's units read the second half of one tile and the first half of the next;
// V^T as whole 64-key tiles, double-buffered, through registers: each thread transposes
// 4-key x 8-feature blocks, converting them to fp16 on the way, and stores them in the key
// order of the P^T fragments, in rows padded by 16 bytes so that fragment reads (32
// consecutive rows) are conflict-free 16-byte loads.  Rows past the end of the frame lie
// outside the buffer descriptors and read as zeros.
//
// Precision.  The P V product runs in fp16 (same MFMA rate as bf16): P, at most 2^8 (see
// below), is rounded to nearest fp16 (relative step 2^-11, eight times finer than bf16, whose
// rounding of P alone puts the output error at the edge of a 2e-2 budget on long streams),
// and V converts from bf16 to fp16 exactly for 2^-14 <= |v| <= 65504 (smaller values round
// to fp16 subnormals, absolute step 2^-24; larger ones become infinite, so they show up
// instead of being clipped).  Q K^T and the Q W term stay bf16 x bf16 with
// fp32 accumulation.
//
// Scores are transposed so that every lane holds one query row and 16 of the unit's keys:
// the row max needs one cross-lane exchange (l, l ^ 32), the row sum none until the end,
// and rescaling the transposed accumulator is a per-lane multiply.  Softmax: exp2 with the
// scale folded in; the running max is only raised when a unit's max exceeds it by more than
// 8 (in log2 units) in some lane of the wave, so P stays below 2^8 and the rescale of the
// accumulator is skipped on almost every unit.  Row sums add the rounded P that enters the
// MFMA, two fp16 values per dot-product instruction with fp32 accumulation.
#include <type_traits>

#include "arl2_device.h"
#include "arl2_kernels.h"
#include "arl2_write_partial.h"

namespace arl2 {
namespace {

constexpr int kQTile = 128;  // query rows per work-group
constexpr int kKV = 64;      // keys per staging iteration (two units)
constexpr int kUnit = 32;    // keys per pipeline unit
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kHalfThreads = kThreads / 2;  // staging threads of one key half (its four waves)
constexpr float kRescaleSlack = 8.f;        // log2 headroom before the running max is raised

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
// Lambdas of the kernel are always inlined (large generic lambdas would otherwise become calls
// with their captures on the stack).
#define ARL2_INLINE __attribute__((always_inline))

using On = std::true_type;
using Off = std::false_type;
template <int N>
using Ic = std::integral_constant<int, N>;

template <int D>
struct FwdShape {
  static constexpr int DP = D < 32 ? 32 : D;  // padded feature rows of the O^T / V^T blocks
  static constexpr int KS = D / 16;          // 16-wide k-steps over features
  static constexpr int MB = DP / 32;         // 32-row blocks over output features
  static constexpr int CPR = D / 8;          // 16-byte chunks per token row
  static constexpr int VBLK = 16 * CPR;      // 4-key x 8-feature blocks per V tile
  static constexpr int VPT = (VBLK + kHalfThreads - 1) / kHalfThreads;  // such blocks per staging thread
  static constexpr int VLD = kKV + 8;        // V^T row stride in fp16 (64 keys + 16 bytes of padding)
  // K half-tile: 32 rows of 2D bytes, row-major, with the 16-byte granules of row r permuted
  // (granule g holds feature chunk g ^ (r mod CPR)).  Every direct-to-LDS load then brings
  // RPI whole rows (contiguous in memory), and the 32 rows of an MFMA fragment read land on
  // distinct banks.
  static constexpr int KH_BYTES = KS * kUnit * 32;
  static constexpr int RB = 2 * D;                  // bytes per row
  static constexpr int RPI = 1024 / RB;             // rows per 1-KB load
  static constexpr int NKV = CPR * CPR / 64 > 1 ? CPR * CPR / 64 : 1;  // distinct lane offsets of the loads
  static constexpr int VT_BYTES = DP * VLD * 2;
  static constexpr int NA = KS < 4 ? KS : 4;          // stages of phase A
  static constexpr int NB = 2 * MB < 4 ? 2 * MB : 4;  // stages of phase B
  static constexpr int FA = KS / NA;                  // K fragments per A stage
  static constexpr int FB = 2 * MB / NB;              // V^T fragments per B stage
  static constexpr int KPW = (2 * KS + 3) / 4;        // K half-tile loads per wave per iteration
};

// Buffer resource over rows [first_row, T) of one (stream, head) slice of a [B][T][H][d]
// tensor: anything past the frame lies outside num_records, and loads there return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const bf16* base, int T, int64_t rs, int d, int first_row) {
  const int64_t start = (int64_t)first_row * rs;
  const int64_t left = (int64_t)(T - 1) * rs + d - start;
  const bool any = left > 0;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16*>(any ? base + start : base), (short)0,
                                           any ? (int)(left * 2) : 0, 0x00020000);
}

// voff: per-lane byte offset; soff: wave-uniform byte offset (kept in a scalar register).
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  return make_uint4(x.x, x.y, x.z, x.w);
}

// 16 bytes per lane from the buffer straight into LDS at lds + 16 * lane (lds wave-uniform).
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, void* lds, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, voff, soff, 0, 0);
}

// Pins a value to the architectural VGPRs at this point.  MFMA results may land in AGPRs; a
// score block that the VALU is about to read moves over once, here.
__device__ __forceinline__ void to_vgpr(f32x16& x) { asm volatile("" : "+v"(x)); }

// Marks a value as produced at this point, so that the compiler does not sink its computation
// into a later stage (stages are laid out so that VALU work overlaps the MFMAs of its stage).
template <class T>
__device__ __forceinline__ void pin(T& x) {
  asm volatile("" : "+v"(x));
}

// Wait until all of this wave's vector memory operations (including loads into LDS) are done.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Wait until at most n of this wave's vector memory loads are in flight (n < 16).  Loads
// complete in issue order, so this waits for every load issued before the last n.
template <int N>
__device__ __forceinline__ void wait_vmem_but() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

// INTER: the ARL2 pass (the Q W term; state-write work-groups after n_pass_blocks).  Without it,
// plain softmax attention of the T queries over keys [0, Tk) of k / v (whose stream slices are
// kv_rows rows apart): the retained softmax layers' attention over their K/V cache, or, with
// `add` (fp32, the output's layout) added to the result, the softmax branch of the
// token-level access variant.
template <int D, bool OUT_BF16, bool INTER>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void arl2_fwd_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ wt_hi, const bf16* __restrict__ wt_lo, void* __restrict__ out,
    int T, int Tk, int kv_rows, int H, int nq, int n_bh, float scale_log2, int n_pass_blocks,
    const WritePartialArgs wa, int n_write, const float* __restrict__ add, float* __restrict__ lse) {
  using S = FwdShape<D>;
  constexpr int DP = S::DP, KS = S::KS, MB = S::MB, VLD = S::VLD, VBLK = S::VBLK, VPT = S::VPT,
                KH_BYTES = S::KH_BYTES, VT_BYTES = S::VT_BYTES, NA = S::NA, NB = S::NB, FA = S::FA, FB = S::FB,
                KPW = S::KPW;

  // LDS: the four K ring slots and the two V^T buffers are separate arrays ([key half][...]
  // each), addressed with compile-time slot numbers (the steady loop is unrolled by iteration
  // parity), so that the compiler can tell the LDS accesses of an iteration from the
  // direct-to-LDS loads in flight into other slots and does not wait for those loads.  After
  // the loop the K arrays hold W^T (hi, lo) and the V arrays the exchange between the halves.
  constexpr int KA_BYTES = 2 * KH_BYTES, VA_BYTES = 2 * VT_BYTES;
  __shared__ __attribute__((aligned(64))) unsigned char ks0[KA_BYTES], ks1[KA_BYTES], ks2[KA_BYTES], ks3[KA_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char vs0[VA_BYTES], vs1[VA_BYTES];
  auto karr = [&](auto slot_c) ARL2_INLINE -> unsigned char* {
    constexpr int sl = decltype(slot_c)::value & 3;
    if constexpr (sl == 0) return ks0;
    else if constexpr (sl == 1) return ks1;
    else if constexpr (sl == 2) return ks2;
    else return ks3;
  };
  auto varr = [&](auto buf_c) ARL2_INLINE -> unsigned char* {
    if constexpr ((decltype(buf_c)::value & 1) == 0) return vs0;
    else return vs1;
  };

  // The exchange between the key halves in the epilogue (for d < 128 an array of its own; LDS
  // is plentiful there).
  constexpr int MBH = MB >= 2 ? MB / 2 : 1;
  constexpr int NXV = MBH * 4 + 1;     // exported 16-byte rows: accumulator quads, then (m, l)
  constexpr int NX = MB >= 2 ? 8 : 4;  // exporting waves
  constexpr int XS_BYTES = NXV * 64 * 16, XS_PER = VA_BYTES / XS_BYTES;  // exchange slots per V array
  constexpr bool XFIT = XS_PER >= 1 && (NX + XS_PER - 1) / XS_PER <= 2;
  __shared__ __attribute__((aligned(16))) unsigned char xs_own[XFIT ? 16 : NX * XS_BYTES];

  // Work-groups past the pass's: the state write's per-chunk partial sums of the clean pass's
  // launch, in the same LDS arrays (region A: the K arrays, or the exchange array where the
  // K arrays are too small; region B: the V arrays).
  if (INTER && (int)blockIdx.x >= n_pass_blocks) {
    using WS = WriteShape<D>;
    constexpr int KA_KB = KA_BYTES / 1024, VA_KB = VA_BYTES / 1024;
    constexpr bool A_IN_K = 4 * KA_KB >= WS::A_SLOTS;
    static_assert(A_IN_K || (int)sizeof(xs_own) >= WS::A_SLOTS * 1024, "state-write region A must fit");
    static_assert(2 * VA_KB >= WS::B_SLOTS, "state-write region B must fit");
    auto slot_a = [&](int i) ARL2_INLINE -> unsigned char* {
      if constexpr (A_IN_K) {
        const int a = i / KA_KB;
        return (a == 0 ? ks0 : a == 1 ? ks1 : a == 2 ? ks2 : ks3) + (i % KA_KB) * 1024;
      } else {
        return xs_own + i * 1024;
      }
    };
    auto slot_b = [&](int i) ARL2_INLINE -> unsigned char* { return i < VA_KB ? vs0 + i * 1024 : vs1 + (i - VA_KB) * 1024; };
    // XCD-aware like the pass's items below: each XCD gets a contiguous run of chunks.
    const int wp = (int)blockIdx.x - n_pass_blocks, per = (n_write + 7) / 8;
    const int witem = (wp & 7) * per + (wp >> 3);
    if (witem < n_write) write_partial<D>(wa, T, H, witem, slot_a, slot_b);
    return;
  }

  // XCD-aware order: work-groups are dealt to the 8 XCDs round-robin (work-group i runs on XCD
  // i % 8), so each XCD gets a contiguous run of items (the query tiles of one head, then the
  // next head's): a head's K and V come into one or two L2 caches, and every XCD gets the same
  // number of work-groups.  (Dealing whole heads to XCDs saves the second L2 fill but leaves
  // the XCDs unevenly loaded, which costs more.)
  const int n_items = nq * n_bh, per_xcd = (n_items + 7) / 8;
  const int item = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (item >= n_items) return;
  const int qt = item % nq, bh = item / nq;
  const int h = bh % H, b = bh / H;

  // wave-uniform indices are made explicitly uniform (scalar registers), so that buffer
  // descriptors and LDS bases built from them need no per-lane handling
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rb = wave & 3, grp = wave >> 2;  // 32-row block and key half of this wave
  const int64_t rs = (int64_t)H * D;
  const int64_t base = ((int64_t)b * T * H + h) * D;  // this (stream, head)'s queries and output
  const int64_t kv_base = ((int64_t)b * kv_rows * H + h) * D;
  const bf16* qb = q + base;
  const bf16* kb = k + kv_base;
  const bf16* vb = v + kv_base;

  // The halves split the keys (the frame's, or a cache's) at 32-key units: half 0 takes the first u0 = ceil(U / 2)
  // of the U units, half 1 the rest.  Every wave runs u0 pipeline steps (one per unit; the
  // work-group barriers keep the halves together), in iters full iterations of two units and,
  // for odd u0, a last single step.  Units past the end of a wave's keys (half 1's last when U
  // is odd, the one after each half's last) are masked to -inf, so they add nothing.
  const int units = (Tk + kUnit - 1) / kUnit;
  const int u0 = (units + 1) >> 1;
  const int steps = u0, iters = steps >> 1;
  const int key0 = grp ? u0 * kUnit : 0;  // first key of this wave's half
  const int key_end = grp ? Tk : min(Tk, u0 * kUnit);

  if (D < DP) {  // padded V^T rows stay zero for the whole kernel
    for (int i = tid; i < VA_BYTES / 16; i += kThreads) {
      reinterpret_cast<uint4*>(vs0)[i] = make_uint4(0, 0, 0, 0);
      reinterpret_cast<uint4*>(vs1)[i] = make_uint4(0, 0, 0, 0);
    }
    __syncthreads();
  }

  // Staging: the four waves of a key half stage its keys (wave sw of the four: 256 threads).
  const int st_t = tid & (kHalfThreads - 1), sw = rb;
  // K half-tile u (keys key0 + 32 u ..): KS direct-to-LDS loads; load i brings rows RPI i ..
  // RPI i + RPI - 1, lane l the granule l % CPR of row RPI i + l / CPR, i.e. feature chunk
  // (l % CPR) ^ (row % CPR).  The lane offset repeats every NKV loads.
  constexpr int RB = S::RB, RPI = S::RPI, NKV = S::NKV, CPR = S::CPR;
  int k_vo[NKV];
#pragma unroll
  for (int q = 0; q < NKV; ++q) {
    const int row = RPI * q + lane / CPR;
    k_vo[q] = (int)((lane / CPR) * rs * 2) + 16 * ((lane % CPR) ^ (row % CPR));
  }
  auto dma_k = [&](__amdgpu_buffer_rsrc_t r, unsigned char* dst, int i) ARL2_INLINE {
    dma16(r, dst + i * 1024, k_vo[i % NKV], (int)(RPI * i * rs * 2));
  };
  // K fragment of k-step st (row lane % 32, feature chunk 2 st + lane / 32) within this key
  // half's part of a ring slot.
  int k_fo[KS];
#pragma unroll
  for (int st = 0; st < KS; ++st) {
    const int row = lane & 31;
    k_fo[st] = grp * KH_BYTES + row * RB + 16 * ((2 * st + (lane >> 5)) ^ (row % CPR));
  }
  // V: blocks of 4 keys (4 va .. 4 va + 3) x 8 features (8 vbb ..) through registers, with the
  // 16 lanes of a quarter-wave on the 16 key blocks of one feature block, transposed (and
  // converted to fp16) on the way into LDS so that the stores of a quarter-wave fill one V^T
  // row.  Every thread issues the same number of loads (a thread without a block of its own
  // reloads block 0).
  int v_off[VPT];  // byte offset of the block's first key row (key kk adds kk rows)
  int v_dst[VPT];  // V^T element offset of the block's first row and key slot
  bool v_mine[VPT];
#pragma unroll
  for (int r = 0; r < VPT; ++r) {
    const int blk = st_t + kHalfThreads * r;
    v_mine[r] = blk < VBLK;
    const int bb = v_mine[r] ? blk : 0;
    const int va = bb & 15, vbb = bb >> 4;
    v_off[r] = (int)((4 * va * rs + 8 * vbb) * 2);
    // keys of block va sit at slot {0, 2, 1, 3}[va % 4] of their 16-key group (the P^T order)
    const int v_slot = ((va & 1) << 1) | ((va >> 1) & 1);
    v_dst[r] = (8 * vbb) * VLD + 16 * (va >> 2) + 4 * v_slot;
  }
  uint4 vreg[VPT][4];
  auto load_v = [&](int tile) ARL2_INLINE {
    const __amdgpu_buffer_rsrc_t r = rows_rsrc(vb, Tk, rs, D, key0 + kKV * tile);
#pragma unroll
    for (int rr = 0; rr < VPT; ++rr)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) vreg[rr][kk] = buf_load16(r, v_off[rr], (int)(kk * rs * 2));
  };
  // store_v_part: block rr, word pairs i in [i0, i1) (rows 2 i, 2 i + 1 of the block's V^T
  // rows); load_v_part: block rr, keys kk in [k0, k1).
  auto store_v_part = [&](auto buf_c, int rr, int i0, int i1) ARL2_INLINE {
    if (v_mine[rr]) {
      f16* vrow = reinterpret_cast<f16*>(varr(buf_c) + grp * VT_BYTES) + v_dst[rr];
      const unsigned w[4][4] = {{vreg[rr][0].x, vreg[rr][0].y, vreg[rr][0].z, vreg[rr][0].w},
                                {vreg[rr][1].x, vreg[rr][1].y, vreg[rr][1].z, vreg[rr][1].w},
                                {vreg[rr][2].x, vreg[rr][2].y, vreg[rr][2].z, vreg[rr][2].w},
                                {vreg[rr][3].x, vreg[rr][3].y, vreg[rr][3].z, vreg[rr][3].w}};
      // word i of key kk holds features 2i (low half) and 2i + 1 (high half) as bf16; a bf16 is
      // the upper half of the fp32 with the same value
      auto feat = [&](int kk, int i, int odd) ARL2_INLINE {
        return __uint_as_float(odd ? (w[kk][i] & 0xFFFF0000u) : (w[kk][i] << 16));
      };
#pragma unroll
      for (int i = i0; i < i1; ++i)
#pragma unroll
        for (int odd = 0; odd < 2; ++odd) {
          const f16x2 k01 = __builtin_convertvector((f32x2{feat(0, i, odd), feat(1, i, odd)}), f16x2);
          const f16x2 k23 = __builtin_convertvector((f32x2{feat(2, i, odd), feat(3, i, odd)}), f16x2);
          *reinterpret_cast<uint2*>(vrow + (2 * i + odd) * VLD) =
              make_uint2(__builtin_bit_cast(unsigned, k01), __builtin_bit_cast(unsigned, k23));
        }
    }
  };
  auto load_v_part = [&](__amdgpu_buffer_rsrc_t r, int rr, int k0, int k1) ARL2_INLINE {
#pragma unroll
    for (int kk = k0; kk < k1; ++kk) vreg[rr][kk] = buf_load16(r, v_off[rr], (int)(kk * rs * 2));
  };
  auto store_v = [&](auto buf_c) ARL2_INLINE {
#pragma unroll
    for (int rr = 0; rr < VPT; ++rr) store_v_part(buf_c, rr, 0, 4);
  };
  // W^T = (phi_q S)^T, hi then lo, into the K arrays after the loop, as planes of DP rows x 32
  // bytes: plane (hl, st) holds features 16 st .. 16 st + 15 of every output feature.  Its
  // kilobyte c sits in K array c / KA_KB at kilobyte c % KA_KB.
  constexpr int W_INSTR = 2 * KS * DP / 32, KA_KB = KA_BYTES / 1024;
  auto w_kb = [&](int c) ARL2_INLINE -> unsigned char* {
    const int a = c / KA_KB;
    return (a == 0 ? ks0 : a == 1 ? ks1 : a == 2 ? ks2 : ks3) + (c % KA_KB) * 1024;
  };
  const int64_t wbase = ((int64_t)b * H + h) * DP * D;
  auto load_w = [&]() ARL2_INLINE {
    const __amdgpu_buffer_rsrc_t rh = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16*>(wt_hi + wbase), (short)0,
                                                                        DP * D * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t rl = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16*>(wt_lo + wbase), (short)0,
                                                                        DP * D * 2, 0x00020000);
#pragma unroll
    for (int c = 0; c < (W_INSTR + kWaves - 1) / kWaves; ++c) {
      const int i = wave + kWaves * c;  // kilobyte i: plane i / (DP / 32), 32-row block i % (DP / 32)
      if (i < W_INSTR) {
        const int hl = i / (W_INSTR / 2), kb_in = i % (W_INSTR / 2);
        dma16(hl ? rl : rh, w_kb(i), 16 * lane, kb_in * 1024);
      }
    }
  };

  // This lane's query row as B fragments of Q^T (k-step st = features 16 st .. 16 st + 15),
  // read from LDS in the prologue.
  bf16x8 qf[KS];

  f32x16 acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = zero16();
  float m_run = -INFINITY;  // running max (raw score units), equal in lanes l and l ^ 32
  float mc = 0.f;           // m_run * scale_log2 (0 while m_run = -inf: a half without keys gets P = 0, not NaN)
  float thr = -INFINITY;    // raw score above which the running max is raised
  float l_run = 0.f;        // this lane's share of the running sum
  const float slack_raw = kRescaleSlack / scale_log2;

  // Fragment offsets of this lane inside a W^T plane (32-byte rows) and, in bytes, inside this
  // key half's part of a V^T buffer.
  const int k_frag = (lane & 31) * 32 + (lane >> 5) * 16;
  const int v_frag = grp * VT_BYTES + 2 * ((lane & 31) * VLD + 8 * (lane >> 5));

  // Fragments in flight.  K fragment st of a unit = k-step st; V^T fragment f of a unit =
  // k-step f / MB of the unit (16 keys), feature block f % MB.
  bf16x8 kfr[KS];
  f16x8 vfr[2 * MB];

  // Softmax of score registers [v0, v1) of a unit (v1 - v0 a multiple of 4) into fp16 pairs:
  // registers i, i + 1 of the score block become word (i / 2) % 4 of pw[i / 8], the P^T
  // fragment of k-step i / 8; and adds the rounded P that enters the MFMA to the running row sum
  // (fp32).  A fragment is pinned once complete.
  const f16x2 ones = {(f16)1.f, (f16)1.f};
  auto softmax_part = [&](const f32x16& sa, u32x4 (&pw)[2], int v0, int v1, float mc) ARL2_INLINE {
#pragma unroll
    for (int jj = v0; jj < v1; jj += 4) {
      f16x2 p[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int i = jj + 2 * e;
        const f32x2 x = {__builtin_amdgcn_exp2f(fmaf(sa[i], scale_log2, -mc)),
                         __builtin_amdgcn_exp2f(fmaf(sa[i + 1], scale_log2, -mc))};
        p[e] = __builtin_convertvector(x, f16x2);
        pw[i >> 3][(i >> 1) & 3] = __builtin_bit_cast(unsigned, p[e]);
      }
      l_run = __builtin_amdgcn_fdot2(p[0], ones, l_run, false);
      l_run = __builtin_amdgcn_fdot2(p[1], ones, l_run, false);
    }
    if (v1 % 8 == 0) pin(pw[(v1 - 1) >> 3]);
    pin(l_run);
  };
  // Keys of unit u past the end of this wave's keys do not take part.
  auto mask_unit = [&](int u, f32x16& sc) ARL2_INLINE {
    const int k0 = key0 + kUnit * u;
    if (k0 + kUnit > key_end) {
      const int lid = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (k0 + c_row(i, lid) >= key_end) sc[i] = -INFINITY;
    }
  };
  // Raise the running max to a unit's max when it exceeds it by more than the slack in some
  // lane of the wave (the accumulator and sum are rescaled); otherwise keep it, so P <= 2^8.
  // mp is this lane's max over its 16 keys of the unit; the row max (lanes l and l ^ 32) is
  // only needed when raising.
  auto rescale_to = [&](float mp) ARL2_INLINE {
    if (__builtin_amdgcn_ballot_w64(mp > thr) != 0) {
      const float mx = fmaxf(mp, other_half(mp, lane));
      const float m_new = fmaxf(m_run, mx);
      const float corr = __builtin_amdgcn_exp2f((m_run - m_new) * scale_log2);
      m_run = m_new;
      mc = m_new * scale_log2;
      thr = m_new + slack_raw;
      l_run *= corr;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[mb][i] *= corr;
    }
  };

  // Step u: phase A = scores of unit u + 1 (into sb) with the softmax of unit u (from sa);
  // phase B = O^T += V^T P^T for unit u with the row max of unit u + 1.  next_sw / cur_sw
  // switch the work on unit u + 1 / unit u on or off at compile time (On / Off), so that every
  // variant is branch-free.  Stage s of the step (A stages, then B stages) reads the fragments
  // of stage s + 2.
  // kslot_c / vbuf_c: compile-time ring slot of unit u + 1 and V^T buffer of unit u.
  // hook(s) issues the staging work of stage s (A stages 0 .. NA - 1, then B stages) first.
  auto step = [&](int u, const f32x16& sa, f32x16& sb, auto next_sw, auto cur_sw, auto kslot_c, auto vbuf_c,
                  auto&& hook) ARL2_INLINE {
    constexpr bool nx = decltype(next_sw)::value, cu = decltype(cur_sw)::value;
    const unsigned char* kt = karr(kslot_c);
    const unsigned char* vt = varr(vbuf_c) + v_frag + 64 * (u & 1);
    auto read_stage = [&](int s) ARL2_INLINE {
      if (s < NA) {
        if (nx)
#pragma unroll
          for (int f = s * FA; f < (s + 1) * FA; ++f) kfr[f] = *reinterpret_cast<const bf16x8*>(kt + k_fo[f]);
      } else if (s < NA + NB) {
        if (cu)
#pragma unroll
          for (int f = (s - NA) * FB; f < (s - NA + 1) * FB; ++f)
            vfr[f] = *reinterpret_cast<const f16x8*>(vt + 64 * (f % MB) * VLD + 32 * (f / MB));
      }
    };
    u32x4 pw[2];
    read_stage(0);
    read_stage(1);
#pragma unroll
    for (int t = 0; t < NA; ++t) {
      hook(t);
      read_stage(t + 2);
      if (cu) softmax_part(sa, pw, t * 16 / NA, (t + 1) * 16 / NA, mc);
      if (nx)
#pragma unroll
        for (int f = t * FA; f < (t + 1) * FA; ++f) sb = mfma32(kfr[f], qf[f], f ? sb : zero16());
      __builtin_amdgcn_sched_barrier(0);
    }
    float mp = -INFINITY;
    if (nx) {
      mask_unit(u + 1, sb);
      to_vgpr(sb);
    }
#pragma unroll
    for (int t = 0; t < NB; ++t) {
      hook(NA + t);
      read_stage(NA + t + 2);
      if (nx) {
#pragma unroll
        for (int i = t * 16 / NB; i < (t + 1) * 16 / NB; ++i) mp = fmaxf(mp, sb[i]);
        pin(mp);
      }
      if (cu)
#pragma unroll
        for (int f = t * FB; f < (t + 1) * FB; ++f)
          acc[f % MB] = mfma32(vfr[f], __builtin_bit_cast(f16x8, pw[f / MB]), acc[f % MB]);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (nx) rescale_to(mp);
  };

  // Prologue.  The work-group's query tile comes into V^T buffer 1 (unused until the first
  // iteration stores into it) with the swizzled row-major loads of K, and each key half's K
  // half-tiles 0-2 into its ring slots 0-2; V tile 0 comes into registers.  The first barrier
  // waits for the loads into LDS only; each wave then takes its Q fragments from LDS and
  // computes the scores and max of unit 0, while V tile 0 arrives, goes to V^T buffer 0, and
  // tile 1 comes into registers.  The second barrier publishes V tile 0 and keeps the first
  // iteration's loads into slot 0 (and stores into buffer 1) behind every wave's reads.
  // Only the query tile and K half-tile 0 are waited for before unit 0's scores; half-tiles
  // 1-2 and V tile 0 are issued after the first barrier, so that the vector-memory path
  // drains them while those MFMAs run.
  {
    const __amdgpu_buffer_rsrc_t qr = rows_rsrc(qb, T, rs, D, qt * kQTile);
    constexpr int QI = kQTile / RPI;  // 1-KB loads of the query tile
#pragma unroll
    for (int c = 0; c < (QI + kWaves - 1) / kWaves; ++c)
      if (wave + kWaves * c < QI) dma_k(qr, vs1, wave + kWaves * c);
    const __amdgpu_buffer_rsrc_t r0 = rows_rsrc(kb, Tk, rs, D, key0);
#pragma unroll
    for (int m = 0; m < (KS + 3) / 4; ++m)
      if (sw + 4 * m < KS) dma_k(r0, ks0 + grp * KH_BYTES, sw + 4 * m);
  }
  wait_vmem();
  __syncthreads();
#pragma unroll
  for (int st = 0; st < KS; ++st)
    qf[st] = *reinterpret_cast<const bf16x8*>(vs1 + rb * 32 * RB + k_fo[st] - grp * KH_BYTES);
  {
    constexpr int NKI = 2 * KS;  // loads of this key half's K half-tiles 1-2
#pragma unroll
    for (int m = 0; m < (NKI + 3) / 4; ++m) {
      const int i = sw + 4 * m;
      if (i < NKI) {
        const int hh = 1 + i / KS;
        const __amdgpu_buffer_rsrc_t r = rows_rsrc(kb, Tk, rs, D, key0 + kUnit * hh);
        dma_k(r, (hh == 1 ? ks1 : ks2) + grp * KH_BYTES, i % KS);
      }
    }
  }
  asm volatile("" ::: "memory");  // the V loads stay behind the loads into LDS
  __builtin_amdgcn_sched_barrier(0);
  load_v(0);
  f32x16 s0, s1 = zero16();  // (s1 is not read by the first step)
  auto no_staging = [](int) ARL2_INLINE {};
  step(-1, s1, s0, On(), Off(), Ic<0>(), Ic<1>(), no_staging);
  store_v(Ic<0>());
  if (steps > 2) load_v(1);
  wait_vmem_but<4 * VPT>();  // half-tiles 1-2 have landed (V tile 1 may still be in flight)
  if (D < DP) {  // the query tile overlapped padded V^T rows of buffer 1, which stay zero
    __syncthreads();
    for (int i = tid; i < VA_BYTES / 16; i += kThreads) reinterpret_cast<uint4*>(vs1)[i] = make_uint4(0, 0, 0, 0);
  }
  __syncthreads();

  // Iteration j (parity P = j % 2, a compile-time constant): units 2j and 2j + 1 (tile j of
  // this key half).  Staging, spread over the stages so that the vector-memory path drains
  // while the MFMAs run: K half-tiles 2j + 3 and 2j + 4 into the ring slots that held 2j - 1
  // and 2j (the 2 KS loads dealt over the four waves of the half, in the A stages of step
  // 2j); V tile j + 1 from registers into the buffer that held tile j - 1 (B stages of step
  // 2j), then the registers reloaded with tile j + 2 (B stages of step 2j + 1).  All K loads
  // precede the V loads, so waiting for all but the V loads before the barrier leaves the K
  // loads complete and the V loads in flight until their use.  Staging past the last tile
  // reads zeros (outside the buffer descriptors) into slots and buffers that nothing reads
  // again.
  auto iteration = [&](int j, auto par_c) ARL2_INLINE {
    constexpr int P = decltype(par_c)::value;
    unsigned char* kd0 = karr(Ic<2 * P + 3>()) + grp * KH_BYTES;
    unsigned char* kd1 = karr(Ic<2 * P + 4>()) + grp * KH_BYTES;
    const __amdgpu_buffer_rsrc_t kr0 = rows_rsrc(kb, Tk, rs, D, key0 + kUnit * (2 * j + 3));
    const __amdgpu_buffer_rsrc_t kr1 = rows_rsrc(kb, Tk, rs, D, key0 + kUnit * (2 * j + 4));
    const __amdgpu_buffer_rsrc_t vr = rows_rsrc(vb, Tk, rs, D, key0 + kKV * (j + 2));
    // The K loads are dealt over both phases of step 2j (half each, on every other stage) and the
    // V loads over both phases of step 2j + 1, so that the vector-memory path has work in every
    // phase instead of bursts in two.
    auto k_loads = [&](int m0, int m1) ARL2_INLINE {
#pragma unroll
      for (int m = m0; m < m1; ++m) {
        const int i = sw + 4 * m;
        if (i < KS) dma_k(kr0, kd0, i);
        else if (i < 2 * KS) dma_k(kr1, kd1, i - KS);
      }
    };
    // share [s * n / (2 ns), (s + 1) * n / (2 ns)) of n items for stage s of ns in half h of the step
    auto share = [](int h, int s, int ns, int n, int& i0, int& i1) ARL2_INLINE {
      i0 = (h * ns + s) * n / (2 * ns);
      i1 = (h * ns + s + 1) * n / (2 * ns);
    };
    auto hook0 = [&](int st) ARL2_INLINE {
      const bool pa = st < NA;
      const int s = pa ? st : st - NA, ns = pa ? NA : NB;
      int m0, m1;
      share(pa ? 0 : 1, s, ns, KPW, m0, m1);
      k_loads(m0, m1);
      if (!pa)
#pragma unroll
        for (int rr = 0; rr < VPT; ++rr) store_v_part(Ic<P + 1>(), rr, 4 * s / NB, 4 * (s + 1) / NB);
    };
    auto hook1 = [&](int st) ARL2_INLINE {
      const bool pa = st < NA;
      const int s = pa ? st : st - NA, ns = pa ? NA : NB;
      if (st == 0) asm volatile("" ::: "memory");  // the V loads stay behind the K loads
      int k0, k1;
      share(pa ? 0 : 1, s, ns, 4, k0, k1);
#pragma unroll
      for (int rr = 0; rr < VPT; ++rr) load_v_part(vr, rr, k0, k1);
    };
    step(2 * j, s0, s1, On(), On(), Ic<2 * P + 1>(), Ic<P>(), hook0);
    step(2 * j + 1, s1, s0, On(), On(), Ic<2 * P + 2>(), Ic<P>(), hook1);
    wait_vmem_but<4 * VPT>();
    __syncthreads();
  };
  int j = 0;
  for (; j + 1 < iters; j += 2) {
    iteration(j, Ic<0>());
    iteration(j + 1, Ic<1>());
  }
  if (j < iters) {
    iteration(j, Ic<0>());
    ++j;
  }
  // W^T (for the epilogue) comes into the K arrays, which the last single step does not read.
  if constexpr (INTER) load_w();
  if (steps & 1) {  // the last unit, 2j: its scores are in s0 and its V^T tile j in buffer j % 2
    if (j & 1) step(2 * j, s0, s1, Off(), On(), Ic<0>(), Ic<1>(), no_staging);
    else step(2 * j, s0, s1, Off(), On(), Ic<0>(), Ic<0>(), no_staging);
    __syncthreads();  // every wave is done with the V arrays before the exchange writes them
  }

  // Epilogue.  W^T comes into the K arrays while the two waves of a row block exchange,
  // through the V arrays, the halves of the accumulator that the other one finalises (with
  // their running max and sum): the wave of key half g finalises output feature blocks
  // [g * MBH, (g + 1) * MBH) (for d < 64 key half 0 finalises the single block).
  static_assert(W_INSTR <= 4 * KA_KB, "W must fit in the K arrays");
  const int partner = wave ^ 4;
  const bool owner = MB >= 2 || grp == 0;
  const bool partner_owns = MB >= 2 || grp == 1;
  auto xslot = [&](int w) ARL2_INLINE {  // [NXV][64] f32x4 of exporter w
    const int xs = MB >= 2 ? w : (w & 3);
    if constexpr (XFIT) return reinterpret_cast<f32x4*>((xs / XS_PER ? vs1 : vs0) + (xs % XS_PER) * XS_BYTES);
    else return reinterpret_cast<f32x4*>(xs_own + xs * XS_BYTES);
  };
  if (partner_owns) {
    f32x4* xo = xslot(wave);
    const int p0 = MB >= 2 ? (1 - grp) * MBH : 0;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
      if (mb >= p0 && mb < p0 + MBH)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          xo[((mb - p0) * 4 + g) * 64 + lane] =
              f32x4{acc[mb][4 * g], acc[mb][4 * g + 1], acc[mb][4 * g + 2], acc[mb][4 * g + 3]};
    xo[(NXV - 1) * 64 + lane] = f32x4{m_run, l_run, 0.f, 0.f};
  }
  __syncthreads();

  const f32x4* xi = xslot(partner);
  const int o0 = MB >= 2 ? grp * MBH : 0;
  if (owner) {
    const f32x4 ml = xi[(NXV - 1) * 64 + lane];
    const float m1 = ml[0], l1 = ml[1];
    const float m = fmaxf(m_run, m1);
    const float e0 = __builtin_amdgcn_exp2f((m_run - m) * scale_log2);
    const float e1 = __builtin_amdgcn_exp2f((m1 - m) * scale_log2);
    const float lsum = l_run * e0 + l1 * e1;
    const float ltot = lsum + other_half(lsum, lane);
    const float inv = 1.f / ltot;
    // plain attention: the row's log-sum-exp of the scaled scores in log2 units, for a backward
    if (!INTER && lse && grp == 0 && lane < 32 && qt * kQTile + rb * 32 + lane < T)
      lse[(int64_t)bh * T + qt * kQTile + rb * 32 + lane] = m * scale_log2 + log2f(ltot);
    const float a0 = e0 * inv, a1 = e1 * inv;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      if (mb < o0 || mb >= o0 + MBH) continue;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 x = xi[((mb - o0) * 4 + g) * 64 + lane];
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[mb][4 * g + e] = acc[mb][4 * g + e] * a0 + x[e] * a1;
      }
    }
  }
  wait_vmem();  // W^T has landed (every wave waits for its own loads, then the barrier)
  __syncthreads();
  if (!owner) return;

  // Add Q W = Q (phi_q S) with W^T split in two bf16 terms (A fragments from LDS).
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    if (!INTER || mb < o0 || mb >= o0 + MBH) continue;
#pragma unroll
    for (int st = 0; st < KS; ++st)
#pragma unroll
      for (int hl = 0; hl < 2; ++hl) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(w_kb((hl * KS + st) * (DP / 32) + mb) + k_frag);
        acc[mb] = mfma32(a, qf[st], acc[mb]);
      }
  }

  // Output.  The wave's 32 rows x OWN_D finished features go through LDS (the V arrays, free
  // since the barrier) into row-major order, 16-byte chunks of row r at granule
  // chunk ^ (r % OC), so that each store instruction writes whole row segments.
  constexpr int OWN_D = D < 32 * MBH ? D : 32 * MBH;  // features this wave finalises
  constexpr int OC = OWN_D / 4, ORB = 16 * OC, RPS = 64 / OC;  // chunks per row, row bytes, rows per store
  static_assert(4 * 32 * ORB <= VA_BYTES, "output staging must fit in the V arrays");
  unsigned char* ost = (wave >> 2 ? vs1 : vs0) + (wave & 3) * 32 * ORB;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    if (mb < o0 || mb >= o0 + MBH) continue;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int ld = 32 * (mb - o0) + 8 * g + 4 * (lane >> 5);
      if (ld < OWN_D) {
        const int r = lane & 31, c = ld >> 2;
        *reinterpret_cast<f32x4*>(ost + r * ORB + 16 * (c ^ (r % OC))) =
            f32x4{acc[mb][4 * g], acc[mb][4 * g + 1], acc[mb][4 * g + 2], acc[mb][4 * g + 3]};
      }
    }
  }
  const int row0 = qt * kQTile + rb * 32;
#pragma unroll
  for (int i = 0; i < 32 / RPS; ++i) {
    const int r = RPS * i + lane / OC, c = lane % OC;
    f32x4 x = *reinterpret_cast<const f32x4*>(ost + r * ORB + 16 * (c ^ (r % OC)));
    if (row0 + r < T) {
      const int64_t o = base + (int64_t)(row0 + r) * rs + 32 * o0 + 4 * c;
      if (!INTER && add) x += *reinterpret_cast<const f32x4*>(add + o);
      // The ARL2 pass stores with streaming (non-temporal) stores: its output is written once and
      // read only by later kernels, so it need not hold L2 lines that the other work-groups' K and
      // V tiles use.  The plain-attention instance keeps ordinary stores: a backward's recompute
      // is read by the very next kernel.  (The choice is made at compile time: with a run-time
      // branch the compiler merges the two stores into an ordinary one.)
      if (OUT_BF16) {
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (bf16)x[e];
        bf16x4* dst = reinterpret_cast<bf16x4*>(reinterpret_cast<bf16*>(out) + o);
        if constexpr (INTER) __builtin_nontemporal_store(w, dst);
        else *dst = w;
      } else {
        f32x4* dst = reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + o);
        if constexpr (INTER) __builtin_nontemporal_store(x, dst);
        else *dst = x;
      }
    }
  }
}

template <int D>
hipError_t launch_fwd_d(const FwdArgs& a, const WritePartialArgs* w, hipStream_t stream) {
  const int nq = (a.T + kQTile - 1) / kQTile;
  const int n_bh = a.H * a.B;
  const bool inter = a.Tk < 0;  // the ARL2 pass: keys are the frame's own
  const int Tk = inter ? a.T : a.Tk, kv_rows = inter ? a.T : a.kv_rows;
  const int n_pass_blocks = a.out ? 8 * ((nq * n_bh + 7) / 8) : 0;
  const int n_write = inter && w ? commit_chunks(a.T) * n_bh : 0;
  if (n_pass_blocks + n_write == 0) return hipSuccess;
  const WritePartialArgs wa = w ? *w : WritePartialArgs{};
  dim3 grid(n_pass_blocks + 8 * ((n_write + 7) / 8));
  const bf16* q = static_cast<const bf16*>(a.q);
  const bf16* k = static_cast<const bf16*>(a.k);
  const bf16* v = static_cast<const bf16*>(a.v);
  const bf16* wh = static_cast<const bf16*>(a.wt_hi);
  const bf16* wl = static_cast<const bf16*>(a.wt_lo);
#define ARL2_LAUNCH_FWD(OB, IN)                                                                              \
  hipLaunchKernelGGL((arl2_fwd_kernel<D, OB, IN>), grid, dim3(kThreads), 0, stream, q, k, v, wh, wl, a.out, a.T, Tk, \
                     kv_rows, a.H, nq, n_bh, a.scale_log2, n_pass_blocks, wa, n_write, a.add, a.lse)
  if (inter) {
    if (a.out_bf16) ARL2_LAUNCH_FWD(true, true);
    else ARL2_LAUNCH_FWD(false, true);
  } else {
    if (a.out_bf16) ARL2_LAUNCH_FWD(true, false);
    else ARL2_LAUNCH_FWD(false, false);
  }
#undef ARL2_LAUNCH_FWD
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd(int d, const FwdArgs& a, const WritePartialArgs* w, hipStream_t stream) {
  switch (d) {
    case 16: return launch_fwd_d<16>(a, w, stream);
    case 64: return launch_fwd_d<64>(a, w, stream);
    case 128: return launch_fwd_d<128>(a, w, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace arl2
