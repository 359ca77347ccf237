// Fused per-pass kernel of the ARL2 layer:
//   out = softmax(Q K^T * scale) V + Q W,   W = phi_q S_{N-1}
// ("Attend Locally, Remember Linearly", gist.science technical summary, section 2.1:
// intra-frame softmax branch and inter-frame output Q' S_{N-1} with Q' = Q phi_q; section
// 2.2: every token of the frame reads the same pre-update state).  Q' S = Q (phi_q S) by
// associativity; W is formed once per frame by the state-write kernels, so a pass only
// adds a Q x W product to the attention accumulator.
//
// Work decomposition.  One work-group of 8 waves per (stream, head, 128-query tile), two
// waves per SIMD.  Waves 0-3 and 4-7 form two groups that own the same 128 query rows (32
// per wave) but opposite halves of the frame's keys; the halves are merged through LDS at
// the end (max / sum rescaling), so no partial result leaves the chip.  Each group streams
// its half in 64-key tiles, double-buffered in LDS and staged by all 512 threads.
//
// Scores are computed transposed, S^T = K Q^T, so that every lane holds one query row and
// 32 of the tile's keys: the row max needs one cross-lane exchange (l, l ^ 32), the row sum
// none until the end.  The output is accumulated transposed too, O^T += V^T P^T, one query
// row per lane, so rescaling is a per-lane multiply.  V^T is written to LDS while staging:
// each thread transposes a 4-key x 8-feature block in registers (v_perm) and stores it in
// the key order of the P^T fragments; rows are padded by 16 bytes so that fragment reads
// (32 consecutive rows) are conflict-free 16-byte loads.  K and V come in through buffer
// loads: rows past the end of the frame lie outside the buffer and read as zeros.
//
// Softmax: exp2 with the scale folded in; the running max is only raised when a tile's max
// exceeds it by more than 8 (in log2 units) in some lane of the wave, so P stays below 2^8
// and the rescale of the accumulator is skipped on almost every tile.  Row sums use dot2 on
// the bf16 P that enters the MFMA.
#include <type_traits>

#include "arl2_device.h"
#include "arl2_kernels.h"

namespace arl2 {
namespace {

constexpr int kQTile = 128;  // query rows per work-group
constexpr int kKV = 64;      // keys per LDS tile
constexpr int kThreads = 512;
constexpr float kRescaleSlack = 8.f;  // log2 headroom before the running max is raised

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

template <int D>
struct FwdShape {
  static constexpr int DP = D < 32 ? 32 : D;  // padded feature rows of the O^T / V^T blocks
  static constexpr int KS = D / 16;          // 16-wide k-steps over features
  static constexpr int MB = DP / 32;         // 32-row blocks over output features
  static constexpr int CPR = D / 8;          // 16-byte chunks per token row
  static constexpr int VBLK = 16 * CPR;      // 4-key x 8-feature blocks per V tile
  static constexpr int VLD = kKV + 8;        // V^T row stride in bf16 (64 keys + 16 bytes of padding)
  // K tile: one plane of 64 rows x 32 bytes per k-step (features 16 st .. 16 st + 15), so that
  // every MFMA fragment is one contiguous kilobyte.
  static constexpr int K_BYTES = KS * kKV * 32;
  static constexpr int VT_BYTES = DP * VLD * 2;
  static constexpr int K_INSTR = 2 * KS;     // 1-KB direct-to-LDS loads per K tile
};

// Buffer resource over rows [tile * 64, T) of one (stream, head) slice of a [B][T][H][d]
// tensor: anything past the frame lies outside num_records, and loads there return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const bf16* base, int T, int64_t rs, int d, int tile) {
  const int64_t start = (int64_t)tile * kKV * rs;
  const int64_t left = (int64_t)(T - 1) * rs + d - start;
  const bool any = left > 0;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16*>(any ? base + start : base), (short)0,
                                           any ? (int)(left * 2) : 0, 0x00020000);
}

__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, int off) {
  const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(x.x, x.y, x.z, x.w);
}

// 16 bytes per lane from the buffer straight into LDS at lds + 16 * lane (lds wave-uniform).
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, void* lds, int off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, off, 0, 0, 0);
}

// Wait until all of this wave's vector memory operations (including loads into LDS) are done.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

template <int D, bool OUT_BF16>
__global__ __launch_bounds__(kThreads) void arl2_fwd_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ wt_hi, const bf16* __restrict__ wt_lo, void* __restrict__ out,
    int T, int H, int nq, int n_items, int per_xcd, float scale_log2) {
  using S = FwdShape<D>;
  constexpr int DP = S::DP, KS = S::KS, MB = S::MB, VLD = S::VLD, CPR = S::CPR, VBLK = S::VBLK,
                K_BYTES = S::K_BYTES, VT_BYTES = S::VT_BYTES, K_INSTR = S::K_INSTR;

  // LDS: K tiles [group][buffer] then V^T tiles [group][buffer].  After the loop the K part
  // holds W^T (hi, lo) and the V part the exchange between the two groups.
  __shared__ __attribute__((aligned(16))) unsigned char smem[4 * K_BYTES + 4 * VT_BYTES];
  unsigned char* const kreg_lds = smem;
  unsigned char* const vreg_lds = smem + 4 * K_BYTES;
  auto ktile = [&](int g, int buf) { return kreg_lds + (2 * g + buf) * K_BYTES; };
  auto vtile = [&](int g, int buf) { return reinterpret_cast<bf16*>(vreg_lds + (2 * g + buf) * VT_BYTES); };

  // XCD-aware order: work-groups are dealt to the 8 XCDs round-robin, so consecutive items
  // (the query tiles of one head) are given to work-groups on the same XCD and share its L2.
  const int item = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (item >= n_items) return;
  const int qt = item % nq, bh = item / nq;
  const int h = bh % H, b = bh / H;

  // wave-uniform indices are made explicitly uniform (scalar registers), so that buffer
  // descriptors and LDS bases built from them need no per-lane handling
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2, wq = wave & 3;
  const int64_t rs = (int64_t)H * D;
  const int64_t base = ((int64_t)b * T * H + h) * D;
  const bf16* qb = q + base;
  const bf16* kb = k + base;
  const bf16* vb = v + base;

  const int ntiles = (T + kKV - 1) / kKV;
  const int nt0 = (ntiles + 1) >> 1;  // group 0: tiles [0, nt0); group 1: [nt0, ntiles)
  const int my_first = grp ? nt0 : 0, my_count = grp ? ntiles - nt0 : nt0;
  const int iters = nt0;

  if (D < DP) {  // padded V^T rows stay zero for the whole kernel
    for (int i = tid; i < 4 * VT_BYTES / 16; i += kThreads)
      reinterpret_cast<uint4*>(vreg_lds)[i] = make_uint4(0, 0, 0, 0);
    __syncthreads();
  }

  // Staging roles: waves 0-3 stage group 0's tiles, waves 4-7 group 1's.
  const int sg = wave >> 2, st_t = tid & 255, sw = wave & 3;
  const int sg_first = sg ? nt0 : 0;
  // K: direct-to-LDS loads; instruction i (st = i / 2, 32-row block i % 2) puts rows
  // 32 (i % 2) + lane / 2, features 16 st + 8 (lane % 2) .. + 7 at 16 lane.
  const int k_lane_off = (int)(((lane >> 1) * rs + 8 * (lane & 1)) * 2);
  auto load_k = [&](int tile, int buf) {
    const __amdgpu_buffer_rsrc_t r = tile_rsrc(kb, T, rs, D, sg_first + tile);
    unsigned char* dst = ktile(sg, buf);
#pragma unroll
    for (int c = 0; c < (K_INSTR + 3) / 4; ++c) {
      const int i = sw + 4 * c;
      if (i < K_INSTR)
        dma16(r, dst + (i >> 1) * (kKV * 32) + (i & 1) * 1024,
              k_lane_off + (int)((i & 1) * 32 * rs * 2) + (i >> 1) * 32);
    }
  };
  // V: a block of 4 keys (4 va .. 4 va + 3) x 8 features (8 vbb ..) through registers, with the
  // 16 lanes of a quarter-wave on 16 key blocks of one feature block, transposed on the way
  // into LDS so that the stores of a quarter-wave fill one V^T row.
  const int va = st_t & 15, vbb = st_t >> 4;
  const bool v_stager = st_t < VBLK;
  int v_off[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) v_off[kk] = (int)(((4 * va + kk) * rs + 8 * vbb) * 2);
  uint4 vreg[4];
  auto load_v = [&](int tile) {
    const __amdgpu_buffer_rsrc_t r = tile_rsrc(vb, T, rs, D, sg_first + tile);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) vreg[kk] = v_stager ? buf_load16(r, v_off[kk]) : make_uint4(0, 0, 0, 0);
  };
  // keys of block va sit at slot {0, 2, 1, 3}[va % 4] of their 16-key group (the P^T order)
  const int v_slot = ((va & 1) << 1) | ((va >> 1) & 1);
  const int v_col = 16 * (va >> 2) + 4 * v_slot;  // key position within a V^T row
  auto store_v = [&](int buf) {
    if (!v_stager) return;
    bf16* vrow = vtile(sg, buf) + (8 * vbb) * VLD + v_col;
    const unsigned w0[4] = {vreg[0].x, vreg[0].y, vreg[0].z, vreg[0].w};
    const unsigned w1[4] = {vreg[1].x, vreg[1].y, vreg[1].z, vreg[1].w};
    const unsigned w2[4] = {vreg[2].x, vreg[2].y, vreg[2].z, vreg[2].w};
    const unsigned w3[4] = {vreg[3].x, vreg[3].y, vreg[3].z, vreg[3].w};
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int odd = 0; odd < 2; ++odd) {
        const unsigned sel = odd ? 0x07060302u : 0x05040100u;
        const uint2 val = make_uint2(__builtin_amdgcn_perm(w1[i], w0[i], sel), __builtin_amdgcn_perm(w3[i], w2[i], sel));
        *reinterpret_cast<uint2*>(vrow + (2 * i + odd) * VLD) = val;
      }
  };
  // W^T = (phi_q S)^T, hi then lo, into the K part of LDS (free during the last iteration), in
  // the same plane layout: plane (hl, st) holds rows 0 .. DP-1 x 32 bytes.
  constexpr int W_INSTR = 2 * KS * DP / 32;
  const int64_t wbase = ((int64_t)b * H + h) * DP * D;
  const int w_lane_off = (int)(((lane >> 1) * D + 8 * (lane & 1)) * 2);
  auto load_w = [&]() {
    const __amdgpu_buffer_rsrc_t rh = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16*>(wt_hi + wbase), (short)0,
                                                                        DP * D * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t rl = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16*>(wt_lo + wbase), (short)0,
                                                                        DP * D * 2, 0x00020000);
#pragma unroll
    for (int c = 0; c < (W_INSTR + 7) / 8; ++c) {
      const int i = wave + 8 * c;  // 1 KB each: plane i / (DP / 32), 32-row block i % (DP / 32)
      if (i < W_INSTR) {
        const int plane = i / (DP / 32), rb = i % (DP / 32);
        const int hl = plane / KS, st = plane % KS;
        dma16(hl ? rl : rh, kreg_lds + i * 1024, w_lane_off + (32 * rb * D + 16 * st) * 2);
      }
    }
  };

  // This lane's query row as B fragments of Q^T (k-step st = features 16 st .. 16 st + 15).
  const int qrow = qt * kQTile + wq * 32 + (lane & 31);
  bf16x8 qf[KS];
#pragma unroll
  for (int st = 0; st < KS; ++st)
    qf[st] = qrow < T ? ld_bf16x8(qb + qrow * rs + 16 * st + 8 * (lane >> 5)) : zero_bf16x8();

  f32x16 acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = zero16();
  float m_run = -INFINITY;  // running max (raw score units), equal in lanes l and l ^ 32
  float l_run = 0.f;        // this lane's share of the running sum

  // Fragment offsets of this lane inside a K plane and a V^T tile.
  const int k_frag = (lane & 31) * 32 + (lane >> 5) * 16;
  const int v_frag = (lane & 31) * VLD + 8 * (lane >> 5);

  // Scores of one K tile (S^T, two 32-key blocks) and their per-row max, with keys past the
  // frame masked (lanes l and l ^ 32 hold the two halves of a row).
  auto scores = [&](int kbuf, f32x16 (&sc)[2]) {
    const unsigned char* kt = ktile(grp, kbuf) + k_frag;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
      sc[kb2] = zero16();
#pragma unroll
      for (int st = 0; st < KS; ++st)
        sc[kb2] = mfma32(*reinterpret_cast<const bf16x8*>(kt + st * (kKV * 32) + kb2 * 1024), qf[st], sc[kb2]);
    }
  };
  auto tile_max = [&](int tile, f32x16 (&sc)[2]) {
    if ((tile + 1) * kKV > T) {  // ragged last tile: keys beyond the frame do not exist
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (tile * kKV + 32 * kb2 + c_row(i, lane) >= T) sc[kb2][i] = -INFINITY;
    }
    float mx = sc[0][0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sc[0][i]);
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sc[1][i]);
    return fmaxf(mx, other_half(mx, lane));
  };

  // Raise the running max to a tile's max when it exceeds it by more than the slack in some
  // lane of the wave (the accumulator and sum are rescaled); otherwise keep it, so P <= 2^8.
  auto rescale_to = [&](float mx) {
    if (__builtin_amdgcn_ballot_w64((mx - m_run) * scale_log2 > kRescaleSlack) != 0) {
      const float m_new = fmaxf(m_run, mx);
      const float corr = __builtin_amdgcn_exp2f((m_run - m_new) * scale_log2);
      m_run = m_new;
      l_run *= corr;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[mb][i] *= corr;
    }
  };
  const bf16x2 ones = {(bf16)1.f, (bf16)1.f};
  // P = exp2(S scale - m scale) of one tile as bf16 B fragments, the row sums, and O^T += V^T P^T
  // with the tile's V^T from LDS buffer vbuf.
  auto softmax_pv = [&](const f32x16 (&sa)[2], int vbuf) {
    const float mc = m_run * scale_log2;
    const bf16* vt = vtile(grp, vbuf) + v_frag;
#pragma unroll
    for (int ks4 = 0; ks4 < 4; ++ks4) {
      bf16x8 pf;  // k-step ks4 = 16 keys: element jj <-> register 8 (ks4 % 2) + jj of block ks4 / 2
#pragma unroll
      for (int jj = 0; jj < 8; ++jj)
        pf[jj] = (bf16)__builtin_amdgcn_exp2f(fmaf(sa[ks4 >> 1][8 * (ks4 & 1) + jj], scale_log2, -mc));
#pragma unroll
      for (int jj = 0; jj < 8; jj += 2)
        l_run = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pf[jj], pf[jj + 1]}, ones, l_run, false);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        acc[mb] = mfma32(*reinterpret_cast<const bf16x8*>(vt + 32 * mb * VLD + 16 * ks4), pf, acc[mb]);
    }
  };

  // Prologue: K of the group's first two tiles, V of the first; scores of the first tile.
  load_k(0, 0);
  load_k(1, 1);
  load_v(0);
  store_v(0);
  wait_vmem();
  __syncthreads();

  f32x16 s0[2], s1[2];
  if (my_count > 0) {
    scores(0, s0);
    rescale_to(tile_max(my_first, s0));
  }
  if (iters == 1) __syncthreads();  // W goes over K tile 0 during the only iteration

  // Steady iteration j (j + 2 < iters, so tiles j and j + 1 exist for both groups): the MFMAs
  // of tile j+1's scores, tile j's softmax (VALU) and tile j's P V MFMAs form one branch-free
  // block that the compiler can interleave; the max of tile j+1 and the staging of K_{j+2}
  // (already in flight) and V_{j+1} follow.
  auto step_full = [&](int j, f32x16 (&sa)[2], f32x16 (&sb)[2]) {
    load_k(j + 2, j & 1);
    load_v(j + 1);
    scores((j + 1) & 1, sb);
    softmax_pv(sa, j & 1);
    // interleave each score MFMA (with its fragment read) with a share of the softmax VALU
    // work, then each P V MFMA likewise
#pragma unroll
    for (int i = 0; i < 2 * KS + 4 * MB; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
    }
    rescale_to(tile_max(my_first + j + 1, sb));
    store_v((j + 1) & 1);
    wait_vmem();
    __syncthreads();
  };
  // The last two iterations: a group may have no tile j or j + 1, and W comes in last.
  auto step_tail = [&](int j, f32x16 (&sa)[2], f32x16 (&sb)[2]) {
    if (j + 1 < iters) load_v(j + 1);
    if (j == iters - 1) load_w();
    const bool next = j + 1 < my_count;
    if (next) scores((j + 1) & 1, sb);
    if (j < my_count) softmax_pv(sa, j & 1);
    if (next) rescale_to(tile_max(my_first + j + 1, sb));
    if (j + 1 < iters) store_v((j + 1) & 1);
    wait_vmem();
    __syncthreads();
  };
  int j = 0;
  for (; j + 2 < iters; ++j) {
    step_full(j, s0, s1);
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) s0[kb2] = s1[kb2];
  }
  for (; j < iters; ++j) {
    step_tail(j, s0, s1);
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) s0[kb2] = s1[kb2];
  }

  // Epilogue.  W^T is in the K part of LDS.  The two groups exchange, through the V part, the
  // halves of the accumulator that the other one finalises (with their running max and sum):
  // group g finalises output feature blocks [g * MBH, (g + 1) * MBH) (for d < 64 group 0
  // finalises the single block).
  constexpr int MBH = MB >= 2 ? MB / 2 : 1;
  constexpr int NXR = MBH * 16 + 2;  // exported rows: accumulator blocks, then max, then sum
  static_assert((MB >= 2 ? 2 : 1) * NXR * 256 * 4 <= 4 * VT_BYTES, "exchange must fit in the V part");
  static_assert(W_INSTR * 1024 <= 4 * K_BYTES, "W must fit in the K part");
  float* xb = reinterpret_cast<float*>(vreg_lds);  // [exporter][NXR][256]
  const int xl = wq * 64 + lane;
  const int partner = 1 - grp;
  const bool owner = MB >= 2 || grp == 0;
  const bool partner_owns = MB >= 2 || partner == 0;
  if (partner_owns) {
    float* xo = xb + (MB >= 2 ? grp : 0) * NXR * 256;
    const int p0 = MB >= 2 ? partner * MBH : 0;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
      if (mb >= p0 && mb < p0 + MBH)
#pragma unroll
        for (int i = 0; i < 16; ++i) xo[((mb - p0) * 16 + i) * 256 + xl] = acc[mb][i];
    xo[(MBH * 16) * 256 + xl] = m_run;
    xo[(MBH * 16 + 1) * 256 + xl] = l_run;
  }
  __syncthreads();
  if (!owner) return;

  const float* xi = xb + (MB >= 2 ? partner : 0) * NXR * 256;
  const float m1 = xi[(MBH * 16) * 256 + xl], l1 = xi[(MBH * 16 + 1) * 256 + xl];
  const float m = fmaxf(m_run, m1);
  const float a0 = __builtin_amdgcn_exp2f((m_run - m) * scale_log2);
  const float a1 = __builtin_amdgcn_exp2f((m1 - m) * scale_log2);
  const float lsum = l_run * a0 + l1 * a1;
  const float inv = 1.f / (lsum + other_half(lsum, lane));
  const int o0 = MB >= 2 ? grp * MBH : 0;

  // Normalise, then add Q W = Q (phi_q S) with W^T split in two bf16 terms (A fragments from LDS).
  const unsigned char* wfrag = kreg_lds + k_frag;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    if (mb < o0 || mb >= o0 + MBH) continue;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[mb][i] = (acc[mb][i] * a0 + xi[((mb - o0) * 16 + i) * 256 + xl] * a1) * inv;
#pragma unroll
    for (int st = 0; st < KS; ++st)
#pragma unroll
      for (int hl = 0; hl < 2; ++hl)
        acc[mb] = mfma32(*reinterpret_cast<const bf16x8*>(wfrag + ((hl * KS + st) * DP + 32 * mb) * 32), qf[st], acc[mb]);
  }

  if (qrow < T) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      if (mb < o0 || mb >= o0 + MBH) continue;
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
}

template <int D>
hipError_t launch_fwd_d(const FwdArgs& a, hipStream_t stream) {
  const int nq = (a.T + kQTile - 1) / kQTile;
  const int n_items = nq * a.H * a.B;
  const int per_xcd = (n_items + 7) / 8;
  dim3 grid(per_xcd * 8);
  const bf16* q = static_cast<const bf16*>(a.q);
  const bf16* k = static_cast<const bf16*>(a.k);
  const bf16* v = static_cast<const bf16*>(a.v);
  const bf16* wh = static_cast<const bf16*>(a.wt_hi);
  const bf16* wl = static_cast<const bf16*>(a.wt_lo);
  if (a.out_bf16)
    hipLaunchKernelGGL((arl2_fwd_kernel<D, true>), grid, dim3(kThreads), 0, stream, q, k, v, wh, wl, a.out, a.T,
                       a.H, nq, n_items, per_xcd, a.scale_log2);
  else
    hipLaunchKernelGGL((arl2_fwd_kernel<D, false>), grid, dim3(kThreads), 0, stream, q, k, v, wh, wl, a.out, a.T,
                       a.H, nq, n_items, per_xcd, a.scale_log2);
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
