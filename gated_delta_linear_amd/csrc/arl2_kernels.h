// Host-side launchers of the ARL2 kernels.  All pointers are device pointers; shapes are
// validated by the caller (arl2_host.cpp) before any launcher runs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace arl2 {

// Feature dimension padded to a whole 32-row MFMA block.
inline int padded_dim(int d) { return d < 32 ? 32 : d; }
// Tokens per work-group of the state-write kernel, and the number of such chunks.
constexpr int kCommitChunk = 128;
__host__ __device__ inline int commit_chunks(int T) { return (T + kCommitChunk - 1) / kCommitChunk; }

// Per-chunk partial sums of the state write, P_c = K'_c^T diag(beta_c) (V'_c - K'_c S), written
// to partial [B][H][chunks][dp/16][dp/16][4][64] (16 x 16 blocks, each in the C-register order
// of the 16x16 MFMA: block (r, c), register i, lane l = P[16 r + 4 (l / 16) + i][16 c + l % 16]).
struct WritePartialArgs {
  const void* k;
  const void* v;
  const float* beta;    // [B][T][H]
  const void* pkt;      // phi_k^T, [H][dp][dp] (zero beyond d)
  const void* pvt;      // phi_v^T, [H][dp][dp]
  const void* sneg_hi;  // -S_{N-1} as 16x16x32 B fragments, [B][H][dp/32][dp/16][64][8]
  const void* sneg_lo;
  float* partial;
  float knorm_eps;
};

// One launch of the pass kernel, with either part optional: the pass (out = softmax(Q K^T *
// scale) V + Q (phi_q S), when a.out is not null) and the state write's per-chunk partial sums
// (when w is not null), the latter as extra work-groups after the pass's in dispatch order.
// wt_hi / wt_lo hold (phi_q S)^T split into two bf16 terms, layout [B][H][d / 16][dp][16]:
// W^T[j][i] at [i / 16][j][i % 16] (k-step planes of the pass kernel's MFMA fragments).
//
// With Tk >= 0 the launch is plain softmax attention instead (no Q W term, no state write): the
// T queries of q against keys / values [0, Tk) of k / v, whose per-stream slices hold kv_rows
// rows ([B][kv_rows][H][d]): the retained softmax layers' attention over their K/V cache.
struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* wt_hi;
  const void* wt_lo;
  void* out;
  int B, H, T;
  float scale_log2;  // softmax scale * log2(e)
  bool out_bf16;
  int Tk = -1;       // keys of plain attention; -1: the ARL2 pass
  int kv_rows = 0;   // rows per stream slice of k and v (plain attention)
  const float* add = nullptr;  // plain attention: fp32 [B][T][H][d] added to the output, or null
  float* lse = nullptr;        // plain attention: fp32 [B][H][T] row log-sum-exp (log2 units), or null
};
hipError_t launch_fwd(int d, const FwdArgs& a, const WritePartialArgs* w, hipStream_t stream);

// Gate projections from the hidden states x [B][T][H d] bf16 and the weights w [2H][H d] bf16
// (rows 0..H-1 beta, H..2H-1 alpha), bias [2H] fp32: beta [B][T][H] = beta_scale *
// sigmoid(x w_beta^T + bias), and per 16-token block the sums of x w_alpha^T over its tokens,
// alpha_part [B][gate_blocks(T)][H].
struct GateArgs {
  const void* x;
  const void* w;
  const float* bias;
  float beta_scale;
  float* beta;
  float* alpha_part;
  int B, H, d, T;
};
int gate_blocks(int T);
hipError_t launch_gates(const GateArgs& a, hipStream_t stream);

// S_new = alpha S_prev + sum over chunks of the partials (fixed order), then the derived
// forms of S_new: -S_new as 16x16x32 B fragments (hi/lo) and (phi_q S_new)^T (hi/lo).
// alpha == nullptr means alpha = 1, unless alpha_part is given: then alpha = sigmoid(sum of the
// n_ablk partials / T + alpha_bias[h]) (the gate projection's per-frame decay).  chunks == 0
// means no partials (used to load a state).
struct CommitReduceArgs {
  const float* s_prev;  // [B][H][d][d]
  const float* alpha;   // [B][H] or nullptr
  const float* alpha_part = nullptr;  // [B][n_ablk][H] logit sums, or nullptr
  const float* alpha_bias = nullptr;  // [H]
  int n_ablk = 0, T = 0;
  const float* partial; // [B][H][chunks][dp/16][dp/16][4][64]
  int chunks;
  const void* pq;       // phi_q, [H][dp][d] (rows >= d zero)
  float* s_new;         // [B][H][d][d]
  void* sneg_hi;
  void* sneg_lo;
  void* wt_hi;
  void* wt_lo;
  int B, H;
};
hipError_t launch_commit_reduce(int d, const CommitReduceArgs& a, hipStream_t stream);

// Token-level (sequential) access variant, the inter-frame part of one pass: per (stream, head)
// the chunked recurrence over the frame's tokens from S_{N-1} = s_prev, writing o_inter
// [B][T][H][d] fp32 (q'_t S^(t-1)) and, if s_new is not null, S_N = S^(T) - (1 - alpha) S_{N-1}
// into s_new [B][H][d][d].  ws: workspace of seq_workspace_bytes(d, B, H, T).  d = 64 or 128.
struct SeqArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* beta;  // [B][T][H]
  const void* pqt;    // phi_q^T [H][d][d]
  const void* pkt;
  const void* pvt;
  void* ws;
  const float* s_prev;
  const float* alpha;  // [B][H] (used with s_new)
  float* s_new;
  float* o_inter;
  int B, H, T;
  float eps;
};
int seq_chunks(int T);
size_t seq_workspace_bytes(int d, int B, int H, int T);
hipError_t launch_seq(int d, const SeqArgs& a, hipStream_t stream);

// Copy one frame's k, v ([B][T][H][d] bf16) into rows [row0, row0 + T) of the K/V caches
// kc, vc ([B][rows][H][d] bf16).
struct KvAppendArgs {
  const void* k;
  const void* v;
  void* kc;
  void* vc;
  int B, H, d, T;
  int64_t row0, rows;
};
hipError_t launch_kv_append(const KvAppendArgs& a, hipStream_t stream);

// Working layouts of the maps from the caller's phi_q, phi_k, phi_v (bf16 [H][d][d]):
// pq = phi_q padded to [H][dp][d]; pkt = phi_k^T, pvt = phi_v^T and pqt = phi_q^T padded to
// [H][dp][dp].
struct PrepMapsArgs {
  const void* phi_q;
  const void* phi_k;
  const void* phi_v;
  void* pq;
  void* pkt;
  void* pvt;
  void* pqt;
  int H;
};
hipError_t launch_prep_maps(int d, const PrepMapsArgs& a, hipStream_t stream);

// fp32 -> bf16 (round to nearest even) of up to three tensors of n values each (n % 8 == 0,
// 16-byte aligned): the staging of fp32 inputs (io_dtype ARL2_F32).
struct CvtJobs {
  const float* src[3];
  void* dst[3];
};
hipError_t launch_cvt_bf16(const CvtJobs& jobs, int n_jobs, int64_t n, hipStream_t stream);

// y = x W with W given as W^T [N][K] (bf16), x [M][K] bf16, y [M][N] fp32 or bf16, the N output
// features dealt to `parts` row-major outputs of N / parts features each (K % 64 == 0, N % 8 == 0,
// (N / parts) % 4 == 0; 16-byte aligned pointers).
constexpr int kLinearMaxParts = 4;
struct LinearOut {
  void* ptr[kLinearMaxParts];
  int parts;
};
struct LinearArgs {
  const void* x;
  const void* wt;
  LinearOut y;
  int M, N, K;
  bool out_bf16;
};
int linear_tile_n(int M, int N);  // feature width of a work-group's tile (64 or 128)
hipError_t launch_linear(const LinearArgs& a, hipStream_t stream);

// --- backward (arl2_bwd.hip) -------------------------------------------------------------------
// Per (stream, head) d x d matrices in 16x16x32 B-fragment order ([d/32][d/16][64][8] bf16:
// lane l of fragment (s, nb) holds M[32 s + 8 (l / 16) + j][16 nb + l % 16]), split into hi + lo
// for fp32 matrices.  Token tensors are [B][T][H][d].
int bwd_chunks(int T);  // 128-token chunks of the token kernels
// dst = src (n floats, n % 4 == 0), or zeros when src is null
hipError_t launch_bwd_fill(float* dst, const float* src, size_t n, hipStream_t stream);

struct BwdTokArgs {
  const void* q;          // bf16 inputs of the pass (read) or of the clean pass (write)
  const void* k;
  const void* v;
  const float* d_out;     // fp32 output gradient of the pass (read kernel)
  const float* beta;      // [B][T][H] (write kernel)
  float* dq;              // accumulated (+=) by the token kernels
  float* dk;
  float* dv;
  float* dbeta;           // [B][T][H], written by the write kernel
  const void* s_hi;       // S_{N-1}, S_{N-1}^T, G = dL/dS_N, G^T as split fragments, [B][H]
  const void* s_lo;
  const void* st_hi;
  const void* st_lo;
  const void* g_hi;
  const void* g_lo;
  const void* gt_hi;
  const void* gt_lo;
  const void* phik;       // phi_k, phi_v, phi_k^T, phi_v^T, phi_q^T fragments, [H]
  const void* phiv;
  const void* phikt;
  const void* phivt;
  const void* pqt;
  float* part;            // chunk partials: read [B][H][chunks][d][d]; write [B][H][3][d/16][chunks][d][16]
                          // (the sums K^T dR, V^T dR, K^T dU in 16-column strips)
  int B, H, T;
  float knorm_eps;
};

struct BwdPassArgs {
  BwdTokArgs tok;         // q, k, v, d_out, dq, dk, dv (written), st, pqt, part (read partials)
  const float* d_out;
  const float* o_sm;      // the softmax branch's output of the pass, recomputed, fp32
  const float* lse;       // its rows' log-sum-exp (log2 units), [B][H][T]
  void* do_h;             // workspace: d_out in fp16
  float* dvec;            // workspace: dO . O per row, [B][H][T]
  float* gr;              // sum over the frame's passes of Q^T dO, [B][H][d][d]
  bool gr_first;          // first pass of the frame: gr is overwritten
  void* v16;              // workspace: v in fp16, [B][T][H][d]
  void* kt16;             // workspace: k^T, q^T, dO^T in fp16, [B][H][d][tp] (tokens past T zero)
  void* qt16;
  void* dot16;
  int tp;                 // T rounded up to whole 64-key blocks
  float* dq_read;         // workspace: the inter-frame read's part of dq, [B][T][H][d]
  int B, H, T;
  float scale, scale_log2;
};
// The pass backward in stages, which the host orders on two streams:
//   kRead:   the inter-frame read (needs the S fragments): dq_read, and the chunk partials of Q^T dO;
//   kPrep:   dO in fp16, dO . O per row, and the fp16 operands of the attention kernels, in one
//            kernel (needs the recomputed softmax output);
//   kAttn:   dK, dV and dQ of the softmax branch in one launch (needs kPrep; overwrites dk, dv, dq);
//   kFinish: the chunk partials summed into gr, and dq += dq_read (needs kRead and kAttn).
enum class BwdStage { kRead, kPrep, kAttn, kFinish };
hipError_t launch_bwd_stage(int d, BwdStage stage, const BwdPassArgs& a, hipStream_t stream);
int bwd_key_pitch(int T);  // tp: T rounded up to a multiple of 64

struct BwdFragJobs {
  struct Job {
    const float* src;     // [B][H][d][d] fp32
    void* hi;             // fragment order, [B][H]
    void* lo;
    int transpose;        // fragments of src^T
  } job[4];
};
hipError_t launch_bwd_frags(int d, const BwdFragJobs& j, int BH, int n_jobs, hipStream_t stream);

struct BwdFrameArgs {
  const float* g;         // dL/dS_N [B][H][d][d]
  const float* s_prev;    // S_{N-1}
  const float* alpha;     // [B][H]
  const float* gr;        // sum of Q^T dO over the frame's passes, or null (no pass)
  const float* part;      // write partials
  const void* phi_q;      // bf16 [H][d][d]
  float* ds_prev;         // dL/dS_{N-1}
  float* dalpha;          // [B][H]
  float* dphi_q;          // accumulated, [H][d][d]
  float* dphi_k;
  float* dphi_v;
  int B, H, chunks;
};
hipError_t launch_bwd_commit(int d, const BwdTokArgs& t, const BwdFrameArgs& f, hipStream_t stream);
hipError_t launch_bwd_phi_frags(int d, const void* phi, void* dst, int H, bool transpose, hipStream_t stream);

}  // namespace arl2
