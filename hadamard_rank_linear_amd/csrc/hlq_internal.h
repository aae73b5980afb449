// Internal launch interface between the C ABI layer (hlq_api.cpp) and the
// gfx950 kernels (hlq_tr.hip, hlq_gemm.hip, hlq_lqs.hip, hlq_acbp.hip).
// Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace hlq {

enum GemmEpi { EPI_F32 = 0, EPI_I32 = 1, EPI_PARTIAL = 2, EPI_BF16 = 3 };
enum TrPass { PASS_MAX = 0, PASS_QUANT = 1 };

// Rows and columns of one transform tile (see the tile engine in
// hlq_tr.hip); the host sizes the partial-maximum arrays with them.
constexpr int TR_ROWS = 128;
constexpr int TR_COLS = 128;
// Atomic slots per tensor maximum: reduce block b folds into slot b % 64, so
// same-address atomics queue 64 times less; readers fold the 64 slots (one
// load per lane and a wave maximum).
constexpr int TMAX_SLOTS = 64;
constexpr int TR_GY_REG_ROWS = 64;   // token rows of a register-resident g_y tile (one wave)
constexpr int TR_GY_REG_SPAN = 256;  // token rows of a register workgroup (four tiles)

// Everything the three transform launches (MAX, reduce, QUANT) read and write.
struct TrArgs {
  const void* gy;  int gy_dt;
  const uint8_t* xc; const float* xs;
  const void* w;   int w_dt;
  int64_t T, I, O, kxb, kwb, tl;
  int gx_tok, gw_tok;
  uint8_t *q_gy, *q_w, *q_gyl, *q_xl;
  float *s_gy, *s_w, *s_gyl, *s_xl;
  // partial maxima: rows of H.g_y per column chunk [nch_o][T]; low-rank g_y
  // columns per token range [ntr_gy][O] (ntr_gy <= ceil(T / TR_ROWS));
  // low-rank x [ntr_t][I]; H.w [ntr_o][I]
  float *part_gy, *part_gyl, *part_xl, *part_w;
  // reciprocal scales qmax / max of the folded maxima (per-token modes)
  float *inv_gy, *inv_gyl, *inv_xl, *inv_w;
  // tensor maxima as float bit patterns, [4][TMAX_SLOTS] (the maximum of
  // list l is the maximum of its slots): list 0 H.g_y, 1 H.w, 2 low-rank
  // g_y, 3 low-rank x (zeroed by the MAX pass, folded into by reduce)
  unsigned* tmax;
  // tok_tmax: reduce also folds the per-token lists' tensor maxima (the LQS
  // statistics read them; the backward reads only the per-tensor lists')
  int tok_tmax;
  int64_t nch_o, nch_i, ntr_t, ntr_o;
  // gy_reg: the MAX pass runs g_y on the register-resident kernel (bf16 g_y,
  // n <= 64, TR_GY_REG_ROWS-token tiles, four per workgroup: wg_gy
  // workgroups of TR_GY_REG_SPAN tokens x TR_COLS channels); ntr_gy = its
  // token spans (rows of part_gyl).  The LDS engine uses TR_ROWS-token tiles.
  int gy_reg;
  int64_t ntr_gy;
  int64_t wg_gy, wg_x, wg_w;  // tiles (register g_y: workgroups) of each job
  int64_t gy_workers;         // LDS-engine g_y tiles of the transform launch (set per launch)
  int64_t gyreg_wgs;          // register-path g_y workgroups of that launch (4 tiles each)
  // Convolution (conv = 1): the x job gathers im2col of the ACBP-coded input
  // [N][Hc][Wc][Cc] (one scale per pixel) for the output grid P x Q, taps
  // R x S (feature (r*S + s)*Cc + c, so I = R*S*Cc), stride, zero padding.
  int conv;
  int64_t Hc, Wc, Cc, P, Q, S, cstride, cpad;
  uint8_t* zero_row;          // kxb zero bytes written by QUANT (conv), else null
  unsigned* pair_ctr;         // arrival counters of the pair GEMM, cleared by QUANT
  int64_t pair_nctr;
};

// Launch configuration of one integer GEMM C[m][n] = sum_k A[m][k] B[n][k],
// both operands K-contiguous ("NT").
struct GemmPlan {
  int cfg;         // tile configuration index (see plan_gemm)
  int bm, bn;      // block tile
  int kb;          // K bytes per pipeline stage (the operand pitch is a multiple)
  int splits;      // split-K factor (partials summed by gemm_finalize)
  int64_t stages;  // K stages in total
  int64_t sps;     // stages per split (the last split takes the remainder)
};

GemmPlan plan_gemm(bool int4, int64_t M, int64_t N, int64_t kbytes);

// Layer-wise quantizer selection statistics (one calibration batch).  The
// per-token scales and the tensor maxima come from the backward's MAX and
// reduce launches run with both paths per token.
constexpr int LQS_STRIP = 4;  // blocks per thread along a column operand
// row blocks per thread of the LQS row pass (two while they fit registers)
constexpr int lqs_row_blocks(int n) { return n <= 32 ? 2 : 1; }
struct LqsArgs {
  const void* gy; int gy_dt;
  const uint8_t* xc; const float* xs;
  const void* w; int w_dt;
  int64_t T, I, O;
  int r;
  // per operand (0 H.g_y, 1 H.w, 2 low-rank g_y, 3 low-rank x): per-token
  // reciprocal scales and scales, [T], [I], [O], [I]
  const float* tok_inv[4];
  const float* tok_s[4];
  const unsigned* tmax;  // [4][TMAX_SLOTS] slots of the tensor maxima (float bits)
  double* part;          // [wg0[4]][3] per-workgroup sums of v^2, e_tok^2, e_ten^2
  double* stats;         // [16] the caller's accumulated statistics
  int64_t items[4];      // op 0: threads (one row block each); ops 1-3: tiles of
                         // 64 columns x LQS_STRIP blocks (one wave each)
  int64_t wg0[5];        // first partial-sum slot of each operand (op 0: one per
                         // 256-thread workgroup, ops 1-3: one per tile); wg0[4] = total
  double count[4];       // elements per operand
};

// ERR pass and the final fold (after launch_tr MAX and launch_tr_reduce).
hipError_t launch_lqs(const LqsArgs& a, int n, hipStream_t s);

// Device address of the current device's static scratch array
// (hlq_linear_backward_noalloc), nullptr on a runtime error.
void* noalloc_scratch();

hipError_t launch_acbp(const void* x, int dtype, int64_t T, int64_t I, uint8_t* codes,
                       float* scales, hipStream_t s);

// Transform pass over g_y, the ACBP codes of x and w (one grid for all three).
hipError_t launch_tr(const TrArgs& a, int pass, int n, int r, hipStream_t s);
// The same for one block size (one object file each; grid already sized).
hipError_t launch_tr_n16(const TrArgs& a, int pass, int r, dim3 g, hipStream_t s);
hipError_t launch_tr_n32(const TrArgs& a, int pass, int r, dim3 g, hipStream_t s);
hipError_t launch_tr_n64(const TrArgs& a, int pass, int r, dim3 g, hipStream_t s);
hipError_t launch_tr_n128(const TrArgs& a, int pass, int r, dim3 g, hipStream_t s);
// Fold the partial maxima of the MAX pass (per-token maxima, scales, tensor maxima).
hipError_t launch_tr_reduce(const TrArgs& a, hipStream_t s);

hipError_t launch_gemm(bool int4, const uint8_t* A, const uint8_t* B, int64_t M,
                       int64_t N, int64_t pitch, const GemmPlan& plan,
                       const float* sa, int sa_step, const float* sb, int sb_step,
                       float alpha, GemmEpi epi, float* C, int32_t* Ci,
                       int32_t* partial, hipStream_t s);

// Tiles of the pair launch (both GEMMs of the backward in one grid).  The g_w
// tiles (long K = T') may split K over nsplit workgroups: each stores its INT32
// sums to `part` (device-coherent), counts itself into its tile's counter, and
// the last to arrive adds the others' sums and runs the epilogue.
struct PairPlan {
  bool big;             // 256 x 256 tiles, 512-thread workgroups (one per CU)
  int wcfg, wbm, wbn;   // g_w tile configuration (rows of O x rows of I)
  int64_t wstages;      // K stages of a g_w tile (its KB may differ from the plan's)
  int64_t tw, tx;       // g_w and g_x tiles
  int nsplit;           // K splits of each g_w tile (1: none)
  int64_t sps;          // K stages per split (the last takes the remainder)
  size_t part_bytes;    // INT32 partial sums, tw * nsplit * wbm * wbn * 4 (0 without split)
  int64_t nctr;         // arrival counters, one per g_w tile (0 without split)
};
PairPlan plan_pair(int64_t T, int64_t I, int64_t O, const GemmPlan& px, const GemmPlan& pw);

// Both GEMMs of the backward in one launch.  EPI_F32 (the backward): g_x =
// acc(q_gy, q_w) * s_gy * s_w * gx_alpha, g_w = acc(q_gyl, q_xl) * s_gyl *
// s_xl * gw_alpha (scale steps 1 per-token, 0 per-tensor).  EPI_I32: the
// same launch stores the INT32 accumulators to acc_x [T][I] and acc_w [O][I]
// instead (scales and fp32 outputs unused).  With pp.nsplit > 1, part holds
// pp.part_bytes and ctr pp.nctr counters that must read zero at launch (the
// QUANT transform pass clears them; every launch leaves them zero);
// zero_ctr clears them first with a small kernel.
hipError_t launch_gemm_pair(const uint8_t* gxA, const uint8_t* gxB, int64_t T, int64_t I,
                            int64_t kx_pitch, const GemmPlan& px, const float* s_gy,
                            const float* s_w, int gx_step, float gx_alpha, float* g_x,
                            const uint8_t* gwA, const uint8_t* gwB, int64_t O, int64_t kw_pitch,
                            const GemmPlan& pw, const float* s_gyl, const float* s_xl,
                            int gw_step, float gw_alpha, float* g_w, const PairPlan& pp,
                            int32_t* part, unsigned* ctr, bool zero_ctr, hipStream_t s,
                            GemmEpi epi = EPI_F32, int32_t* acc_x = nullptr,
                            int32_t* acc_w = nullptr);

// Input gradient of a convolution, implicit GEMM over the taps:
// g_x[(n,h,w)][c] = alpha * s_gy * s_w * sum_{tap, o} q_gy[(n,p,q)][o] *
// q_w[tap * C + c][o] over the taps whose (p, q) is a whole in-range output
// position (per-tensor scales only).  EPI_I32 stores the INT32 sums instead.
struct ConvGemm {
  const uint8_t* q_gy;  // N*P*Q rows x kx_pitch: FP6 codes of H.g_y (96-byte K planes)
  const uint8_t* q_w;   // R*S*C rows x kx_pitch: FP6 codes of H.w (96-byte K planes)
  const uint8_t* zero;  // kx_pitch (>= 96) zero bytes
  int64_t kx_pitch, N, H, W, C, P, Q, S, taps;
  int stride, pad;
  const float* s_gy;    // [1]
  const float* s_w;     // [1]
  float alpha;          // 1 / n
  GemmEpi epi;
  float* g_x;           // [N*H*W][C]
  int32_t* acc_x;       // [N*H*W][C]
};
hipError_t launch_dgrad(const ConvGemm& c, hipStream_t s);

// One GEMM operand of an ablation variant (hlq_ablation.hip): V[k][m] read
// from src (dt 0 fp32 / 1 bf16 matrix [rows][cols], dt 2 ACBP codes with
// per-row scales), V = S^T (m_is_row) or S; transform along M (along_m) or
// K over blocks of n: kind 0 none, 1 full Hadamard, 2 low rank (rows j*n/r).
// Threads: lines x blocks (lines = the other axis' length, blocks = the
// transformed axis / n).  Output codes q [Mo][Kpad] (K' = Ko valid), scales
// s [Mo] or [1], maxima maxbits (float bits) of the same size.
struct AblOperand {
  const void* src; int dt;
  const uint8_t* codes; const float* cscales;
  int64_t rows, cols;
  int m_is_row, along_m, kind, r, qmax, per_token;
  int64_t lines, blocks, Mo, Ko, Kpad;
  int8_t* q; float* s; unsigned* maxbits;
};
hipError_t launch_abl_operand(const AblOperand& o, int n, hipStream_t s);
hipError_t launch_abl_expand(const float* G, int64_t rows, int64_t cols, int n, int r,
                             float alpha, float* out, hipStream_t s);

// Forward product y = x . w^T (bf16 x [T][I], w [O][I]; I % 32 == 0) into
// y32 (fp32) or y16 (bf16, round to nearest even), and the ACBP codes
// [T][I/2] and scales [T] of x when codes is set.
hipError_t launch_forward(const uint16_t* x, const uint16_t* w, int64_t T, int64_t I, int64_t O,
                          float* y32, uint16_t* y16, uint8_t* codes, float* scales,
                          hipStream_t s);

hipError_t launch_gemm_finalize(const int32_t* partial, int splits, int64_t M,
                                int64_t N, const float* sa, int sa_step,
                                const float* sb, int sb_step, float alpha, float* C,
                                hipStream_t s);

}  // namespace hlq
