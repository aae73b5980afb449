/*
 * hlq.h - C ABI of the HLQ/HOT linear-layer backward on AMD Instinct MI355X
 * (gfx950).
 *
 * The method: "HLQ: Fast and Efficient Backpropagation via Hadamard Low-rank
 * Quantization" (Kim, Park; arXiv 2406.15102), TL;DR, and "HOT:
 * Hadamard-based Optimized Training" (HF paper page abstract; scime.ai summary,
 * section "Approach").  For y = x . w^T the backward needs
 *     g_x = g_y . w            (T x I)
 *     g_w = g_y^T . x          (O x I)
 * g_x runs through 4-bit Hadamard quantization along O; g_w through a
 * Hadamard low-rank approximation along the token dimension T followed by
 * INT8 quantization; x is kept as INT4 from the forward pass (activation
 * buffer compression, ACBP); per-token or per-tensor scales are chosen per
 * path (layer-wise quantizer selection).
 *
 * Conventions for every entry point
 *  - Data pointers are DEVICE pointers owned by the caller; the library never
 *    allocates, frees or keeps them.  Matrices are row-major and densely
 *    packed.  Every data pointer must be 16-byte aligned.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *    enqueue work on it and return; nothing is synchronised.  A kernel fault
 *    surfaces at the caller's next synchronisation.
 *  - Arguments are validated on the host before anything is enqueued; on an
 *    error no work is enqueued and outputs are untouched.
 *  - Thread-safe for distinct (stream, workspace) pairs.  Outputs must not
 *    alias inputs or the workspace.
 *  - Hadamard blocks are aligned and non-overlapping; the transform is the
 *    unnormalised Sylvester matrix H[i][j] = (-1)^popcount(i&j), applied with
 *    fp32 radix-2 butterflies in ascending stage order; the normalising 1/n is
 *    applied once in the GEMM epilogue.
 *  - Quantizer: symmetric absmax; for a scale group with maximum magnitude a,
 *    scale s = fl(a/qmax), code q = clamp(rne(fl(v * fl(qmax/a))), +-qmax);
 *    a == 0 gives s = 0 and all codes 0.  qmax = 7 (INT4) or 127 (INT8).
 */
#ifndef HLQ_H
#define HLQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum hlq_status {
  HLQ_OK = 0,
  HLQ_ERR_NULL = 1,      /* a required pointer is NULL                        */
  HLQ_ERR_SHAPE = 2,     /* T, I or O non-positive or not a required multiple */
  HLQ_ERR_BLOCK = 3,     /* block not in {16, 32, 64, 128}                    */
  HLQ_ERR_RANK = 4,      /* rank not a power of two in [1, block]             */
  HLQ_ERR_MODE = 5,      /* quantizer mode or reduction out of range          */
  HLQ_ERR_DTYPE = 6,     /* dtype code out of range                           */
  HLQ_ERR_ALIGN = 7,     /* a data pointer is not 16-byte aligned             */
  HLQ_ERR_OVERFLOW = 8,  /* an INT32 accumulator could overflow              */
  HLQ_ERR_WORKSPACE = 9, /* workspace NULL or smaller than required           */
  HLQ_ERR_HIP = 10       /* the HIP runtime refused a launch                  */
} hlq_status;

/* Element type of g_y, w and of the forward activation x. */
enum { HLQ_F32 = 0, HLQ_BF16 = 1 };
/* Scale granularity per path (layer-wise quantizer selection, HOT). */
enum { HLQ_PER_TOKEN = 0, HLQ_PER_TENSOR = 1 };
/* Reduction of g_w: MEAN multiplies g_w by 1/T (the "1/B" of the HLQ TL;DR
   identity for g_w, read as a mean over tokens). */
enum { HLQ_SUM = 0, HLQ_MEAN = 1 };

/*
 * ACBP - activation buffer compression (HLQ TL;DR: int4 activation
 * compression; HOT summary, "Approach": stored activations compressed at
 * forward time).
 *   x        [T][I] f32 or bf16 (x_dtype), the layer input.
 *   x_codes  [T][I/2] bytes out: two's-complement INT4 codes, element 2k in
 *            bits 3:0 and element 2k+1 in bits 7:4 of byte k.
 *   x_scales [T] f32 out: one scale per token (qmax 7).
 * Requires T >= 1, I >= 8, I % 8 == 0.
 */
hlq_status hlq_compress_act(const void* x, int x_dtype, int64_t T, int64_t I,
                            uint8_t* x_codes, float* x_scales, void* stream);

/*
 * Forward product of a bf16 linear layer, y = x . w^T, with ACBP fused in
 * (HOT summary, "Approach": stored activations compressed at forward time;
 * HOT abstract: activation buffer compression): the same launch writes the
 * INT4 codes and per-token scales of x that hlq_compress_act would, without a
 * separate read of x from HBM (the first column of output tiles tracks each
 * token row's maximum |x| from the operand fragments of its MFMAs, then
 * re-reads its rows from cache for the codes).
 *   x        [T][I] bf16;  w [O][I] bf16;  I % 32 == 0.
 *   y        [T][O] out, y_dtype HLQ_F32 (fp32 sums) or HLQ_BF16 (rounded to
 *            nearest even).
 *   x_codes  [T][I/2], x_scales [T] out (both NULL: the product only);
 *            bit-identical to hlq_compress_act of x.
 */
hlq_status hlq_linear_forward(const void* x, const void* w, int64_t T, int64_t I, int64_t O,
                              void* y, int y_dtype, uint8_t* x_codes, float* x_scales,
                              void* stream);

/*
 * Bytes of device workspace hlq_linear_backward needs for this shape
 * (0 if the shape or block/rank is invalid).  Independent of modes/dtypes.
 */
size_t hlq_linear_backward_workspace_size(int64_t T, int64_t I, int64_t O,
                                          int block, int rank);

/*
 * The HLQ/HOT backward of one linear layer (HLQ TL;DR; HOT summary,
 * "Approach").
 *   g_y      [T][O] f32 or bf16 (gy_dtype), upstream gradient.
 *   x_codes  [T][I/2], x_scales [T]: the ACBP buffer of hlq_compress_act.
 *   w        [O][I] f32 or bf16 (w_dtype).
 *   block    Hadamard block n in {16, 32, 64, 128}; T % n == 0, O % n == 0.
 *   rank     r, power of two, 1 <= r <= n: rows kept per block of n tokens
 *            on the g_w path (the r lowest-sequency rows, j*n/r).
 *   gx_mode  HLQ_PER_TOKEN: one scale per token of H.g_y and per input channel
 *            of H.w; HLQ_PER_TENSOR: one scale per operand.
 *   gw_mode  HLQ_PER_TOKEN: one scale per output channel of the low-rank g_y
 *            and per input channel of the low-rank x; HLQ_PER_TENSOR: one each.
 *   reduction HLQ_SUM or HLQ_MEAN (g_w only).
 *   g_x      [T][I] f32 out = acc_x * s_gy * s_w / n.
 *   g_w      [O][I] f32 out = acc_w * s_gyl * s_xl / n  (/ T for MEAN).
 *   workspace device buffer of at least hlq_linear_backward_workspace_size()
 *            bytes; holds the quantized operands and scales afterwards (layout
 *            from hlq_workspace_layout).
 * Also requires I % 8 == 0 (stricter than the even I that nibble packing
 * alone needs: every kernel moves a row's codes in whole 32-bit words of 8
 * codes, so rows never split a word; HLQ_ERR_SHAPE otherwise) and that no
 * accumulator can lose exactness: O <= 342391 (49 * O < 2^24, the fp32 sums of
 * the FP6 g_x product) and T*rank/block <= 133143 (127^2 * T' < 2^31, INT32).
 */
hlq_status hlq_linear_backward(const void* g_y, int gy_dtype,
                               const uint8_t* x_codes, const float* x_scales,
                               const void* w, int w_dtype,
                               int64_t T, int64_t I, int64_t O,
                               int block, int rank,
                               int gx_mode, int gw_mode, int reduction,
                               float* g_x, float* g_w,
                               void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * hlq_linear_backward for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, no workspace.  The intermediates go to a static
 * device array owned by the library, HLQ_NOALLOC_SCRATCH_BYTES on each GPU the
 * library runs on, held until the process ends; the call allocates and frees
 * nothing.  Its first call on a device resolves that device's copy of the
 * array (hipGetSymbolAddress, a runtime query; make one call before any graph
 * capture).  A shape whose intermediates do not fit (the workspace of
 * hlq_linear_backward_workspace_size less its split-K partial region, which
 * this call never uses) returns HLQ_ERR_WORKSPACE before anything is
 * enqueued.  All calls on one GPU share its array: calls that can overlap on
 * one GPU (other streams, other host threads) race and must be serialised by
 * the caller.  Each call writes every intermediate before reading it, so the
 * array needs no clearing between calls.
 */
#define HLQ_NOALLOC_SCRATCH_BYTES (64u << 20)
hlq_status hlq_linear_backward_noalloc(const void* g_y, int gy_dtype,
                                       const uint8_t* x_codes, const float* x_scales,
                                       const void* w, int w_dtype,
                                       int64_t T, int64_t I, int64_t O,
                                       int block, int rank,
                                       int gx_mode, int gw_mode, int reduction,
                                       float* g_x, float* g_w, void* stream);

/*
 * The launches hlq_linear_backward enqueues, in order.  Bit k of a step mask
 * selects HLQ_STEP k.
 */
enum {
  HLQ_STEP_TR_MAX = 0,     /* partial maxima of H.g_y (along O), the low-rank
                              g_y and x (along T) and H.w (along O)          */
  HLQ_STEP_TR_REDUCE = 1,  /* fold partials: per-token maxima, scales,
                              tensor maxima                                  */
  HLQ_STEP_TR_QUANT = 2,   /* transforms again -> INT4 / INT8 GEMM operands  */
  HLQ_STEP_GEMM_GX = 3,    /* INT4 GEMM + dequantizing epilogue -> g_x       */
  HLQ_STEP_GEMM_GW = 4,    /* INT8 GEMM + dequantizing epilogue -> g_w       */
  HLQ_STEP_COUNT = 5
};
#define HLQ_STEPS_ALL 0x1Fu

/*
 * hlq_linear_backward restricted to the steps whose bit is set in step_mask
 * (same arguments, same validation).  All steps in one call equal
 * hlq_linear_backward.  A subset re-runs those launches on a workspace that
 * the earlier steps have filled (every step is idempotent given its inputs),
 * which lets a caller time or inspect one kernel of the sequence in place.
 * The GEMM steps read what the QUANT step last wrote to the workspace,
 * including the arrival counters of the K-split g_w tiles it clears.
 */
hlq_status hlq_linear_backward_steps(const void* g_y, int gy_dtype,
                                     const uint8_t* x_codes, const float* x_scales,
                                     const void* w, int w_dtype,
                                     int64_t T, int64_t I, int64_t O,
                                     int block, int rank,
                                     int gx_mode, int gw_mode, int reduction,
                                     float* g_x, float* g_w,
                                     void* workspace, size_t workspace_bytes,
                                     uint32_t step_mask, void* stream);

/*
 * Where hlq_linear_backward leaves its intermediates inside the workspace
 * (byte offsets), for tests and diagnostics.
 * The four code operands are matrices of `rows` rows whose K run is pitch
 * bytes per row, stored in K planes of U bytes: plane p (p = 0 ..
 * pitch/U - 1) holds bytes [p*U, (p+1)*U) of every row's run, row after row,
 * so byte k of row m is at (k / U) * rows * U + m * U + k % U.  U = 96 for
 * q_gy and q_w, 64 for q_gyl and q_xl.
 *   q_gy   T rows, kx_pitch bytes: INT4 codes of H.g_y (along O), stored as
 *          FP6 E2M3 fields (exact for -7..7: sign bit 5, exponent bits 4-3
 *          with bias 1, mantissa bits 2-0) in groups of 128 codes (96 bytes,
 *          one plane): quarter Q of a group (codes 32Q .. 32Q+31) is a
 *          24-byte stream, code j at bits 6j .. 6j+5, and the quarters are
 *          stored in the order 0, 2, 1, 3.  Codes past O are zero fields
 *          (kx_pitch = 96 * ceil(O / 128)).
 *   s_gy   [T] (PER_TOKEN) or [1] f32.
 *   q_w    I rows, kx_pitch bytes: INT4 codes of H.w, transposed (K = O), in
 *          the same FP6 groups.
 *   s_w    [I] or [1] f32.
 *   q_gyl  O rows, kw_pitch bytes: INT8 codes of the low-rank g_y, transposed
 *          (K = T'), zero past T' = T*rank/block.
 *   s_gyl  [O] or [1] f32.
 *   q_xl   I rows, kw_pitch bytes: INT8 codes of the low-rank x, transposed.
 *   s_xl   [I] or [1] f32.
 *   partial  scratch of the split-K GEMMs (contents unspecified).
 * The workspace also holds, after these, the INT32 partial sums and arrival
 * counters of the K-split g_w tiles of the pair launch (contents unspecified).
 */
typedef struct hlq_workspace_layout {
  size_t q_gy, s_gy, q_w, s_w, q_gyl, s_gyl, q_xl, s_xl;
  int64_t kx_pitch;  /* K bytes per row of q_gy and q_w (96-byte planes)  */
  int64_t kw_pitch;  /* K bytes per row of q_gyl and q_xl (64-byte planes) */
  int64_t t_low;     /* T' = T * rank / block           */
  size_t total;      /* == hlq_linear_backward_workspace_size() */
  size_t partial;    /* INT32 split-K partial sums shared by both GEMMs */
  size_t partial_bytes;
  int32_t gx_splits; /* split-K factor of the g_x GEMM (1 = none) */
  int32_t gw_splits; /* split-K factor of the g_w GEMM            */
} hlq_workspace_layout;

hlq_status hlq_workspace_layout_query(int64_t T, int64_t I, int64_t O, int block,
                                      int rank, hlq_workspace_layout* out);

/*
 * INT32 accumulators of the two integer GEMMs, recomputed from a workspace
 * that hlq_linear_backward has filled (tests and diagnostics; HLQ TL;DR:
 * "int8-accelerated" products).  acc_x [T][I] = sum_o q_gy[t,o] q_w[o,i];
 * acc_w [O][I] = sum_t' q_gyl[t',o] q_xl[t',i].
 *   hlq_gemm_pair_acc: the one launch hlq_linear_backward runs for both
 *     GEMMs (same tile grids, K splits and schedule), its epilogue storing
 *     the INT32 sums instead of the fp32 gradients.  It writes the
 *     workspace's split-K partial sums and arrival counters (the codes and
 *     scales are only read), hence the non-const workspace.
 *   hlq_gemm_gx_acc / hlq_gemm_gw_acc: the single-GEMM launches that
 *     hlq_linear_backward_steps runs when only one GEMM step is selected.
 * workspace_bytes is checked against hlq_linear_backward_workspace_size
 * (HLQ_ERR_WORKSPACE); acc_* are device buffers of the sizes above.
 */
hlq_status hlq_gemm_pair_acc(void* workspace, size_t workspace_bytes, int64_t T, int64_t I,
                             int64_t O, int block, int rank, int32_t* acc_x, int32_t* acc_w,
                             void* stream);
hlq_status hlq_gemm_gx_acc(const void* workspace, size_t workspace_bytes, int64_t T,
                           int64_t I, int64_t O, int block, int rank, int32_t* acc_x,
                           void* stream);
hlq_status hlq_gemm_gw_acc(const void* workspace, size_t workspace_bytes, int64_t T,
                           int64_t I, int64_t O, int block, int rank, int32_t* acc_w,
                           void* stream);

/*
 * The HLQ/HOT backward of one 2-D convolution (HLQ abstract: backpropagation
 * of convolutional and linear layers; HOT summary, "Key results": ResNet-50
 * at batch 256), as implicit GEMMs: no im2col or col2im buffer.
 *   y[n,p,q,o] = sum_{r,s,c} x[n, p*stride - pad + r, q*stride - pad + s, c]
 *                * w[o,r,s,c]   (zero padding; P = (H + 2 pad - R)/stride + 1,
 *                                Q = (W + 2 pad - S)/stride + 1)
 * is the linear layer y = im2col(x) . w^T with tokens t = (n, p, q) and
 * features i = (r*S + s)*C + c; the backward is that layer's (same
 * transforms, quantizers, codes and g_w), with the g_w path's low-rank x
 * gathered from the ACBP codes of x itself and g_x the sum over the taps
 * that read each input pixel (col2im).
 *   g_y      [N][P][Q][O] f32 or bf16.
 *   x_codes, x_scales: hlq_compress_act of x viewed as [N*H*W][C] (one scale
 *            per pixel).
 *   w        [O][R][S][C] f32 or bf16.
 *   g_x      [N][H][W][C] f32 out = s_gy * s_w / n * sum over taps and O of
 *            the INT4 code products (an implicit GEMM over the taps).
 *   g_w      [O][R][S][C] f32 out, as hlq_linear_backward's g_w.
 * Requires C % 8 == 0, N*P*Q and O multiples of block, gx_mode ==
 * HLQ_PER_TENSOR (HLQ_ERR_MODE otherwise: per-token scales of H.g_y and H.w
 * do not factor out of the sum over the taps), O*R*S <= 342391 and
 * T' = N*P*Q*rank/block <= 133143 (HLQ_ERR_OVERFLOW), pixel and position
 * counts below 2^31.  workspace: hlq_conv_backward_workspace_size bytes.
 * Launches: the transform MAX, reduce and QUANT passes, the INT8 g_w GEMM
 * (with split-K partials when its grid is small), the INT4 input-gradient GEMM.
 */
size_t hlq_conv_backward_workspace_size(int64_t N, int64_t H, int64_t W, int64_t C, int64_t O,
                                        int R, int S, int stride, int pad, int block,
                                        int rank);
hlq_status hlq_conv_backward(const void* g_y, int gy_dtype, const uint8_t* x_codes,
                             const float* x_scales, const void* w, int w_dtype, int64_t N,
                             int64_t H, int64_t W, int64_t C, int64_t O, int R, int S,
                             int stride, int pad, int block, int rank, int gx_mode,
                             int gw_mode, int reduction, float* g_x, float* g_w,
                             void* workspace, size_t workspace_bytes, void* stream);
/*
 * INT32 accumulators of the convolution backward's two GEMMs from a workspace
 * hlq_conv_backward has filled (tests): acc_x [N*H*W][C] (sums over taps and
 * O, before the per-tensor scales), acc_w [O][R*S*C].
 */
hlq_status hlq_conv_gemm_acc(const void* workspace, size_t workspace_bytes, int64_t N,
                             int64_t H, int64_t W, int64_t C, int64_t O, int R, int S,
                             int stride, int pad, int block, int rank, int32_t* acc_x,
                             int32_t* acc_w, void* stream);

/*
 * Ablation variants: the backward with another transform / quantizer on
 * either path, for synthetic error studies (HOT summary, "Measured effects":
 * the ResNet50 ablation rows; "Surprising findings": internal and external
 * Hadamard low-rank approximation on the activation-gradient path,
 * quantization sensitivity of the weight-gradient path).  Each path is one
 * integer GEMM over its contracted dimension K (O for g_x, T for g_w):
 *   HLQ_VAR_HQ4       block Hadamard along K on both operands, INT4 (the
 *                     method's g_x path);
 *   HLQ_VAR_Q4        no transform, INT4;
 *   HLQ_VAR_HLA8_INT  low-rank rows j*n/r of the block Hadamard along K on
 *                     both operands ("internal" HLA), INT8 (the method's g_w
 *                     path);
 *   HLQ_VAR_HLA8_EXT  low-rank Hadamard along the left operand's output
 *                     dimension (T for g_x, O for g_w: "external" HLA), none
 *                     on the right operand, INT8; the r rows per block of the
 *                     product are expanded back to n by H_low^T / n.
 * The pages list HLA without a quantizer; HOT pairs it with INT8, as here.
 * Scale groups and modes as hlq_linear_backward.  Plain kernels, one thread
 * per block of n source values, then the library's INT8 GEMM (INT4 codes are
 * stored one per byte): not the hot path.  acc_x [T or T*r/n][I] and acc_w
 * [O or O*r/n][I] (device, may be NULL) receive the GEMMs' INT32 sums.
 * Errors as hlq_linear_backward; HLQ_ERR_MODE for an unknown variant.
 */
enum { HLQ_VAR_HQ4 = 0, HLQ_VAR_Q4 = 1, HLQ_VAR_HLA8_INT = 2, HLQ_VAR_HLA8_EXT = 3 };
size_t hlq_ablation_workspace_size(int64_t T, int64_t I, int64_t O, int block, int rank,
                                   int gx_variant, int gw_variant);
hlq_status hlq_linear_backward_ablation(const void* g_y, int gy_dtype, const uint8_t* x_codes,
                                        const float* x_scales, const void* w, int w_dtype,
                                        int64_t T, int64_t I, int64_t O, int block, int rank,
                                        int gx_variant, int gw_variant, int gx_mode,
                                        int gw_mode, int reduction, float* g_x, float* g_w,
                                        int32_t* acc_x, int32_t* acc_w, void* workspace,
                                        size_t workspace_bytes, void* stream);

/*
 * Layer-wise quantizer selection (LQS).  "HOT: Hadamard-based Optimized
 * Training": HF page abstract (layer-wise quantizer selection), scime.ai
 * summary "Approach" (per-token vs per-tensor chosen per layer) and
 * "Limitations" (chosen from a calibration set with a 50% MSE-difference
 * threshold).  The pages name the threshold, not the error measure; the
 * reading taken here: the squared reconstruction error of each quantized
 * GEMM operand under each mode.
 *
 * hlq_lqs_accumulate adds one calibration batch (the same inputs as
 * hlq_linear_backward) to `stats`, a DEVICE array of 16 doubles the caller
 * zeroes once and keeps across batches.  For operand k = 0 (H.g_y along O,
 * INT4), 1 (H.w along O, INT4), 2 (low-rank g_y along T, INT8), 3 (low-rank
 * x along T, INT8), with v the fp32 transformed values of the backward:
 *   stats[4k]   += sum v^2
 *   stats[4k+1] += sum e^2 with PER_TOKEN scales (one per group of reading R6)
 *   stats[4k+2] += sum e^2 with a PER_TENSOR scale
 *   stats[4k+3] += number of elements
 * where e = fl32(v - fl32(s * q)) with the code q and scale s the backward's
 * quantizer gives v; e^2 and the sums are fp64 (fixed summation order, so a
 * call is reproducible).  Five launches on `stream`: the backward's MAX and
 * reduce launches with both paths per token (group and tensor maxima,
 * scales), two error passes (row and column operands) and a fixed-order
 * fold.  The workspace (at least
 * hlq_lqs_workspace_size bytes) holds the backward's workspace regions
 * followed by per-workgroup partial sums.  Shape
 * rules and errors as for hlq_linear_backward; `stats` must be 16-byte
 * aligned; HLQ_ERR_OVERFLOW also when g_y, w or the ACBP codes hold 4 GiB or
 * more (the statistics kernels use 32-bit byte offsets).
 *
 * hlq_lqs_select is a host function on a HOST copy of the 16 statistics.
 * A path's error in a mode is the sum over its two operands of
 * SSE / sum v^2 (0 for an all-zero operand).  The path takes HLQ_PER_TOKEN
 * when its per-tensor error exceeds (1 + threshold) times its per-token
 * error, else HLQ_PER_TENSOR (the single-scale quantizer).  The pages'
 * threshold is 0.5.  Errors: HLQ_ERR_NULL, HLQ_ERR_MODE (threshold negative
 * or NaN).
 */
size_t hlq_lqs_workspace_size(int64_t T, int64_t I, int64_t O, int block, int rank);
hlq_status hlq_lqs_accumulate(const void* g_y, int gy_dtype, const uint8_t* x_codes,
                              const float* x_scales, const void* w, int w_dtype,
                              int64_t T, int64_t I, int64_t O, int block, int rank,
                              double* stats, void* workspace, size_t workspace_bytes,
                              void* stream);
hlq_status hlq_lqs_select(const double* stats, double threshold, int* gx_mode,
                          int* gw_mode);

/* Static text for a status code (never NULL). */
const char* hlq_status_string(int status);

/* Library ABI version (major*100 + minor). */
int hlq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* HLQ_H */
