// C ABI of the HLQ/HOT linear-layer backward: argument validation, workspace
// carving and the launch sequence.  Everything here runs on the host; all
// arithmetic of the method happens in the kernels of hlq_*.hip.
//
// Launch sequence of hlq_linear_backward (one stream, no host sync; each
// line is one HLQ_STEP_* of hlq.h):
//   1. MAX pass of the transform engine over g_y, the ACBP codes of x and w:
//      partial maxima of H.g_y rows, low-rank g_y / x columns, H.w columns
//   2. fold the partials: per-token maxima and scales, tensor maxima
//   3. QUANT pass: the same transforms again, quantized and written as the
//      GEMM operands (INT4 H.g_y rows, INT4 H.w transposed, INT8 low-rank g_y
//      and x transposed), K padding zeroed
//   4. INT4 GEMM with fused dequantizing epilogue -> g_x
//   5. INT8 GEMM with fused dequantizing epilogue -> g_w
// Steps 4 and 5 requested together run as one launch holding both tile grids
// (no split-K); either alone uses split-K partials + a finalize pass when its
// tile grid is smaller than the CU count.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include "../../include/hlq.h"
#include "hlq_internal.h"

namespace {

constexpr int64_t kMaxO = 342391;       // 49 * O < 2^24: the FP6 product's fp32 sums stay exact
constexpr int64_t kMaxTLow = 133143;    // 127^2 * T' < 2^31

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

bool pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Layout {
  hlq_workspace_layout pub;
  size_t part_gy, part_gyl, part_xl, part_w;  // partial maxima of the MAX pass
  size_t inv_gy, inv_gyl, inv_xl, inv_w;      // reciprocal scales of per-token maxima
  size_t tmax;                                // tensor maxima (float bits) [4][TMAX_SLOTS]
  size_t partial;                             // int32 split-K partials
  int64_t nch_o, nch_i, ntr_t, ntr_o;         // transform tile grid
  hlq::GemmPlan plan_gx, plan_gw;
  hlq::PairPlan pair;                         // tiles and g_w K splits of the pair launch
  size_t pair_part, pair_ctr;                 // its INT32 partial sums, arrival counters
};

hlq_status check_shape(int64_t T, int64_t I, int64_t O, int block, int rank) {
  if (T <= 0 || I <= 0 || O <= 0) return HLQ_ERR_SHAPE;
  if (block != 16 && block != 32 && block != 64 && block != 128) return HLQ_ERR_BLOCK;
  if (!pow2(rank) || rank > block) return HLQ_ERR_RANK;
  if (T % block || O % block || I % 8) return HLQ_ERR_SHAPE;
  if (O > kMaxO || T / block * rank > kMaxTLow) return HLQ_ERR_OVERFLOW;
  return HLQ_OK;
}

Layout make_layout(int64_t T, int64_t I, int64_t O, int block, int rank) {
  Layout L;
  memset(&L, 0, sizeof(L));
  const int64_t t_low = T / block * rank;
  const int64_t kx = (O + 127) / 128 * 128;  // codes per row: FP6 groups of 128 in 96 bytes
  const int64_t kxb = kx / 128 * 96;
  const int64_t kwb = (t_low + 127) / 128 * 128;  // INT8 codes, 128-byte stages
  L.pub.kx_pitch = kxb;
  L.pub.kw_pitch = kwb;
  L.pub.t_low = t_low;
  L.plan_gx = hlq::plan_gemm(true, T, I, kxb);
  L.plan_gw = hlq::plan_gemm(false, O, I, kwb);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off = align256(off + bytes);
    return at;
  };
  L.pub.q_gy = take((size_t)T * kxb);
  L.pub.s_gy = take((size_t)T * 4);
  L.pub.q_w = take((size_t)I * kxb);
  L.pub.s_w = take((size_t)I * 4);
  L.pub.q_gyl = take((size_t)O * kwb);
  L.pub.s_gyl = take((size_t)O * 4);
  L.pub.q_xl = take((size_t)I * kwb);
  L.pub.s_xl = take((size_t)I * 4);
  L.nch_o = (O + hlq::TR_COLS - 1) / hlq::TR_COLS;
  L.nch_i = (I + hlq::TR_COLS - 1) / hlq::TR_COLS;
  L.ntr_t = (T + hlq::TR_ROWS - 1) / hlq::TR_ROWS;
  L.ntr_o = (O + hlq::TR_ROWS - 1) / hlq::TR_ROWS;
  L.part_gy = take((size_t)L.nch_o * T * 4);
  L.part_gyl = take((size_t)L.ntr_t * O * 4);  // 128-token tiles or 256-token register spans
  L.part_xl = take((size_t)L.ntr_t * I * 4);
  L.part_w = take((size_t)L.ntr_o * I * 4);
  L.inv_gy = take((size_t)T * 4);
  L.inv_gyl = take((size_t)O * 4);
  L.inv_xl = take((size_t)I * 4);
  L.inv_w = take((size_t)I * 4);
  L.tmax = take(4 * hlq::TMAX_SLOTS * 4);
  // split-K partials: the two GEMMs run one after the other on one stream and
  // share this buffer
  size_t part = 0;
  if (L.plan_gx.splits > 1) part = (size_t)L.plan_gx.splits * T * I * 4;
  if (L.plan_gw.splits > 1 && (size_t)L.plan_gw.splits * O * I * 4 > part)
    part = (size_t)L.plan_gw.splits * O * I * 4;
  L.pub.partial_bytes = part;
  L.pub.gx_splits = L.plan_gx.splits;
  L.pub.gw_splits = L.plan_gw.splits;
  L.partial = take(part);
  L.pub.partial = L.partial;
  L.pair = hlq::plan_pair(T, I, O, L.plan_gx, L.plan_gw);
  L.pair_part = take(L.pair.part_bytes);
  L.pair_ctr = take((size_t)L.pair.nctr * 4);
  L.pub.total = off;
  return L;
}

// Workspace of hlq_lqs_accumulate: the backward's (its MAX and reduce
// launches run on it) followed by the per-workgroup partial sums.
struct LqsLayout {
  size_t part, total;
  int64_t items[4], wg0[5];
  double count[4];
};

LqsLayout make_lqs_layout(int64_t T, int64_t I, int64_t O, int block, int rank) {
  LqsLayout L;
  memset(&L, 0, sizeof(L));
  const int64_t n = block, S = hlq::LQS_STRIP;
  // op 0: one thread per row block, 256-thread workgroups; ops 1-3: one
  // 64-column x LQS_STRIP-block tile per single-wave workgroup
  L.items[0] = T * (O / n);
  L.items[1] = (I + 63) / 64 * ((O / n + S - 1) / S);
  L.items[2] = (O + 63) / 64 * ((T / n + S - 1) / S);
  L.items[3] = (I + 63) / 64 * ((T / n + S - 1) / S);
  L.count[0] = (double)(T * O);
  L.count[1] = (double)(O * I);
  L.count[2] = (double)(T / n * rank * O);
  L.count[3] = (double)(T / n * rank * I);
  L.wg0[0] = 0;
  const int64_t rows_per_wg = 256 * hlq::lqs_row_blocks(block);
  L.wg0[1] = (L.items[0] + rows_per_wg - 1) / rows_per_wg;
  for (int k = 1; k < 4; ++k) L.wg0[k + 1] = L.wg0[k] + L.items[k];
  L.part = align256(make_layout(T, I, O, block, rank).pub.total);
  L.total = align256(L.part + (size_t)L.wg0[4] * 3 * 8);
  return L;
}

// Arguments of the transform launches (MAX, reduce, QUANT) over the
// backward's workspace layout.
hlq::TrArgs make_tr_args(const Layout& L, const void* g_y, int gy_dtype, const uint8_t* x_codes,
                         const float* x_scales, const void* w, int w_dtype, int64_t T,
                         int64_t I, int64_t O, int block, bool gx_tok, bool gw_tok,
                         uint8_t* ws) {
  auto f32 = [&](size_t off) { return reinterpret_cast<float*>(ws + off); };
  hlq::TrArgs a;
  a.gy = g_y; a.gy_dt = gy_dtype;
  a.xc = x_codes; a.xs = x_scales;
  a.w = w; a.w_dt = w_dtype;
  a.T = T; a.I = I; a.O = O;
  a.kxb = L.pub.kx_pitch; a.kwb = L.pub.kw_pitch; a.tl = L.pub.t_low;
  a.gx_tok = gx_tok; a.gw_tok = gw_tok;
  a.q_gy = ws + L.pub.q_gy; a.q_w = ws + L.pub.q_w;
  a.q_gyl = ws + L.pub.q_gyl; a.q_xl = ws + L.pub.q_xl;
  a.s_gy = f32(L.pub.s_gy); a.s_w = f32(L.pub.s_w);
  a.s_gyl = f32(L.pub.s_gyl); a.s_xl = f32(L.pub.s_xl);
  a.part_gy = f32(L.part_gy); a.part_gyl = f32(L.part_gyl);
  a.part_xl = f32(L.part_xl); a.part_w = f32(L.part_w);
  a.inv_gy = f32(L.inv_gy); a.inv_gyl = f32(L.inv_gyl);
  a.inv_xl = f32(L.inv_xl); a.inv_w = f32(L.inv_w);
  a.tmax = reinterpret_cast<unsigned*>(ws + L.tmax);
  a.tok_tmax = 0;
  a.nch_o = L.nch_o; a.nch_i = L.nch_i; a.ntr_t = L.ntr_t; a.ntr_o = L.ntr_o;
  // bf16 g_y with n <= 64 runs the register-resident kernel (64-token tiles,
  // one partial of the low-rank column maxima per 256 tokens)
  a.gy_reg = (gy_dtype == HLQ_BF16 && block <= 64) ? 1 : 0;
  a.ntr_gy = a.gy_reg ? (T + hlq::TR_GY_REG_SPAN - 1) / hlq::TR_GY_REG_SPAN : L.ntr_t;
  a.wg_gy = a.ntr_gy * L.nch_o;
  a.gy_workers = 0;  // both chosen per pass by launch_tr
  a.gyreg_wgs = 0;
  a.wg_x = L.ntr_t * L.nch_i;
  a.wg_w = L.ntr_o * L.nch_i;
  a.conv = 0;
  a.Hc = a.Wc = a.Cc = a.P = a.Q = a.S = a.cstride = a.cpad = 0;
  a.zero_row = nullptr;
  a.pair_ctr = reinterpret_cast<unsigned*>(ws + L.pair_ctr);
  a.pair_nctr = L.pair.nctr;
  return a;
}

#define HLQ_TRY(expr)                       \
  do {                                      \
    if ((expr) != hipSuccess) return HLQ_ERR_HIP; \
  } while (0)

}  // namespace

extern "C" {

int hlq_version(void) { return 200; }

const char* hlq_status_string(int status) {
  switch (status) {
    case HLQ_OK: return "ok";
    case HLQ_ERR_NULL: return "a required pointer is NULL";
    case HLQ_ERR_SHAPE: return "invalid shape (T, I, O > 0; T, O multiples of block; I multiple of 8)";
    case HLQ_ERR_BLOCK: return "block must be 16, 32, 64 or 128";
    case HLQ_ERR_RANK: return "rank must be a power of two in [1, block]";
    case HLQ_ERR_MODE: return "quantizer mode or reduction out of range";
    case HLQ_ERR_DTYPE: return "dtype must be HLQ_F32 or HLQ_BF16";
    case HLQ_ERR_ALIGN: return "data pointers must be 16-byte aligned";
    case HLQ_ERR_OVERFLOW: return "an INT32 accumulator could overflow (O or T*rank/block too large)";
    case HLQ_ERR_WORKSPACE: return "workspace missing or too small";
    case HLQ_ERR_HIP: return "HIP runtime error while enqueueing";
    default: return "unknown status";
  }
}

hlq_status hlq_compress_act(const void* x, int x_dtype, int64_t T, int64_t I,
                            uint8_t* x_codes, float* x_scales, void* stream) {
  if (!x || !x_codes || !x_scales) return HLQ_ERR_NULL;
  if (x_dtype != HLQ_F32 && x_dtype != HLQ_BF16) return HLQ_ERR_DTYPE;
  if (T <= 0 || I < 8 || I % 8) return HLQ_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(x_codes) || !aligned16(x_scales)) return HLQ_ERR_ALIGN;
  HLQ_TRY(hlq::launch_acbp(x, x_dtype, T, I, x_codes, x_scales,
                           static_cast<hipStream_t>(stream)));
  return HLQ_OK;
}

hlq_status hlq_linear_forward(const void* x, const void* w, int64_t T, int64_t I, int64_t O,
                              void* y, int y_dtype, uint8_t* x_codes, float* x_scales,
                              void* stream) {
  if (!x || !w || !y) return HLQ_ERR_NULL;
  if ((x_codes == nullptr) != (x_scales == nullptr)) return HLQ_ERR_NULL;
  if (y_dtype != HLQ_F32 && y_dtype != HLQ_BF16) return HLQ_ERR_DTYPE;
  if (T <= 0 || O <= 0 || I < 32 || I % 32) return HLQ_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(w) || !aligned16(y) || (x_codes && !aligned16(x_codes)) ||
      (x_scales && !aligned16(x_scales)))
    return HLQ_ERR_ALIGN;
  HLQ_TRY(hlq::launch_forward(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w),
                              T, I, O, y_dtype == HLQ_F32 ? static_cast<float*>(y) : nullptr,
                              y_dtype == HLQ_BF16 ? static_cast<uint16_t*>(y) : nullptr, x_codes,
                              x_scales, static_cast<hipStream_t>(stream)));
  return HLQ_OK;
}

size_t hlq_linear_backward_workspace_size(int64_t T, int64_t I, int64_t O, int block,
                                          int rank) {
  if (check_shape(T, I, O, block, rank) != HLQ_OK) return 0;
  return make_layout(T, I, O, block, rank).pub.total;
}

hlq_status hlq_workspace_layout_query(int64_t T, int64_t I, int64_t O, int block,
                                      int rank, hlq_workspace_layout* out) {
  if (!out) return HLQ_ERR_NULL;
  hlq_status st = check_shape(T, I, O, block, rank);
  if (st != HLQ_OK) return st;
  *out = make_layout(T, I, O, block, rank).pub;
  return HLQ_OK;
}

// Argument checks shared by the backward's entry points (everything but the
// workspace).
static hlq_status check_backward(const void* g_y, int gy_dtype, const uint8_t* x_codes,
                                 const float* x_scales, const void* w, int w_dtype, int64_t T,
                                 int64_t I, int64_t O, int block, int rank, int gx_mode,
                                 int gw_mode, int reduction, const float* g_x, const float* g_w) {
  if (!g_y || !x_codes || !x_scales || !w || !g_x || !g_w) return HLQ_ERR_NULL;
  if ((gy_dtype != HLQ_F32 && gy_dtype != HLQ_BF16) ||
      (w_dtype != HLQ_F32 && w_dtype != HLQ_BF16))
    return HLQ_ERR_DTYPE;
  hlq_status st = check_shape(T, I, O, block, rank);
  if (st != HLQ_OK) return st;
  if ((gx_mode != HLQ_PER_TOKEN && gx_mode != HLQ_PER_TENSOR) ||
      (gw_mode != HLQ_PER_TOKEN && gw_mode != HLQ_PER_TENSOR) ||
      (reduction != HLQ_SUM && reduction != HLQ_MEAN))
    return HLQ_ERR_MODE;
  if (!aligned16(g_y) || !aligned16(x_codes) || !aligned16(x_scales) || !aligned16(w) ||
      !aligned16(g_x) || !aligned16(g_w))
    return HLQ_ERR_ALIGN;
  return HLQ_OK;
}

// The launch sequence of a validated call.
static hlq_status run_backward(const Layout& L, const void* g_y, int gy_dtype,
                               const uint8_t* x_codes, const float* x_scales, const void* w,
                               int w_dtype, int64_t T, int64_t I, int64_t O, int block,
                               int rank, int gx_mode, int gw_mode, int reduction, float* g_x,
                               float* g_w, uint8_t* ws, uint32_t step_mask, hipStream_t s) {
  const bool gx_tok = gx_mode == HLQ_PER_TOKEN;
  const bool gw_tok = gw_mode == HLQ_PER_TOKEN;
  const hlq::TrArgs a = make_tr_args(L, g_y, gy_dtype, x_codes, x_scales, w, w_dtype, T, I, O,
                                     block, gx_tok, gw_tok, ws);
  int32_t* partial = reinterpret_cast<int32_t*>(ws + L.partial);
  auto on = [&](int step) { return (step_mask >> step) & 1u; };

  if (on(HLQ_STEP_TR_MAX)) HLQ_TRY(hlq::launch_tr(a, hlq::PASS_MAX, block, rank, s));
  if (on(HLQ_STEP_TR_REDUCE)) HLQ_TRY(hlq::launch_tr_reduce(a, s));
  if (on(HLQ_STEP_TR_QUANT)) HLQ_TRY(hlq::launch_tr(a, hlq::PASS_QUANT, block, rank, s));
  const float inv_n = 1.0f / (float)block;
  const float gw_alpha =
      reduction == HLQ_MEAN ? (float)(1.0 / ((double)block * (double)T)) : inv_n;
  if (on(HLQ_STEP_GEMM_GX) && on(HLQ_STEP_GEMM_GW)) {  // both GEMMs, one launch
    // the QUANT pass (this call's or, for a GEMM-only step call, the one that
    // wrote the codes) cleared the g_w split counters; every launch leaves them zero
    HLQ_TRY(hlq::launch_gemm_pair(a.q_gy, a.q_w, T, I, a.kxb, L.plan_gx, a.s_gy, a.s_w,
                                  gx_tok ? 1 : 0, inv_n, g_x, a.q_gyl, a.q_xl, O, a.kwb,
                                  L.plan_gw, a.s_gyl, a.s_xl, gw_tok ? 1 : 0, gw_alpha, g_w,
                                  L.pair, reinterpret_cast<int32_t*>(ws + L.pair_part),
                                  a.pair_ctr, false, s));
    return HLQ_OK;
  }
  if (on(HLQ_STEP_GEMM_GX))  // g_x = acc * s_gy[t] * s_w[i] / n
    HLQ_TRY(hlq::launch_gemm(true, a.q_gy, a.q_w, T, I, a.kxb, L.plan_gx, a.s_gy,
                             gx_tok ? 1 : 0, a.s_w, gx_tok ? 1 : 0, inv_n, hlq::EPI_F32,
                             g_x, nullptr, partial, s));
  if (on(HLQ_STEP_GEMM_GW))  // g_w = acc * s_gyl[o] * s_xl[i] / n  (/ T)
    HLQ_TRY(hlq::launch_gemm(false, a.q_gyl, a.q_xl, O, I, a.kwb, L.plan_gw, a.s_gyl,
                             gw_tok ? 1 : 0, a.s_xl, gw_tok ? 1 : 0, gw_alpha, hlq::EPI_F32,
                             g_w, nullptr, partial, s));
  return HLQ_OK;
}

hlq_status hlq_linear_backward_steps(const void* g_y, int gy_dtype,
                                     const uint8_t* x_codes, const float* x_scales,
                                     const void* w, int w_dtype, int64_t T, int64_t I,
                                     int64_t O, int block, int rank, int gx_mode,
                                     int gw_mode, int reduction, float* g_x, float* g_w,
                                     void* workspace, size_t workspace_bytes,
                                     uint32_t step_mask, void* stream) {
  hlq_status st = check_backward(g_y, gy_dtype, x_codes, x_scales, w, w_dtype, T, I, O, block,
                                 rank, gx_mode, gw_mode, reduction, g_x, g_w);
  if (st != HLQ_OK) return st;
  const Layout L = make_layout(T, I, O, block, rank);
  if (!workspace || workspace_bytes < L.pub.total) return HLQ_ERR_WORKSPACE;
  if (!aligned16(workspace)) return HLQ_ERR_ALIGN;
  return run_backward(L, g_y, gy_dtype, x_codes, x_scales, w, w_dtype, T, I, O, block, rank,
                      gx_mode, gw_mode, reduction, g_x, g_w, static_cast<uint8_t*>(workspace),
                      step_mask, static_cast<hipStream_t>(stream));
}

hlq_status hlq_linear_backward(const void* g_y, int gy_dtype, const uint8_t* x_codes,
                               const float* x_scales, const void* w, int w_dtype,
                               int64_t T, int64_t I, int64_t O, int block, int rank,
                               int gx_mode, int gw_mode, int reduction, float* g_x,
                               float* g_w, void* workspace, size_t workspace_bytes,
                               void* stream) {
  return hlq_linear_backward_steps(g_y, gy_dtype, x_codes, x_scales, w, w_dtype, T, I, O,
                                   block, rank, gx_mode, gw_mode, reduction, g_x, g_w,
                                   workspace, workspace_bytes, HLQ_STEPS_ALL, stream);
}

hlq_status hlq_linear_backward_noalloc(const void* g_y, int gy_dtype, const uint8_t* x_codes,
                                       const float* x_scales, const void* w, int w_dtype,
                                       int64_t T, int64_t I, int64_t O, int block, int rank,
                                       int gx_mode, int gw_mode, int reduction, float* g_x,
                                       float* g_w, void* stream) {
  hlq_status st = check_backward(g_y, gy_dtype, x_codes, x_scales, w, w_dtype, T, I, O, block,
                                 rank, gx_mode, gw_mode, reduction, g_x, g_w);
  if (st != HLQ_OK) return st;
  // All five steps run, the GEMMs as the one paired launch, which uses no
  // split-K partials: the intermediates end where the partial region begins.
  const Layout L = make_layout(T, I, O, block, rank);
  if (L.partial > (size_t)HLQ_NOALLOC_SCRATCH_BYTES) return HLQ_ERR_WORKSPACE;
  uint8_t* scratch = static_cast<uint8_t*>(hlq::noalloc_scratch());
  if (!scratch) return HLQ_ERR_HIP;
  return run_backward(L, g_y, gy_dtype, x_codes, x_scales, w, w_dtype, T, I, O, block, rank,
                      gx_mode, gw_mode, reduction, g_x, g_w, scratch, HLQ_STEPS_ALL,
                      static_cast<hipStream_t>(stream));
}

// Shared checks of the accumulator exports: the workspace holds the layout of
// hlq_linear_backward for this shape.
static hlq_status acc_checks(const void* workspace, size_t workspace_bytes, int64_t T,
                             int64_t I, int64_t O, int block, int rank, Layout* L) {
  if (!workspace) return HLQ_ERR_NULL;
  hlq_status st = check_shape(T, I, O, block, rank);
  if (st != HLQ_OK) return st;
  *L = make_layout(T, I, O, block, rank);
  if (workspace_bytes < L->pub.total) return HLQ_ERR_WORKSPACE;
  if (!aligned16(workspace)) return HLQ_ERR_ALIGN;
  return HLQ_OK;
}

hlq_status hlq_gemm_gx_acc(const void* workspace, size_t workspace_bytes, int64_t T,
                           int64_t I, int64_t O, int block, int rank, int32_t* acc_x,
                           void* stream) {
  if (!acc_x) return HLQ_ERR_NULL;
  Layout L;
  hlq_status st = acc_checks(workspace, workspace_bytes, T, I, O, block, rank, &L);
  if (st != HLQ_OK) return st;
  if (!aligned16(acc_x)) return HLQ_ERR_ALIGN;
  const uint8_t* ws = static_cast<const uint8_t*>(workspace);
  HLQ_TRY(hlq::launch_gemm(true, ws + L.pub.q_gy, ws + L.pub.q_w, T, I, L.pub.kx_pitch,
                           L.plan_gx, nullptr, 0, nullptr, 0, 1.f, hlq::EPI_I32, nullptr,
                           acc_x, nullptr, static_cast<hipStream_t>(stream)));
  return HLQ_OK;
}

hlq_status hlq_gemm_gw_acc(const void* workspace, size_t workspace_bytes, int64_t T,
                           int64_t I, int64_t O, int block, int rank, int32_t* acc_w,
                           void* stream) {
  if (!acc_w) return HLQ_ERR_NULL;
  Layout L;
  hlq_status st = acc_checks(workspace, workspace_bytes, T, I, O, block, rank, &L);
  if (st != HLQ_OK) return st;
  if (!aligned16(acc_w)) return HLQ_ERR_ALIGN;
  const uint8_t* ws = static_cast<const uint8_t*>(workspace);
  HLQ_TRY(hlq::launch_gemm(false, ws + L.pub.q_gyl, ws + L.pub.q_xl, O, I, L.pub.kw_pitch,
                           L.plan_gw, nullptr, 0, nullptr, 0, 1.f, hlq::EPI_I32, nullptr,
                           acc_w, nullptr, static_cast<hipStream_t>(stream)));
  return HLQ_OK;
}

hlq_status hlq_gemm_pair_acc(void* workspace, size_t workspace_bytes, int64_t T, int64_t I,
                             int64_t O, int block, int rank, int32_t* acc_x, int32_t* acc_w,
                             void* stream) {
  if (!acc_x || !acc_w) return HLQ_ERR_NULL;
  Layout L;
  hlq_status st = acc_checks(workspace, workspace_bytes, T, I, O, block, rank, &L);
  if (st != HLQ_OK) return st;
  if (!aligned16(acc_x) || !aligned16(acc_w)) return HLQ_ERR_ALIGN;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  HLQ_TRY(hlq::launch_gemm_pair(ws + L.pub.q_gy, ws + L.pub.q_w, T, I, L.pub.kx_pitch,
                                L.plan_gx, nullptr, nullptr, 0, 1.f, nullptr, ws + L.pub.q_gyl,
                                ws + L.pub.q_xl, O, L.pub.kw_pitch, L.plan_gw, nullptr, nullptr,
                                0, 1.f, nullptr, L.pair,
                                reinterpret_cast<int32_t*>(ws + L.pair_part),
                                reinterpret_cast<unsigned*>(ws + L.pair_ctr), true,
                                static_cast<hipStream_t>(stream), hlq::EPI_I32, acc_x, acc_w));
  return HLQ_OK;
}

// ---------------------------------------------------------------- convolution

namespace {

struct ConvShape {
  int64_t N, H, W, C, O, R, S, P, Q, T, I;
  int stride, pad;
};

hlq_status check_conv(int64_t N, int64_t H, int64_t W, int64_t C, int64_t O, int R, int S,
                      int stride, int pad, int block, int rank, ConvShape* cs) {
  if (N <= 0 || H <= 0 || W <= 0 || C <= 0 || O <= 0 || R <= 0 || S <= 0 || stride <= 0 ||
      pad < 0)
    return HLQ_ERR_SHAPE;
  if (H + 2 * pad < R || W + 2 * pad < S) return HLQ_ERR_SHAPE;
  ConvShape c;
  c.N = N; c.H = H; c.W = W; c.C = C; c.O = O; c.R = R; c.S = S;
  c.stride = stride; c.pad = pad;
  c.P = (H + 2 * pad - R) / stride + 1;
  c.Q = (W + 2 * pad - S) / stride + 1;
  c.T = N * c.P * c.Q;
  c.I = (int64_t)R * S * C;
  if (C % 8) return HLQ_ERR_SHAPE;
  // the kernels index pixels, output positions and channels in 32 bits
  const int64_t lim = (int64_t)1 << 31;
  if (N * H * W >= lim || c.T >= lim || c.I >= lim) return HLQ_ERR_OVERFLOW;
  hlq_status st = check_shape(c.T, c.I, O, block, rank);
  if (st != HLQ_OK) return st;
  // the input gradient's INT32 sums run over every (tap, O) pair
  if (O * R * S > kMaxO) return HLQ_ERR_OVERFLOW;
  *cs = c;
  return HLQ_OK;
}

// Workspace of the convolution backward: the linear backward's for
// (T = N*P*Q, I = R*S*C, O), then the zero row of the input-gradient GEMM.
struct ConvLayout {
  Layout L;
  size_t zero, total;
};

ConvLayout make_conv_layout(const ConvShape& c, int block, int rank) {
  ConvLayout cl;
  cl.L = make_layout(c.T, c.I, c.O, block, rank);
  cl.zero = cl.L.pub.total;
  cl.total = align256(cl.zero + (size_t)cl.L.pub.kx_pitch);
  return cl;
}

hlq::ConvGemm conv_gemm(const ConvShape& c, const ConvLayout& cl, const uint8_t* ws) {
  hlq::ConvGemm g;
  memset(&g, 0, sizeof(g));
  g.q_gy = ws + cl.L.pub.q_gy;
  g.q_w = ws + cl.L.pub.q_w;
  g.zero = ws + cl.zero;
  g.kx_pitch = cl.L.pub.kx_pitch;
  g.N = c.N; g.H = c.H; g.W = c.W; g.C = c.C; g.P = c.P; g.Q = c.Q; g.S = c.S;
  g.taps = c.R * c.S;
  g.stride = c.stride; g.pad = c.pad;
  return g;
}

}  // namespace

size_t hlq_conv_backward_workspace_size(int64_t N, int64_t H, int64_t W, int64_t C, int64_t O,
                                        int R, int S, int stride, int pad, int block,
                                        int rank) {
  ConvShape c;
  if (check_conv(N, H, W, C, O, R, S, stride, pad, block, rank, &c) != HLQ_OK) return 0;
  return make_conv_layout(c, block, rank).total;
}

hlq_status hlq_conv_backward(const void* g_y, int gy_dtype, const uint8_t* x_codes,
                             const float* x_scales, const void* w, int w_dtype, int64_t N,
                             int64_t H, int64_t W, int64_t C, int64_t O, int R, int S,
                             int stride, int pad, int block, int rank, int gx_mode,
                             int gw_mode, int reduction, float* g_x, float* g_w,
                             void* workspace, size_t workspace_bytes, void* stream) {
  if (!g_y || !x_codes || !x_scales || !w || !g_x || !g_w) return HLQ_ERR_NULL;
  if ((gy_dtype != HLQ_F32 && gy_dtype != HLQ_BF16) ||
      (w_dtype != HLQ_F32 && w_dtype != HLQ_BF16))
    return HLQ_ERR_DTYPE;
  ConvShape c;
  hlq_status st = check_conv(N, H, W, C, O, R, S, stride, pad, block, rank, &c);
  if (st != HLQ_OK) return st;
  // g_x: per-tensor scales only (per-token scales of H.g_y and H.w would not
  // factor out of the sum over the taps)
  if (gx_mode != HLQ_PER_TENSOR || (gw_mode != HLQ_PER_TOKEN && gw_mode != HLQ_PER_TENSOR) ||
      (reduction != HLQ_SUM && reduction != HLQ_MEAN))
    return HLQ_ERR_MODE;
  const ConvLayout cl = make_conv_layout(c, block, rank);
  if (!workspace || workspace_bytes < cl.total) return HLQ_ERR_WORKSPACE;
  if (!aligned16(g_y) || !aligned16(x_codes) || !aligned16(x_scales) || !aligned16(w) ||
      !aligned16(g_x) || !aligned16(g_w) || !aligned16(workspace))
    return HLQ_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  const bool gw_tok = gw_mode == HLQ_PER_TOKEN;
  hlq::TrArgs a = make_tr_args(cl.L, g_y, gy_dtype, x_codes, x_scales, w, w_dtype, c.T, c.I,
                               c.O, block, false, gw_tok, ws);
  a.conv = 1;
  a.Hc = c.H; a.Wc = c.W; a.Cc = c.C; a.P = c.P; a.Q = c.Q; a.S = c.S;
  a.cstride = c.stride; a.cpad = c.pad;
  a.zero_row = ws + cl.zero;
  HLQ_TRY(hlq::launch_tr(a, hlq::PASS_MAX, block, rank, s));
  HLQ_TRY(hlq::launch_tr_reduce(a, s));
  HLQ_TRY(hlq::launch_tr(a, hlq::PASS_QUANT, block, rank, s));
  const float gw_alpha =
      reduction == HLQ_MEAN ? (float)(1.0 / ((double)block * (double)c.T)) : 1.0f / (float)block;
  HLQ_TRY(hlq::launch_gemm(false, a.q_gyl, a.q_xl, c.O, c.I, a.kwb, cl.L.plan_gw, a.s_gyl,
                           gw_tok ? 1 : 0, a.s_xl, gw_tok ? 1 : 0, gw_alpha, hlq::EPI_F32, g_w,
                           nullptr, reinterpret_cast<int32_t*>(ws + cl.L.partial), s));
  hlq::ConvGemm g = conv_gemm(c, cl, ws);
  g.s_gy = a.s_gy;
  g.s_w = a.s_w;
  g.alpha = 1.0f / (float)block;
  g.epi = hlq::EPI_F32;
  g.g_x = g_x;
  HLQ_TRY(hlq::launch_dgrad(g, s));
  return HLQ_OK;
}

hlq_status hlq_conv_gemm_acc(const void* workspace, size_t workspace_bytes, int64_t N,
                             int64_t H, int64_t W, int64_t C, int64_t O, int R, int S,
                             int stride, int pad, int block, int rank, int32_t* acc_x,
                             int32_t* acc_w, void* stream) {
  if (!workspace || !acc_x || !acc_w) return HLQ_ERR_NULL;
  ConvShape c;
  hlq_status st = check_conv(N, H, W, C, O, R, S, stride, pad, block, rank, &c);
  if (st != HLQ_OK) return st;
  const ConvLayout cl = make_conv_layout(c, block, rank);
  if (workspace_bytes < cl.total) return HLQ_ERR_WORKSPACE;
  if (!aligned16(workspace) || !aligned16(acc_x) || !aligned16(acc_w)) return HLQ_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint8_t* ws = static_cast<const uint8_t*>(workspace);
  HLQ_TRY(hlq::launch_gemm(false, ws + cl.L.pub.q_gyl, ws + cl.L.pub.q_xl, c.O, c.I,
                           cl.L.pub.kw_pitch, cl.L.plan_gw, nullptr, 0, nullptr, 0, 1.f,
                           hlq::EPI_I32, nullptr, acc_w, nullptr, s));
  hlq::ConvGemm g = conv_gemm(c, cl, ws);
  g.epi = hlq::EPI_I32;
  g.acc_x = acc_x;
  HLQ_TRY(hlq::launch_dgrad(g, s));
  return HLQ_OK;
}

// ---------------------------------------------------------------- ablation variants

namespace {

// One path's operands and GEMM under a variant (HLQ_VAR_*).  K = the
// contracted dimension, Ma / Nb = the two output dimensions.
struct AblPath {
  int variant;
  int64_t K, Ma, Nb;       // source sizes
  int64_t MoA, Ko, Kpad;   // operand A rows (Ma or its low rank), K' (K or low rank)
  float alpha;             // Hadamard along K: 1/n
  size_t qA, qB, sA, sB, mA, mB, G, part, end;
  hlq::GemmPlan plan;
};

bool var_ok(int v) { return v >= HLQ_VAR_HQ4 && v <= HLQ_VAR_HLA8_EXT; }

AblPath abl_path(int variant, int64_t K, int64_t Ma, int64_t Nb, int n, int r, size_t off) {
  AblPath p;
  memset(&p, 0, sizeof(p));
  p.variant = variant; p.K = K; p.Ma = Ma; p.Nb = Nb;
  p.MoA = variant == HLQ_VAR_HLA8_EXT ? Ma / n * r : Ma;
  p.Ko = variant == HLQ_VAR_HLA8_INT ? K / n * r : K;
  p.Kpad = (p.Ko + 127) / 128 * 128;
  p.alpha = (variant == HLQ_VAR_HQ4 || variant == HLQ_VAR_HLA8_INT) ? 1.0f / (float)n : 1.0f;
  p.plan = hlq::plan_gemm(false, p.MoA, Nb, p.Kpad);
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align256(off + bytes);
    return at;
  };
  p.qA = take((size_t)p.MoA * p.Kpad);
  p.qB = take((size_t)Nb * p.Kpad);
  p.sA = take((size_t)p.MoA * 4);
  p.sB = take((size_t)Nb * 4);
  p.mA = take((size_t)p.MoA * 4);
  p.mB = take((size_t)Nb * 4);
  p.G = take(variant == HLQ_VAR_HLA8_EXT ? (size_t)p.MoA * Nb * 4 : 0);
  p.part = take(p.plan.splits > 1 ? (size_t)p.plan.splits * p.MoA * Nb * 4 : 0);
  p.end = off;
  return p;
}

// Operand A (left, rows MoA) or B of one path.  src_a_rows: the source holds
// the K axis along its columns (g_y for the g_x path) rather than its rows.
hlq::AblOperand abl_operand(const AblPath& p, bool left, const void* src, int dt,
                            const uint8_t* codes, const float* cscales, int64_t rows,
                            int64_t cols, bool m_is_row, int n, int r, bool per_token,
                            uint8_t* ws) {
  hlq::AblOperand o;
  memset(&o, 0, sizeof(o));
  o.src = src; o.dt = dt; o.codes = codes; o.cscales = cscales;
  o.rows = rows; o.cols = cols; o.m_is_row = m_is_row ? 1 : 0;
  o.r = r;
  o.qmax = (p.variant == HLQ_VAR_HQ4 || p.variant == HLQ_VAR_Q4) ? 7 : 127;
  o.per_token = per_token ? 1 : 0;
  const int64_t M = left ? p.Ma : p.Nb;
  if (p.variant == HLQ_VAR_HLA8_EXT) {
    o.along_m = left ? 1 : 0;
    o.kind = left ? 2 : 0;
  } else {
    o.along_m = 0;
    o.kind = p.variant == HLQ_VAR_Q4 ? 0 : p.variant == HLQ_VAR_HQ4 ? 1 : 2;
  }
  o.lines = o.along_m ? p.K : M;
  o.blocks = (o.along_m ? M : p.K) / n;
  o.Mo = left ? p.MoA : p.Nb;
  o.Ko = p.Ko;
  o.Kpad = p.Kpad;
  o.q = reinterpret_cast<int8_t*>(ws + (left ? p.qA : p.qB));
  o.s = reinterpret_cast<float*>(ws + (left ? p.sA : p.sB));
  o.maxbits = reinterpret_cast<unsigned*>(ws + (left ? p.mA : p.mB));
  return o;
}

struct AblLayout {
  AblPath x, w;
  size_t total;
};

AblLayout abl_layout(int64_t T, int64_t I, int64_t O, int n, int r, int gxv, int gwv) {
  AblLayout L;
  L.x = abl_path(gxv, O, T, I, n, r, 0);
  L.w = abl_path(gwv, T, O, I, n, r, L.x.end);
  L.total = L.w.end;
  return L;
}

// GEMM of one path; fp32 result (or the external variant's expansion), and
// the INT32 sums when acc is given.
hlq_status abl_gemm(const AblPath& p, uint8_t* ws, bool tok, float out_alpha, float* out,
                    int32_t* acc, int n, int r, hipStream_t s) {
  const uint8_t* A = ws + p.qA;
  const uint8_t* B = ws + p.qB;
  const float* sa = reinterpret_cast<const float*>(ws + p.sA);
  const float* sb = reinterpret_cast<const float*>(ws + p.sB);
  int32_t* part = reinterpret_cast<int32_t*>(ws + p.part);
  const bool ext = p.variant == HLQ_VAR_HLA8_EXT;
  float* C = ext ? reinterpret_cast<float*>(ws + p.G) : out;
  const float alpha = ext ? 1.0f : p.alpha * out_alpha;
  HLQ_TRY(hlq::launch_gemm(false, A, B, p.MoA, p.Nb, p.Kpad, p.plan, sa, tok ? 1 : 0, sb,
                           tok ? 1 : 0, alpha, hlq::EPI_F32, C, nullptr, part, s));
  if (ext)
    HLQ_TRY(hlq::launch_abl_expand(C, p.Ma, p.Nb, n, r, out_alpha / (float)n, out, s));
  if (acc)
    HLQ_TRY(hlq::launch_gemm(false, A, B, p.MoA, p.Nb, p.Kpad, p.plan, nullptr, 0, nullptr, 0,
                             1.f, hlq::EPI_I32, nullptr, acc, nullptr, s));
  return HLQ_OK;
}

}  // namespace

size_t hlq_ablation_workspace_size(int64_t T, int64_t I, int64_t O, int block, int rank,
                                   int gx_variant, int gw_variant) {
  if (check_shape(T, I, O, block, rank) != HLQ_OK || !var_ok(gx_variant) || !var_ok(gw_variant))
    return 0;
  return abl_layout(T, I, O, block, rank, gx_variant, gw_variant).total;
}

hlq_status hlq_linear_backward_ablation(const void* g_y, int gy_dtype, const uint8_t* x_codes,
                                        const float* x_scales, const void* w, int w_dtype,
                                        int64_t T, int64_t I, int64_t O, int block, int rank,
                                        int gx_variant, int gw_variant, int gx_mode,
                                        int gw_mode, int reduction, float* g_x, float* g_w,
                                        int32_t* acc_x, int32_t* acc_w, void* workspace,
                                        size_t workspace_bytes, void* stream) {
  hlq_status st = check_backward(g_y, gy_dtype, x_codes, x_scales, w, w_dtype, T, I, O, block,
                                 rank, gx_mode, gw_mode, reduction, g_x, g_w);
  if (st != HLQ_OK) return st;
  if (!var_ok(gx_variant) || !var_ok(gw_variant)) return HLQ_ERR_MODE;
  const AblLayout L = abl_layout(T, I, O, block, rank, gx_variant, gw_variant);
  if (!workspace || workspace_bytes < L.total) return HLQ_ERR_WORKSPACE;
  if (!aligned16(workspace) || (acc_x && !aligned16(acc_x)) || (acc_w && !aligned16(acc_w)))
    return HLQ_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  const bool gx_tok = gx_mode == HLQ_PER_TOKEN, gw_tok = gw_mode == HLQ_PER_TOKEN;
  // g_x = g_y . w over O: A from g_y [T][O] (m = row t), B from w [O][I] (m = column i)
  HLQ_TRY(hlq::launch_abl_operand(abl_operand(L.x, true, g_y, gy_dtype, nullptr, nullptr, T, O,
                                              true, block, rank, gx_tok, ws), block, s));
  HLQ_TRY(hlq::launch_abl_operand(abl_operand(L.x, false, w, w_dtype, nullptr, nullptr, O, I,
                                              false, block, rank, gx_tok, ws), block, s));
  st = abl_gemm(L.x, ws, gx_tok, 1.0f, g_x, acc_x, block, rank, s);
  if (st != HLQ_OK) return st;
  // g_w = g_y^T . x over T: A from g_y [T][O] (m = column o), B from the
  // ACBP codes of x [T][I] (m = column i)
  HLQ_TRY(hlq::launch_abl_operand(abl_operand(L.w, true, g_y, gy_dtype, nullptr, nullptr, T, O,
                                              false, block, rank, gw_tok, ws), block, s));
  HLQ_TRY(hlq::launch_abl_operand(abl_operand(L.w, false, nullptr, 2, x_codes, x_scales, T, I,
                                              false, block, rank, gw_tok, ws), block, s));
  const float mean = reduction == HLQ_MEAN ? (float)(1.0 / (double)T) : 1.0f;
  return abl_gemm(L.w, ws, gw_tok, mean, g_w, acc_w, block, rank, s);
}

size_t hlq_lqs_workspace_size(int64_t T, int64_t I, int64_t O, int block, int rank) {
  if (check_shape(T, I, O, block, rank) != HLQ_OK) return 0;
  return make_lqs_layout(T, I, O, block, rank).total;
}

hlq_status hlq_lqs_accumulate(const void* g_y, int gy_dtype, const uint8_t* x_codes,
                              const float* x_scales, const void* w, int w_dtype, int64_t T,
                              int64_t I, int64_t O, int block, int rank, double* stats,
                              void* workspace, size_t workspace_bytes, void* stream) {
  if (!g_y || !x_codes || !x_scales || !w || !stats) return HLQ_ERR_NULL;
  if ((gy_dtype != HLQ_F32 && gy_dtype != HLQ_BF16) ||
      (w_dtype != HLQ_F32 && w_dtype != HLQ_BF16))
    return HLQ_ERR_DTYPE;
  hlq_status st = check_shape(T, I, O, block, rank);
  if (st != HLQ_OK) return st;
  // the statistics kernels address every input with 32-bit byte offsets
  const int64_t lim = (int64_t)1 << 32;
  const int64_t gy_b = T * O * (gy_dtype == HLQ_F32 ? 4 : 2);
  const int64_t w_b = O * I * (w_dtype == HLQ_F32 ? 4 : 2);
  if (gy_b >= lim || w_b >= lim || T * I / 2 >= lim || T * 4 >= lim) return HLQ_ERR_OVERFLOW;
  const LqsLayout L = make_lqs_layout(T, I, O, block, rank);
  if (!workspace || workspace_bytes < L.total) return HLQ_ERR_WORKSPACE;
  if (!aligned16(g_y) || !aligned16(x_codes) || !aligned16(x_scales) || !aligned16(w) ||
      !aligned16(stats) || !aligned16(workspace))
    return HLQ_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  // group maxima, per-token scales and tensor maxima: the backward's MAX and
  // reduce launches with both paths per token
  const Layout B = make_layout(T, I, O, block, rank);
  hlq::TrArgs t = make_tr_args(B, g_y, gy_dtype, x_codes, x_scales, w, w_dtype, T, I, O,
                               block, true, true, ws);
  t.tok_tmax = 1;  // the statistics compare against the tensor maxima too
  HLQ_TRY(hlq::launch_tr(t, hlq::PASS_MAX, block, rank, s));
  HLQ_TRY(hlq::launch_tr_reduce(t, s));
  hlq::LqsArgs a;
  memset(&a, 0, sizeof(a));
  a.gy = g_y; a.gy_dt = gy_dtype;
  a.xc = x_codes; a.xs = x_scales;
  a.w = w; a.w_dt = w_dtype;
  a.T = T; a.I = I; a.O = O; a.r = rank;
  a.tok_inv[0] = t.inv_gy; a.tok_s[0] = t.s_gy;
  a.tok_inv[1] = t.inv_w; a.tok_s[1] = t.s_w;
  a.tok_inv[2] = t.inv_gyl; a.tok_s[2] = t.s_gyl;
  a.tok_inv[3] = t.inv_xl; a.tok_s[3] = t.s_xl;
  a.tmax = t.tmax;
  a.part = reinterpret_cast<double*>(ws + L.part);
  a.stats = stats;
  for (int k = 0; k < 4; ++k) {
    a.items[k] = L.items[k];
    a.count[k] = L.count[k];
  }
  for (int k = 0; k < 5; ++k) a.wg0[k] = L.wg0[k];
  HLQ_TRY(hlq::launch_lqs(a, block, s));
  return HLQ_OK;
}

hlq_status hlq_lqs_select(const double* stats, double threshold, int* gx_mode,
                          int* gw_mode) {
  if (!stats || !gx_mode || !gw_mode) return HLQ_ERR_NULL;
  if (!(threshold >= 0.0)) return HLQ_ERR_MODE;
  // relative error of operand k in mode column c (1 per-token, 2 per-tensor)
  auto rel = [&](int k, int c) {
    const double ss = stats[4 * k];
    return ss == 0.0 ? 0.0 : stats[4 * k + c] / ss;
  };
  const double gx_tok = rel(0, 1) + rel(1, 1), gx_ten = rel(0, 2) + rel(1, 2);
  const double gw_tok = rel(2, 1) + rel(3, 1), gw_ten = rel(2, 2) + rel(3, 2);
  *gx_mode = gx_ten > (1.0 + threshold) * gx_tok ? HLQ_PER_TOKEN : HLQ_PER_TENSOR;
  *gw_mode = gw_ten > (1.0 + threshold) * gw_tok ? HLQ_PER_TOKEN : HLQ_PER_TENSOR;
  return HLQ_OK;
}

}  // extern "C"
