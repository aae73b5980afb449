// gfx950 (CDNA4) kernels of the HLQ/HOT linear-layer backward: integer GEMMs.
//
// Method: "HLQ: Fast and Efficient Backpropagation via Hadamard Low-rank
// Quantization" (TL;DR: g_x = g_y.w with 4-bit Hadamard quantization, g_w with
// low-rank int8 processing, int4 activation compression) and "HOT:
// Hadamard-based Optimized Training" (scime.ai summary, "Approach": INT4
// Hadamard quantization for gx, Hadamard low-rank approximation plus INT8 for
// gw, per-token or per-tensor scales chosen per layer).
//
// Numerics every kernel keeps (so codes are unique and reproducible):
//  * Walsh-Hadamard butterflies in fp32, ascending stage distance
//    h = 1, 2, 4, ...; pair (k, k+h) -> (a + b, a - b).  Built with
//    -ffp-contract=off so nothing is fused into an FMA.
//  * Quantizer: a = max|v| (exact), inv = qmax / a (IEEE division),
//    q = clamp(rne(v * inv), -qmax, qmax), s = a / qmax; a == 0 -> q = 0, s = 0.
//  * Cross-block maxima use atomicMax on the fp32 bit pattern of non-negative
//    values, which orders like the values and commutes, so results do not
//    depend on scheduling.
#include <hip/hip_runtime.h>
#include <algorithm>
#include <cmath>
#include <stdint.h>

#include <type_traits>

#include "hlq_device.h"
#include "hlq_internal.h"

namespace hlq {

// ------------------------------------------------------------ integer GEMM
// C[m][n] = sum_k A[m][k] * B[n][k]; the K run of every row is pitch bytes,
// zero-padded to a multiple of the stage depth KB, and the integer operands
// are stored in K planes (hlq_device.h: plane p = bytes [p U, (p + 1) U) of
// every row, rows consecutive; U = 96 for FP6, 64 for INT8), so one stage of
// a tile is one contiguous block per operand.  The bf16 operands of the
// forward are plain row-major [M][pitch] / [N][pitch].
//
// Matrix cores: INT8 operands (the g_w product) on v_mfma_i32_32x32x32_i8
// (32 cycles of the matrix pipe for a 32x32x32 product; the 16x16x64 form
// needs more independent accumulators than a wave has to stay busy); lane l
// feeds row l%32 with 16 consecutive K bytes of half l/32.  The INT4 codes of
// the g_x product arrive as FP6 E2M3 fields (exact for [-7, 7]; see
// hlq_device.h) and run on v_mfma_scale_f32_32x32x64_f8f6f4 (unit scales):
// twice the K of the INT8 instruction in the same 32 cycles, no unpacking,
// and fp32 sums that are exact integers below 2^24.  Lane l feeds row l%32
// with the 32 K values 32*(l/32) .. of the K step (6 dwords); a 96-byte
// stage row (128 K values, two K steps) holds those of half h at bytes
// 48 h .. 48 h + 47, read as three 16-byte chunks whose first and last six
// dwords are the operands of the two steps.
// Operand X holds 32 rows of A, operand Y 32 rows of B.
// Lane l then holds D[8*(r/4) + 4*(l/32) + r%4][l%32] in accumulator r: one
// column n of C per lane, so a store of register r writes 128 contiguous
// bytes of a C row per half-wave.
//
// Pipeline (256 threads, 2x2 waves, wave tile (BM/2) x (BN/2)):
//   * K advances in stages of KB bytes held in an NS-deep LDS ring.  Stages
//     are fetched with LDS DMA (global_load_lds_dwordx4: lane i of a wave
//     instruction fills bytes 16i..16i+15 of a 1 KB LDS run), NS stages
//     ahead; no VGPR staging.  Each row's 16-byte chunks are XOR-swizzled
//     (chunk c of row r sits at c ^ swz(r)) so the fragment reads of 32 rows
//     at one chunk hit distinct banks.
//   * Fragments are double-buffered in registers: the reads of k-step kk+1
//     are issued between the MFMAs of step kk.
//   * One barrier per stage, after the stage's last MFMAs are issued: it
//     publishes the next stage (every wave has waited for its own DMA with
//     vmcnt) and frees the stage just read, which is refilled at once.
// Workgroups map to tiles XCD-aware: consecutive workgroup ids go to the 8
// XCDs in turn, so each XCD takes a contiguous run of tiles (n fastest) and
// its L2 serves the A rows those tiles share.  blockIdx.y selects a split of
// the K stages (partials summed by k_gemm_finalize).

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef unsigned short us2 __attribute__((ext_vector_type(2)));

// fp32 -> bf16 bits, round to nearest even (finite values)
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}


typedef unsigned int v12u __attribute__((ext_vector_type(12)));
typedef unsigned int v8u __attribute__((ext_vector_type(8)));
typedef int v8i __attribute__((ext_vector_type(8)));

// The three 16-byte chunks of a lane's FP6 stage row as one 12-dword value.
__device__ __forceinline__ v12u join12(u32x4 a, u32x4 b, u32x4 c) {
  const v8u ab = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  const v8u cc = __builtin_shufflevector(c, c, 0, 1, 2, 3, -1, -1, -1, -1);
  return __builtin_shufflevector(ab, cc, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11);
}
// Operand of K step K (0, 1): six dwords of FP6 fields (the instruction reads six).
template <int K>
__device__ __forceinline__ v8i step_op(v12u r) {
  return __builtin_bit_cast(
      v8i, __builtin_shufflevector(r, r, 6 * K, 6 * K + 1, 6 * K + 2, 6 * K + 3, 6 * K + 4,
                                   6 * K + 5, -1, -1));
}
// One 32x32x64 product of FP6 E2M3 operands, unit block scales (E8M0 127).
__device__ __forceinline__ v16f mfma_fp6(v8i a, v8i b, v16f c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 2, 2, 0, 127, 0, 127);
}

__device__ __forceinline__ bool xcd_tile(int64_t w, int64_t nt_m, int64_t nt_n, int64_t& tm,
                                         int64_t& tn) {
  const int64_t total = nt_m * nt_n;
  const int64_t per = (total + 7) / 8;
  const int64_t t = (w % 8) * per + w / 8;
  if (t >= total) return false;
  tm = t / nt_n;
  tn = t % nt_n;
  return true;
}

// s_waitcnt with vmcnt = N and the other counters left alone.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Wait for this wave's LDS reads, then a workgroup barrier.  Written with
// the builtins so the compiler knows the reads are complete and adds no wait
// of its own before their first use (an asm wait is opaque to it, and the one
// it would add also covers the next stage's reads issued after the barrier);
// the empty asm statements keep every memory access on its side.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt left alone
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// 16 bytes per lane from global memory into LDS run l (lane i -> l + 16 i).
__device__ __forceinline__ void lds_dma16(const uint8_t* g, uint8_t* l) {
  __builtin_amdgcn_global_load_lds(g, l, 16, 0, 0);
}

// Physical 16-byte chunk slot of logical chunk 0 in row r (XOR with it).
// Depends on r & 15 only, so fragment bases (multiples of 32 rows) keep it.
// The LDS serves a 16-byte read 16 lanes (16 rows) at a time from 64 banks
// (16 groups of 16 bytes).  KB 96 (six chunks per row): rows 8..15 of every
// 16 swap chunk pairs, so those 16 rows at one chunk fall in 16 distinct
// groups (rows 0..7 at 6 r cover the even groups, the swap the odd ones;
// measured 132 against 94 B/clk per CU for a swap on row bit 2).
template <int KB>
__device__ __forceinline__ int chunk_swz(int r) {
  if constexpr (KB == 128) return (r & 7) ^ ((r >> 3) & 1);
  else if constexpr (KB == 96) return (r >> 3) & 1;
  else return (r >> 2) & 3;
}

// WNW waves along N (2 x WNW waves, NT = 128 * WNW threads per workgroup).
template <bool FP6, int BM, int BN, int KB, int NS, int WNW = 2>
struct GemmShape {
  static constexpr int NT = 128 * WNW;
  static constexpr int WTM = BM / 2, WTN = BN / WNW, FM = WTM / 32, FN = WTN / 32;
  static constexpr int CPR = KB / 16;                              // chunks per row
  static constexpr int IA = BM * CPR / NT, IB = BN * CPR / NT;     // DMA ops per wave
  static constexpr int IPW = IA + IB;
  static constexpr int STAGE = (BM + BN) * KB;
  static constexpr int KK = FP6 ? KB / 48 : KB / 32;               // k-steps per stage
  static_assert(FM >= 1 && FN >= 1, "wave tile smaller than one MFMA tile");
  static_assert(IA * NT == BM * CPR && IB * NT == BN * CPR, "stage load split");
  static_assert(KK % 2 == 0, "fragment slots alternate per k-step");
  static_assert(FP6 ? KB == 96 : (KB == 64 || KB == 128), "swizzle covers 4, 6 or 8 chunks per row");
  static_assert(NS >= 2 && NS <= 4, "ring depth");
  static_assert(NS * STAGE <= 160 * 1024, "LDS ring fits the CU");
};

#define HLQ_SGB(mask, n) __builtin_amdgcn_sched_group_barrier(mask, n, 0)

// One GEMM of a launch: operands, shape, K stages (split into sps-stage
// pieces) and the dequantizing epilogue's scales.
struct GemmArgs {
  const uint8_t* A;
  const uint8_t* B;
  int64_t M, N, pitch, S_total, sps;
  const float* sa;
  int sa_step;
  const float* sb;
  int sb_step;
  float alpha;
  float* C;
  int32_t* Ci;
  // Implicit-GEMM input gradient of a convolution (gemm_tile CONV): output
  // rows m = input pixels (n, h, w) of an [N][cH][cW] image, columns the cC
  // channels; K stage st belongs to tap (st / cSO) = r * cS + s and is plane
  // st % cSO of the operands.  A (the H.g_y codes, one row per output pixel
  // of the cP x cQ grid) is read at the output pixel (n, (h + pad - r) /
  // stride, (w + pad - s) / stride) when that is a whole in-range position,
  // else at `zero` (96 zero bytes); B (the H.w codes) at row tap * cC +
  // channel.
  int32_t cH, cW, cP, cQ, cS, cC, cstride, cpad, cSO;
  int64_t cArows, cBrows;  // rows of A (output pixels) and B (taps x channels): plane heights
  const uint8_t* zero;
  // bf16 forward (gemm_tile BF16): y [M][N] as bf16 bits (EPI_BF16) and, when
  // acbp_codes is set, the ACBP codes [M][K/2] and scales [M] of A (= x),
  // emitted by the workgroups of the first column of tiles.
  uint16_t* Cb;
  uint8_t* acbp_codes;
  float* acbp_scales;
  // K split across workgroups (INT8 tiles of the pair launch): with nsplit > 1,
  // split s of tile t stores its INT32 sums to part + (t * nsplit + s) * BM * BN
  // (thread-major, device-coherent write-through), then counts itself into
  // ctr[t]; the workgroup that arrives last adds the other splits' sums (loads
  // that bypass the XCD's own L2) and alone runs the epilogue, resetting ctr[t]
  // to zero.  No workgroup waits on another.
  int32_t nsplit;
  int32_t* part;
  unsigned* ctr;
};

// One output tile (workgroup w of the tile grid, K split `split`) of one GEMM.
// Every thread of the workgroup calls it; `lds` holds NS * STAGE bytes.
//
// BF16: bf16 operands (8 per 16-byte fragment, v_mfma_f32_32x32x16_bf16, fp32
// sums), the forward product y = x . w^T; EPI_F32 stores y in fp32 (no
// scales), EPI_BF16 rounds it to bf16.  With g.acbp_codes set, every tile's
// waves of the first column keep the running maximum of |x| of the tile's A
// rows (packed 16-bit maxima of the magnitude bits of the fragments they
// feed to the MFMAs, no extra load: every tile streams the whole K of its
// rows); after the K loop each tile re-reads (from cache) an equal slice of
// its rows' columns and writes their INT4 codes, the first column of tiles
// also the scales.
template <bool FP6, int BM, int BN, int KB, int NS, int EPI, bool CONV = false,
          bool BF16 = false, int WNW = 2>
__device__ __forceinline__ void gemm_tile(const GemmArgs& g, int64_t w, int64_t split,
                                          uint8_t* lds, float* sc) {
  static_assert(!(FP6 && BF16), "one operand type");
  using G = GemmShape<FP6, BM, BN, KB, NS, WNW>;
  constexpr int NT = G::NT;
  constexpr int FM = G::FM, FN = G::FN, IA = G::IA, IB = G::IB, IPW = G::IPW;
  constexpr int CPR = G::CPR, KK = G::KK;
  const uint8_t* __restrict__ A = g.A;
  const uint8_t* __restrict__ B = g.B;
  const int64_t M = g.M, N = g.N, pitch = g.pitch, S_total = g.S_total, sps = g.sps;
  const float* __restrict__ sa = g.sa;
  const float* __restrict__ sb = g.sb;
  const int sa_step = g.sa_step, sb_step = g.sb_step;
  const float alpha = g.alpha;
  float* __restrict__ C = g.C;
  int32_t* __restrict__ Ci = g.Ci;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WNW, wn = wave % WNW;
  int64_t tm, tn;
  if (!xcd_tile(w, (M + BM - 1) / BM, (N + BN - 1) / BN, tm, tn)) return;
  const int64_t m0 = tm * BM, n0 = tn * BN;
  const int64_t s_first = split * sps;
  const int64_t S = (S_total - s_first < sps ? S_total - s_first : sps);  // >= 1 by plan
  const int64_t kbase = s_first * KB;

  // DMA sources of this lane for stage 0 (rows past M / N re-read the last row).
  // The integer operands are in K planes of U bytes (FP6: 96, one plane per
  // stage; INT8: 64, one or two per stage): chunk c of row r of a stage sits
  // in plane c * 16 / U of it at r * U + c * 16 % U, and a stage is M * KB
  // (N * KB) bytes on.  The bf16 operands of the forward are plain row-major.
  constexpr int U = FP6 ? FP6_PLANE : I8_PLANE;
  const int64_t sta = BF16 ? KB : M * KB, stb = BF16 ? KB : N * KB;
  const uint8_t* src[IPW];
  // CONV: input pixel (n, h, w) of each A slot's row, channel of each B
  // slot's row, byte offset of each slot's 16-byte chunk
  int32_t cv_n[CONV ? IA : 1], cv_h[CONV ? IA : 1], cv_w[CONV ? IA : 1];
  int32_t cv_c[CONV ? IB : 1], cv_off[CONV ? IPW : 1];
#pragma unroll
  for (int j = 0; j < IA; ++j) {
    const int slot = (wave * IA + j) * 64 + lane;
    const int row = slot / CPR, c = (slot % CPR) ^ chunk_swz<KB>(row);
    const int64_t r = m0 + row < M ? m0 + row : M - 1;
    if constexpr (CONV) {
      const int32_t hw = g.cH * g.cW, m = (int32_t)r;
      cv_n[j] = m / hw;
      cv_h[j] = (m - cv_n[j] * hw) / g.cW;
      cv_w[j] = m - cv_n[j] * hw - cv_h[j] * g.cW;
      cv_off[j] = c * 16;
      src[j] = nullptr;
    } else {
      src[j] = BF16 ? A + r * pitch + kbase + c * 16
                    : A + s_first * sta + ((c * 16 / U) * M + r) * U + c * 16 % U;
    }
  }
#pragma unroll
  for (int j = 0; j < IB; ++j) {
    const int slot = (wave * IB + j) * 64 + lane;
    const int row = slot / CPR, c = (slot % CPR) ^ chunk_swz<KB>(row);
    const int64_t r = n0 + row < N ? n0 + row : N - 1;
    if constexpr (CONV) {
      cv_c[j] = (int32_t)r;
      cv_off[IA + j] = c * 16;
      src[IA + j] = nullptr;
    } else {
      src[IA + j] = BF16 ? B + r * pitch + kbase + c * 16
                         : B + s_first * stb + ((c * 16 / U) * N + r) * U + c * 16 % U;
    }
  }
  // Issue the LDS DMA of K stage st into ring buffer bf.
  auto issue = [&](int64_t st, int bf) {
    uint8_t* base_ = lds + bf * G::STAGE;
    if constexpr (CONV) {
      const int32_t tap = (int32_t)st / g.cSO, ko = (int32_t)st - tap * g.cSO;
      const int32_t tr = tap / g.cS, ts = tap - tr * g.cS;
#pragma unroll
      for (int j = 0; j < IA; ++j) {
        int32_t p = cv_h[j] + g.cpad - tr, q = cv_w[j] + g.cpad - ts;
        bool ok = p >= 0 && q >= 0;
        if (g.cstride != 1) {
          ok = ok && p % g.cstride == 0 && q % g.cstride == 0;
          p /= g.cstride;
          q /= g.cstride;
        }
        ok = ok && p < g.cP && q < g.cQ;
        // plane ko of the output pixel's row (FP6 planes of KB bytes)
        const uint8_t* row =
            ok ? A + ((int64_t)ko * g.cArows + (int64_t)(cv_n[j] * g.cP + p) * g.cQ + q) * KB
               : g.zero;
        lds_dma16(row + cv_off[j], base_ + (wave * IA + j) * 1024);
      }
#pragma unroll
      for (int j = 0; j < IB; ++j)
        lds_dma16(B + ((int64_t)ko * g.cBrows + tap * g.cC + cv_c[j]) * KB + cv_off[IA + j],
                  base_ + BM * KB + (wave * IB + j) * 1024);
    } else {
#pragma unroll
      for (int j = 0; j < IA; ++j) lds_dma16(src[j] + st * sta, base_ + (wave * IA + j) * 1024);
#pragma unroll
      for (int j = 0; j < IB; ++j)
        lds_dma16(src[IA + j] + st * stb, base_ + BM * KB + (wave * IB + j) * 1024);
    }
  };
#define HLQ_GEMM_ISSUE(st, bf) issue((st), (bf))
  // wait until at most k stages of this wave's DMA are still in flight
#define HLQ_GEMM_WAIT(k)                                        \
  do {                                                          \
    const int64_t k_ = (k);                                     \
    if (k_ <= 0) wait_vmcnt<0>();                               \
    else if (k_ == 1) wait_vmcnt<IPW>();                        \
    else if (k_ == 2) wait_vmcnt<(2 * IPW < 63 ? 2 * IPW : 63)>(); \
    else wait_vmcnt<(3 * IPW < 63 ? 3 * IPW : 63)>();           \
  } while (0)

  const int fr = lane & 31, fh = lane >> 5;
  const int a_off = (wm * G::WTM + fr) * KB;
  const int b_off = BM * KB + (wn * G::WTN + fr) * KB;
  const int sw = chunk_swz<KB>(fr);
  int coff[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) coff[kk] = ((kk * 2 + fh) ^ sw) * 16;
  // FP6: chunks 3 fh .. 3 fh + 2 of a stage row
  int c6[3];
#pragma unroll
  for (int m = 0; m < 3; ++m) c6[m] = ((3 * fh + m) ^ sw) * 16;

  // Dequantization scales of the tile's rows (times alpha) and columns, read
  // before the K loop and parked in LDS (sc, an array of its own, so the
  // ring's DMA does not order its accesses): the epilogue then waits on no
  // global load while its stores are in flight.
  constexpr int NSC = (BM + BN + NT - 1) / NT;
  float scv[NSC];
  if constexpr (EPI == EPI_F32 && !BF16) {
#pragma unroll
    for (int q = 0; q < NSC; ++q) {
      // one unconditional load per slot (a select of the address, so the
      // loaded value is not merged across branches, which would wait on it)
      const int i = tid + NT * q;
      const int64_t m = m0 + i, n = n0 + (i - BM);
      const float* src = i < BM ? sa + (m < M ? m : M - 1) * sa_step
                                : sb + (n < N ? (n >= 0 ? n : 0) : N - 1) * sb_step;
      scv[q] = *src;
    }
  }

#pragma unroll
  for (int p = 0; p < NS; ++p)
    if (p < S) HLQ_GEMM_ISSUE(p, p);
  // keep the scales' LDS writes below the ring's first wait (no stall on
  // the scale loads before the stage loads are in flight)
  asm volatile("" ::: "memory");

  using AccT = std::conditional_t<BF16 || FP6, v16f, v16i>;
  AccT acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0;
  // ACBP row maxima (BF16 forward): packed 16-bit maxima of |x| bits
  const bool acbp = BF16 && g.acbp_codes != nullptr;
  const bool track = acbp && wn == 0;
  // (a plain array: bit casts of ext-vector elements read element 0 here)
  unsigned amax[FM][4];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int d = 0; d < 4; ++d) amax[i][d] = 0u;

  u32x4 fa[2][FM], fb[2][FN];
  HLQ_GEMM_WAIT((S - 1 < NS - 1 ? S - 1 : NS - 1));
  if constexpr (EPI == EPI_F32 && !BF16) {
#pragma unroll
    for (int q = 0; q < NSC; ++q)
      if (tid + NT * q < BM + BN) sc[tid + NT * q] = tid + NT * q < BM ? scv[q] * alpha : scv[q];
  }
  asm volatile("s_barrier" ::: "memory");
  // FP6: chunks 0 and 1 of each fragment row (K step 0 and the first half of
  // step 1), chunk 2 (the rest of step 1) loads under step 0's MFMAs
  u32x4 p0a[FM], p1a[FM], p2a[FM], p0b[FN], p1b[FN], p2b[FN];
  if constexpr (FP6) {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      p0a[i] = *reinterpret_cast<const u32x4*>(lds + a_off + i * 32 * KB + c6[0]);
      p1a[i] = *reinterpret_cast<const u32x4*>(lds + a_off + i * 32 * KB + c6[1]);
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      p0b[j] = *reinterpret_cast<const u32x4*>(lds + b_off + j * 32 * KB + c6[0]);
      p1b[j] = *reinterpret_cast<const u32x4*>(lds + b_off + j * 32 * KB + c6[1]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < FM; ++i)
      fa[0][i] = *reinterpret_cast<const u32x4*>(lds + a_off + i * 32 * KB + coff[0]);
#pragma unroll
    for (int j = 0; j < FN; ++j)
      fb[0][j] = *reinterpret_cast<const u32x4*>(lds + b_off + j * 32 * KB + coff[0]);
  }

  // One K stage.  MODE 0: steady state (refill a buffer, prefetch the next
  // stage's first fragments); 1: the last NS-1 stages but one (prefetch, no
  // refill); 2: the last stage.  Separate bodies keep each stage one block
  // of straight-line code for the scheduler.
  int buf = 0;
  auto stage = [&](int64_t st, auto mode_tag) {
    constexpr int MODE = decltype(mode_tag)::value;
    const uint8_t* base = lds + buf * G::STAGE;
    if constexpr (FP6) {
      // K step 0: chunk 2 of every fragment row loads under its MFMAs
#pragma unroll
      for (int i = 0; i < FM; ++i)
        p2a[i] = *reinterpret_cast<const u32x4*>(base + a_off + i * 32 * KB + c6[2]);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        p2b[j] = *reinterpret_cast<const u32x4*>(base + b_off + j * 32 * KB + c6[2]);
      v12u ra[FM], rb[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) ra[i] = join12(p0a[i], p1a[i], p2a[i]);
#pragma unroll
      for (int j = 0; j < FN; ++j) rb[j] = join12(p0b[j], p1b[j], p2b[j]);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = mfma_fp6(step_op<0>(ra[i]), step_op<0>(rb[j]), acc[i][j]);
      if constexpr (MODE != 2) {
        // stage st+1 landed in every wave and no wave reads stage st any
        // more: its chunks 0 and 1 load under step 1's MFMAs, and stage st's
        // buffer is refilled (after those reads are issued)
        if constexpr (MODE == 0) wait_vmcnt<(NS - 2) * IPW>();
        else HLQ_GEMM_WAIT((S - st - 2 < NS - 2 ? S - st - 2 : NS - 2));
        lds_barrier();
        const int ob = buf;
        buf = buf + 1 == NS ? 0 : buf + 1;
        const uint8_t* nb = lds + buf * G::STAGE;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          p0a[i] = *reinterpret_cast<const u32x4*>(nb + a_off + i * 32 * KB + c6[0]);
          p1a[i] = *reinterpret_cast<const u32x4*>(nb + a_off + i * 32 * KB + c6[1]);
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          p0b[j] = *reinterpret_cast<const u32x4*>(nb + b_off + j * 32 * KB + c6[0]);
          p1b[j] = *reinterpret_cast<const u32x4*>(nb + b_off + j * 32 * KB + c6[1]);
        }
        if constexpr (MODE == 0) HLQ_GEMM_ISSUE(st + NS, ob);
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = mfma_fp6(step_op<1>(ra[i]), step_op<1>(rb[j]), acc[i][j]);
    } else {
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const int cur = kk & 1, nxt = cur ^ 1;
      const bool reads = kk + 1 < KK || MODE != 2;
      if (kk + 1 < KK) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
          fa[nxt][i] = *reinterpret_cast<const u32x4*>(base + a_off + i * 32 * KB + coff[kk + 1]);
#pragma unroll
        for (int j = 0; j < FN; ++j)
          fb[nxt][j] = *reinterpret_cast<const u32x4*>(base + b_off + j * 32 * KB + coff[kk + 1]);
      } else if constexpr (MODE != 2) {
        // Before the stage's last k-step (its fragments are already in
        // registers): stage st+1 landed in every wave (st+2 .. st+NS-1 may
        // still fly) and no wave reads stage st any more ...
        if constexpr (MODE == 0) wait_vmcnt<(NS - 2) * IPW>();
        else HLQ_GEMM_WAIT((S - st - 2 < NS - 2 ? S - st - 2 : NS - 2));
        lds_barrier();
        // ... so the first fragments of stage st+1 load under this step's
        // MFMAs, and stage st's buffer is refilled (after those reads are
        // issued: an LDS read behind a DMA into LDS would wait for the DMA).
        const int ob = buf;
        buf = buf + 1 == NS ? 0 : buf + 1;
        const uint8_t* nb = lds + buf * G::STAGE;
#pragma unroll
        for (int i = 0; i < FM; ++i)
          fa[nxt][i] = *reinterpret_cast<const u32x4*>(nb + a_off + i * 32 * KB + coff[0]);
#pragma unroll
        for (int j = 0; j < FN; ++j)
          fb[nxt][j] = *reinterpret_cast<const u32x4*>(nb + b_off + j * 32 * KB + coff[0]);
        if constexpr (MODE == 0) HLQ_GEMM_ISSUE(st + NS, ob);
      }
      if constexpr (BF16) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(v8bf, fa[cur][i]), __builtin_bit_cast(v8bf, fb[cur][j]),
                acc[i][j], 0, 0, 0);
        if (track) {
#pragma unroll
          for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int d = 0; d < 4; ++d) {
              const unsigned run = amax[i][d], mag = fa[cur][i][d] & 0x7FFF7FFFu;
              amax[i][d] = __builtin_bit_cast(
                  unsigned, __builtin_elementwise_max(__builtin_bit_cast(us2, run),
                                                      __builtin_bit_cast(us2, mag)));
            }
        }
        if (reads) {
          HLQ_SGB(0x100, FM + FN);
          HLQ_SGB(0x008, FM * FN);
        }
      } else {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            const u32x4 xa = fa[cur][i], yb = fb[cur][j];
            acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(
                v4i{(int)xa[0], (int)xa[1], (int)xa[2], (int)xa[3]},
                v4i{(int)yb[0], (int)yb[1], (int)yb[2], (int)yb[3]}, acc[i][j], 0, 0, 0);
          }
        if (reads) {
          // every fragment read of the next k-step ahead of this step's
          // MFMAs: the reads get a whole step to land (interleaved one per
          // MFMA, the last one landed just before the next step needed it;
          // qkv pair 42.4 -> 40.3 us)
          HLQ_SGB(0x100, FM + FN);
          HLQ_SGB(0x008, FM * FN);
        }
      }
    }
    }
  };
  int64_t st = 0;
  for (; st + NS < S; ++st) stage(st, std::integral_constant<int, 0>());
  for (; st + 1 < S; ++st) stage(st, std::integral_constant<int, 1>());
  stage(st, std::integral_constant<int, 2>());  // S >= 1
#undef HLQ_GEMM_ISSUE
#undef HLQ_GEMM_WAIT

  if constexpr (!BF16 && !FP6 && !CONV && EPI != EPI_PARTIAL) {
    if (g.nsplit > 1) {
      typedef int v4i __attribute__((ext_vector_type(4)));
      constexpr int NQ = FM * FN * 4;  // 16-byte groups of this thread's sums
      const int64_t tile = tm * ((N + BN - 1) / BN) + tn;
      const int ns = g.nsplit, sp = (int)split;
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          g.part + tile * ns * (int64_t)(BM * BN), 0, ns * BM * BN * 4, 0x00020000);
      constexpr int SC1 = 16;  // cache policy: device scope (write-through / coherent load)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const v4i v = {acc[i][j][4 * k], acc[i][j][4 * k + 1], acc[i][j][4 * k + 2],
                           acc[i][j][4 * k + 3]};
            __builtin_amdgcn_raw_buffer_store_b128(
                v, rs, ((sp * NQ + (i * FN + j) * 4 + k) * NT + tid) * 16, 0, SC1);
          }
      wait_vmcnt<0>();  // this thread's sums have reached device scope
      __shared__ unsigned arrived;
      __syncthreads();
      if (tid == 0)
        arrived = __hip_atomic_fetch_add(g.ctr + tile, 1u, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
      __syncthreads();
      if (arrived != (unsigned)(ns - 1)) return;
      if (tid == 0) __hip_atomic_store(g.ctr + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      for (int o = 0; o < ns; ++o) {
        if (o == sp) continue;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              const v4i v = __builtin_amdgcn_raw_buffer_load_b128(
                  rs, ((o * NQ + (i * FN + j) * 4 + k) * NT + tid) * 16, 0, SC1);
              acc[i][j][4 * k] += v[0];
              acc[i][j][4 * k + 1] += v[1];
              acc[i][j][4 * k + 2] += v[2];
              acc[i][j][4 * k + 3] += v[3];
            }
      }
    }
  }

  if constexpr (BF16) {
    if (acbp) {
      // row maxima: the 8 packed maxima of a fragment, then the other K half
      // (lane ^ 32); rows wm*WTM + i*32 + lane % 32 -> sc[row] (|x| max),
      // sc[BM + row] (reciprocal scale)
      // sc: the row maxima and reciprocal scales of the tile's BM rows (2 BM floats)
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      if (wn == 0) {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          unsigned m = 0u;
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            const unsigned v = amax[i][d];
            m = max(m, max(v & 0xFFFFu, v >> 16));
          }
          m = max(m, (unsigned)__shfl_xor((int)m, 32));
          if (lane < 32) {
            const int row = wm * G::WTM + i * 32 + lane;
            const float a = bf16_to_f32(m);
            sc[row] = a;
            sc[BM + row] = inv_of(a, 7.f);
          }
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      // codes of this tile's slice of its rows' 8-element chunks (16 bytes
      // of x each, read again from cache): eight loads in flight per thread
      const int64_t c8 = pitch / 16;  // 8-element chunks per row
      const int64_t nt_n = (N + BN - 1) / BN;
      const int64_t per = (c8 + nt_n - 1) / nt_n;
      const int64_t cb = tn * per, cw = (c8 - cb < per ? c8 - cb : per);
      const int64_t rows = M - m0 < BM ? M - m0 : BM;
      const int64_t items = cw > 0 ? rows * cw : 0;
      for (int64_t base = tid; base < items; base += NT * 8) {
        uint4 raw[8];
        int64_t off[8];
        int rw[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int64_t it = base + u * NT;
          rw[u] = -1;
          if (it < items) {
            const int64_t row = it / cw, c = cb + (it - row * cw);
            rw[u] = (int)row;
            off[u] = (m0 + row) * pitch + c * 16;
            raw[u] = *reinterpret_cast<const uint4*>(A + off[u]);
          }
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (rw[u] < 0) continue;
          float v[8] = {bf16_lo(raw[u].x), bf16_hi(raw[u].x), bf16_lo(raw[u].y), bf16_hi(raw[u].y),
                        bf16_lo(raw[u].z), bf16_hi(raw[u].z), bf16_lo(raw[u].w), bf16_hi(raw[u].w)};
          *reinterpret_cast<uint32_t*>(g.acbp_codes + off[u] / 4) = quant_pack8_int4(v, sc[BM + rw[u]]);
        }
      }
      if (tn == 0 && tid < rows) g.acbp_scales[m0 + tid] = scale_of(sc[tid], 7.f);
    }
  }

  int32_t* Cp = Ci + (EPI == EPI_PARTIAL ? split * M * N : 0);
  // Scales from LDS (written before the K loop; its barriers published them).
  float s_n[FN], s_m[FM][16];
  if constexpr (EPI == EPI_F32 && !BF16) {
#pragma unroll
    for (int j = 0; j < FN; ++j) s_n[j] = sc[BM + wn * G::WTN + j * 32 + fr];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) s_m[i][r] = sc[wm * G::WTM + i * 32 + 8 * (r / 4) + 4 * fh + (r % 4)];
  }
  // Interior tiles store without per-lane guards: branch-free code lets the
  // counter waits before the stores be exact instead of full drains.  The fp32
  // outputs are written once and not read again here: non-temporal stores
  // stream them to HBM instead of leaving them dirty in L2 / the last-level
  // cache, where the next layer's transform passes would have to evict them
  // (ViT-B qkv: the following MAX pass 20 -> 17.6 us).
  const bool full = m0 + BM <= M && n0 + BN <= N;
  if (full) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + wm * G::WTM + i * 32 + 8 * (r / 4) + 4 * fh + (r % 4);
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int64_t n = n0 + wn * G::WTN + j * 32 + fr;
          if constexpr (BF16) {
            if constexpr (EPI == EPI_BF16) g.Cb[m * N + n] = f32_to_bf16_rne(acc[i][j][r]);
            else C[m * N + n] = acc[i][j][r];
          } else {
            const int32_t v = (int32_t)acc[i][j][r];  // exact (FP6: an integer-valued float)
            if constexpr (EPI == EPI_F32) __builtin_nontemporal_store((float)v * s_m[i][r] * s_n[j], &C[m * N + n]);
            else Cp[m * N + n] = v;
          }
        }
      }
    return;
  }
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t m = m0 + wm * G::WTM + i * 32 + 8 * (r / 4) + 4 * fh + (r % 4);
      if (m >= M) continue;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int64_t n = n0 + wn * G::WTN + j * 32 + fr;
        if (n >= N) continue;
        if constexpr (BF16) {
          if constexpr (EPI == EPI_BF16) g.Cb[m * N + n] = f32_to_bf16_rne(acc[i][j][r]);
          else C[m * N + n] = acc[i][j][r];
        } else {
          const int32_t v = (int32_t)acc[i][j][r];
          if constexpr (EPI == EPI_F32) __builtin_nontemporal_store((float)v * s_m[i][r] * s_n[j], &C[m * N + n]);
          else Cp[m * N + n] = v;
        }
      }
  }
}

template <bool FP6, int BM, int BN, int KB, int NS, int EPI>
__global__ __launch_bounds__(256, 2) void k_gemm(GemmArgs g) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[NS * GemmShape<FP6, BM, BN, KB, NS>::STAGE];
  __shared__ float sc[BM + BN];
  gemm_tile<FP6, BM, BN, KB, NS, EPI>(g, blockIdx.x, blockIdx.y, lds, sc);
}

// Forward product y = x . w^T of a bf16 linear layer, with the ACBP codes of
// x emitted by the first column of tiles (gemm_tile BF16).
// BM = 256 where the grid still fills every workgroup slot of the chip (two
// per CU), else BM = 128 (more, shorter tiles).
template <int BM, int EPI>
__global__ __launch_bounds__(256, 2) void k_forward(GemmArgs g) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[3 * GemmShape<false, BM, 128, 64, 3>::STAGE];
  __shared__ float sc[BM + (BM > 128 ? BM : 128)];
  gemm_tile<false, BM, 128, 64, 3, EPI, false, true>(g, blockIdx.x, 0, lds, sc);
}

// Input gradient of a convolution as an implicit GEMM over the taps (CONV
// addressing in gemm_tile): no im2col / col2im buffer; the INT32 sum runs over
// every (tap, O) pair of an input pixel, so one per-tensor epilogue finishes it.
template <int BM, int BN, int KB, int NS, int EPI>
__global__ __launch_bounds__(256, 2) void k_dgrad(GemmArgs g) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[NS * GemmShape<true, BM, BN, KB, NS>::STAGE];
  __shared__ float sc[BM + BN];
  gemm_tile<true, BM, BN, KB, NS, EPI, true>(g, blockIdx.x, 0, lds, sc);
}

// Both GEMMs of the backward in one launch (fp32 epilogues, no split-K): the
// first n1 workgroups take the g_w tiles (longer K, so they start first), the
// rest the g_x tiles, which fill the CUs around them.  One launch instead of
// two plus a split-K pass, and neither GEMM's tail leaves the GPU idle.
// EPI_I32 stores the INT32 accumulators instead of the fp32 gradients (tests
// compare them bit for bit); everything else is the same launch.
// With gw.nsplit > 1 the first n1 = nsplit * n1w workgroups are split s =
// b / n1w of g_w workgroup b % n1w (n1w a multiple of 8, so every split of a
// tile runs on the XCD the tile mapping gives it).
// WNW = 4: 512 threads (2 x 4 waves), one workgroup per CU.
// MINW: waves per SIMD the registers must allow (three workgroups of 256
// threads per CU take 3: at most 168 VGPRs).
template <int WNW, int BM1, int BN1, int KB1, int NS1, int BM0, int BN0, int KB0, int NS0, int EPI,
          int MINW = (WNW == 2 ? 2 : 1)>
__global__ __launch_bounds__(128 * WNW, MINW) void k_gemm_pair(GemmArgs gw, int64_t n1,
                                                                           int64_t n1w, GemmArgs gx) {
  constexpr int L1 = NS1 * GemmShape<false, BM1, BN1, KB1, NS1, WNW>::STAGE;
  constexpr int L0 = NS0 * GemmShape<true, BM0, BN0, KB0, NS0, WNW>::STAGE;
  constexpr int SC = BM1 + BN1 > BM0 + BN0 ? BM1 + BN1 : BM0 + BN0;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[L1 > L0 ? L1 : L0];
  __shared__ float sc[SC];
  const int64_t b = blockIdx.x;
  if (b < n1) gemm_tile<false, BM1, BN1, KB1, NS1, EPI, false, false, WNW>(gw, b % n1w, b / n1w, lds, sc);
  else gemm_tile<true, BM0, BN0, KB0, NS0, EPI, false, false, WNW>(gx, b - n1, 0, lds, sc);
}

__global__ void k_zero_u32(unsigned* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    p[i] = 0u;
}

// Sum of split-K INT32 partials (exact) followed by the dequantizing epilogue.
__global__ __launch_bounds__(256) void k_gemm_finalize(const int32_t* __restrict__ P,
                                                       int splits, int64_t M, int64_t N,
                                                       const float* __restrict__ sa,
                                                       int sa_step,
                                                       const float* __restrict__ sb,
                                                       int sb_step, float alpha,
                                                       float* __restrict__ C) {
  const int64_t q4 = (int64_t)blockIdx.x * 256 + threadIdx.x;  // index of 4 outputs
  if (q4 * 4 >= M * N) return;
  const int64_t e = q4 * 4;
  const int64_t m = e / N, nn = e % N;
  int4 s = *reinterpret_cast<const int4*>(P + e);
  for (int z = 1; z < splits; ++z) {
    int4 p = *reinterpret_cast<const int4*>(P + (int64_t)z * M * N + e);
    s.x += p.x; s.y += p.y; s.z += p.z; s.w += p.w;
  }
  const float s_m = sa[m * sa_step] * alpha;
  float4 o;
  o.x = (float)s.x * s_m * sb[(nn + 0) * sb_step];
  o.y = (float)s.y * s_m * sb[(nn + 1) * sb_step];
  o.z = (float)s.z * s_m * sb[(nn + 2) * sb_step];
  o.w = (float)s.w * s_m * sb[(nn + 3) * sb_step];
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  __builtin_nontemporal_store(f32x4{o.x, o.y, o.z, o.w}, reinterpret_cast<f32x4*>(C + e));
}

// Tile configurations (rows of A x rows of B, stage depth, ring depth):
//   INT8: 0: 128 x 128, KB  64, 3 stages  (48 KB LDS, two workgroups per CU)
//         1: 256 x 128, KB  64, 3 stages  (72 KB LDS, two workgroups per CU)
//         2: 128 x 128, KB 128, 2 stages  (64 KB LDS, two workgroups per CU)
//   FP6:  0: 128 x 128, KB  96, 3 stages  (72 KB LDS, two workgroups per CU)
//         (a 256 x 128 FP6 tile needs more than the 256 VGPRs of two
//         workgroups per CU)
// Large INT8 grids take the 256 x 128 tile; INT8 operands with K a multiple
// of 128 bytes take the deeper stage; grids below the CU count split K.
GemmPlan plan_gemm(bool fp6, int64_t M, int64_t N, int64_t kbytes) {
  static const int cfg_bm[3] = {128, 256, 128}, cfg_bn[3] = {128, 128, 128};
  static const int cfg_kb[3] = {64, 64, 128};
  GemmPlan p;
  auto tiles = [&](int c) { return (int64_t)cdiv(M, cfg_bm[c]) * cdiv(N, cfg_bn[c]); };
  if (!fp6 && tiles(1) >= 1024) p.cfg = 1;
  else if (!fp6 && kbytes % 128 == 0) p.cfg = 2;
  else p.cfg = 0;
  p.bm = cfg_bm[p.cfg];
  p.bn = cfg_bn[p.cfg];
  p.kb = fp6 ? 96 : cfg_kb[p.cfg];
  p.stages = kbytes / p.kb;
  const int64_t t = tiles(p.cfg);
  int64_t sp = 1;
  while (t * sp < 256 && sp < 8 && p.stages / (sp * 2) >= 8) sp *= 2;
  p.sps = (p.stages + sp - 1) / sp;
  p.splits = (int)((p.stages + p.sps - 1) / p.sps);  // every split non-empty
  return p;
}

template <bool F6, int EPI>
static void gemm_dispatch(int cfg, dim3 g, hipStream_t s, const GemmArgs& a) {
#define HLQ_GEMM(BM_, BN_, KB_, NS_) \
  hipLaunchKernelGGL((k_gemm<F6, BM_, BN_, KB_, NS_, EPI>), g, dim3(256), 0, s, a)
  if constexpr (F6) {
    HLQ_GEMM(128, 128, 96, 3);
  } else {
    switch (cfg) {
      case 1: HLQ_GEMM(256, 128, 64, 3); break;
      case 2: HLQ_GEMM(128, 128, 128, 2); break;
      default: HLQ_GEMM(128, 128, 64, 3); break;
    }
  }
#undef HLQ_GEMM
}

hipError_t launch_gemm(bool fp6, const uint8_t* A, const uint8_t* B, int64_t M,
                       int64_t N, int64_t pitch, const GemmPlan& plan,
                       const float* sa, int sa_step, const float* sb, int sb_step,
                       float alpha, GemmEpi epi, float* C, int32_t* Ci,
                       int32_t* partial, hipStream_t s) {
  if (pitch % plan.kb != 0 || plan.stages * plan.kb != pitch) return hipErrorInvalidValue;
  const int splits = epi == EPI_I32 ? 1 : plan.splits;
  const int64_t sps = splits == 1 ? plan.stages : plan.sps;
  const int64_t tiles = (int64_t)cdiv(M, plan.bm) * cdiv(N, plan.bn);
  dim3 grid((unsigned)((tiles + 7) / 8 * 8), splits);
  const bool use_partial = (epi == EPI_F32 && splits > 1);
  if (use_partial && partial == nullptr) return hipErrorInvalidValue;
  if (epi == EPI_F32 && (C == nullptr || sa == nullptr || sb == nullptr))
    return hipErrorInvalidValue;
  if (epi == EPI_I32 && Ci == nullptr) return hipErrorInvalidValue;
  const int e = use_partial ? EPI_PARTIAL : epi;
  GemmArgs a{A, B, M, N, pitch, plan.stages, sps, sa, sa_step, sb, sb_step, alpha, C,
             use_partial ? partial : Ci};
  if (fp6) {
    if (e == EPI_F32) gemm_dispatch<true, EPI_F32>(plan.cfg, grid, s, a);
    else if (e == EPI_I32) gemm_dispatch<true, EPI_I32>(plan.cfg, grid, s, a);
    else gemm_dispatch<true, EPI_PARTIAL>(plan.cfg, grid, s, a);
  } else {
    if (e == EPI_F32) gemm_dispatch<false, EPI_F32>(plan.cfg, grid, s, a);
    else if (e == EPI_I32) gemm_dispatch<false, EPI_I32>(plan.cfg, grid, s, a);
    else gemm_dispatch<false, EPI_PARTIAL>(plan.cfg, grid, s, a);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || !use_partial) return err;
  return launch_gemm_finalize(partial, splits, M, N, sa, sa_step, sb, sb_step, alpha, C, s);
}

// g_w tile of the pair launch: the plan's, except that a grid of at most 128
// tiles of 128 x 128 takes the deep-ring configuration (wcfg 5: 128 x 128, KB
// 64, 4 stages), and a larger one beside g_x tiles of at most 8 stages the
// three-workgroup configuration (wcfg 6: KB 64 in 3 stages, the g_x ring 2
// deep).  Then K splits: the g_w tiles start first, so a g_w tile
// longer than the launch's mean work per workgroup slot (two per CU) sets its
// length; nsplit cuts it (at most 4 splits of at least 4 stages each) when it
// is more than twice that mean.  Work is counted in MACs, an FP6 MAC (twice
// the INT8 rate on the matrix cores, more LDS bytes per MAC) at 0.7 INT8 MACs.
static int pair_splits(double dw, double dx, int64_t tw, int64_t tx, int64_t slots,
                       int64_t wstages) {
  const double mean = (tw * dw + tx * dx) / (double)slots;
  // a split costs a merge (the partial sums written and read back once): split
  // only tiles that cost more than twice a slot's mean load
  int ns = (int)std::ceil(dw / mean - 1.0);
  ns = std::max(1, std::min(ns, 4));
  while (ns > 1 && wstages / ns < 4) --ns;
  return ns;
}

PairPlan plan_pair(int64_t T, int64_t I, int64_t O, const GemmPlan& px, const GemmPlan& pw) {
  PairPlan pp;
  // 256 x 256 tiles (8 waves, one workgroup per CU) for long-K grids that
  // 128-tiles would run in many rounds: each 128 x 128 tile re-reads its
  // operand rows from L2 twice as often (Llama-3 down-proj pair 336 -> 264
  // us).  Grids of one or two rounds keep 128-tiles (ViT-B qkv: 42.6 us
  // against 59.6 for 256-tiles in one round, whose K-split g_w tiles run
  // longest); so do short-K grids, bound by their fp32 output.
  {
    const int64_t sx = (int64_t)cdiv(T, 128) * cdiv(I, 128), sw = (int64_t)cdiv(O, 128) * cdiv(I, 128);
    pp.big = px.kb == 96 && pw.kb % 64 == 0 && sx + sw >= 8 * 512 && px.stages >= 8;
  }
  int64_t wstages = pw.stages, xbm = px.bm, xbn = px.bn, slots = 512;
  if (pp.big) {
    // 256 x 256 tiles, 8 waves, one workgroup per CU: half the L2 -> LDS
    // bytes per product of 128 x 128 tiles, the LDS rings 4 x 32 KB (INT8,
    // KB 64) and 3 x 48 KB (FP6)
    pp.wcfg = 4; pp.wbm = 256; pp.wbn = 256;
    wstages = pw.stages * pw.kb / 64;
    xbm = 256; xbn = 256; slots = 256;
  } else {
    pp.wcfg = pw.cfg; pp.wbm = pw.bm; pp.wbn = pw.bn;
    if (pw.kb % 64 == 0 && (int64_t)cdiv(O, 128) * cdiv(I, 128) <= 128) {
      // a small g_w grid (its tiles run beside the g_x tiles, K long): 64-byte
      // stages in a four-deep ring, three stages (48 KB) in flight per
      // workgroup instead of one 32 KB stage of the two-deep 128-byte ring
      // (64 KB of LDS, inside the FP6 ring's 72 KB; ViT-B qkv pair 41.5 ->
      // 39.4 us, ResNet-50 stage-3 shape 89.5 -> 80.7; fc2's 144-tile grid
      // is faster with the 128-byte stages)
      pp.wcfg = 5; pp.wbm = 128; pp.wbn = 128;
      wstages = pw.stages * pw.kb / 64;
    } else if (pw.kb % 64 == 0 && px.kb == 96 && px.stages <= 8) {
      // a larger g_w grid beside short-K g_x tiles (their fixed per-tile
      // costs, prologue loads and fp32 epilogue, dominate): three workgroups
      // per CU, a two-deep FP6 ring and a three-deep ring of 64-byte INT8
      // stages (48 KB each; ViT-B fc2 pair 54.7 -> 50.6 us median of 21
      // interleaved rounds, T = 25216 95.6 -> 86.3; qkv and the ResNet-50
      // shape are slower this way)
      pp.wcfg = 6; pp.wbm = 128; pp.wbn = 128;
      wstages = pw.stages * pw.kb / 64;
      slots = 768;
    }
  }
  pp.wstages = wstages;
  pp.tx = (int64_t)cdiv(T, xbm) * cdiv(I, xbn);
  pp.tw = (int64_t)cdiv(O, pp.wbm) * cdiv(I, pp.wbn);
  // tile costs in K values: the K loop, plus the fp32 epilogue, which costs
  // about as much as six 128-value stages (it sets the time of short-K
  // tiles: ResNet-50 stage-3 shape pair 94.8 -> 88.5 us without the K split
  // this term removes)
  constexpr double kEpi = 768;
  const double dw = (double)pp.wbm * pp.wbn * (pw.stages * pw.kb + kEpi);
  const double dx = 0.7 * xbm * xbn * (px.stages * (px.kb * 4 / 3) + kEpi);
  int ns = pair_splits(dw, dx, pp.tw, pp.tx, slots, wstages);
  pp.sps = (wstages + ns - 1) / ns;
  pp.nsplit = (int)((wstages + pp.sps - 1) / pp.sps);  // every split non-empty
  pp.part_bytes = pp.nsplit > 1 ? (size_t)pp.tw * pp.nsplit * pp.wbm * pp.wbn * 4 : 0;
  pp.nctr = pp.nsplit > 1 ? pp.tw : 0;
  return pp;
}

hipError_t launch_gemm_pair(const uint8_t* gxA, const uint8_t* gxB, int64_t T, int64_t I,
                            int64_t kx_pitch, const GemmPlan& px, const float* s_gy,
                            const float* s_w, int gx_step, float gx_alpha, float* g_x,
                            const uint8_t* gwA, const uint8_t* gwB, int64_t O, int64_t kw_pitch,
                            const GemmPlan& pw, const float* s_gyl, const float* s_xl,
                            int gw_step, float gw_alpha, float* g_w, const PairPlan& pp,
                            int32_t* part, unsigned* ctr, bool zero_ctr, hipStream_t s,
                            GemmEpi epi, int32_t* acc_x, int32_t* acc_w) {
  if (kx_pitch % px.kb || px.stages * px.kb != kx_pitch) return hipErrorInvalidValue;
  if (kw_pitch % pw.kb || pw.stages * pw.kb != kw_pitch) return hipErrorInvalidValue;
  if (epi == EPI_F32 && (!g_x || !g_w || !s_gy || !s_w || !s_gyl || !s_xl))
    return hipErrorInvalidValue;
  if (epi == EPI_I32 && (!acc_x || !acc_w)) return hipErrorInvalidValue;
  if (epi != EPI_F32 && epi != EPI_I32) return hipErrorInvalidValue;
  if (pp.nsplit < 1 || pp.nsplit > 4 || (pp.nsplit > 1 && (!part || !ctr))) return hipErrorInvalidValue;
  if ((pp.nsplit - 1) * pp.sps >= pp.wstages) return hipErrorInvalidValue;  // an empty split
  if (pp.wstages * (pp.big || pp.wcfg >= 5 ? 64 : pw.kb) != kw_pitch) return hipErrorInvalidValue;
  const GemmArgs ax{gxA, gxB, T, I, kx_pitch, px.stages, px.stages, s_gy, gx_step, s_w, gx_step,
                    gx_alpha, g_x, acc_x};
  GemmArgs aw{gwA, gwB, O, I, kw_pitch, pp.wstages, pp.sps, s_gyl, gw_step, s_xl, gw_step,
              gw_alpha, g_w, acc_w};
  aw.nsplit = pp.nsplit;
  aw.part = part;
  aw.ctr = ctr;
  if (pp.nsplit > 1 && zero_ctr) {
    hipLaunchKernelGGL(k_zero_u32, dim3((unsigned)std::min<int64_t>(cdiv(pp.nctr, 256), 64)),
                       dim3(256), 0, s, ctr, pp.nctr);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t n1w = (pp.tw + 7) / 8 * 8, n0 = (pp.tx + 7) / 8 * 8;
  const int64_t n1 = n1w * pp.nsplit;
  const dim3 g((unsigned)(n1 + n0));
#define HLQ_PAIR(W_, X_)                                                                 \
  do {                                                                                   \
    if (epi == EPI_F32) hipLaunchKernelGGL((k_gemm_pair<2, W_, X_, EPI_F32>), g, dim3(256), 0, s, aw, n1, n1w, ax); \
    else hipLaunchKernelGGL((k_gemm_pair<2, W_, X_, EPI_I32>), g, dim3(256), 0, s, aw, n1, n1w, ax); \
  } while (0)
  if (pp.big) {
    if (epi == EPI_F32)
      hipLaunchKernelGGL((k_gemm_pair<4, 256, 256, 64, 4, 256, 256, 96, 3, EPI_F32>), g, dim3(512), 0, s, aw, n1, n1w, ax);
    else
      hipLaunchKernelGGL((k_gemm_pair<4, 256, 256, 64, 4, 256, 256, 96, 3, EPI_I32>), g, dim3(512), 0, s, aw, n1, n1w, ax);
    return hipGetLastError();
  }
#define HLQ_W0 128, 128, 64, 3
#define HLQ_W1 256, 128, 64, 3
#define HLQ_W2 128, 128, 128, 2
#define HLQ_W5 128, 128, 64, 4
#define HLQ_W6 128, 128, 64, 3
#define HLQ_X0 128, 128, 96, 3
#define HLQ_X6 128, 128, 96, 2
  if (px.cfg != 0 || px.kb != 96) return hipErrorInvalidValue;
  switch (pp.wcfg) {
    case 1: HLQ_PAIR(HLQ_W1, HLQ_X0); break;
    case 2: HLQ_PAIR(HLQ_W2, HLQ_X0); break;
    case 5: HLQ_PAIR(HLQ_W5, HLQ_X0); break;
    case 6:
      if (epi == EPI_F32) hipLaunchKernelGGL((k_gemm_pair<2, HLQ_W6, HLQ_X6, EPI_F32, 3>), g, dim3(256), 0, s, aw, n1, n1w, ax);
      else hipLaunchKernelGGL((k_gemm_pair<2, HLQ_W6, HLQ_X6, EPI_I32, 3>), g, dim3(256), 0, s, aw, n1, n1w, ax);
      break;
    default: HLQ_PAIR(HLQ_W0, HLQ_X0); break;
  }
#undef HLQ_PAIR
#undef HLQ_W0
#undef HLQ_W1
#undef HLQ_W2
#undef HLQ_W5
#undef HLQ_W6
#undef HLQ_X6
#undef HLQ_X0
  return hipGetLastError();
}

hipError_t launch_dgrad(const ConvGemm& c, hipStream_t s) {
  if (c.kx_pitch % 96 || c.taps <= 0 || c.C % 8) return hipErrorInvalidValue;
  if ((c.epi == EPI_F32 && (!c.g_x || !c.s_gy || !c.s_w)) || (c.epi == EPI_I32 && !c.acc_x))
    return hipErrorInvalidValue;
  const int64_t M = c.N * c.H * c.W;
  const int64_t so = c.kx_pitch / 96;  // 96-byte (128-value) stages per tap
  GemmArgs a{c.q_gy, c.q_w, M, c.C, c.kx_pitch, so * c.taps, so * c.taps, c.s_gy, 0, c.s_w, 0,
             c.alpha, c.g_x, c.acc_x};
  a.cH = (int32_t)c.H; a.cW = (int32_t)c.W; a.cP = (int32_t)c.P; a.cQ = (int32_t)c.Q;
  a.cS = (int32_t)c.S; a.cC = (int32_t)c.C; a.cstride = c.stride; a.cpad = c.pad;
  a.cSO = (int32_t)so;
  a.cArows = c.N * c.P * c.Q;
  a.cBrows = c.taps * c.C;
  a.zero = c.zero;
  const int64_t tiles = (int64_t)cdiv(M, 128) * cdiv(c.C, 128);
  const dim3 g((unsigned)((tiles + 7) / 8 * 8));
  if (c.epi == EPI_F32) hipLaunchKernelGGL((k_dgrad<128, 128, 96, 3, EPI_F32>), g, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((k_dgrad<128, 128, 96, 3, EPI_I32>), g, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_forward(const uint16_t* x, const uint16_t* w, int64_t T, int64_t I, int64_t O,
                          float* y32, uint16_t* y16, uint8_t* codes, float* scales,
                          hipStream_t s) {
  if (I % 32 || (!y32 && !y16) || (codes && !scales)) return hipErrorInvalidValue;
  const int64_t pitch = 2 * I, stages = pitch / 64;
  GemmArgs a{reinterpret_cast<const uint8_t*>(x), reinterpret_cast<const uint8_t*>(w), T, O, pitch,
             stages, stages, nullptr, 0, nullptr, 0, 1.f, y32, nullptr};
  a.Cb = y16;
  a.acbp_codes = codes;
  a.acbp_scales = scales;
  const int64_t tiles256 = (int64_t)cdiv(T, 256) * cdiv(O, 128);
  const bool big = tiles256 >= 2 * 256;  // two workgroups per CU, 256 CUs
  const int64_t tiles = big ? tiles256 : (int64_t)cdiv(T, 128) * cdiv(O, 128);
  const dim3 g((unsigned)((tiles + 7) / 8 * 8));
  if (big) {
    if (y16) hipLaunchKernelGGL((k_forward<256, EPI_BF16>), g, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((k_forward<256, EPI_F32>), g, dim3(256), 0, s, a);
  } else {
    if (y16) hipLaunchKernelGGL((k_forward<128, EPI_BF16>), g, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((k_forward<128, EPI_F32>), g, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_gemm_finalize(const int32_t* partial, int splits, int64_t M,
                                int64_t N, const float* sa, int sa_step,
                                const float* sb, int sb_step, float alpha, float* C,
                                hipStream_t s) {
  const int64_t q4 = M * N / 4;
  hipLaunchKernelGGL(k_gemm_finalize, dim3(cdiv(q4, 256)), dim3(256), 0, s, partial, splits,
                     M, N, sa, sa_step, sb, sb_step, alpha, C);
  return hipGetLastError();
}

}  // namespace hlq
