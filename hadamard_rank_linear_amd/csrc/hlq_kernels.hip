// gfx950 (CDNA4) kernels of the HLQ/HOT linear-layer backward.
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
#include <stdint.h>

#include <type_traits>

#include "hlq_internal.h"

namespace hlq {

typedef int v4i __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------ helpers

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// 8 consecutive elements starting at element index `e` of a row.
template <int DT>
__device__ __forceinline__ void load8(const void* base, int64_t e, float (&v)[8]) {
  if constexpr (DT == 0) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + e);
    float4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
    const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + e);
    v[0] = bf16_to_f32(u.x & 0xFFFFu); v[1] = bf16_to_f32(u.x >> 16);
    v[2] = bf16_to_f32(u.y & 0xFFFFu); v[3] = bf16_to_f32(u.y >> 16);
    v[4] = bf16_to_f32(u.z & 0xFFFFu); v[5] = bf16_to_f32(u.z >> 16);
    v[6] = bf16_to_f32(u.w & 0xFFFFu); v[7] = bf16_to_f32(u.w >> 16);
  }
}

template <int DT>
__device__ __forceinline__ float load1(const void* base, int64_t e) {
  if constexpr (DT == 0) return static_cast<const float*>(base)[e];
  else return bf16_to_f32(static_cast<const uint16_t*>(base)[e]);
}

__device__ __forceinline__ float wave_max(float a) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) a = fmaxf(a, __shfl_xor(a, m));
  return a;
}

// In-lane butterflies over 8 consecutive elements (stages h = 1, 2, 4).
__device__ __forceinline__ void fwht8(float (&v)[8]) {
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if ((k & h) == 0) {
        float a = v[k], b = v[k + h];
        v[k] = a + b;
        v[k + h] = a - b;
      }
    }
  }
}

// Cross-lane butterflies: element distance 8*m lives in lane ^ m.  Lower lane
// keeps a + b, upper lane keeps a - b where a is the lower lane's value.
__device__ __forceinline__ void fwht_lanes(float (&v)[8], int lane, int lanes_per_block) {
  for (int m = 1; m < lanes_per_block; m <<= 1) {
    const bool upper = (lane & m) != 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      float p = __shfl_xor(v[k], m);
      v[k] = upper ? (p - v[k]) : (v[k] + p);
    }
  }
}

// Quantizer code of v: rne(fl(v * inv)) as the low bits of a two's-complement
// integer.  Adding 1.5 * 2^23 to fl(v * inv) (|.| < 2^22) lands in [2^23, 2^24),
// where the fp32 spacing is 1, so that one IEEE add performs the
// round-half-to-even and leaves the integer in the low mantissa bits (the
// build forbids contracting the multiply into the add).  No clamp is needed:
// |v| <= a gives |fl(v * fl(QMAX / a))| <= QMAX * (1 + 2^-24), which rounds to
// at most QMAX.  Mask the result to 4 (INT4) or 8 (INT8) bits.
template <int QMAX>
__device__ __forceinline__ uint32_t quant_bits(float v, float inv) {
  const float p = v * inv;
  return __float_as_uint(p + 12582912.0f);
}

// Low bytes of four words gathered into one word (byte i <- w_i), 3 v_perm.
__device__ __forceinline__ uint32_t pack_lo_bytes(uint32_t w0, uint32_t w1, uint32_t w2,
                                                  uint32_t w3) {
  const uint32_t lo = __builtin_amdgcn_perm(w1, w0, 0x0c0c0400u);  // w0.b0 w1.b0 0 0
  const uint32_t hi = __builtin_amdgcn_perm(w3, w2, 0x0c0c0400u);  // w2.b0 w3.b0 0 0
  return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

// 8 INT4 codes packed two per byte, element 2k in the low nibble: the low
// bytes of the even and odd elements are gathered, then nibble-merged.
__device__ __forceinline__ uint32_t pack8_nibbles(const uint32_t (&q)[8]) {
  const uint32_t ev = pack_lo_bytes(q[0], q[2], q[4], q[6]);
  const uint32_t od = pack_lo_bytes(q[1], q[3], q[5], q[7]);
  return (ev & 0x0F0F0F0Fu) | ((od << 4) & 0xF0F0F0F0u);
}

__device__ __forceinline__ uint32_t quant_pack8_int4(const float (&v)[8], float inv) {
  uint32_t q[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) q[k] = quant_bits<7>(v[k], inv);
  return pack8_nibbles(q);
}

// Reciprocal scale of a group with absmax a.  A zero group, and a group so
// small that qmax / a overflows fp32, get 0: all their codes are zero.
__device__ __forceinline__ float inv_of(float a, float qmax) {
  const float r = qmax / a;
  return (a == 0.f || r == __builtin_huge_valf()) ? 0.f : r;
}
__device__ __forceinline__ float scale_of(float a, float qmax) { return a == 0.f ? 0.f : a / qmax; }

// ------------------------------------------------------------ ACBP pack
// One wave per token row: absmax over the row, then INT4 codes (qmax 7).

// One wave per token row.  RC > 0: the row (at most RC * 512 elements) stays
// in registers between the maximum and the codes, all of its loads issued
// before the reduction (qkv rows: 8.9 -> 8.0 us; two rows per wave measured no
// better); RC == 0: longer rows are read twice (the second time from cache).
template <int DT, int RC>
__global__ __launch_bounds__(256) void k_acbp(const void* __restrict__ x, int64_t T,
                                              int64_t I, uint8_t* __restrict__ codes,
                                              float* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= T) return;
  const int64_t base = row * I;
  uint8_t* out = codes + row * (I / 2);
  float a = 0.f;
  if constexpr (RC > 0) {
    float v[RC][8];
#pragma unroll
    for (int j = 0; j < RC; ++j) {
      const int64_t c = lane * 8 + j * 512;
      if (c < I) load8<DT>(x, base + c, v[j]);
      else
#pragma unroll
        for (int k = 0; k < 8; ++k) v[j][k] = 0.f;
    }
#pragma unroll
    for (int j = 0; j < RC; ++j)
#pragma unroll
      for (int k = 0; k < 8; ++k) a = fmaxf(a, fabsf(v[j][k]));
    a = wave_max(a);
    const float inv = inv_of(a, 7.f);
#pragma unroll
    for (int j = 0; j < RC; ++j) {
      const int64_t c = lane * 8 + j * 512;
      if (c < I) *reinterpret_cast<uint32_t*>(out + c / 2) = quant_pack8_int4(v[j], inv);
    }
  } else {
    for (int64_t c = lane * 8; c < I; c += 512) {
      float v[8];
      load8<DT>(x, base + c, v);
#pragma unroll
      for (int k = 0; k < 8; ++k) a = fmaxf(a, fabsf(v[k]));
    }
    a = wave_max(a);
    const float inv = inv_of(a, 7.f);
    for (int64_t c = lane * 8; c < I; c += 512) {
      float v[8];
      load8<DT>(x, base + c, v);
      *reinterpret_cast<uint32_t*>(out + c / 2) = quant_pack8_int4(v, inv);
    }
  }
  if (lane == 0) scales[row] = scale_of(a, 7.f);
}


// Value of lane ^ M of the wave (M = 1, 2: DPP quad permute; 8: DPP row
// rotate by 8; 4, 16: swizzle inside 32 lanes; 32: bpermute).
template <int M>
__device__ __forceinline__ float lane_xor(float v) {
  const int b = __float_as_int(v);
  if constexpr (M == 1) return __int_as_float(__builtin_amdgcn_mov_dpp(b, 0xB1, 0xF, 0xF, true));
  else if constexpr (M == 2) return __int_as_float(__builtin_amdgcn_mov_dpp(b, 0x4E, 0xF, 0xF, true));
  else if constexpr (M == 8) return __int_as_float(__builtin_amdgcn_mov_dpp(b, 0x128, 0xF, 0xF, true));
  else if constexpr (M == 4) return __int_as_float(__builtin_amdgcn_ds_swizzle(b, 0x101F));
  else if constexpr (M == 16) return __int_as_float(__builtin_amdgcn_ds_swizzle(b, 0x401F));
  else return __int_as_float(__builtin_amdgcn_ds_bpermute((int)((threadIdx.x ^ 32) & 63) * 4, b));
}

// Max over the 8 lanes c16 = 0..7 of a row group (quad swaps, then the
// half-row mirror pairs each lane with one of the other quad).
__device__ __forceinline__ float group8_max(float m) {
  m = fmaxf(m, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(m), 0xB1, 0xF, 0xF, true)));
  m = fmaxf(m, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(m), 0x4E, 0xF, 0xF, true)));
  m = fmaxf(m, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(m), 0x141, 0xF, 0xF, true)));
  return m;
}

// Butterfly stage with the partner lane ^ M: the lower lane keeps
// own + partner, the upper partner - own; fma(+-1, own, partner) is that one
// IEEE add, so the result equals the in-register butterfly bit for bit.
template <int M>
__device__ __forceinline__ float xbfly(float v, float sgn) {
  return __builtin_fmaf(sgn, v, lane_xor<M>(v));
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// ------------------------------------------------------------ operand transforms
// All four GEMM operands come from one tile engine.  A tile is TT rows x CW
// columns of a row-major source: g_y [T][O] (rows = tokens), the ACBP codes of
// x [T][I], or w [O][I] (rows = output features).  Each tile is loaded once
// with coalesced 16-byte loads (all of a thread's loads issued before any
// arithmetic) and parked in LDS in its source form - bf16 or fp32 values, or
// the packed INT4 codes plus one scale per row - with 16-byte LDS writes.
// Every column is then transformed along the rows by one thread per (column,
// block) task reading LDS column-wise (consecutive threads take consecutive
// columns: no bank conflicts):
//   * g_y and x: the low-rank rows of H_n along tokens (g_w path);
//   * w: the full H_n along O (g_x path, operand B).
// g_y rows are also transformed along O in registers while loading (g_x path,
// operand A): each lane owns 8 consecutive columns, n/8 lanes form a block,
// butterflies cross lanes with xor shuffles.
//
// Two launches of the same kernel:
//   MAX:   every tile writes its partial maxima (per row chunk, per column
//          range) to plain arrays - no atomics;
//   QUANT: after k_tr_reduce has folded the partials, every tile recomputes
//          its transforms and writes codes; the transposed operands are
//          staged in LDS so each column's run of codes leaves in wide stores.
// Workgroups of the three sources share one grid (g_y first: largest tiles).
// Keeping the tile in its source form (35 KB for bf16) lets four workgroups
// share a CU, which the load/transform/store phases need to overlap.

constexpr int TT = TR_ROWS;     // rows per tile
constexpr int CW = TR_COLS;     // columns per tile
constexpr int P_F32 = CW + 4;   // LDS pitches (elements); rows stay 16-byte aligned
constexpr int P_B16 = CW + 8;
constexpr int P_I4 = CW / 2 + 16;  // bytes: two codes per byte
constexpr int OUT_BYTES = 128;  // staging bytes per column (>= TT*r/n and TT/2)
// Pitch of a staged column: 36 banks apart, so the 4-byte writes of 64
// consecutive columns spread over 16 banks instead of 2.
constexpr int OUT_PITCH = 144;

template <bool F32>
struct TileSmem {
  static constexpr int bytes = F32 ? TT * P_F32 * 4 : TT * P_B16 * 2;
};

// Column readers: value of (row, c) of the tile as fp32, exactly as the
// source holds it (bf16 widened; INT4 code times its row scale, one rounding).
struct RdF32 {
  const float* t;
  __device__ __forceinline__ float operator()(int r, int c) const { return t[r * P_F32 + c]; }
};
struct RdB16 {
  const uint16_t* t;
  __device__ __forceinline__ float operator()(int r, int c) const {
    return __uint_as_float((uint32_t)t[r * P_B16 + c] << 16);
  }
};
struct RdI4 {
  const uint8_t* q;
  const float* s;
  __device__ __forceinline__ float operator()(int r, int c) const {
    const int byte = q[r * P_I4 + (c >> 1)];
    const int code = __builtin_amdgcn_sbfe(byte, (c & 1) * 4, 4);
    return s[r] * (float)code;
  }
};

__device__ __forceinline__ float max_over_16_lanes(float a) {
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) a = fmaxf(a, __shfl_xor(a, m));
  return a;
}

// Butterflies across the lanes of one 16-lane row group (element distance
// 8*m lives in lane ^ m; m < 16 keeps the exchange inside the group).  The
// lower lane keeps p + v, the upper lane p - v = p + (-v) (a is the lower
// lane's value): both exact IEEE adds.
template <int N>
__device__ __forceinline__ void fwht_lanes_n(float (&v)[8], int lc) {
#pragma unroll
  for (int m = 1; m < N / 8; m <<= 1) {
    const bool upper = (lc & m) != 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float p = __shfl_xor(v[k], m);
      v[k] = p + (upper ? -v[k] : v[k]);
    }
  }
}

// Low-rank rows of H_N for one column block: group sums of N/R consecutive
// rows in adjacent-pair tree order (the first log2(N/R) butterfly stages on
// the kept rows), then H_R in registers.
template <int N, int R, class RD>
__device__ __forceinline__ void lowrank_col(const RD& rd, int r0, int c, float (&g)[R]) {
  constexpr int G = N / R;
#pragma unroll
  for (int j = 0; j < R; ++j) {
    float s[G];
#pragma unroll
    for (int k = 0; k < G; ++k) s[k] = rd(r0 + j * G + k, c);
#pragma unroll
    for (int h = 1; h < G; h <<= 1)
#pragma unroll
      for (int k = 0; k < G; k += 2 * h) s[k] = s[k] + s[k + h];
    g[j] = s[0];
  }
#pragma unroll
  for (int h = 1; h < R; h <<= 1)
#pragma unroll
    for (int j = 0; j < R; ++j)
      if ((j & h) == 0) {
        float x0 = g[j], x1 = g[j + h];
        g[j] = x0 + x1;
        g[j + h] = x0 - x1;
      }
}

// Full H_N of one column block.
template <int N, class RD>
__device__ __forceinline__ void full_col(const RD& rd, int r0, int c, float (&v)[N]) {
#pragma unroll
  for (int k = 0; k < N; ++k) v[k] = rd(r0 + k, c);
#pragma unroll
  for (int h = 1; h < N; h <<= 1)
#pragma unroll
    for (int k = 0; k < N; ++k)
      if ((k & h) == 0) {
        float x0 = v[k], x1 = v[k + h];
        v[k] = x0 + x1;
        v[k + h] = x0 - x1;
      }
}

// 8 consecutive source elements as raw 16 bytes (bf16) or 32 bytes (fp32).
struct Raw8 {
  uint4 a, b;
};
__device__ __forceinline__ void load_raw8(const void* base, int dt, int64_t e, Raw8& r) {
  if (dt == 0) {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const float*>(base) + e);
    r.a = p[0];
    r.b = p[1];
  } else {
    r.a = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + e);
  }
}
__device__ __forceinline__ void raw8_to_f32(const Raw8& r, int dt, float (&v)[8]) {
  if (dt == 0) {
    v[0] = __uint_as_float(r.a.x); v[1] = __uint_as_float(r.a.y);
    v[2] = __uint_as_float(r.a.z); v[3] = __uint_as_float(r.a.w);
    v[4] = __uint_as_float(r.b.x); v[5] = __uint_as_float(r.b.y);
    v[6] = __uint_as_float(r.b.z); v[7] = __uint_as_float(r.b.w);
  } else {
    v[0] = bf16_to_f32(r.a.x & 0xFFFFu); v[1] = bf16_to_f32(r.a.x >> 16);
    v[2] = bf16_to_f32(r.a.y & 0xFFFFu); v[3] = bf16_to_f32(r.a.y >> 16);
    v[4] = bf16_to_f32(r.a.z & 0xFFFFu); v[5] = bf16_to_f32(r.a.z >> 16);
    v[6] = bf16_to_f32(r.a.w & 0xFFFFu); v[7] = bf16_to_f32(r.a.w >> 16);
  }
}
// Park 8 source elements of (row, col..col+7) in the tile (16-byte writes).
// A fp32 tile widens bf16 exactly; a bf16 tile only ever holds bf16 sources.
template <bool F32>
__device__ __forceinline__ void park8(uint8_t* smem, int row, int col, const Raw8& r, int dt) {
  if constexpr (F32) {
    float v[8];
    raw8_to_f32(r, dt, v);
    float* t = reinterpret_cast<float*>(smem) + row * P_F32 + col;
    *reinterpret_cast<float4*>(t) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(t + 4) = make_float4(v[4], v[5], v[6], v[7]);
  } else {
    *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(smem) + row * P_B16 + col) = r.a;
  }
}

// Column maxima of a tile: thread tid covers column tid % CW; the two threads
// of a column meet in LDS.
__device__ __forceinline__ void tile_colmax_store(float m, float* red, int tid, int cols,
                                                  float* dst) {
  red[tid] = m;
  __syncthreads();
  if (tid < CW && tid < cols) dst[tid] = fmaxf(red[tid], red[tid + CW]);
}

// Store the staged transposed codes: column c of the tile owns `len` bytes at
// dst + c * pitch (dst already offset to the tile's first K byte).  Byte runs
// go out in the widest unit that divides both the run and its offset.
__device__ __forceinline__ void store_staged(const uint8_t (*outs)[OUT_PITCH], int cols,
                                             int len, uint8_t* dst, int64_t pitch,
                                             int64_t koff, int tid) {
  int wdt = 16;
  while (wdt > 1 && ((len % wdt) || (koff % wdt))) wdt >>= 1;
  const int per_col = len / wdt;
  const int total = cols * per_col;
  for (int i = tid; i < total; i += 256) {
    const int c = i / per_col, k = (i % per_col) * wdt;
    uint8_t* d = dst + (int64_t)c * pitch + k;
    const uint8_t* s = &outs[c][k];
    if (wdt == 16) *reinterpret_cast<uint4*>(d) = *reinterpret_cast<const uint4*>(s);
    else if (wdt == 8) *reinterpret_cast<uint2*>(d) = *reinterpret_cast<const uint2*>(s);
    else if (wdt == 4) *reinterpret_cast<uint32_t*>(d) = *reinterpret_cast<const uint32_t*>(s);
    else if (wdt == 2) *reinterpret_cast<uint16_t*>(d) = *reinterpret_cast<const uint16_t*>(s);
    else *d = *s;
  }
}

// store_staged for a full tile whose runs are LEN bytes (a multiple of 16)
// at a 16-byte aligned offset: every column, 16-byte stores.
template <int LEN>
__device__ __forceinline__ void store_staged_full(const uint8_t (*outs)[OUT_PITCH], uint8_t* dst,
                                                  int64_t pitch, int tid) {
  static_assert(LEN % 16 == 0 && LEN <= OUT_BYTES, "16-byte runs");
  constexpr int PER = LEN / 16;
#pragma unroll
  for (int i = tid; i < CW * PER; i += 256) {
    const int c = i / PER, k = (i % PER) * 16;
    *reinterpret_cast<uint4*>(dst + (int64_t)c * pitch + k) =
        *reinterpret_cast<const uint4*>(&outs[c][k]);
  }
}

// Zero bytes [from, to) of `cols` rows of a K-major operand (K padding);
// nthr threads share the work.
__device__ __forceinline__ void zero_tail(uint8_t* dst, int64_t pitch, int cols, int64_t from,
                                          int64_t to, int tid, int nthr = 256) {
  const int64_t w = to - from;
  if (w <= 0) return;
  for (int64_t i = tid; i < (int64_t)cols * w; i += nthr) dst[(i / w) * pitch + from + i % w] = 0;
}

// Column pass, low-rank rows of H_N (g_w operands).  Thread tid owns column
// c = tid % CW and blocks b = tid / CW + 2t.  MAX: the tile's column maxima ->
// part[0..cols).  QUANT: INT8 codes (reciprocal scale colinv[c], or that of tensor
// list `list` when colinv is null) staged in LDS over the tile (after a
// barrier) and stored K-contiguous at q[(c0 + c) * pitch + t0 / N * R ...].
template <int PASS, int N, int R, class RD>
__device__ __forceinline__ void colpass_lowrank(const TrArgs& a, const RD& rd, uint8_t* smem,
                                                float* red, int rows, int cols, int64_t c0,
                                                const float* colinv, int list, float* part,
                                                uint8_t* q, int64_t pitch, int64_t tl,
                                                int64_t t0, bool last) {
  constexpr int TPT = (TT / N) / 2 > 0 ? (TT / N) / 2 : 1;  // tasks per thread
  constexpr int WPR = (R + 3) / 4;                           // code words per task
  const int tid = threadIdx.x;
  const int c = tid % CW;
  const int nb = rows / N;
  float inv_c = 0.f;
  if constexpr (PASS == PASS_QUANT) {
    const float tinv = colinv ? 0.f : inv_of(__uint_as_float(a.tmax[list]), list == 1 ? 7.f : 127.f);
    inv_c = colinv ? (c < cols ? colinv[c0 + c] : 0.f) : tinv;
  }
  float cm = 0.f;
  uint32_t words[TPT][WPR];
#pragma unroll
  for (int t = 0; t < TPT; ++t) {
#pragma unroll
    for (int w = 0; w < WPR; ++w) words[t][w] = 0;
    const int b = tid / CW + 2 * t;
    if (b < nb && c < cols) {
      float g[R];
      lowrank_col<N, R>(rd, b * N, c, g);
      if constexpr (PASS == PASS_MAX) {
#pragma unroll
        for (int j = 0; j < R; ++j) cm = fmaxf(cm, fabsf(g[j]));
      } else {
#pragma unroll
        for (int j = 0; j < R; ++j)
          words[t][j / 4] |= (quant_bits<127>(g[j], inv_c) & 0xFFu) << (8 * (j % 4));
      }
    }
  }
  if constexpr (PASS == PASS_MAX) {
    tile_colmax_store(cm, red, tid, cols, part);
  } else {
    uint8_t (*outs)[OUT_PITCH] = reinterpret_cast<uint8_t (*)[OUT_PITCH]>(smem);
    __syncthreads();  // every thread is done reading the tile
#pragma unroll
    for (int t = 0; t < TPT; ++t) {
      const int b = tid / CW + 2 * t;
      if (b < nb && c < cols) {
        if constexpr (R >= 4) {
#pragma unroll
          for (int w = 0; w < WPR; ++w)
            *reinterpret_cast<uint32_t*>(&outs[c][b * R + 4 * w]) = words[t][w];
        } else {
#pragma unroll
          for (int j = 0; j < R; ++j) outs[c][b * R + j] = (uint8_t)(words[t][0] >> (8 * j));
        }
      }
    }
    __syncthreads();
    const int64_t koff = t0 / N * R;
    constexpr int LEN = (TT / N) * R;
    if (LEN % 16 == 0 && rows == TT && cols == CW)
      store_staged_full<(LEN % 16 == 0 ? LEN : 16)>(outs, q + c0 * pitch + koff, pitch, tid);
    else
      store_staged(outs, cols, nb * R, q + c0 * pitch + koff, pitch, koff, tid);
    if (last) zero_tail(q + c0 * pitch, pitch, cols, tl, pitch, tid);
  }
}

// Column pass with the full H_N along the rows (w -> INT4 codes for g_x).
template <int PASS, int N, class RD>
__device__ __forceinline__ void colpass_full(const TrArgs& a, const RD& rd, uint8_t* smem,
                                             float* red, int rows, int cols, int64_t c0,
                                             const float* colinv, int list, float* part,
                                             uint8_t* q, int64_t pitch, int64_t o0, int64_t O,
                                             bool last) {
  constexpr int TPT = (TT / N) / 2 > 0 ? (TT / N) / 2 : 1;
  constexpr int WPT = N / 8;  // code words (8 nibbles) per task
  const int tid = threadIdx.x;
  const int c = tid % CW;
  const int nb = rows / N;
  float inv_c = 0.f;
  if constexpr (PASS == PASS_QUANT) {
    const float tinv = colinv ? 0.f : inv_of(__uint_as_float(a.tmax[list]), list == 1 ? 7.f : 127.f);
    inv_c = colinv ? (c < cols ? colinv[c0 + c] : 0.f) : tinv;
  }
  float cm = 0.f;
  uint32_t words[TPT][WPT];
#pragma unroll
  for (int t = 0; t < TPT; ++t) {
#pragma unroll
    for (int w = 0; w < WPT; ++w) words[t][w] = 0;
    const int b = tid / CW + 2 * t;
    if (b < nb && c < cols) {
      float v[N];
      full_col<N>(rd, b * N, c, v);
      if constexpr (PASS == PASS_MAX) {
#pragma unroll
        for (int k = 0; k < N; ++k) cm = fmaxf(cm, fabsf(v[k]));
      } else {
#pragma unroll
        for (int k = 0; k < N; ++k)
          words[t][k / 8] |= (quant_bits<7>(v[k], inv_c) & 0xFu) << (4 * (k % 8));
      }
    }
  }
  if constexpr (PASS == PASS_MAX) {
    tile_colmax_store(cm, red, tid, cols, part);
  } else {
    uint8_t (*outs)[OUT_PITCH] = reinterpret_cast<uint8_t (*)[OUT_PITCH]>(smem);
    __syncthreads();
#pragma unroll
    for (int t = 0; t < TPT; ++t) {
      const int b = tid / CW + 2 * t;
      if (b < nb && c < cols) {
#pragma unroll
        for (int w = 0; w < WPT; ++w)
          *reinterpret_cast<uint32_t*>(&outs[c][b * (N / 2) + 4 * w]) = words[t][w];
      }
    }
    __syncthreads();
    const int64_t koff = o0 / 2;
    if (rows == TT && cols == CW)
      store_staged_full<TT / 2>(outs, q + c0 * pitch + koff, pitch, tid);
    else
      store_staged(outs, cols, rows / 2, q + c0 * pitch + koff, pitch, koff, tid);
    if (last) zero_tail(q + c0 * pitch, pitch, cols, O / 2, pitch, tid);
  }
}

// Cross-lane butterfly stages h = 8, 16, .. N/2 of the row transform (lane
// lc of a 16-lane row holds elements 8 lc .. 8 lc + 7): DPP / swizzle
// exchanges, one fma(+-1, own, partner) per element (the exact IEEE add).
template <int N>
__device__ __forceinline__ void fwht_lanes_dpp(float (&v)[8], int lc) {
  if constexpr (N >= 16) {
    const float sg = (lc & 1) ? -1.f : 1.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = xbfly<1>(v[k], sg);
  }
  if constexpr (N >= 32) {
    const float sg = (lc & 2) ? -1.f : 1.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = xbfly<2>(v[k], sg);
  }
  if constexpr (N >= 64) {
    const float sg = (lc & 4) ? -1.f : 1.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = xbfly<4>(v[k], sg);
  }
  if constexpr (N >= 128) {
    const float sg = (lc & 8) ? -1.f : 1.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = xbfly<8>(v[k], sg);
  }
}

// Row phase of a full bf16 g_y tile (TT rows x CW columns inside T and O):
// the same per-row work as the general loop of tr_job_gy, with tile-uniform
// base pointers and 32-bit lane offsets, no bounds guards, and DPP exchanges.
// 16 bytes of a source tile.  The QUANT pass reads g_y for the last time:
// non-temporal loads keep it from displacing the GEMM operands the pass is
// writing (ViT-B qkv QUANT 25.5 -> 24.5 us, GEMM -0.5 us).
template <bool NT>
__device__ __forceinline__ uint4 ld16(const uint8_t* p) {
  if constexpr (NT) {
    typedef unsigned v4u __attribute__((ext_vector_type(4)));
    const v4u x = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
    return make_uint4(x[0], x[1], x[2], x[3]);
  } else {
    return *reinterpret_cast<const uint4*>(p);
  }
}

template <int PASS, int N>
__device__ __forceinline__ void gy_rows_bf16_full(const TrArgs& a, int64_t t0, int64_t c0,
                                                  int64_t ch, uint8_t* smem, float inv_tensor) {
  constexpr int SW = TT / 16;
  const int tid = threadIdx.x, lr = tid >> 4, lc = tid & 15, col = lc * 8;
  const uint32_t O32 = (uint32_t)a.O;
  const uint8_t* gbase = static_cast<const uint8_t*>(a.gy) + (t0 * a.O + c0) * 2;
  const uint32_t goff = ((uint32_t)lr * O32 + (uint32_t)col) * 2u;
  uint4 raw[SW];
#pragma unroll
  for (int sw = 0; sw < SW; ++sw)
    raw[sw] = ld16<PASS == PASS_QUANT>(gbase + goff + (uint32_t)sw * 32u * O32);
  float inv[SW];
  if constexpr (PASS == PASS_QUANT) {
    const float* ib = a.inv_gy + t0;
#pragma unroll
    for (int sw = 0; sw < SW; ++sw) inv[sw] = a.gx_tok ? ib[sw * 16 + lr] : inv_tensor;
  }
  const uint32_t K32 = (uint32_t)a.kxb;
  uint8_t* qbase = a.q_gy + t0 * a.kxb + c0 / 2;
  const uint32_t qoff = (uint32_t)lr * K32 + (uint32_t)(col / 2);
#pragma unroll
  for (int sw = 0; sw < SW; ++sw) {
    const int row = sw * 16 + lr;
    *reinterpret_cast<uint4*>(smem + (row * P_B16 + col) * 2) = raw[sw];
    float v[8] = {bf16_lo(raw[sw].x), bf16_hi(raw[sw].x), bf16_lo(raw[sw].y), bf16_hi(raw[sw].y),
                  bf16_lo(raw[sw].z), bf16_hi(raw[sw].z), bf16_lo(raw[sw].w), bf16_hi(raw[sw].w)};
    fwht8(v);
    fwht_lanes_dpp<N>(v, lc);
    if constexpr (PASS == PASS_MAX) {
      float m = 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k) m = fmaxf(m, fabsf(v[k]));
      m = fmaxf(m, lane_xor<1>(m));
      m = fmaxf(m, lane_xor<2>(m));
      m = fmaxf(m, lane_xor<4>(m));
      m = fmaxf(m, lane_xor<8>(m));
      if (lc == 0) a.part_gy[ch * a.T + t0 + row] = m;
    } else {
      *reinterpret_cast<uint32_t*>(qbase + qoff + (uint32_t)sw * 16u * K32) =
          quant_pack8_int4(v, inv[sw]);
    }
  }
}

// ---- job: g_y tile (rows along O for g_x, low-rank columns along T for g_w)
template <int PASS, int N, int R, bool F32>
__device__ void tr_job_gy(const TrArgs& a, int64_t bid, uint8_t* smem, float* red) {
  const int tid = threadIdx.x;
  // tile ids and chunk counts fit 32 bits (grids are 32-bit)
  const uint32_t b32 = (uint32_t)bid, n32 = (uint32_t)a.nch_o;
  const int64_t tr = b32 / n32, ch = b32 % n32;
  const int64_t t0 = tr * TT, c0 = ch * CW;
  const int rows = (int)(a.T - t0 < TT ? a.T - t0 : TT);
  const int cols = (int)(a.O - c0 < CW ? a.O - c0 : CW);
  float inv_tensor = 0.f;
  if constexpr (PASS == PASS_QUANT) {
    if (!a.gx_tok) inv_tensor = inv_of(__uint_as_float(a.tmax[0]), 7.f);
  }
  if (!F32 && rows == TT && cols == CW) {
    gy_rows_bf16_full<PASS, N>(a, t0, c0, ch, smem, inv_tensor);
  } else {
  // 16 rows per sweep, 16 lanes x 8 columns per row
  constexpr int SW = TT / 16;
  const int lr = tid >> 4, lc = tid & 15;
  const int col = lc * 8;
  Raw8 raw[SW];
#pragma unroll
  for (int sw = 0; sw < SW; ++sw) {
    const int row = sw * 16 + lr;
    raw[sw].a = make_uint4(0, 0, 0, 0);
    raw[sw].b = make_uint4(0, 0, 0, 0);
    if (row < rows && col < cols) load_raw8(a.gy, a.gy_dt, (t0 + row) * a.O + c0 + col, raw[sw]);
  }
#pragma unroll
  for (int sw = 0; sw < SW; ++sw) {
    const int row = sw * 16 + lr;
    park8<F32>(smem, row, col, raw[sw], a.gy_dt);
    float v[8];
    raw8_to_f32(raw[sw], a.gy_dt, v);
    fwht8(v);
    fwht_lanes_n<N>(v, lc);
    if constexpr (PASS == PASS_MAX) {
      float m = 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k) m = fmaxf(m, fabsf(v[k]));
      m = max_over_16_lanes(m);
      if (lc == 0 && row < rows) a.part_gy[ch * a.T + t0 + row] = m;
    } else if (row < rows) {
      const float inv = a.gx_tok ? a.inv_gy[t0 + row] : inv_tensor;
      // columns past O inside the chunk are zero -> zero codes (K padding)
      *reinterpret_cast<uint32_t*>(a.q_gy + (t0 + row) * a.kxb + (c0 + col) / 2) =
          col < cols ? quant_pack8_int4(v, inv) : 0u;
    }
  }
  }
  __syncthreads();
  const bool last = t0 + rows == a.T;
  if constexpr (F32) {
    RdF32 rd{reinterpret_cast<const float*>(smem)};
    colpass_lowrank<PASS, N, R>(a, rd, smem, red, rows, cols, c0, a.gw_tok ? a.inv_gyl : nullptr,
                                2, a.part_gyl + tr * a.O + c0, a.q_gyl, a.kwb, a.tl, t0, last);
  } else {
    RdB16 rd{reinterpret_cast<const uint16_t*>(smem)};
    colpass_lowrank<PASS, N, R>(a, rd, smem, red, rows, cols, c0, a.gw_tok ? a.inv_gyl : nullptr,
                                2, a.part_gyl + tr * a.O + c0, a.q_gyl, a.kwb, a.tl, t0, last);
  }
}

// ---- MAX pass over g_y tiles held in registers (bf16 g_y, n <= 64)
// One wave per tile of GYR_ROWS = 64 tokens x CW = 128 channels; the four
// waves of a workgroup take four tiles, never wait for each other and finish
// independently.  These workgroups run in the same MAX launch as the x and w
// tiles of the LDS engine.
// Lane c16 = lane & 7 owns channels c0 + 16 c16 .. +15 and row group
// rg = lane >> 3 owns tokens t0 + 8 rg .. +7, loaded once into registers
// (8 tokens x 32 bytes).  A Hadamard block of n
// channels spans n/16 adjacent lanes; a block of n tokens spans n/8 row
// groups of one wave, i.e. lanes 8 apart.  Nothing goes through LDS:
//   * along O (g_x operand A): per token, stages h = 1..8 in-lane, stages
//     h >= 16 across lanes c16 ^ h/16 (DPP quad permutes);
//   * along T (g_w operand): per channel, stages h = 1, 2, 4 over the lane's
//     8 tokens, stages h = 8, 16, 32 across lanes 8, 16, 32 apart.
// The low-rank rows are the butterfly network pruned to its surviving
// entries: stages with h < n/r keep only a + b (the pairwise-tree group sums),
// the later stages are full butterflies over the group sums (H_r), all in
// ascending h as the full transform runs them.
constexpr int GYR_ROWS = TR_GY_REG_ROWS;

// max |v[i]| over 16 values with three-input maxima
__device__ __forceinline__ float absmax16(const float (&v)[16]) {
  float m = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fabsf(v[2]));
#pragma unroll
  for (int i = 3; i < 15; i += 2) m = fmaxf(fmaxf(m, fabsf(v[i])), fabsf(v[i + 1]));
  return fmaxf(m, fabsf(v[15]));
}

// Registers of one tile (zero outside T and O).
__device__ __forceinline__ void gyr_load(const TrArgs& a, int64_t bid, uint4 (&raw)[8][2]) {
  const int lane = threadIdx.x & 63;
  // tile ids and chunk counts fit 32 bits (grids are 32-bit)
  const uint32_t b32 = (uint32_t)bid, n32 = (uint32_t)a.nch_o;
  const int64_t tr = b32 / n32, ch = b32 % n32;
  const int64_t t0 = tr * GYR_ROWS, c0 = ch * CW;
  const int rows = (int)(a.T - t0 < GYR_ROWS ? a.T - t0 : GYR_ROWS);
  const int cols = (int)(a.O - c0 < CW ? a.O - c0 : CW);
  const int col = (lane & 7) * 16, r0 = (lane >> 3) * 8;
  const bool ok = r0 < rows && col < cols;
  const uint16_t* gy = static_cast<const uint16_t*>(a.gy);
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    raw[k][0] = make_uint4(0, 0, 0, 0);
    raw[k][1] = make_uint4(0, 0, 0, 0);
    if (ok) {
      const uint4* src = reinterpret_cast<const uint4*>(gy + (t0 + r0 + k) * a.O + c0 + col);
      raw[k][0] = src[0];
      raw[k][1] = src[1];
    }
  }
}

// Maxima of one tile: row maxima of H.g_y along O -> part_gy[ch][t], column
// maxima of the low-rank g_y along T -> part_gyl[tr][o].
template <int N, int R>
__device__ __forceinline__ void gyr_tile_max(const TrArgs& a, int64_t bid,
                                             const uint4 (&raw)[8][2]) {
  static_assert(N >= 16 && N <= 64, "a token block spans 2..8 row groups of one wave");
  constexpr int G = N / R;             // tokens per low-rank group
  constexpr int GL = G < 8 ? G : 8;    // in-lane span of a group
  constexpr int RGB = N / 8;           // row groups per token block
  const int lane = threadIdx.x & 63;
  const int c16 = lane & 7, rg = lane >> 3;
  // tile ids and chunk counts fit 32 bits (grids are 32-bit)
  const uint32_t b32 = (uint32_t)bid, n32 = (uint32_t)a.nch_o;
  const int64_t tr = b32 / n32, ch = b32 % n32;
  const int64_t t0 = tr * GYR_ROWS, c0 = ch * CW;
  const int rows = (int)(a.T - t0 < GYR_ROWS ? a.T - t0 : GYR_ROWS);
  const int cols = (int)(a.O - c0 < CW ? a.O - c0 : CW);
  const int col = c16 * 16;
  const int r0 = rg * 8;               // first token of this lane in the tile
  const bool act = r0 < rows;          // rows is a multiple of n >= 16
  const bool cact = col < cols;        // cols is a multiple of n >= 16

  // ---- along O: one token per iteration
  const float sgn1 = (c16 & 1) ? -1.f : 1.f, sgn2 = (c16 & 2) ? -1.f : 1.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    float v[16];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      v[8 * q + 0] = bf16_lo(raw[k][q].x); v[8 * q + 1] = bf16_hi(raw[k][q].x);
      v[8 * q + 2] = bf16_lo(raw[k][q].y); v[8 * q + 3] = bf16_hi(raw[k][q].y);
      v[8 * q + 4] = bf16_lo(raw[k][q].z); v[8 * q + 5] = bf16_hi(raw[k][q].z);
      v[8 * q + 6] = bf16_lo(raw[k][q].w); v[8 * q + 7] = bf16_hi(raw[k][q].w);
    }
#pragma unroll
    for (int h = 1; h < 16; h <<= 1)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if ((e & h) == 0) {
          const float p = v[e], q = v[e + h];
          v[e] = p + q;
          v[e + h] = p - q;
        }
    if constexpr (N >= 32) {
#pragma unroll
      for (int e = 0; e < 16; ++e) v[e] = xbfly<1>(v[e], sgn1);
    }
    if constexpr (N >= 64) {
#pragma unroll
      for (int e = 0; e < 16; ++e) v[e] = xbfly<2>(v[e], sgn2);
    }
    const float m = group8_max(absmax16(v));
    if (c16 == 0 && act) a.part_gy[ch * a.T + t0 + r0 + k] = m;
  }

  // ---- along T: one channel per iteration
  const int rib = rg % RGB;                                  // row group inside its block
  const bool owner = (G <= 8) || (rib % (G / 8) == 0);       // holds surviving entries
  const float sg8 = (rib & 1) ? -1.f : 1.f, sg16 = (rib & 2) ? -1.f : 1.f;
  const float sg32 = (rib & 4) ? -1.f : 1.f;
  float cmax[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    float x[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint4& w4 = raw[k][j / 8];
      const int jj = j % 8;
      const uint32_t w = jj < 2 ? w4.x : jj < 4 ? w4.y : jj < 6 ? w4.z : w4.w;
      x[k] = (jj & 1) ? bf16_hi(w) : bf16_lo(w);
    }
#pragma unroll
    for (int h = 1; h < 8; h <<= 1) {
      if (h < G) {  // group sums: pairwise tree
#pragma unroll
        for (int k = 0; k < 8; k += 2 * h) x[k] = x[k] + x[k + h];
      } else {      // full butterflies over the surviving group sums
#pragma unroll
        for (int k = 0; k < 8; ++k)
          if ((k & h) == 0 && k % G == 0) {
            const float p = x[k], q = x[k + h];
            x[k] = p + q;
            x[k + h] = p - q;
          }
      }
    }
    if constexpr (N >= 16) {
#pragma unroll
      for (int k = 0; k < 8; k += GL) x[k] = (8 < G) ? x[k] + lane_xor<8>(x[k]) : xbfly<8>(x[k], sg8);
    }
    if constexpr (N >= 32) {
#pragma unroll
      for (int k = 0; k < 8; k += GL) x[k] = (16 < G) ? x[k] + lane_xor<16>(x[k]) : xbfly<16>(x[k], sg16);
    }
    if constexpr (N >= 64) {
#pragma unroll
      for (int k = 0; k < 8; k += GL) x[k] = (32 < G) ? x[k] + lane_xor<32>(x[k]) : xbfly<32>(x[k], sg32);
    }
    float m = 0.f;
#pragma unroll
    for (int k = 0; k < 8; k += GL) m = fmaxf(m, fabsf(x[k]));
    cmax[j] = owner && act && cact ? m : 0.f;
  }
  // fold the eight row groups (lanes 8, 16, 32 apart)
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    float m = cmax[j];
    m = fmaxf(m, lane_xor<8>(m));
    m = fmaxf(m, lane_xor<16>(m));
    m = fmaxf(m, lane_xor<32>(m));
    cmax[j] = m;
  }
  if (lane < 8 && cact) {
#pragma unroll
    for (int j = 0; j < 16; ++j) a.part_gyl[tr * a.O + c0 + col + j] = cmax[j];
  }
}

// ---- job: x tile (ACBP codes, low-rank columns along T for g_w)
template <int PASS, int N, int R>
__device__ void tr_job_x(const TrArgs& a, int64_t bid, uint8_t* smem, float* red) {
  const int tid = threadIdx.x;
  // tile ids and chunk counts fit 32 bits (grids are 32-bit)
  const uint32_t b32 = (uint32_t)bid, n32 = (uint32_t)a.nch_i;
  const int64_t tr = b32 / n32, ch = b32 % n32;
  const int64_t t0 = tr * TT, c0 = ch * CW;
  const int rows = (int)(a.T - t0 < TT ? a.T - t0 : TT);
  const int cols = (int)(a.I - c0 < CW ? a.I - c0 : CW);
  uint8_t* codes = smem;                                          // [TT][P_I4] bytes
  float* scales = reinterpret_cast<float*>(smem + TT * P_I4);     // [TT]
  // 64 code bytes per tile row: 4 lanes x 16 bytes, 64 rows per sweep.  Rows
  // are I/2 bytes (a multiple of 4, not of 16), so the loads are dwords.
  constexpr int SW = TT / 64;
  const int lr = tid >> 2, lq = tid & 3;
  const int col = lq * 32;
  uint32_t w4[SW][4];
#pragma unroll
  for (int sw = 0; sw < SW; ++sw) {
    const int row = sw * 64 + lr;
#pragma unroll
    for (int d = 0; d < 4; ++d) w4[sw][d] = 0u;
    if (row < rows && col < cols) {
      const uint32_t* src =
          reinterpret_cast<const uint32_t*>(a.xc + (t0 + row) * (a.I / 2) + (c0 + col) / 2);
#pragma unroll
      for (int d = 0; d < 4; ++d)
        if (col + 8 * d < cols) w4[sw][d] = src[d];
    }
  }
  if (tid < TT) scales[tid] = tid < rows ? a.xs[t0 + tid] : 0.f;
#pragma unroll
  for (int sw = 0; sw < SW; ++sw)
    *reinterpret_cast<uint4*>(codes + (sw * 64 + lr) * P_I4 + col / 2) =
        make_uint4(w4[sw][0], w4[sw][1], w4[sw][2], w4[sw][3]);
  __syncthreads();
  RdI4 rd{codes, scales};
  colpass_lowrank<PASS, N, R>(a, rd, smem, red, rows, cols, c0, a.gw_tok ? a.inv_xl : nullptr, 3,
                              a.part_xl + tr * a.I + c0, a.q_xl, a.kwb, a.tl, t0,
                              t0 + rows == a.T);
}

// ---- job: w tile (full H_N along O, INT4 stored transposed for g_x)
template <int PASS, int N, bool F32>
__device__ void tr_job_w(const TrArgs& a, int64_t bid, uint8_t* smem, float* red) {
  const int tid = threadIdx.x;
  // tile ids and chunk counts fit 32 bits (grids are 32-bit)
  const uint32_t b32 = (uint32_t)bid, n32 = (uint32_t)a.nch_i;
  const int64_t tr = b32 / n32, ch = b32 % n32;
  const int64_t o0 = tr * TT, c0 = ch * CW;
  const int rows = (int)(a.O - o0 < TT ? a.O - o0 : TT);
  const int cols = (int)(a.I - c0 < CW ? a.I - c0 : CW);
  constexpr int SW = TT / 16;
  const int lr = tid >> 4, lc = tid & 15;
  const int col = lc * 8;
  Raw8 raw[SW];
#pragma unroll
  for (int sw = 0; sw < SW; ++sw) {
    const int row = sw * 16 + lr;
    raw[sw].a = make_uint4(0, 0, 0, 0);
    raw[sw].b = make_uint4(0, 0, 0, 0);
    if (row < rows && col < cols) load_raw8(a.w, a.w_dt, (o0 + row) * a.I + c0 + col, raw[sw]);
  }
#pragma unroll
  for (int sw = 0; sw < SW; ++sw) park8<F32>(smem, sw * 16 + lr, col, raw[sw], a.w_dt);
  __syncthreads();
  const bool last = o0 + rows == a.O;
  if constexpr (F32) {
    RdF32 rd{reinterpret_cast<const float*>(smem)};
    colpass_full<PASS, N>(a, rd, smem, red, rows, cols, c0, a.gx_tok ? a.inv_w : nullptr, 1,
                          a.part_w + tr * a.I + c0, a.q_w, a.kxb, o0, a.O, last);
  } else {
    RdB16 rd{reinterpret_cast<const uint16_t*>(smem)};
    colpass_full<PASS, N>(a, rd, smem, red, rows, cols, c0, a.gx_tok ? a.inv_w : nullptr, 1,
                          a.part_w + tr * a.I + c0, a.q_w, a.kxb, o0, a.O, last);
  }
}

// F32: the g_y / w tiles hold fp32 (any fp32 source); otherwise bf16.
template <int PASS, int N, int R, bool F32>
__global__ __launch_bounds__(256) void k_tr(TrArgs a) {
  static_assert(TT * P_I4 + TT * 4 <= TileSmem<F32>::bytes, "x tile fits the smem buffer");
  static_assert(CW * OUT_PITCH <= TileSmem<F32>::bytes, "staging fits the smem buffer");
  __shared__ __attribute__((aligned(16))) uint8_t smem[TileSmem<F32>::bytes];
  __shared__ float red[4 * CW];
  if (blockIdx.x == 0 && threadIdx.x < 4) {
    if constexpr (PASS == PASS_MAX) {
      a.tmax[threadIdx.x] = 0u;  // k_tr_reduce folds into it
    } else {  // tensor scales of the per-tensor modes
      const int l = threadIdx.x;
      const float qmax = l < 2 ? 7.f : 127.f;
      if (l < 2 ? !a.gx_tok : !a.gw_tok) {
        float* sc = l == 0 ? a.s_gy : l == 1 ? a.s_w : l == 2 ? a.s_gyl : a.s_xl;
        sc[0] = scale_of(__uint_as_float(a.tmax[l]), qmax);
      }
    }
  }
  // Workgroup -> job: consecutive ids go to the 8 XCDs in turn; slot s of an
  // XCD walks that XCD's eighth of each job list in the order register g_y,
  // LDS g_y, x, w (longest tiles first).  Every XCD gets the same mix of
  // jobs, and within a job list a contiguous range of tiles.
  const int64_t xcd = blockIdx.x % 8;
  int64_t slot = blockIdx.x / 8;
  const int64_t per_r = (a.gyreg_wgs + 7) / 8, per_g = (a.gy_workers + 7) / 8;
  const int64_t per_x = (a.wg_x + 7) / 8, per_w = (a.wg_w + 7) / 8;
  if constexpr (PASS == PASS_MAX && N <= 64) {
    // register-resident g_y tiles: four independent waves, one tile each
    if (slot < per_r) {
      const int64_t bid = xcd * per_r + slot;
      const int64_t tile = bid * 4 + (threadIdx.x >> 6);
      if (bid < a.gyreg_wgs && tile < a.wg_gy) {
        uint4 raw[8][2];
        gyr_load(a, tile, raw);
        gyr_tile_max<N, R>(a, tile, raw);
      }
      return;
    }
  }
  slot -= per_r;
  if (slot < per_g) {  // g_y tiles on the LDS engine
    const int64_t bid = xcd * per_g + slot;
    if (bid < a.gy_workers) tr_job_gy<PASS, N, R, F32>(a, bid, smem, red);
    return;
  }
  slot -= per_g;
  if (slot < per_x) {
    const int64_t bid = xcd * per_x + slot;
    if (bid < a.wg_x) tr_job_x<PASS, N, R>(a, bid, smem, red);
    return;
  }
  slot -= per_x;
  if (slot < per_w) {
    const int64_t bid = xcd * per_w + slot;
    if (bid < a.wg_w) tr_job_w<PASS, N, F32>(a, bid, smem, red);
  }
}

// Fold the partial maxima.  Entry e of each list takes the max over its
// partials; per-token modes store its scale and reciprocal scale (the QUANT
// pass multiplies by the latter).  Every block folds its per-list maxima into
// the four tensor maxima with one atomicMax each (lists: 0 H.g_y rows, 1 H.w
// columns, 2 low-rank g_y columns, 3 low-rank x columns).  Max is exact and
// commutes, so the result does not depend on the schedule.  A block covers 64 consecutive entries; its 16
// waves split each entry's partials (stride 16) so every wave keeps several
// loads in flight.
constexpr int RED_ENTRIES = TR_RED_ENTRIES;
constexpr int RED_WAVES = 16;

__global__ __launch_bounds__(64 * RED_WAVES) void k_tr_reduce(TrArgs a) {
  __shared__ float wpart[RED_WAVES][RED_ENTRIES];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t e = (int64_t)blockIdx.x * RED_ENTRIES + lane;
  const int64_t n0 = a.T, n1 = n0 + a.O, n2 = n1 + a.I, n3 = n2 + a.I;
  const float* p = nullptr;
  int64_t np = 0, stride = 0;
  int list = -1;
  if (e < n0) { list = 0; p = a.part_gy + e; np = a.nch_o; stride = a.T; }
  else if (e < n1) { list = 2; p = a.part_gyl + (e - n0); np = a.ntr_gy; stride = a.O; }
  else if (e < n2) { list = 3; p = a.part_xl + (e - n1); np = a.ntr_t; stride = a.I; }
  else if (e < n3) { list = 1; p = a.part_w + (e - n2); np = a.ntr_o; stride = a.I; }
  // wave wv folds partials wv, wv + 16, ...; four loads in flight per step
  float m0 = 0.f, m1 = 0.f, m2 = 0.f, m3 = 0.f;
  int64_t k = wv;
  constexpr int W = RED_WAVES;
  for (; k + 3 * W < np; k += 4 * W) {
    m0 = fmaxf(m0, p[k * stride]);
    m1 = fmaxf(m1, p[(k + W) * stride]);
    m2 = fmaxf(m2, p[(k + 2 * W) * stride]);
    m3 = fmaxf(m3, p[(k + 3 * W) * stride]);
  }
  for (; k < np; k += W) m0 = fmaxf(m0, p[k * stride]);
  wpart[wv][lane] = fmaxf(fmaxf(m0, m1), fmaxf(m2, m3));
  __syncthreads();
  if (wv == 0) {
  float m = wpart[0][lane];
#pragma unroll
  for (int q = 1; q < RED_WAVES; ++q) m = fmaxf(m, wpart[q][lane]);
  if (list == 0) {
    if (a.gx_tok) { a.inv_gy[e] = inv_of(m, 7.f); a.s_gy[e] = scale_of(m, 7.f); }
  } else if (list == 2) {
    if (a.gw_tok) { a.inv_gyl[e - n0] = inv_of(m, 127.f); a.s_gyl[e - n0] = scale_of(m, 127.f); }
  } else if (list == 3) {
    if (a.gw_tok) { a.inv_xl[e - n1] = inv_of(m, 127.f); a.s_xl[e - n1] = scale_of(m, 127.f); }
  } else if (list == 1) {
    if (a.gx_tok) { a.inv_w[e - n2] = inv_of(m, 7.f); a.s_w[e - n2] = scale_of(m, 7.f); }
  }
#pragma unroll
  for (int l = 0; l < 4; ++l) {
    // tensor maxima: max over blocks by atomicMax on the bit patterns of
    // non-negative floats (they order like the values), exact and
    // schedule-independent; zeroed by the MAX pass
    const float v = wave_max(list == l ? m : 0.f);
    if (lane == 0 && v > 0.f) atomicMax(a.tmax + l, __float_as_uint(v));
  }
  }
}

// ------------------------------------------------------------ integer GEMM
// C[m][n] = sum_k A[m][k] * B[n][k]; A [M][pitch], B [N][pitch] bytes, K
// contiguous and zero-padded to a multiple of the stage depth KB.  INT4
// operands hold two codes per byte and stay packed in HBM, L2 and LDS; each
// 16-byte fragment is widened on the LDS->register path into two int8
// fragments holding 16*code (low nibble shifted up, high nibble masked in
// place), so the INT32 sum is 256 times the code product sum and is shifted
// back exactly.  Both operands are widened the same way, so the nibble order
// inside a lane leaves the dot product unchanged.
//
// Matrix core: v_mfma_i32_32x32x32_i8 (32 cycles of the matrix pipe for a
// 32x32x32 product; the 16x16x64 form needs more independent accumulators
// than a wave has to stay busy).  Operand X holds 32 rows of A, operand Y 32
// rows of B; lane l feeds row l%32 with 16 consecutive K bytes of half l/32.
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

__device__ __forceinline__ void widen_int4x2(u32x4 p, v4i& a, v4i& b) {
  a[0] = (int)((p[0] << 4) & 0xF0F0F0F0u); a[1] = (int)(p[0] & 0xF0F0F0F0u);
  a[2] = (int)((p[1] << 4) & 0xF0F0F0F0u); a[3] = (int)(p[1] & 0xF0F0F0F0u);
  b[0] = (int)((p[2] << 4) & 0xF0F0F0F0u); b[1] = (int)(p[2] & 0xF0F0F0F0u);
  b[2] = (int)((p[3] << 4) & 0xF0F0F0F0u); b[3] = (int)(p[3] & 0xF0F0F0F0u);
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

// 16 bytes per lane from global memory into LDS run l (lane i -> l + 16 i).
__device__ __forceinline__ void lds_dma16(const uint8_t* g, uint8_t* l) {
  __builtin_amdgcn_global_load_lds(g, l, 16, 0, 0);
}

// Physical 16-byte chunk slot of logical chunk 0 in row r (XOR with it).
// Depends on r & 15 only, so fragment bases (multiples of 32 rows) keep it.
template <int KB>
__device__ __forceinline__ int chunk_swz(int r) {
  if constexpr (KB == 128) return (r & 7) ^ ((r >> 3) & 1);
  else return (r >> 2) & 3;
}

template <bool INT4, int BM, int BN, int KB, int NS>
struct GemmShape {
  static constexpr int WTM = BM / 2, WTN = BN / 2, FM = WTM / 32, FN = WTN / 32;
  static constexpr int CPR = KB / 16;                              // chunks per row
  static constexpr int IA = BM * CPR / 256, IB = BN * CPR / 256;   // DMA ops per wave
  static constexpr int IPW = IA + IB;
  static constexpr int STAGE = (BM + BN) * KB;
  static constexpr int KK = KB / 32;                               // k-steps per stage
  static_assert(FM >= 1 && FN >= 1, "wave tile smaller than one MFMA tile");
  static_assert(IA * 256 == BM * CPR && IB * 256 == BN * CPR, "stage load split");
  static_assert(KK % 2 == 0, "fragment slots alternate per k-step");
  static_assert(KB == 64 || KB == 128, "swizzle covers 4 or 8 chunks per row");
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
};

// One output tile (workgroup w of the tile grid, K split `split`) of one GEMM.
// Every thread of the workgroup calls it; `lds` holds NS * STAGE bytes.
template <bool INT4, int BM, int BN, int KB, int NS, int EPI>
__device__ __forceinline__ void gemm_tile(const GemmArgs& g, int64_t w, int64_t split,
                                          uint8_t* lds, float* sc) {
  using G = GemmShape<INT4, BM, BN, KB, NS>;
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
  const int wm = wave >> 1, wn = wave & 1;
  int64_t tm, tn;
  if (!xcd_tile(w, (M + BM - 1) / BM, (N + BN - 1) / BN, tm, tn)) return;
  const int64_t m0 = tm * BM, n0 = tn * BN;
  const int64_t s_first = split * sps;
  const int64_t S = (S_total - s_first < sps ? S_total - s_first : sps);  // >= 1 by plan
  const int64_t kbase = s_first * KB;

  // DMA sources of this lane for stage 0 (rows past M / N re-read the last row)
  const uint8_t* src[IPW];
#pragma unroll
  for (int j = 0; j < IA; ++j) {
    const int slot = (wave * IA + j) * 64 + lane;
    const int row = slot / CPR, c = (slot % CPR) ^ chunk_swz<KB>(row);
    const int64_t r = m0 + row < M ? m0 + row : M - 1;
    src[j] = A + r * pitch + kbase + c * 16;
  }
#pragma unroll
  for (int j = 0; j < IB; ++j) {
    const int slot = (wave * IB + j) * 64 + lane;
    const int row = slot / CPR, c = (slot % CPR) ^ chunk_swz<KB>(row);
    const int64_t r = n0 + row < N ? n0 + row : N - 1;
    src[IA + j] = B + r * pitch + kbase + c * 16;
  }
#define HLQ_GEMM_ISSUE(st, bf)                                                           \
  do {                                                                                   \
    uint8_t* base_ = lds + (bf) * G::STAGE;                                              \
    for (int j = 0; j < IA; ++j) lds_dma16(src[j] + (st) * KB, base_ + (wave * IA + j) * 1024); \
    for (int j = 0; j < IB; ++j)                                                         \
      lds_dma16(src[IA + j] + (st) * KB, base_ + BM * KB + (wave * IB + j) * 1024);      \
  } while (0)
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

  // Dequantization scales of the tile's rows (times alpha) and columns, read
  // before the K loop and parked in LDS (sc, an array of its own, so the
  // ring's DMA does not order its accesses): the epilogue then waits on no
  // global load while its stores are in flight.
  constexpr int NSC = (BM + BN + 255) / 256;
  float scv[NSC];
  if constexpr (EPI == EPI_F32) {
#pragma unroll
    for (int q = 0; q < NSC; ++q) {
      // one unconditional load per slot (a select of the address, so the
      // loaded value is not merged across branches, which would wait on it)
      const int i = tid + 256 * q;
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

  v16i acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0;

  u32x4 fa[2][FM], fb[2][FN];
  HLQ_GEMM_WAIT((S - 1 < NS - 1 ? S - 1 : NS - 1));
  if constexpr (EPI == EPI_F32) {
#pragma unroll
    for (int q = 0; q < NSC; ++q)
      if (tid + 256 * q < BM + BN) sc[tid + 256 * q] = tid + 256 * q < BM ? scv[q] * alpha : scv[q];
  }
  asm volatile("s_barrier" ::: "memory");
#pragma unroll
  for (int i = 0; i < FM; ++i)
    fa[0][i] = *reinterpret_cast<const u32x4*>(lds + a_off + i * 32 * KB + coff[0]);
#pragma unroll
  for (int j = 0; j < FN; ++j)
    fb[0][j] = *reinterpret_cast<const u32x4*>(lds + b_off + j * 32 * KB + coff[0]);

  // One K stage.  MODE 0: steady state (refill a buffer, prefetch the next
  // stage's first fragments); 1: the last NS-1 stages but one (prefetch, no
  // refill); 2: the last stage.  Separate bodies keep each stage one block
  // of straight-line code for the scheduler.
  int buf = 0;
  auto stage = [&](int64_t st, auto mode_tag) {
    constexpr int MODE = decltype(mode_tag)::value;
    const uint8_t* base = lds + buf * G::STAGE;
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
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
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
      if constexpr (INT4) {
        v4i xa0[FM], xa1[FM], yb0[FN], yb1[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i) widen_int4x2(fa[cur][i], xa0[i], xa1[i]);
#pragma unroll
        for (int j = 0; j < FN; ++j) widen_int4x2(fb[cur][j], yb0[j], yb1[j]);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(xa0[i], yb0[j], acc[i][j], 0, 0, 0);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(xa1[i], yb1[j], acc[i][j], 0, 0, 0);
        // INT4: the compiler's own interleaving of reads, widening and MFMAs
        // (explicit groups measured no better: fc2 pair 52.5 vs 51 us)
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
  };
  int64_t st = 0;
  for (; st + NS < S; ++st) stage(st, std::integral_constant<int, 0>());
  for (; st + 1 < S; ++st) stage(st, std::integral_constant<int, 1>());
  stage(st, std::integral_constant<int, 2>());  // S >= 1
#undef HLQ_GEMM_ISSUE
#undef HLQ_GEMM_WAIT

  constexpr int SH = INT4 ? 8 : 0;
  int32_t* Cp = Ci + (EPI == EPI_PARTIAL ? split * M * N : 0);
  // Scales from LDS (written before the K loop; its barriers published them).
  float s_n[FN], s_m[FM][16];
  if constexpr (EPI == EPI_F32) {
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
          const int32_t v = acc[i][j][r] >> SH;
          if constexpr (EPI == EPI_F32) __builtin_nontemporal_store((float)v * s_m[i][r] * s_n[j], &C[m * N + n]);
          else Cp[m * N + n] = v;
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
        const int32_t v = acc[i][j][r] >> SH;
        if constexpr (EPI == EPI_F32) __builtin_nontemporal_store((float)v * s_m[i][r] * s_n[j], &C[m * N + n]);
        else Cp[m * N + n] = v;
      }
  }
}

template <bool INT4, int BM, int BN, int KB, int NS, int EPI>
__global__ __launch_bounds__(256, 2) void k_gemm(GemmArgs g) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[NS * GemmShape<INT4, BM, BN, KB, NS>::STAGE];
  __shared__ float sc[BM + BN];
  gemm_tile<INT4, BM, BN, KB, NS, EPI>(g, blockIdx.x, blockIdx.y, lds, sc);
}

// Both GEMMs of the backward in one launch (fp32 epilogues, no split-K): the
// first n1 workgroups take the g_w tiles (longer K, so they start first), the
// rest the g_x tiles, which fill the CUs around them.  One launch instead of
// two plus a split-K pass, and neither GEMM's tail leaves the GPU idle.
template <int BM1, int BN1, int KB1, int NS1, int BM0, int BN0, int KB0, int NS0>
__global__ __launch_bounds__(256, 2) void k_gemm_pair(GemmArgs gw, int64_t n1, GemmArgs gx) {
  constexpr int L1 = NS1 * GemmShape<false, BM1, BN1, KB1, NS1>::STAGE;
  constexpr int L0 = NS0 * GemmShape<true, BM0, BN0, KB0, NS0>::STAGE;
  constexpr int SC = BM1 + BN1 > BM0 + BN0 ? BM1 + BN1 : BM0 + BN0;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[L1 > L0 ? L1 : L0];
  __shared__ float sc[SC];
  const int64_t b = blockIdx.x;
  if (b < n1) gemm_tile<false, BM1, BN1, KB1, NS1, EPI_F32>(gw, b, 0, lds, sc);
  else gemm_tile<true, BM0, BN0, KB0, NS0, EPI_F32>(gx, b - n1, 0, lds, sc);
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

// ------------------------------------------------------------ LQS statistics
// Layer-wise quantizer selection ("HOT: Hadamard-based Optimized Training",
// abstract; scime.ai summary, "Approach" and "Limitations": per-token or
// per-tensor chosen per layer from calibration data with a 50% MSE-difference
// threshold).  For each of the four operands the backward quantizes, the
// squared reconstruction error under per-token and under per-tensor scales,
// with sum(v^2) and the element count.  The group maxima, per-token scales,
// reciprocal scales and tensor maxima come from the backward's own MAX and
// reduce launches (both paths per token); this ERR pass then recomputes the
// transformed values.  One thread (one lane) transforms one block of n values:
//   op 0  H.g_y          row t, block beta along O      group: token t
//   op 1  H.w            column i, block beta along O   group: input channel i
//   op 2  low-rank g_y   column o, token block b        group: channel o
//   op 3  low-rank x     column i, token block b        group: channel i
// with the fp32 butterfly network of the backward (ascending stages); the
// low-rank operands keep outputs j * (n / r).  Calibration work, not the
// backward's hot path.

template <int N>
__device__ __forceinline__ void fwht_reg(float (&v)[N]) {
#pragma unroll
  for (int h = 1; h < N; h <<= 1)
#pragma unroll
    for (int k = 0; k < N; ++k)
      if ((k & h) == 0) {
        const float p = v[k], q = v[k + h];
        v[k] = p + q;
        v[k + h] = p - q;
      }
}

// Quantizer of a group: scale s and reciprocal scale inv (0 for a group whose
// codes are all 0: a zero group, or qmax / a overflowing).
struct LqsQuant {
  float inv, s, qmax;
};

// fl(v - fl(s * q)) with q = clamp(rne(fl(v * inv)), +-qmax).
__device__ __forceinline__ float lqs_err(float v, const LqsQuant& z) {
  const float q = fminf(fmaxf(rintf(v * z.inv), -z.qmax), z.qmax);
  const float d = z.s * q;
  return v - d;
}

// Element e of a uniform base pointer through a 32-bit byte offset (the host
// keeps every input below 4 GiB): one VGPR per address, no 64-bit adds.
__device__ __forceinline__ float ld_off(const void* base, int dt, uint32_t e) {
  const char* b = static_cast<const char*>(base);
  if (dt == 0) return *reinterpret_cast<const float*>(b + (e << 2));
  return bf16_to_f32(*reinterpret_cast<const uint16_t*>(b + (e << 1)));
}

// Row operand (op 0, H.g_y): a thread takes LQS_ROW_BLOCKS(N) blocks of n
// values of token rows (blocks tid and tid + 256 of its workgroup's range, so
// each load instruction of a wave reads contiguous bytes), every load issued
// before the arithmetic; 16-byte loads.
template <int N>
__global__ __launch_bounds__(256) void k_lqs_rows(LqsArgs a) {
  constexpr int RPT = lqs_row_blocks(N);
  __shared__ double red[3][256];
  const int tid = threadIdx.x;
  const int64_t b = blockIdx.x;
  const uint32_t O = (uint32_t)a.O;
  const char* base = static_cast<const char*>(a.gy);
  double ss = 0.0, e_tok = 0.0, e_ten = 0.0;
  float v[RPT][N];
  uint32_t tq[RPT];
  bool ok[RPT];
#pragma unroll
  for (int q = 0; q < RPT; ++q) {
    const uint32_t item = (uint32_t)((b * RPT + q) * 256 + tid);
    ok[q] = item < (uint32_t)a.items[0];
    tq[q] = item / (O / N);
    if (!ok[q]) continue;
    const uint32_t e0 = tq[q] * O + item % (O / N) * N;
#pragma unroll
    for (int k = 0; k < N; k += 8) {
      if (a.gy_dt == 0) {
        const float4* p = reinterpret_cast<const float4*>(base + ((e0 + k) << 2));
        const float4 x0 = p[0], x1 = p[1];
        v[q][k] = x0.x; v[q][k + 1] = x0.y; v[q][k + 2] = x0.z; v[q][k + 3] = x0.w;
        v[q][k + 4] = x1.x; v[q][k + 5] = x1.y; v[q][k + 6] = x1.z; v[q][k + 7] = x1.w;
      } else {
        const uint4 u = *reinterpret_cast<const uint4*>(base + ((e0 + k) << 1));
        v[q][k] = bf16_to_f32(u.x & 0xFFFFu); v[q][k + 1] = bf16_to_f32(u.x >> 16);
        v[q][k + 2] = bf16_to_f32(u.y & 0xFFFFu); v[q][k + 3] = bf16_to_f32(u.y >> 16);
        v[q][k + 4] = bf16_to_f32(u.z & 0xFFFFu); v[q][k + 5] = bf16_to_f32(u.z >> 16);
        v[q][k + 6] = bf16_to_f32(u.w & 0xFFFFu); v[q][k + 7] = bf16_to_f32(u.w >> 16);
      }
    }
  }
  const float at = __uint_as_float(a.tmax[0]);
  const LqsQuant zT{inv_of(at, 7.f), scale_of(at, 7.f), 7.f};
#pragma unroll
  for (int q = 0; q < RPT; ++q) {
    if (!ok[q]) continue;
    const LqsQuant zt{a.tok_inv[0][tq[q]], a.tok_s[0][tq[q]], 7.f};
    fwht_reg<N>(v[q]);
#pragma unroll
    for (int k = 0; k < N; ++k) {
      const float x = v[q][k];
      const float d1 = lqs_err(x, zt), d2 = lqs_err(x, zT);
      ss += (double)x * (double)x;
      e_tok += (double)d1 * (double)d1;
      e_ten += (double)d2 * (double)d2;
    }
  }
  red[0][tid] = ss;
  red[1][tid] = e_tok;
  red[2][tid] = e_ten;
  __syncthreads();
  for (int h = 128; h > 0; h >>= 1) {  // fixed order: the sums are reproducible
    if (tid < h) {
      red[0][tid] += red[0][tid + h];
      red[1][tid] += red[1][tid + h];
      red[2][tid] += red[2][tid + h];
    }
    __syncthreads();
  }
  if (tid < 3) a.part[b * 3 + tid] = red[tid][0];
}

// Column operands (op 1 H.w, op 2 low-rank g_y, op 3 low-rank x): one wave
// per workgroup, 64 columns and a strip of LQS_STRIP blocks.  Each block of n
// rows x 64 columns is staged in LDS in its source form with 16-byte (bf16,
// fp32) or 4-byte (ACBP codes) loads, whole pieces of a row since I and O are
// multiples of 8; then lane c transforms column c from LDS.
template <int N>
__global__ __launch_bounds__(64) void k_lqs_cols(LqsArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[N * 256];
  __shared__ float tsc[N];
  const int lane = threadIdx.x;
  const int64_t g = a.wg0[1] + blockIdx.x;  // workgroup slot of the partial sums
  const int op = 1 + (g >= a.wg0[2]) + (g >= a.wg0[3]);
  const uint32_t T = (uint32_t)a.T, I = (uint32_t)a.I, O = (uint32_t)a.O;
  const uint32_t ncol = op == 2 ? O : I;
  const uint32_t nblk = op == 1 ? O / N : T / N;
  const uint32_t nct = (ncol + 63) / 64;
  const uint32_t local = (uint32_t)(g - a.wg0[op]);
  const uint32_t c0 = local % nct * 64, col = c0 + lane;
  const uint32_t blk0 = local / nct * LQS_STRIP;
  const uint32_t blk1 = blk0 + LQS_STRIP < nblk ? blk0 + LQS_STRIP : nblk;
  const bool valid = col < ncol;
  const int step = op >= 2 ? N / a.r : 1;  // outputs k with k % step == 0 are kept
  const float qmax = op >= 2 ? 127.f : 7.f;
  const int dt = op == 1 ? a.w_dt : a.gy_dt;
  const char* src = static_cast<const char*>(op == 1 ? a.w : a.gy);
  LqsQuant zt{0.f, 0.f, qmax}, zT{0.f, 0.f, qmax};
  if (valid) {
    zt.inv = a.tok_inv[op][col];
    zt.s = a.tok_s[op][col];
    const float at = __uint_as_float(a.tmax[op]);
    zT.inv = inv_of(at, qmax);
    zT.s = scale_of(at, qmax);
  }
  double ss = 0.0, e_tok = 0.0, e_ten = 0.0;
  for (uint32_t bb = blk0; bb < blk1; ++bb) {
    const uint32_t r0 = bb * N;
    if (op == 3) {
      // codes: 32 bytes per row of the tile, 8 lanes x 4 bytes, 8 rows a step
      const uint32_t half = I / 2, pc = lane & 7;
#pragma unroll
      for (int k0 = 0; k0 < N; k0 += 8) {
        const uint32_t r = k0 + (lane >> 3);
        uint32_t u = 0u;
        if (c0 + pc * 8 < I)
          u = *reinterpret_cast<const uint32_t*>(a.xc + (r0 + r) * half + c0 / 2 + pc * 4);
        *reinterpret_cast<uint32_t*>(tile + r * 32 + pc * 4) = u;
      }
      for (int k = lane; k < N; k += 64) tsc[k] = a.xs[r0 + k];
    } else if (dt == 1) {
      // bf16: 128 bytes per row, 8 lanes x 16 bytes, 8 rows a step
      const uint32_t pc = lane & 7;
#pragma unroll
      for (int k0 = 0; k0 < N; k0 += 8) {
        const uint32_t r = k0 + (lane >> 3);
        uint4 u = make_uint4(0, 0, 0, 0);
        if (c0 + pc * 8 < ncol)
          u = *reinterpret_cast<const uint4*>(src + (((r0 + r) * ncol + c0 + pc * 8) << 1));
        *reinterpret_cast<uint4*>(tile + r * 128 + pc * 16) = u;
      }
    } else {
      // fp32: 256 bytes per row, 16 lanes x 16 bytes, 4 rows a step
      const uint32_t pc = lane & 15;
#pragma unroll
      for (int k0 = 0; k0 < N; k0 += 4) {
        const uint32_t r = k0 + (lane >> 4);
        uint4 u = make_uint4(0, 0, 0, 0);
        if (c0 + pc * 4 < ncol)
          u = *reinterpret_cast<const uint4*>(src + (((r0 + r) * ncol + c0 + pc * 4) << 2));
        *reinterpret_cast<uint4*>(tile + r * 256 + pc * 16) = u;
      }
    }
    __syncthreads();
    if (valid) {
      float v[N];
#pragma unroll
      for (int k = 0; k < N; ++k) {
        if (op == 3) {
          const unsigned byte = tile[k * 32 + lane / 2];
          const int code = (int)(((lane & 1) ? byte >> 4 : byte) & 15u);
          v[k] = tsc[k] * (float)((code ^ 8) - 8);  // x = fl(s_x[t] * q)
        } else if (dt == 1) {
          v[k] = bf16_to_f32(*reinterpret_cast<const uint16_t*>(tile + k * 128 + lane * 2));
        } else {
          v[k] = *reinterpret_cast<const float*>(tile + k * 256 + lane * 4);
        }
      }
      fwht_reg<N>(v);
#pragma unroll
      for (int k = 0; k < N; ++k)
        if ((k & (step - 1)) == 0) {
          const float x = v[k];
          const float d1 = lqs_err(x, zt), d2 = lqs_err(x, zT);
          ss += (double)x * (double)x;
          e_tok += (double)d1 * (double)d1;
          e_ten += (double)d2 * (double)d2;
        }
    }
    __syncthreads();  // the next block overwrites the tile
  }
  // fixed-order butterfly over the wave: the sums are reproducible
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    ss += __shfl_xor(ss, m);
    e_tok += __shfl_xor(e_tok, m);
    e_ten += __shfl_xor(e_ten, m);
  }
  if (lane == 0) {
    a.part[g * 3 + 0] = ss;
    a.part[g * 3 + 1] = e_tok;
    a.part[g * 3 + 2] = e_ten;
  }
}

// Sum the per-workgroup partials of operand blockIdx.x in a fixed order and
// add them (and its element count) to the caller's statistics.
__global__ __launch_bounds__(1024) void k_lqs_final(LqsArgs a) {
  __shared__ double red[3][1024];
  const int tid = threadIdx.x, op = blockIdx.x;
  // four independent partial sums per thread (loads in flight), combined in
  // a fixed order
  double acc[4][3] = {};
  const int64_t e = a.wg0[op + 1];
  int64_t g = a.wg0[op] + tid;
  for (; g + 3 * 1024 < e; g += 4 * 1024)
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int c = 0; c < 3; ++c) acc[u][c] += a.part[(g + u * 1024) * 3 + c];
  for (; g < e; g += 1024)
#pragma unroll
    for (int c = 0; c < 3; ++c) acc[0][c] += a.part[g * 3 + c];
#pragma unroll
  for (int c = 0; c < 3; ++c) red[c][tid] = (acc[0][c] + acc[1][c]) + (acc[2][c] + acc[3][c]);
  __syncthreads();
  for (int h = 512; h > 0; h >>= 1) {
    if (tid < h)
#pragma unroll
      for (int c = 0; c < 3; ++c) red[c][tid] += red[c][tid + h];
    __syncthreads();
  }
  if (tid < 3) a.stats[4 * op + tid] += red[tid][0];
  if (tid == 3) a.stats[4 * op + 3] += a.count[op];
}

// ------------------------------------------------------------ launchers

static inline unsigned cdiv(int64_t a, int64_t b) { return (unsigned)((a + b - 1) / b); }

hipError_t launch_acbp(const void* x, int dtype, int64_t T, int64_t I, uint8_t* codes,
                       float* scales, hipStream_t s) {
  dim3 grid(cdiv(T, 4)), block(256);
#define HLQ_ACBP(RC)                                                                    \
  if (dtype == 0) hipLaunchKernelGGL((k_acbp<0, RC>), grid, block, 0, s, x, T, I, codes, scales); \
  else hipLaunchKernelGGL((k_acbp<1, RC>), grid, block, 0, s, x, T, I, codes, scales)
  if (I <= 512) { HLQ_ACBP(1); }
  else if (I <= 1024) { HLQ_ACBP(2); }
  else if (I <= 2048) { HLQ_ACBP(4); }
  else { HLQ_ACBP(0); }
#undef HLQ_ACBP
  return hipGetLastError();
}

template <int PASS, bool F32>
static hipError_t tr_dispatch(int n, int r, dim3 g, hipStream_t s, const TrArgs& a) {
#define HLQ_TR(NN, RR) hipLaunchKernelGGL((k_tr<PASS, NN, RR, F32>), g, dim3(256), 0, s, a)
#define HLQ_TR_N(NN)                                                      \
  switch (r) {                                                            \
    case 1: HLQ_TR(NN, 1); break;                                         \
    case 2: HLQ_TR(NN, 2); break;                                         \
    case 4: HLQ_TR(NN, 4); break;                                         \
    case 8: HLQ_TR(NN, 8); break;                                         \
    case 16: HLQ_TR(NN, 16); break;                                       \
    case 32: if (NN >= 32) HLQ_TR(NN, (NN >= 32 ? 32 : 1)); break;        \
    case 64: if (NN >= 64) HLQ_TR(NN, (NN >= 64 ? 64 : 1)); break;        \
    case 128: if (NN >= 128) HLQ_TR(NN, (NN >= 128 ? 128 : 1)); break;    \
    default: return hipErrorInvalidValue;                                 \
  }
  switch (n) {
    case 16: HLQ_TR_N(16); break;
    case 32: HLQ_TR_N(32); break;
    case 64: HLQ_TR_N(64); break;
    case 128: HLQ_TR_N(128); break;
    default: return hipErrorInvalidValue;
  }
#undef HLQ_TR_N
#undef HLQ_TR
  return hipGetLastError();
}

hipError_t launch_tr(const TrArgs& args, int pass, int n, int r, hipStream_t s) {
  if (r > n) return hipErrorInvalidValue;
  TrArgs a = args;
  // g_y tiles: the LDS engine's, except in the MAX pass of the register path,
  // where workgroups of four register-resident waves take them
  a.gy_workers = a.ntr_t * a.nch_o;
  a.gyreg_wgs = 0;
  if (pass == PASS_MAX && a.gy_reg) {
    if (a.gy_dt != 1 || n > 64) return hipErrorInvalidValue;
    a.gy_workers = 0;
    a.gyreg_wgs = (a.wg_gy + 3) / 4;
  }
  // eight slots per XCD row: each XCD takes an eighth of every job list
  const int64_t slots = (a.gyreg_wgs + 7) / 8 + (a.gy_workers + 7) / 8 + (a.wg_x + 7) / 8 +
                        (a.wg_w + 7) / 8;
  if (slots <= 0) return hipSuccess;
  dim3 g((unsigned)(slots * 8));
  const bool f32 = a.gy_dt == 0 || a.w_dt == 0;
  if (pass == PASS_MAX)
    return f32 ? tr_dispatch<PASS_MAX, true>(n, r, g, s, a) : tr_dispatch<PASS_MAX, false>(n, r, g, s, a);
  return f32 ? tr_dispatch<PASS_QUANT, true>(n, r, g, s, a)
             : tr_dispatch<PASS_QUANT, false>(n, r, g, s, a);
}

hipError_t launch_tr_reduce(const TrArgs& a, hipStream_t s) {
  if (a.nred != (int64_t)cdiv(a.T + a.O + 2 * a.I, RED_ENTRIES)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_tr_reduce, dim3((unsigned)a.nred), dim3(64 * RED_WAVES), 0, s, a);
  return hipGetLastError();
}

// Tile configurations (rows of A x rows of B, stage depth, ring depth):
//   0: 128 x 128, KB  64, 3 stages  (48 KB LDS, two workgroups per CU)
//   1: 256 x 128, KB  64, 3 stages  (72 KB LDS, two workgroups per CU)
//   2: 128 x 128, KB 128, 2 stages  (64 KB LDS, two workgroups per CU)
// Large grids take the 256 x 128 tile; INT8 operands with K a multiple of 128
// bytes take the deeper stage; grids below the CU count split K.
GemmPlan plan_gemm(bool int4, int64_t M, int64_t N, int64_t kbytes) {
  static const int cfg_bm[3] = {128, 256, 128}, cfg_bn[3] = {128, 128, 128};
  static const int cfg_kb[3] = {64, 64, 128};
  GemmPlan p;
  auto tiles = [&](int c) { return (int64_t)cdiv(M, cfg_bm[c]) * cdiv(N, cfg_bn[c]); };
  if (tiles(1) >= 1024) p.cfg = 1;
  else if (!int4 && kbytes % 128 == 0) p.cfg = 2;
  else p.cfg = 0;
  p.bm = cfg_bm[p.cfg];
  p.bn = cfg_bn[p.cfg];
  p.kb = cfg_kb[p.cfg];
  p.stages = kbytes / p.kb;
  const int64_t t = tiles(p.cfg);
  int64_t sp = 1;
  while (t * sp < 256 && sp < 8 && p.stages / (sp * 2) >= 8) sp *= 2;
  p.sps = (p.stages + sp - 1) / sp;
  p.splits = (int)((p.stages + p.sps - 1) / p.sps);  // every split non-empty
  return p;
}

template <bool I4, int EPI>
static void gemm_dispatch(int cfg, dim3 g, hipStream_t s, const GemmArgs& a) {
#define HLQ_GEMM(BM_, BN_, KB_, NS_) \
  hipLaunchKernelGGL((k_gemm<I4, BM_, BN_, KB_, NS_, EPI>), g, dim3(256), 0, s, a)
  switch (cfg) {
    case 1: HLQ_GEMM(256, 128, 64, 3); break;
    case 2: HLQ_GEMM(128, 128, 128, 2); break;
    default: HLQ_GEMM(128, 128, 64, 3); break;
  }
#undef HLQ_GEMM
}

hipError_t launch_gemm(bool int4, const uint8_t* A, const uint8_t* B, int64_t M,
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
  if (int4) {
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

hipError_t launch_gemm_pair(const uint8_t* gxA, const uint8_t* gxB, int64_t T, int64_t I,
                            int64_t kx_pitch, const GemmPlan& px, const float* s_gy,
                            const float* s_w, int gx_step, float gx_alpha, float* g_x,
                            const uint8_t* gwA, const uint8_t* gwB, int64_t O, int64_t kw_pitch,
                            const GemmPlan& pw, const float* s_gyl, const float* s_xl,
                            int gw_step, float gw_alpha, float* g_w, hipStream_t s) {
  if (kx_pitch % px.kb || px.stages * px.kb != kx_pitch) return hipErrorInvalidValue;
  if (kw_pitch % pw.kb || pw.stages * pw.kb != kw_pitch) return hipErrorInvalidValue;
  if (!g_x || !g_w || !s_gy || !s_w || !s_gyl || !s_xl) return hipErrorInvalidValue;
  const GemmArgs ax{gxA, gxB, T, I, kx_pitch, px.stages, px.stages, s_gy, gx_step, s_w, gx_step,
                    gx_alpha, g_x, nullptr};
  const GemmArgs aw{gwA, gwB, O, I, kw_pitch, pw.stages, pw.stages, s_gyl, gw_step, s_xl, gw_step,
                    gw_alpha, g_w, nullptr};
  // g_w tile: the plan's, except that a long-K g_w grid of fewer than 64
  // tiles (a quarter of the CU count; its tiles are the launch's critical
  // path) takes 64-row tiles (cfg 3: 64 x 128, KB 128, 3 stages): twice the
  // tiles, half the K work each.  Larger grids keep 128 x 128, which reads
  // fewer LDS bytes per MFMA (ViT-B qkv, 108 tiles: 46 -> 43 us).
  int wcfg = pw.cfg, wbm = pw.bm;
  if (pw.cfg == 2 && (int64_t)cdiv(O, 128) * cdiv(I, 128) < 64) { wcfg = 3; wbm = 64; }
  const int64_t tx = (int64_t)cdiv(T, px.bm) * cdiv(I, px.bn);
  const int64_t tw = (int64_t)cdiv(O, wbm) * cdiv(I, pw.bn);
  const int64_t n1 = (tw + 7) / 8 * 8, n0 = (tx + 7) / 8 * 8;
  const dim3 g((unsigned)(n1 + n0));
#define HLQ_PAIR(W_, X_) hipLaunchKernelGGL((k_gemm_pair<W_, X_>), g, dim3(256), 0, s, aw, n1, ax)
#define HLQ_W0 128, 128, 64, 3
#define HLQ_W1 256, 128, 64, 3
#define HLQ_W2 128, 128, 128, 2
#define HLQ_W3 64, 128, 128, 3
#define HLQ_X0 128, 128, 64, 3
#define HLQ_X1 256, 128, 64, 3
  const bool x1 = px.cfg == 1;
  switch (wcfg) {
    case 1: if (x1) HLQ_PAIR(HLQ_W1, HLQ_X1); else HLQ_PAIR(HLQ_W1, HLQ_X0); break;
    case 2: if (x1) HLQ_PAIR(HLQ_W2, HLQ_X1); else HLQ_PAIR(HLQ_W2, HLQ_X0); break;
    case 3: if (x1) HLQ_PAIR(HLQ_W3, HLQ_X1); else HLQ_PAIR(HLQ_W3, HLQ_X0); break;
    default: if (x1) HLQ_PAIR(HLQ_W0, HLQ_X1); else HLQ_PAIR(HLQ_W0, HLQ_X0); break;
  }
#undef HLQ_PAIR
#undef HLQ_W0
#undef HLQ_W1
#undef HLQ_W2
#undef HLQ_W3
#undef HLQ_X0
#undef HLQ_X1
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


hipError_t launch_lqs(const LqsArgs& a, int n, hipStream_t s) {
  const dim3 gr((unsigned)a.wg0[1]), gc((unsigned)(a.wg0[4] - a.wg0[1]));
#define HLQ_LQS(NN)                                                              \
  if (gr.x) hipLaunchKernelGGL((k_lqs_rows<NN>), gr, dim3(256), 0, s, a);       \
  if (gc.x) hipLaunchKernelGGL((k_lqs_cols<NN>), gc, dim3(64), 0, s, a)
  switch (n) {
    case 16: HLQ_LQS(16); break;
    case 32: HLQ_LQS(32); break;
    case 64: HLQ_LQS(64); break;
    case 128: HLQ_LQS(128); break;
    default: return hipErrorInvalidValue;
  }
#undef HLQ_LQS
  hipLaunchKernelGGL(k_lqs_final, dim3(4), dim3(1024), 0, s, a);
  return hipGetLastError();
}

}  // namespace hlq
