// gfx950 (CDNA4) kernels of the HLQ/HOT linear-layer backward: operand transforms (MAX, reduce, QUANT).
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

#include <algorithm>
#include <type_traits>

#include "hlq_device.h"
#include "hlq_internal.h"

namespace hlq {

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
// Readers of a parked tile.  operator()(r, c): element (r, c) as fp32;
// row<K>(r, c, v): the K adjacent elements c .. c + K - 1 of row r (c a
// multiple of K, K = 1, 2 or 4) with one LDS read.  (The bit-field extract
// builtin returns an unsigned int: the INT4 codes go through int before the
// conversion to float.)
struct RdF32 {
  const float* t;
  __device__ __forceinline__ float operator()(int r, int c) const { return t[r * P_F32 + c]; }
  template <int K>
  __device__ __forceinline__ void row(int r, int c, float (&v)[K]) const {
    const float* p = t + r * P_F32 + c;
    if constexpr (K == 4) {
      const float4 u = *reinterpret_cast<const float4*>(p);
      v[0] = u.x; v[1] = u.y; v[2] = u.z; v[3] = u.w;
    } else if constexpr (K == 2) {
      const float2 u = *reinterpret_cast<const float2*>(p);
      v[0] = u.x; v[1] = u.y;
    } else {
      v[0] = p[0];
    }
  }
};
struct RdB16 {
  const uint16_t* t;
  __device__ __forceinline__ float operator()(int r, int c) const {
    return __uint_as_float((uint32_t)t[r * P_B16 + c] << 16);
  }
  template <int K>
  __device__ __forceinline__ void row(int r, int c, float (&v)[K]) const {
    const uint16_t* p = t + r * P_B16 + c;
    if constexpr (K == 4) {
      const uint2 u = *reinterpret_cast<const uint2*>(p);
      v[0] = __uint_as_float(u.x << 16); v[1] = __uint_as_float(u.x & 0xFFFF0000u);
      v[2] = __uint_as_float(u.y << 16); v[3] = __uint_as_float(u.y & 0xFFFF0000u);
    } else if constexpr (K == 2) {
      const uint32_t u = *reinterpret_cast<const uint32_t*>(p);
      v[0] = __uint_as_float(u << 16); v[1] = __uint_as_float(u & 0xFFFF0000u);
    } else {
      v[0] = __uint_as_float((uint32_t)p[0] << 16);
    }
  }
};
// ACBP codes of a linear layer's x tile: one scale per row (token).
struct RdI4 {
  const uint8_t* q;
  const float* s;
  __device__ __forceinline__ float operator()(int r, int c) const {
    const int byte = q[r * P_I4 + (c >> 1)];
    const int code = __builtin_amdgcn_sbfe(byte, (c & 1) * 4, 4);
    return s[r] * (float)code;
  }
  template <int K>
  __device__ __forceinline__ void row(int r, int c, float (&v)[K]) const {
    const float sr = s[r];
    int bits;
    if constexpr (K == 4) bits = *reinterpret_cast<const uint16_t*>(q + r * P_I4 + (c >> 1));
    else bits = q[r * P_I4 + (c >> 1)];
#pragma unroll
    for (int k = 0; k < K; ++k)
      v[k] = sr * (float)(int)__builtin_amdgcn_sbfe(bits, ((K == 1 ? c & 1 : 0) + k) * 4, 4);
  }
};
// ACBP codes of a convolution's im2col tile: one scale per (row, 8-column
// chunk), s[r][c / 8] (the input pixel, hence the scale, can change at every
// tap boundary).
constexpr int X_CHUNKS = CW / 8;
struct RdI4c {
  const uint8_t* q;
  const float* s;
  __device__ __forceinline__ float operator()(int r, int c) const {
    const int byte = q[r * P_I4 + (c >> 1)];
    const int code = __builtin_amdgcn_sbfe(byte, (c & 1) * 4, 4);
    return s[r * X_CHUNKS + (c >> 3)] * (float)code;
  }
  // the K columns share one 8-column chunk, hence one scale
  template <int K>
  __device__ __forceinline__ void row(int r, int c, float (&v)[K]) const {
    const float sr = s[r * X_CHUNKS + (c >> 3)];
    int bits;
    if constexpr (K == 4) bits = *reinterpret_cast<const uint16_t*>(q + r * P_I4 + (c >> 1));
    else bits = q[r * P_I4 + (c >> 1)];
#pragma unroll
    for (int k = 0; k < K; ++k)
      v[k] = sr * (float)(int)__builtin_amdgcn_sbfe(bits, ((K == 1 ? c & 1 : 0) + k) * 4, 4);
  }
};

__device__ __forceinline__ float max_over_16_lanes(float a) {
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) a = nnmax(a, __shfl_xor(a, m));
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

// lowrank_col for the K adjacent columns c .. c + K - 1 (one LDS read per
// row for all of them); per column the same additions in the same order.
template <int N, int R, int K, class RD>
__device__ __forceinline__ void lowrank_cols(const RD& rd, int r0, int c, float (&g)[K][R]) {
  constexpr int G = N / R;
#pragma unroll
  for (int j = 0; j < R; ++j) {
    float s[G][K];
#pragma unroll
    for (int k = 0; k < G; ++k) rd.template row<K>(r0 + j * G + k, c, s[k]);
#pragma unroll
    for (int h = 1; h < G; h <<= 1)
#pragma unroll
      for (int k = 0; k < G; k += 2 * h)
#pragma unroll
        for (int q = 0; q < K; ++q) s[k][q] = s[k][q] + s[k + h][q];
#pragma unroll
    for (int q = 0; q < K; ++q) g[q][j] = s[0][q];
  }
#pragma unroll
  for (int q = 0; q < K; ++q)
#pragma unroll
    for (int h = 1; h < R; h <<= 1)
#pragma unroll
      for (int j = 0; j < R; ++j)
        if ((j & h) == 0) {
          float x0 = g[q][j], x1 = g[q][j + h];
          g[q][j] = x0 + x1;
          g[q][j + h] = x0 - x1;
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
  if (tid < CW && tid < cols) dst[tid] = nnmax(red[tid], red[tid + CW]);
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

// Store the staged INT8 codes of a tile into the K planes of an operand with
// `nrows` rows: column c of the tile (operand row c0 + c) owns `len` bytes at
// K offset koff.  Units of the widest width dividing len and koff (at most
// 16, so no unit crosses a 64-byte plane).
__device__ __forceinline__ void store_staged_i8(const uint8_t (*outs)[OUT_PITCH], int cols,
                                                int len, uint8_t* q, int64_t nrows, int64_t c0,
                                                int64_t koff, int tid) {
  int wdt = 16;
  while (wdt > 1 && ((len % wdt) || (koff % wdt))) wdt >>= 1;
  const int per_col = len / wdt;
  const int total = cols * per_col;
  for (int i = tid; i < total; i += 256) {
    const int c = i / per_col, k = (i % per_col) * wdt;
    uint8_t* d = q + i8_plane_off(nrows, c0 + c, koff + k);
    const uint8_t* s = &outs[c][k];
    if (wdt == 16) *reinterpret_cast<uint4*>(d) = *reinterpret_cast<const uint4*>(s);
    else if (wdt == 8) *reinterpret_cast<uint2*>(d) = *reinterpret_cast<const uint2*>(s);
    else if (wdt == 4) *reinterpret_cast<uint32_t*>(d) = *reinterpret_cast<const uint32_t*>(s);
    else if (wdt == 2) *reinterpret_cast<uint16_t*>(d) = *reinterpret_cast<const uint16_t*>(s);
    else *d = *s;
  }
}

// store_staged_i8 for a full tile whose runs are LEN bytes, LEN a multiple of
// 16 that divides 64 (koff a multiple of LEN: every run inside one plane):
// the tile's runs are CW consecutive 64-byte rows of that plane.
template <int LEN>
__device__ __forceinline__ void store_staged_i8_full(const uint8_t (*outs)[OUT_PITCH],
                                                     uint8_t* q, int64_t nrows, int64_t c0,
                                                     int64_t koff, int tid) {
  static_assert(LEN % 16 == 0 && I8_PLANE % LEN == 0, "16-byte runs inside one plane");
  constexpr int PER = LEN / 16;
  uint8_t* dst = q + i8_plane_off(nrows, c0, koff);
#pragma unroll
  for (int i = tid; i < CW * PER; i += 256) {
    const int c = i / PER, k = (i % PER) * 16;
    *reinterpret_cast<uint4*>(dst + (int64_t)c * I8_PLANE + k) =
        *reinterpret_cast<const uint4*>(&outs[c][k]);
  }
}

// Zero K bytes [from, to) of operand rows c0 .. c0 + cols - 1 (INT8 K planes,
// `nrows` rows; K padding); nthr threads share the work.
__device__ __forceinline__ void zero_tail_i8(uint8_t* q, int64_t nrows, int64_t c0, int cols,
                                             int64_t from, int64_t to, int tid, int nthr = 256) {
  const int64_t w = to - from;
  if (w <= 0) return;
  for (int64_t i = tid; i < (int64_t)cols * w; i += nthr)
    q[i8_plane_off(nrows, c0 + i / w, from + i % w)] = 0;
}

// Adjacent columns per thread of a low-rank column pass: 64 / n (4, 2, 1), so
// that the tile's (CW / CPT) column groups x (TT / n) blocks are the 256
// threads' tasks (n = 128: 128 tasks).
template <int N>
constexpr int lowrank_cpt() { return N <= 16 ? 4 : N == 32 ? 2 : 1; }

// Reciprocal scales of a thread's CPT columns c0 + (tid % (CW / CPT)) * CPT ..
// of a low-rank column pass (QUANT): colinv[column] in per-token mode (0 past
// cols), else that of tensor list `list` (INT8).  Every thread of the
// workgroup calls it (the tensor maximum is a wave fold).
template <int N>
__device__ __forceinline__ void lowrank_col_inv(const TrArgs& a, const float* colinv, int list,
                                                int64_t c0, int cols,
                                                float (&inv)[lowrank_cpt<N>()]) {
  constexpr int CPT = lowrank_cpt<N>();
  const int c = (threadIdx.x % (CW / CPT)) * CPT;
  if (colinv) {
#pragma unroll
    for (int k = 0; k < CPT; ++k) inv[k] = c + k < cols ? colinv[c0 + c + k] : 0.f;
  } else {
    const float t = inv_of(tensor_max_slots(a.tmax + list * TMAX_SLOTS), 127.f);
#pragma unroll
    for (int k = 0; k < CPT; ++k) inv[k] = t;
  }
}

// Column pass, low-rank rows of H_N (g_w operands).  Thread tid owns the CPT
// adjacent columns c = (tid % NCG) * CPT .. and block b = tid / NCG (NCG =
// CW / CPT column groups), reading a row of its columns with one LDS read.
// MAX: the tile's column maxima -> part[0..cols).  QUANT: INT8 codes
// (reciprocal scales inv of the thread's columns, lowrank_col_inv) staged in
// LDS over the tile (after a barrier) and stored as operand rows c0 + c, K
// bytes t0 / N * R ..., of the INT8 K planes of q (nrows rows, kpitch bytes
// of K per row).
template <int PASS, int N, int R, class RD>
__device__ __forceinline__ void colpass_lowrank(const TrArgs& a, const RD& rd, uint8_t* smem,
                                                float* red, int rows, int cols, int64_t c0,
                                                const float (&inv)[lowrank_cpt<N>()], float* part,
                                                uint8_t* q, int64_t nrows, int64_t kpitch,
                                                int64_t tl, int64_t t0, bool last) {
  constexpr int CPT = lowrank_cpt<N>(), NCG = CW / CPT;
  constexpr int WPR = (R + 3) / 4;  // code words per column
  static_assert(NCG * (TT / N) <= 256, "one task per thread");
  const int tid = threadIdx.x;
  const int c = (tid % NCG) * CPT, b = tid / NCG;
  const int nb = rows / N;
  const bool act = b < nb && c < cols;
  float cm[CPT];
  uint32_t words[CPT][WPR];
#pragma unroll
  for (int k = 0; k < CPT; ++k) {
    cm[k] = 0.f;
#pragma unroll
    for (int w = 0; w < WPR; ++w) words[k][w] = 0;
  }
  if (act) {
    float g[CPT][R];
    lowrank_cols<N, R, CPT>(rd, b * N, c, g);
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      if constexpr (PASS == PASS_MAX) {
#pragma unroll
        for (int j = 0; j < R; ++j) cm[k] = fmaxf(cm[k], fabsf(g[k][j]));
      } else {
#pragma unroll
        for (int j = 0; j < R; ++j)
          words[k][j / 4] |= (quant_bits<127>(g[k][j], inv[k]) & 0xFFu) << (8 * (j % 4));
      }
    }
  }
  if constexpr (PASS == PASS_MAX) {
    // maxima over the column's blocks: with NCG = 32 the two blocks of a
    // wave meet by a lane exchange, then at most four slots per column in LDS
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      if constexpr (NCG == 32) cm[k] = nnmax(cm[k], __shfl_xor(cm[k], 32));
    }
    constexpr int SLOTS = (TT / N) / (NCG == 32 ? 2 : 1);  // <= 4
    static_assert(SLOTS >= 1 && SLOTS <= 4, "red holds four slots per column");
    const int slot = NCG == 32 ? b / 2 : b;
    if (NCG != 32 || (tid & 32) == 0) {
      if (slot < SLOTS) {
#pragma unroll
        for (int k = 0; k < CPT; ++k) red[slot * CW + c + k] = cm[k];
      }
    }
    __syncthreads();
    if (tid < CW && tid < cols) {
      float m = red[tid];
#pragma unroll
      for (int sl = 1; sl < SLOTS; ++sl) m = nnmax(m, red[sl * CW + tid]);
      part[tid] = m;
    }
  } else {
    uint8_t (*outs)[OUT_PITCH] = reinterpret_cast<uint8_t (*)[OUT_PITCH]>(smem);
    __syncthreads();  // every thread is done reading the tile
    if (act) {
      // column groups of CPT columns are CPT * OUT_PITCH bytes apart, which
      // maps 16 lanes onto 4 banks; each lane writes its columns starting
      // at a rotation (cg / 4 or cg / 8 mod CPT), so that the 16 lanes of
      // one write cover 16 columns mod 16 (16 distinct banks)
      const int cg = tid % NCG;
      const int rot = CPT == 1 ? 0 : (cg >> (CPT == 4 ? 2 : 3)) & (CPT - 1);
#pragma unroll
      for (int kk = 0; kk < CPT; ++kk) {
        const int k = (kk + rot) & (CPT - 1);
        uint32_t wv[WPR];
#pragma unroll
        for (int w = 0; w < WPR; ++w) {
          wv[w] = words[0][w];
#pragma unroll
          for (int q = 1; q < CPT; ++q) wv[w] = k == q ? words[q][w] : wv[w];
        }
        if (c + k >= cols) continue;
        if constexpr (R >= 4) {
#pragma unroll
          for (int w = 0; w < WPR; ++w)
            *reinterpret_cast<uint32_t*>(&outs[c + k][b * R + 4 * w]) = wv[w];
        } else {
#pragma unroll
          for (int j = 0; j < R; ++j) outs[c + k][b * R + j] = (uint8_t)(wv[0] >> (8 * j));
        }
      }
    }
    __syncthreads();
    const int64_t koff = t0 / N * R;
    constexpr int LEN = (TT / N) * R;
    constexpr bool FULL_OK = LEN % 16 == 0 && I8_PLANE % LEN == 0;
    if (FULL_OK && rows == TT && cols == CW)
      store_staged_i8_full<(FULL_OK ? LEN : 16)>(outs, q, nrows, c0, koff, tid);
    else
      store_staged_i8(outs, cols, nb * R, q, nrows, c0, koff, tid);
    if (last) zero_tail_i8(q, nrows, c0, cols, tl, kpitch, tid);
  }
}

// Column pass with the full H_N along the rows (w -> INT4 codes for g_x, stored
// as FP6 E2M3 groups of 128 K values).
template <int PASS, int N, class RD>
__device__ __forceinline__ void colpass_full(const TrArgs& a, const RD& rd, uint8_t* smem,
                                             float* red, int rows, int cols, int64_t c0,
                                             const float* colinv, int list, float* part,
                                             uint8_t* q, int64_t nrows, int64_t o0, int64_t O,
                                             bool last) {
  constexpr int TPT = (TT / N) / 2 > 0 ? (TT / N) / 2 : 1;
  constexpr int NB = TT / N;  // blocks of the tile's group
  static_assert(TT == 128, "one tile of rows is one 128-value FP6 group");
  const int tid = threadIdx.x;
  const int c = tid % CW;
  const int nb = rows / N;
  float inv_c = 0.f;
  if constexpr (PASS == PASS_QUANT) {
    const float tinv =
        colinv ? 0.f : inv_of(tensor_max_slots(a.tmax + list * TMAX_SLOTS), list == 1 ? 7.f : 127.f);
    inv_c = colinv ? (c < cols ? colinv[c0 + c] : 0.f) : tinv;
  }
  if constexpr (PASS == PASS_MAX) {
    float cm = 0.f;
#pragma unroll
    for (int t = 0; t < TPT; ++t) {
      const int b = tid / CW + 2 * t;
      if (b < nb && c < cols) {
        float v[N];
        full_col<N>(rd, b * N, c, v);
#pragma unroll
        for (int k = 0; k < N; ++k) cm = fmaxf(cm, fabsf(v[k]));
      }
    }
    tile_colmax_store(cm, red, tid, cols, part);
  } else {
    // FP6 codes of the thread's blocks (zero codes for blocks past O or
    // columns past I), 32 values per conversion: a block of 16 is paired
    // with the thread's next (16 rows on, the same half of the next quarter)
    uint8_t (*outs)[OUT_PITCH] = reinterpret_cast<uint8_t (*)[OUT_PITCH]>(smem);
    float r[TPT][N];
#pragma unroll
    for (int t = 0; t < TPT; ++t) {
      const int b = tid / CW + 2 * t;
#pragma unroll
      for (int k = 0; k < N; ++k) r[t][k] = 0.f;
      if (b < nb && c < cols) {
        float v[N];
        full_col<N>(rd, b * N, c, v);
#pragma unroll
        for (int k = 0; k < N; ++k) r[t][k] = quant_code_f32(v[k], inv_c);
      }
    }
    __syncthreads();  // the column reads of the tile are done: smem is staging now
    if constexpr (N == 16) {
#pragma unroll
      for (int t = 0; t < TPT; t += 2) {
        const int b = tid / CW + 2 * t;  // blocks b and b + 2: quarters b/2 and b/2 + 1
        float f[32];
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          f[k] = r[t][k];
          f[16 + k] = r[t + 1][k];
        }
        uint32_t d[6];
        fp6_pack32(f, d);
        const int e = b & 1, qa = b >> 1;
        uint8_t* pa = &outs[c][fp6_quarter_pos(qa) * 24 + 12 * e];
        uint8_t* pb = &outs[c][fp6_quarter_pos(qa + 1) * 24 + 12 * e];
#pragma unroll
        for (int k = 0; k < 3; ++k) {
          reinterpret_cast<uint32_t*>(pa)[k] = d[k];
          reinterpret_cast<uint32_t*>(pb)[k] = d[3 + k];
        }
      }
    } else {
#pragma unroll
      for (int t = 0; t < TPT; ++t) {
        const int b = tid / CW + 2 * t;
        if (b < NB) {
#pragma unroll
          for (int p = 0; p < N / 32; ++p) {
            float f[32];
#pragma unroll
            for (int k = 0; k < 32; ++k) f[k] = r[t][32 * p + k];
            uint32_t d[6];
            fp6_pack32(f, d);
            uint32_t* dst = reinterpret_cast<uint32_t*>(
                &outs[c][fp6_quarter_pos(b * (N / 32) + p) * 24]);
#pragma unroll
            for (int k = 0; k < 6; ++k) dst[k] = d[k];
          }
        }
      }
    }
    __syncthreads();
    // the whole 96-byte group of each column, K padding (zero codes)
    // included: rows c0 .. of FP6 plane o0 / TT (nrows rows of 96 bytes)
    uint8_t* dst = q + ((o0 / TT) * nrows + c0) * FP6_PLANE;
    if (cols == CW)
      store_staged_full<96>(outs, dst, FP6_PLANE, tid);
    else
      store_staged(outs, cols, 96, dst, FP6_PLANE, 0, tid);
  }
  (void)last;
  (void)O;
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

// FP6 codes of H.g_y: lane lc (0..15) of a row's 16 lanes holds the 48-bit
// fields (lo: bits 0-31, hi: bits 32-47) of the codes of columns 8 lc ..
// 8 lc + 7 of one 128-value group, i.e. bits 48 (lc & 3) .. of quarter lc >> 2.
// An even lane takes its odd neighbour's field (DPP quad permute) and writes
// the pair's 96 bits, bytes 12 (lc & 3) / 2 .. + 11 of the quarter's 24-byte
// stream, with one 12-byte store.  Every lane of the quad calls it (the
// exchange reads lane ^ 1); `store` masks the write.
__device__ __forceinline__ void store_fp6_lane8(uint8_t* group, int lc, uint32_t lo, uint32_t hi,
                                                bool store) {
  const uint32_t nlo = (uint32_t)__builtin_amdgcn_mov_dpp((int)lo, 0xB1, 0xF, 0xF, true);
  const uint32_t nhi = (uint32_t)__builtin_amdgcn_mov_dpp((int)hi, 0xB1, 0xF, 0xF, true);
  if (!store || (lc & 1)) return;
  uint32_t* q = reinterpret_cast<uint32_t*>(group + fp6_quarter_pos(lc >> 2) * 24 + 6 * (lc & 2));
  typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
  *reinterpret_cast<u32x3*>(q) = u32x3{lo, hi | (nlo << 16), (nlo >> 16) | (nhi << 16)};
}

// FP6 codes of four rows' 8-value lane slices (rc[k][0..7], integer-valued
// floats) in one conversion; row k's 48-bit field is bits 48 k .. 48 k + 47.
__device__ __forceinline__ void fp6_rows4(const float (&rc)[4][8], uint32_t (&lo)[4],
                                          uint32_t (&hi)[4]) {
  float f[32];
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int e = 0; e < 8; ++e) f[8 * k + e] = rc[k][e];
  uint32_t d[6];
  fp6_pack32(f, d);
  lo[0] = d[0];                                 hi[0] = d[1] & 0xFFFFu;
  lo[1] = __builtin_amdgcn_alignbit(d[2], d[1], 16); hi[1] = d[2] >> 16;
  lo[2] = d[3];                                 hi[2] = d[4] & 0xFFFFu;
  lo[3] = __builtin_amdgcn_alignbit(d[5], d[4], 16); hi[3] = d[5] >> 16;
}

template <int PASS, int N>
__device__ __forceinline__ void gy_rows_bf16_full(const TrArgs& a, int64_t t0, int64_t c0,
                                                  int64_t ch, uint8_t* smem, float inv_tensor) {
  constexpr int SW = TT / 16;
  const int tid = threadIdx.x, lr = tid >> 4, lc = tid & 15, col = lc * 8;
  const uint32_t O32 = (uint32_t)a.O;
  const uint8_t* gbase = static_cast<const uint8_t*>(a.gy) + (t0 * a.O + c0) * 2;
  const uint32_t goff = ((uint32_t)lr * O32 + (uint32_t)col) * 2u;
  // The row scales are loaded before the tile and in either mode (the array
  // holds T floats): each sweep then waits only for its own tile rows.
  // Loaded after the tile, or under a per-mode branch (the compiler moves
  // loads used on one side into it), they made the first sweep wait for the
  // whole tile.  Per-tensor mode masks the loaded bits to +0 and takes the
  // tensor scale (scales are >= +0, never NaN).
  float inv[SW];
  if constexpr (PASS == PASS_QUANT) {
    const float* ib = a.inv_gy + t0;
    const uint32_t keep = a.gx_tok ? 0xFFFFFFFFu : 0u;
    const float base = a.gx_tok ? 0.f : inv_tensor;
#pragma unroll
    for (int sw = 0; sw < SW; ++sw) inv[sw] = ib[sw * 16 + lr];
#pragma unroll
    for (int sw = 0; sw < SW; ++sw) inv[sw] = nnmax(__uint_as_float(__float_as_uint(inv[sw]) & keep), base);
  }
  uint4 raw[SW];
#pragma unroll
  for (int sw = 0; sw < SW; ++sw)
    raw[sw] = ld16<PASS == PASS_QUANT>(gbase + goff + (uint32_t)sw * 32u * O32);
  static_assert(SW % 4 == 0 && CW == 128, "four rows per FP6 conversion, one group per tile");
  // the tile's 128 columns are one FP6 group of each row: rows t0 .. of FP6
  // plane c0 / CW (T rows of 96 bytes)
  uint8_t* qbase = a.q_gy + ((c0 / CW) * a.T + t0) * FP6_PLANE;
  float rc[4][8];
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
      m = nnmax(m, lane_xor<1>(m));
      m = nnmax(m, lane_xor<2>(m));
      m = nnmax(m, lane_xor<4>(m));
      m = nnmax(m, lane_xor<8>(m));
      if (lc == 0) a.part_gy[ch * a.T + t0 + row] = m;
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) rc[sw & 3][k] = quant_code_f32(v[k], inv[sw]);
      if ((sw & 3) == 3) {
        uint32_t lo[4], hi[4];
        fp6_rows4(rc, lo, hi);
#pragma unroll
        for (int k = 0; k < 4; ++k)
          store_fp6_lane8(qbase + (uint32_t)((sw - 3 + k) * 16 + lr) * FP6_PLANE, lc, lo[k], hi[k],
                          true);
      }
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
    if (!a.gx_tok) inv_tensor = inv_of(tensor_max_slots(a.tmax), 7.f);
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
  float rc[4][8];
  uint8_t* qbase = a.q_gy + ((c0 / CW) * a.T + t0) * FP6_PLANE;
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
    } else {
      // rows past T quantize nothing; columns past O inside the group are
      // zero codes (K padding)
      const float inv = row < rows ? (a.gx_tok ? a.inv_gy[t0 + row] : inv_tensor) : 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k) rc[sw & 3][k] = col < cols ? quant_code_f32(v[k], inv) : 0.f;
      if ((sw & 3) == 3) {
        uint32_t lo[4], hi[4];
        fp6_rows4(rc, lo, hi);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int rk = (sw - 3 + k) * 16 + lr;
          store_fp6_lane8(qbase + (int64_t)rk * FP6_PLANE, lc, lo[k], hi[k], rk < rows);
        }
      }
    }
  }
  }
  __syncthreads();
  const bool last = t0 + rows == a.T;
  float inv_c[lowrank_cpt<N>()] = {};
  if constexpr (PASS == PASS_QUANT)
    lowrank_col_inv<N>(a, a.gw_tok ? a.inv_gyl : nullptr, 2, c0, cols, inv_c);
  if constexpr (F32) {
    RdF32 rd{reinterpret_cast<const float*>(smem)};
    colpass_lowrank<PASS, N, R>(a, rd, smem, red, rows, cols, c0, inv_c,
                                a.part_gyl + tr * a.O + c0, a.q_gyl, a.O, a.kwb, a.tl, t0, last);
  } else {
    RdB16 rd{reinterpret_cast<const uint16_t*>(smem)};
    colpass_lowrank<PASS, N, R>(a, rd, smem, red, rows, cols, c0, inv_c,
                                a.part_gyl + tr * a.O + c0, a.q_gyl, a.O, a.kwb, a.tl, t0, last);
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

// Registers of tile (tr, ch): tokens tr * 64 .., channels ch * 128 .. (zero
// outside T and O).
__device__ __forceinline__ void gyr_load(const TrArgs& a, int64_t tr, int64_t ch,
                                         uint4 (&raw)[8][2]) {
  const int lane = threadIdx.x & 63;
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

// Whether tile (tr, ch) lies wholly inside T and O (uniform over the wave).
__device__ __forceinline__ bool gyr_full(const TrArgs& a, int64_t tr, int64_t ch) {
  return (tr + 1) * GYR_ROWS <= a.T && (ch + 1) * CW <= a.O;
}

// gyr_load for a whole tile: the sixteen loads back to back with no per-lane
// guards.  (Guarded, the compiler placed register moves between the loads
// that waited for the first ones to arrive, a memory latency per tile.)
__device__ __forceinline__ void gyr_load_full(const TrArgs& a, int64_t tr, int64_t ch,
                                              uint4 (&raw)[8][2]) {
  const int lane = threadIdx.x & 63;
  const int64_t t0 = tr * GYR_ROWS + (lane >> 3) * 8, c0 = ch * CW + (lane & 7) * 16;
  const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.gy) + t0 * a.O + c0);
  const int64_t pitch = a.O / 8;  // uint4 per row (O is a multiple of 16)
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    raw[k][0] = src[k * pitch];
    raw[k][1] = src[k * pitch + 1];
  }
}

// Maxima of tile (tr, ch): row maxima of H.g_y along O -> part_gy[ch][t];
// column maxima of the low-rank g_y along T -> cm[0 .. 128) (the workgroup
// folds its four tiles' into part_gyl).
template <int N, int R, bool LEAN>
__device__ __forceinline__ void gyr_tile_max(const TrArgs& a, int64_t tr, int64_t ch,
                                             uint4 (&raw)[8][2], float* cm) {
  static_assert(N >= 16 && N <= 64, "a token block spans 2..8 row groups of one wave");
  constexpr int G = N / R;             // tokens per low-rank group
  constexpr int GL = G < 8 ? G : 8;    // in-lane span of a group
  constexpr int RGB = N / 8;           // row groups per token block
  const int lane = threadIdx.x & 63;
  const int c16 = lane & 7, rg = lane >> 3;
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

  // LEAN: the tile's words pass through an empty asm statement, so the fp32
  // values unpacked along O are not kept for the pass along T (which unpacks
  // the same words again, two VALU operations per element).  Kept, they
  // double the live registers of the whole launch (154 VGPRs against 90:
  // three waves per SIMD instead of four), which the LDS-engine jobs of the
  // same launch feel; the host takes LEAN when those jobs outnumber the
  // register tiles' workgroups (ResNet-50 stage-3 shape MAX 49 -> 39 us,
  // ViT-B qkv, mostly register tiles, 18.1 -> 19.2 with it).
  if constexpr (LEAN) {
#pragma unroll
    for (int k = 0; k < 8; ++k)
#pragma unroll
      for (int q = 0; q < 2; ++q)
        asm volatile("" : "+v"(raw[k][q].x), "+v"(raw[k][q].y), "+v"(raw[k][q].z), "+v"(raw[k][q].w));
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
    m = nnmax(m, lane_xor<8>(m));
    m = nnmax(m, lane_xor<16>(m));
    m = nnmax(m, lane_xor<32>(m));
    cmax[j] = m;
  }
  if (lane < 8) {  // lane c16 < 8 holds columns 16 c16 .. + 15 (zero past O)
#pragma unroll
    for (int j = 0; j < 16; ++j) cm[col + j] = cact ? cmax[j] : 0.f;
  }
}

// ---- job: x tile (ACBP codes, low-rank columns along T for g_w)
// Linear layer: rows are tokens of the code matrix [T][I/2].  Convolution
// (a.conv): rows are output pixels t = (n, p, q) and columns the im2col
// features (r*S + s)*C + c; each 8-column chunk (C is a multiple of 8, so a
// chunk stays inside one tap) gathers 4 code bytes of input pixel
// (n, p*stride - pad + r, q*stride - pad + s) with that pixel's scale, or
// zeros outside the image.
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
  float* scales = reinterpret_cast<float*>(smem + TT * P_I4);     // [TT] or [TT][X_CHUNKS]
  // 64 code bytes per tile row: 4 lanes x 16 bytes, 64 rows per sweep.  Rows
  // are I/2 bytes, a multiple of 4: whole tiles of rows that are a multiple
  // of 16 bytes take one 16-byte load per lane and sweep, the rest dwords
  // (four dword loads per lane touched every 64-byte run four times).
  constexpr int SW = TT / 64;
  const int lr = tid >> 2, lq = tid & 3;
  const int col = lq * 32;
  uint32_t w4[SW][4];
  if (!a.conv && rows == TT && cols == CW && a.I % 32 == 0) {
    // whole tile with 16-byte aligned rows (uniform): one 16-byte load per
    // sweep, no guards
#pragma unroll
    for (int sw = 0; sw < SW; ++sw) {
      const uint4 u = *reinterpret_cast<const uint4*>(a.xc + (t0 + sw * 64 + lr) * (a.I / 2) +
                                                      (c0 + col) / 2);
      w4[sw][0] = u.x; w4[sw][1] = u.y; w4[sw][2] = u.z; w4[sw][3] = u.w;
    }
    if (tid < TT) scales[tid] = a.xs[t0 + tid];
  } else if (!a.conv) {
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
  } else if (a.Cc % 32 == 0 && cols == CW) {
    // the thread's four chunks are 32 consecutive channels of one tap (the
    // channel count a multiple of 32): one 16-byte load of one pixel's codes
    // and one scale per row
    const int64_t cc = c0 + col, rs = cc / a.Cc, chan = cc - rs * a.Cc;
    const int tap_r = (int)(rs / a.S), tap_s = (int)(rs - (int64_t)tap_r * a.S);
    float sv[SW];
#pragma unroll
    for (int sw = 0; sw < SW; ++sw) {
      const int row = sw * 64 + lr;
      const int64_t t = t0 + row;
      const int64_t pq = a.P * a.Q;
      const int64_t nn = t / pq, rem = t - nn * pq;
      const int64_t p = rem / a.Q, q = rem - p * a.Q;
      const int64_t hh = p * a.cstride - a.cpad + tap_r;
      const int64_t ww = q * a.cstride - a.cpad + tap_s;
#pragma unroll
      for (int d = 0; d < 4; ++d) w4[sw][d] = 0u;
      sv[sw] = 0.f;
      if (row < rows && hh >= 0 && hh < a.Hc && ww >= 0 && ww < a.Wc) {
        const int64_t pix = (nn * a.Hc + hh) * a.Wc + ww;
        const uint4 u = *reinterpret_cast<const uint4*>(a.xc + pix * (a.Cc / 2) + chan / 2);
        w4[sw][0] = u.x; w4[sw][1] = u.y; w4[sw][2] = u.z; w4[sw][3] = u.w;
        sv[sw] = a.xs[pix];
      }
    }
#pragma unroll
    for (int sw = 0; sw < SW; ++sw)
      *reinterpret_cast<float4*>(scales + (sw * 64 + lr) * X_CHUNKS + lq * 4) =
          make_float4(sv[sw], sv[sw], sv[sw], sv[sw]);
  } else {
    // taps and channels of this thread's four chunks
    int tap_r[4], tap_s[4];
    int64_t chan[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const int64_t cc = c0 + col + 8 * d;
      const int64_t rs = cc / a.Cc;
      chan[d] = cc - rs * a.Cc;
      tap_r[d] = (int)(rs / a.S);
      tap_s[d] = (int)(rs - (int64_t)tap_r[d] * a.S);
    }
    float sv[SW][4];
#pragma unroll
    for (int sw = 0; sw < SW; ++sw) {
      const int row = sw * 64 + lr;
      const int64_t t = t0 + row;
      const int64_t pq = a.P * a.Q;
      const int64_t nn = t / pq, rem = t - nn * pq;
      const int64_t p = rem / a.Q, q = rem - p * a.Q;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        w4[sw][d] = 0u;
        sv[sw][d] = 0.f;
        const int64_t hh = p * a.cstride - a.cpad + tap_r[d];
        const int64_t ww = q * a.cstride - a.cpad + tap_s[d];
        if (row < rows && col + 8 * d < cols && hh >= 0 && hh < a.Hc && ww >= 0 && ww < a.Wc) {
          const int64_t pix = (nn * a.Hc + hh) * a.Wc + ww;
          w4[sw][d] = *reinterpret_cast<const uint32_t*>(a.xc + pix * (a.Cc / 2) + chan[d] / 2);
          sv[sw][d] = a.xs[pix];
        }
      }
    }
#pragma unroll
    for (int sw = 0; sw < SW; ++sw)
      *reinterpret_cast<float4*>(scales + (sw * 64 + lr) * X_CHUNKS + lq * 4) =
          make_float4(sv[sw][0], sv[sw][1], sv[sw][2], sv[sw][3]);
  }
#pragma unroll
  for (int sw = 0; sw < SW; ++sw)
    *reinterpret_cast<uint4*>(codes + (sw * 64 + lr) * P_I4 + col / 2) =
        make_uint4(w4[sw][0], w4[sw][1], w4[sw][2], w4[sw][3]);
  __syncthreads();
  float inv_c[lowrank_cpt<N>()] = {};
  if constexpr (PASS == PASS_QUANT)
    lowrank_col_inv<N>(a, a.gw_tok ? a.inv_xl : nullptr, 3, c0, cols, inv_c);
  if (!a.conv) {
    RdI4 rd{codes, scales};
    colpass_lowrank<PASS, N, R>(a, rd, smem, red, rows, cols, c0, inv_c,
                                a.part_xl + tr * a.I + c0, a.q_xl, a.I, a.kwb, a.tl, t0,
                                t0 + rows == a.T);
  } else {
    RdI4c rd{codes, scales};
    colpass_lowrank<PASS, N, R>(a, rd, smem, red, rows, cols, c0, inv_c,
                                a.part_xl + tr * a.I + c0, a.q_xl, a.I, a.kwb, a.tl, t0,
                                t0 + rows == a.T);
  }
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
                          a.part_w + tr * a.I + c0, a.q_w, a.I, o0, a.O, last);
  } else {
    RdB16 rd{reinterpret_cast<const uint16_t*>(smem)};
    colpass_full<PASS, N>(a, rd, smem, red, rows, cols, c0, a.gx_tok ? a.inv_w : nullptr, 1,
                          a.part_w + tr * a.I + c0, a.q_w, a.I, o0, a.O, last);
  }
}

// F32: the g_y / w tiles hold fp32 (any fp32 source); otherwise bf16.
// LEAN (MAX pass): the register-resident g_y tiles in the register-lean form.
template <int PASS, int N, int R, bool F32, bool LEAN = false>
__global__ __launch_bounds__(256) void k_tr(TrArgs a) {
  static_assert(TT * P_I4 + TT * X_CHUNKS * 4 <= TileSmem<F32>::bytes, "x tile fits the smem buffer");
  static_assert(CW * OUT_PITCH <= TileSmem<F32>::bytes, "staging fits the smem buffer");
  __shared__ __attribute__((aligned(16))) uint8_t smem[TileSmem<F32>::bytes];
  __shared__ float red[4 * CW];
  if constexpr (PASS == PASS_QUANT) {
    // the zero row the convolution's input-gradient GEMM reads for taps
    // outside the image
    if (a.zero_row && blockIdx.x == 0)
      for (int64_t i = threadIdx.x; i < a.kxb / 16; i += 256)
        reinterpret_cast<uint4*>(a.zero_row)[i] = make_uint4(0, 0, 0, 0);
    // arrival counters of the GEMM launch that follows (K-split g_w tiles)
    if (blockIdx.x == 1 % gridDim.x)
      for (int64_t i = threadIdx.x; i < a.pair_nctr; i += 256) a.pair_ctr[i] = 0u;
  }
  if (blockIdx.x == 0) {
    if constexpr (PASS == PASS_MAX) {
      static_assert(4 * TMAX_SLOTS <= 256, "one slot per thread");
      if (threadIdx.x < 4 * TMAX_SLOTS) a.tmax[threadIdx.x] = 0u;  // k_tr_reduce folds into them
    } else if (threadIdx.x < 64) {  // tensor scales of the per-tensor modes (wave 0)
#pragma unroll
      for (int l = 0; l < 4; ++l) {
        const float m = tensor_max_slots(a.tmax + l * TMAX_SLOTS);
        const float qmax = l < 2 ? 7.f : 127.f;
        if (threadIdx.x == 0 && (l < 2 ? !a.gx_tok : !a.gw_tok)) {
          float* sc = l == 0 ? a.s_gy : l == 1 ? a.s_w : l == 2 ? a.s_gyl : a.s_xl;
          sc[0] = scale_of(m, qmax);
        }
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
    // register-resident g_y tiles: a workgroup takes four consecutive
    // 64-token tiles of one 128-channel chunk, one per wave; the waves run
    // independently and meet once, to fold their low-rank column maxima into
    // one partial per 256 tokens (a quarter of the partials to fold)
    if (slot < per_r) {
      const int64_t bid = xcd * per_r + slot;
      if (bid < a.gyreg_wgs) {  // uniform over the workgroup
        // workgroup ids and chunk counts fit 32 bits (grids are 32-bit)
        const uint32_t b32 = (uint32_t)bid, n32 = (uint32_t)a.nch_o;
        const int64_t trg = b32 / n32, ch = b32 % n32;
        const int w = threadIdx.x >> 6;
        const int64_t tr = trg * 4 + w;
        float* cm = red + w * CW;
        if (tr * GYR_ROWS < a.T) {
          uint4 raw[8][2];
          if (gyr_full(a, tr, ch)) {  // separate copies: no register moves between the loads
            gyr_load_full(a, tr, ch, raw);
            gyr_tile_max<N, R, LEAN>(a, tr, ch, raw, cm);
          } else {
            gyr_load(a, tr, ch, raw);
            gyr_tile_max<N, R, LEAN>(a, tr, ch, raw, cm);
          }
        } else {
          cm[threadIdx.x & 63] = 0.f;
          cm[64 + (threadIdx.x & 63)] = 0.f;
        }
        __syncthreads();
        const int c = threadIdx.x;
        const int64_t c0 = ch * CW;
        if (c < CW && c0 + c < a.O)
          a.part_gyl[trg * a.O + c0 + c] =
              nnmax(nnmax(red[c], red[CW + c]), nnmax(red[2 * CW + c], red[3 * CW + c]));
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

// Fold the partial maxima.  Lists: 0 H.g_y rows, 1 H.w columns, 2 low-rank
// g_y columns, 3 low-rank x columns.
//  * A list in per-token mode is folded entry by entry: entry e takes the max
//    over its partials and stores its scale s = a/qmax and qmax/a (the QUANT
//    pass multiplies by the latter).  A 256-thread block folds E consecutive
//    entries of one list, its threads splitting each entry's partials
//    256 / E ways with up to eight loads in flight per thread: E = 64 for
//    lists of at most 32 partials per entry, 32 up to 64, else 16 (one round
//    of loads up to 128 partials).  Blocks of 16 waves for 64 entries of any
//    list left most waves idle on the short lists (ViT-B qkv fold 3.9 ->
//    3.0 us).
//  * A list in per-tensor mode needs only its maximum: its partial array is
//    folded flat, RED_FLAT floats per block with 16-byte loads (entry by
//    entry, a long low-rank column list made a few blocks long).
// A flat block folds its list's maximum into the tensor maximum with one
// atomicMax, on slot blockIdx % 64 of the list (same-address atomics
// serialize: the ResNet shape's reduce 13.6 -> 6.4 us without the slots).
// Per-entry blocks do the same for their list only when the tensor maxima of
// per-token lists are asked for (tok_tmax: the LQS statistics); the backward
// reads only the per-tensor lists'.  Max of non-negative float bit patterns
// is exact and commutes, so the result does not depend on the schedule.
constexpr int64_t RED_FLAT = 256 * 16;

// partials per entry, entries, per-token mode of list l
__host__ __device__ __forceinline__ int64_t red_np(const TrArgs& a, int l) {
  return l == 0 ? a.nch_o : l == 1 ? a.ntr_o : l == 2 ? a.ntr_gy : a.ntr_t;
}
__host__ __device__ __forceinline__ int64_t red_len(const TrArgs& a, int l) {
  return l == 0 ? a.T : l == 2 ? a.O : a.I;
}
__host__ __device__ __forceinline__ bool red_tok(const TrArgs& a, int l) {
  return l < 2 ? a.gx_tok != 0 : a.gw_tok != 0;
}
__host__ __device__ __forceinline__ int red_ent(int64_t np) {
  return np <= 32 ? 64 : np <= 64 ? 32 : 16;
}

// Blocks of the reduce: the per-entry blocks of the per-token lists (order
// 0, 2, 3, 1), then the flat blocks of the per-tensor lists (same order).
// Host and device use the same counts.
__host__ __device__ __forceinline__ int64_t red_tok_blocks(const TrArgs& a, int l) {
  if (!red_tok(a, l)) return 0;
  const int e = red_ent(red_np(a, l));
  return (red_len(a, l) + e - 1) / e;
}
__host__ __device__ __forceinline__ int64_t red_flat_blocks(const TrArgs& a, int l) {
  if (red_tok(a, l)) return 0;
  return (red_np(a, l) * red_len(a, l) + RED_FLAT - 1) / RED_FLAT;
}
__host__ __device__ __forceinline__ int64_t red_blocks(const TrArgs& a) {
  return red_tok_blocks(a, 0) + red_tok_blocks(a, 2) + red_tok_blocks(a, 3) +
         red_tok_blocks(a, 1) + red_flat_blocks(a, 0) + red_flat_blocks(a, 2) +
         red_flat_blocks(a, 3) + red_flat_blocks(a, 1);
}

#if HLQ_TR_N == 16
// The fields of list L (chosen at compile time: selected at run time, the
// argument block was copied to scratch memory).
template <int L>
__device__ __forceinline__ const float* red_part(const TrArgs& a) {
  if constexpr (L == 0) return a.part_gy;
  else if constexpr (L == 1) return a.part_w;
  else if constexpr (L == 2) return a.part_gyl;
  else return a.part_xl;
}

// Flat block b of per-tensor list L: its maximum into slot blockIdx % 64.
template <int L>
__device__ void red_flat_block(const TrArgs& a, int64_t b, float* wpart) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const float* lp = red_part<L>(a);
  const int64_t n = red_np(a, L) * red_len(a, L), c0 = b * RED_FLAT;
  float m = 0.f;
  if ((n & 3) == 0) {
    float4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t i = c0 + 4 * ((int64_t)u * 256 + tid);
      v[u] = i < n ? *reinterpret_cast<const float4*>(lp + i) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) m = nnmax(m, nnmax(nnmax(v[u].x, v[u].y), nnmax(v[u].z, v[u].w)));
  } else {
    for (int64_t i = c0 + tid; i < c0 + RED_FLAT && i < n; i += 256) m = nnmax(m, lp[i]);
  }
  m = wave_max(m);
  if (lane == 0) wpart[wv] = m;
  __syncthreads();
  if (tid == 0) {
    const float r = nnmax(nnmax(wpart[0], wpart[1]), nnmax(wpart[2], wpart[3]));
    if (r > 0.f) atomicMax(a.tmax + L * TMAX_SLOTS + (int)(blockIdx.x % TMAX_SLOTS), __float_as_uint(r));
  }
}

// Entries b * E .. of per-token list L: thread (s, e) folds partials
// s, s + S, ... of entry e, rounds of eight loads issued before their maxima
// (every load issued, past the list's end from partial 0, then dropped:
// predicated loads became one branch each).
template <int L>
__device__ void red_entry_block(const TrArgs& a, int64_t b, float* wpart) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t lnp = red_np(a, L), len = red_len(a, L);
  const int E = red_ent(lnp), S = 256 / E;
  const int e_loc = tid % E, sub = tid / E;
  const int64_t idx = b * E + e_loc;
  const bool valid = idx < len;
  const float* p = red_part<L>(a) + idx;
  const int64_t np = valid ? lnp : 0;
  constexpr int U = 8;
  float mx[U];
#pragma unroll
  for (int u = 0; u < U; ++u) mx[u] = 0.f;
  for (int64_t k = sub; k < np; k += (int64_t)U * S) {
    float v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t kk = k + (int64_t)u * S;
      v[u] = p[(kk < np ? kk : 0) * len];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) mx[u] = nnmax(mx[u], k + (int64_t)u * S < np ? v[u] : 0.f);
  }
#pragma unroll
  for (int u = 1; u < U; ++u) mx[0] = nnmax(mx[0], mx[u]);
  wpart[sub * E + e_loc] = mx[0];
  __syncthreads();
  float m = 0.f;
  if (tid < E) {
    m = wpart[tid];
    for (int q = 1; q < S; ++q) m = nnmax(m, wpart[q * E + tid]);
    if (valid) {
      if constexpr (L == 0) {
        a.inv_gy[idx] = inv_of(m, 7.f); a.s_gy[idx] = scale_of(m, 7.f);
      } else if constexpr (L == 2) {
        a.inv_gyl[idx] = inv_of(m, 127.f); a.s_gyl[idx] = scale_of(m, 127.f);
      } else if constexpr (L == 3) {
        a.inv_xl[idx] = inv_of(m, 127.f); a.s_xl[idx] = scale_of(m, 127.f);
      } else {
        a.inv_w[idx] = inv_of(m, 7.f); a.s_w[idx] = scale_of(m, 7.f);
      }
    }
  }
  if (a.tok_tmax && wv == 0) {  // uniform; the E <= 64 entries are wave 0's threads
    const float v = wave_max(m);
    if (lane == 0 && v > 0.f)
      atomicMax(a.tmax + L * TMAX_SLOTS + (int)(blockIdx.x % TMAX_SLOTS), __float_as_uint(v));
  }
}

__global__ __launch_bounds__(256) void k_tr_reduce(TrArgs a) {
  __shared__ float wpart[256];
  int64_t b = blockIdx.x;
  int64_t nb = red_tok_blocks(a, 0);
  if (b < nb) { red_entry_block<0>(a, b, wpart); return; }
  b -= nb; nb = red_tok_blocks(a, 2);
  if (b < nb) { red_entry_block<2>(a, b, wpart); return; }
  b -= nb; nb = red_tok_blocks(a, 3);
  if (b < nb) { red_entry_block<3>(a, b, wpart); return; }
  b -= nb; nb = red_tok_blocks(a, 1);
  if (b < nb) { red_entry_block<1>(a, b, wpart); return; }
  b -= nb; nb = red_flat_blocks(a, 0);
  if (b < nb) { red_flat_block<0>(a, b, wpart); return; }
  b -= nb; nb = red_flat_blocks(a, 2);
  if (b < nb) { red_flat_block<2>(a, b, wpart); return; }
  b -= nb; nb = red_flat_blocks(a, 3);
  if (b < nb) { red_flat_block<3>(a, b, wpart); return; }
  b -= nb; nb = red_flat_blocks(a, 1);
  if (b < nb) red_flat_block<1>(a, b, wpart);
}
#endif

// One object per block size n: the build compiles this file with
// HLQ_TR_N = 16, 32, 64 and 128 (the k_tr instantiations dominate the build
// time).  The object of n = 16 also holds the generic launchers.
#ifndef HLQ_TR_N
#error "compile hlq_tr.hip with -DHLQ_TR_N=16, 32, 64 or 128"
#endif
#define HLQ_CAT2(a, b) a##b
#define HLQ_CAT(a, b) HLQ_CAT2(a, b)

template <int PASS, bool F32, bool LEAN = false>
static hipError_t tr_dispatch(int r, dim3 g, hipStream_t s, const TrArgs& a) {
  constexpr int NN = HLQ_TR_N;
#define HLQ_TR(RR) hipLaunchKernelGGL((k_tr<PASS, NN, RR, F32, LEAN>), g, dim3(256), 0, s, a)
  switch (r) {
    case 1: HLQ_TR(1); break;
    case 2: HLQ_TR(2); break;
    case 4: HLQ_TR(4); break;
    case 8: HLQ_TR(8); break;
    case 16: HLQ_TR(16); break;
    case 32: if constexpr (NN >= 32) { HLQ_TR((NN >= 32 ? 32 : 1)); break; } else return hipErrorInvalidValue;
    case 64: if constexpr (NN >= 64) { HLQ_TR((NN >= 64 ? 64 : 1)); break; } else return hipErrorInvalidValue;
    case 128: if constexpr (NN >= 128) { HLQ_TR((NN >= 128 ? 128 : 1)); break; } else return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
#undef HLQ_TR
  return hipGetLastError();
}

hipError_t HLQ_CAT(launch_tr_n, HLQ_TR_N)(const TrArgs& a, int pass, int r, dim3 g, hipStream_t s) {
  const bool f32 = a.gy_dt == 0 || a.w_dt == 0;
  // register-lean g_y tiles when the LDS-engine workgroups outnumber theirs
  const bool lean = a.gyreg_wgs > 0 && a.gyreg_wgs < a.gy_workers + a.wg_x + a.wg_w;
  if (pass == PASS_MAX && lean)
    return f32 ? tr_dispatch<PASS_MAX, true, true>(r, g, s, a)
               : tr_dispatch<PASS_MAX, false, true>(r, g, s, a);
  if (pass == PASS_MAX)
    return f32 ? tr_dispatch<PASS_MAX, true>(r, g, s, a) : tr_dispatch<PASS_MAX, false>(r, g, s, a);
  return f32 ? tr_dispatch<PASS_QUANT, true>(r, g, s, a) : tr_dispatch<PASS_QUANT, false>(r, g, s, a);
}

#if HLQ_TR_N == 16
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
    a.gyreg_wgs = a.wg_gy;
  }
  // eight slots per XCD row: each XCD takes an eighth of every job list
  const int64_t slots = (a.gyreg_wgs + 7) / 8 + (a.gy_workers + 7) / 8 + (a.wg_x + 7) / 8 +
                        (a.wg_w + 7) / 8;
  if (slots <= 0) return hipSuccess;
  dim3 g((unsigned)(slots * 8));
  switch (n) {
    case 16: return launch_tr_n16(a, pass, r, g, s);
    case 32: return launch_tr_n32(a, pass, r, g, s);
    case 64: return launch_tr_n64(a, pass, r, g, s);
    case 128: return launch_tr_n128(a, pass, r, g, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_tr_reduce(const TrArgs& a, hipStream_t s) {
  const int64_t nb = red_blocks(a);
  if (nb <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_tr_reduce, dim3((unsigned)nb), dim3(256), 0, s, a);
  return hipGetLastError();
}
#endif

}  // namespace hlq
