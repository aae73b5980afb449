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

template <int QMAX>
__device__ __forceinline__ int quant1(float v, float inv) {
  float q = __builtin_rintf(v * inv);
  q = fminf(fmaxf(q, -(float)QMAX), (float)QMAX);
  return (int)q;
}

__device__ __forceinline__ uint32_t pack8_int4(const int (&q)[8]) {
  uint32_t u = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) u |= (uint32_t)(q[k] & 0xF) << (4 * k);
  return u;
}

__device__ __forceinline__ float inv_of(float a, float qmax) { return a == 0.f ? 0.f : qmax / a; }
__device__ __forceinline__ float scale_of(float a, float qmax) { return a == 0.f ? 0.f : a / qmax; }

// ------------------------------------------------------------ small utility kernels

__global__ void k_fill_u32(uint32_t* p, int64_t n, uint32_t v) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// Zero bytes [from, pitch) of each of `rows` rows (K padding of GEMM operands).
__global__ void k_zero_pad(uint8_t* p, int64_t rows, int64_t pitch, int64_t from) {
  const int64_t w = pitch - from;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= rows * w) return;
  int64_t r = i / w, c = i % w;
  p[r * pitch + from + c] = 0;
}

// ------------------------------------------------------------ ACBP pack
// One wave per token row: absmax over the row, then INT4 codes (qmax 7).

template <int DT>
__global__ __launch_bounds__(256) void k_acbp(const void* __restrict__ x, int64_t T,
                                              int64_t I, uint8_t* __restrict__ codes,
                                              float* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= T) return;
  const int64_t base = row * I;
  float a = 0.f;
  for (int64_t c = lane * 8; c < I; c += 512) {
    float v[8];
    load8<DT>(x, base + c, v);
#pragma unroll
    for (int k = 0; k < 8; ++k) a = fmaxf(a, fabsf(v[k]));
  }
  a = wave_max(a);
  const float inv = inv_of(a, 7.f);
  uint8_t* out = codes + row * (I / 2);
  for (int64_t c = lane * 8; c < I; c += 512) {
    float v[8];
    load8<DT>(x, base + c, v);
    int q[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) q[k] = quant1<7>(v[k], inv);
    *reinterpret_cast<uint32_t*>(out + c / 2) = pack8_int4(q);
  }
  if (lane == 0) scales[row] = scale_of(a, 7.f);
}

// ------------------------------------------------------------ g_x operand A
// Rows of g_y [T][O]: block FWHT along O (n/8 lanes per block, 8 elements per
// lane), absmax per row, INT4 codes into [T][kxb] with zero K padding.
// NCH > 0: the transformed row (<= NCH*512 elements) stays in registers;
// NCH == 0: the second pass reloads and transforms again.

template <int DT, int MODE, int NCH>
__global__ __launch_bounds__(256) void k_rows(const void* __restrict__ gy, int64_t T,
                                              int64_t O, int n, int64_t kxb,
                                              uint8_t* __restrict__ q,
                                              float* __restrict__ scale,
                                              uint32_t* __restrict__ gmax) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= T) return;
  const int lpb = n / 8;
  const int64_t base = row * O;
  const int64_t kx = kxb * 2;
  const int nch = (int)((kx + 511) / 512);

  float buf[NCH > 0 ? NCH : 1][8];
  float a = 0.f;
  if constexpr (MODE != QUANT_GLOBAL) {
    for (int ch = 0; ch < nch; ++ch) {
      const int64_t c = (int64_t)ch * 512 + lane * 8;
      float v[8];
      if (c < O) load8<DT>(gy, base + c, v);
      else {
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = 0.f;
      }
      fwht8(v);
      fwht_lanes(v, lane, lpb);
#pragma unroll
      for (int k = 0; k < 8; ++k) a = fmaxf(a, fabsf(v[k]));
      if constexpr (NCH > 0) {
#pragma unroll
        for (int cc = 0; cc < NCH; ++cc)
          if (cc == ch) {
#pragma unroll
            for (int k = 0; k < 8; ++k) buf[cc][k] = v[k];
          }
      }
    }
    a = wave_max(a);
  }
  if constexpr (MODE == ABS_ONLY) {
    if (lane == 0) atomicMax(gmax, __float_as_uint(a));
    return;
  } else {
    if constexpr (MODE == QUANT_GLOBAL) a = __uint_as_float(*gmax);
    const float inv = inv_of(a, 7.f);
    uint8_t* out = q + row * kxb;
    for (int ch = 0; ch < nch; ++ch) {
      const int64_t c = (int64_t)ch * 512 + lane * 8;
      float v[8];
      if constexpr (NCH > 0 && MODE == QUANT_OWN) {
#pragma unroll
        for (int cc = 0; cc < NCH; ++cc)
          if (cc == ch) {
#pragma unroll
            for (int k = 0; k < 8; ++k) v[k] = buf[cc][k];
          }
      } else {
        if (c < O) load8<DT>(gy, base + c, v);
        else {
#pragma unroll
          for (int k = 0; k < 8; ++k) v[k] = 0.f;
        }
        fwht8(v);
        fwht_lanes(v, lane, lpb);
      }
      if (c < kx) {
        int qq[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) qq[k] = quant1<7>(v[k], inv);
        *reinterpret_cast<uint32_t*>(out + c / 2) = (c < O) ? pack8_int4(qq) : 0u;
      }
    }
    if (lane == 0) {
      if constexpr (MODE == QUANT_OWN) scale[row] = scale_of(a, 7.f);
      else if (row == 0) scale[0] = scale_of(a, 7.f);
    }
  }
}

// ------------------------------------------------------------ g_x operand B
// Columns of w [O][I]: one thread per column i, a run of SEG = max(n, 64) rows
// per block row of the grid.  FWHT of n rows in registers; absmax per column
// (pass ABS_ONLY, into colmax and gmax) or INT4 codes stored transposed into
// [I][kxb] (pass QUANT_OWN: per-column scale, QUANT_GLOBAL: tensor scale).

template <int DT, int MODE, int N>
__global__ __launch_bounds__(64) void k_cols(const void* __restrict__ w, int64_t O,
                                             int64_t I, int64_t kxb, int seg,
                                             uint8_t* __restrict__ q,
                                             float* __restrict__ scale,
                                             uint32_t* __restrict__ colmax,
                                             uint32_t* __restrict__ gmax) {
  const int64_t i = (int64_t)blockIdx.x * 64 + threadIdx.x;
  const bool active = i < I;
  const int64_t ic = active ? i : I - 1;
  const int64_t o_begin = (int64_t)blockIdx.y * seg;
  float a = 0.f;
  float inv = 0.f;
  if constexpr (MODE == QUANT_OWN) {
    a = __uint_as_float(colmax[ic]);
    inv = inv_of(a, 7.f);
  } else if constexpr (MODE == QUANT_GLOBAL) {
    a = __uint_as_float(*gmax);
    inv = inv_of(a, 7.f);
  }
  for (int64_t o0 = o_begin; o0 < o_begin + seg && o0 < O; o0 += N) {
    float v[N];
#pragma unroll
    for (int k = 0; k < N; ++k) v[k] = load1<DT>(w, (o0 + k) * I + ic);
#pragma unroll
    for (int h = 1; h < N; h <<= 1) {
#pragma unroll
      for (int k = 0; k < N; ++k) {
        if ((k & h) == 0) {
          float x0 = v[k], x1 = v[k + h];
          v[k] = x0 + x1;
          v[k + h] = x0 - x1;
        }
      }
    }
    if constexpr (MODE == ABS_ONLY) {
#pragma unroll
      for (int k = 0; k < N; ++k) a = fmaxf(a, fabsf(v[k]));
    } else {
      uint32_t packed[N / 8];
#pragma unroll
      for (int g = 0; g < N / 8; ++g) {
        int qq[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) qq[k] = quant1<7>(v[g * 8 + k], inv);
        packed[g] = pack8_int4(qq);
      }
      if (active) {
        uint8_t* dst = q + i * kxb + o0 / 2;
        if constexpr (N == 16) {
          *reinterpret_cast<uint2*>(dst) = make_uint2(packed[0], packed[1]);
        } else {
#pragma unroll
          for (int g = 0; g < N / 8; g += 4)
            *reinterpret_cast<uint4*>(dst + g * 4) =
                make_uint4(packed[g], packed[g + 1], packed[g + 2], packed[g + 3]);
        }
      }
    }
  }
  if constexpr (MODE == ABS_ONLY) {
    if (active) atomicMax(colmax + i, __float_as_uint(a));
    float wm = wave_max(active ? a : 0.f);
    if (threadIdx.x == 0) atomicMax(gmax, __float_as_uint(wm));
  } else {
    if (active && blockIdx.y == 0) {
      if constexpr (MODE == QUANT_OWN) scale[i] = scale_of(a, 7.f);
      else if (i == 0) scale[0] = scale_of(a, 7.f);
    }
  }
}

// ------------------------------------------------------------ g_w operands
// Low-rank Hadamard along T.  In block b of n tokens the kept rows j*(n/r) of
// H_n equal H_r applied to the r sums of n/r consecutive tokens (the low
// bits of the row index are zero), so each thread forms those group sums in
// adjacent-pair tree order (identical fp32 result to the first log2(n/r)
// butterfly stages) and then applies H_r in registers.
//
// Block = 32 column chunks (x) * 8 token segments (y); a chunk is CPT
// consecutive columns, a segment SEGB consecutive blocks of n tokens.
// ABS_ONLY: per-column maxima -> colmax (atomicMax) and the tensor max ->
// gmax.  QUANT_*: INT8 codes stored transposed into [C][kwb].

template <int KIND, int CPT>
__device__ __forceinline__ void hla_load(const void* src, const float* sx, int64_t t,
                                         int64_t C, int64_t c0, float (&v)[CPT]) {
  if constexpr (KIND == SRC_INT4) {
    const uint8_t* p = static_cast<const uint8_t*>(src) + t * (C / 2) + c0 / 2;
    uint32_t u;
    if constexpr (CPT == 8) u = *reinterpret_cast<const uint32_t*>(p);
    else if constexpr (CPT == 4) u = *reinterpret_cast<const uint16_t*>(p);
    else u = *p;
    const float s = sx[t];
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      int nib = (int)((u >> (4 * k)) & 0xFu);
      nib = (nib ^ 8) - 8;
      v[k] = s * (float)nib;
    }
  } else if constexpr (KIND == SRC_BF16) {
    const uint16_t* p = static_cast<const uint16_t*>(src) + t * C + c0;
    if constexpr (CPT == 8) {
      uint4 u = *reinterpret_cast<const uint4*>(p);
      uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        v[2 * k] = bf16_to_f32(w4[k] & 0xFFFFu);
        v[2 * k + 1] = bf16_to_f32(w4[k] >> 16);
      }
    } else if constexpr (CPT == 4) {
      uint2 u = *reinterpret_cast<const uint2*>(p);
      v[0] = bf16_to_f32(u.x & 0xFFFFu); v[1] = bf16_to_f32(u.x >> 16);
      v[2] = bf16_to_f32(u.y & 0xFFFFu); v[3] = bf16_to_f32(u.y >> 16);
    } else {
      uint32_t u = *reinterpret_cast<const uint32_t*>(p);
      v[0] = bf16_to_f32(u & 0xFFFFu); v[1] = bf16_to_f32(u >> 16);
    }
  } else {
    const float* p = static_cast<const float*>(src) + t * C + c0;
#pragma unroll
    for (int k = 0; k < CPT; k += 2) {
      float2 f = *reinterpret_cast<const float2*>(p + k);
      v[k] = f.x;
      v[k + 1] = f.y;
    }
  }
}

template <int R>
struct HlaLevels {  // stack depth for group sums of up to 128/R tokens
  static constexpr int value = (R >= 128) ? 1 : (R >= 64) ? 2 : (R >= 32) ? 3 : (R >= 16) ? 4
                             : (R >= 8) ? 5 : (R >= 4) ? 6 : (R >= 2) ? 7 : 8;
};

template <int KIND, int MODE, int R, int CPT>
__global__ __launch_bounds__(256) void k_hla(const void* __restrict__ src,
                                             const float* __restrict__ sx, int64_t T,
                                             int64_t C, int n, int segb, int64_t kwb,
                                             uint8_t* __restrict__ q,
                                             float* __restrict__ scale,
                                             uint32_t* __restrict__ colmax,
                                             uint32_t* __restrict__ gmax) {
  constexpr int LV = HlaLevels<R>::value;
  __shared__ float red[8][32][CPT];
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  const int64_t ncc = C / CPT;
  const int64_t cc = (int64_t)blockIdx.x * 32 + tx;
  const bool col_ok = cc < ncc;
  const int64_t c0 = (col_ok ? cc : ncc - 1) * CPT;
  const int64_t nblk = T / n;
  const int64_t b_begin = ((int64_t)blockIdx.y * 8 + ty) * segb;
  const int g = n / R;
  int logg = 0;
  while ((1 << logg) < g) ++logg;

  float amax[CPT];
  float inv[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    amax[c] = 0.f;
    inv[c] = 0.f;
  }
  if constexpr (MODE == QUANT_OWN) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      amax[c] = __uint_as_float(colmax[c0 + c]);
      inv[c] = inv_of(amax[c], 127.f);
    }
  } else if constexpr (MODE == QUANT_GLOBAL) {
    const float a = __uint_as_float(*gmax);
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      amax[c] = a;
      inv[c] = inv_of(a, 127.f);
    }
  }

  for (int64_t b = b_begin; b < b_begin + segb && b < nblk; ++b) {
    float gs[R][CPT];
#pragma unroll
    for (int j = 0; j < R; ++j) {
      float stk[LV][CPT];
      const int64_t t0 = b * n + (int64_t)j * g;
      for (int k = 0; k < g; ++k) {
        float v[CPT];
        hla_load<KIND, CPT>(src, sx, t0 + k, C, c0, v);
        const int tz = __builtin_ctz(~(unsigned)k);  // trailing ones of k
#pragma unroll
        for (int l = 0; l < LV - 1; ++l) {
          if (l < tz) {
#pragma unroll
            for (int c = 0; c < CPT; ++c) v[c] = stk[l][c] + v[c];
          }
        }
#pragma unroll
        for (int l = 0; l < LV; ++l) {
          if (l == tz) {
#pragma unroll
            for (int c = 0; c < CPT; ++c) stk[l][c] = v[c];
          }
        }
      }
#pragma unroll
      for (int l = 0; l < LV; ++l) {
        if (l == logg) {
#pragma unroll
          for (int c = 0; c < CPT; ++c) gs[j][c] = stk[l][c];
        }
      }
    }
#pragma unroll
    for (int h = 1; h < R; h <<= 1) {
#pragma unroll
      for (int j = 0; j < R; ++j) {
        if ((j & h) == 0) {
#pragma unroll
          for (int c = 0; c < CPT; ++c) {
            float x0 = gs[j][c], x1 = gs[j + h][c];
            gs[j][c] = x0 + x1;
            gs[j + h][c] = x0 - x1;
          }
        }
      }
    }
    if constexpr (MODE == ABS_ONLY) {
#pragma unroll
      for (int j = 0; j < R; ++j)
#pragma unroll
        for (int c = 0; c < CPT; ++c) amax[c] = fmaxf(amax[c], fabsf(gs[j][c]));
    } else if (col_ok) {
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        uint8_t* dst = q + (c0 + c) * kwb + b * R;
        uint32_t words[(R + 3) / 4];
#pragma unroll
        for (int wi = 0; wi < (R + 3) / 4; ++wi) words[wi] = 0;
#pragma unroll
        for (int j = 0; j < R; ++j)
          words[j / 4] |= (uint32_t)(quant1<127>(gs[j][c], inv[c]) & 0xFF) << (8 * (j % 4));
        if constexpr (R == 1) *dst = (uint8_t)words[0];
        else if constexpr (R == 2) *reinterpret_cast<uint16_t*>(dst) = (uint16_t)words[0];
        else if constexpr (R == 4) *reinterpret_cast<uint32_t*>(dst) = words[0];
        else if constexpr (R == 8) *reinterpret_cast<uint2*>(dst) = make_uint2(words[0], words[1]);
        else {
#pragma unroll
          for (int wi = 0; wi < R / 4; wi += 4)
            *reinterpret_cast<uint4*>(dst + wi * 4) =
                make_uint4(words[wi], words[wi + 1], words[wi + 2], words[wi + 3]);
        }
      }
    }
  }

  if constexpr (MODE == ABS_ONLY) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) red[ty][tx][c] = amax[c];
    __syncthreads();
    if (ty == 0) {
      float bm = 0.f;
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        float m = red[0][tx][c];
#pragma unroll
        for (int y = 1; y < 8; ++y) m = fmaxf(m, red[y][tx][c]);
        if (col_ok) {
          atomicMax(colmax + c0 + c, __float_as_uint(m));
          bm = fmaxf(bm, m);
        }
      }
      // ty == 0 is the low half of wave 0: reduce over its 32 lanes
#pragma unroll
      for (int m = 16; m >= 1; m >>= 1) bm = fmaxf(bm, __shfl_xor(bm, m));
      if (tx == 0) atomicMax(gmax, __float_as_uint(bm));
    }
  } else {
    if (col_ok && blockIdx.y == 0 && ty == 0) {
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        if constexpr (MODE == QUANT_OWN) scale[c0 + c] = scale_of(amax[c], 127.f);
        else if (c0 + c == 0) scale[0] = scale_of(amax[c], 127.f);
      }
    }
  }
}

// ------------------------------------------------------------ integer GEMM
// C[m][n] = sum_k A[m][k] * B[n][k]; A [M][pitch], B [N][pitch] bytes, K
// contiguous and zero-padded to a multiple of 64 bytes.  INT4 operands hold
// two codes per byte; they are widened on the LDS->register path into int8
// lanes holding 16*code (low nibble shifted up, high nibble masked in place),
// so the INT32 sum is 256 times the code product sum and is shifted back
// exactly.  The nibble order inside a lane is permuted the same way for both
// operands, which leaves the dot product unchanged.
//
// v_mfma_i32_16x16x64_i8: operand X (16 rows of D) comes from B's rows (n),
// operand Y (16 columns of D) from A's rows (m); lane l then holds
// D[4*(l/16)+e][l%16] = C[m0 + l%16][n0 + 4*(l/16) + e], four consecutive n,
// which the epilogue stores as one 16-byte vector.
//
// 256 threads = 4 waves in a 2x2 grid, wave tile (BM/2) x (BN/2), 64-byte K
// stages double-buffered in LDS (one barrier per stage).

constexpr int KST = 64;        // bytes of K per stage
constexpr int LROW = KST + 16; // LDS row pitch (padding spreads banks)

__device__ __forceinline__ v4i widen_int4(uint2 p) {
  v4i r;
  r[0] = (int)((p.x << 4) & 0xF0F0F0F0u);
  r[1] = (int)(p.x & 0xF0F0F0F0u);
  r[2] = (int)((p.y << 4) & 0xF0F0F0F0u);
  r[3] = (int)(p.y & 0xF0F0F0F0u);
  return r;
}

template <int L, int ROWS>
__device__ __forceinline__ void gemm_gload(uint4 (&r)[L], const uint8_t* __restrict__ P,
                                           int64_t row0, int64_t rows, int64_t pitch,
                                           int64_t kb, int tid) {
#pragma unroll
  for (int i = 0; i < L; ++i) {
    const int c = tid + 256 * i;
    int64_t rr = row0 + (c >> 2);
    rr = rr < rows ? rr : rows - 1;
    r[i] = *reinterpret_cast<const uint4*>(P + rr * pitch + kb + (c & 3) * 16);
  }
}

template <int L>
__device__ __forceinline__ void gemm_sstore(const uint4 (&r)[L], uint8_t* lds, int tid) {
#pragma unroll
  for (int i = 0; i < L; ++i) {
    const int c = tid + 256 * i;
    *reinterpret_cast<uint4*>(lds + (c >> 2) * LROW + (c & 3) * 16) = r[i];
  }
}

template <bool INT4, int BM, int BN, int EPI>
__global__ __launch_bounds__(256) void k_gemm(const uint8_t* __restrict__ A,
                                              const uint8_t* __restrict__ B, int64_t M,
                                              int64_t N, int64_t pitch,
                                              int64_t stages_per_split,
                                              const float* __restrict__ sa, int sa_step,
                                              const float* __restrict__ sb, int sb_step,
                                              float alpha, float* __restrict__ C,
                                              int32_t* __restrict__ Ci) {
  constexpr int TM = BM / 32, TN = BN / 32;   // 16x16 tiles per wave
  constexpr int LA = BM * KST / 16 / 256;     // 16-byte loads per thread
  constexpr int LB = BN * KST / 16 / 256;
  __shared__ __attribute__((aligned(16))) uint8_t As[2][BM * LROW];
  __shared__ __attribute__((aligned(16))) uint8_t Bs[2][BN * LROW];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t m0 = (int64_t)blockIdx.x * BM;
  const int64_t n0 = (int64_t)blockIdx.y * BN;
  const int64_t kb0 = (int64_t)blockIdx.z * stages_per_split * KST;
  const int64_t kb1 = kb0 + stages_per_split * KST;

  uint4 ra[LA], rb[LB];
  v4i acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = v4i{0, 0, 0, 0};

  const int fr = lane & 15, fg = lane >> 4;
  gemm_gload<LA, BM>(ra, A, m0, M, pitch, kb0, tid);
  gemm_gload<LB, BN>(rb, B, n0, N, pitch, kb0, tid);
  gemm_sstore<LA>(ra, As[0], tid);
  gemm_sstore<LB>(rb, Bs[0], tid);
  __syncthreads();
  int cur = 0;
  for (int64_t kb = kb0; kb < kb1; kb += KST) {
    // prefetch the next stage (the last iteration reloads its own stage, in
    // bounds, and parks it in the idle buffer)
    const int64_t kn = kb + KST < kb1 ? kb + KST : kb;
    gemm_gload<LA, BM>(ra, A, m0, M, pitch, kn, tid);
    gemm_gload<LB, BN>(rb, B, n0, N, pitch, kn, tid);
    const uint8_t* as = As[cur];
    const uint8_t* bs = Bs[cur];
    if constexpr (INT4) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        v4i ya[TM], xb[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i)
          ya[i] = widen_int4(*reinterpret_cast<const uint2*>(
              as + (wm * (BM / 2) + i * 16 + fr) * LROW + ks * 32 + fg * 8));
#pragma unroll
        for (int j = 0; j < TN; ++j)
          xb[j] = widen_int4(*reinterpret_cast<const uint2*>(
              bs + (wn * (BN / 2) + j * 16 + fr) * LROW + ks * 32 + fg * 8));
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(xb[j], ya[i], acc[i][j], 0, 0, 0);
      }
    } else {
      v4i ya[TM], xb[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        ya[i] = *reinterpret_cast<const v4i*>(as + (wm * (BM / 2) + i * 16 + fr) * LROW + fg * 16);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        xb[j] = *reinterpret_cast<const v4i*>(bs + (wn * (BN / 2) + j * 16 + fr) * LROW + fg * 16);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(xb[j], ya[i], acc[i][j], 0, 0, 0);
    }
    gemm_sstore<LA>(ra, As[cur ^ 1], tid);
    gemm_sstore<LB>(rb, Bs[cur ^ 1], tid);
    __syncthreads();
    cur ^= 1;
  }

  constexpr int SH = INT4 ? 8 : 0;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int64_t m = m0 + wm * (BM / 2) + i * 16 + fr;
    if (m >= M) continue;
    const float s_m = (EPI == EPI_F32) ? sa[m * sa_step] * alpha : 0.f;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int64_t nn = n0 + wn * (BN / 2) + j * 16 + fg * 4;
      if (nn >= N) continue;
      v4i r = acc[i][j];
      if constexpr (EPI == EPI_F32) {
        float4 o;
        o.x = (float)(r[0] >> SH) * s_m * sb[(nn + 0) * sb_step];
        o.y = (float)(r[1] >> SH) * s_m * sb[(nn + 1) * sb_step];
        o.z = (float)(r[2] >> SH) * s_m * sb[(nn + 2) * sb_step];
        o.w = (float)(r[3] >> SH) * s_m * sb[(nn + 3) * sb_step];
        *reinterpret_cast<float4*>(C + m * N + nn) = o;
      } else {
        int32_t* dst = Ci + (EPI == EPI_PARTIAL ? (int64_t)blockIdx.z * M * N : 0) + m * N + nn;
        *reinterpret_cast<int4*>(dst) = make_int4(r[0] >> SH, r[1] >> SH, r[2] >> SH, r[3] >> SH);
      }
    }
  }
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
  *reinterpret_cast<float4*>(C + e) = o;
}

// ------------------------------------------------------------ launchers

static inline unsigned cdiv(int64_t a, int64_t b) { return (unsigned)((a + b - 1) / b); }

hipError_t launch_fill_u32(uint32_t* p, int64_t n, uint32_t v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill_u32, dim3(cdiv(n, 256)), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

hipError_t launch_zero_pad(uint8_t* p, int64_t rows, int64_t pitch, int64_t from,
                           hipStream_t s) {
  const int64_t total = rows * (pitch - from);
  if (total <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_zero_pad, dim3(cdiv(total, 256)), dim3(256), 0, s, p, rows, pitch,
                     from);
  return hipGetLastError();
}

hipError_t launch_acbp(const void* x, int dtype, int64_t T, int64_t I, uint8_t* codes,
                       float* scales, hipStream_t s) {
  dim3 grid(cdiv(T, 4)), block(256);
  if (dtype == 0) hipLaunchKernelGGL(k_acbp<0>, grid, block, 0, s, x, T, I, codes, scales);
  else hipLaunchKernelGGL(k_acbp<1>, grid, block, 0, s, x, T, I, codes, scales);
  return hipGetLastError();
}

template <int DT, int MODE>
static void rows_dispatch(int nch, dim3 g, dim3 b, hipStream_t s, const void* gy,
                          int64_t T, int64_t O, int n, int64_t kxb, uint8_t* q,
                          float* scale, uint32_t* gmax) {
#define HLQ_ROWS(NC) hipLaunchKernelGGL((k_rows<DT, MODE, NC>), g, b, 0, s, gy, T, O, n, kxb, q, scale, gmax)
  switch (nch) {
    case 1: HLQ_ROWS(1); break;
    case 2: HLQ_ROWS(2); break;
    case 3: HLQ_ROWS(3); break;
    case 4: HLQ_ROWS(4); break;
    case 5: case 6: HLQ_ROWS(6); break;
    case 7: case 8: HLQ_ROWS(8); break;
    default: HLQ_ROWS(0); break;
  }
#undef HLQ_ROWS
}

hipError_t launch_rows(const void* gy, int dtype, int64_t T, int64_t O, int n,
                       int64_t kxb, uint8_t* q, float* scale, uint32_t* gmax,
                       AbsMode mode, hipStream_t s) {
  dim3 grid(cdiv(T, 4)), block(256);
  const int nch = (int)cdiv(kxb * 2, 512);
  if (dtype == 0) {
    if (mode == ABS_ONLY) rows_dispatch<0, ABS_ONLY>(nch, grid, block, s, gy, T, O, n, kxb, q, scale, gmax);
    else if (mode == QUANT_OWN) rows_dispatch<0, QUANT_OWN>(nch, grid, block, s, gy, T, O, n, kxb, q, scale, gmax);
    else rows_dispatch<0, QUANT_GLOBAL>(0, grid, block, s, gy, T, O, n, kxb, q, scale, gmax);
  } else {
    if (mode == ABS_ONLY) rows_dispatch<1, ABS_ONLY>(nch, grid, block, s, gy, T, O, n, kxb, q, scale, gmax);
    else if (mode == QUANT_OWN) rows_dispatch<1, QUANT_OWN>(nch, grid, block, s, gy, T, O, n, kxb, q, scale, gmax);
    else rows_dispatch<1, QUANT_GLOBAL>(0, grid, block, s, gy, T, O, n, kxb, q, scale, gmax);
  }
  return hipGetLastError();
}

template <int DT, int MODE>
static void cols_dispatch(int n, dim3 g, dim3 b, hipStream_t s, const void* w,
                          int64_t O, int64_t I, int64_t kxb, int seg, uint8_t* q,
                          float* scale, uint32_t* colmax, uint32_t* gmax) {
#define HLQ_COLS(NN) hipLaunchKernelGGL((k_cols<DT, MODE, NN>), g, b, 0, s, w, O, I, kxb, seg, q, scale, colmax, gmax)
  switch (n) {
    case 16: HLQ_COLS(16); break;
    case 32: HLQ_COLS(32); break;
    case 64: HLQ_COLS(64); break;
    default: HLQ_COLS(128); break;
  }
#undef HLQ_COLS
}

hipError_t launch_cols(const void* w, int dtype, int64_t O, int64_t I, int n,
                       int64_t kxb, uint8_t* q, float* scale, uint32_t* colmax,
                       uint32_t* gmax, AbsMode mode, hipStream_t s) {
  const int seg = n > 64 ? n : 64;
  dim3 grid(cdiv(I, 64), cdiv(O, seg)), block(64);
  if (dtype == 0) {
    if (mode == ABS_ONLY) cols_dispatch<0, ABS_ONLY>(n, grid, block, s, w, O, I, kxb, seg, q, scale, colmax, gmax);
    else if (mode == QUANT_OWN) cols_dispatch<0, QUANT_OWN>(n, grid, block, s, w, O, I, kxb, seg, q, scale, colmax, gmax);
    else cols_dispatch<0, QUANT_GLOBAL>(n, grid, block, s, w, O, I, kxb, seg, q, scale, colmax, gmax);
  } else {
    if (mode == ABS_ONLY) cols_dispatch<1, ABS_ONLY>(n, grid, block, s, w, O, I, kxb, seg, q, scale, colmax, gmax);
    else if (mode == QUANT_OWN) cols_dispatch<1, QUANT_OWN>(n, grid, block, s, w, O, I, kxb, seg, q, scale, colmax, gmax);
    else cols_dispatch<1, QUANT_GLOBAL>(n, grid, block, s, w, O, I, kxb, seg, q, scale, colmax, gmax);
  }
  return hipGetLastError();
}

template <int KIND, int MODE>
static void hla_dispatch(int r, dim3 g, dim3 b, hipStream_t s, const void* src,
                         const float* sx, int64_t T, int64_t C, int n, int segb,
                         int64_t kwb, uint8_t* q, float* scale, uint32_t* colmax,
                         uint32_t* gmax) {
#define HLQ_HLA(RR, CP) hipLaunchKernelGGL((k_hla<KIND, MODE, RR, CP>), g, b, 0, s, src, sx, T, C, n, segb, kwb, q, scale, colmax, gmax)
  switch (r) {
    case 1: HLQ_HLA(1, 8); break;
    case 2: HLQ_HLA(2, 8); break;
    case 4: HLQ_HLA(4, 8); break;
    case 8: HLQ_HLA(8, 8); break;
    case 16: HLQ_HLA(16, 8); break;
    case 32: HLQ_HLA(32, 4); break;
    case 64: HLQ_HLA(64, 2); break;
    default: HLQ_HLA(128, 2); break;
  }
#undef HLQ_HLA
}

static int hla_cpt(int r) { return r <= 16 ? 8 : (r == 32 ? 4 : 2); }

hipError_t launch_hla(const void* src, const float* src_scale, HlaSource kind,
                      int64_t T, int64_t C, int n, int r, int64_t kwb, uint8_t* q,
                      float* scale, uint32_t* colmax, uint32_t* gmax, AbsMode mode,
                      hipStream_t s) {
  const int cpt = hla_cpt(r);
  const int64_t ncc = C / cpt;
  const int64_t nblk = T / n;
  // enough token segments to give ~96k threads, at most 16 blocks each
  int64_t want_segs = (98304 + ncc - 1) / ncc;
  int64_t segb = (nblk + want_segs - 1) / want_segs;
  if (segb < 1) segb = 1;
  if (segb > 16) segb = 16;
  const int64_t nseg = (nblk + segb - 1) / segb;
  dim3 grid(cdiv(ncc, 32), cdiv(nseg, 8)), block(256);
#define HLQ_HLA_K(KD)                                                                        \
  do {                                                                                       \
    if (mode == ABS_ONLY) hla_dispatch<KD, ABS_ONLY>(r, grid, block, s, src, src_scale, T, C, n, (int)segb, kwb, q, scale, colmax, gmax); \
    else if (mode == QUANT_OWN) hla_dispatch<KD, QUANT_OWN>(r, grid, block, s, src, src_scale, T, C, n, (int)segb, kwb, q, scale, colmax, gmax); \
    else hla_dispatch<KD, QUANT_GLOBAL>(r, grid, block, s, src, src_scale, T, C, n, (int)segb, kwb, q, scale, colmax, gmax); \
  } while (0)
  if (kind == SRC_F32) HLQ_HLA_K(SRC_F32);
  else if (kind == SRC_BF16) HLQ_HLA_K(SRC_BF16);
  else HLQ_HLA_K(SRC_INT4);
#undef HLQ_HLA_K
  return hipGetLastError();
}

GemmPlan plan_gemm(int64_t M, int64_t N, int64_t kbytes) {
  GemmPlan p;
  p.stages = kbytes / KST;
  const int64_t target = 512;  // two blocks per CU
  auto tiles = [&](int bm, int bn) { return (int64_t)cdiv(M, bm) * cdiv(N, bn); };
  if (tiles(128, 128) >= target) { p.bm = 128; p.bn = 128; }
  else if (tiles(64, 128) >= target) { p.bm = 64; p.bn = 128; }
  else if (tiles(128, 64) >= target) { p.bm = 128; p.bn = 64; }
  else { p.bm = 64; p.bn = 64; }
  const int64_t t = tiles(p.bm, p.bn);
  int64_t sp = 1;
  while (t * sp * 2 <= target && p.stages / (sp * 2) >= 8 && sp < 8) sp *= 2;
  // splits must divide the stage count
  while (sp > 1 && p.stages % sp) sp /= 2;
  p.splits = (int)sp;
  return p;
}

template <bool I4, int EPI>
static void gemm_dispatch(int bm, int bn, dim3 g, hipStream_t s, const uint8_t* A,
                          const uint8_t* B, int64_t M, int64_t N, int64_t pitch,
                          int64_t sps, const float* sa, int sa_step, const float* sb,
                          int sb_step, float alpha, float* C, int32_t* Ci) {
#define HLQ_GEMM(BM_, BN_) hipLaunchKernelGGL((k_gemm<I4, BM_, BN_, EPI>), g, dim3(256), 0, s, A, B, M, N, pitch, sps, sa, sa_step, sb, sb_step, alpha, C, Ci)
  if (bm == 128 && bn == 128) HLQ_GEMM(128, 128);
  else if (bm == 64 && bn == 128) HLQ_GEMM(64, 128);
  else if (bm == 128 && bn == 64) HLQ_GEMM(128, 64);
  else HLQ_GEMM(64, 64);
#undef HLQ_GEMM
}

hipError_t launch_gemm(bool int4, const uint8_t* A, const uint8_t* B, int64_t M,
                       int64_t N, int64_t pitch, const GemmPlan& plan,
                       const float* sa, int sa_step, const float* sb, int sb_step,
                       float alpha, GemmEpi epi, float* C, int32_t* Ci,
                       int32_t* partial, hipStream_t s) {
  const int splits = epi == EPI_I32 ? 1 : plan.splits;
  const int64_t sps = plan.stages / splits;
  dim3 grid(cdiv(M, plan.bm), cdiv(N, plan.bn), splits);
  const bool use_partial = (epi == EPI_F32 && splits > 1);
  if (use_partial && partial == nullptr) return hipErrorInvalidValue;
  if (epi == EPI_F32 && (C == nullptr || sa == nullptr || sb == nullptr))
    return hipErrorInvalidValue;
  if (epi == EPI_I32 && Ci == nullptr) return hipErrorInvalidValue;
  const int e = use_partial ? EPI_PARTIAL : epi;
  int32_t* dst = use_partial ? partial : Ci;
  if (int4) {
    if (e == EPI_F32) gemm_dispatch<true, EPI_F32>(plan.bm, plan.bn, grid, s, A, B, M, N, pitch, sps, sa, sa_step, sb, sb_step, alpha, C, dst);
    else if (e == EPI_I32) gemm_dispatch<true, EPI_I32>(plan.bm, plan.bn, grid, s, A, B, M, N, pitch, sps, sa, sa_step, sb, sb_step, alpha, C, dst);
    else gemm_dispatch<true, EPI_PARTIAL>(plan.bm, plan.bn, grid, s, A, B, M, N, pitch, sps, sa, sa_step, sb, sb_step, alpha, C, dst);
  } else {
    if (e == EPI_F32) gemm_dispatch<false, EPI_F32>(plan.bm, plan.bn, grid, s, A, B, M, N, pitch, sps, sa, sa_step, sb, sb_step, alpha, C, dst);
    else if (e == EPI_I32) gemm_dispatch<false, EPI_I32>(plan.bm, plan.bn, grid, s, A, B, M, N, pitch, sps, sa, sa_step, sb, sb_step, alpha, C, dst);
    else gemm_dispatch<false, EPI_PARTIAL>(plan.bm, plan.bn, grid, s, A, B, M, N, pitch, sps, sa, sa_step, sb, sb_step, alpha, C, dst);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || !use_partial) return err;
  return launch_gemm_finalize(partial, splits, M, N, sa, sa_step, sb, sb_step, alpha, C, s);
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
