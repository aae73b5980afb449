// Device helpers shared by the gfx950 kernels of the HLQ/HOT backward:
// bf16 widening, in-register and cross-lane Walsh-Hadamard butterflies, the
// quantizer's rounding, nibble and FP6 packing.  Header-only, internal.
#pragma once

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

// Maximum of two values that are >= +0 and not NaN (maxima of magnitudes):
// their bit patterns order like the values, so one integer maximum does it.
// Unlike fmaxf it needs no NaN canonicalization of operands that come from
// lane exchanges or memory, and a DPP lane exchange folds into it.
__device__ __forceinline__ float nnmax(float a, float b) {
  return __uint_as_float(max(__float_as_uint(a), __float_as_uint(b)));
}

// Maximum over the wave of values >= +0 (every lane gets it).
__device__ __forceinline__ float wave_max(float a) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) a = nnmax(a, __shfl_xor(a, m));
  return a;
}

// Maximum of one list's 64 slots of non-negative float bit patterns (the
// tensor maxima of the transform passes).  Every lane of the wave must call
// it (one load per lane, then a wave maximum); every lane gets the result.
__device__ __forceinline__ float tensor_max_slots(const unsigned* slots64) {
  return wave_max(__uint_as_float(slots64[threadIdx.x & 63]));
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

// ---- g_x GEMM operands: INT4 codes stored as FP6 E2M3
// Every code q in [-7, 7] is exact in FP6 E2M3 (sign, 2 exponent bits with
// bias 1, 3 mantissa bits), so are the products (|q q'| <= 49) and every fp32
// partial sum below 2^24: the g_x product runs on the FP6 matrix cores with
// exact integer results.  A row of codes is stored in groups of 128 K values
// (96 bytes): quarter Q of a group (its values 32 Q .. 32 Q + 31) is a 24-byte
// stream of 6-bit fields (value j at bits 6 j .. 6 j + 5), and the quarters
// sit in the order 0, 2, 1, 3.  Lane half h of the matrix instruction then
// finds its K values of both K steps of a group (quarters h and 2 + h) in
// the 48 contiguous bytes 48 h .. 48 h + 47.
__device__ __forceinline__ constexpr int fp6_quarter_pos(int q) { return ((q & 1) << 1) | (q >> 1); }

// K-plane storage of the integer GEMM operands.  An operand of `rows` rows
// and a K run of kpitch bytes per row is stored as kpitch / U planes of
// rows * U bytes: plane p holds bytes [p U, (p + 1) U) of every row's run,
// row after row.  U = 96 for the FP6 codes (one 128-value group per plane)
// and 64 for the INT8 codes.  A GEMM stage then reads one contiguous block
// per operand (tile rows x U bytes) instead of rows x U bytes scattered at
// the row pitch, which leaves most of each cache line it touches unused.
constexpr int FP6_PLANE = 96;
constexpr int I8_PLANE = 64;
// Byte offset of byte k of row m of an INT8 operand with `rows` rows.
__device__ __forceinline__ int64_t i8_plane_off(int64_t rows, int64_t m, int64_t k) {
  return (k >> 6) * rows * I8_PLANE + m * I8_PLANE + (k & (I8_PLANE - 1));
}

// The code rne(fl(v * inv)) as an integer-valued float (the magic add of
// quant_bits, then an exact subtraction; never -0).
__device__ __forceinline__ float quant_code_f32(float v, float inv) {
  const float p = v * inv;
  return (p + 12582912.0f) - 12582912.0f;
}

typedef float v16f_cvt __attribute__((ext_vector_type(16)));
typedef int v6i_cvt __attribute__((ext_vector_type(6)));

// 32 integer-valued floats in [-7, 7] -> 6 dwords of FP6 E2M3 fields, value j
// at bits 6 j (exact conversion; the instruction interleaves its two 16-value
// operands, the first at the even positions).
__device__ __forceinline__ void fp6_pack32(const float (&v)[32], uint32_t (&d)[6]) {
  v16f_cvt ev, od;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    ev[k] = v[2 * k];
    od[k] = v[2 * k + 1];
  }
  const v6i_cvt r = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(ev, od, 1.0f);
#pragma unroll
  for (int k = 0; k < 6; ++k) d[k] = (uint32_t)r[k];
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
// half-row mirror pairs each lane with one of the other quad); m >= +0.
__device__ __forceinline__ float group8_max(float m) {
  m = nnmax(m, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(m), 0xB1, 0xF, 0xF, true)));
  m = nnmax(m, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(m), 0x4E, 0xF, 0xF, true)));
  m = nnmax(m, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(m), 0x141, 0xF, 0xF, true)));
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

static inline unsigned cdiv(int64_t a, int64_t b) { return (unsigned)((a + b - 1) / b); }

}  // namespace hlq
