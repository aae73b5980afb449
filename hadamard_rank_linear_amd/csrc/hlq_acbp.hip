// gfx950 (CDNA4) kernels of the HLQ/HOT linear-layer backward: ACBP pack.
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

#include "hlq_device.h"
#include "hlq_internal.h"

namespace hlq {

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

}  // namespace hlq
