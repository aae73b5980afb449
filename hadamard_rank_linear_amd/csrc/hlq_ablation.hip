// gfx950 kernels of the HLQ/HOT backward's ablation variants: each path's
// GEMM operands under another transform / quantizer ("HOT: Hadamard-based
// Optimized Training", scime.ai summary, "Measured effects" ablation rows and
// "Surprising findings": Hadamard or not before INT4, internal HLA along the
// contracted dimension, external HLA along an output dimension).  Synthetic
// error studies, not the hot path: one plain thread per block of n source
// values, no tiling.  The integer GEMMs are the library's.
//
// An operand is a matrix V[k][m] (k the contracted dimension, m the GEMM
// output index) read from a source matrix S (fp32, bf16, or the ACBP codes
// of x decoded as fl(s_t * q)), V[k][m] = S[m][k] or S[k][m].  Its transform
// runs along X = K or X = M over aligned blocks of n: none, the full block
// Hadamard, or its low-rank rows j*n/r (the full butterfly network in fp32,
// ascending stages, then the kept outputs).  Codes: symmetric absmax with
// round-half-even, one scale per output index m' (PER_TOKEN) or per operand;
// stored one signed byte per code (INT4 values fit), M' rows of Kpad K bytes
// in the INT8 K planes the library's GEMM reads (hlq_device.h), zero past K'.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hlq_device.h"
#include "hlq_internal.h"

namespace hlq {

// fp32 value of source element (row, col).
__device__ __forceinline__ float abl_src(const AblOperand& o, int64_t row, int64_t col) {
  if (o.dt == 0) return static_cast<const float*>(o.src)[row * o.cols + col];
  if (o.dt == 1) return bf16_to_f32(static_cast<const uint16_t*>(o.src)[row * o.cols + col]);
  const int byte = o.codes[row * (o.cols / 2) + (col >> 1)];
  const int code = __builtin_amdgcn_sbfe(byte, (int)(col & 1) * 4, 4);
  return o.cscales[row] * (float)code;  // ACBP decode, one rounding
}

// The nout transformed values of one block: line `line` of the other axis,
// block `blk` along X.  Returns nout (n, or r for low rank).
template <int N>
__device__ __forceinline__ int abl_block(const AblOperand& o, int64_t line, int64_t blk,
                                         float (&v)[N]) {
#pragma unroll
  for (int e = 0; e < N; ++e) {
    const int64_t x = blk * N + e;
    // (k, m) of element e
    const int64_t k = o.along_m ? line : x, m = o.along_m ? x : line;
    v[e] = o.m_is_row ? abl_src(o, m, k) : abl_src(o, k, m);
  }
  if (o.kind == 0) return N;
#pragma unroll
  for (int h = 1; h < N; h <<= 1)
#pragma unroll
    for (int e = 0; e < N; ++e)
      if ((e & h) == 0) {
        const float p = v[e], q = v[e + h];
        v[e] = p + q;
        v[e + h] = p - q;
      }
  if (o.kind == 1) return N;
  const int step = N / o.r;  // low rank: outputs j*step, compacted
  for (int j = 0; j < o.r; ++j) v[j] = v[j * step];
  return o.r;
}

// (m', k') of output j of a block, and the scale group.
__device__ __forceinline__ void abl_out_index(const AblOperand& o, int64_t line, int64_t blk,
                                              int nout, int j, int64_t& mo, int64_t& ko) {
  if (o.along_m) { mo = blk * nout + j; ko = line; }
  else { mo = line; ko = blk * nout + j; }
}

// Zero the maxima and the K padding of every output row.
__global__ __launch_bounds__(256) void k_abl_init(AblOperand o) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t groups = o.per_token ? o.Mo : 1;
  if (i < groups) o.maxbits[i] = 0u;
  const int64_t pad = o.Kpad - o.Ko;
  if (pad > 0 && i < o.Mo * pad) o.q[i8_plane_off(o.Mo, i / pad, o.Ko + i % pad)] = 0;
}

template <int N, int PASS>
__global__ __launch_bounds__(256) void k_abl_operand(AblOperand o) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= o.lines * o.blocks) return;
  const int64_t line = i % o.lines, blk = i / o.lines;  // consecutive threads: consecutive lines
  float v[N];
  const int nout = abl_block<N>(o, line, blk, v);
  const float qmax = (float)o.qmax;
  if constexpr (PASS == PASS_MAX) {
    float m = 0.f;
    for (int j = 0; j < nout; ++j) {
      int64_t mo, ko;
      abl_out_index(o, line, blk, nout, j, mo, ko);
      if (o.per_token && o.along_m) atomicMax(o.maxbits + mo, __float_as_uint(fabsf(v[j])));
      else m = fmaxf(m, fabsf(v[j]));
    }
    if (!(o.per_token && o.along_m)) {
      int64_t mo, ko;
      abl_out_index(o, line, blk, nout, 0, mo, ko);
      atomicMax(o.maxbits + (o.per_token ? mo : 0), __float_as_uint(m));
    }
  } else {
    for (int j = 0; j < nout; ++j) {
      int64_t mo, ko;
      abl_out_index(o, line, blk, nout, j, mo, ko);
      const int64_t g = o.per_token ? mo : 0;
      const float a = __uint_as_float(o.maxbits[g]);
      const float inv = inv_of(a, qmax);
      const float q = fminf(fmaxf(rintf(v[j] * inv), -qmax), qmax);
      o.q[i8_plane_off(o.Mo, mo, ko)] = (int8_t)(int)q;
      if (ko == 0 && (o.per_token || mo == 0)) o.s[g] = scale_of(a, qmax);
    }
  }
}

// g[(b*n + k)][c] = alpha * sum_j H[j*n/r][k] * G[(b*r + j)][c] (fp32, j
// ascending): the expansion of an external-HLA product back to n rows per
// block.
__global__ __launch_bounds__(256) void k_abl_expand(const float* __restrict__ G, int64_t rows,
                                                    int64_t cols, int n, int r, float alpha,
                                                    float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= rows * cols) return;
  const int64_t row = i / cols, c = i % cols;
  const int64_t b = row / n;
  const int k = (int)(row % n), step = n / r;
  float acc = 0.f;
  for (int j = 0; j < r; ++j) {
    const float g = G[(b * r + j) * cols + c];
    acc = (__builtin_popcount((unsigned)(j * step) & (unsigned)k) & 1) ? acc - g : acc + g;
  }
  out[i] = acc * alpha;
}

hipError_t launch_abl_operand(const AblOperand& o, int n, hipStream_t s) {
  const int64_t groups = o.per_token ? o.Mo : 1;
  const int64_t init = groups > o.Mo * (o.Kpad - o.Ko) ? groups : o.Mo * (o.Kpad - o.Ko);
  if (init > 0) hipLaunchKernelGGL(k_abl_init, dim3(cdiv(init, 256)), dim3(256), 0, s, o);
  const dim3 g(cdiv(o.lines * o.blocks, 256));
#define HLQ_ABL(NN)                                                               \
  hipLaunchKernelGGL((k_abl_operand<NN, PASS_MAX>), g, dim3(256), 0, s, o);      \
  hipLaunchKernelGGL((k_abl_operand<NN, PASS_QUANT>), g, dim3(256), 0, s, o)
  switch (n) {
    case 16: HLQ_ABL(16); break;
    case 32: HLQ_ABL(32); break;
    case 64: HLQ_ABL(64); break;
    case 128: HLQ_ABL(128); break;
    default: return hipErrorInvalidValue;
  }
#undef HLQ_ABL
  return hipGetLastError();
}

hipError_t launch_abl_expand(const float* G, int64_t rows, int64_t cols, int n, int r,
                             float alpha, float* out, hipStream_t s) {
  hipLaunchKernelGGL(k_abl_expand, dim3(cdiv(rows * cols, 256)), dim3(256), 0, s, G, rows, cols,
                     n, r, alpha, out);
  return hipGetLastError();
}

}  // namespace hlq
