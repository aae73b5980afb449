// gfx950 (CDNA4) kernels of the HLQ/HOT linear-layer backward: layer-wise quantizer selection statistics.
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
  const float at = tensor_max_slots(a.tmax);  // every lane of every wave
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
  const float at = tensor_max_slots(a.tmax + op * TMAX_SLOTS);  // the whole wave
  if (valid) {
    zt.inv = a.tok_inv[op][col];
    zt.s = a.tok_s[op][col];
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
