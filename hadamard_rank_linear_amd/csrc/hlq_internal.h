// Internal launch interface between the C ABI layer (hlq_api.cpp) and the
// gfx950 kernels (hlq_kernels.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace hlq {

enum AbsMode { ABS_ONLY = 0, QUANT_OWN = 1, QUANT_GLOBAL = 2 };
enum HlaSource { SRC_F32 = 0, SRC_BF16 = 1, SRC_INT4 = 2 };
enum GemmEpi { EPI_F32 = 0, EPI_I32 = 1, EPI_PARTIAL = 2 };

// Launch configuration of one integer GEMM C[m][n] = sum_k A[m][k] B[n][k],
// both operands K-contiguous ("NT").
struct GemmPlan {
  int bm, bn;      // block tile
  int splits;      // split-K factor (partials summed by gemm_finalize)
  int64_t stages;  // 64-byte K stages in total
};

GemmPlan plan_gemm(int64_t M, int64_t N, int64_t kbytes);

hipError_t launch_fill_u32(uint32_t* p, int64_t n, uint32_t v, hipStream_t s);
hipError_t launch_zero_pad(uint8_t* p, int64_t rows, int64_t pitch, int64_t from,
                           hipStream_t s);

hipError_t launch_acbp(const void* x, int dtype, int64_t T, int64_t I, uint8_t* codes,
                       float* scales, hipStream_t s);

// H along O of each row of g_y [T][O] -> INT4 rows [T][kxb] (+ scales).
hipError_t launch_rows(const void* gy, int dtype, int64_t T, int64_t O, int n,
                       int64_t kxb, uint8_t* q, float* scale, uint32_t* gmax,
                       AbsMode mode, hipStream_t s);

// H along O of each column of w [O][I] -> INT4 stored [I][kxb] (+ scales).
hipError_t launch_cols(const void* w, int dtype, int64_t O, int64_t I, int n,
                       int64_t kxb, uint8_t* q, float* scale, uint32_t* colmax,
                       uint32_t* gmax, AbsMode mode, hipStream_t s);

// Low-rank H along T of [T][C] -> INT8 stored [C][kwb] (+ scales).
hipError_t launch_hla(const void* src, const float* src_scale, HlaSource kind,
                      int64_t T, int64_t C, int n, int r, int64_t kwb, uint8_t* q,
                      float* scale, uint32_t* colmax, uint32_t* gmax, AbsMode mode,
                      hipStream_t s);

hipError_t launch_gemm(bool int4, const uint8_t* A, const uint8_t* B, int64_t M,
                       int64_t N, int64_t pitch, const GemmPlan& plan,
                       const float* sa, int sa_step, const float* sb, int sb_step,
                       float alpha, GemmEpi epi, float* C, int32_t* Ci,
                       int32_t* partial, hipStream_t s);

hipError_t launch_gemm_finalize(const int32_t* partial, int splits, int64_t M,
                                int64_t N, const float* sa, int sa_step,
                                const float* sb, int sb_step, float alpha, float* C,
                                hipStream_t s);

}  // namespace hlq
