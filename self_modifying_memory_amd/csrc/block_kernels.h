// Internal launch interface of the block kernels (block_kernels.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hope {

enum { kEpiF32 = 0, kEpiGeluBf16 = 1, kEpiResidualF32 = 2 };

// out[m][n] = epi(sum_k A[m][k] Wt[n][k] + bias[n]): kEpiF32 -> fp32 out; kEpiGeluBf16 ->
// bf16 GELU(.) (erf form, erf by Abramowitz-Stegun 7.1.26); kEpiResidualF32 -> fp32 res[m][n] + (.) (res may equal out).
// bias may be null.  N % 4 == 0, K % 8 == 0 (ragged tiles); A, Wt, bias, res, out 16-byte
// aligned.
hipError_t launch_gemm_bf16(int epi, const uint16_t* A, const uint16_t* Wt, int M, int N, int K,
                            const float* bias, const float* res, void* out, hipStream_t s);

// x1 = x + DW(x) (the conditional positional encoding), a = bf16(LayerNorm(x1) g + lb),
// r = x1 + addv, x1 itself not stored.  C % 128 == 0, C <= 1024.
hipError_t launch_cpe_layernorm(const float* x, const float* w, const float* b, const float* g,
                                const float* lb, const float* addv, uint16_t* a, float* r, int B,
                                int H, int W, int C, float eps, hipStream_t s);
// z = bf16(u + SiLU(DW(u))) (the gated depthwise branch)
hipError_t launch_dwconv_gated(const float* u, const float* w, const float* b, uint16_t* z, int B,
                               int H, int W, int C, hipStream_t s);
// out = bf16(y' + DW(z)) (the local positional branch added to the operator output), where
// y' = y + planes[0] + ... + planes[n_planes - 1] (left to right, planes plane_stride floats
// apart: the operator's unsummed route planes; n_planes may be 0)
hipError_t launch_dwconv_lpe(const uint16_t* z, const float* y, const float* planes,
                             int64_t plane_stride, int n_planes, const float* w, const float* b,
                             uint16_t* out, int B, int H, int W, int C, hipStream_t s);
// x1 = x + bias + DW(x) (the conditional positional encoding alone, fp32), any C % 4 == 0.
hipError_t launch_cpe(const float* x, const float* w, const float* b, float* x1, int B, int H, int W,
                      int C, hipStream_t s);
// y = bf16(LayerNorm(x) g + b); if x_plus: x_plus = x + addv (x_plus may equal x).  C <= 1024.
hipError_t launch_layernorm(const float* x, const float* g, const float* b, uint16_t* y,
                            const float* addv, float* x_plus, int64_t M, int C, float eps,
                            hipStream_t s);

}  // namespace hope
