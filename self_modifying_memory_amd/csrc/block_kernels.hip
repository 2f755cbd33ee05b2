// Kernels of the VisionHOPE block around the scan, gfx950 ("VisionHOPE: Visual Backbones as
// Self-Modifying Learning Systems", Sec. 2.3 Eq. 27 and App. B.5): the pointwise
// projections as bf16 matrix-core GEMMs with fused epilogues (bias, GELU, residual), the
// 3x3 depthwise convolutions with their residual / gate fused, and LayerNorm.
// Feature maps are channels-last [M = B*H*W][C]; linear weights are [out][in] bf16.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "block_kernels.h"

namespace hope {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// two floats to bf16, round to nearest even (one v_cvt_pk_bf16_f32): a in the low half
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
__device__ __forceinline__ uint16_t to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// erf by Abramowitz and Stegun 7.1.26 (|error| <= 1.5e-7): for x >= 0,
// erf(x) = 1 - (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) e^{-x^2}, t = 1 / (1 + p x); odd.
__device__ __forceinline__ float erf_as(float x) {
  const float ax = fabsf(x);
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, ax, 1.f));
  float y = fmaf(1.061405429f, t, -1.453152027f);
  y = fmaf(y, t, 1.421413741f);
  y = fmaf(y, t, -0.284496736f);
  y = fmaf(y, t, 0.254829592f);
  y = 1.f - y * t * __builtin_amdgcn_exp2f(-ax * ax * 1.4426950408889634f);
  return copysignf(y, x);
}

// Workgroups are dealt to the 8 XCDs (each with its own L2) round robin by their index.  The
// logical tile index below gives each XCD one contiguous range of the G tiles instead, so
// that the tiles sharing an operand panel (GEMM) or a halo row (convolution) meet in one L2:
// with G = 8 q + r, XCD x < r takes q + 1 tiles, the others q.
__device__ __forceinline__ int xcd_tile(int bid, int G) {
  const int x = bid & 7, j = bid >> 3, q = G >> 3, r = G & 7;
  return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + j;
}

// ---- GEMM: out[m][n] = epilogue(sum_k A[m][k] Wt[n][k]) -----------------------------------
// Block tile 128 x 128, 4 waves as 2 x 2, each 64 x 64 = 4 x 4 tiles of v_mfma_f32_16x16x32_bf16;
// K in steps of 32 (one MFMA k-step) through double-buffered LDS (rows padded to 40 bf16:
// 40 KB a workgroup, so that four share a CU and hide each other's barriers), one barrier a
// step.  The MFMA computes the transposed tile (weights as its A operand), so that a lane's
// four results are four consecutive output columns of one row: lane (r16, q4) feeds row r16
// of the weight tile and row r16 of the activation tile with the 8 consecutive k values
// 8 q4 .. 8 q4 + 7 (the same k order on both sides), and holds
// C[m = 16 i + r16][n = 16 j + 4 q4 + v].
// Requires N % 128 == 0 and K % 64 == 0; rows past M are read clamped and not written.
constexpr int kBM = 128, kBN = 128, kBK = 32, kLDK = kBK + 8;

template <int EPI>
__global__ __launch_bounds__(256, 4) void gemm_bf16_kernel(const uint16_t* __restrict__ A,
                                                            const uint16_t* __restrict__ Wt, int M,
                                                            int N, int K, const float* bias,
                                                            const float* res, void* out) {
  __shared__ __align__(16) uint16_t sA[2][kBM * kLDK];
  __shared__ __align__(16) uint16_t sB[2][kBN * kLDK];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r16 = lane & 15, q4 = lane >> 4, wm = w >> 1, wn = w & 1;
  const int tiles_n = N / kBN;
  const int tile = xcd_tile(blockIdx.x, gridDim.x);
  const int m0 = (tile / tiles_n) * kBM, n0 = (tile % tiles_n) * kBN;

  // global -> registers -> LDS: 2 chunks of 8 bf16 per thread for each operand
  // (rows tid / 4 and tid / 4 + 64, k chunk 8 (tid % 4))
  const int row = tid >> 2, ch = 8 * (tid & 3);
  const uint16_t* pa = A + (int64_t)min(m0 + row, M - 1) * K + ch;
  const int64_t da1 = (int64_t)(min(m0 + row + 64, M - 1) - min(m0 + row, M - 1)) * K;
  const uint16_t* pb = Wt + (int64_t)(n0 + row) * K + ch;
  const int64_t db = (int64_t)64 * K;
  uint4 ga00, ga01, gb00, gb01;
#define HOPE_GEMM_FETCH(S, k)                                 \
  ga##S##0 = *reinterpret_cast<const uint4*>(pa + (k));       \
  ga##S##1 = *reinterpret_cast<const uint4*>(pa + da1 + (k)); \
  gb##S##0 = *reinterpret_cast<const uint4*>(pb + (k));       \
  gb##S##1 = *reinterpret_cast<const uint4*>(pb + db + (k));
#define HOPE_GEMM_STORE(S, buf)                                            \
  *reinterpret_cast<uint4*>(&sA[buf][(row + 0) * kLDK + ch]) = ga##S##0;   \
  *reinterpret_cast<uint4*>(&sA[buf][(row + 64) * kLDK + ch]) = ga##S##1;  \
  *reinterpret_cast<uint4*>(&sB[buf][(row + 0) * kLDK + ch]) = gb##S##0;   \
  *reinterpret_cast<uint4*>(&sB[buf][(row + 64) * kLDK + ch]) = gb##S##1;
#define HOPE_GEMM_COMPUTE(buf)                                                                   \
  {                                                                                              \
    bf16x8 a[4], bv[4];                                                                          \
    _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                              \
      a[i] = *reinterpret_cast<const bf16x8*>(&sA[buf][(wm * 64 + 16 * i + r16) * kLDK + 8 * q4]); \
      bv[i] = *reinterpret_cast<const bf16x8*>(&sB[buf][(wn * 64 + 16 * i + r16) * kLDK + 8 * q4]); \
    }                                                                                            \
    _Pragma("unroll") for (int i = 0; i < 4; ++i)                                                \
      _Pragma("unroll") for (int j = 0; j < 4; ++j)                                              \
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bv[j], a[i], acc[i][j], 0, 0, 0);    \
  }

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // tile t (32 deep) is loaded into registers during step t - 2, stored into LDS buffer
  // t % 2 during step t - 1 and multiplied at step t; the barrier closing step t - 1 retires
  // every read of the buffer that step t - 1 stores to (the four workgroups on a CU hide
  // the latency that the single register set leaves)
  HOPE_GEMM_FETCH(0, 0)
  HOPE_GEMM_STORE(0, 0)
  HOPE_GEMM_FETCH(0, kBK)
  __syncthreads();
  for (int k0 = 0; k0 < K; k0 += 2 * kBK) {
    HOPE_GEMM_STORE(0, 1)
    if (k0 + 2 * kBK < K) {
      HOPE_GEMM_FETCH(0, k0 + 2 * kBK)
    }
    HOPE_GEMM_COMPUTE(0)
    __syncthreads();
    if (k0 + 2 * kBK < K) {
      HOPE_GEMM_STORE(0, 0)
      if (k0 + 3 * kBK < K) {
        HOPE_GEMM_FETCH(0, k0 + 3 * kBK)
      }
    }
    HOPE_GEMM_COMPUTE(1)
    __syncthreads();
  }

#undef HOPE_GEMM_FETCH
#undef HOPE_GEMM_STORE
#undef HOPE_GEMM_COMPUTE
  // epilogue: acc[i][j][v] = C[m0 + 64 wm + 16 i + r16][n0 + 64 wn + 16 j + 4 q4 + v]
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = n0 + wn * 64 + 16 * j + 4 * q4;
    const f32x4 bn = bias ? *reinterpret_cast<const f32x4*>(&bias[n]) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + wm * 64 + 16 * i + r16;
      if (m >= M) continue;
      const int64_t o = (int64_t)m * N + n;
      const f32x4 t = acc[i][j] + bn;
      if (EPI == kEpiF32) {
        *reinterpret_cast<f32x4*>(&static_cast<float*>(out)[o]) = t;
      } else if (EPI == kEpiGeluBf16) {
        f32x4 gv;
#pragma unroll
        for (int v = 0; v < 4; ++v) {  // GELU(t) = t / 2 + (t / 2) erf(t / sqrt 2)
          const float hv = 0.5f * t[v];
          gv[v] = fmaf(hv, erf_as(t[v] * 0.70710678118654752f), hv);
        }
        uint2 u;
        u.x = pack_bf16(gv[0], gv[1]);
        u.y = pack_bf16(gv[2], gv[3]);
        *reinterpret_cast<uint2*>(&static_cast<uint16_t*>(out)[o]) = u;
      } else {
        const f32x4 rv = *reinterpret_cast<const f32x4*>(&res[o]);
        *reinterpret_cast<f32x4*>(&static_cast<float*>(out)[o]) = rv + t;
      }
    }
  }
}

// ---- depthwise 3x3 convolution with a fused residual --------------------------------------
// out[p][c] = res'[p][c] + act(bias[c] + sum over the 3x3 neighbourhood (zero padding) of
// w[dy][dx][c] src[p + (dy - 1, dx - 1)][c]), res' = res + planes[0] + ... + planes[n - 1]
// (added left to right); four channels per thread.
template <typename T>
__device__ __forceinline__ f32x4 load4(const T* p);
template <>
__device__ __forceinline__ f32x4 load4<float>(const float* p) {
  return *reinterpret_cast<const f32x4*>(p);
}
template <>
__device__ __forceinline__ f32x4 load4<uint16_t>(const uint16_t* p) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  return f32x4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u),
               __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xFFFF0000u)};
}
template <typename T>
__device__ __forceinline__ void store4(T* p, f32x4 v);
template <>
__device__ __forceinline__ void store4<float>(float* p, f32x4 v) {
  *reinterpret_cast<f32x4*>(p) = v;
}
template <>
__device__ __forceinline__ void store4<uint16_t>(uint16_t* p, f32x4 v) {
  uint2 u;
  u.x = pack_bf16(v[0], v[1]);
  u.y = pack_bf16(v[2], v[3]);
  *reinterpret_cast<uint2*>(p) = u;
}

template <typename SrcT, typename ResT, typename OutT, bool SILU>
__global__ __launch_bounds__(256) void dwconv3x3_kernel(const SrcT* __restrict__ src,
                                                         const ResT* __restrict__ res,
                                                         const float* __restrict__ wgt,
                                                         const float* __restrict__ bias, OutT* out,
                                                         int B, int H, int W, int C,
                                                         const float* __restrict__ planes,
                                                         int64_t plane_stride, int n_planes) {
  // one thread: four channels of four consecutive pixels of a row (x0 .. x0 + 3), so that
  // the 3 x 6 input neighbourhood and the nine weights are read once for four outputs
  // (32-bit index arithmetic: the host bounds B * H * ceil(W / 4) * C / 4 below 2^31)
  const int cq = C / 4, xq = (W + 3) / 4;
  const int total = B * H * xq * cq;
  for (int i = xcd_tile(blockIdx.x, gridDim.x) * blockDim.x + threadIdx.x; i < total;
       i += gridDim.x * blockDim.x) {
    const int c = (i % cq) * 4;
    const int rest = i / cq;
    const int x0 = (rest % xq) * 4;
    const int y = (rest / xq) % H;
    const int64_t img = rest / (xq * H);
    const f32x4 b4 = *reinterpret_cast<const f32x4*>(&bias[c]);
    f32x4 acc[4] = {b4, b4, b4, b4};
#pragma unroll
    for (int dy = 0; dy < 3; ++dy) {
      const int yy = y + dy - 1;
      if (yy < 0 || yy >= H) continue;
      const f32x4 w0 = *reinterpret_cast<const f32x4*>(&wgt[(dy * 3 + 0) * C + c]);
      const f32x4 w1 = *reinterpret_cast<const f32x4*>(&wgt[(dy * 3 + 1) * C + c]);
      const f32x4 w2 = *reinterpret_cast<const f32x4*>(&wgt[(dy * 3 + 2) * C + c]);
      const SrcT* row = src + ((img * H + yy) * W) * (int64_t)C + c;
      f32x4 v[6];
#pragma unroll
      for (int k = 0; k < 6; ++k) {
        const int xx = x0 - 1 + k;
        v[k] = (xx >= 0 && xx < W) ? load4(row + (int64_t)xx * C) : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int o = 0; o < 4; ++o)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          acc[o][e] = fmaf(w2[e], v[o + 2][e], fmaf(w1[e], v[o + 1][e], fmaf(w0[e], v[o][e], acc[o][e])));
    }
#pragma unroll
    for (int o = 0; o < 4; ++o) {
      if (x0 + o >= W) break;
      f32x4 a = acc[o];
      if (SILU) {
#pragma unroll
        for (int e = 0; e < 4; ++e)  // SiLU; hardware exp2 and reciprocal (about 1 ulp each, the
                                     // result is rounded to bf16)
          a[e] = a[e] * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-a[e] * 1.4426950408889634f));
      }
      const int64_t p = (img * H + y) * W + x0 + o;
      f32x4 r = load4(&res[p * C + c]);
      if (n_planes == 3) {  // the four-route operator: the three loads issued together
        const float* pp = &planes[p * C + c];
        const f32x4 p0 = load4(pp), p1 = load4(pp + plane_stride), p2 = load4(pp + 2 * plane_stride);
        r = ((r + p0) + p1) + p2;
      } else {
        for (int k = 0; k < n_planes; ++k) r += load4(&planes[k * plane_stride + p * C + c]);
      }
      store4(&out[p * C + c], r + a);
    }
  }
}

// ---- CPE and LayerNorm 1 fused -----------------------------------------------------------
// x1 = x + bias + DW(x) (the conditional positional encoding), then a = bf16(LN(x1) g + lb)
// (biased variance) and r = x1 + addv, without x1 leaving the chip.  A workgroup of D / 2
// threads covers two groups of four consecutive pixels of a row; thread (slot, c) holds
// channels 4c .. 4c + 3 of its group's four pixels (the stencil of dwconv3x3_kernel).  The
// per-pixel sums go through 32-lane halves (D / 4 is a multiple of 32) and LDS; the
// variance is taken about the mean from the values in registers.
__global__ __launch_bounds__(512) void cpe_layernorm_kernel(
    const float* __restrict__ x, const float* __restrict__ wgt, const float* __restrict__ bias,
    const float* __restrict__ g, const float* __restrict__ lb, const float* __restrict__ addv,
    uint16_t* __restrict__ a, float* __restrict__ r, int B, int H, int W, int C, float eps) {
  __shared__ float red[2][16][4];  // [pass][half-wave][pixel]: up to 512 threads
  const int cq = C / 4, xq = (W + 3) / 4;
  const int slot = threadIdx.x / cq, c = (threadIdx.x % cq) * 4;
  const int half = threadIdx.x >> 5, halves = cq / 32;  // a slot's halves: slot * halves + i
  const int grp = xcd_tile(blockIdx.x, gridDim.x) * 2 + slot;
  const int total = B * H * xq;
  const bool on = grp < total;
  const int gq = on ? grp : total - 1;  // a missing second group computes in bounds, stores nothing
  const int x0 = (gq % xq) * 4;
  const int y = (gq / xq) % H;
  const int64_t img = gq / (xq * H);
  const f32x4 b4 = *reinterpret_cast<const f32x4*>(&bias[c]);
  f32x4 acc[4] = {b4, b4, b4, b4};
#pragma unroll
  for (int dy = 0; dy < 3; ++dy) {
    const int yy = y + dy - 1;
    if (yy < 0 || yy >= H) continue;
    const f32x4 w0 = *reinterpret_cast<const f32x4*>(&wgt[(dy * 3 + 0) * C + c]);
    const f32x4 w1 = *reinterpret_cast<const f32x4*>(&wgt[(dy * 3 + 1) * C + c]);
    const f32x4 w2 = *reinterpret_cast<const f32x4*>(&wgt[(dy * 3 + 2) * C + c]);
    const float* row = x + ((img * H + yy) * W) * (int64_t)C + c;
    f32x4 v[6];
#pragma unroll
    for (int k = 0; k < 6; ++k) {
      const int xx = x0 - 1 + k;
      v[k] = (xx >= 0 && xx < W) ? *reinterpret_cast<const f32x4*>(row + (int64_t)xx * C) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int o = 0; o < 4; ++o)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        acc[o][e] = fmaf(w2[e], v[o + 2][e], fmaf(w1[e], v[o + 1][e], fmaf(w0[e], v[o][e], acc[o][e])));
  }
  // residual (pixels past the row end read the last pixel: in bounds, never stored)
#pragma unroll
  for (int o = 0; o < 4; ++o) {
    const int64_t p = (img * H + y) * W + min(x0 + o, W - 1);
    acc[o] += *reinterpret_cast<const f32x4*>(&x[p * C + c]);
  }
  // per-pixel sums over the slot's channels: 32-lane halves, then LDS
  float mean[4], rstd[4];
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    float s[4];
#pragma unroll
    for (int o = 0; o < 4; ++o) {
      float t = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float dv = pass == 0 ? acc[o][e] : acc[o][e] - mean[o];
        t = pass == 0 ? t + dv : fmaf(dv, dv, t);
      }
#pragma unroll
      for (int off = 16; off >= 1; off >>= 1) t += __shfl_xor(t, off, 64);
      s[o] = t;
    }
    if ((threadIdx.x & 31) == 0) {
#pragma unroll
      for (int o = 0; o < 4; ++o) red[pass][half][o] = s[o];
    }
    __syncthreads();
#pragma unroll
    for (int o = 0; o < 4; ++o) {
      float t = 0.f;
      for (int i = 0; i < halves; ++i) t += red[pass][slot * halves + i][o];
      if (pass == 0) mean[o] = t / C;
      else rstd[o] = 1.f / sqrtf(t / C + eps);
    }
  }
  if (!on) return;
  const f32x4 g4 = *reinterpret_cast<const f32x4*>(&g[c]);
  const f32x4 lb4 = *reinterpret_cast<const f32x4*>(&lb[c]);
  const f32x4 ad4 = *reinterpret_cast<const f32x4*>(&addv[c]);
#pragma unroll
  for (int o = 0; o < 4; ++o) {
    if (x0 + o >= W) break;
    const int64_t p = (img * H + y) * W + x0 + o;
    f32x4 nv;
#pragma unroll
    for (int e = 0; e < 4; ++e) nv[e] = (acc[o][e] - mean[o]) * rstd[o] * g4[e] + lb4[e];
    uint2 u;
    u.x = pack_bf16(nv[0], nv[1]);
    u.y = pack_bf16(nv[2], nv[3]);
    *reinterpret_cast<uint2*>(&a[p * C + c]) = u;
    *reinterpret_cast<f32x4*>(&r[p * C + c]) = acc[o] + ad4;
  }
}

// ---- LayerNorm over the channels of each pixel (one wave per pixel) ------------------------
// y = bf16((x - mean) / sqrt(var + eps) * g + b) with the biased variance; optionally
// x_plus = x + addv (fp32).  VPL = C / 64 values per lane.
template <int VPL>
__global__ __launch_bounds__(256) void layernorm_kernel(const float* __restrict__ x,
                                                         const float* __restrict__ g,
                                                         const float* __restrict__ b,
                                                         uint16_t* __restrict__ y,
                                                         const float* __restrict__ addv,
                                                         float* __restrict__ x_plus, int64_t M,
                                                         float eps) {
  constexpr int C = 64 * VPL;
  const int lane = threadIdx.x & 63;
  const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) >> 6;
  for (int64_t p = wave; p < M; p += nwaves) {
    float v[VPL];
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      v[k] = x[p * C + lane + 64 * k];
      s += v[k];
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
    const float mean = s * (1.f / C);
    float q = 0.f;
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      const float dv = v[k] - mean;
      q = fmaf(dv, dv, q);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) q += __shfl_xor(q, off, 64);
    const float rstd = 1.f / sqrtf(q * (1.f / C) + eps);
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      const int c = lane + 64 * k;
      y[p * C + c] = to_bf16((v[k] - mean) * rstd * g[c] + b[c]);
      if (x_plus) x_plus[p * C + c] = v[k] + addv[c];
    }
  }
}

unsigned grid_for(int64_t work, int per_block) {
  const int64_t g = (work + per_block - 1) / per_block;
  return (unsigned)(g < 65535 * 16 ? (g < 1 ? 1 : g) : 65535 * 16);
}

}  // namespace

hipError_t launch_gemm_bf16(int epi, const uint16_t* A, const uint16_t* Wt, int M, int N, int K,
                            const float* bias, const float* res, void* out, hipStream_t s) {
  if (N % kBN || K % (2 * kBK) || M <= 0 || K <= 0) return hipErrorInvalidValue;
  const int64_t tiles = (int64_t)((M + kBM - 1) / kBM) * (N / kBN);
  if (tiles > INT32_MAX) return hipErrorInvalidValue;
  const dim3 grid((unsigned)tiles), block(256);
  switch (epi) {
    case kEpiF32: gemm_bf16_kernel<kEpiF32><<<grid, block, 0, s>>>(A, Wt, M, N, K, bias, res, out); break;
    case kEpiGeluBf16: gemm_bf16_kernel<kEpiGeluBf16><<<grid, block, 0, s>>>(A, Wt, M, N, K, bias, res, out); break;
    case kEpiResidualF32: gemm_bf16_kernel<kEpiResidualF32><<<grid, block, 0, s>>>(A, Wt, M, N, K, bias, res, out); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_cpe_layernorm(const float* x, const float* w, const float* b, const float* g,
                                const float* lb, const float* addv, uint16_t* a, float* r, int B,
                                int H, int W, int C, float eps, hipStream_t s) {
  if (C % 128 || C > 1024) return hipErrorInvalidValue;
  const int64_t groups = (int64_t)B * H * ((W + 3) / 4);
  const int64_t blocks = (groups + 1) / 2;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  cpe_layernorm_kernel<<<(unsigned)blocks, C / 2, 0, s>>>(x, w, b, g, lb, addv, a, r, B, H, W, C, eps);
  return hipGetLastError();
}

hipError_t launch_dwconv_gated(const float* u, const float* w, const float* b, uint16_t* z, int B,
                               int H, int W, int C, hipStream_t s) {
  const int64_t work = (int64_t)B * H * ((W + 3) / 4) * (C / 4);
  dwconv3x3_kernel<float, float, uint16_t, true><<<grid_for(work, 256), 256, 0, s>>>(u, u, w, b, z, B, H, W, C, nullptr, 0, 0);
  return hipGetLastError();
}

hipError_t launch_dwconv_lpe(const uint16_t* z, const float* y, const float* planes,
                             int64_t plane_stride, int n_planes, const float* w, const float* b,
                             uint16_t* out, int B, int H, int W, int C, hipStream_t s) {
  const int64_t work = (int64_t)B * H * ((W + 3) / 4) * (C / 4);
  dwconv3x3_kernel<uint16_t, float, uint16_t, false><<<grid_for(work, 256), 256, 0, s>>>(z, y, w, b, out, B, H, W, C, planes, plane_stride, n_planes);
  return hipGetLastError();
}

hipError_t launch_layernorm(const float* x, const float* g, const float* b, uint16_t* y,
                            const float* addv, float* x_plus, int64_t M, int C, float eps,
                            hipStream_t s) {
  const unsigned grid = grid_for(M * 64, 256);
  switch (C / 64) {
#define HOPE_LN(V) \
  case V: layernorm_kernel<V><<<grid, 256, 0, s>>>(x, g, b, y, addv, x_plus, M, eps); break;
    HOPE_LN(1) HOPE_LN(2) HOPE_LN(3) HOPE_LN(4) HOPE_LN(6) HOPE_LN(8) HOPE_LN(12) HOPE_LN(16)
#undef HOPE_LN
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace hope
