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
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

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
// Block tile 128 x BN (BN = 128, or 64 when N is not a multiple of 128, so that N = 192 is not
// covered by a three-quarters-empty tile), 4 waves as 2 x 2, each 64 x (BN / 2) = 4 x NJ tiles
// of v_mfma_f32_16x16x32_bf16; K in steps of 32 (one MFMA k-step) through double-buffered LDS,
// one barrier a step (32 KB a workgroup at BN = 128, so that four share a CU and hide each
// other's barriers).  The MFMA computes the transposed tile (weights as its A operand), so
// that a lane's four results are four consecutive output columns of one row: lane (r16, q4)
// feeds row r16 of the weight tile and row r16 of the activation tile with the 8 consecutive
// k values 8 q4 .. 8 q4 + 7 (the same k order on both sides), and holds
// C[m = 16 i + r16][n = 16 j + 4 q4 + v].
//
// LDS rows are the 64 bytes of one row's 32-deep k-slice, unpadded, as four 16-byte chunks;
// chunk c of row r sits at chunk c ^ swz(r), swz(r) = ((r >> 1) & 3) ^ ((r >> 3) & 1).  A
// read of one chunk by 16 consecutive rows and a write of four rows' four chunks by 16
// consecutive threads then touch 16 distinct 4-bank groups of a 64-bank LDS (and 8 distinct
// groups per 8 lanes of a 32-bank one): no bank conflicts either way.
//
// Ragged edges: rows past M and weight rows past N are read clamped (in bounds) and not
// written; k chunks past K are zero on both operands.  Requires K % 8 == 0 and N % 4 == 0.
constexpr int kBK = 32;

__device__ __forceinline__ int lds_chunk(int row, int c) {
  return row * 4 + (c ^ (((row >> 1) & 3) ^ ((row >> 3) & 1)));
}

template <int EPI, int BN>
__global__ __launch_bounds__(256, BN == 128 ? 4 : 5) void gemm_bf16_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ Wt, int M, int N, int K,
    const float* bias, const float* res, void* out) {
  constexpr int BM = 128, NI = BM / 32, NJ = BN / 32;  // MFMA tiles of a wave: rows, columns
  constexpr int RB = BN / 64;  // 16-byte weight staging loads per thread
  static_assert(BN == 64 || BN == 128, "tile");
  __shared__ __align__(16) u32x4 sA[2][BM * 4];
  __shared__ __align__(16) u32x4 sB[2][BN * 4];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r16 = lane & 15, q4 = lane >> 4, wm = w >> 1, wn = w & 1;
  const int tiles_n = (N + BN - 1) / BN;
  const int tile = xcd_tile(blockIdx.x, gridDim.x);
  const int m0 = (tile / tiles_n) * BM, n0 = (tile % tiles_n) * BN;

  // global -> registers -> LDS: for each operand, rows tid / 4 (and tid / 4 + 64 when the tile
  // has 128 of them) of the tile, 16-byte chunk tid % 4 of the step's 32-deep k-slice (named
  // registers and native vector types: arrays, or selects between 16-byte structs, are placed
  // in scratch memory)
  const int row = tid >> 2, ch = tid & 3;
  const uint16_t* const pa0 = A + (int64_t)min(m0 + row, M - 1) * K + 8 * ch;
  const uint16_t* const pa1 = A + (int64_t)min(m0 + row + 64, M - 1) * K + 8 * ch;
  const uint16_t* const pb0 = Wt + (int64_t)min(n0 + row, N - 1) * K + 8 * ch;
  const uint16_t* const pb1 = Wt + (int64_t)min(n0 + row + 64, N - 1) * K + 8 * ch;
  const int st0 = lds_chunk(row, ch), st1 = lds_chunk(row + 64, ch);
  struct Slice {
    u32x4 a0, a1, b0, b1;
    bool in;  // the chunk lies below K (else it is stored as zeros)
  };
  // A chunk past K loads chunk 0 of its row (in bounds) and is replaced by zeros when it is
  // stored, not when it arrives: a select right after the load would wait for it there.  The
  // loads are unconditional, so no branch or select of addresses enters the step loop; the
  // helpers are forced inline, as a call would keep the captured registers in scratch memory.
  auto fetch = [&](Slice& r, int k0) __attribute__((always_inline)) {
    r.in = k0 + 8 * ch < K;
    const int kk = r.in ? k0 : 0;
    r.a0 = *reinterpret_cast<const u32x4*>(pa0 + kk);
    r.b0 = *reinterpret_cast<const u32x4*>(pb0 + kk);
    r.a1 = *reinterpret_cast<const u32x4*>(pa1 + kk);
    if constexpr (RB > 1) r.b1 = *reinterpret_cast<const u32x4*>(pb1 + kk);
  };
  auto store = [&](const Slice& r, int buf) __attribute__((always_inline)) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    sA[buf][st0] = r.in ? r.a0 : z;
    sB[buf][st0] = r.in ? r.b0 : z;
    sA[buf][st1] = r.in ? r.a1 : z;
    if constexpr (RB > 1) sB[buf][st1] = r.in ? r.b1 : z;
  };

  f32x4 acc[NI][NJ];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  int rd_a[NI], rd_b[NJ];
#pragma unroll
  for (int i = 0; i < NI; ++i) rd_a[i] = lds_chunk(wm * (BM / 2) + 16 * i + r16, q4);
#pragma unroll
  for (int j = 0; j < NJ; ++j) rd_b[j] = lds_chunk(wn * (BN / 2) + 16 * j + r16, q4);
  auto compute = [&](int buf) __attribute__((always_inline)) {
    bf16x8 a[NI], bv[NJ];
#pragma unroll
    for (int i = 0; i < NI; ++i) a[i] = __builtin_bit_cast(bf16x8, sA[buf][rd_a[i]]);
#pragma unroll
    for (int j = 0; j < NJ; ++j) bv[j] = __builtin_bit_cast(bf16x8, sB[buf][rd_b[j]]);
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bv[j], a[i], acc[i][j], 0, 0, 0);
  };

  // Step s multiplies k-slice s from LDS buffer s % 2: slice s + 1 (fetched during step s - 1)
  // is stored into the other buffer at the start of step s, and slice s + 2 fetched into the
  // same registers.  The barrier closing step s - 1 retires every read of the buffer that step
  // s stores to.  (A second register set, fetching two slices ahead, was measured slower: the
  // registers it takes cost more occupancy than the latency it hides.)
  const int steps = (K + kBK - 1) / kBK;
  Slice X;
  fetch(X, 0);
  store(X, 0);
  if (steps > 1) fetch(X, kBK);
  __syncthreads();
  for (int s = 0; s < steps; ++s) {
    const int buf = s & 1;
    if (s + 1 < steps) store(X, buf ^ 1);
    if (s + 2 < steps) fetch(X, (s + 2) * kBK);
    compute(buf);
    __syncthreads();
  }

  // epilogue: acc[i][j][v] = C[m0 + (BM / 2) wm + 16 i + r16][n0 + (BN / 2) wn + 16 j + 4 q4 + v]
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int n = n0 + wn * (BN / 2) + 16 * j + 4 * q4;
    if (n >= N) continue;  // N % 4 == 0: the lane's four columns are all in or all out
    const f32x4 bn = bias ? *reinterpret_cast<const f32x4*>(&bias[n]) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int m = m0 + wm * (BM / 2) + 16 * i + r16;
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
// x_plus = x + addv (fp32; x_plus may equal x).  Lane l holds channels l + 64 k, k < VPL,
// those below C (C <= 64 VPL).
template <int VPL>
__global__ __launch_bounds__(256) void layernorm_kernel(const float* x,
                                                         const float* __restrict__ g,
                                                         const float* __restrict__ b,
                                                         uint16_t* __restrict__ y,
                                                         const float* __restrict__ addv,
                                                         float* x_plus, int64_t M, int C,
                                                         float eps) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) >> 6;
  const float inv_c = 1.f / C;
  for (int64_t p = wave; p < M; p += nwaves) {
    float v[VPL];
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      const int c = lane + 64 * k;
      v[k] = c < C ? x[p * C + c] : 0.f;
      s += v[k];
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
    const float mean = s * inv_c;
    float q = 0.f;
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      const float dv = lane + 64 * k < C ? v[k] - mean : 0.f;
      q = fmaf(dv, dv, q);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) q += __shfl_xor(q, off, 64);
    const float rstd = 1.f / sqrtf(q * inv_c + eps);
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      const int c = lane + 64 * k;
      if (c >= C) break;
      y[p * C + c] = to_bf16((v[k] - mean) * rstd * g[c] + b[c]);
      if (x_plus) x_plus[p * C + c] = v[k] + addv[c];
    }
  }
}

unsigned grid_for(int64_t work, int per_block) {
  const int64_t g = (work + per_block - 1) / per_block;
  return (unsigned)(g < 65535 * 16 ? (g < 1 ? 1 : g) : 65535 * 16);
}

template <int BN>
hipError_t launch_gemm_tile(int epi, const uint16_t* A, const uint16_t* Wt, int M, int N, int K,
                            const float* bias, const float* res, void* out, hipStream_t s) {
  const int64_t tiles = (int64_t)((M + 127) / 128) * ((N + BN - 1) / BN);
  if (tiles > INT32_MAX) return hipErrorInvalidValue;
  const dim3 grid((unsigned)tiles), block(256);
  switch (epi) {
    case kEpiF32: gemm_bf16_kernel<kEpiF32, BN><<<grid, block, 0, s>>>(A, Wt, M, N, K, bias, res, out); break;
    case kEpiGeluBf16: gemm_bf16_kernel<kEpiGeluBf16, BN><<<grid, block, 0, s>>>(A, Wt, M, N, K, bias, res, out); break;
    case kEpiResidualF32: gemm_bf16_kernel<kEpiResidualF32, BN><<<grid, block, 0, s>>>(A, Wt, M, N, K, bias, res, out); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_bf16(int epi, const uint16_t* A, const uint16_t* Wt, int M, int N, int K,
                            const float* bias, const float* res, void* out, hipStream_t s) {
  if (N % 4 || K % 8 || M <= 0 || N <= 0 || K <= 0) return hipErrorInvalidValue;
  if (N % 128) return launch_gemm_tile<64>(epi, A, Wt, M, N, K, bias, res, out, s);
  return launch_gemm_tile<128>(epi, A, Wt, M, N, K, bias, res, out, s);
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
  if (C <= 0 || C > 1024) return hipErrorInvalidValue;
  const unsigned grid = grid_for(M * 64, 256);
  const int vpl = (C + 63) / 64;
#define HOPE_LN(V)                                                                        \
  if (vpl <= V) {                                                                         \
    layernorm_kernel<V><<<grid, 256, 0, s>>>(x, g, b, y, addv, x_plus, M, C, eps);        \
    return hipGetLastError();                                                             \
  }
  HOPE_LN(1) HOPE_LN(2) HOPE_LN(3) HOPE_LN(4) HOPE_LN(6) HOPE_LN(8) HOPE_LN(12) HOPE_LN(16)
#undef HOPE_LN
  return hipErrorInvalidValue;
}

hipError_t launch_cpe(const float* x, const float* w, const float* b, float* x1, int B, int H, int W,
                      int C, hipStream_t s) {
  if (C % 4) return hipErrorInvalidValue;
  const int64_t work = (int64_t)B * H * ((W + 3) / 4) * (C / 4);
  dwconv3x3_kernel<float, float, float, false><<<grid_for(work, 256), 256, 0, s>>>(x, x, w, b, x1, B, H, W, C, nullptr, 0, 0);
  return hipGetLastError();
}

}  // namespace hope
