// Route permutations and the fixed-order route sum, gfx950.
//
// Orders: "VMamba: Visual State Space Model" (explainer), the four scan orders:
// row-major, the flatten of the spatial transpose, and the full reversal of each;
// "VisionHOPE: Visual Backbones as Self-Modifying Learning Systems" Sec. 2.3 Eq. 24.
// Merge: restore each route to its pixel, then add (VisionHOPE Eq. 26, unit scales).
// All kernels are HBM-bound streaming kernels: consecutive threads touch
// consecutive channels of one pixel, so every wave reads/writes contiguous runs.
#include "kernels.h"

namespace hope {
namespace {

struct Routes4 {
  int r[4];
};

__device__ __forceinline__ int64_t route_pixel64(int r, int64_t t, int H, int W, int64_t N) {
  if (r & 1) t = N - 1 - t;
  if (r < 2) return t;
  return (t % H) * W + (t / H);
}

// inverse: sequence index of pixel p on route r
__device__ __forceinline__ int64_t route_step64(int r, int64_t p, int H, int W, int64_t N) {
  int64_t t = p;
  if (r >= 2) {
    const int64_t hh = p / W, ww = p % W;
    t = ww * H + hh;
  }
  if (r & 1) t = N - 1 - t;
  return t;
}

template <typename T>
__global__ void cross_scan_kernel(const T* __restrict__ x, int B, int H, int W, int D, Routes4 rs,
                                  int n_sel, T* __restrict__ routes) {
  const int64_t N = (int64_t)H * W;
  const int64_t per_route = (int64_t)B * N * D;
  const int64_t total = per_route * n_sel;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int slot = (int)(e / per_route);
    int64_t rem = e - slot * per_route;
    const int c = (int)(rem % D);
    rem /= D;
    const int64_t t = rem % N;
    const int64_t b = rem / N;
    const int64_t p = route_pixel64(rs.r[slot], t, H, W, N);
    routes[e] = x[(b * N + p) * D + c];
  }
}

// Vector forms: 16 bytes per thread (8 bf16 or 4 fp32 channels of one pixel), 32-bit index
// arithmetic (the host checks the sizes); D a multiple of the vector width.
template <typename T>
__global__ void cross_scan_vec_kernel(const T* __restrict__ x, int B, int H, int W, int D,
                                      Routes4 rs, int n_sel, T* __restrict__ routes) {
  constexpr int V = 16 / sizeof(T);
  const unsigned N = (unsigned)H * W, DV = (unsigned)D / V;
  const unsigned total = (unsigned)n_sel * B * N * DV;
  for (unsigned i = blockIdx.x * blockDim.x + threadIdx.x; i < total; i += gridDim.x * blockDim.x) {
    const unsigned cv = i % DV;
    unsigned rem = i / DV;
    const unsigned t = rem % N;
    rem /= N;
    const unsigned b = rem % B, slot = rem / B;
    const int r = rs.r[slot];
    unsigned tt = (r & 1) ? N - 1 - t : t;
    const unsigned p = r < 2 ? tt : (tt % H) * W + tt / H;
    const uint4 v = *reinterpret_cast<const uint4*>(x + ((int64_t)b * N + p) * D + (int64_t)cv * V);
    *reinterpret_cast<uint4*>(routes + (int64_t)i * V) = v;
  }
}

template <bool BF16>
__global__ void cross_merge_vec_kernel(const void* __restrict__ routes, int B, int H, int W, int D,
                                       Routes4 rs, int n_sel, float* __restrict__ out) {
  const unsigned N = (unsigned)H * W, DQ = (unsigned)D / 4;
  const unsigned total = (unsigned)B * N * DQ;
  const int64_t per_route = (int64_t)B * N * D;
  for (unsigned i = blockIdx.x * blockDim.x + threadIdx.x; i < total; i += gridDim.x * blockDim.x) {
    const unsigned cq = i % DQ;
    const unsigned rem = i / DQ;
    const unsigned p = rem % N, b = rem / N;
    float4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < n_sel; ++s) {
      const int r = rs.r[s];
      unsigned t = r < 2 ? p : (p % W) * H + p / W;
      if (r & 1) t = N - 1 - t;
      const int64_t idx = s * per_route + ((int64_t)b * N + t) * D + (int64_t)cq * 4;
      float4 v;
      if (BF16) {
        const uint2 u = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(routes) + idx);
        v = float4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u),
                   __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xFFFF0000u)};
      } else {
        v = *reinterpret_cast<const float4*>(static_cast<const float*>(routes) + idx);
      }
      if (s == 0) {
        acc = v;
      } else {
        acc.x += v.x;
        acc.y += v.y;
        acc.z += v.z;
        acc.w += v.w;
      }
    }
    *reinterpret_cast<float4*>(out + (int64_t)i * 4) = acc;
  }
}

template <bool BF16>
__global__ void cross_merge_kernel(const void* __restrict__ routes, int B, int H, int W, int D,
                                   Routes4 rs, int n_sel, float* __restrict__ out) {
  const int64_t N = (int64_t)H * W;
  const int64_t per_route = (int64_t)B * N * D;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < per_route;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int c = (int)(e % D);
    const int64_t rem = e / D;
    const int64_t p = rem % N;
    const int64_t b = rem / N;
    float acc = 0.f;
    for (int s = 0; s < n_sel; ++s) {
      const int64_t t = route_step64(rs.r[s], p, H, W, N);
      const int64_t idx = s * per_route + (b * N + t) * D + c;
      float v;
      if (BF16) {
        v = __uint_as_float((uint32_t)static_cast<const uint16_t*>(routes)[idx] << 16);
      } else {
        v = static_cast<const float*>(routes)[idx];
      }
      acc = s == 0 ? v : acc + v;
    }
    out[e] = acc;
  }
}

// Restore-and-sum of the routes (VisionHOPE Eq. 26 with unit scales): slot 0 is already
// in out, slots 1.. are workspace planes of the same layout; added in slot order so the
// result is bit-for-bit reproducible.
__global__ void plane_sum_vec4(float4* __restrict__ out, const float4* __restrict__ planes,
                               int64_t stride4, int n_planes, int64_t n4) {
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n4;
       e += (int64_t)gridDim.x * blockDim.x) {
    float4 a = out[e];
    for (int k = 0; k < n_planes; ++k) {
      const float4 v = planes[k * stride4 + e];
      a.x += v.x;
      a.y += v.y;
      a.z += v.z;
      a.w += v.w;
    }
    out[e] = a;
  }
}

__global__ void plane_sum_scalar(float* __restrict__ out, const float* __restrict__ planes,
                                 int64_t stride, int n_planes, int64_t n) {
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n;
       e += (int64_t)gridDim.x * blockDim.x) {
    float a = out[e];
    for (int k = 0; k < n_planes; ++k) a += planes[k * stride + e];
    out[e] = a;
  }
}

// bf16 out: the fp32 sum of the route planes in slot order, rounded once
__global__ void plane_sum_bf16_vec4(uint2* __restrict__ out, const float4* __restrict__ planes,
                                    int64_t stride4, int n_planes, int64_t n4) {
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n4;
       e += (int64_t)gridDim.x * blockDim.x) {
    float4 a = planes[e];
    for (int k = 1; k < n_planes; ++k) {
      const float4 v = planes[k * stride4 + e];
      a.x += v.x;
      a.y += v.y;
      a.z += v.z;
      a.w += v.w;
    }
    const __bf16 b0 = (__bf16)a.x, b1 = (__bf16)a.y, b2 = (__bf16)a.z, b3 = (__bf16)a.w;
    uint2 o;
    o.x = (unsigned)__builtin_bit_cast(unsigned short, b0) | ((unsigned)__builtin_bit_cast(unsigned short, b1) << 16);
    o.y = (unsigned)__builtin_bit_cast(unsigned short, b2) | ((unsigned)__builtin_bit_cast(unsigned short, b3) << 16);
    out[e] = o;
  }
}

__global__ void plane_sum_bf16_scalar(unsigned short* __restrict__ out, const float* __restrict__ planes,
                                      int64_t stride, int n_planes, int64_t n) {
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n;
       e += (int64_t)gridDim.x * blockDim.x) {
    float a = planes[e];
    for (int k = 1; k < n_planes; ++k) a += planes[k * stride + e];
    out[e] = __builtin_bit_cast(unsigned short, (__bf16)a);
  }
}

unsigned grid_for(int64_t n, int block) {
  int64_t g = (n + block - 1) / block;
  const int64_t cap = 256 * 64;  // enough waves to saturate HBM; grid-stride beyond
  if (g > cap) g = cap;
  if (g < 1) g = 1;
  return (unsigned)g;
}

}  // namespace

hipError_t launch_plane_sum(float* out, const float* planes, int64_t plane_stride, int n_planes,
                            int64_t n_elem, hipStream_t stream) {
  if (n_planes <= 0 || n_elem <= 0) return hipSuccess;
  if (n_elem % 4 == 0 && plane_stride % 4 == 0) {
    const int64_t n4 = n_elem / 4;
    hipLaunchKernelGGL(plane_sum_vec4, dim3(grid_for(n4, 256)), dim3(256), 0, stream,
                       reinterpret_cast<float4*>(out), reinterpret_cast<const float4*>(planes),
                       plane_stride / 4, n_planes, n4);
  } else {
    hipLaunchKernelGGL(plane_sum_scalar, dim3(grid_for(n_elem, 256)), dim3(256), 0, stream, out,
                       planes, plane_stride, n_planes, n_elem);
  }
  return hipGetLastError();
}

hipError_t launch_plane_sum_bf16(unsigned short* out, const float* planes, int64_t plane_stride,
                                 int n_planes, int64_t n_elem, hipStream_t stream) {
  if (n_planes <= 0 || n_elem <= 0) return hipSuccess;
  if (n_elem % 4 == 0 && plane_stride % 4 == 0) {
    const int64_t n4 = n_elem / 4;
    hipLaunchKernelGGL(plane_sum_bf16_vec4, dim3(grid_for(n4, 256)), dim3(256), 0, stream,
                       reinterpret_cast<uint2*>(out), reinterpret_cast<const float4*>(planes),
                       plane_stride / 4, n_planes, n4);
  } else {
    hipLaunchKernelGGL(plane_sum_bf16_scalar, dim3(grid_for(n_elem, 256)), dim3(256), 0, stream,
                       out, planes, plane_stride, n_planes, n_elem);
  }
  return hipGetLastError();
}

hipError_t launch_cross_scan(const void* x, int elem_bytes, int B, int H, int W, int D,
                             const int* route_of_slot, int n_sel, void* routes,
                             hipStream_t stream) {
  Routes4 rs{{0, 0, 0, 0}};
  for (int i = 0; i < n_sel; ++i) rs.r[i] = route_of_slot[i];
  const int64_t total = (int64_t)n_sel * B * H * W * D;
  const int vec = 16 / elem_bytes;
  if (D % vec == 0 && total / vec < ((int64_t)1 << 31) && total < ((int64_t)1 << 40)) {
    const dim3 grid(grid_for(total / vec, 256)), block(256);
    if (elem_bytes == 2)
      hipLaunchKernelGGL(cross_scan_vec_kernel<uint16_t>, grid, block, 0, stream,
                         static_cast<const uint16_t*>(x), B, H, W, D, rs, n_sel,
                         static_cast<uint16_t*>(routes));
    else
      hipLaunchKernelGGL(cross_scan_vec_kernel<uint32_t>, grid, block, 0, stream,
                         static_cast<const uint32_t*>(x), B, H, W, D, rs, n_sel,
                         static_cast<uint32_t*>(routes));
    return hipGetLastError();
  }
  const dim3 grid(grid_for(total, 256)), block(256);
  if (elem_bytes == 2) {
    hipLaunchKernelGGL(cross_scan_kernel<uint16_t>, grid, block, 0, stream,
                       static_cast<const uint16_t*>(x), B, H, W, D, rs, n_sel,
                       static_cast<uint16_t*>(routes));
  } else {
    hipLaunchKernelGGL(cross_scan_kernel<uint32_t>, grid, block, 0, stream,
                       static_cast<const uint32_t*>(x), B, H, W, D, rs, n_sel,
                       static_cast<uint32_t*>(routes));
  }
  return hipGetLastError();
}

hipError_t launch_cross_merge(const void* routes, int bf16, int B, int H, int W, int D,
                              const int* route_of_slot, int n_sel, float* out,
                              hipStream_t stream) {
  Routes4 rs{{0, 0, 0, 0}};
  for (int i = 0; i < n_sel; ++i) rs.r[i] = route_of_slot[i];
  const int64_t total = (int64_t)B * H * W * D;
  if (D % 4 == 0 && total / 4 < ((int64_t)1 << 31)) {
    const dim3 grid(grid_for(total / 4, 256)), block(256);
    if (bf16)
      hipLaunchKernelGGL(cross_merge_vec_kernel<true>, grid, block, 0, stream, routes, B, H, W, D,
                         rs, n_sel, out);
    else
      hipLaunchKernelGGL(cross_merge_vec_kernel<false>, grid, block, 0, stream, routes, B, H, W, D,
                         rs, n_sel, out);
    return hipGetLastError();
  }
  const dim3 grid(grid_for(total, 256)), block(256);
  if (bf16) {
    hipLaunchKernelGGL(cross_merge_kernel<true>, grid, block, 0, stream, routes, B, H, W, D, rs,
                       n_sel, out);
  } else {
    hipLaunchKernelGGL(cross_merge_kernel<false>, grid, block, 0, stream, routes, B, H, W, D, rs,
                       n_sel, out);
  }
  return hipGetLastError();
}

}  // namespace hope
