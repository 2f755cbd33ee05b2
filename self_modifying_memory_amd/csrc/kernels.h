// Internal launch interface between the C-ABI host code and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace hope {

// One (image, head, route) recurrence per workgroup.
struct ChainParams {
  const void* x;          // [B][H][W][D], fp32 or bf16
  const float* init;      // [4][nh][S] or [B][4][nh][S]
  float* out;             // [B][H][W][D] fp32: plane of slot 0
  float* planes;          // slots 1..n_sel-1: planes + (slot-1)*plane_stride
  float* final_mem;       // [B][4][nh][S] or nullptr
  int64_t plane_stride;   // elements between consecutive workspace planes
  int x_bf16;
  int B, H, W, D, nh;
  int n_sel;              // number of selected routes
  int route_of_slot[4];   // route index of each slot, increasing
  int chunk;              // 0 = aligned
  int init_per_image;
  int eta_map;            // 0 sigmoid, 1 softplus
  float eta_scale, alpha_bias, eps;
  int readout;            // 0 boundary (chunk-start memory), 1 running (memory after the
                          // chunk's earlier tokens)
  // variants
  const float* route_scales;     // [4][D] channel-wise direction scales, or nullptr (ones)
  const float* skip;             // [D] channel-wise skip, or nullptr
  unsigned long long* counts;    // [3] step-control counters (accumulated), or nullptr
  int injection, spectral;       // step controls (GateParams)
  unsigned frozen;               // 1: M_k, M_v; 2: m_eta, m_alpha; 4: M_q held fixed
  int no_dgd;                    // 1: drop the key-dependent correction of the update
  int shared_init;               // 1: init is [nh][S] for every route
  const void* queries;           // [B][H][W][D] queries of a fixed projection, or nullptr
  int queries_bf16;
  int mem_chunk;                 // 0: one chunk length; > 0: the working memory's own
  float* steps;                  // [B][4][nh][H*W] executed step of each token at its pixel,
                                 // or nullptr
};

// Raw query component c of pixel pix of image b (fixed-projection variant).
__device__ inline float query_at(const ChainParams& p, int b, int pix, int64_t c) {
  const int64_t i = ((int64_t)b * p.H * p.W + pix) * p.D + c;
  if (p.queries_bf16) return __uint_as_float((unsigned)static_cast<const unsigned short*>(p.queries)[i] << 16);
  return static_cast<const float*>(p.queries)[i];
}

// Offset (in floats) of the initial state of (image b, route r, head h).
__host__ __device__ inline int64_t init_offset(const ChainParams& p, int b, int r, int h, int64_t SS) {
  if (p.shared_init) return (int64_t)h * SS;
  return (p.init_per_image ? ((int64_t)b * 4 + r) * p.nh + h : (int64_t)r * p.nh + h) * SS;
}

// Backward pass, one chain per workgroup (fp32).  Per chain the workspace holds nck
// checkpoints of the state, the state adjoint and the gain trajectory of one chunk:
// chain_floats >= (nck + 1) * (4d^2 + 2d) + min(C, N) * d^2.
struct BackParams {
  const void* x;          // [B][H][W][D], fp32 or bf16
  const float* init;      // [4][nh][S] or [B][4][nh][S]
  const float* grad_out;  // [B][H][W][D] fp32
  float* grad_x;          // [B][H][W][D] fp32: plane of slot 0
  float* planes;          // slots 1..n_sel-1 of the map adjoint
  float* chain_ws;        // per-chain workspace, chain_floats apart
  int64_t plane_stride, chain_floats, nck;
  int x_bf16;
  int B, H, W, D, nh;
  int n_sel;
  int route_of_slot[4];
  int chunk;              // 0 = aligned
  int init_per_image;
  int eta_map;
  float eta_scale, alpha_bias, eps;
  int readout;            // 0 boundary, 1 running (d = 32 only)
};
// longest chunk the token-serial backward kernel holds in LDS (d = 16 and 64)
__host__ __device__ constexpr int backward_max_chunk(int d) { return d == 64 ? 32 : 128; }
// writes grad_x (slot 0 plane) and the route planes, then grad_init; the caller adds the planes
hipError_t launch_chain_backward(const BackParams& p, int d, float* grad_init, hipStream_t stream);
// chunk-parallel backward on the fp32 matrix cores: d = 64, every chunk <= 16 tokens
bool backward_wy_supported(const BackParams& p, int d);
hipError_t launch_chain_backward_wy(const BackParams& p, hipStream_t stream);
// chunk-parallel backward on the fp32 matrix cores in 16-token blocks: d = 32, any chunk
// length; its workspace per chain (the state adjoint first, then the chunk records)
bool backward_wy32_supported(const BackParams& p, int d);
int64_t backward_wy32_chain_floats(int64_t nck, int64_t cmax);
hipError_t launch_chain_backward_wy32(const BackParams& p, hipStream_t stream);

// The scan kernel a forward call launches (host-side dispatch, api.hip).
enum ScanPath { kPathChain = 0, kPathMfma = 1, kPathChunk = 2 };
ScanPath select_scan_path(const ChainParams& p, int d);
const char* scan_path_kernel(ScanPath path);
hipError_t launch_scan(const ChainParams& p, int d, hipStream_t stream);

// fp32 VALU kernel: any supported head dimension and dtype (exact fp32 arithmetic).
hipError_t launch_chain(const ChainParams& p, int d, hipStream_t stream);

// Chunk-parallel MFMA kernel for bf16 maps at d = 16 or 32 (any chunk length; boundary
// readout, one chunk length).
bool chunk_path_supported(const ChainParams& p, int d);
hipError_t launch_chain_chunk(const ChainParams& p, int d, hipStream_t stream);
// true when the call asks for any variant that only the variant instantiations implement
bool needs_variants(const ChainParams& p);

// MFMA kernel for bf16 maps (d = 32, or d = 64 with every chunk <= 16 tokens).
bool mfma_path_supported(const ChainParams& p, int d);
hipError_t launch_chain_mfma(const ChainParams& p, int d, hipStream_t stream);

// out = bf16(planes[0] + planes[1] + ...) in that order, rounded once to nearest even
hipError_t launch_plane_sum_bf16(unsigned short* out, const float* planes, int64_t plane_stride,
                                 int n_planes, int64_t n_elem, hipStream_t stream);
// out[i] += planes[0][i] + ... + planes[n-1][i], left to right, fp32 (route sum).
hipError_t launch_plane_sum(float* out, const float* planes, int64_t plane_stride, int n_planes,
                            int64_t n_elem, hipStream_t stream);

// Bit-exact permutation of x into route order: routes[slot][b][t][c] = x[b][p_r(t)][c].
hipError_t launch_cross_scan(const void* x, int elem_bytes, int B, int H, int W, int D,
                             const int* route_of_slot, int n_sel, void* routes, hipStream_t stream);

// out[b][p][c] = sum over slots (increasing route) of routes[slot][b][p_r^-1(p)][c].
hipError_t launch_cross_merge(const void* routes, int bf16, int B, int H, int W, int D,
                              const int* route_of_slot, int n_sel, float* out, hipStream_t stream);

}  // namespace hope
