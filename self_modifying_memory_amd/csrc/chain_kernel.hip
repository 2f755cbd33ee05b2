// Fused chunked recurrence of one (image, head, route) chain per workgroup, gfx950.
//
// Method ("VisionHOPE: Visual Backbones as Self-Modifying Learning Systems"):
//   Sec. 2.3 Eq. 24-25   route order and row/column-aligned chunks;
//   Sec. 2.1.3 Eq. 15-16 k, v, q, eta, alpha and y = M_mem q from the chunk-start state;
//                        or the running readout y_t = M_mem,b G_{t-1} q_t ("Nested
//                        Learning", Eq. 94 applied inside the chunk);
//   Sec. 2.2 Eq. 19-20   executed step (soft injection cap, spectral clamp) with the
//                        App. B.3 inward factors, |k|^2 floor and one-ulp rounding;
//   App. B.4 Eq. 46      one gain G per chunk, G_t = alpha_t G_{t-1} - step_t (G_{t-1} k_t
//                        + delta_t) k_t^T, shared by all six memories: S_end = S_b G_C;
//   "Nested Learning"    two chunk sizes (one for the working memory, one for the
//                        projection memories): M_mem then carries a second gain of the same
//                        recurrence, reset at its own boundaries.
//
// Layout: the fp32 state (4d+2 rows of d: M_mem, M_k, M_v, M_q, m_eta, m_alpha) stays
// in LDS for the whole sequence; tokens are processed in blocks of kTB; each thread
// keeps a strip of one row of G in registers.
#include "device_common.h"
#include "kernels.h"

namespace hope {
namespace {

constexpr int kThreads = 256;
constexpr int kTB = 16;  // tokens per LDS block

__device__ __forceinline__ float load_x(const void* x, int bf16, int64_t idx) {
  if (bf16) {
    uint32_t b = static_cast<const uint16_t*>(x)[idx];
    return __uint_as_float(b << 16);
  }
  return static_cast<const float*>(x)[idx];
}

template <int D>
__global__ __launch_bounds__(kThreads) void chain_kernel(ChainParams p) {
  constexpr int R = 4 * D + 2;        // state rows
  constexpr int SP = D + 1;           // padded LDS row stride of state / tokens / gain
  constexpr int NP = 3 * D + 2;       // projected rows: k, v, q, s_eta, s_alpha
  constexpr int PS = NP + 1;          // padded per-token stride of the projections
  constexpr int TPR = kThreads / D;   // threads per gain row
  constexpr int CPT = D / TPR;        // gain columns per thread
  constexpr int NG = kThreads / D;    // row groups of the state update

  __shared__ float S[R * SP];
  __shared__ float X[kTB * SP];
  __shared__ float P[kTB * PS];
  __shared__ float Gl[D * SP];
  __shared__ float Glm[D * SP];   // the working memory's gain (two chunk sizes)
  __shared__ float Wq[kTB * SP];  // running readout: w_t = G_{t-1} q_t per token
  const bool running = p.readout != 0;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int nh = p.nh;
  const int h = blockIdx.x % nh;
  const int b = (blockIdx.x / nh) % p.B;
  const int slot = blockIdx.x / (nh * p.B);
  const int r = p.route_of_slot[slot];
  const int H = p.H, W = p.W, N = H * W, Dt = p.D;
  const int C = p.chunk > 0 ? p.chunk : (r < 2 ? W : H);
  const int Cm = p.mem_chunk > 0 ? p.mem_chunk : C;  // the working memory's chunk length
  const bool two = Cm != C;
  const int64_t SS = 4 * D * D + 2 * D;

  float* dst = slot == 0 ? p.out : p.planes + (int64_t)(slot - 1) * p.plane_stride;
  const float* init = p.init + init_offset(p, b, r, h, SS);
  for (int e = tid; e < R * D; e += kThreads) S[(e / D) * SP + e % D] = init[e];

  const int grow = tid / TPR;         // gain row owned by this thread
  const int gcol0 = (tid % TPR) * CPT;
  const GateParams gp{p.eta_map, p.eta_scale, p.alpha_bias, p.eps, p.injection, p.spectral};
  unsigned long long n_upd = 0, n_inj = 0, n_spec = 0;  // step-control counters (lane 0)
  // rows held fixed within the image: M_k, M_v (bit 0), the gate rows (bit 1), M_q (bit 2)
  const unsigned frozen = p.frozen | (p.queries ? 4u : 0u);  // given queries: M_q takes no part
  auto frozen_row = [&](int row) {
    return ((frozen & 1u) && row >= D && row < 3 * D) || ((frozen & 4u) && row >= 3 * D && row < 4 * D) ||
           ((frozen & 2u) && row >= 4 * D);
  };
  __syncthreads();

  // Segments run to the next boundary of either chunk grid; g is the gain of the memories
  // on the projection grid (all six with one chunk size), gm that of M_mem on its own.
  float g[CPT], gm[CPT];
  for (int s0 = 0; s0 < N;) {
    const int end_p = min((s0 / C + 1) * C, N);
    const int end_m = two ? min((s0 / Cm + 1) * Cm, N) : end_p;
    const int s1 = min(end_p, end_m);
    if (s0 % C == 0) {
#pragma unroll
      for (int c = 0; c < CPT; ++c) g[c] = (gcol0 + c == grow) ? 1.f : 0.f;
    }
    if (two && s0 % Cm == 0) {
#pragma unroll
      for (int c = 0; c < CPT; ++c) gm[c] = (gcol0 + c == grow) ? 1.f : 0.f;
    }

    for (int tb = s0; tb < s1; tb += kTB) {
      const int nt = min(kTB, s1 - tb);
      // gather the block's tokens in route order
      for (int e = tid; e < nt * D; e += kThreads) {
        const int t = e / D, i = e % D;
        const int pix = route_pixel(r, tb + t, H, W, N);
        X[t * SP + i] = load_x(p.x, p.x_bf16, ((int64_t)b * N + pix) * Dt + (int64_t)h * D + i);
      }
      __syncthreads();
      // projections from the chunk-start memories (Eq. 15): rows D.. of the state
      for (int e = tid; e < nt * NP; e += kThreads) {
        const int t = e % nt, j = e / nt;
        const float* srow = &S[(D + j) * SP];
        const float* xrow = &X[t * SP];
        float acc = 0.f;
#pragma unroll 16
        for (int i = 0; i < D; ++i) acc = fmaf(srow[i], xrow[i], acc);
        P[t * PS + j] = acc;
      }
      __syncthreads();
      // gates and executed step (Eq. 19-20), one wave per token
      for (int t = wave; t < nt; t += kThreads / 64) {
        float* pt = &P[t * PS];
        const float kr = lane < D ? pt[lane] : 0.f;
        const float vr = lane < D ? pt[D + lane] : 0.f;
        float qr = 0.f;
        if (lane < D) {
          qr = p.queries ? query_at(p, b, route_pixel(r, tb + t, H, W, N), (int64_t)h * D + lane)
                         : pt[2 * D + lane];
        }
        const TokenGates tg = token_gates(kr, vr, qr, pt[3 * D], pt[3 * D + 1], gp);
        const float k = tg.k, q = tg.q, dl = tg.delta, step = tg.step, alpha = tg.alpha;
        if (lane < D) {
          pt[lane] = k;
          pt[D + lane] = dl;
          pt[2 * D + lane] = q;
        }
        if (lane == 0) {
          pt[3 * D] = step;
          pt[3 * D + 1] = alpha;
          if (p.steps)
            p.steps[(((int64_t)b * 4 + r) * p.nh + h) * N + route_pixel(r, tb + t, H, W, N)] = step;
          n_upd += 1;
          n_inj += tg.flags & 1;
          n_spec += (tg.flags >> 1) & 1;
        }
      }
      __syncthreads();
      // readout y_t = M_mem,b v_t with v_t = q_t (Eq. 16, boundary) or v_t = G_{t-1} q_t
      // (running: M_mem,b G_{t-1} is the memory after the chunk's earlier tokens),
      // written at the token's pixel
      // then the channel-wise skip and direction scale: (y + skip x) lambda_r
      auto readout = [&](const float* vbase, int vstride) {
        for (int e = tid; e < nt * D; e += kThreads) {
          const int t = e / D, i = e % D;
          const float* mrow = &S[i * SP];
          const float* qv = vbase + t * vstride;
          float acc = 0.f;
#pragma unroll 16
          for (int j = 0; j < D; ++j) acc = fmaf(mrow[j], qv[j], acc);
          const int64_t c = (int64_t)h * D + i;
          if (p.skip) acc = fmaf(p.skip[c], X[t * SP + i], acc);
          if (p.route_scales) acc *= p.route_scales[(int64_t)r * Dt + c];
          const int pix = route_pixel(r, tb + t, H, W, N);
          dst[((int64_t)b * N + pix) * Dt + c] = acc;
        }
      };
      if (!running) readout(&P[2 * D], PS);
      // shared gain, token by token (Eq. 46)
      for (int t = 0; t < nt; ++t) {
        const float* pt = &P[t * PS];
        float w = 0.f, wm = 0.f, wq = 0.f;
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
          w = fmaf(g[c], pt[gcol0 + c], w);
          if (two) wm = fmaf(gm[c], pt[gcol0 + c], wm);
          if (running) wq = fmaf(two ? gm[c] : g[c], pt[2 * D + gcol0 + c], wq);
        }
#pragma unroll
        for (int off = TPR / 2; off >= 1; off >>= 1) {
          w += __shfl_xor(w, off, 64);
          if (two) wm += __shfl_xor(wm, off, 64);
          if (running) wq += __shfl_xor(wq, off, 64);
        }
        if (running && tid % TPR == 0) Wq[t * SP + grow] = wq;
        const float step = pt[3 * D], alpha = pt[3 * D + 1];
        const float u = -step * (p.no_dgd ? pt[D + grow] : w + pt[D + grow]);
#pragma unroll
        for (int c = 0; c < CPT; ++c) g[c] = fmaf(alpha, g[c], u * pt[gcol0 + c]);
        if (two) {
          const float um = -step * (p.no_dgd ? pt[D + grow] : wm + pt[D + grow]);
#pragma unroll
          for (int c = 0; c < CPT; ++c) gm[c] = fmaf(alpha, gm[c], um * pt[gcol0 + c]);
        }
      }
      __syncthreads();
      if (running) {
        readout(Wq, SP);
        __syncthreads();
      }
    }
    // carry S <- S_b G at the end of a chunk: rows [rb, re) with the gain in Gs.  Rows are
    // independent, so the product runs in passes of kRB rows per thread; a barrier
    // separates each pass's reads from its in-place writes
    auto carry = [&](const float* Gs, int rb, int re) {
      constexpr int kRB = 8;
      const int col = tid % D, grp = tid / D;
      float gc[D];
#pragma unroll
      for (int j = 0; j < D; ++j) gc[j] = Gs[j * SP + col];
#pragma unroll 1
      for (int r0 = rb; r0 < re; r0 += kRB * NG) {
        float acc[kRB];
#pragma unroll
        for (int k = 0; k < kRB; ++k) {
          const int row = r0 + grp + k * NG;
          float a = 0.f;
          if (row < re) {
            const float* srow = &S[row * SP];
#pragma unroll
            for (int j = 0; j < D; ++j) a = fmaf(srow[j], gc[j], a);
          }
          acc[k] = a;
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < kRB; ++k) {
          const int row = r0 + grp + k * NG;
          if (row < re && !frozen_row(row)) S[row * SP + col] = acc[k];
        }
      }
    };
    const bool carry_p = s1 == end_p, carry_m = s1 == end_m;
#pragma unroll
    for (int c = 0; c < CPT; ++c) Gl[grow * SP + gcol0 + c] = g[c];
    if (two) {
#pragma unroll
      for (int c = 0; c < CPT; ++c) Glm[grow * SP + gcol0 + c] = gm[c];
    }
    __syncthreads();
    if (!two) {
      carry(Gl, 0, R);  // all six memories at once
    } else {
      if (carry_m) carry(Glm, 0, D);  // M_mem at its own boundary
      if (carry_p) carry(Gl, D, R);   // the projection memories at theirs
    }
    __syncthreads();
    s0 = s1;
  }

  if (p.final_mem) {
    float* fin = p.final_mem + (((int64_t)b * 4 + r) * nh + h) * SS;
    for (int e = tid; e < R * D; e += kThreads) fin[e] = S[(e / D) * SP + e % D];
  }
  if (p.counts && lane == 0) {
    atomicAdd(&p.counts[0], n_upd);
    atomicAdd(&p.counts[1], n_inj);
    atomicAdd(&p.counts[2], n_spec);
  }

}

}  // namespace

hipError_t launch_chain(const ChainParams& p, int d, hipStream_t stream) {
  const int64_t blocks = (int64_t)p.n_sel * p.B * p.nh;
  dim3 grid((unsigned)blocks), block(kThreads);
  switch (d) {
    case 16: hipLaunchKernelGGL(chain_kernel<16>, grid, block, 0, stream, p); break;
    case 32: hipLaunchKernelGGL(chain_kernel<32>, grid, block, 0, stream, p); break;
    case 64: hipLaunchKernelGGL(chain_kernel<64>, grid, block, 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace hope
