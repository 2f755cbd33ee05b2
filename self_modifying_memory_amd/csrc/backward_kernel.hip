// Backward pass of the four-direction scan, gfx950: gradients of a loss L(out) with
// respect to the feature map and the initial memories, one (image, head, route) chain per
// workgroup, exact fp32 arithmetic.
//
// Forward per chunk [s, e) from the boundary state S_b ("VisionHOPE: Visual Backbones as
// Self-Modifying Learning Systems"): projections (Sec. 2.1.3 Eq. 15), normalisation
// (App. C.1), gates and executed step (Sec. 2.2 Eq. 19-20 with the App. B.3 safeguards),
// readout y_t = M_mem,b q_t (Eq. 16), the shared gain G_t = G_{t-1} A_t + B_t with
// A_t = alpha_t I - step_t k_t k_t^T and B_t = -step_t delta_t k_t^T (App. B.4 Eq. 46),
// and the carry S_end = S_b G_e.  The memory trajectory is explicit and differentiable
// (Sec. 1); reverse mode per chunk, last chunk first, with dS the adjoint of the chunk's
// end state:
//   dG_e = S_b^T dS,  dS_b = dS G_e^T + (projection and readout terms);
//   for t = e-1 .. s, with a = dG_t k_t and b = G_{t-1} k_t:
//     dalpha_t += <G_{t-1}, dG_t>,  dstep_t += -(b + delta_t)^T a,
//     dk_t += -step_t (G_{t-1}^T a + dG_t^T (b + delta_t)),  ddelta_t += -step_t a,
//     dG_{t-1} = alpha_t dG_t - step_t a k_t^T;
//   then, token by token, the readout, the step, the gates, the normalisation and the
//   projections.  Where the step is not differentiable: min(eta_bar, eta_spec) follows
//   eta_bar when eta_bar <= eta_spec; no derivative through the |k|^2 floor or the
//   one-ulp rounding of eta_spec; eta_bar = 0 (eta = 0 or eta_inj = 0) has derivative 0.
//
// A forward sweep stores each chunk's boundary state in the workspace (checkpoints); per
// chunk of the reverse sweep the gain trajectory G_{t-1} is recomputed into the workspace.
// Layout per chain: the state S_b and the gain adjoint in LDS; the state adjoint in
// registers, thread (col, grp) holding column col of rows grp, grp + NG, ...; per-token
// quantities of the chunk in LDS.  The state adjoint reaches the workspace once, at the
// end, for the initial-state gradient.
#include <algorithm>

#include "device_common.h"
#include "kernels.h"

namespace hope {
namespace {

constexpr int kTB = 16;  // tokens per block of the projection passes
// threads per chain: 512 at d = 64 (8 waves, two per SIMD: half the state-adjoint rows
// per thread of 256), 256 below (measured faster at d = 32)
constexpr int back_threads(int d) { return d == 64 ? 512 : 256; }

__device__ __forceinline__ float load_xb(const void* x, int bf16, int64_t idx) {
  if (bf16) return __uint_as_float((uint32_t) static_cast<const uint16_t*>(x)[idx] << 16);
  return static_cast<const float*>(x)[idx];
}

template <int D>
__global__ __launch_bounds__(back_threads(D)) void chain_backward_kernel(BackParams p) {
  constexpr int kThreads = back_threads(D);
  constexpr int R = 4 * D + 2;        // state rows
  constexpr int SP = D + 1;           // padded LDS row stride
  constexpr int NP = 3 * D + 2;       // projected rows: k, v, q, s_eta, s_alpha
  constexpr int PS = NP + 1;
  constexpr int TPR = kThreads / D;   // threads per gain row
  constexpr int CPT = D / TPR;        // gain columns per thread
  constexpr int NG = kThreads / D;    // row groups
  constexpr int MC = backward_max_chunk(D);
  constexpr int RPT = (R + NG - 1) / NG;  // state-adjoint rows per thread
  constexpr int kSR = 4;                  // row slots staged per pass of dS G^T
  constexpr float kInjInward = 1.f - 1e-3f, kSpecInward = 1.f - 1e-6f, kKappaFloor = 1e-20f;

  __shared__ float S[R * SP];         // boundary state of the chunk
  __shared__ float X[kTB * SP];       // token block
  __shared__ float P[kTB * PS];       // its projections, then their adjoints
  __shared__ float Kc[MC * SP];       // k_t of the chunk, then dL/dk_t (gain part)
  __shared__ float Dc[MC * SP];       // delta_t, then dL/ddelta_t (gain part)
  __shared__ float Ec[MC], Ac[MC];    // step_t, alpha_t, then their adjoints (gain part)
  __shared__ float Gb[D * SP];        // G_end, then G_{t-1} in the reverse loop
  __shared__ float dG[D * SP];        // adjoint of the gain
  __shared__ float Qb[kTB * SP];      // q_t of the block
  __shared__ float DY[kTB * SP];      // dL/dy_t of the block
  __shared__ float va[D], vb[D], vk[D];
  __shared__ float red[kThreads / 64];
  __shared__ float red2[kThreads];       // column partial sums, [row group][column]
  __shared__ int pixb[kTB];
  __shared__ float Stg[kSR * kThreads];  // staging of dS rows (kSR slots x NG rows x D)

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
  const int nck = (N + C - 1) / C;
  const int64_t SS = (int64_t)R * D;

  float* const ckpt = p.chain_ws + (int64_t)blockIdx.x * p.chain_floats;
  float* const dSg = ckpt + p.nck * SS;
  float* const gtr = dSg + SS;
  float* const gdst = slot == 0 ? p.grad_x : p.planes + (int64_t)(slot - 1) * p.plane_stride;
  const GateParams gp{p.eta_map, p.eta_scale, p.alpha_bias, p.eps, 0, 0};
  const int grow = tid / TPR, gcol0 = (tid % TPR) * CPT;
  const int col = tid % D, grp = tid / D;  // state-adjoint ownership
  float dsr[RPT];                          // dS[grp + k NG][col]

  {
    const float* init = p.init + (p.init_per_image ? ((int64_t)b * 4 + r) * nh + h : (int64_t)r * nh + h) * SS;
    for (int e = tid; e < R * D; e += kThreads) S[(e / D) * SP + e % D] = init[e];
  }
  __syncthreads();

  // tokens tb .. tb+nt-1: x into X, pixels, projections P = S_b[rows D..] x
  auto load_block = [&](int tb, int nt) {
    for (int e = tid; e < nt * D; e += kThreads) {
      const int t = e / D, i = e % D;
      const int pix = route_pixel(r, tb + t, H, W, N);
      X[t * SP + i] = load_xb(p.x, p.x_bf16, ((int64_t)b * N + pix) * Dt + (int64_t)h * D + i);
    }
    if (tid < kTB) pixb[tid] = tid < nt ? route_pixel(r, tb + tid, H, W, N) : 0;
    __syncthreads();
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
  };
  // k, delta, step, alpha of every token of the chunk into Kc, Dc, Ec, Ac
  auto chunk_gates = [&](int s0, int s1) {
    for (int tb = s0; tb < s1; tb += kTB) {
      const int nt = min(kTB, s1 - tb);
      load_block(tb, nt);
      for (int t = wave; t < nt; t += kThreads / 64) {
        const float* pt = &P[t * PS];
        const float kr = lane < D ? pt[lane] : 0.f;
        const float vr = lane < D ? pt[D + lane] : 0.f;
        const float qr = lane < D ? pt[2 * D + lane] : 0.f;
        const TokenGates tg = token_gates(kr, vr, qr, pt[3 * D], pt[3 * D + 1], gp);
        const int tl = tb - s0 + t;
        if (lane < D) {
          Kc[tl * SP + lane] = tg.k;
          Dc[tl * SP + lane] = tg.delta;
        }
        if (lane == 0) {
          Ec[tl] = tg.step;
          Ac[tl] = tg.alpha;
        }
      }
      __syncthreads();
    }
  };
  // the chunk's gain, row strips in registers; store: G_{t-1} of every token to gtr.
  // Leaves G_end in Gb.
  auto gain_forward = [&](int s0, int s1, bool store) {
    float g[CPT];
#pragma unroll
    for (int c = 0; c < CPT; ++c) g[c] = (gcol0 + c == grow) ? 1.f : 0.f;
    for (int t = s0; t < s1; ++t) {
      const int tl = t - s0;
      if (store) {
#pragma unroll
        for (int c = 0; c < CPT; ++c) gtr[(int64_t)tl * D * D + grow * D + gcol0 + c] = g[c];
      }
      float w = 0.f;
#pragma unroll
      for (int c = 0; c < CPT; ++c) w = fmaf(g[c], Kc[tl * SP + gcol0 + c], w);
#pragma unroll
      for (int off = TPR / 2; off >= 1; off >>= 1) w += __shfl_xor(w, off, 64);
      const float step = Ec[tl], alpha = Ac[tl];
      const float u = -step * (w + Dc[tl * SP + grow]);
#pragma unroll
      for (int c = 0; c < CPT; ++c) g[c] = fmaf(alpha, g[c], u * Kc[tl * SP + gcol0 + c]);
    }
#pragma unroll
    for (int c = 0; c < CPT; ++c) Gb[grow * SP + gcol0 + c] = g[c];
    __syncthreads();
  };
  // rows of M (LDS, stride SP, or global, stride D) times G_end (transposed when trans):
  // M[row] <- M[row] G (forward carry) or M[row] G^T (adjoint carry), in place, rows in
  // passes of kRB per thread with a barrier between each pass's reads and writes
  auto rows_times_gain = [&](float* M, int stride, bool trans) {
    constexpr int kRB = 8;
    float gc[D];
#pragma unroll
    for (int j = 0; j < D; ++j) gc[j] = trans ? Gb[col * SP + j] : Gb[j * SP + col];
#pragma unroll 1
    for (int r0 = 0; r0 < R; r0 += kRB * NG) {
      float acc[kRB];
#pragma unroll
      for (int k = 0; k < kRB; ++k) {
        const int row = r0 + grp + k * NG;
        float a = 0.f;
        if (row < R) {
          const float* mrow = M + (int64_t)row * stride;
#pragma unroll
          for (int j = 0; j < D; ++j) a = fmaf(mrow[j], gc[j], a);
        }
        acc[k] = a;
      }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < kRB; ++k) {
        const int row = r0 + grp + k * NG;
        if (row < R) M[(int64_t)row * stride + col] = acc[k];
      }
    }
    __syncthreads();
  };

  // ---- forward sweep: checkpoints of every chunk's boundary state ----------------
  for (int c = 0; c < nck; ++c) {
    const int s0 = c * C, s1 = min(s0 + C, N);
    for (int e = tid; e < R * D; e += kThreads) ckpt[(int64_t)c * SS + e] = S[(e / D) * SP + e % D];
    if (c == nck - 1) break;  // the state after the last chunk is not needed
    chunk_gates(s0, s1);
    gain_forward(s0, s1, false);
    rows_times_gain(S, SP, false);
  }
#pragma unroll
  for (int k = 0; k < RPT; ++k) dsr[k] = 0.f;  // no loss on the final state

  // ---- reverse sweep ------------------------------------------------------------------
  for (int c = nck - 1; c >= 0; --c) {
    const int s0 = c * C, s1 = min(s0 + C, N);
    for (int e = tid; e < R * D; e += kThreads) S[(e / D) * SP + e % D] = ckpt[(int64_t)c * SS + e];
    __syncthreads();
    chunk_gates(s0, s1);
    gain_forward(s0, s1, true);

    // dG_e = S_b^T dS: each thread's partial over its rows, added into dG one row group
    // at a time (a fixed order)
    // (16 rows of dG per pass, to bound the partials held in registers)
    for (int i0 = 0; i0 < D; i0 += 16) {
      float part[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) part[i] = 0.f;
#pragma unroll
      for (int k = 0; k < RPT; ++k) {
        const int row = grp + k * NG;
        if (row < R) {
#pragma unroll
          for (int i = 0; i < 16; ++i) part[i] = fmaf(S[row * SP + i0 + i], dsr[k], part[i]);
        }
      }
      for (int gsel = 0; gsel < NG; ++gsel) {
        if (grp == gsel) {
#pragma unroll
          for (int i = 0; i < 16; ++i)
            dG[(i0 + i) * SP + col] = gsel == 0 ? part[i] : dG[(i0 + i) * SP + col] + part[i];
        }
        __syncthreads();
      }
    }
    // dS <- dS G_e^T: rows staged through LDS, kSR row slots per pass (unrolled, so that
    // the register array is indexed statically)
#pragma unroll
    for (int k0 = 0; k0 < RPT; k0 += kSR) {
#pragma unroll
      for (int kk = 0; kk < kSR; ++kk)
        if (k0 + kk < RPT) Stg[kk * kThreads + tid] = dsr[k0 + kk];  // = [slot][grp][col]
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < kSR; ++kk) {
        if (k0 + kk < RPT) {
          const float* srow = &Stg[kk * kThreads + grp * D];
          float acc = 0.f;
#pragma unroll
          for (int i = 0; i < D; ++i) acc = fmaf(srow[i], Gb[col * SP + i], acc);
          dsr[k0 + kk] = acc;
        }
      }
      __syncthreads();
    }

    // gain recurrence backwards, token by token
    constexpr int GPT = D * D / kThreads;
    float gpre[GPT];
#pragma unroll
    for (int m = 0; m < GPT; ++m) gpre[m] = gtr[(int64_t)(s1 - 1 - s0) * D * D + tid + m * kThreads];
    for (int t = s1 - 1; t >= s0; --t) {
      const int tl = t - s0;
#pragma unroll
      for (int m = 0; m < GPT; ++m) {
        const int e = tid + m * kThreads;
        Gb[(e / D) * SP + e % D] = gpre[m];
      }
      if (tl > 0) {
#pragma unroll
        for (int m = 0; m < GPT; ++m) gpre[m] = gtr[(int64_t)(tl - 1) * D * D + tid + m * kThreads];
      }
      if (tid < D) vk[tid] = Kc[tl * SP + tid];
      __syncthreads();
      const float step = Ec[tl], alpha = Ac[tl];
      // row parts: a_i = (dG k)_i, b_i = (G k)_i, and <G, dG>
      float trp = 0.f, pa = 0.f, pb = 0.f;
#pragma unroll
      for (int cc = 0; cc < CPT; ++cc) {
        const int j = gcol0 + cc;
        const float gv = Gb[grow * SP + j], dv = dG[grow * SP + j], kj = vk[j];
        trp = fmaf(gv, dv, trp);
        pa = fmaf(dv, kj, pa);
        pb = fmaf(gv, kj, pb);
      }
#pragma unroll
      for (int off = TPR / 2; off >= 1; off >>= 1) {
        pa += __shfl_xor(pa, off, 64);
        pb += __shfl_xor(pb, off, 64);
      }
      trp = wave_sum(trp);
      if (lane == 0) red[wave] = trp;
      if (tid % TPR == 0) {
        va[grow] = pa;
        vb[grow] = pb + Dc[tl * SP + grow];  // b + delta
      }
      __syncthreads();
      // column parts: (G^T a + dG^T (b + delta))_j over rows q, q + NG, ...
      {
        const int q = tid / D;
        float ce = 0.f;
#pragma unroll 4
        for (int i = q; i < D; i += NG) ce = fmaf(Gb[i * SP + col], va[i], fmaf(dG[i * SP + col], vb[i], ce));
        red2[q * D + col] = ce;
      }
      __syncthreads();
      if (wave == 0) {
        float dk = 0.f, ddl = 0.f, part = 0.f;
        if (lane < D) {
          float ce = 0.f;
          for (int q = 0; q < NG; ++q) ce += red2[q * D + lane];
          dk = -step * ce;
          ddl = -step * va[lane];
          part = vb[lane] * va[lane];
        }
        part = wave_sum(part);
        if (lane < D) {
          Kc[tl * SP + lane] = dk;
          Dc[tl * SP + lane] = ddl;
        }
        if (lane == 0) {
          float tr = 0.f;
#pragma unroll
          for (int q = 0; q < kThreads / 64; ++q) tr += red[q];
          Ec[tl] = -part;
          Ac[tl] = tr;
        }
      }
      __syncthreads();  // the column sums have read dG
#pragma unroll
      for (int cc = 0; cc < CPT; ++cc) {
        const int j = gcol0 + cc;
        dG[grow * SP + j] = fmaf(alpha, dG[grow * SP + j], -step * va[grow] * vk[j]);
      }
      __syncthreads();
    }

    // token by token: readout, step, gates, normalisation, projections
    for (int tb = s0; tb < s1; tb += kTB) {
      const int nt = min(kTB, s1 - tb);
      load_block(tb, nt);
      for (int e = tid; e < kTB * D; e += kThreads) {
        const int t = e / D, i = e % D;
        if (t < nt) {
          DY[t * SP + i] = p.grad_out[((int64_t)b * N + pixb[t]) * Dt + (int64_t)h * D + i];
        } else {  // padding tokens: zero rows, so the sums below run over all kTB
          DY[t * SP + i] = 0.f;
          X[t * SP + i] = 0.f;
          Qb[t * SP + i] = 0.f;
        }
      }
      for (int e = tid; e < (kTB - nt) * NP; e += kThreads) P[(nt + e / NP) * PS + e % NP] = 0.f;
      __syncthreads();
      for (int t = wave; t < nt; t += kThreads / 64) {
        float* pt = &P[t * PS];
        const int tl = tb - s0 + t;
        const bool on = lane < D;
        const float kr = on ? pt[lane] : 0.f;
        const float vr = on ? pt[D + lane] : 0.f;
        const float qr = on ? pt[2 * D + lane] : 0.f;
        const float se = pt[3 * D], sa = pt[3 * D + 1];
        // forward values, as in token_gates / executed_step
        const float nk = sqrtf(wave_sum(kr * kr) + gp.eps);
        const float nq = sqrtf(wave_sum(qr * qr) + gp.eps);
        const float k = kr / nk, q = qr / nq;
        const float dl = k - vr;
        const float dd = wave_sum(dl * dl), kk = wave_sum(k * k);
        float eta, deta_dse;
        if (gp.eta_map == 0) {
          const float sg = fast_rcp(1.f + fast_exp(-se));
          eta = gp.eta_scale * sg;
          deta_dse = gp.eta_scale * sg * (1.f - sg);
        } else {
          eta = gp.eta_scale * (fmaxf(se, 0.f) + log1pf(fast_exp(-fabsf(se))));
          deta_dse = gp.eta_scale * fast_rcp(1.f + fast_exp(-se));
        }
        const float ez = fast_exp(-(sa + gp.alpha_bias));
        const float alpha = fast_rcp(1.f + ez);
        const float oma = ez * alpha;  // 1 - alpha
        const float rr0 = fast_sqrt(dd + gp.eps * gp.eps);
        const float rr = rr0 + gp.eps;
        const float inj = kInjInward * oma * fast_rcp(rr);
        const bool ok = eta != 0.f && inj != 0.f;
        const float xr = ok ? eta * fast_rcp(inj) : 0.f;
        const float ex = fast_exp(-xr);
        const float bar = ok ? inj * one_minus_exp_neg(xr) : 0.f;
        const float kap = fmaxf(kk, kKappaFloor);
        const float spec_raw = kSpecInward * 2.f * alpha * fast_rcp(kap);
        const float spec = spec_raw > 0.f ? __uint_as_float(__float_as_uint(spec_raw) - 1u) : spec_raw;
        // adjoints from the gain and the readout
        float dk = on ? Kc[tl * SP + lane] : 0.f;
        float ddl = on ? Dc[tl * SP + lane] : 0.f;
        const float dstep = Ec[tl];
        float dalpha = Ac[tl];
        float dq = 0.f;
        if (on)
          for (int rr2 = 0; rr2 < D; ++rr2) dq = fmaf(S[rr2 * SP + lane], DY[t * SP + rr2], dq);
        // step = min(eta_bar, eta_spec)
        float deta = 0.f, ddd = 0.f, dkk = 0.f;
        if (bar <= spec) {
          if (ok) {
            deta = dstep * ex;
            const float dinj = dstep * ((1.f - ex) - xr * ex);
            dalpha -= dinj * kInjInward * fast_rcp(rr);
            const float drr = -dinj * inj * fast_rcp(rr);
            ddd = drr * 0.5f * fast_rcp(rr0);
          }
        } else {
          dalpha += dstep * kSpecInward * 2.f * fast_rcp(kap);
          if (kk > kKappaFloor) dkk = -dstep * spec_raw * fast_rcp(kap);
        }
        ddl = fmaf(2.f * dl, ddd, ddl);
        dk = fmaf(2.f * k, dkk, dk);
        dk += ddl;                       // delta = k - v
        const float dv = -ddl;
        const float kdk = wave_sum(k * dk), qdq = wave_sum(q * dq);
        const float dkr = (dk - k * kdk) / nk;
        const float dqr = (dq - q * qdq) / nq;
        if (on) {
          pt[lane] = dkr;
          pt[D + lane] = dv;
          pt[2 * D + lane] = dqr;
          Qb[t * SP + lane] = q;
        }
        if (lane == 0) {
          pt[3 * D] = deta * deta_dse;
          pt[3 * D + 1] = dalpha * alpha * oma;
        }
      }
      __syncthreads();
      // state adjoint: dM_mem += dy q^T; the projection rows += (their adjoint) x^T
      {
#pragma unroll
        for (int k = 0; k < RPT; ++k) {
          const int rr = grp + k * NG;
          if (rr < R) {
            float acc = 0.f;
            if (rr < D) {
#pragma unroll 4
              for (int t = 0; t < kTB; ++t) acc = fmaf(DY[t * SP + rr], Qb[t * SP + col], acc);
            } else {
#pragma unroll 4
              for (int t = 0; t < kTB; ++t) acc = fmaf(P[t * PS + rr - D], X[t * SP + col], acc);
            }
            dsr[k] += acc;
          }
          __builtin_amdgcn_sched_barrier(0);  // one row's loads in flight at a time
        }
      }
      // map adjoint of this route: dx_t = sum over projection rows of (their adjoint) row
      for (int e = tid; e < nt * D; e += kThreads) {
        const int t = e / D, j = e % D;
        float acc = 0.f;
        for (int rr = D; rr < R; ++rr) acc = fmaf(P[t * PS + rr - D], S[rr * SP + j], acc);
        gdst[((int64_t)b * N + pixb[t]) * Dt + (int64_t)h * D + j] = acc;
      }
      __syncthreads();
    }
  }
  // the initial-state adjoint of this chain, for the gradient reduction
#pragma unroll
  for (int k = 0; k < RPT; ++k) {
    const int rr = grp + k * NG;
    if (rr < R) dSg[(int64_t)rr * D + col] = dsr[k];
  }
}

// grad_init from the chains' state adjoints, summed over images in order when the initial
// state is shared by the batch; zero rows for unselected routes
__global__ void init_grad_kernel(BackParams p, float* grad_init, int64_t SS, int64_t dS_off) {
  const int64_t n_out = (p.init_per_image ? (int64_t)p.B : 1) * 4 * p.nh * SS;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_out;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t e = i % SS;
    const int h = (int)((i / SS) % p.nh);
    const int r = (int)((i / (SS * p.nh)) % 4);
    const int b0 = p.init_per_image ? (int)(i / (SS * p.nh * 4)) : 0;
    int slot = -1;
    for (int s = 0; s < p.n_sel; ++s)
      if (p.route_of_slot[s] == r) slot = s;
    float acc = 0.f;
    if (slot >= 0) {
      const int b_lo = p.init_per_image ? b0 : 0, b_hi = p.init_per_image ? b0 + 1 : p.B;
      for (int b = b_lo; b < b_hi; ++b) {
        const int64_t chain = ((int64_t)slot * p.B + b) * p.nh + h;
        acc += p.chain_ws[chain * p.chain_floats + dS_off + e];
      }
    }
    grad_init[i] = acc;
  }
}

}  // namespace

hipError_t launch_chain_backward(const BackParams& p, int d, float* grad_init, hipStream_t stream) {
  const int64_t blocks = (int64_t)p.n_sel * p.B * p.nh;
  dim3 grid((unsigned)blocks), block(back_threads(d));
  hipError_t err = hipSuccess;
  const int64_t SS = 4LL * d * d + 2LL * d;
  int64_t dS_off = p.nck * SS;  // where a chain's state adjoint sits in its workspace
  if (backward_wy_supported(p, d)) {
    err = launch_chain_backward_wy(p, stream);
  } else if (backward_wy32_supported(p, d)) {
    err = launch_chain_backward_wy32(p, stream);
    dS_off = 0;
  } else {
    switch (d) {
      case 16: chain_backward_kernel<16><<<grid, block, 0, stream>>>(p); break;
      case 64: chain_backward_kernel<64><<<grid, block, 0, stream>>>(p); break;
      default: return hipErrorInvalidValue;
    }
    err = hipGetLastError();
  }
  if (err != hipSuccess) return err;
  const int64_t n_out = (p.init_per_image ? (int64_t)p.B : 1) * 4 * p.nh * SS;
  const int64_t nb = std::min<int64_t>((n_out + 255) / 256, 65535);
  init_grad_kernel<<<dim3((unsigned)nb), dim3(256), 0, stream>>>(p, grad_init, SS, dS_off);
  return hipGetLastError();
}

}  // namespace hope
