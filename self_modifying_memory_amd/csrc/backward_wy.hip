// Backward pass of the four-direction scan at d = 64 with chunks of at most 16 tokens,
// gfx950: the chunk-parallel form, fp32 matrix cores (v_mfma_f32_16x16x4_f32, exact fp32
// products and fp32 sums), one (image, head, route) chain per workgroup of 8 waves.
//
// Forward, per chunk c of a chain ("VisionHOPE: Visual Backbones as Self-Modifying Learning
// Systems", Sec. 2.1.3 Eq. 15-16, Sec. 2.2 Eq. 19-20 with the App. B.3 safeguards, App. B.4
// Eq. 46): all six memories share the chunk's gain G_c, so the boundary state of chunk c is
// S_0 P_c with P_c = G_0 G_1 ... G_{c-1} (d x d) and the state S_0 (4d+2 rows) fixed.  The
// chunk's projections are S_0 (P_c x_t), its readout S_0[mem] (P_c q_t), and its gain, with
// A_t = alpha_t I - step_t k_t k_t^T, is
//   G_t = alpha_t G_{t-1} + u_t k_t^T,  u_t = -step_t w_t,  w_t = G_{t-1} k_t + delta_t,
//   G_{t-1} = Gam_{t-1} I + sum_{j<t} beta_{j,t-1} u_j k_j^T   (Gam prefix products of alpha,
//   beta_{j,t} = alpha_{j+1} ... alpha_t),
// so u_t follows from a C x C triangular recurrence over the Gram matrix K^T K, and
// P_{c+1} = Gam_C P_c + (P_c U) diag(beta_{., C-1}) K^T.
//
// Reverse (the memory trajectory is explicit and differentiable, Sec. 1), with dP the
// adjoint of P_{c+1} and D_e = P_c^T dP the adjoint of the chunk's end gain:
//   dG_t = Gam'_t D_e - sum_{m>t} beta_{t,m-1} step_m a_m k_m^T  (Gam'_t = alpha_{t+1} ...),
//   a_t = dG_t k_t = Gam'_t D_e k_t - sum_{m>t} beta_{t,m-1} step_m (k_m^T k_t) a_m,
//   dstep_t = -w_t^T a_t,  ddelta_t = -step_t a_t,  dalpha_t = <G_{t-1}, dG_t>,
//   dk_t = -step_t (G_{t-1}^T a_t + dG_t^T w_t),
// each expanded through the two low-rank forms into C x C Gram matrices (U^T A, A^T W,
// K^T A, (P U)^T (dP K)) and the vectors D_e k_t = P^T (dP k_t), D_e^T w_t = dP^T (P w_t);
// then the gates, the normalisation and the projections token by token, and
//   dP_c = Gam_C dP + (dP K) diag(beta_{., C-1}) U^T + sum_t (dx~_t x_t^T + dq~_t q_t^T),
//   dS_0 += sum_t [dy_t (P q_t)^T ; dp_t (P x_t)^T],  dx_t = P^T dx~_t,
// with dx~_t = S_0[proj]^T dp_t and dq~_t = S_0[mem]^T dy_t.  Where the step is not
// differentiable: min(eta_bar, eta_spec) follows eta_bar when eta_bar <= eta_spec; no
// derivative through the |k|^2 floor or the one-ulp rounding of eta_spec; eta_bar = 0
// (eta = 0 or eta_inj = 0) has derivative 0.
//
// A forward sweep writes P_c of every chunk to the workspace; the reverse sweep recomputes
// the chunk's projections and gates from it.  S_0 stays in registers for the whole chain:
// waves 0-3 hold column tile w of every row (for S_0^T products), waves 4-7 the rows of
// their projection row tiles (for S_0 products); the state adjoint dS_0 is accumulated in
// registers as 68 16 x 16 tiles spread over the 8 waves.  P_c, dP and the chunk's per-token
// vectors (token-major, 16 token slots, padding slots zero) live in LDS.
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace hope {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kD = 64;            // head dimension
constexpr int kTT = 16;           // token slots per chunk
constexpr int kLD = kD + 4;       // LDS row stride of d-vectors and d x d matrices
constexpr int kR = 4 * kD + 2;    // state rows: M_mem, M_k, M_v, M_q, m_eta, m_alpha
constexpr int kPL = 212;          // stride of a token's projection row (13 row tiles = 208)
constexpr int kCL = 17;           // stride of the C x C matrices
constexpr float kInjInward = 1.f - 1e-3f, kSpecInward = 1.f - 1e-6f, kKappaFloor = 1e-20f;

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

struct Lane {
  int lane, r16, q4;
};

// Sum over the wave, in every lane: DPP sums within the four 16-lane rows, then the four
// row totals read as scalars.
__device__ __forceinline__ float wave_total(float v) {
  v = row16_sum(v);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
  return (r0 + r1) + (r2 + r3);
}

// The thread index through an opaque copy: LDS addresses derived from it are recomputed in
// each stage instead of being hoisted out of the chunk loops and held for the whole kernel.
__device__ __forceinline__ int stage_lane(int tid) {
  asm volatile("" : "+v"(tid));
  return tid;
}
__device__ __forceinline__ Lane stage_lane_of(int tid) {
  const int t = stage_lane(tid);
  return Lane{t & 63, t & 15, (t & 63) >> 4};
}

// Rows 16m..16m+15 of M (or of M^T) times the 16 token vectors of In (token-major):
// Out[t][16m + i] = sum_k M(16m + i, k) In[t][k].  MFMA operands: in step s, lane (r16, q4)
// feeds A[r16][k] and B[k][t = r16] with k = 16 q4 + s, so that a lane's operands are 16
// consecutive floats (four 16-byte LDS reads; the transposed A is read column-wise), all
// loaded before the products; result D[4 q4 + v][r16].
__device__ __forceinline__ f32x4 dmat_tokens(const float* M, bool trans, const float* In, int m,
                                             const Lane& L) {
  float a[16], bv[16];
  if (trans) {
#pragma unroll
    for (int s = 0; s < 16; ++s) a[s] = M[(16 * L.q4 + s) * kLD + 16 * m + L.r16];
  } else {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(&M[(16 * m + L.r16) * kLD + 16 * L.q4 + 4 * g]);
#pragma unroll
      for (int e = 0; e < 4; ++e) a[4 * g + e] = v[e];
    }
  }
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(&In[L.r16 * kLD + 16 * L.q4 + 4 * g]);
#pragma unroll
    for (int e = 0; e < 4; ++e) bv[4 * g + e] = v[e];
  }
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 16; ++s) acc = mfma4(a[s], bv[s], acc);
  return acc;
}

__device__ __forceinline__ void store_tokens(float* Out, int m, f32x4 acc, const Lane& L) {
  *reinterpret_cast<f32x4*>(&Out[L.r16 * kLD + 16 * m + 4 * L.q4]) = acc;
}

// C x C Gram matrix Out[j][t] = A_j . B_t of two token-major arrays (same operand mapping).
__device__ __forceinline__ f32x4 gram_tokens(const float* A, const float* B, const Lane& L) {
  float a[16], bv[16];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const f32x4 va = *reinterpret_cast<const f32x4*>(&A[L.r16 * kLD + 16 * L.q4 + 4 * g]);
    const f32x4 vb = *reinterpret_cast<const f32x4*>(&B[L.r16 * kLD + 16 * L.q4 + 4 * g]);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      a[4 * g + e] = va[e];
      bv[4 * g + e] = vb[e];
    }
  }
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 16; ++s) acc = mfma4(a[s], bv[s], acc);
  return acc;
}

__device__ __forceinline__ void store_cc(float* Out, f32x4 acc, const Lane& L) {
#pragma unroll
  for (int v = 0; v < 4; ++v) Out[(4 * L.q4 + v) * kCL + L.r16] = acc[v];
}

// diagonal of a C x C result tile into Out[16]
__device__ __forceinline__ void store_diag(float* Out, f32x4 acc, const Lane& L) {
#pragma unroll
  for (int v = 0; v < 4; ++v)
    if (4 * L.q4 + v == L.r16) Out[L.r16] = acc[v];
}

// Per-chunk record in the workspace, written by the forward sweep and read back by the
// reverse sweep (floats): P_c (d x d), the token-major [16][d] arrays x~, k, delta, q, u, w,
// and eight per-token scalars (step, alpha, the two reciprocal norms, |k|^2, |delta|^2, s_eta,
// s_alpha).
constexpr int kRecTok = kTT * kD;
constexpr int kRec = kD * kD + 6 * kRecTok + 8 * kTT;

template <bool XBF>  // the map is bf16 (else fp32)
__global__ __launch_bounds__(512) void chain_backward_wy_kernel(BackParams p) {
  // One LDS block, small and uniformly read arrays first so that their addresses fit the
  // 16-bit immediate offset of the LDS instructions (one base register serves them all).
  constexpr int kTok = kTT * kLD;
  constexpr int oSc = 0;                      // per-token scalars, 16 x 16
  constexpr int oCC = oSc + 16 * kTT;         // C x C matrices, 6 x 16 x 17
  constexpr int oRow = oCC + 6 * kTT * kCL;   // solve coefficient columns, 16 x 16
  constexpr int oTok = oRow + kTT * kTT;      // token-major d-vectors, 18 of them
  constexpr int oProj = oTok + 18 * kTok;     // projections [16][kPL], then their adjoints
  constexpr int oP = oProj + kTT * kPL;       // P_c, dP, P_c^T
  constexpr int kSmem = oP + 3 * kD * kLD;
  __shared__ __align__(16) float smem[kSmem];
  // per-token scalars; the first eight in record order
  float* const tSt = smem + oSc;  // step_t
  float* const tAl = tSt + kTT;   // alpha_t
  float* const tNk = tAl + kTT;   // 1 / sqrt(|k_raw|^2 + eps)
  float* const tNq = tNk + kTT;   // 1 / sqrt(|q_raw|^2 + eps)
  float* const tKk = tNq + kTT;   // |k|^2
  float* const tDd = tKk + kTT;   // |delta|^2
  float* const tSe = tDd + kTT;   // s_eta
  float* const tSa = tSe + kTT;   // s_alpha
  float* const tGam = tSa + kTT;  // Gam_{t-1}
  float* const tGp = tGam + kTT;  // Gam'_t
  float* const tL = tGp + kTT;    // k_t . a_t
  float* const tUd = tL + kTT;    // u_t . D_e k_t
  float* const tDal = tUd + kTT;  // dalpha_t from the gain
  float* const tMisc = tDal + kTT;  // [0] Gam_C, [8..11] parts of <P, dP> = tr(D_e)
  int* const pixb = reinterpret_cast<int*>(tMisc + kTT);
  float* const sGm = smem + oCC;       // K^T K
  float* const sBt = sGm + kTT * kCL;  // beta[j][t]
  float* const sH = sBt + kTT * kCL;   // U^T A
  float* const sJ = sH + kTT * kCL;    // A^T W
  float* const sCm = sJ + kTT * kCL;   // c[t][m] = beta_{t,m-1} step_m for m > t
  float* const sCf = sCm + kTT * kCL;  // coefficient of k_j in dk_t
  // a solve's coefficient columns: [j][t] = beta_{j,t-1} (k_j . k_t) for t > j (u), or
  // [m][t] = -c[t][m] (k_m . k_t) for t < m (a)
  float* const sRow = smem + oRow;
  // token-major arrays; the first six in record order
  float* const sXt = smem + oTok;
  float* const sK = sXt + kTok;
  float* const sDl = sK + kTok;
  float* const sQ = sDl + kTok;
  float* const sU = sQ + kTok;
  float* const sW = sU + kTok;
  float* const sA = sW + kTok;
  float* const sZ = sA + kTok;
  float* const sE = sZ + kTok;
  float* const sF = sE + kTok;
  float* const sX = sF + kTok;
  float* const sDY = sX + kTok;
  float* const sQt = sDY + kTok;
  float* const sdQt = sQt + kTok;
  float* const sdQ = sdQt + kTok;
  float* const sPU = sdQ + kTok;
  float* const sdXt = sPU + kTok;
  float* const sY = sdXt + kTok;
  float* const sProj = smem + oProj;
  float* const sP = smem + oP;         // P_c
  float* const sdP = sP + kD * kLD;    // adjoint of P_{c+1}, then of P_c
  float* const sPT = sdP + kD * kLD;   // P_c^T (reverse sweep)

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
  const int nh = p.nh;
  const int h = blockIdx.x % nh;
  const int b = (blockIdx.x / nh) % p.B;
  const int slot = blockIdx.x / (nh * p.B);
  const int r = p.route_of_slot[slot];
  const int H = p.H, W = p.W, N = H * W, Dt = p.D;
  const int C = p.chunk > 0 ? p.chunk : (r < 2 ? W : H);
  const int nck = (N + C - 1) / C;
  const int64_t SS = (int64_t)kR * kD;
  float* const ckpt = p.chain_ws + (int64_t)blockIdx.x * p.chain_floats;
  float* const dSg = ckpt + p.nck * SS;
  float* const gdst = slot == 0 ? p.grad_x : p.planes + (int64_t)(slot - 1) * p.plane_stride;
  const GateParams gp{p.eta_map, p.eta_scale, p.alpha_bias, p.eps, 0, 0};
  const float* init = p.init + (p.init_per_image ? ((int64_t)b * 4 + r) * nh + h : (int64_t)r * nh + h) * SS;

  // S_0 in registers.  Waves 0-3 (column tile w): s0f[4T + s] = S_0[16T + 4q4 + s][16w + r16]
  // for the 17 row tiles T.  Waves 4-7: row tiles 4 + j + 4 slot (slot 0-2) and, on wave 4,
  // tile 16: s0f[16 slot + s] = S_0[16T + r16][16q4 + s].  (k = 16 q4 + s, or 4 q4 + s within
  // a row tile, as in the products below.)
  float s0f[68];
  {
    const Lane L = stage_lane_of(tid);
    if (w < 4) {
#pragma unroll
      for (int e = 0; e < 68; ++e) {
        const int row = 16 * (e >> 2) + 4 * L.q4 + (e & 3);
        s0f[e] = row < kR ? init[(int64_t)row * kD + 16 * w + L.r16] : 0.f;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 64; ++e) {
        const int sl = e >> 4, s = e & 15;
        const int T = sl < 3 ? 4 + (w - 4) + 4 * sl : 16;
        const int row = 16 * T + L.r16;
        s0f[e] = ((sl < 3 || w == 4) && row < kR) ? init[(int64_t)row * kD + 16 * L.q4 + s] : 0.f;
      }
#pragma unroll
      for (int e = 64; e < 68; ++e) s0f[e] = 0.f;
    }
  }
  f32x4 dsa[9];  // dS_0 tiles o = w + 8 i: rows 16 (o >> 2) .., columns 16 (o & 3) ..
#pragma unroll
  for (int i = 0; i < 9; ++i) dsa[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  // identity P_0, zero dP
  for (int e = tid; e < kD * kD; e += 512) {
    const int i = e >> 6, j = e & 63;
    sP[i * kLD + j] = i == j ? 1.f : 0.f;
    sdP[i * kLD + j] = 0.f;
  }

  // Inputs of a chunk, fetched into registers one chunk ahead and written to LDS when the
  // chunk starts.  The loads are unconditional (padding slots read the chunk's last token
  // and are zeroed when written to LDS), so nothing waits for them before then.
  uint32_t fx[2];  // raw bits of x (bf16 in the low half, or fp32)
  float fdy[2], fP[8], fT[12], fS;
  auto fetch = [&](int c, bool rev) {
    const int t0 = stage_lane(tid), s0 = c * C, cl = min(C, N - s0);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int e = t0 + 512 * k, t = min(e >> 6, cl - 1), i = e & 63;
      const int pix = route_pixel(r, s0 + t, H, W, N);
      const int64_t idx = ((int64_t)b * N + pix) * Dt + (int64_t)h * kD + i;
      if (XBF) fx[k] = static_cast<const uint16_t*>(p.x)[idx];
      else fx[k] = __float_as_uint(static_cast<const float*>(p.x)[idx]);
      if (rev) fdy[k] = p.grad_out[idx];
    }
    if (rev) {
      const float* rec = ckpt + (int64_t)c * kRec;
#pragma unroll
      for (int k = 0; k < 8; ++k) fP[k] = rec[t0 + 512 * k];
#pragma unroll
      for (int k = 0; k < 12; ++k) fT[k] = rec[kD * kD + t0 + 512 * k];
      fS = rec[kD * kD + 6 * kRecTok + (t0 & 127)];
    }
  };
  auto commit = [&](int c, bool rev) {
    const int t0 = stage_lane(tid), s0 = c * C, cl = min(C, N - s0);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int e = t0 + 512 * k, t = e >> 6, i = e & 63;
      const float xv = XBF ? __uint_as_float(fx[k] << 16) : __uint_as_float(fx[k]);
      sX[t * kLD + i] = t < cl ? xv : 0.f;
      if (rev) sDY[t * kLD + i] = t < cl ? fdy[k] : 0.f;
    }
    if (rev) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int e = t0 + 512 * k;
        sP[(e >> 6) * kLD + (e & 63)] = fP[k];
        sPT[(e & 63) * kLD + (e >> 6)] = fP[k];
      }
#pragma unroll
      for (int k = 0; k < 12; ++k) {
        const int e = t0 + 512 * k, a = e >> 10, t = (e >> 6) & 15, i = e & 63;
        sXt[a * kTok + t * kLD + i] = fT[k];
      }
      if (t0 < 8 * kTT) tSt[t0] = fS;
    }
    if (t0 < kTT) pixb[t0] = t0 < cl ? route_pixel(r, s0 + t0, H, W, N) : 0;
  };
  // the forward sweep's record of chunk c: P_c, or the token arrays and scalars
  auto store_P = [&](int c) {
    const int t0 = stage_lane(tid);
    float* rec = ckpt + (int64_t)c * kRec;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int e = t0 + 512 * k;
      rec[e] = sP[(e >> 6) * kLD + (e & 63)];
    }
  };
  auto store_tokens_rec = [&](int c) {
    const int t0 = stage_lane(tid);
    float* rec = ckpt + (int64_t)c * kRec;
#pragma unroll
    for (int k = 0; k < 12; ++k) {
      const int e = t0 + 512 * k, a = e >> 10, t = (e >> 6) & 15, i = e & 63;
      rec[kD * kD + e] = sXt[a * kTok + t * kLD + i];
    }
    if (t0 < 8 * kTT) rec[kD * kD + 6 * kRecTok + t0] = tSt[t0];
  };
  // projections of the chunk: waves 4-7, Proj[t][pr] = S_0[64 + pr] . x~_t
  auto projections = [&]() {
    const Lane L = stage_lane_of(tid);
#pragma unroll
    for (int sl = 0; sl < 4; ++sl) {
      const int T = sl < 3 ? 4 + (w - 4) + 4 * sl : 16;
      if (sl < 3 || w == 4) {
        float bv[16];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(&sXt[L.r16 * kLD + 16 * L.q4 + 4 * g]);
#pragma unroll
          for (int e = 0; e < 4; ++e) bv[4 * g + e] = v[e];
        }
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 16; ++s) acc = mfma4(s0f[16 * sl + s], bv[s], acc);
        *reinterpret_cast<f32x4*>(&sProj[L.r16 * kPL + 16 * T - 64 + 4 * L.q4]) = acc;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // the stabilised normalisation of k and q (App. C.1), delta = k - v and the step of every
  // token slot (wave per token), with the norms and gate inputs the backward reuses
  auto gates = [&](int cl) {
    const int lane = stage_lane(tid) & 63;
    float kr[2], vr[2], qr[2], se[2], sa[2], nk[2], nq[2], k[2], q[2], dl[2], kk[2], dd[2], al[2], st[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const float* pt = &sProj[(w + 8 * u) * kPL];
      kr[u] = pt[lane];
      vr[u] = pt[kD + lane];
      qr[u] = pt[2 * kD + lane];
      se[u] = pt[3 * kD];
      sa[u] = pt[3 * kD + 1];
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      nk[u] = fast_rsqrt(wave_total(kr[u] * kr[u]) + gp.eps);
      nq[u] = fast_rsqrt(wave_total(qr[u] * qr[u]) + gp.eps);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      k[u] = kr[u] * nk[u];
      q[u] = qr[u] * nq[u];
      dl[u] = k[u] - vr[u];
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      kk[u] = wave_total(k[u] * k[u]);
      dd[u] = wave_total(dl[u] * dl[u]);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) st[u] = executed_step(kk[u], dd[u], se[u], sa[u], gp, &al[u]);
    // padding slots (t >= cl): zero vectors, step 0, alpha 1, unit norms
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int t = w + 8 * u;
      const bool on = t < cl;
      sK[t * kLD + lane] = on ? k[u] : 0.f;
      sDl[t * kLD + lane] = on ? dl[u] : 0.f;
      sQ[t * kLD + lane] = on ? q[u] : 0.f;
      if (lane == 0) {
        tSt[t] = on ? st[u] : 0.f;
        tAl[t] = on ? al[u] : 1.f;
        tNk[t] = on ? nk[u] : 1.f;
        tNq[t] = on ? nq[u] : 1.f;
        tKk[t] = on ? kk[u] : 0.f;
        tDd[t] = on ? dd[u] : 0.f;
        tSe[t] = on ? se[u] : 0.f;
        tSa[t] = on ? sa[u] : 0.f;
      }
    }
  };
  // products of alpha over token ranges (lanes of waves 4-7, one (j, t) pair each):
  // Bt[j][t] = alpha_{j+1} .. alpha_t (j <= t, else 0), Gam_{t-1}, Gam'_t, Gam_C
  auto alpha_products = [&]() {
    const int e = stage_lane(tid) - 256, t = e >> 4, j = e & 15;
    float al[kTT];
#pragma unroll
    for (int i = 0; i < kTT; ++i) al[i] = tAl[i];
    float bt = 1.f, gm = 1.f, gq = 1.f, gc = 1.f;
#pragma unroll
    for (int i = 0; i < kTT; ++i) {
      bt *= (i > j && i <= t) ? al[i] : 1.f;
      gm *= i < t ? al[i] : 1.f;
      gq *= i > t ? al[i] : 1.f;
      gc *= al[i];
    }
    sBt[j * kCL + t] = j <= t ? bt : 0.f;
    if (j == 0) tGam[t] = gm;
    else if (j == 1) tGp[t] = gq;
    else if (j == 2 && t == 0) tMisc[0] = gc;
  };
  // A one-wave triangular recurrence over the 16 token slots, lane = component,
  // right-looking: slot t starts from base_t = g0_t B0_t (+ B1_t), and once v_j is final
  // every later slot t (t > j forward, t < j backward) adds sCol[j][t] v_j, so one FMA per
  // step is on the critical path; the coefficient columns are loaded two steps ahead.
  // kU: the u-recurrence (forward, with the B1 term, v = -gscale * pre to Out and pre to
  // Out2); else the a-recurrence (backward, v = pre to Out).  (Which operands are present is
  // a template argument: a test of a pointer into LDS against null is not folded by the
  // compiler, and the branches it leaves serialise the steps' LDS reads.)
  auto solve_cols = [&](auto kU_tag, int cl, const float* g0, const float* B0, const float* B1,
                        float* Out, float* Out2, const float* gscale) {
    constexpr bool kU = decltype(kU_tag)::value;
    constexpr bool kBack = !kU;
    const int lane = stage_lane(tid) & 63;
    float acc[kTT], gs[kTT];
#pragma unroll
    for (int t = 0; t < kTT; ++t) {
      const float b0 = B0[t * kLD + lane];
      if constexpr (kU) {
        acc[t] = fmaf(g0[t], b0, B1[t * kLD + lane]);
        gs[t] = gscale[t];
      } else {
        acc[t] = g0[t] * b0;
      }
    }
    f32x4 col[3][4];
    auto load_col = [&](int n) {
      const int j = kBack ? kTT - 1 - n : n;
#pragma unroll
      for (int q = 0; q < 4; ++q) col[n % 3][q] = *reinterpret_cast<const f32x4*>(&sRow[j * kTT + 4 * q]);
    };
    load_col(0);
    load_col(1);
#pragma unroll
    for (int n = 0; n < kTT; ++n) {
      const int j = kBack ? kTT - 1 - n : n;
      if (n + 2 < kTT) load_col(n + 2);
      const float pre = j < cl ? acc[j] : 0.f;
      const float val = kU ? -gs[j] * pre : pre;
      Out[j * kLD + lane] = val;
      if constexpr (kU) Out2[j * kLD + lane] = pre;
#pragma unroll
      for (int t = 0; t < kTT; ++t)
        if (kBack ? t < j : t > j) acc[t] = fmaf(col[n % 3][t >> 2][t & 3], val, acc[t]);
    }
  };
  // tile idx (0-15) of a d x d matrix in LDS: M <- gc M + sum over the 16 token slots of
  // (A1_t, scaled by beta_{t,cl-1} if kScale) B1_t^T [+ A2_t B2_t^T if kTwo]
  auto dd_update = [&](auto kScale_tag, auto kTwo_tag, float* M, int idx, float gc, const float* A1,
                       const float* B1, int cl, const float* A2, const float* B2) {
    constexpr bool kScale = decltype(kScale_tag)::value, kTwo = decltype(kTwo_tag)::value;
    const Lane L = stage_lane_of(tid);
    const int r16 = L.r16, q4 = L.q4, mi = idx >> 2, nj = idx & 3;
    f32x4 acc;
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[v] = gc * M[(16 * mi + 4 * q4 + v) * kLD + 16 * nj + r16];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int tk = 4 * s + q4;
      const float a = A1[tk * kLD + 16 * mi + r16];
      acc = mfma4(kScale ? a * sBt[tk * kCL + cl - 1] : a, B1[tk * kLD + 16 * nj + r16], acc);
      if constexpr (kTwo) acc = mfma4(A2[tk * kLD + 16 * mi + r16], B2[tk * kLD + 16 * nj + r16], acc);
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) M[(16 * mi + 4 * q4 + v) * kLD + 16 * nj + r16] = acc[v];
  };
  auto dtok = [&](float* Out, const float* M, bool trans, const float* In, int m) {
    const Lane L = stage_lane_of(tid);
    store_tokens(Out, m, dmat_tokens(M, trans, In, m, L), L);
  };
  auto gram = [&](float* Out, const float* A, const float* B) {
    const Lane L = stage_lane_of(tid);
    store_cc(Out, gram_tokens(A, B, L), L);
  };
  auto gram_diag = [&](float* Out, const float* A, const float* B) {
    const Lane L = stage_lane_of(tid);
    store_diag(Out, gram_tokens(A, B, L), L);
  };

  // dS_0[M_mem rows] += dy q~^T for this wave's two M_mem tiles (i = 0, 1)
  auto mem_rows_dS0 = [&]() {
    const Lane L = stage_lane_of(tid);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int o = w + 8 * i, RT = o >> 2, n = o & 3;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int tk = 4 * s + L.q4;
        dsa[i] = mfma4(sDY[tk * kLD + 16 * RT + L.r16], sQt[tk * kLD + 16 * n + L.r16], dsa[i]);
      }
    }
  };

  fetch(0, false);
  __syncthreads();

  // ---- forward sweep: the record of every chunk into the workspace --------------------
  // (barriers order LDS only; global loads stay in flight across them, and the stores are
  // issued after each chunk's prefetch so that waiting for the prefetch skips them)
  for (int c = 0; c < nck; ++c) {
    const int s0 = c * C, cl = min(C, N - s0);
    commit(c, false);
    fetch(min(c + 1, nck - 1), false);  // (the last fetch is not used)
    store_P(c);
    if (c > 0) store_tokens_rec(c - 1);
    lds_barrier();
    if (w < 4) dtok(sXt, sP, false, sX, w);
    lds_barrier();
    if (w >= 4) projections();
    lds_barrier();
    gates(cl);
    lds_barrier();
    if (w == 0) gram(sGm, sK, sK);
    if (w >= 4) alpha_products();
    lds_barrier();
    if (w == 0) {
      // coefficient columns beta_{j,t-1} (k_j . k_t), t > j, then the recurrence for w and u
      const int lane = stage_lane(tid) & 63;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int e = lane + 64 * k, t = e >> 4, j = e & 15;
        sRow[j * kTT + t] = j < t ? sBt[j * kCL + t - 1] * sGm[j * kCL + t] : 0.f;
      }
      solve_cols(std::true_type{}, cl, tGam, sK, sDl, sU, sW, tSt);
    }
    lds_barrier();
    if (c == nck - 1) break;
    if (w < 4) dtok(sPU, sP, false, sU, w);
    lds_barrier();
    // P <- Gam_C P + (P U) diag(beta_{., cl-1}) K^T
    {
      const float gc = tMisc[0];
      dd_update(std::true_type{}, std::false_type{}, sP, w, gc, sPU, sK, cl, nullptr, nullptr);
      dd_update(std::true_type{}, std::false_type{}, sP, w + 8, gc, sPU, sK, cl, nullptr, nullptr);
      (void)s0;
    }
    lds_barrier();
  }
  store_tokens_rec(nck - 1);

  // ---- reverse sweep ---------------------------------------------------------------------
  __syncthreads();  // the records written above are visible to every thread
  fetch(nck - 1, true);
  // dx of a chunk is stored after the next chunk's prefetch is issued (same reason)
  f32x4 dxv = {0.f, 0.f, 0.f, 0.f};
  float* dxdst = gdst;
  bool dxok = false;
  for (int c = nck - 1; c >= 0; --c) {
    const int cl = min(C, N - c * C);
    lds_barrier();
    commit(c, true);
    fetch(max(c - 1, 0), true);  // (the last fetch is not used)
    if (dxok) *reinterpret_cast<f32x4*>(dxdst) = dxv;
    lds_barrier();
    // dq~ = S_0[mem]^T dy and parts of <P, dP> (waves 0-3); Z = dP K, Y = P W (waves 4-7);
    // K^T K (wave 4); beta (waves 4-7)
    if (w < 4) {
      const Lane L = stage_lane_of(tid);
      f32x4 dy4[4];
#pragma unroll
      for (int T = 0; T < 4; ++T) dy4[T] = *reinterpret_cast<const f32x4*>(&sDY[L.r16 * kLD + 16 * T + 4 * L.q4]);
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int T = 0; T < 4; ++T)
#pragma unroll
        for (int s = 0; s < 4; ++s) acc = mfma4(s0f[4 * T + s], dy4[T][s], acc);
      store_tokens(sdQt, w, acc, L);
      float tr = 0.f;
#pragma unroll 4
      for (int k = 0; k < 16; ++k) {
        const int e = 64 * w + L.lane + 256 * k, o = (e >> 6) * kLD + (e & 63);
        tr = fmaf(sP[o], sdP[o], tr);
      }
      tr = wave_total(tr);
      if (L.lane == 0) tMisc[8 + w] = tr;
    } else {
      dtok(sZ, sdP, false, sK, w - 4);
      dtok(sY, sP, false, sW, w - 4);
      if (w == 4) gram(sGm, sK, sK);
      alpha_products();
    }
    lds_barrier();
    // E = P^T Z = D_e K, F = dP^T Y = D_e^T W, q~ = P q, dq = P^T dq~; c and the a-solve rows
    for (int jb = w; jb < 16; jb += 8) {
      const int kind = jb >> 2, m = jb & 3;
      if (kind == 0) dtok(sE, sPT, false, sZ, m);
      else if (kind == 1) dtok(sF, sdP, true, sY, m);
      else if (kind == 2) dtok(sQt, sP, false, sQ, m);
      else dtok(sdQ, sPT, false, sdQt, m);
    }
    if (w >= 4) {
      const int e = stage_lane(tid) - 256, t = e >> 4, m = e & 15;
      const float cm = m > t ? sBt[t * kCL + m - 1] * tSt[m] : 0.f;
      sCm[t * kCL + m] = cm;
      sRow[m * kTT + t] = -cm * sGm[m * kCL + t];
    }
    lds_barrier();
    // a (wave 0); the adjoint carry's first part on waves 1-7:
    // dP <- Gam_C dP + (dP K) diag(beta_{., cl-1}) U^T + dq~ q^T
    if (w == 0) {
      solve_cols(std::false_type{}, cl, tGp, sE, nullptr, sA, nullptr, nullptr);
    } else {
      const float gc = tMisc[0];
      for (int idx = w - 1; idx < 16; idx += 7)
        dd_update(std::true_type{}, std::true_type{}, sdP, idx, gc, sZ, sU, cl, sdQt, sQ);
      mem_rows_dS0();
    }
    lds_barrier();
    // H = U^T A, J = A^T W, diag(K^T A), diag(U^T E)
    if (w == 4) gram(sH, sU, sA);
    else if (w == 5) gram(sJ, sA, sW);
    else if (w == 6) gram_diag(tL, sK, sA);
    else if (w == 7) gram_diag(tUd, sU, sE);
    lds_barrier();
    // dalpha_t from the gain (wave 0, through the C x C product inner = (H o K^T K) c^T);
    // the coefficients of k_j in dk_t (waves 1-4)
    if (w == 0) {
      const Lane L = stage_lane_of(tid);
      const int r16 = L.r16, q4 = L.q4;
      f32x4 inner = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int m = 4 * s + q4;
        inner = mfma4(sH[r16 * kCL + m] * sGm[r16 * kCL + m], sCm[r16 * kCL + m], inner);
      }
      // inner[j = 4 q4 + v][t = r16]
      const int t = r16;
      const float gp1 = tGp[t];
      float part = 0.f;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int j = 4 * q4 + v;
        if (j < t) part = fmaf(sBt[j * kCL + t - 1], gp1 * tUd[j] - inner[v], part);
      }
      part += __shfl_xor(part, 16, 64);
      part += __shfl_xor(part, 32, 64);
      if (q4 == 0) {
        float lsum = 0.f;
#pragma unroll
        for (int m = 0; m < kTT; ++m) lsum = fmaf(sCm[t * kCL + m], tL[m], lsum);
        const float trd = (tMisc[8] + tMisc[9]) + (tMisc[10] + tMisc[11]);
        tDal[t] = part + tGam[t] * (gp1 * trd - lsum);
      }
    } else if (w <= 4) {
      const int e = stage_lane(tid) - 64, t = e >> 4, j = e & 15;
      float cf = 0.f;
      if (j < t) cf = sBt[j * kCL + t - 1] * sH[j * kCL + t];
      else if (j > t) cf = -sCm[t * kCL + j] * sJ[j * kCL + t];
      sCf[j * kCL + t] = cf;
    }
    lds_barrier();
    // token by token: the gain adjoints, then the readout, the step, the gates, the
    // normalisation and the projections; dProj replaces Proj (zero rows in padding slots)
    {
      const int lane = stage_lane(tid) & 63;
      float dk[2], ddl[2], dstep[2], dalpha[2], dq[2], k[2], q[2], dl[2];
      float eta[2], deta_dse[2], alpha[2], oma[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int t = w + 8 * u;
        const float st = tSt[t];
        const float at = sA[t * kLD + lane];
        float gk = fmaf(tGam[t], at, tGp[t] * sF[t * kLD + lane]);
#pragma unroll
        for (int j = 0; j < kTT; ++j) gk = fmaf(sCf[j * kCL + t], sK[j * kLD + lane], gk);
        dk[u] = -st * gk;
        ddl[u] = -st * at;
        dstep[u] = -sJ[t * kCL + t];
        dalpha[u] = tDal[t];
        dq[u] = sdQ[t * kLD + lane];
        k[u] = sK[t * kLD + lane];
        q[u] = sQ[t * kLD + lane];
        dl[u] = sDl[t * kLD + lane];
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        // forward values, as in the gates and executed_step
        const int t = w + 8 * u;
        const float kk = tKk[t], dd = tDd[t], se = tSe[t], sa = tSa[t];
        if (gp.eta_map == 0) {
          const float sg = fast_rcp(1.f + fast_exp(-se));
          eta[u] = gp.eta_scale * sg;
          deta_dse[u] = gp.eta_scale * sg * (1.f - sg);
        } else {
          eta[u] = gp.eta_scale * (fmaxf(se, 0.f) + log1pf(fast_exp(-fabsf(se))));
          deta_dse[u] = gp.eta_scale * fast_rcp(1.f + fast_exp(-se));
        }
        const float ez = fast_exp(-(sa + gp.alpha_bias));
        alpha[u] = fast_rcp(1.f + ez);
        oma[u] = ez * alpha[u];  // 1 - alpha
        const float rr0 = fast_sqrt(dd + gp.eps * gp.eps);
        const float rr = rr0 + gp.eps;
        const float inj = kInjInward * oma[u] * fast_rcp(rr);
        const bool ok = eta[u] != 0.f && inj != 0.f;
        const float xr = ok ? eta[u] * fast_rcp(inj) : 0.f;
        const float ex = fast_exp(-xr);
        const float bar = ok ? inj * one_minus_exp_neg(xr) : 0.f;
        const float kap = fmaxf(kk, kKappaFloor);
        const float spec_raw = kSpecInward * 2.f * alpha[u] * fast_rcp(kap);
        const float spec = spec_raw > 0.f ? __uint_as_float(__float_as_uint(spec_raw) - 1u) : spec_raw;
        // step = min(eta_bar, eta_spec)
        float deta = 0.f, ddd = 0.f, dkk = 0.f;
        if (bar <= spec) {
          if (ok) {
            deta = dstep[u] * ex;
            const float dinj = dstep[u] * ((1.f - ex) - xr * ex);
            dalpha[u] -= dinj * kInjInward * fast_rcp(rr);
            const float drr = -dinj * inj * fast_rcp(rr);
            ddd = drr * 0.5f * fast_rcp(rr0);
          }
        } else {
          dalpha[u] += dstep[u] * kSpecInward * 2.f * fast_rcp(kap);
          if (kk > kKappaFloor) dkk = -dstep[u] * spec_raw * fast_rcp(kap);
        }
        ddl[u] = fmaf(2.f * dl[u], ddd, ddl[u]);
        dk[u] = fmaf(2.f * k[u], dkk, dk[u]);
        dk[u] += ddl[u];  // delta = k - v
        deta_dse[u] *= deta;
      }
      float kdk[2], qdq[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        kdk[u] = wave_total(k[u] * dk[u]);
        qdq[u] = wave_total(q[u] * dq[u]);
      }
      // dProj rows; zero in padding slots
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int t = w + 8 * u;
        const bool on = t < cl;
        float* pt = &sProj[t * kPL];
        pt[lane] = on ? (dk[u] - k[u] * kdk[u]) * tNk[t] : 0.f;
        pt[kD + lane] = on ? -ddl[u] : 0.f;
        pt[2 * kD + lane] = on ? (dq[u] - q[u] * qdq[u]) * tNq[t] : 0.f;
        if (lane < 16) {
          const float g = lane == 0 ? deta_dse[u] : (lane == 1 ? dalpha[u] * alpha[u] * oma[u] : 0.f);
          pt[3 * kD + lane] = on ? g : 0.f;
        }
      }
    }
    lds_barrier();
    // dx~ = S_0[proj]^T dProj (waves 0-3); dS_0 += [dy q~^T ; dProj x~^T] (all waves)
    {
      const Lane L = stage_lane_of(tid);
      const int r16 = L.r16, q4 = L.q4;
      if (w < 4) {
        f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int T0 = 4; T0 < 17; T0 += 5) {
          f32x4 pv[5];
#pragma unroll
          for (int T = T0; T < T0 + 5 && T < 17; ++T)
            pv[T - T0] = *reinterpret_cast<const f32x4*>(&sProj[r16 * kPL + 16 * T - 64 + 4 * q4]);
#pragma unroll
          for (int T = T0; T < T0 + 5 && T < 17; ++T)
#pragma unroll
            for (int s = 0; s < 4; ++s) {
              if (s & 1) acc1 = mfma4(s0f[4 * T + s], pv[T - T0][s], acc1);
              else acc0 = mfma4(s0f[4 * T + s], pv[T - T0][s], acc0);
            }
          __builtin_amdgcn_sched_barrier(0);  // bounded operand prefetch
        }
        store_tokens(sdXt, w, acc0 + acc1, L);
      }
#pragma unroll
      for (int i = 0; i < 9; ++i) {
        const int o = w + 8 * i;
        if (o < 68 && (i >= 2 || w == 0)) {
          const int RT = o >> 2, n = o & 3;
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const int tk = 4 * s + q4;
            const float av = RT < 4 ? sDY[tk * kLD + 16 * RT + r16] : sProj[tk * kPL + 16 * RT - 64 + r16];
            const float bv = RT < 4 ? sQt[tk * kLD + 16 * n + r16] : sXt[tk * kLD + 16 * n + r16];
            dsa[i] = mfma4(av, bv, dsa[i]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    lds_barrier();
    // dx = P^T dx~ (waves 0-3, stored next chunk); the adjoint carry's last part
    // dP <- dP + dx~ x^T
    if (w < 4) {
      const Lane L = stage_lane_of(tid);
      dxv = dmat_tokens(sPT, false, sdXt, w, L);
      dxok = L.r16 < cl;
      dxdst = gdst + ((int64_t)b * N + pixb[L.r16]) * Dt + (int64_t)h * kD + 16 * w + 4 * L.q4;
    }
    dd_update(std::false_type{}, std::false_type{}, sdP, w, 1.f, sdXt, sX, cl, nullptr, nullptr);
    dd_update(std::false_type{}, std::false_type{}, sdP, w + 8, 1.f, sdXt, sX, cl, nullptr, nullptr);
  }
  if (dxok) *reinterpret_cast<f32x4*>(dxdst) = dxv;

  // the initial-state adjoint of this chain, for the gradient reduction
  {
    const Lane L = stage_lane_of(tid);
#pragma unroll
    for (int i = 0; i < 9; ++i) {
      const int o = w + 8 * i;
      if (o < 68) {
        const int RT = o >> 2, n = o & 3;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int row = 16 * RT + 4 * L.q4 + v;
          if (row < kR) dSg[(int64_t)row * kD + 16 * n + L.r16] = dsa[i][v];
        }
      }
    }
  }
}

}  // namespace

bool backward_wy_supported(const BackParams& p, int d) {
  if (d != kD) return false;
  for (int s = 0; s < p.n_sel; ++s) {
    const int r = p.route_of_slot[s];
    const int C = p.chunk > 0 ? p.chunk : (r < 2 ? p.W : p.H);
    if (C > kTT) return false;
  }
  return true;
}

hipError_t launch_chain_backward_wy(const BackParams& p, hipStream_t stream) {
  const int64_t blocks = (int64_t)p.n_sel * p.B * p.nh;
  if (p.x_bf16) chain_backward_wy_kernel<true><<<dim3((unsigned)blocks), dim3(512), 0, stream>>>(p);
  else chain_backward_wy_kernel<false><<<dim3((unsigned)blocks), dim3(512), 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace hope
