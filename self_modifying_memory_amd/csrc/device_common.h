// Device helpers shared by the chain kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hope {

// Flat pixel visited at step t of route r ("VMamba: Visual State Space Model",
// the four scan orders; VisionHOPE Sec. 2.3 Eq. 24).
__device__ __forceinline__ int route_pixel(int r, int t, int H, int W, int N) {
  if (r & 1) t = N - 1 - t;          // routes 1 and 3 are full reversals
  if (r < 2) return t;               // row-major
  return (t % H) * W + (t / H);      // column-major: flatten of the spatial transpose
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

struct GateParams {
  int eta_map;   // 0 sigmoid, 1 softplus
  float eta_scale, alpha_bias, eps;
  int injection;  // 0 soft cap (Eq. 19), 1 hard clamp at the same limit, 2 none
  int spectral;   // 0 clamp (Eq. 20), 1 smooth map to the same limit, 2 none
};

// Which step-control limits bind for one token: bit 0 the raw eta exceeds the injection
// limit, bit 1 eta_bar exceeds the spectral limit.
struct StepFlags {
  int bits;
};

struct TokenGates {
  float k, q, delta;  // this lane's component (0 for lanes >= d)
  float alpha, step;  // per token (same in every lane)
  int flags;          // StepFlags bits (same in every lane)
};

// Executed step from the token's norms ("VisionHOPE: Visual Backbones as Self-Modifying
// Learning Systems", Sec. 2.2 Definition 1, Eq. 19-20 with the App. B.3 safeguards):
//   r = sqrt(|delta|^2 + eps^2) + eps,  eta_inj = (1 - 1e-3)(1 - alpha) / r,
//   eta_bar = eta_inj (1 - exp(-eta / eta_inj)),
//   eta_spec = (1 - 1e-6) 2 alpha / max(|k|^2, 1e-20), one ulp toward zero,
//   step = min(eta_bar, eta_spec);
// gate maps of App. C.1 Eq. 53 (eta_scale * sigmoid or softplus; alpha = sigmoid(s + bias)).
// 1 - alpha is evaluated as e^-z sigmoid(z) = sigmoid(-z) to keep its relative accuracy
// near alpha = 1.
// Reciprocals, square roots and exponentials use the hardware approximations (about
// 1 ulp; with eps > 0 no argument here is denormal).
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float fast_exp(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }
__device__ __forceinline__ float fast_sqrt(float x) { return __builtin_amdgcn_sqrtf(x); }
__device__ __forceinline__ float fast_rsqrt(float x) { return __builtin_amdgcn_rsqf(x); }

// 1 - e^-x for x >= 0 to a few ulp: below 1/4, where 1 - e^-x would cancel, the Taylor
// series through x^7 (truncation below 2e-9 relative); above, the hardware exponential
// (the subtraction then loses at most two bits).
__device__ __forceinline__ float one_minus_exp_neg(float x) {
  float p = fmaf(x, 1.f / 5040.f, -1.f / 720.f);
  p = fmaf(x, p, 1.f / 120.f);
  p = fmaf(x, p, -1.f / 24.f);
  p = fmaf(x, p, 1.f / 6.f);
  p = fmaf(x, p, -0.5f);
  p = fmaf(x, p, 1.f);
  const float series = x * p;
  return x < 0.25f ? series : 1.f - fast_exp(-x);
}

// Retention alpha = sigmoid(s_alpha + bias) (App. C.1 Eq. 53), with e^-z for 1 - alpha; the
// chain kernels that need alpha outside the gate phase call this same function, so both
// uses agree bit for bit.
__device__ __forceinline__ float gate_alpha(float s_alpha, const GateParams& g, float* ez_out) {
  const float z = s_alpha + g.alpha_bias;
  const float ez = fast_exp(-z);
  *ez_out = ez;
  return fast_rcp(1.f + ez);
}

// Variants ("VisionHOPE", Sec. 3.5 ablations): a hard clamp min(eta, eta_inj) or no
// injection control; the smooth spectral map eta_spec (1 - exp(-eta_bar / eta_spec)) or no
// spectral control.
__device__ __forceinline__ float executed_step(float kk, float dd, float s_eta, float s_alpha,
                                               const GateParams& g, float* alpha_out,
                                               StepFlags* flags = nullptr) {
  float eta;
  if (g.eta_map == 0) {
    eta = g.eta_scale * fast_rcp(1.f + fast_exp(-s_eta));
  } else {
    eta = g.eta_scale * (fmaxf(s_eta, 0.f) + log1pf(fast_exp(-fabsf(s_eta))));
  }
  float ez;
  const float alpha = gate_alpha(s_alpha, g, &ez);
  const float one_minus_alpha = ez * alpha;  // sigmoid(-z), accurate near alpha = 1
  const float rr = fast_sqrt(dd + g.eps * g.eps) + g.eps;
  const float inj = (1.f - 1e-3f) * one_minus_alpha * fast_rcp(rr);
  float bar;
  if (g.injection == 0) {
    bar = (eta == 0.f || inj == 0.f) ? 0.f : inj * one_minus_exp_neg(eta * fast_rcp(inj));
  } else {
    bar = g.injection == 1 ? fminf(eta, inj) : eta;
  }
  float spec = (1.f - 1e-6f) * 2.f * alpha * fast_rcp(fmaxf(kk, 1e-20f));
  if (spec > 0.f) spec = __uint_as_float(__float_as_uint(spec) - 1u);  // one ulp toward 0
  *alpha_out = alpha;
  if (flags) flags->bits = (eta > inj ? 1 : 0) | (bar > spec ? 2 : 0);
  if (g.spectral == 0) return fminf(bar, spec);
  if (g.spectral == 2) return bar;
  return (bar == 0.f || spec == 0.f) ? 0.f : spec * one_minus_exp_neg(bar * fast_rcp(spec));
}

// One token on one wave, lane i holding component i of the raw projections: the
// stabilised normalisation of k (App. C.1; q the same way), delta = k - v, and the step.
__device__ __forceinline__ TokenGates token_gates(float kr, float vr, float qr, float s_eta,
                                                  float s_alpha, const GateParams& g) {
  TokenGates o;
  o.k = kr / sqrtf(wave_sum(kr * kr) + g.eps);
  o.q = qr / sqrtf(wave_sum(qr * qr) + g.eps);
  o.delta = o.k - vr;
  const float dd = wave_sum(o.delta * o.delta);
  const float kk = wave_sum(o.k * o.k);
  StepFlags f;
  o.step = executed_step(kk, dd, s_eta, s_alpha, g, &o.alpha, &f);
  o.flags = f.bits;
  return o;
}

// Sum over the 16 lanes of a DPP row; every lane of the row receives the total.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                                0xF, 0xF, false));
}
// Value held by lane k (0-3) of each quad, in every lane of that quad (k is a constant
// once the caller's loop is unrolled).
template <int CTRL>
__device__ __forceinline__ float dpp_bcast(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float quad_bcast(float v, int k) {
  switch (k) {
    case 0: return dpp_bcast<0x00>(v);   // quad_perm [0,0,0,0]
    case 1: return dpp_bcast<0x55>(v);   // quad_perm [1,1,1,1]
    case 2: return dpp_bcast<0xAA>(v);   // quad_perm [2,2,2,2]
    default: return dpp_bcast<0xFF>(v);  // quad_perm [3,3,3,3]
  }
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_move<0x128>(v);  // row_ror:8
  v += dpp_move<0x124>(v);  // row_ror:4
  v += dpp_move<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_move<0xB1>(v);   // quad_perm [1,0,3,2]
  return v;
}

// Product over lanes j..15 of a DPP row (suffix product); lanes past the row end count as 1.
__device__ __forceinline__ float row16_suffix_prod(float v) {
  const int one = __builtin_bit_cast(int, 1.f);
  v *= __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(one, __builtin_bit_cast(int, v), 0x101, 0xF, 0xF, false));
  v *= __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(one, __builtin_bit_cast(int, v), 0x102, 0xF, 0xF, false));
  v *= __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(one, __builtin_bit_cast(int, v), 0x104, 0xF, 0xF, false));
  v *= __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(one, __builtin_bit_cast(int, v), 0x108, 0xF, 0xF, false));
  return v;
}

// Product over lanes 0..j of a DPP row (prefix product); lanes before the row start count as 1.
__device__ __forceinline__ float row16_prefix_prod(float v) {
  const int one = __builtin_bit_cast(int, 1.f);
  v *= __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(one, __builtin_bit_cast(int, v), 0x111, 0xF, 0xF, false));
  v *= __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(one, __builtin_bit_cast(int, v), 0x112, 0xF, 0xF, false));
  v *= __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(one, __builtin_bit_cast(int, v), 0x114, 0xF, 0xF, false));
  v *= __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(one, __builtin_bit_cast(int, v), 0x118, 0xF, 0xF, false));
  return v;
}

// Workgroup barrier that orders LDS only: global loads in flight (prefetches) and global
// stores (readouts) stay outstanding across it, unlike __syncthreads().
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace hope
