// Backward pass of the four-direction scan at d = 32 with chunks of any length, gfx950: the
// chunk-parallel form in 16-token blocks, fp32 matrix cores (v_mfma_f32_16x16x4_f32, exact
// fp32 products and fp32 sums), one (image, head, route) chain per workgroup of 4 waves.
//
// Forward, per chunk c of a chain ("VisionHOPE: Visual Backbones as Self-Modifying Learning
// Systems", Sec. 2.1.3 Eq. 15-16, Sec. 2.2 Eq. 19-20 with the App. B.3 safeguards, App. B.4
// Eq. 46): all six memories share the chunk's gain, so the boundary state of chunk c is
// S_0 P_c with P_c the product of the earlier chunks' end gains (d x d) and the state S_0
// (4d+2 rows) fixed.  The chunk's projections are S_0 (P_c x_t), its readout
// S_0[mem] (P_c q_t), and its gain runs G_t = alpha_t G_{t-1} + u_t k_t^T from G = I with
// u_t = -step_t w_t, w_t = G_{t-1} k_t + delta_t.  The chunk is cut into blocks of 16
// tokens; with G_s the gain before a block and, inside it, Gam_{t-1} = alpha_0 .. alpha_{t-1}
// and beta_{j,t} = alpha_{j+1} .. alpha_t,
//   G_{t-1} = Gam_{t-1} G_s + sum_{j<t} beta_{j,t-1} u_j k_j^T,
//   w_t = Gam_{t-1} (G_s k_t) + delta_t + sum_{j<t} beta_{j,t-1} (k_j . k_t) u_j,
// a 16-step triangular recurrence, and the block's end gain is
// G_e = Gam_15 G_s + sum_t beta_{t,15} u_t k_t^T.  P_{c+1} = P_c G_C with G_C the chunk's
// last block end gain.
//
// Reverse (the memory trajectory is explicit and differentiable, Sec. 1), per block with
// dG_e the adjoint of its end gain (dG_e = P_c^T dP_{c+1} for the chunk's last block):
//   dG_t = Gam'_t dG_e - sum_{m>t} c_{t,m} a_m k_m^T  (Gam'_t = alpha_{t+1} .. alpha_15,
//   c_{t,m} = beta_{t,m-1} step_m),  a_t = dG_t k_t, so
//   a_t = Gam'_t (dG_e k_t) - sum_{m>t} c_{t,m} (k_m . k_t) a_m (backward recurrence);
//   dstep_t = -w_t . a_t,  ddelta_t = -step_t a_t,
//   dk_t = -step_t (G_{t-1}^T a_t + dG_t^T w_t),  dalpha_t = <G_{t-1}, dG_t>,
// both expanded through the low-rank forms into 16 x 16 Gram matrices (U^T A, A^T W,
// K^T K) and the vectors G_s k_t, G_s^T a_t, dG_e k_t, dG_e^T w_t, <G_s, dG_e>; then
//   dG_s = Gam_15 dG_e - sum_t Gam_{t-1} step_t a_t k_t^T   (the previous block's dG_e),
// the gates, the normalisation and the projections token by token, and
//   dP_c = dP_{c+1} G_C^T + sum_t (dx~_t x_t^T + dq~_t q_t^T),
//   dS_0 += sum_t [dy_t (P q_t)^T ; dp_t (P x_t)^T],  dx_t = P^T dx~_t,
// with dx~_t = S_0[proj]^T dp_t and dq~_t = S_0[mem]^T dy_t.  Where the step is not
// differentiable: min(eta_bar, eta_spec) follows eta_bar when eta_bar <= eta_spec; no
// derivative through the |k|^2 floor or the one-ulp rounding of eta_spec; eta_bar = 0
// (eta = 0 or eta_inj = 0) has derivative 0.
//
// A forward sweep writes P_c and, per block, its end gain, its token vectors (x~, k, delta,
// q, u, w) and gates to the workspace; the reverse sweep reads them back one block ahead.  S_0 stays in
// registers for the whole chain: waves 0 and 1 hold column tile w of every row (for S_0^T
// products), and waves 0-3 the rows of their projection row tiles (for S_0 products); the
// state adjoint dS_0 is accumulated in registers as 18 16 x 16 tiles, 8 on each of waves
// 2-3 and one on each of waves 0-1 (which also form S_0^T products in that phase).  P_c,
// P_c^T, the two adjoints of P, G_s, dG and the block's per-token vectors (token-major, 16
// token slots, padding slots zero) live in LDS: 76 KiB, two chains per CU.  The triangular
// recurrences run right-looking (column by column) on one wave.
#include "device_common.h"
#include "kernels.h"

namespace hope {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kD = 32;            // head dimension
constexpr int kTT = 16;           // token slots of a block
constexpr int kLD = kD + 4;       // LDS row stride of d-vectors and d x d matrices
constexpr int kR = 4 * kD + 2;    // state rows: M_mem, M_k, M_v, M_q, m_eta, m_alpha
constexpr int kPL = 116;          // stride of a token's projection row (7 row tiles = 112)
constexpr int kCL = 17;           // stride of the 16 x 16 token matrices
constexpr int kDD = kD * kD;
constexpr int kSS = kR * kD;      // state floats
// Workspace record of a 16-token block, written by the forward sweep: its end gain, then the
// token-major [16][d] arrays x~, k, delta, q, u, w and eight per-token scalars (step, alpha,
// the two reciprocal norms, |k|^2, |delta|^2, s_eta, s_alpha).
constexpr int kBTok = 16 * kD;
constexpr int kBR = kD * kD + 6 * kBTok + 8 * 16;
constexpr int kNT = 256;          // threads per chain
constexpr float kInjInward = 1.f - 1e-3f, kSpecInward = 1.f - 1e-6f, kKappaFloor = 1e-20f;

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

struct Lane {
  int lane, r16, q4;
};

// Sum over the 32 lanes of a half wave, in every lane of that half: DPP sums within the
// 16-lane rows, then v_permlane16_swap of the row totals with themselves, which hands each
// row of a pair (0-1, 2-3) the total of the even row in one result and of the odd row in
// the other.
__device__ __forceinline__ float half_total(float v) {
  v = row16_sum(v);
  const unsigned u = __builtin_bit_cast(unsigned, v);
  const auto sw = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return __builtin_bit_cast(float, (unsigned)sw[0]) + __builtin_bit_cast(float, (unsigned)sw[1]);
}

// The thread index through an opaque copy: LDS addresses derived from it are recomputed in
// each stage instead of being held across the block loops.
__device__ __forceinline__ int stage_lane(int tid) {
  asm volatile("" : "+v"(tid));
  return tid;
}
__device__ __forceinline__ Lane stage_lane_of(int tid) {
  const int t = stage_lane(tid);
  return Lane{t & 63, t & 15, (t & 63) >> 4};
}

// Eight consecutive floats of an LDS row (two 16-byte reads).
__device__ __forceinline__ void load8(const float* src, float* dst) {
  const f32x4 v0 = *reinterpret_cast<const f32x4*>(src);
  const f32x4 v1 = *reinterpret_cast<const f32x4*>(src + 4);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    dst[e] = v0[e];
    dst[4 + e] = v1[e];
  }
}

// Column tile m of the 16 token vectors times a d x d matrix:
// Out[t][16m + i] = sum_k M(16m + i, k) In[t][k], M(i, k) = M[i][k] (or M[k][i] if trans).
// MFMA operands: in step s, lane (r16, q4) feeds A[r16][k] and B[k][t = r16] with
// k = 8 q4 + s; result D[4 q4 + v][r16], i.e. component 16m + 4 q4 + v of token r16.
__device__ __forceinline__ f32x4 tok_prod(const float* M, bool trans, const float* In, int m,
                                          const Lane& L) {
  float a[8], bv[8];
  if (trans) {
#pragma unroll
    for (int s = 0; s < 8; ++s) a[s] = M[(8 * L.q4 + s) * kLD + 16 * m + L.r16];
  } else {
    load8(&M[(16 * m + L.r16) * kLD + 8 * L.q4], a);
  }
  load8(&In[L.r16 * kLD + 8 * L.q4], bv);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 8; ++s) acc = mfma4(a[s], bv[s], acc);
  return acc;
}

__device__ __forceinline__ void store_tokens(float* Out, int m, f32x4 acc, const Lane& L) {
  *reinterpret_cast<f32x4*>(&Out[L.r16 * kLD + 16 * m + 4 * L.q4]) = acc;
}

// 16 x 16 Gram matrix of two token-major arrays: D[j][t] = A_j . B_t (same operand mapping).
__device__ __forceinline__ f32x4 gram_tokens(const float* A, const float* B, const Lane& L) {
  float a[8], bv[8];
  load8(&A[L.r16 * kLD + 8 * L.q4], a);
  load8(&B[L.r16 * kLD + 8 * L.q4], bv);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 8; ++s) acc = mfma4(a[s], bv[s], acc);
  return acc;
}

__device__ __forceinline__ void store_cc(float* Out, f32x4 acc, const Lane& L) {
#pragma unroll
  for (int v = 0; v < 4; ++v) Out[(4 * L.q4 + v) * kCL + L.r16] = acc[v];
}

__device__ __forceinline__ void store_diag(float* Out, f32x4 acc, const Lane& L) {
#pragma unroll
  for (int v = 0; v < 4; ++v)
    if (4 * L.q4 + v == L.r16) Out[L.r16] = acc[v];
}

// Tile (mi, nj) of X Y for d x d matrices in LDS (Y read transposed if yT):
// D[4 q4 + v][r16] = sum_k X[16 mi + 4 q4 + v][k] Y(k, 16 nj + r16).
__device__ __forceinline__ f32x4 mm_tile(const float* X, const float* Y, bool yT, int mi, int nj,
                                         const Lane& L) {
  float a[8], bv[8];
  load8(&X[(16 * mi + L.r16) * kLD + 8 * L.q4], a);
  if (yT) {
    load8(&Y[(16 * nj + L.r16) * kLD + 8 * L.q4], bv);
  } else {
#pragma unroll
    for (int s = 0; s < 8; ++s) bv[s] = Y[(8 * L.q4 + s) * kLD + 16 * nj + L.r16];
  }
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 8; ++s) acc = mfma4(a[s], bv[s], acc);
  return acc;
}

__device__ __forceinline__ void store_dd(float* M, int mi, int nj, f32x4 acc, const Lane& L) {
#pragma unroll
  for (int v = 0; v < 4; ++v) M[(16 * mi + 4 * L.q4 + v) * kLD + 16 * nj + L.r16] = acc[v];
}

// Tile idx (0-3) of a d x d matrix in LDS: M <- gc M + sum over the 16 token slots of
// (A1_t, scaled by sc_t if kScale) B1_t^T.  (Which operands are present is a template
// argument: a test of a pointer into LDS against null is not folded by the compiler.)
template <bool kScale, bool kTwo = false>
__device__ __forceinline__ void dd_update(float* M, int idx, float gc, const float* A1,
                                          const float* B1, const float* sc, const Lane& L,
                                          const float* A2 = nullptr, const float* B2 = nullptr,
                                          const float* sc2 = nullptr) {
  const int mi = idx >> 1, nj = idx & 1;
  f32x4 acc;
#pragma unroll
  for (int v = 0; v < 4; ++v) acc[v] = gc * M[(16 * mi + 4 * L.q4 + v) * kLD + 16 * nj + L.r16];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int tk = 4 * s + L.q4;
    const float a = A1[tk * kLD + 16 * mi + L.r16];
    acc = mfma4(kScale ? a * sc[tk] : a, B1[tk * kLD + 16 * nj + L.r16], acc);
    if constexpr (kTwo) acc = mfma4(A2[tk * kLD + 16 * mi + L.r16] * sc2[tk], B2[tk * kLD + 16 * nj + L.r16], acc);
  }
#pragma unroll
  for (int v = 0; v < 4; ++v) M[(16 * mi + 4 * L.q4 + v) * kLD + 16 * nj + L.r16] = acc[v];
}

// A one-wave triangular recurrence over the 16 token slots, lane = component (the two half
// waves compute the same values; the lower half stores), right-looking: slot t starts from
// base_t = g0_t B0_t (+ B1_t), and once v_j is final every later slot t (t > j forward,
// t < j backward) adds cols[j][t] v_j, so one FMA per step is on the critical path; the
// coefficient columns are loaded two steps ahead.  kU: the u-recurrence (forward, with the
// B1 term, v = -gscale * pre stored to Out and pre to Out2); else the a-recurrence
// (backward, v = pre stored to Out; with kB1 its base has the B1 term too).
template <bool kU, bool kB1 = kU>
__device__ __forceinline__ void solve_cols(int lane, int bl, const float* cols, const float* g0,
                                           const float* B0, const float* B1, float* Out,
                                           float* Out2, const float* gscale) {
  constexpr bool kBack = !kU;
  const int c = lane & 31;
  float acc[kTT], gs[kTT];
#pragma unroll
  for (int t = 0; t < kTT; ++t) {
    const float b0 = B0[t * kLD + c];
    acc[t] = kB1 ? fmaf(g0[t], b0, B1[t * kLD + c]) : g0[t] * b0;
    if constexpr (kU) gs[t] = gscale[t];
  }
  f32x4 col[3][4];
  auto load_col = [&](int n) {
    const int j = kBack ? kTT - 1 - n : n;
#pragma unroll
    for (int q = 0; q < 4; ++q) col[n % 3][q] = *reinterpret_cast<const f32x4*>(&cols[j * kTT + 4 * q]);
  };
  load_col(0);
  load_col(1);
#pragma unroll
  for (int n = 0; n < kTT; ++n) {
    const int j = kBack ? kTT - 1 - n : n;
    if (n + 2 < kTT) load_col(n + 2);
    const float pre = j < bl ? acc[j] : 0.f;
    const float val = kU ? -gs[j] * pre : pre;
    if (lane < 32) {
      Out[j * kLD + c] = val;
      if constexpr (kU) Out2[j * kLD + c] = pre;
    }
#pragma unroll
    for (int t = 0; t < kTT; ++t)
      if (kBack ? t < j : t > j) acc[t] = fmaf(col[n % 3][t >> 2][t & 3], val, acc[t]);
  }
}

// XBF: the map is bf16 (else fp32).  RUN: the running readout y_t = S_0[mem] P_c G_{t-1} q_t
// (the memory after the chunk's earlier tokens): its adjoint r_t = P_c^T S_0[mem]^T dy_t
// enters every earlier gain, dG_{t-1} += r_t q_t^T, which adds to the a-recurrence's base
// sum_{m>t} beta_{t,m-1} (q_m . k_t) r_m, to dk_t the term sum_{m>t} beta_{t,m-1} (r_m . w_t) q_m
// (times -step_t), to dalpha_t Gam_{t-1} sum_{m>t} beta_{t,m-1} r_m . (G_s q_m) +
// sum_{j<t, m>t} beta_{j,t-1} beta_{t,m-1} (u_j . r_m)(k_j . q_m), to dG_s the sum
// sum_t Gam_{t-1} r_t q_t^T, and makes dq_t = G_{t-1}^T r_t; the readout's reads of P_c and
// S_0[mem] take G_{t-1} q_t in place of q_t.  Its extra arrays cost one chain per CU.
template <bool XBF, bool RUN>
__global__ __launch_bounds__(kNT, RUN ? 1 : 2) void chain_backward_wy32_kernel(BackParams p) {
  // One LDS block, small and uniformly read arrays first.
  constexpr int kTok = kTT * kLD;
  constexpr int kMat = kD * kLD;
  constexpr int oSc = 0;                      // per-token scalars, 16 x 16
  constexpr int oCC = oSc + 16 * kTT;         // 16 x 16 token matrices, 5 x 16 x 17
  constexpr int oRow = oCC + 5 * kTT * kCL;   // solve coefficient columns, 2 x 16 x 16
  constexpr int oTok = oRow + 2 * kTT * kTT;  // token-major d-vectors, 15 of them
  constexpr int oProj = oTok + 15 * kTok;     // projections [16][kPL], then their adjoints
  constexpr int oMat = oProj + kTT * kPL;     // P, P^T, two adjoints of P, G_s, dG
  constexpr int kSmem = oMat + 6 * kMat;
  // running readout only: K^T Q, U^T R, R^T W (16 x 16), r . (G_s q) per token, then the
  // token vectors r, G_{t-1} q, G_s q and the a-recurrence's readout base
  constexpr int kRunExtra = 3 * kTT * kCL + kTT + 4 * kTok;
  __shared__ __align__(16) float smem[kSmem + (RUN ? kRunExtra : 0)];
  float* const tSt = smem + oSc;    // step_t
  float* const tAl = tSt + kTT;     // alpha_t
  float* const tNk = tAl + kTT;     // 1 / sqrt(|k_raw|^2 + eps)
  float* const tNq = tNk + kTT;     // 1 / sqrt(|q_raw|^2 + eps)
  float* const tKk = tNq + kTT;     // |k|^2
  float* const tDd = tKk + kTT;     // |delta|^2
  float* const tSe = tDd + kTT;     // s_eta
  float* const tSa = tSe + kTT;     // s_alpha
  float* const tGam = tSa + kTT;    // Gam_{t-1}
  float* const tGp = tGam + kTT;    // Gam'_t (= beta_{t,15})
  float* const tGS = tGp + kTT;     // -Gam_{t-1} step_t
  float* const tL = tGS + kTT;      // a_t . (G_s k_t)
  float* const tUd = tL + kTT;      // u_t . (dG_e k_t)
  float* const tDal = tUd + kTT;    // dalpha_t from the gain
  float* const tMisc = tDal + kTT;  // [0] Gam_15, [1] <G_s, dG_e>
  int* const pixb = reinterpret_cast<int*>(tMisc + kTT);
  float* const sGm = smem + oCC;       // K^T K
  float* const sBt = sGm + kTT * kCL;  // beta[j][t]
  float* const sH = sBt + kTT * kCL;   // U^T A
  float* const sJ = sH + kTT * kCL;    // A^T W
  float* const sCm = sJ + kTT * kCL;   // c[t][m] = beta_{t,m-1} step_m for m > t
  float* const sColU = smem + oRow;    // [j][t]: beta_{j,t-1} (k_j . k_t), t > j
  float* const sColA = sColU + kTT * kTT;  // [m][t]: -c[t][m] (k_m . k_t), t < m
  float* const sX = smem + oTok;   // x
  // x~, k, delta, q, u, w: consecutive, in the order of the block record
  float* const sXt = sX + kTok;    // x~ = P x
  float* const sK = sXt + kTok;    // k
  float* const sDl = sK + kTok;    // delta
  float* const sQ = sDl + kTok;    // q
  float* const sU = sQ + kTok;     // u
  float* const sW = sU + kTok;     // w
  float* const sG = sW + kTok;     // G_s k
  float* const sE = sG + kTok;     // dG_e k, then G_s^T a
  float* const sGA = sE;
  float* const sQt = sE + kTok;    // q~ = P q
  float* const sdQt = sQt + kTok;  // dq~ = S_0[mem]^T dy, then dx~
  float* const sdXt = sdQt;
  float* const sdQ = sdQt + kTok;  // P^T dq~
  float* const sA = sdQ + kTok;    // a
  float* const sF = sA + kTok;     // dG_e^T w, then the gain part of dk / -step
  float* const sDY = sF + kTok;    // dy
  float* const sProj = smem + oProj;
  float* const sP = smem + oMat;   // P_c
  float* const sPT = sP + kMat;    // P_c^T
  float* sdPn = sPT + kMat;        // adjoint of P_{c+1}
  float* sdPc = sdPn + kMat;       // adjoint of P_c (accumulating)
  float* const sGs = sdPc + kMat;  // G_s (block start gain)
  float* const sdG = sGs + kMat;   // adjoint of the block's end gain
  float* const sKQ = smem + kSmem;     // [j][t]: k_j . q_t            (running readout only)
  float* const sUR = sKQ + kTT * kCL;  // [j][t]: u_j . r_t
  float* const sRW = sUR + kTT * kCL;  // [m][t]: r_m . w_t
  float* const tRg = sRW + kTT * kCL;  // r_t . (G_s q_t)
  float* const sR = tRg + kTT;         // r_t = P^T dq~_t
  float* const sRQ = sR + kTok;        // G_{t-1} q_t
  float* const sGQ = sRQ + kTok;       // G_s q_t
  float* const sXB = sGQ + kTok;       // sum_{m>t} beta_{t,m-1} (q_m . k_t) r_m

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
  const int nbc = (min(C, N) + kTT - 1) / kTT;  // blocks of a full chunk
  // chunk record: P_c, then the records of its blocks
  const int64_t kRecC = (int64_t)kDD + (int64_t)nbc * kBR;
  float* const dSg = p.chain_ws + (int64_t)blockIdx.x * p.chain_floats;
  float* const recs = dSg + kSS;
  float* const gdst = slot == 0 ? p.grad_x : p.planes + (int64_t)(slot - 1) * p.plane_stride;
  const GateParams gp{p.eta_map, p.eta_scale, p.alpha_bias, p.eps, 0, 0};
  const float* init = p.init + (p.init_per_image ? ((int64_t)b * 4 + r) * nh + h : (int64_t)r * nh + h) * kSS;

  // Registers held for the whole chain, by role:
  //   waves 0-1: reg4[T][s] = S_0[16T + 4q4 + s][16w + r16] for the 9 row tiles T (column
  //     tile w of S_0, for S_0^T products), and reg4[9] their one tile of dS_0;
  //   waves 2-3: reg4[0..7] their eight tiles of dS_0;
  //   every wave: projection row tiles T = 2 + 2w + sl (sl = 0, 1; T <= 8) of S_0,
  //     s0p[8 sl + s] = S_0[16T + r16][8q4 + s].
  // dS_0 tiles (row tile RT, column tile n): waves 0-1 hold (8, w), the gate rows; wave 2 the
  // row tiles 0, 2, 3, 4 and wave 3 the row tiles 1, 5, 6, 7 (both column tiles each), so
  // that every wave runs the same number of products in the adjoint phase.
  f32x4 reg4[10];
  float s0p[16];
  {
    const Lane L = stage_lane_of(tid);
#pragma unroll
    for (int e = 0; e < 36; ++e) {
      const int row = 16 * (e >> 2) + 4 * L.q4 + (e & 3);
      reg4[e >> 2][e & 3] = (w < 2 && row < kR) ? init[row * kD + 16 * w + L.r16] : 0.f;
    }
    reg4[9] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (w >= 2) {
#pragma unroll
      for (int i = 0; i < 8; ++i) reg4[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int T = 2 + 2 * w + (e >> 3), row = 16 * T + L.r16;
      s0p[e] = row < kR ? init[row * kD + 8 * L.q4 + (e & 7)] : 0.f;
    }
  }
  // row tile of dS_0 tile i (0-7, column tile i & 1) of waves 2-3
  auto dtile_row = [&](int i) {
    const int g = i >> 1;
    return g == 0 ? w - 2 : (w == 2 ? 1 : 4) + g;
  };

  // identity P_0, zero adjoint of P_nck
  for (int e = tid; e < kDD; e += kNT) {
    const int i = e >> 5, j = e & 31;
    sP[i * kLD + j] = i == j ? 1.f : 0.f;
    sdPn[i * kLD + j] = 0.f;
  }

  // Inputs of a block, fetched into registers one block ahead and written to LDS when the
  // block starts.  The loads are unconditional (padding slots read the block's last token
  // and are zeroed when written to LDS), so nothing waits for them before then.
  uint32_t fx[2];  // raw bits of x (bf16 in the low half, or fp32)
  float fdy[2], fg[4], ftk[12], fsc;
  // Route pixel of position s0 + t (t < 16) of this chain's route: for the column routes one
  // division of the block's first position by H (uniform) and a per-slot step from it.
  auto block_pixel = [&](int s0, int t) {
    if (r < 2) return (r & 1) ? N - 1 - s0 - t : s0 + t;
    const int b0 = (r & 1) ? N - 1 - s0 : s0;
    int q = b0 / H, m = b0 - q * H;
    if (r & 1) {
      m -= t;
      while (m < 0) { m += H; --q; }
    } else {
      m += t;
      while (m >= H) { m -= H; ++q; }
    }
    return m * W + q;
  };
  auto block_len = [&](int c, int i) {
    const int cl = min(C, N - c * C);
    return min(kTT, cl - kTT * i);
  };
  auto fetch = [&](int c, int i, bool rev) {
    const int t0 = stage_lane(tid), s0 = c * C + kTT * i, bl = block_len(c, i);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int e = t0 + kNT * k, t = min(e >> 5, bl - 1), j = e & 31;
      const int pix = block_pixel(s0, t);
      const int64_t idx = ((int64_t)b * N + pix) * Dt + (int64_t)h * kD + j;
      if (XBF) fx[k] = static_cast<const uint16_t*>(p.x)[idx];
      else fx[k] = __float_as_uint(static_cast<const float*>(p.x)[idx]);
      if (rev) fdy[k] = p.grad_out[idx];
    }
    if (rev) {
      // block i's record, and the end gain of block i - 1 (for block 0 a load of its own,
      // unused: every load here is unconditional, so that the registers it fills are the
      // ones the commit reads and nothing waits for it before then)
      const float* br = recs + (int64_t)c * kRecC + kDD + (int64_t)i * kBR;
      const float* g = i > 0 ? br - kBR : br;
#pragma unroll
      for (int k = 0; k < 4; ++k) fg[k] = g[t0 + kNT * k];
#pragma unroll
      for (int k = 0; k < 12; ++k) ftk[k] = br[kDD + t0 + kNT * k];
      fsc = br[kDD + 6 * kBTok + (t0 & (8 * kTT - 1))];
    }
  };
  auto commit = [&](int c, int i, bool rev) {
    const int t0 = stage_lane(tid), s0 = c * C + kTT * i, bl = block_len(c, i);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int e = t0 + kNT * k, t = e >> 5, j = e & 31;
      const float xv = XBF ? __uint_as_float(fx[k] << 16) : __uint_as_float(fx[k]);
      sX[t * kLD + j] = t < bl ? xv : 0.f;
      if (rev) sDY[t * kLD + j] = t < bl ? fdy[k] : 0.f;
    }
    if (rev) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int e = t0 + kNT * k, ri = e >> 5, j = e & 31;
        sGs[ri * kLD + j] = i > 0 ? fg[k] : (ri == j ? 1.f : 0.f);
      }
      // x~, k, delta, q, u, w (six consecutive token arrays) and the scalars
#pragma unroll
      for (int k = 0; k < 12; ++k) {
        const int e = t0 + kNT * k, a = e >> 9, t = (e >> 5) & 15, j = e & 31;
        sXt[a * kTok + t * kLD + j] = ftk[k];
      }
      if (t0 < 8 * kTT) tSt[t0] = fsc;
    }
    if (t0 < kTT) pixb[t0] = t0 < bl ? block_pixel(s0, t0) : 0;
  };
  // projections of the block: Proj[t][pr] = S_0[32 + pr] . x~_t, row tiles 2 + 2w + sl
  auto projections = [&]() {
    const Lane L = stage_lane_of(tid);
    float bv[8];
    load8(&sXt[L.r16 * kLD + 8 * L.q4], bv);
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) {
      const int T = 2 + 2 * w + sl;
      if (T <= 8) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 8; ++s) acc = mfma4(s0p[8 * sl + s], bv[s], acc);
        *reinterpret_cast<f32x4*>(&sProj[L.r16 * kPL + 16 * (T - 2) + 4 * L.q4]) = acc;
      }
    }
  };
  // the stabilised normalisation of k and q (App. C.1), delta = k - v and the step of every
  // token slot (half wave per token: tokens w + 4 hh + 8 u), with the norms and gate inputs
  // the backward reuses
  auto gates = [&](int bl) {
    const int lane = stage_lane(tid) & 63, c = lane & 31, hh = lane >> 5;
    float kr[2], vr[2], qr[2], se[2], sa[2], nk[2], nq[2], k[2], q[2], dl[2], kk[2], dd[2], al[2], st[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const float* pt = &sProj[(w + 4 * hh + 8 * u) * kPL];
      kr[u] = pt[c];
      vr[u] = pt[kD + c];
      qr[u] = pt[2 * kD + c];
      se[u] = pt[3 * kD];
      sa[u] = pt[3 * kD + 1];
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      nk[u] = fast_rsqrt(half_total(kr[u] * kr[u]) + gp.eps);
      nq[u] = fast_rsqrt(half_total(qr[u] * qr[u]) + gp.eps);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      k[u] = kr[u] * nk[u];
      q[u] = qr[u] * nq[u];
      dl[u] = k[u] - vr[u];
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      kk[u] = half_total(k[u] * k[u]);
      dd[u] = half_total(dl[u] * dl[u]);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) st[u] = executed_step(kk[u], dd[u], se[u], sa[u], gp, &al[u]);
    // padding slots (t >= bl): zero vectors, step 0, alpha 1, unit norms
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int t = w + 4 * hh + 8 * u;
      const bool on = t < bl;
      sK[t * kLD + c] = on ? k[u] : 0.f;
      sDl[t * kLD + c] = on ? dl[u] : 0.f;
      sQ[t * kLD + c] = on ? q[u] : 0.f;
      if (c == 0) {
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
  // products of alpha over token ranges (one (j, t) pair per thread):
  // Bt[j][t] = alpha_{j+1} .. alpha_t (j <= t, else 0), Gam_{t-1}, Gam'_t, Gam_15,
  // -Gam_{t-1} step_t
  auto alpha_products = [&]() {
    const int e = stage_lane(tid), t = e >> 4, j = e & 15;
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
    else if (j == 2) tGS[t] = -gm * tSt[t];
    else if (j == 3 && t == 0) tMisc[0] = gc;
  };
  auto dtok = [&](float* Out, const float* M, bool trans, const float* In, int m) {
    const Lane L = stage_lane_of(tid);
    store_tokens(Out, m, tok_prod(M, trans, In, m, L), L);
  };
  auto gram = [&](float* Out, const float* A, const float* B) {
    const Lane L = stage_lane_of(tid);
    store_cc(Out, gram_tokens(A, B, L), L);
  };
  auto gram_diag = [&](float* Out, const float* A, const float* B) {
    const Lane L = stage_lane_of(tid);
    store_diag(Out, gram_tokens(A, B, L), L);
  };
  auto ddu = [&](float* M, int idx, float gc, const float* A1, const float* B1) {
    const Lane L = stage_lane_of(tid);
    dd_update<false>(M, idx, gc, A1, B1, nullptr, L);
  };
  auto ddu_scaled = [&](float* M, int idx, float gc, const float* A1, const float* B1, const float* sc) {
    const Lane L = stage_lane_of(tid);
    dd_update<true>(M, idx, gc, A1, B1, sc, L);
  };
  // u-solve coefficient columns: u_j enters w_t with beta_{j,t-1} (k_j . k_t), t > j
  // (wave 0, 4 per lane)
  auto u_cols = [&]() {
    const int lane = stage_lane(tid) & 63;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int e = lane + 64 * k, j = e >> 4, t = e & 15;
      sColU[e] = j < t ? sBt[j * kCL + t - 1] * sGm[j * kCL + t] : 0.f;
    }
  };

  fetch(0, 0, false);
  __syncthreads();

  // ---- forward sweep: P_c and every block's record into the workspace ---------------------
  // (barriers order LDS only; global loads stay in flight across them, and the stores are
  // issued after the next block's prefetch so that waiting for the prefetch skips them)
  for (int c = 0; c < nck; ++c) {
    const int cl = min(C, N - c * C), nb = (cl + kTT - 1) / kTT;
    float* const rec = recs + (int64_t)c * kRecC;
    for (int e = tid; e < kDD; e += kNT) {
      const int i = e >> 5, j = e & 31;
      sGs[i * kLD + j] = i == j ? 1.f : 0.f;
    }
    for (int i = 0; i < nb; ++i) {
      const int bl = block_len(c, i);
      commit(c, i, false);
      {
        // the next block (the current one again after the last: fetched, unused)
        const bool last_in_chunk = i + 1 == nb, more = c + 1 < nck;
        fetch(last_in_chunk ? (more ? c + 1 : c) : c, last_in_chunk ? (more ? 0 : i) : i + 1, false);
      }
      if (i == 0) {
        const int t0 = stage_lane(tid);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int e = t0 + kNT * k;
          rec[e] = sP[(e >> 5) * kLD + (e & 31)];
        }
      }
      lds_barrier();
      if (w >= 2) dtok(sXt, sP, false, sX, w - 2);
      lds_barrier();
      projections();
      lds_barrier();
      gates(bl);
      lds_barrier();
      alpha_products();
      if (w == 0) gram(sGm, sK, sK);
      else if (w == 1) {
        dtok(sG, sGs, false, sK, 0);
        dtok(sG, sGs, false, sK, 1);
      }
      lds_barrier();
      if (w == 0) {
        u_cols();
        solve_cols<true>(stage_lane(tid) & 63, bl, sColU, tGam, sG, sDl, sU, sW, tSt);
      }
      lds_barrier();
      // G_e = Gam_15 G_s + U diag(beta_{., 15}) K^T, in place; the block's record
      ddu_scaled(sGs, w, tMisc[0], sU, sK, tGp);
      float* const br = rec + kDD + (int64_t)i * kBR;
      {
        const int t0 = stage_lane(tid);
#pragma unroll
        for (int k = 0; k < 12; ++k) {
          const int e = t0 + kNT * k, a = e >> 9, t = (e >> 5) & 15, j = e & 31;
          br[kDD + e] = sXt[a * kTok + t * kLD + j];
        }
        if (t0 < 8 * kTT) br[kDD + 6 * kBTok + t0] = tSt[t0];
      }
      lds_barrier();
      {
        const int t0 = stage_lane(tid);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int e = t0 + kNT * k;
          br[e] = sGs[(e >> 5) * kLD + (e & 31)];
        }
      }
    }
    if (c + 1 == nck) break;
    // P_{c+1} = P_c G_C
    f32x4 pn;
    {
      const Lane L = stage_lane_of(tid);
      pn = mm_tile(sP, sGs, false, w >> 1, w & 1, L);
    }
    lds_barrier();
    {
      const Lane L = stage_lane_of(tid);
      store_dd(sP, w >> 1, w & 1, pn, L);
    }
    lds_barrier();
  }

  // ---- reverse sweep ---------------------------------------------------------------------
  __syncthreads();  // the records written above are visible to every thread
  {
    const int cl = min(C, N - (nck - 1) * C);
    fetch(nck - 1, (cl + kTT - 1) / kTT - 1, true);
  }
  // P_c and G_C of a chunk, fetched one chunk ahead
  float fP[4], fGC[4];
  auto fetch_chunk = [&](int c) {
    const int t0 = stage_lane(tid), cl = min(C, N - c * C), nb = (cl + kTT - 1) / kTT;
    const float* rec = recs + (int64_t)c * kRecC;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      fP[k] = rec[t0 + kNT * k];
      fGC[k] = rec[kDD + (int64_t)(nb - 1) * kBR + t0 + kNT * k];  // end gain of the last block
    }
  };
  fetch_chunk(nck - 1);
  // dx of a block is stored after the next block's prefetch is issued (same reason)
  f32x4 dxv = {0.f, 0.f, 0.f, 0.f};
  float* dxdst = gdst;
  bool dxok = false;
  for (int c = nck - 1; c >= 0; --c) {
    const int cl = min(C, N - c * C), nb = (cl + kTT - 1) / kTT;
    // chunk start: P_c, P_c^T and G_C from the record
    lds_barrier();
    {
      const int t0 = stage_lane(tid);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int e = t0 + kNT * k, i = e >> 5, j = e & 31;
        sP[i * kLD + j] = fP[k];
        sPT[j * kLD + i] = fP[k];
        sGs[i * kLD + j] = fGC[k];
      }
    }
    if (c > 0) fetch_chunk(c - 1);
    lds_barrier();
    // dG_e of the last block = P_c^T dP_{c+1}; dP_c = dP_{c+1} G_C^T + (the blocks' terms)
    {
      const Lane L = stage_lane_of(tid);
      const int mi = w & 1;
      if (w < 2) {
        store_dd(sdG, mi, 0, mm_tile(sPT, sdPn, false, mi, 0, L), L);
        store_dd(sdG, mi, 1, mm_tile(sPT, sdPn, false, mi, 1, L), L);
      } else {
        store_dd(sdPc, mi, 0, mm_tile(sdPn, sGs, true, mi, 0, L), L);
        store_dd(sdPc, mi, 1, mm_tile(sdPn, sGs, true, mi, 1, L), L);
      }
    }
    for (int i = nb - 1; i >= 0; --i) {
      const int bl = block_len(c, i);
      lds_barrier();
      commit(c, i, true);
      {
        // the next block in reverse order (the current one again after the first)
        const int cn = i > 0 ? c : (c > 0 ? c - 1 : c);
        const int cln = min(C, N - cn * C);
        const int in = i > 0 ? i - 1 : (c > 0 ? (cln + kTT - 1) / kTT - 1 : i);
        fetch(cn, in, true);
      }
      if (dxok) *reinterpret_cast<f32x4*>(dxdst) = dxv;
      lds_barrier();
      // the block's forward values come from its record; alpha products (every thread);
      // dq~ = S_0[mem]^T dy tile w and K^T K (wave 0) or G_s k (wave 1); dG_e k (wave 2);
      // q~ = P q (wave 3)
      alpha_products();
      if (w < 2) {
        const Lane L = stage_lane_of(tid);
        f32x4 dy4[2];
#pragma unroll
        for (int T = 0; T < 2; ++T) dy4[T] = *reinterpret_cast<const f32x4*>(&sDY[L.r16 * kLD + 16 * T + 4 * L.q4]);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int T = 0; T < 2; ++T)
#pragma unroll
          for (int s = 0; s < 4; ++s) acc = mfma4(reg4[T][s], dy4[T][s], acc);
        store_tokens(sdQt, w, acc, L);
        if (w == 0) {
          gram(sGm, sK, sK);
        } else {
          dtok(sG, sGs, false, sK, 0);
          dtok(sG, sGs, false, sK, 1);
        }
      } else if (w == 2) {
        dtok(sE, sdG, false, sK, 0);
        dtok(sE, sdG, false, sK, 1);
      } else if constexpr (RUN) {
        gram(sKQ, sK, sQ);
        dtok(sGQ, sGs, false, sQ, 0);
        dtok(sGQ, sGs, false, sQ, 1);
      } else {
        dtok(sQt, sP, false, sQ, 0);
        dtok(sQt, sP, false, sQ, 1);
      }
      lds_barrier();
      if constexpr (RUN) {
        // r = P^T dq~ and the a-recurrence's readout base (wave 0); G_{t-1} q_t (wave 1)
        const Lane L = stage_lane_of(tid);
        const int r16 = L.r16, q4 = L.q4;
        if (w == 0) {
          dtok(sR, sPT, false, sdQt, 0);
          dtok(sR, sPT, false, sdQt, 1);
#pragma unroll
          for (int n = 0; n < 2; ++n) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) {
              const int m = 4 * s4 + q4, t = r16;
              const float cq = m > t ? sBt[t * kCL + m - 1] * sKQ[t * kCL + m] : 0.f;
              acc = mfma4(cq, sR[m * kLD + 16 * n + r16], acc);
            }
#pragma unroll
            for (int v = 0; v < 4; ++v) sXB[(4 * q4 + v) * kLD + 16 * n + r16] = acc[v];
          }
        } else if (w == 1) {
#pragma unroll
          for (int n = 0; n < 2; ++n) {
            f32x4 acc;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const int t = 4 * q4 + v;
              acc[v] = tGam[t] * sGQ[t * kLD + 16 * n + r16];
            }
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) {
              const int j = 4 * s4 + q4, t = r16;
              const float aq = j < t ? sBt[j * kCL + t - 1] * sKQ[j * kCL + t] : 0.f;
              acc = mfma4(aq, sU[j * kLD + 16 * n + r16], acc);
            }
#pragma unroll
            for (int v = 0; v < 4; ++v) sRQ[(4 * q4 + v) * kLD + 16 * n + r16] = acc[v];
          }
        }
        lds_barrier();
      }
      // c, the a-solve columns and a (wave 0); F = dG_e^T W (wave 1); dq = P^T dq~ and
      // diag(U^T E) (wave 2); dP_c += dq~ q^T and <G_s, dG_e> (wave 3).  Running readout:
      // the a-recurrence's base adds the readout term; dq = G_{t-1}^T r (wave 2); dP_c takes
      // G_{t-1} q, and wave 3 also forms q~ = P G_{t-1} q, r . (G_s q) and R^T W
      if (w == 0) {
        const int lane = stage_lane(tid) & 63;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int e = lane + 64 * k, t = e >> 4, m = e & 15;
          const float cm = m > t ? sBt[t * kCL + m - 1] * tSt[m] : 0.f;
          sCm[t * kCL + m] = cm;
          sColA[m * kTT + t] = -cm * sGm[m * kCL + t];
        }
        if constexpr (RUN) solve_cols<false, true>(lane, bl, sColA, tGp, sE, sXB, sA, nullptr, nullptr);
        else solve_cols<false>(lane, bl, sColA, tGp, sE, nullptr, sA, nullptr, nullptr);
      } else if (w == 1) {
        dtok(sF, sdG, true, sW, 0);
        dtok(sF, sdG, true, sW, 1);
      } else if (w == 2) {
        if constexpr (RUN) {
          // dq_t = Gam_{t-1} G_s^T r_t + sum_{j<t} beta_{j,t-1} (u_j . r_t) k_j
          gram(sUR, sU, sR);
          dtok(sdQ, sGs, true, sR, 0);
          dtok(sdQ, sGs, true, sR, 1);
          const Lane L = stage_lane_of(tid);
          const int r16 = L.r16, q4 = L.q4;
#pragma unroll
          for (int n = 0; n < 2; ++n) {
            f32x4 acc;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const int t = 4 * q4 + v;
              acc[v] = tGam[t] * sdQ[t * kLD + 16 * n + r16];
            }
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) {
              const int j = 4 * s4 + q4, t = r16;
              const float cu = j < t ? sBt[j * kCL + t - 1] * sUR[j * kCL + t] : 0.f;
              acc = mfma4(cu, sK[j * kLD + 16 * n + r16], acc);
            }
#pragma unroll
            for (int v = 0; v < 4; ++v) sdQ[(4 * q4 + v) * kLD + 16 * n + r16] = acc[v];
          }
        } else {
          dtok(sdQ, sPT, false, sdQt, 0);
          dtok(sdQ, sPT, false, sdQt, 1);
        }
        gram_diag(tUd, sU, sE);
      } else {
        if constexpr (RUN) {
#pragma unroll
          for (int idx = 0; idx < 4; ++idx) ddu(sdPc, idx, 1.f, sdQt, sRQ);
          dtok(sQt, sP, false, sRQ, 0);
          dtok(sQt, sP, false, sRQ, 1);
          gram_diag(tRg, sR, sGQ);
          gram(sRW, sR, sW);
        } else {
#pragma unroll
          for (int idx = 0; idx < 4; ++idx) ddu(sdPc, idx, 1.f, sdQt, sQ);
        }
        const int lane = stage_lane(tid) & 63;
        float tr = 0.f;
#pragma unroll 4
        for (int k = 0; k < 16; ++k) {
          const int e = lane + 64 * k, o = (e >> 5) * kLD + (e & 31);
          tr = fmaf(sGs[o], sdG[o], tr);
        }
        tr = half_total(tr);
        tr += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, tr), 32));
        if (lane == 0) tMisc[1] = tr;
      }
      lds_barrier();
      // H = U^T A, J = A^T W (wave 0); G_s^T a (wave 1); diag(A^T (G_s K)) (wave 2);
      // dG <- Gam_15 dG - sum_t Gam_{t-1} step_t a_t k_t^T (waves 2-3)
      if (w == 0) {
        gram(sH, sU, sA);
        gram(sJ, sA, sW);
      } else if (w == 1) {
        dtok(sGA, sGs, true, sA, 0);
        dtok(sGA, sGs, true, sA, 1);
      } else {
        if (w == 2) gram_diag(tL, sG, sA);
        if constexpr (RUN) {
          // dG_s also gains sum_t Gam_{t-1} r_t q_t^T
          const Lane L = stage_lane_of(tid);
          dd_update<true, true>(sdG, 2 * (w - 2), tMisc[0], sA, sK, tGS, L, sR, sQ, tGam);
          dd_update<true, true>(sdG, 2 * (w - 2) + 1, tMisc[0], sA, sK, tGS, L, sR, sQ, tGam);
        } else {
          ddu_scaled(sdG, 2 * (w - 2), tMisc[0], sA, sK, tGS);
          ddu_scaled(sdG, 2 * (w - 2) + 1, tMisc[0], sA, sK, tGS);
        }
      }
      lds_barrier();
      // dalpha_t from the gain (wave 0, through the 16 x 16 product inner = (H o K^T K) c^T);
      // the gain part of dk_t / -step_t (waves 1-2, column tile w - 1, over F in place):
      // Gam_{t-1} G_s^T a_t + Gam'_t F_t + sum_j cf[j][t] k_j with cf[j][t] =
      // beta_{j,t-1} H[j][t] (j < t) or -c[t][j] J[j][t] (j > t)
      if (w == 0) {
        const Lane L = stage_lane_of(tid);
        const int r16 = L.r16, q4 = L.q4;
        f32x4 inner = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int m = 4 * s + q4;
          inner = mfma4(sH[r16 * kCL + m] * sGm[r16 * kCL + m], sCm[r16 * kCL + m], inner);
          if constexpr (RUN) {
            // minus the readout's part: (U^T R o K^T Q) beta^T, beta[t][m] = beta_{t,m-1} (m > t)
            const float bm = m > r16 ? sBt[r16 * kCL + m - 1] : 0.f;
            inner = mfma4(-sUR[r16 * kCL + m] * sKQ[r16 * kCL + m], bm, inner);
          }
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
          if constexpr (RUN) {
#pragma unroll
            for (int m = 0; m < kTT; ++m)
              if (m > t) lsum = fmaf(-sBt[t * kCL + m - 1], tRg[m], lsum);
          }
          tDal[t] = part + tGam[t] * (gp1 * tMisc[1] - lsum);
        }
      } else if (w <= 2) {
        const Lane L = stage_lane_of(tid);
        const int n = w - 1, r16 = L.r16, q4 = L.q4, col = 16 * n + r16;
        f32x4 acc;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int t = 4 * q4 + v;
          acc[v] = fmaf(tGam[t], sGA[t * kLD + col], tGp[t] * sF[t * kLD + col]);
        }
        // A[t = r16][j = 4 s + q4] = cf[j][t], B[j][c] = k_j[16 n + c]
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
          const int j = 4 * s4 + q4, t = r16;
          float cf = 0.f;
          if (j < t) cf = sBt[j * kCL + t - 1] * sH[j * kCL + t];
          else if (j > t) cf = -sCm[t * kCL + j] * sJ[j * kCL + t];
          acc = mfma4(cf, sK[j * kLD + col], acc);
          if constexpr (RUN) {
            // + sum_{m>t} beta_{t,m-1} (r_m . w_t) q_m
            const float cr = j > t ? sBt[t * kCL + j - 1] * sRW[j * kCL + t] : 0.f;
            acc = mfma4(cr, sQ[j * kLD + col], acc);
          }
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) sF[(4 * q4 + v) * kLD + col] = acc[v];
      }
      lds_barrier();
      // token by token: the gain adjoints, then the readout, the step, the gates, the
      // normalisation and the projections; dProj goes to the projections' area (zero rows in
      // padding slots)
      {
        const int lane = stage_lane(tid) & 63, c = lane & 31, hh = lane >> 5;
        float dk[2], ddl[2], dstep[2], dalpha[2], dq[2], k[2], q[2], dl[2];
        float deta_dse[2], alpha[2], oma[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int t = w + 4 * hh + 8 * u;
          const float st = tSt[t];
          const float at = sA[t * kLD + c];
          dk[u] = -st * sF[t * kLD + c];
          ddl[u] = -st * at;
          dstep[u] = -sJ[t * kCL + t];
          dalpha[u] = tDal[t];
          dq[u] = sdQ[t * kLD + c];
          k[u] = sK[t * kLD + c];
          q[u] = sQ[t * kLD + c];
          dl[u] = sDl[t * kLD + c];
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          // forward values, as in the gates and executed_step
          const int t = w + 4 * hh + 8 * u;
          const float kk = tKk[t], dd = tDd[t], se = tSe[t], sa = tSa[t];
          float eta;
          if (gp.eta_map == 0) {
            const float sg = fast_rcp(1.f + fast_exp(-se));
            eta = gp.eta_scale * sg;
            deta_dse[u] = gp.eta_scale * sg * (1.f - sg);
          } else {
            eta = gp.eta_scale * (fmaxf(se, 0.f) + log1pf(fast_exp(-fabsf(se))));
            deta_dse[u] = gp.eta_scale * fast_rcp(1.f + fast_exp(-se));
          }
          const float ez = fast_exp(-(sa + gp.alpha_bias));
          alpha[u] = fast_rcp(1.f + ez);
          oma[u] = ez * alpha[u];  // 1 - alpha
          const float rr0 = fast_sqrt(dd + gp.eps * gp.eps);
          const float rr = rr0 + gp.eps;
          const float inj = kInjInward * oma[u] * fast_rcp(rr);
          const bool ok = eta != 0.f && inj != 0.f;
          const float xr = ok ? eta * fast_rcp(inj) : 0.f;
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
          kdk[u] = half_total(k[u] * dk[u]);
          qdq[u] = half_total(q[u] * dq[u]);
        }
        // dProj rows; zero in padding slots
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int t = w + 4 * hh + 8 * u;
          const bool on = t < bl;
          float* pt = &sProj[t * kPL];
          pt[c] = on ? (dk[u] - k[u] * kdk[u]) * tNk[t] : 0.f;
          pt[kD + c] = on ? -ddl[u] : 0.f;
          pt[2 * kD + c] = on ? (dq[u] - q[u] * qdq[u]) * tNq[t] : 0.f;
          if (c < 16) {
            const float g = c == 0 ? deta_dse[u] : (c == 1 ? dalpha[u] * alpha[u] * oma[u] : 0.f);
            pt[3 * kD + c] = on ? g : 0.f;
          }
        }
      }
      lds_barrier();
      // dx~ = S_0[proj]^T dProj (waves 0-1); dS_0 += [dy q~^T ; dProj x~^T] (all waves)
      {
        const Lane L = stage_lane_of(tid);
        const int r16 = L.r16, q4 = L.q4;
        if (w < 2) {
          f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
          f32x4 pv[7];
#pragma unroll
          for (int T = 2; T < 9; ++T) pv[T - 2] = *reinterpret_cast<const f32x4*>(&sProj[r16 * kPL + 16 * (T - 2) + 4 * q4]);
#pragma unroll
          for (int T = 2; T < 9; ++T)
#pragma unroll
            for (int s = 0; s < 4; ++s) {
              if (s & 1) acc1 = mfma4(reg4[T][s], pv[T - 2][s], acc1);
              else acc0 = mfma4(reg4[T][s], pv[T - 2][s], acc0);
            }
          store_tokens(sdXt, w, acc0 + acc1, L);
        }
        // acc += sum over the token slots of [dy ; dProj]_t (rows of tile RT) [q~ ; x~]_t^T
        // (columns of tile n)
        // (mem: a tile of the M_mem rows, RT < 2)
        auto ds_update = [&](f32x4 acc, bool mem, int RT, int n) {
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const int tk = 4 * s + q4;
            const float av = mem ? sDY[tk * kLD + 16 * RT + r16] : sProj[tk * kPL + 16 * (RT - 2) + r16];
            const float bv = mem ? sQt[tk * kLD + 16 * n + r16] : sXt[tk * kLD + 16 * n + r16];
            acc = mfma4(av, bv, acc);
          }
          return acc;
        };
        if (w < 2) {
          reg4[9] = ds_update(reg4[9], false, 8, w);
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            reg4[i] = ds_update(reg4[i], i < 2, dtile_row(i), i & 1);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
      lds_barrier();
      // dx = P^T dx~ (waves 0-1, stored after the next prefetch); dP_c += dx~ x^T (waves 2-3)
      if (w < 2) {
        const Lane L = stage_lane_of(tid);
        dxv = tok_prod(sPT, false, sdXt, w, L);
        dxok = L.r16 < bl;
        dxdst = gdst + ((int64_t)b * N + pixb[L.r16]) * Dt + (int64_t)h * kD + 16 * w + 4 * L.q4;
      } else {
        ddu(sdPc, 2 * (w - 2), 1.f, sdXt, sX);
        ddu(sdPc, 2 * (w - 2) + 1, 1.f, sdXt, sX);
      }
    }
    // dP_c is complete: it is the next chunk's dP_{c+1}
    float* const tmp = sdPn;
    sdPn = sdPc;
    sdPc = tmp;
  }
  if (dxok) *reinterpret_cast<f32x4*>(dxdst) = dxv;

  // the initial-state adjoint of this chain, for the gradient reduction
  {
    const Lane L = stage_lane_of(tid);
    auto store_tile = [&](f32x4 acc, int RT, int n) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = 16 * RT + 4 * L.q4 + v;
        if (row < kR) dSg[row * kD + 16 * n + L.r16] = acc[v];
      }
    };
    if (w < 2) {
      store_tile(reg4[9], 8, w);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) store_tile(reg4[i], dtile_row(i), i & 1);
    }
  }
}

}  // namespace

bool backward_wy32_supported(const BackParams& p, int d) {
  (void)p;
  return d == kD;
}

// Workspace floats per chain: the state adjoint, then per chunk P_c and the records of its
// 16-token blocks.
int64_t backward_wy32_chain_floats(int64_t nck, int64_t cmax) {
  const int64_t nb = (cmax + kTT - 1) / kTT;
  return ((int64_t)kSS + nck * ((int64_t)kDD + nb * kBR) + 63) / 64 * 64;
}

hipError_t launch_chain_backward_wy32(const BackParams& p, hipStream_t stream) {
  const int64_t blocks = (int64_t)p.n_sel * p.B * p.nh;
  const dim3 grid((unsigned)blocks), block(kNT);
  if (p.readout) {
    if (p.x_bf16) chain_backward_wy32_kernel<true, true><<<grid, block, 0, stream>>>(p);
    else chain_backward_wy32_kernel<false, true><<<grid, block, 0, stream>>>(p);
  } else {
    if (p.x_bf16) chain_backward_wy32_kernel<true, false><<<grid, block, 0, stream>>>(p);
    else chain_backward_wy32_kernel<false, false><<<grid, block, 0, stream>>>(p);
  }
  return hipGetLastError();
}

}  // namespace hope
