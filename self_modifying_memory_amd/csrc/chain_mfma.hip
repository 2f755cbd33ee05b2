// Chunked recurrence on MFMA: one (image, head, route) chain per workgroup of four
// waves, for bf16 feature maps and head dimension 32 or 64 (gfx950).
//
// Method ("VisionHOPE: Visual Backbones as Self-Modifying Learning Systems"):
//   Sec. 2.1.3 Eq. 15-16  projections k, v, q, eta, alpha and the readout M_mem q are
//                         generated from the chunk-start state S_b;
//   Sec. 2.2 Eq. 19-20    executed step per token (shared helper token_gates);
//   App. B.4 Eq. 46-47    all six memories follow one gain: S_end = S_b G_C with
//                         G_t = alpha_t G_{t-1} + u_t k_t^T,  u_t = -step_t (G_{t-1} k_t + delta_t).
//
// The gain is applied in a compact (WY-like) form over blocks of up to 16 tokens.
// Starting a block from gain G_s, with P(a, b) = prod_{a <= s < b} alpha_s:
//   u_t = -step_t (P(0,t) G_s k_t + delta_t) - step_t sum_{j<t} P(j+1,t) (k_j . k_t) u_j
//   G_end = P(0,n) G_s + sum_j P(j+1,n) u_j k_j^T =: c G_s + Ub^T K.
// The state is then carried as S_b G = c (S_b G_s) + (S_b Ub^T) K, so the block costs two
// thin products with S_b instead of a d x d x (4d+2) product per chunk.
//
// Precision: the state, the gain and every accumulation are fp32.  Each dense
// contraction runs on bf16 MFMA with fp32 operands split as x = hi + lo (hi = bf16(x),
// lo = bf16(x - hi), |x - hi - lo| <= 2^-17 |x|) and three products hi*hi + hi*lo + lo*hi;
// the bf16 input tokens are exact, so the projections need two.
//
// Layout: the state stays in registers in the B-operand layout of a 16x16 MFMA tile:
// lane l of the wave that owns state-row tile m holds, for column tile n,
// S[16 m + (l & 15)][16 n + 4 (l >> 4) + i], i < 4.  Every product below is arranged
// so that its output lands in that same layout (or in the operand layout of the next
// product), so the state never goes through LDS.  A 32-deep k-step pairs column tiles
// (2s, 2s+1); the A operands read their k values in the same pairing.
#include "device_common.h"
#include "kernels.h"

namespace hope {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kSB = 16;  // tokens per block = MFMA tile height

__device__ __forceinline__ f32x4 mma32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(short4v, a),
                                                   __builtin_bit_cast(short4v, b), c, 0, 0, 0);
}
// c += a b with a, b given as hi/lo pairs (the lo*lo term is below fp32 resolution).
// An accumulation chain never mixes the 16x16x32 and 16x16x16 shapes: a 16x16x16 that
// takes a just-issued 16x16x32 result as its accumulator was seen to read the accumulator
// from before that product (no wait states are inserted between the two shapes).
__device__ __forceinline__ f32x4 mma32x3(bf16x8 ah, bf16x8 al, bf16x8 bh, bf16x8 bl, f32x4 c) {
  c = mma32(al, bh, c);
  c = mma32(ah, bl, c);
  return mma32(ah, bh, c);
}
__device__ __forceinline__ f32x4 mma16x3(bf16x4 ah, bf16x4 al, bf16x4 bh, bf16x4 bl, f32x4 c) {
  c = mma16(al, bh, c);
  c = mma16(ah, bl, c);
  return mma16(ah, bh, c);
}

__device__ __forceinline__ void split4(const f32x4 v, bf16x4& hi, bf16x4& lo);

// X Y for 16x16 fp32 matrices in the accumulator layout (lane (g, c), register i holds
// entry [4g + i][c]): a_t holds X^T, b holds Y.  Register i of both then carries the
// summation index 4g + i in the k slot of a 16x16x4 fp32 product, so four of them give
// the exact fp32 product with no operand splitting (VALU-free).
__device__ __forceinline__ f32x4 mm16(const f32x4 a_t, const f32x4 b) {
  f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a_t[i], b[i], c, 0, 0, 0);
  return c;
}

// hi = bf16(x) (round to nearest even), lo = bf16(x - hi), for a pair of floats: one
// packed conversion for hi, its two halves widened back by a shift and a mask, two
// subtractions and one packed conversion for lo (three VALU operations per element)
__device__ __forceinline__ void split_pair(float x0, float x1, unsigned& hi, unsigned& lo) {
  typedef float f32x2v __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
  const f32x2v x = {x0, x1};
  const unsigned h = __builtin_bit_cast(unsigned, __builtin_convertvector(x, bf16x2v));
  const f32x2v r = {x0 - __uint_as_float(h << 16), x1 - __uint_as_float(h & 0xffff0000u)};
  hi = h;
  lo = __builtin_bit_cast(unsigned, __builtin_convertvector(r, bf16x2v));
}
__device__ __forceinline__ void split8(const f32x4 v0, const f32x4 v1, bf16x8& hi, bf16x8& lo) {
  unsigned h0, h1, h2, h3, l0, l1, l2, l3;
  split_pair(v0[0], v0[1], h0, l0);
  split_pair(v0[2], v0[3], h1, l1);
  split_pair(v1[0], v1[1], h2, l2);
  split_pair(v1[2], v1[3], h3, l3);
  const u32x4 h = {h0, h1, h2, h3}, l = {l0, l1, l2, l3};
  hi = __builtin_bit_cast(bf16x8, h);
  lo = __builtin_bit_cast(bf16x8, l);
}
__device__ __forceinline__ void split4(const f32x4 v, bf16x4& hi, bf16x4& lo) {
  unsigned h0, h1, l0, l1;
  split_pair(v[0], v[1], h0, l0);
  split_pair(v[2], v[3], h1, l1);
  const u32x2 h = {h0, h1}, l = {l0, l1};
  hi = __builtin_bit_cast(bf16x4, h);
  lo = __builtin_bit_cast(bf16x4, l);
}

// The same k slots of a token-major bf16 row (8 values, no conversion)
__device__ __forceinline__ bf16x8 load_row_pair_bf16(const unsigned short* row, int s, int g) {
  const u32x2 lo4 = *reinterpret_cast<const u32x2*>(row + 32 * s + 4 * g);
  const u32x2 hi4 = *reinterpret_cast<const u32x2*>(row + 32 * s + 16 + 4 * g);
  const u32x4 both = {lo4[0], lo4[1], hi4[0], hi4[1]};
  return __builtin_bit_cast(bf16x8, both);
}

// A-operand k values of step s for a token-major fp32 row: cols 32s+4g.. and 32s+16+4g..
__device__ __forceinline__ void load_row_pair(const float* row, int s, int g, f32x4& v0, f32x4& v1) {
  v0 = *reinterpret_cast<const f32x4*>(row + 32 * s + 4 * g);
  v1 = *reinterpret_cast<const f32x4*>(row + 32 * s + 16 + 4 * g);
}

// NW waves per chain: 4 for d = 32, 8 for d = 64 (at most three state-row tiles per wave,
// so two waves fit on a SIMD).  Gates use waves 0-3 (16 lanes per token); with eight
// waves the solve coefficients run on waves 4-7 while waves 0-3 read out.
// The d = 64 kernels are held to 4 waves per SIMD (128 registers) so that two chains share
// a CU: the running-readout and variant instantiations then spill (35 and up to 48
// registers), which costs less than running one chain per CU.
// VAR: 0 the default operator, 1 every variant option, 2 only those of the VisionHOPE block
// (skip, direction scales, given queries)
template <int D, bool MULTI, int NW, bool RUN, int VAR>
__global__ __launch_bounds__(64 * NW, D == 64 ? 4 : 1) void chain_mfma_kernel(ChainParams p) {
  constexpr int kWaves = NW;
  constexpr int kThreads = 64 * NW;
  constexpr int NT = D / 16;                       // column tiles of the state
  constexpr int KS = D / 32;                       // 32-deep k-steps over the head dimension
  constexpr int MT = 4 * D / 16;                   // register tiles: rows of M_mem, M_k, M_v, M_q
  constexpr int MTW = MT / kWaves;                 // tiles per wave (round robin)
  static_assert(MT % kWaves == 0, "every wave holds the same number of state-row tiles");
  constexpr int TR = 4 * D;                        // first tail row: m_eta, then m_alpha
  // fp32 stride of token-major tiles: at d = 64, 72 floats (72 = 8 mod 32) puts the four
  // rows a quad reads in the solve (t = 4i + q) on disjoint banks; d = 32 keeps D + 4 (its
  // LDS budget holds four chains on a CU)
  constexpr int LD = D == 64 ? D + 8 : D + 4;
  constexpr int XLD = D + 8;                       // bf16 stride of the token block
  constexpr int PLD = 3 * D + 4;                   // fp32 stride of the projections
  constexpr int KTLD = kSB + 4;                    // bf16 stride of transposed K (per column)
  constexpr int LTLD = kSB + 4;                    // fp32 stride of L^T
  // d = 64, boundary readout, no variant options: the solve waves, idle while waves 0-3
  // form the gates, use that phase for the block's retention products, the Gram matrix of
  // the raw keys and the staging of the next block's tokens, all of which need only the
  // projections
  constexpr bool kEarly = D == 64 && !RUN && VAR != 1;
  // the early form stages the next block while this one's tokens (skip) and given queries
  // may still be read: two buffers of each with the block's options (the default operator
  // reads its tokens only in the projections, before the staging)
  constexpr int kXB = kEarly && VAR != 0 ? 2 : 1;
  // the M_mem tiles' split waits for the readout, off the projections' path, except in the
  // early form, whose readout waves wait for the solve waves' projections anyway
  constexpr bool kDeferMemSplit = D == 64 && !kEarly;

  __shared__ __attribute__((aligned(16))) unsigned short Xs[kXB * kSB * XLD];
  __shared__ __attribute__((aligned(16))) float Pj[kSB * PLD];
  __shared__ __attribute__((aligned(16))) float Ks[kSB * LD];
  __shared__ __attribute__((aligned(16))) float Dls[kSB * LD];
  __shared__ __attribute__((aligned(16))) float Ubs[kSB * LD];  // write vectors Ub, fp32
  // MFMA-ready bf16 hi/lo copies: Ub rows (A operand of S_b Ub^T) and K transposed
  // (A operand of the carry), written once by their producers instead of re-split per wave
  __shared__ __attribute__((aligned(16))) unsigned short UbH[kSB * XLD];
  __shared__ __attribute__((aligned(16))) unsigned short UbL[kSB * XLD];
  __shared__ __attribute__((aligned(16))) unsigned short KtH[D * KTLD];
  __shared__ __attribute__((aligned(16))) unsigned short KtL[D * KTLD];
  // token-major hi/lo copies of the normalised keys and queries (operands of the token
  // Gram products and of the readout)
  __shared__ __attribute__((aligned(16))) unsigned short KH[kSB * XLD];
  __shared__ __attribute__((aligned(16))) unsigned short KL[kSB * XLD];
  __shared__ __attribute__((aligned(16))) unsigned short QH[kSB * XLD];
  __shared__ __attribute__((aligned(16))) unsigned short QL[kSB * XLD];
  __shared__ int pixs[2][kSB];  // token pixels; two buffers when the next block is staged early
  __shared__ float kinvs[kEarly ? kSB : 1];  // 1 / |k_raw| of each token (early Gram)
  // early form: raw-key Gram matrix and retention products, accumulator layout
  __shared__ __attribute__((aligned(16))) float GrS[kEarly ? 256 : 4];
  __shared__ __attribute__((aligned(16))) float PrS[kEarly ? 256 : 4];
  __shared__ __attribute__((aligned(16))) float Gs[MULTI ? D * LD : 4];
  __shared__ __attribute__((aligned(16))) float alph[kSB];
  __shared__ __attribute__((aligned(16))) float stp[kSB];
  __shared__ float cprev[kSB], bco[kSB + 1];  // block retention products
  // L of the block solve, one copy per solve wave
  __shared__ __attribute__((aligned(16))) float LTs[(D / 16) * kSB * LTLD];
  // running readout: the masked token matrix A^T and the unscaled write vectors U
  __shared__ __attribute__((aligned(16))) float Ais[RUN ? 64 * 4 : 4];
  // given queries of the current block (fp32), staged one block ahead like x
  __shared__ __attribute__((aligned(16))) float Qs[VAR && !RUN ? kXB * kSB * D : 4];
  __shared__ __attribute__((aligned(16))) unsigned short UuH[RUN ? kSB * XLD : 4];
  __shared__ __attribute__((aligned(16))) unsigned short UuL[RUN ? kSB * XLD : 4];
  // the two gate rows (m_eta, m_alpha) live in LDS so that every wave holds the same
  // number of register tiles: Tb[cur] is the chunk-start copy, Tb[cur ^ 1] the update
  __shared__ __attribute__((aligned(16))) float Tb[2][2 * D];
  __shared__ unsigned int cnt_lds[3];  // step-control counters of this chain
  __shared__ __attribute__((aligned(16))) float ztl[2 * kSB];  // z_t of the two gate rows

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c16 = lane & 15, g = lane >> 4;
  const int nh = p.nh;
  const int h = blockIdx.x % nh;
  const int b = (blockIdx.x / nh) % p.B;
  const int slot = blockIdx.x / (nh * p.B);
  const int r = p.route_of_slot[slot];
  const int H = p.H, W = p.W, N = H * W, Dt = p.D;
  const int C = p.chunk > 0 ? p.chunk : (r < 2 ? W : H);
  const int64_t SS = 4 * D * D + 2 * D;
  // variants (compiled only into the VAR instantiations; the others see the defaults)
  // (the skip, direction-scale and query pointers are kept in LDS and read where used:
  // held in scalar registers across the block loop they would spill)
  __shared__ const void* vptr[3];
  const bool has_skip = VAR && p.skip, has_scales = VAR && p.route_scales, has_q = VAR && p.queries;
  unsigned long long* const v_counts = VAR == 1 ? p.counts : nullptr;
  float* const v_steps = VAR == 1 ? p.steps : nullptr;
  // M_q unused with given queries
  const unsigned v_frozen = VAR == 1 ? (p.frozen | (p.queries ? 4u : 0u)) : (VAR && p.queries ? 4u : 0u);
  const bool v_nodgd = VAR == 1 && p.no_dgd;
  const GateParams gp{p.eta_map, p.eta_scale, p.alpha_bias, p.eps, VAR == 1 ? p.injection : 0,
                      VAR == 1 ? p.spectral : 0};
  // register tiles held fixed within the image: M_k, M_v (bit 0) and M_q (bit 2); the gate
  // rows (bit 1) are handled with their LDS copy
  auto tile_frozen = [&](int m) {
    return ((v_frozen & 1u) && m >= NT && m < 3 * NT) || ((v_frozen & 4u) && m >= 3 * NT);
  };
  const bool gates_frozen = (v_frozen & 2u) != 0;
  // direction scale and skip of channel c (read once per readout tile) applied to a
  // readout y of token value xc
  auto finish = [&](float y, float skip_c, float scale_c, float xc) {
    if (has_skip) y = fmaf(skip_c, xc, y);
    if (has_scales) y *= scale_c;
    return y;
  };
  const unsigned short* Xcur = Xs;  // this block's tokens (a buffer of Xs)
  auto xs_at = [&](int t, int col) {
    return __uint_as_float((unsigned)Xcur[t * XLD + col] << 16);
  };
  const unsigned short* xg = static_cast<const unsigned short*>(p.x);
  // pixel of token tb + i of this route (tb the same in every lane, 0 <= i < kSB): one
  // division per block on the scalar unit, then each lane steps from it; exact integer
  // arithmetic, so the map is the one of route_pixel
  auto block_pixel = [&](int tb, int i) {
    if (r < 2) return (r & 1) ? N - 1 - tb - i : tb + i;
    const int base = (r & 1) ? N - 1 - tb : tb;
    int q = base / H, rem = base - q * H;
    if (r & 1) {
      rem -= i;
      while (rem < 0) rem += H, --q;
    } else {
      rem += i;
      while (rem >= H) rem -= H, ++q;
    }
    return rem * W + q;
  };
  float* dst = slot == 0 ? p.out : p.planes + (int64_t)(slot - 1) * p.plane_stride;

  // ---- state in registers --------------------------------------------------------
  f32x4 S[MTW][NT];
  f32x4 Acc[MULTI ? MTW : 1][MULTI ? NT : 1];
  {
    const float* init = p.init + init_offset(p, b, r, h, SS);
#pragma unroll
    for (int mi = 0; mi < MTW; ++mi) {
      const int row = (w + kWaves * mi) * 16 + c16;
#pragma unroll
      for (int n = 0; n < NT; ++n) S[mi][n] = *reinterpret_cast<const f32x4*>(init + row * D + n * 16 + 4 * g);
    }
    for (int i = threadIdx.x; i < 2 * D; i += kThreads) Tb[0][i] = init[TR * D + i];
    if (threadIdx.x < 3) cnt_lds[threadIdx.x] = 0u;
    if (VAR && threadIdx.x == 0) {
      vptr[0] = p.skip;
      vptr[1] = p.route_scales;
      vptr[2] = p.queries;
    }
  }
  int cur = 0;  // which Tb copy holds the chunk-start gate rows
  // B-operand values of the gate rows for column tile n (rows past the two are zero)
  auto tail_tile = [&](const float* t, int n, int c, int gg) {
    f32x4 v = *reinterpret_cast<const f32x4*>(t + (c & 1) * D + n * 16 + 4 * gg);
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    return c < 2 ? v : z;
  };

  // Tokens are gathered one block ahead: block k+1's 16-byte loads (8 channels per loader
  // thread) are in flight while block k computes, and are staged into LDS at its end.
  // The loaders are the last threads, on solve waves, which issue no global stores: a
  // wave's wait for its load then never includes the acknowledgements of readout stores.
  constexpr int kLoaders = kSB * (D / 8);
  constexpr int kLoad0 = kThreads - kLoaders;
  static_assert(kLoaders <= kThreads, "one 16-byte load per loader thread");
  // solve waves: the last NSW waves, none of which owns an M_mem (readout) tile; each
  // forms the block's 16x16 triangular system and solves it for its own 16 columns of U
  constexpr int NSW = NT;
  constexpr int SW0 = kWaves - NSW;
  static_assert(SW0 >= NT, "solve waves must not own readout tiles");
  static_assert(kLoad0 >= SW0 * 64, "loader threads sit on solve waves");
  // (loader indices come from a per-block opaque copy of the thread index, so that no
  // address built on them stays live across the phases)
  auto fetch = [&](int lid, int tb, int nt) {
    const int ld_i = lid - kLoad0;
    const int ld_t = ld_i / (D / 8), ld_c8 = ld_i % (D / 8);
    u32x4 v = {0u, 0u, 0u, 0u};
    if (ld_i >= 0 && ld_t < nt) {
      const int pix = block_pixel(tb, ld_t);
      v = *reinterpret_cast<const u32x4*>(xg + ((int64_t)b * N + pix) * Dt + (int64_t)h * D + ld_c8 * 8);
    }
    return v;
  };
  // start and length of the block after the one starting at tb (length 0 past the end)
  auto next_block = [&](int tb, int& tn, int& ntn) {
    const int cend = min((tb / C + 1) * C, N);
    tn = tb + kSB < cend ? tb + kSB : cend;
    ntn = tn < N ? min(kSB, min((tn / C + 1) * C, N) - tn) : 0;
  };
  auto stage_block = [&](int lid, const u32x4& v, int tb, int nt) {
    const int ld_i = lid - kLoad0;
    const int ld_t = ld_i / (D / 8), ld_c8 = ld_i % (D / 8);
    if (ld_i >= 0) *reinterpret_cast<u32x4*>(Xs + ld_t * XLD + ld_c8 * 8) = v;
    if (lid < kSB) pixs[0][lid] = lid < nt ? block_pixel(tb, lid) : 0;
  };
  // given queries (boundary-readout variant instantiations; the running readout reads them
  // directly): 16 bytes per loader thread, threads from 0, fp32 (4 values) or bf16 (8
  // values) per load; staged to Qs as fp32, zero past nt
  constexpr int kQPer32 = 4, kQPer16 = 8;
  constexpr bool kStageQ = VAR && !RUN;
  auto fetch_q = [&](int lid, int tb, int nt, const void* v_queries) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (kStageQ && has_q) {
      const int per = p.queries_bf16 ? kQPer16 : kQPer32;
      const int lt = lid / (D / per), lc = lid % (D / per);
      if (lt < nt) {
        const int64_t e = ((int64_t)b * N + block_pixel(tb, lt)) * Dt + (int64_t)h * D + lc * per;
        v = p.queries_bf16 ? *reinterpret_cast<const u32x4*>(static_cast<const unsigned short*>(v_queries) + e)
                           : *reinterpret_cast<const u32x4*>(static_cast<const float*>(v_queries) + e);
      }
    }
    return v;
  };
  auto stage_q = [&](int lid, const u32x4& v, int buf) {
    if (kStageQ && has_q) {
      const int per = p.queries_bf16 ? kQPer16 : kQPer32;
      const int lt = lid / (D / per), lc = lid % (D / per);
      if (lt < kSB) {
        float* q = Qs + buf * (kSB * D) + lt * D + lc * per;
        if (p.queries_bf16) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            q[2 * e] = __uint_as_float(v[e] << 16);
            q[2 * e + 1] = __uint_as_float(v[e] & 0xFFFF0000u);
          }
        } else {
          *reinterpret_cast<u32x4*>(q) = v;
        }
      }
    }
  };
  u32x4 pf, qpf;
  {
    const int lid = threadIdx.x;
    const int nt0 = min(kSB, min(C, N));
    stage_block(lid, fetch(lid, 0, nt0), 0, nt0);
    stage_q(lid, fetch_q(lid, 0, nt0, p.queries), 0);
    int tn, ntn;
    next_block(0, tn, ntn);
    pf = fetch(lid, tn, ntn);
    qpf = fetch_q(lid, tn, ntn, p.queries);
  }
  lds_barrier();

  // bf16 hi/lo split of the chunk-start state, formed once per chunk and kept in registers:
  // shared by the projections, the readout and the carry of every block of the chunk
  // (S_b is constant over the chunk)
  bf16x8 Sh[MTW][KS], Sl[MTW][KS];
  auto state_split = [&](int mi, int s, bf16x8& hi, bf16x8& lo) {
    hi = Sh[mi][s];
    lo = Sl[mi][s];
  };

  int bpar = 0;  // pixel-table buffer of the current block (early staging)
  for (int s0 = 0; s0 < N; s0 += C) {
    const int s1 = min(s0 + C, N);
    // (at d = 64 outside the early form the M_mem tiles, first read in the readout, are split
    // there, off the projections' path; measured slower at d = 32)
#pragma unroll
    for (int mi = 0; mi < MTW; ++mi)
      if (!kDeferMemSplit || w + kWaves * mi >= NT) {
#pragma unroll
        for (int s = 0; s < KS; ++s) split8(S[mi][2 * s], S[mi][2 * s + 1], Sh[mi][s], Sl[mi][s]);
      }
    if (MULTI) {
#pragma unroll
      for (int mi = 0; mi < MTW; ++mi)
#pragma unroll
        for (int n = 0; n < NT; ++n) Acc[MULTI ? mi : 0][MULTI ? n : 0] = S[mi][n];
    }
    for (int tb = s0; tb < s1; tb += kSB) {
      // lane indices re-derived through an opaque copy each block: the address
      // arithmetic built on them is then recomputed per block instead of being hoisted
      // out of the loop and held in registers across every phase
      int lid = threadIdx.x;
      asm volatile("" : "+v"(lid));
      const int lane = lid & 63;
      const int c16 = lid & 15, g = (lid >> 4) & 3;
      const int nt = min(kSB, s1 - tb);
      const bool first = tb == s0;
      const bool last_block = tb + kSB >= s1;
      const int* const pixc = pixs[kEarly ? bpar : 0];
      Xcur = Xs + (kXB > 1 ? bpar : 0) * (kSB * XLD);

      // A: projections P[t][row] = x_t . S_b[row] for the k, v, q, eta, alpha rows
      {
        bf16x8 xa[KS];
#pragma unroll
        for (int s = 0; s < KS; ++s) xa[s] = load_row_pair_bf16(Xcur + c16 * XLD, s, g);
#pragma unroll
        for (int mi = 0; mi < MTW; ++mi) {
          const int m = w + kWaves * mi;
          if (m < NT) continue;
          if (has_q && m >= 3 * NT) continue;  // queries are given: no q projection
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < KS; ++s) {
            bf16x8 sh, sl;
            state_split(mi, s, sh, sl);
            acc = mma32(xa[s], sl, acc);
            acc = mma32(xa[s], sh, acc);
          }
          const int row = m * 16 + c16;
#pragma unroll
          for (int i = 0; i < 4; ++i) Pj[(4 * g + i) * PLD + row - D] = acc[i];
        }
        if (w == 0) {  // the gate rows: scores s_eta, s_alpha of every token
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < KS; ++s) {
            bf16x8 th, tl;
            split8(tail_tile(Tb[cur], 2 * s, c16, g), tail_tile(Tb[cur], 2 * s + 1, c16, g), th, tl);
            acc = mma32(xa[s], tl, acc);
            acc = mma32(xa[s], th, acc);
          }
          if (c16 < 2) {
#pragma unroll
            for (int i = 0; i < 4; ++i) Pj[(4 * g + i) * PLD + 3 * D + c16] = acc[i];
          }
        }
      }
      lds_barrier();

      // B: normalisation, gates and executed step; 16 lanes per token (one DPP row),
      // each lane holding CPL consecutive components.  Padding tokens get no key, no
      // write and unit retention.
      if (w < 4) {
        __builtin_amdgcn_s_setprio(2);  // gates are on the block's critical path too
        constexpr int CPL = D / 16;
        const int t = 4 * w + g;
        const float* pt = Pj + t * PLD + c16 * CPL;
        float kr[CPL], vr[CPL], qr[CPL];
        float kk = 0.f, qq = 0.f;
#pragma unroll
        for (int e = 0; e < CPL; ++e) {
          kr[e] = pt[e];
          vr[e] = pt[D + e];
          if (!has_q) {
            qr[e] = pt[2 * D + e];
          } else if (kStageQ) {
            qr[e] = Qs[(kXB > 1 ? bpar : 0) * (kSB * D) + t * D + c16 * CPL + e];
          } else {
            const int64_t qi = ((int64_t)b * N + pixc[t]) * Dt + (int64_t)h * D + c16 * CPL + e;
            qr[e] = p.queries_bf16 ? __uint_as_float((unsigned)static_cast<const unsigned short*>(vptr[2])[qi] << 16)
                                   : static_cast<const float*>(vptr[2])[qi];
          }
          kk += kr[e] * kr[e];
          qq += qr[e] * qr[e];
        }
        const float kk_all = row16_sum(kk);
        const float kinv = fast_rsqrt(kk_all + gp.eps);
        const float qinv = fast_rsqrt(row16_sum(qq) + gp.eps);
        float kn[CPL], dl[CPL], qn[CPL];
        float dd = 0.f;
#pragma unroll
        for (int e = 0; e < CPL; ++e) {
          kn[e] = kr[e] * kinv;
          qn[e] = qr[e] * qinv;
          dl[e] = kn[e] - vr[e];
          dd += dl[e] * dl[e];
        }
        // |k|^2 of the normalised key: |k_raw|^2 kinv^2
        const float kk2 = kk_all * kinv * kinv;
        float alpha;
        StepFlags sf;
        const float step = executed_step(kk2, row16_sum(dd), Pj[t * PLD + 3 * D],
                                         Pj[t * PLD + 3 * D + 1], gp, &alpha, &sf);
        const bool live = t < nt;
        if (v_counts && c16 == 0 && live) {
          atomicAdd(&cnt_lds[0], 1u);
          atomicAdd(&cnt_lds[1], (unsigned)(sf.bits & 1));
          atomicAdd(&cnt_lds[2], (unsigned)((sf.bits >> 1) & 1));
        }
        if (v_steps && c16 == 0 && live)
          v_steps[(((int64_t)b * 4 + r) * p.nh + h) * ((int64_t)p.H * p.W) + pixc[t]] = step;
#pragma unroll
        for (int e = 0; e < CPL; e += 2) {
          const int col = c16 * CPL + e;
          // padding tokens have x = 0, so their raw projections, k and delta are exactly
          // zero; only queries read from the map need the mask
          const bool qlive = live || !(has_q && !kStageQ);
          const float k0 = kn[e], k1 = kn[e + 1];
          const float q0 = qlive ? qn[e] : 0.f, q1 = qlive ? qn[e + 1] : 0.f;
          Ks[t * LD + col] = k0;
          Ks[t * LD + col + 1] = k1;
          Dls[t * LD + col] = dl[e];
          Dls[t * LD + col + 1] = dl[e + 1];
          unsigned kh, kl, qh, ql;
          split_pair(k0, k1, kh, kl);
          split_pair(q0, q1, qh, ql);
          if (!kEarly) {  // (the early form's Gram reads the raw keys)
            *reinterpret_cast<unsigned*>(KH + t * XLD + col) = kh;
            *reinterpret_cast<unsigned*>(KL + t * XLD + col) = kl;
          }
          *reinterpret_cast<unsigned*>(QH + t * XLD + col) = qh;
          *reinterpret_cast<unsigned*>(QL + t * XLD + col) = ql;
          KtH[col * KTLD + t] = (unsigned short)kh;
          KtH[(col + 1) * KTLD + t] = (unsigned short)(kh >> 16);
          KtL[col * KTLD + t] = (unsigned short)kl;
          KtL[(col + 1) * KTLD + t] = (unsigned short)(kl >> 16);
        }
        if (c16 == 0) {
          alph[t] = live ? alpha : 1.f;
          stp[t] = live ? step : 0.f;
          if (kEarly) kinvs[t] = kinv;
        }
        __builtin_amdgcn_s_setprio(0);
        if (kEarly && kStageQ && has_q && s1 < N) {
          // the next block's given queries (this block's were read above), and the request
          // for the block after it: chunks of at most 16 tokens, so they start at s1, s1 + C
          stage_q(lid, qpf, bpar ^ 1);
          const int tq2 = s1 + C;
          qpf = fetch_q(lid, tq2, tq2 < N ? min(C, N - tq2) : 0, vptr[2]);
        }
      } else if (kEarly) {
        // the solve waves meanwhile, each part on one wave and published in LDS in the
        // accumulator layout (lane (g, c16), entry i: t = 4g + i, j = c16) for the solve
        // phase.  (1) Wave SW0: the Gram matrix of the raw keys, Graw[t][j] = k_raw,t .
        // k_raw,j (fp32 rows of the projections split into bf16 hi/lo); the normalised Gram
        // is kinv_t kinv_j times it.
        __builtin_amdgcn_s_setprio(2);  // as urgent as the gates: L needs both
        if (w == SW0) {
          f32x4 gr = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < KS; ++s) {
            f32x4 v0, v1;
            load_row_pair(Pj + c16 * PLD, s, g, v0, v1);
            bf16x8 kh, kl;
            split8(v0, v1, kh, kl);
            gr = mma32x3(kh, kl, kh, kl, gr);
          }
          *reinterpret_cast<f32x4*>(GrS + 4 * lane) = gr;
        }
        // (2) Waves SW0 + 1 and SW0 + 3: the retention of token c16, computed from its
        // score exactly as in the gate phase (unit for padding tokens); wave SW0 + 1 forms the
        // masked suffix products P(j+1, t) for L, wave SW0 + 3 (a loader wave, done early)
        // the block products P(0, t), P(t+1, 16)
        if (w == SW0 + 1 || w == SW0 + 3) {
          float ez;
          const float a_self = c16 < nt ? gate_alpha(Pj[c16 * PLD + 3 * D + 1], gp, &ez) : 1.f;
          const int one = __builtin_bit_cast(int, 1.f);
          const float a_next = __builtin_bit_cast(  // row_shl:1, lane 15 reads 1
              float, __builtin_amdgcn_update_dpp(one, __builtin_bit_cast(int, a_self), 0x101, 0xF, 0xF, false));
          if (w == SW0 + 1) {
            f32x4 pr;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float sp = row16_suffix_prod(c16 + 1 < 4 * g + i ? a_next : 1.f);
              pr[i] = c16 < 4 * g + i ? sp : 0.f;  // strictly lower triangle: L's mask
            }
            *reinterpret_cast<f32x4*>(PrS + 4 * lane) = pr;
          } else {
            const float a_prev = __builtin_bit_cast(  // row_shr:1, lane 0 reads 1
                float, __builtin_amdgcn_update_dpp(one, __builtin_bit_cast(int, a_self), 0x111, 0xF, 0xF, false));
            const float pre = row16_prefix_prod(c16 >= 1 ? a_prev : 1.f);
            const float suf = row16_suffix_prod(c16 < kSB - 1 ? a_next : 1.f);
            if (lane < kSB) {
              cprev[lane] = pre;
              bco[lane] = suf;
              if (lane == kSB - 1) bco[kSB] = pre * a_self;
            }
          }
        }
        __builtin_amdgcn_s_setprio(0);
        // (3) The loader threads stage the next block's tokens, fetched a block ago (X was
        // last read in A), with its pixel table in the other buffer, and request the block
        // after it.  At d = 64 every chunk is one block (at most 16 tokens), so the next
        // blocks start at s1 and s1 + C.
        const int tn = s1;
        if (w >= kLoad0 / 64 && tn < N) {  // (the loader waves only)
          const int ntn = min(C, N - tn);
          const int ld_i = lid - kLoad0;
          const int ld_t = ld_i / (D / 8), ld_c8 = ld_i % (D / 8);
          if (ld_i >= 0) *reinterpret_cast<u32x4*>(Xs + (kXB > 1 ? bpar ^ 1 : 0) * (kSB * XLD) + ld_t * XLD + ld_c8 * 8) = pf;
          if (ld_i >= 0 && ld_i < kSB) pixs[bpar ^ 1][ld_i] = ld_i < ntn ? block_pixel(tn, ld_i) : 0;
          const int tn2 = tn + C;
          pf = fetch(lid, tn2, tn2 < N ? min(C, N - tn2) : 0);
        }
      }
      lds_barrier();

      // C1: readout y_t = M_mem,b q_t on the waves that own M_mem tiles.  The running
      // readout keeps R = Q (M_mem,b G_s)^T (G_s: the chunk gain before this block) and the
      // token pixels in registers and completes y in D, once the block's U is known.
      f32x4 rq = {0.f, 0.f, 0.f, 0.f};
      int rpix[4] = {0, 0, 0, 0};
      float rx[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int mi = 0; mi < MTW; ++mi) {
        const int m = w + kWaves * mi;
        if (m >= NT) continue;
        if (kDeferMemSplit && first) {  // the chunk-start split of this M_mem tile
#pragma unroll
          for (int s = 0; s < KS; ++s) split8(S[mi][2 * s], S[mi][2 * s + 1], Sh[mi][s], Sl[mi][s]);
        }
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const bf16x8 ah = load_row_pair_bf16(QH + c16 * XLD, s, g);
          const bf16x8 al = load_row_pair_bf16(QL + c16 * XLD, s, g);
          bf16x8 sh, sl;
          if (RUN && MULTI) {  // the running state of the chunk so far
            split8(Acc[MULTI ? mi : 0][MULTI ? 2 * s : 0], Acc[MULTI ? mi : 0][MULTI ? 2 * s + 1 : 0], sh, sl);
          } else {
            state_split(mi, s, sh, sl);
          }
          acc = mma32x3(ah, al, sh, sl, acc);
        }
        if (RUN) {
          rq = acc;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            rpix[i] = pixc[4 * g + i];
            if (has_skip) rx[i] = xs_at(4 * g + i, m * 16 + c16);
          }
        } else {
          const int64_t c = (int64_t)h * D + m * 16 + c16;
          const float skip_c = has_skip ? static_cast<const float*>(vptr[0])[c] : 0.f;
          const float scale_c = has_scales ? static_cast<const float*>(vptr[1])[(int64_t)r * Dt + c] : 1.f;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int t = 4 * g + i;
            if (t < nt)
              dst[((int64_t)b * N + pixc[t]) * Dt + c] =
                  finish(acc[i], skip_c, scale_c, has_skip ? xs_at(t, m * 16 + c16) : 0.f);
          }
        }
      }
      // C2: the block's write vectors, on the NSW solve waves; wave ws = w - SW0 owns
      // columns 16 ws .. 16 ws + 15 of U.
      //   (I + L) U = RHS,  L[t][j] = step_t P(j+1,t) (k_t . k_j) for j < t,
      //   RHS[t] = -step_t (P(0,t) G_s k_t + delta_t),  Ub[t] = P(t+1,16) U[t].
      // L is strictly lower triangular and the same for every column of RHS, so the solve
      // is a forward substitution in exact fp32.  A quad of lanes shares a column and
      // splits its rows round robin (quad lane q holds rows q, q+4, q+8, q+12): once u_j is
      // final its holder broadcasts it over the quad by DPP, and every later row subtracts
      // L[t][j] u_j.  Each solve wave forms L itself (token Gram product on MFMA) and keeps
      // its own copy in LDS, laid out so that one 16-byte read gives a lane its four
      // coefficients of column j; the solve waves never wait for one another.
      if (w >= SW0) {
        // these waves are the block's critical path: let them win issue slots on their
        // SIMDs over the waves of the other chain sharing the CU
        __builtin_amdgcn_s_setprio(3);
        const int ws = w - SW0;
        float* const LTw = LTs + ws * (kSB * LTLD);
        const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
        // retention products over DPP rows (they need only alpha, so they overlap the
        // Gram product): P(j+1, t) for L (suffix over j), P(r+1, c) for the running
        // readout's A^T (prefix over c), and the block products P(0, t), P(t+1, 16)
        const bool ais_wave = RUN && w == SW0;
        float pj[4], pc[4], st_r[4];
        f32x4 gr = zero4, aq = zero4;
        if (kEarly) {
          // retention products and raw Gram from the gate phase; normalise the Gram here
          const float kv_j = kinvs[c16];
          const f32x4 gr_e = *reinterpret_cast<const f32x4*>(GrS + 4 * lane);
          const f32x4 pj_e = *reinterpret_cast<const f32x4*>(PrS + 4 * lane);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int rr = 4 * g + i;
            st_r[i] = stp[rr];
            pj[i] = pj_e[i];
            pc[i] = 0.f;
            gr[i] = kinvs[rr] * kv_j * gr_e[i];
          }
        } else {
          const float a_self = alph[c16];
          const float a_next = alph[min(c16 + 1, kSB - 1)], a_prev = alph[max(c16 - 1, 0)];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int rr = 4 * g + i;
            st_r[i] = stp[rr];
            pj[i] = row16_suffix_prod(c16 + 1 < rr ? a_next : 1.f);
            pc[i] = ais_wave ? row16_prefix_prod(c16 >= rr + 2 ? a_prev : 1.f) : 0.f;
          }
          {
            // every solve wave stores the same values; each reads back only after its own store
            const float pre = row16_prefix_prod(c16 >= 1 ? a_prev : 1.f);
            const float suf = row16_suffix_prod(c16 < kSB - 1 ? a_next : 1.f);
            if (lane < kSB) {
              cprev[lane] = pre;
              bco[lane] = suf;
              if (lane == kSB - 1) bco[kSB] = pre * a_self;
            }
          }
          // token Gram matrix, gr[i] = k_{4g+i} . k_{c16} (and, for the running readout,
          // aq[i] = k_{4g+i} . q_{c16})
#pragma unroll
          for (int s = 0; s < KS; ++s) {
            const bf16x8 kh = load_row_pair_bf16(KH + c16 * XLD, s, g);
            const bf16x8 kl = load_row_pair_bf16(KL + c16 * XLD, s, g);
            gr = mma32x3(kh, kl, kh, kl, gr);
            if (ais_wave) {
              const bf16x8 qh = load_row_pair_bf16(QH + c16 * XLD, s, g);
              const bf16x8 ql = load_row_pair_bf16(QL + c16 * XLD, s, g);
              aq = mma32x3(kh, kl, qh, ql, aq);
            }
          }
          if (ais_wave) {
            // A^T[j][t] = P(j+1, t) (k_j . q_t) for j < t, in the accumulator layout
            f32x4 at;
#pragma unroll
            for (int i = 0; i < 4; ++i) at[i] = 4 * g + i < c16 ? pc[i] * aq[i] : 0.f;
            *reinterpret_cast<f32x4*>(Ais + 4 * lane) = at;
          }
        }
        // L[t][j] (t = 4g+i, j = c16) goes to LTw[j][4 (t mod 4) + t / 4]; without the
        // key-dependent correction the writes do not interact (L = 0)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rr = 4 * g + i;
          const float lv = st_r[i] * pj[i] * gr[i];  // (the early pj is already masked)
          LTw[c16 * LTLD + 4 * i + g] = kEarly || (c16 < rr && !v_nodgd) ? lv : 0.f;
        }
        // RHS of a later block of a multi-block chunk: G_s k_t on MFMA for this wave's
        // column tile, staged token-major in Ubs (overwritten below with the write vectors)
        const bool gk_mfma = MULTI && !first && !v_nodgd;
        if (gk_mfma) {
          const int n = ws;
          f32x4 gk = zero4;
#pragma unroll
          for (int s = 0; s < KS; ++s) {
            f32x4 g0, g1;
            load_row_pair(Gs + (n * 16 + c16) * LD, s, g, g0, g1);
            const bf16x8 kh = load_row_pair_bf16(KH + c16 * XLD, s, g);
            const bf16x8 kl = load_row_pair_bf16(KL + c16 * XLD, s, g);
            bf16x8 gh, gl;
            split8(g0, g1, gh, gl);
            gk = mma32x3(kh, kl, gh, gl, gk);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int t = 4 * g + i;
            Ubs[t * LD + n * 16 + c16] = -stp[t] * (cprev[t] * gk[i] + Dls[t * LD + n * 16 + c16]);
          }
        }
        // forward substitution: column `col`, rows q + 4i of this lane
        const int col = 16 * ws + (lane >> 2), q = lane & 3;
        float u[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = 4 * i + q;
          if (gk_mfma) {
            u[i] = Ubs[t * LD + col];
          } else {  // G_s = I (first block) or no G_s k term (no DGD)
            const float gk = v_nodgd ? 0.f : Ks[t * LD + col];
            u[i] = -stp[t] * (cprev[t] * gk + Dls[t * LD + col]);
          }
        }
        if (!v_nodgd) {
          // (padding rows have zero RHS and zero L; they run through unchanged.  L is zero on
          // and above the diagonal, so the rows t <= j of step j subtract an exact zero and
          // need no mask)
          // Coefficient rows are read kPF steps ahead of their use (a rotating set of
          // registers), so that each step's LDS latency hides behind the steps before it.
          constexpr int kPF = 7;
          f32x4 crow[kPF];
#pragma unroll
          for (int j = 0; j < kPF; ++j) crow[j] = *reinterpret_cast<const f32x4*>(LTw + j * LTLD + 4 * q);
#pragma unroll
          for (int j = 0; j < kSB - 1; ++j) {
            const f32x4 c = crow[j % kPF];
            if (j + kPF < kSB - 1) crow[j % kPF] = *reinterpret_cast<const f32x4*>(LTw + (j + kPF) * LTLD + 4 * q);
            const float uj = quad_bcast(u[j >> 2], j & 3);
#pragma unroll
            for (int i = j >> 2; i < 4; ++i) u[i] = fmaf(-c[i], uj, u[i]);
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = 4 * i + q;
          const float ub = bco[t] * u[i];
          Ubs[t * LD + col] = ub;
          const __bf16 uh = (__bf16)ub;
          UbH[t * XLD + col] = __builtin_bit_cast(unsigned short, uh);
          UbL[t * XLD + col] = __builtin_bit_cast(unsigned short, (__bf16)(ub - (float)uh));
          if (RUN) {
            const __bf16 vh = (__bf16)u[i];
            UuH[t * XLD + col] = __builtin_bit_cast(unsigned short, vh);
            UuL[t * XLD + col] = __builtin_bit_cast(unsigned short, (__bf16)(u[i] - (float)vh));
          }
        }
        __builtin_amdgcn_s_setprio(0);
      }
      lds_barrier();

      // D: carry.  Z^T = Ub S_b^T (per state-row tile), then
      //     (S_b G)_new = c (S_b G) + Z K, evaluated transposed so it lands in place.
      {
        const float cc = bco[kSB];
        bf16x8 uh[KS], ul[KS];
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const unsigned short* hr = UbH + c16 * XLD + 32 * s + 4 * g;
          const unsigned short* lr = UbL + c16 * XLD + 32 * s + 4 * g;
          const u32x2 h0 = *reinterpret_cast<const u32x2*>(hr), h1 = *reinterpret_cast<const u32x2*>(hr + 16);
          const u32x2 l0 = *reinterpret_cast<const u32x2*>(lr), l1 = *reinterpret_cast<const u32x2*>(lr + 16);
          const u32x4 hv = {h0[0], h0[1], h1[0], h1[1]}, lv = {l0[0], l0[1], l1[0], l1[1]};
          uh[s] = __builtin_bit_cast(bf16x8, hv);
          ul[s] = __builtin_bit_cast(bf16x8, lv);
        }
        bf16x4 kah[NT], kal[NT];
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          kah[n] = __builtin_bit_cast(bf16x4, *reinterpret_cast<const u32x2*>(KtH + (n * 16 + c16) * KTLD + 4 * g));
          kal[n] = __builtin_bit_cast(bf16x4, *reinterpret_cast<const u32x2*>(KtL + (n * 16 + c16) * KTLD + 4 * g));
        }
        // all Z tiles first, so the state split dies before the updates start
        bf16x4 zh[MTW], zl[MTW];
        f32x4 zu = {0.f, 0.f, 0.f, 0.f};  // running readout: (M_mem,b u_t) for this tile
#pragma unroll
        for (int mi = 0; mi < MTW; ++mi) {
          f32x4 z = {0.f, 0.f, 0.f, 0.f};
          if (tile_frozen(w + kWaves * mi)) {  // no update: Z unused (never an M_mem tile)
            split4(z, zh[mi], zl[mi]);
            continue;
          }
#pragma unroll
          for (int s = 0; s < KS; ++s) {
            bf16x8 sh, sl;
            state_split(mi, s, sh, sl);
            z = mma32x3(uh[s], ul[s], sh, sl, z);
            if (RUN && mi == 0 && w < NT) {
              const unsigned short* hr = UuH + c16 * XLD + 32 * s + 4 * g;
              const unsigned short* lr = UuL + c16 * XLD + 32 * s + 4 * g;
              const u32x2 h0 = *reinterpret_cast<const u32x2*>(hr), h1 = *reinterpret_cast<const u32x2*>(hr + 16);
              const u32x2 l0 = *reinterpret_cast<const u32x2*>(lr), l1 = *reinterpret_cast<const u32x2*>(lr + 16);
              const u32x4 hv = {h0[0], h0[1], h1[0], h1[1]}, lv = {l0[0], l0[1], l1[0], l1[1]};
              zu = mma32x3(__builtin_bit_cast(bf16x8, hv), __builtin_bit_cast(bf16x8, lv), sh, sl, zu);
            }
          }
          split4(z, zh[mi], zl[mi]);
        }
        if (RUN && w < NT) {
          // y_t = P(0,t) (M_mem,b G_s q_t) + sum_{j<t} P(j+1,t) (k_j . q_t) (M_mem,b u_j)
          const f32x4 at = *reinterpret_cast<const f32x4*>(Ais + 4 * lane);
          const f32x4 y = mm16(at, zu);
          const int64_t c = (int64_t)h * D + w * 16 + c16;
          const float skip_c = has_skip ? static_cast<const float*>(vptr[0])[c] : 0.f;
          const float scale_c = has_scales ? static_cast<const float*>(vptr[1])[(int64_t)r * Dt + c] : 1.f;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int t = 4 * g + i;
            if (t < nt)
              dst[((int64_t)b * N + rpix[i]) * Dt + c] = finish(cprev[t] * rq[i] + y[i], skip_c, scale_c, rx[i]);
          }
        }
        // gate rows at d = 32: every readout wave forms their Z tile and updates column
        // tile w on MFMA (at d = 64 they are carried in fp32 below)
        constexpr bool tail_mfma = D != 64;
        bf16x4 tzh, tzl;
        if (tail_mfma && w < NT && !gates_frozen) {
          f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < KS; ++s) {
            bf16x8 th, tl;
            split8(tail_tile(Tb[cur], 2 * s, c16, g), tail_tile(Tb[cur], 2 * s + 1, c16, g), th, tl);
            z = mma32x3(uh[s], ul[s], th, tl, z);
          }
          split4(z, tzh, tzl);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int mi = 0; mi < MTW; ++mi) {
          if (tile_frozen(w + kWaves * mi)) continue;
#pragma unroll
          for (int n = 0; n < NT; ++n) {
            f32x4 acc = MULTI ? Acc[MULTI ? mi : 0][MULTI ? n : 0] : S[mi][n];
            acc *= cc;
            acc = mma16x3(kah[n], kal[n], zh[mi], zl[mi], acc);
            if (MULTI) {
              Acc[MULTI ? mi : 0][MULTI ? n : 0] = acc;
            } else {
              S[mi][n] = acc;
            }
          }
        }
        if (tail_mfma && w < NT && !gates_frozen) {
          f32x4 acc = tail_tile(first ? Tb[cur] : Tb[cur ^ 1], w, c16, g);
          acc *= cc;
          // K operand of column tile w, read again (an index into kah by wave id would not
          // stay in registers)
          const bf16x4 kh = __builtin_bit_cast(bf16x4, *reinterpret_cast<const u32x2*>(KtH + (w * 16 + c16) * KTLD + 4 * g));
          const bf16x4 kl = __builtin_bit_cast(bf16x4, *reinterpret_cast<const u32x2*>(KtL + (w * 16 + c16) * KTLD + 4 * g));
          acc = mma16x3(kh, kl, tzh, tzl, acc);
          if (c16 < 2) *reinterpret_cast<f32x4*>(Tb[cur ^ 1] + c16 * D + w * 16 + 4 * g) = acc;
        }
        // gate rows at d = 64, in exact fp32 on the vector ALUs (two rows fill an eighth of an
        // MFMA tile), on readout waves 0 and 1, which finish their carry before the solve
        // waves, two of which then stage the next block (measured: 1% faster than on two
        // solve waves): wave r takes row r,  z_t = Ub_t . m_b,  m <- c m + sum_t z_t k_t.
        // (Measured: at d = 32, four chains per CU, the MFMA form above is faster.)
        if (!tail_mfma && !gates_frozen && (w == 0 || w == 1)) {
          const int rrow = w;
          const float* mb = Tb[cur] + rrow * D;  // chunk-start row
          const int t = lane >> 2, qq = lane & 3;
          float z = 0.f;
#pragma unroll
          for (int j4 = 0; j4 < D / 16; ++j4) {  // 16-byte reads: D/4 columns per lane
            const int j = qq * (D / 4) + 4 * j4;
            const f32x4 u4 = *reinterpret_cast<const f32x4*>(Ubs + t * LD + j);
            const f32x4 m4 = *reinterpret_cast<const f32x4*>(mb + j);
            z = fmaf(u4[0], m4[0], fmaf(u4[1], m4[1], fmaf(u4[2], m4[2], fmaf(u4[3], m4[3], z))));
          }
          z += dpp_move<0xB1>(z);  // quad_perm [1,0,3,2]
          z += dpp_move<0x4E>(z);  // quad_perm [2,3,0,1]
          if (qq == 0) ztl[rrow * kSB + t] = z;
          // (this wave's LDS writes above precede its reads below)
          if (lane < D) {
            float acc = cc * (first ? Tb[cur] : Tb[cur ^ 1])[rrow * D + lane];
#pragma unroll
            for (int t4 = 0; t4 < kSB / 4; ++t4) {
              const f32x4 z4 = *reinterpret_cast<const f32x4*>(ztl + rrow * kSB + 4 * t4);
#pragma unroll
              for (int e = 0; e < 4; ++e) acc = fmaf(Ks[(4 * t4 + e) * LD + lane], z4[e], acc);
            }
            Tb[cur ^ 1][rrow * D + lane] = acc;
          }
        }
        // gain of the chunk so far, needed by the next block of the same chunk
        if (MULTI && !last_block) {
          for (int tile = w; tile < NT * NT; tile += kWaves) {
            const int ti = tile / NT, tn = tile % NT;
            f32x4 acc;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int gi = ti * 16 + 4 * g + e, gn = tn * 16 + c16;
              acc[e] = first ? (gi == gn ? cc : 0.f) : cc * Gs[gi * LD + gn];
            }
            f32x4 uv;
#pragma unroll
            for (int e = 0; e < 4; ++e) uv[e] = Ubs[(4 * g + e) * LD + ti * 16 + c16];
            bf16x4 ah, al;
            split4(uv, ah, al);
            acc = mma16x3(ah, al, kah[tn], kal[tn], acc);
#pragma unroll
            for (int e = 0; e < 4; ++e) Gs[(ti * 16 + 4 * g + e) * LD + tn * 16 + c16] = acc[e];
          }
        }
      }
      // stage the next block (X was last read in A, the pixel table in C) and request
      // the one after it (done during the gate phase in the early form)
      if (!kEarly) {
        int tn, ntn;
        next_block(tb, tn, ntn);
        if (ntn > 0) {
          int lid2 = threadIdx.x;
          asm volatile("" : "+v"(lid2));
          stage_block(lid2, pf, tn, ntn);
          stage_q(lid2, qpf, 0);
          int tn2, ntn2;
          next_block(tn, tn2, ntn2);
          pf = fetch(lid2, tn2, ntn2);
          qpf = fetch_q(lid2, tn2, ntn2, vptr[2]);
        }
      }
      bpar ^= 1;
      lds_barrier();
    }
    if (MULTI) {
#pragma unroll
      for (int mi = 0; mi < MTW; ++mi)
#pragma unroll
        for (int n = 0; n < NT; ++n) S[mi][n] = Acc[MULTI ? mi : 0][MULTI ? n : 0];
    }
    if (!gates_frozen) cur ^= 1;  // frozen gate rows stay in the chunk-start copy
  }

  if (p.final_mem) {
    float* fin = p.final_mem + (((int64_t)b * 4 + r) * nh + h) * SS;
#pragma unroll
    for (int mi = 0; mi < MTW; ++mi) {
      const int row = (w + kWaves * mi) * 16 + c16;
#pragma unroll
      for (int n = 0; n < NT; ++n)
        *reinterpret_cast<f32x4*>(fin + row * D + n * 16 + 4 * g) = S[mi][n];
    }
    for (int i = threadIdx.x; i < 2 * D; i += kThreads) fin[TR * D + i] = Tb[cur][i];
  }
  if (v_counts && threadIdx.x < 3) atomicAdd(&v_counts[threadIdx.x], (unsigned long long)cnt_lds[threadIdx.x]);

}

}  // namespace

bool mfma_path_supported(const ChainParams& p, int d) {
  if (!p.x_bf16) return false;
  if (p.mem_chunk > 0) return false;  // two chunk sizes: the fp32 kernel
  if (d == 32) return true;
  if (d != 64) return false;
  for (int s = 0; s < p.n_sel; ++s) {
    const int r = p.route_of_slot[s];
    const int C = p.chunk > 0 ? p.chunk : (r < 2 ? p.W : p.H);
    if (C > kSB) return false;  // the d = 64 variant keeps one state copy: one block per chunk
  }
  return true;
}

// true when the call asks for any variant that only the VAR instantiations implement
bool needs_variants(const ChainParams& p) {
  return p.route_scales || p.skip || p.counts || p.frozen || p.no_dgd || p.injection || p.spectral ||
         p.queries || p.steps;
}

template <int D, bool MULTI, int NW>
hipError_t launch_d(const ChainParams& p, dim3 grid, hipStream_t stream) {
  const dim3 block(64 * NW);
  // 0: no variant; 2: only the block's (skip, direction scales, given queries); 1: any
  const int var = !needs_variants(p) ? 0
                  : !(p.counts || p.frozen || p.no_dgd || p.injection || p.spectral || p.steps) ? 2 : 1;
  if (p.readout) {
    if (var == 1) hipLaunchKernelGGL((chain_mfma_kernel<D, MULTI, NW, true, 1>), grid, block, 0, stream, p);
    else if (var == 2) hipLaunchKernelGGL((chain_mfma_kernel<D, MULTI, NW, true, 2>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((chain_mfma_kernel<D, MULTI, NW, true, 0>), grid, block, 0, stream, p);
  } else {
    if (var == 1) hipLaunchKernelGGL((chain_mfma_kernel<D, MULTI, NW, false, 1>), grid, block, 0, stream, p);
    else if (var == 2) hipLaunchKernelGGL((chain_mfma_kernel<D, MULTI, NW, false, 2>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((chain_mfma_kernel<D, MULTI, NW, false, 0>), grid, block, 0, stream, p);
  }
  return hipGetLastError();
}

hipError_t launch_chain_mfma(const ChainParams& p, int d, hipStream_t stream) {
  const int64_t blocks = (int64_t)p.n_sel * p.B * p.nh;
  const dim3 grid((unsigned)blocks);
  if (d == 32) return launch_d<32, true, 4>(p, grid, stream);
  if (d == 64) return launch_d<64, false, 8>(p, grid, stream);
  return hipErrorInvalidValue;
}

}  // namespace hope
