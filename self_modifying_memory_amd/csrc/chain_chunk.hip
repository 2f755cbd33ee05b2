// Chunk-parallel recurrence on MFMA: one (image, head, route) chain per workgroup, for bf16
// feature maps at head dimension 16, 32 or 64 and chunks of any length (gfx950).
//
// Method ("VisionHOPE: Visual Backbones as Self-Modifying Learning Systems"):
//   Sec. 2.1.3 Eq. 15-16  projections k, v, q, eta, alpha and the readout M_mem q come from
//                         the chunk-start state S_b, so every token of a chunk can generate
//                         them at once;
//   Sec. 2.2 Eq. 19-20    executed step per token (shared helper executed_step);
//   App. B.4 Eq. 45-47    all six memories follow one gain, G_t = alpha_t G_{t-1} + w_t k_t^T
//                         with w_t = -step_t (G_{t-1} k_t + delta_t).
//
// A chunk is processed in segments of up to SEG tokens (16 or 64 at d = 16, 64 at d = 32, 32
// at d = 64; one segment when the chunk fits).  With P(a, b) = prod_{a <= s < b} alpha_s over the segment's
// tokens and G_s the chunk gain at the segment's start (the identity for the first segment),
// the segment's write vectors solve the unit lower-triangular system
//   (I + L) W = R,   L[t][j] = step_t P(j+1, t) (k_j . k_t)  for j < t,
//                    R[t]    = -step_t (P(0, t) G_s k_t + delta_t),
// and the gain at its end is G_e = P(0, n) G_s + sum_t P(t+1, n) w_t k_t^T.  The state is
// carried as S_b G_e = P(0, n) (S_b G_s) + (S_b Ub^T) K with Ub_t = P(t+1, n) w_t.
//
// The system is solved by 16-token tiles.  Every diagonal tile's inverse T_JJ = (I + L_JJ)^-1
// is formed at once (forward substitution in exact fp32, one tile per wave), then one wave
// per 16 columns of W runs W_J = T_JJ R_J and R_I -= L_IJ W_J for every later tile I on the
// matrix cores: the sequential part of a segment is a dependent pair of 16x16x16 products
// per tile.  Retention products are formed without division: within a tile by DPP prefix
// and suffix products, across tiles from the tiles' totals.
//
// Precision: the state, the gain and every accumulation are fp32; each dense contraction is
// a bf16 MFMA with fp32 operands split hi/lo (three products; the bf16 tokens are exact, so
// the projections need two); the diagonal inverses are exact fp32 substitutions.
//
// Layout: wave w holds state-row tile w (rows 16 w .. 16 w + 15 of M_mem, M_k, M_v, M_q) in
// registers, in the B-operand layout of a 16x16 tile: lane 16 g + c holds
// S[16 w + c][16 n + 4 g + i] for column tile n.  Waves 0 .. NT-1 (the M_mem rows) read out;
// the last NT waves solve for W, one 16-column tile each.
#include <algorithm>

#include "device_common.h"
#include "kernels.h"
#include "mfma_ops.h"

namespace hope {
namespace {

// Contraction over the head dimension: one 16x16x16 step at d = 16, one 16x16x32 step at
// d = 32, two at d = 64.
template <int D>
struct HeadOps;
template <>
struct HeadOps<32> {
  typedef bf16x8 V;
  static __device__ __forceinline__ V row(const unsigned short* r, int g) { return load_row_pair_bf16(r, 0, g); }
  static __device__ __forceinline__ void split(const f32x4* s, V& hi, V& lo) { split8(s[0], s[1], hi, lo); }
  static __device__ __forceinline__ f32x4 mma(V a, V b, f32x4 c) { return mma32(a, b, c); }
  static __device__ __forceinline__ f32x4 mma3(V ah, V al, V bh, V bl, f32x4 c) { return mma32x3(ah, al, bh, bl, c); }
};
// d = 64: two 32-deep steps (column tiles 0-1, then 2-3)
struct Bf16x8x2 {
  bf16x8 s[2];
};
template <>
struct HeadOps<64> {
  typedef Bf16x8x2 V;
  static __device__ __forceinline__ V row(const unsigned short* r, int g) {
    return V{{load_row_pair_bf16(r, 0, g), load_row_pair_bf16(r, 1, g)}};
  }
  static __device__ __forceinline__ void split(const f32x4* s, V& hi, V& lo) {
    split8(s[0], s[1], hi.s[0], lo.s[0]);
    split8(s[2], s[3], hi.s[1], lo.s[1]);
  }
  static __device__ __forceinline__ f32x4 mma(V a, V b, f32x4 c) {
    return mma32(a.s[1], b.s[1], mma32(a.s[0], b.s[0], c));
  }
  static __device__ __forceinline__ f32x4 mma3(V ah, V al, V bh, V bl, f32x4 c) {
    return mma32x3(ah.s[1], al.s[1], bh.s[1], bl.s[1], mma32x3(ah.s[0], al.s[0], bh.s[0], bl.s[0], c));
  }
};
template <>
struct HeadOps<16> {
  typedef bf16x4 V;
  static __device__ __forceinline__ V row(const unsigned short* r, int g) { return load_row_quad_bf16(r, 0, g); }
  static __device__ __forceinline__ void split(const f32x4* s, V& hi, V& lo) { split4(s[0], hi, lo); }
  static __device__ __forceinline__ f32x4 mma(V a, V b, f32x4 c) { return mma16(a, b, c); }
  static __device__ __forceinline__ f32x4 mma3(V ah, V al, V bh, V bl, f32x4 c) { return mma16x3(ah, al, bh, bl, c); }
};

// D head dimension, SEG_ tokens per segment, NW_ waves per chain (one or two per state-row tile)
template <int D, int SEG_, int NW_>
struct ChunkShape {
  static constexpr int NT = D / 16;           // column tiles of the state = solve waves
  static constexpr int MT = D / 4;            // state-row tiles (of the 4D rows)
  static constexpr int NW = NW_;
  static constexpr int RW = NW / MT;          // waves per state-row tile
  static constexpr int SEG = SEG_;
  static constexpr int TMAX = SEG / 16;       // token tiles per segment
  static_assert(NW % MT == 0 && (RW == 1 || (RW == 2 && NT % 2 == 0)), "wave layout");
  static constexpr int XLD = D + 8;           // bf16 stride of token-major rows
  static constexpr int LD = D + 4;            // fp32 stride of token-major rows
  static constexpr int PLD = 3 * D + 4;       // fp32 stride of the projections
  static constexpr int LTLD = 20;             // fp32 stride of the substitution's L copy
};

// LDS carve-up for segments of TT token tiles (the host sizes the launch with the same
// function).  Offsets in bytes, each 16-byte aligned.
struct ChunkLds {
  int xs, pj, ks, dls, kh, kl, qh, ql, kth, ktl, ubh, ubl, gs, alph, stp, pix, p0, sf, sc, pre, suf, tt,
      lts, xch, total;
  int ktld;
};
template <int D>
__host__ __device__ constexpr ChunkLds chunk_lds(int TT, bool multi, bool exchange) {
  typedef ChunkShape<D, 16, D / 4> S;  // (the strides do not depend on the segment or waves)
  ChunkLds L{};
  const int nt = 16 * TT;
  int o = 0;
  auto take = [&o](int bytes) {
    const int at = o;
    o += (bytes + 15) / 16 * 16;
    return at;
  };
  L.ktld = nt + 4;
  L.xs = take(nt * S::XLD * 2);
  // the projections are dead once the gates are written: the L tiles take their place
  const int nl = TT * (TT + 1) / 2;
  const int pj_bytes = nt * S::PLD * 4, lt_bytes = nl * 64 * 16;
  L.pj = take(pj_bytes > lt_bytes ? pj_bytes : lt_bytes);
  // normalised keys and delta, column-major (stride nt + 4): the right-hand side reads four
  // consecutive tokens of a column at once
  L.ks = take(D * (nt + 4) * 4);
  L.dls = take(D * (nt + 4) * 4);
  L.kh = take(nt * S::XLD * 2);
  L.kl = take(nt * S::XLD * 2);
  L.qh = take(nt * S::XLD * 2);
  L.ql = take(nt * S::XLD * 2);
  L.kth = take(D * L.ktld * 2);
  L.ktl = take(D * L.ktld * 2);
  L.ubh = take(nt * S::XLD * 2);
  L.ubl = take(nt * S::XLD * 2);
  L.alph = take(nt * 4);
  L.stp = take(nt * 4);
  L.pix = take(nt * 4);
  L.p0 = take(nt * 4);
  L.sf = take(nt * 4);
  L.sc = take(4 * nt * 4);
  L.pre = take(nt * 4);
  L.suf = take(nt * 4);
  L.tt = take(16 * 4);
  L.lts = take(TT * 16 * S::LTLD * 4);
  // two waves per state-row tile: their partial carries meet here at each chunk end
  L.xch = take(exchange ? 2 * S::MT * S::NT * 64 * 16 : 16);
  L.gs = take(multi ? D * S::LD * 4 : 16);  // last: the gain of multi-segment chunks
  L.total = o;
  return L;
}

// Register budgets of the throughput-bound launches: the one-tile d = 16 launches (the
// block's operator, thousands of four-wave chains) are held to 72 registers, seven chains per
// CU; the eight-wave d = 32 launches with up to three token tiles to 128, two chains per CU
// (four tiles would spill)
// VAR: 0 the default operator, 1 every variant option, 2 only those of the VisionHOPE block
// (skip, direction scales, given queries: fewer live scalars, no register spills)
template <int D, int SEG_, int NW_, int TT, int VAR>
__global__ __launch_bounds__(64 * NW_, (D == 16 && SEG_ == 16) ? 7 : (D == 32 && NW_ == 8 && TT <= 3) ? 4 : 1) void chain_chunk_kernel(ChainParams p, int multi) {
  typedef ChunkShape<D, SEG_, NW_> S;
  typedef HeadOps<D> Ops;
  typedef typename Ops::V V;
  constexpr int NT = S::NT, NW = S::NW, MT = S::MT, RW = S::RW, SEG = S::SEG, TMAX = S::TMAX;
  constexpr int XLD = S::XLD, LD = S::LD, PLD = S::PLD, LTLD = S::LTLD;
  constexpr int kThreads = 64 * NW;
  constexpr int SW0 = NW - NT;  // first solve wave
  constexpr int TR = 4 * D;     // first gate row (m_eta, then m_alpha) of the flat state

  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  // TT (token tiles per segment) is a compile-time constant, so every LDS offset below is
  // one too (immediate offsets of the LDS instructions); the gain area sits last
  constexpr ChunkLds Lo = chunk_lds<D>(TT, true, RW > 1);
  unsigned short* const Xs = reinterpret_cast<unsigned short*>(lds + Lo.xs);
  float* const Pj = reinterpret_cast<float*>(lds + Lo.pj);
  u32x4* const Lt = reinterpret_cast<u32x4*>(lds + Lo.pj);  // [tile pair][lane]: hi bf16x4, lo bf16x4
  float* const Ks = reinterpret_cast<float*>(lds + Lo.ks);
  float* const Dls = reinterpret_cast<float*>(lds + Lo.dls);
  unsigned short* const KH = reinterpret_cast<unsigned short*>(lds + Lo.kh);
  unsigned short* const KL = reinterpret_cast<unsigned short*>(lds + Lo.kl);
  unsigned short* const QH = reinterpret_cast<unsigned short*>(lds + Lo.qh);
  unsigned short* const QL = reinterpret_cast<unsigned short*>(lds + Lo.ql);
  unsigned short* const KtH = reinterpret_cast<unsigned short*>(lds + Lo.kth);
  unsigned short* const KtL = reinterpret_cast<unsigned short*>(lds + Lo.ktl);
  unsigned short* const UbH = reinterpret_cast<unsigned short*>(lds + Lo.ubh);
  unsigned short* const UbL = reinterpret_cast<unsigned short*>(lds + Lo.ubl);
  float* const Gs = reinterpret_cast<float*>(lds + Lo.gs);
  float* const alph = reinterpret_cast<float*>(lds + Lo.alph);
  float* const stp = reinterpret_cast<float*>(lds + Lo.stp);
  int* const pixs = reinterpret_cast<int*>(lds + Lo.pix);
  float* const P0s = reinterpret_cast<float*>(lds + Lo.p0);  // P(0, t) from the segment start
  float* const Sfs = reinterpret_cast<float*>(lds + Lo.sf);  // P(t+1, n) to the segment end
  float* const Sc = reinterpret_cast<float*>(lds + Lo.sc);    // per token: |k|^2, |delta|^2, s_eta, s_alpha
  float* const pre_ex = reinterpret_cast<float*>(lds + Lo.pre);  // prod of alpha before t, within its tile
  float* const suf_ex = reinterpret_cast<float*>(lds + Lo.suf);  // prod of alpha after t, within its tile
  float* const Tt = reinterpret_cast<float*>(lds + Lo.tt);    // prod of alpha over each tile
  float* const LTs = reinterpret_cast<float*>(lds + Lo.lts);
  constexpr int KTLD = Lo.ktld;
  constexpr int KSLD = 16 * TT + 4;  // fp32 stride of the column-major keys and delta
  // the two gate rows (m_eta, m_alpha): Tb[cur] the chunk-start copy, Tb[cur ^ 1] the running one
  __shared__ __attribute__((aligned(16))) float Tb[2][2 * D];
  __shared__ unsigned int cnt_lds[3];

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
  // the skip, direction-scale and query pointers are kept in LDS and read where used: held
  // in scalar registers across the loop they would spill (these kernels are at the scalar
  // register limit)
  __shared__ const void* vptr[3];
  const bool has_skip = VAR && p.skip, has_scales = VAR && p.route_scales;
  unsigned long long* const v_counts = VAR == 1 ? p.counts : nullptr;
  float* const v_steps = VAR == 1 ? p.steps : nullptr;
  const bool has_q = VAR && p.queries;
  const unsigned v_frozen = VAR == 1 ? (p.frozen | (p.queries ? 4u : 0u)) : (VAR && p.queries ? 4u : 0u);
  const bool v_nodgd = VAR == 1 && p.no_dgd;
  const GateParams gp{p.eta_map, p.eta_scale, p.alpha_bias, p.eps, VAR == 1 ? p.injection : 0,
                      VAR == 1 ? p.spectral : 0};
  const int m = w % MT, u = w / MT;  // this wave's state-row tile, and its share of the tile's work
  // row tiles held fixed within the image: M_k, M_v (bit 0) and M_q (bit 2)
  const bool my_tile_frozen = ((v_frozen & 1u) && m >= NT && m < 3 * NT) || ((v_frozen & 4u) && m >= 3 * NT);
  const bool gates_frozen = (v_frozen & 2u) != 0;
  float* dst = slot == 0 ? p.out : p.planes + (int64_t)(slot - 1) * p.plane_stride;
  const unsigned short* xg = static_cast<const unsigned short*>(p.x);

  // pixel of token t of this route (exact integers; the map of route_pixel)
  auto pixel_of = [&](int t) {
    if (r & 1) t = N - 1 - t;
    if (r < 2) return t;
    const int q = t / H;
    return (t - q * H) * W + q;
  };

  // ---- state in registers -------------------------------------------------------------
  f32x4 St[NT];    // the chunk-start state S_b of this row tile
  f32x4 Acc[NT];   // S_b G_s, the state after the chunk's earlier segments; with two waves per
                   // row tile each carries its own token tiles' share (the two shares sum to it)
  // At d = 32 one wave per row tile keeps the two shares apart too (Acc2: the odd token tiles)
  // and adds them in the same order, so that 8 and 16 waves per chain (chosen by the number
  // of chains in the call) give bitwise the same result
  constexpr bool kTwoShares = D == 32 && RW == 1;
  f32x4 Acc2[kTwoShares ? NT : 1];
  {
    const float* init = p.init + init_offset(p, b, r, h, SS);
    const int row = 16 * m + c16;
#pragma unroll
    for (int n = 0; n < NT; ++n) St[n] = *reinterpret_cast<const f32x4*>(init + row * D + 16 * n + 4 * g);
    for (int i = threadIdx.x; i < 2 * D; i += kThreads) Tb[0][i] = init[TR * D + i];
    if (threadIdx.x < 3) cnt_lds[threadIdx.x] = 0u;
    if (VAR && threadIdx.x == 0) {
      vptr[0] = p.skip;
      vptr[1] = p.route_scales;
      vptr[2] = p.queries;
    }
  }
  int cur = 0;

  // tokens are fetched one segment ahead: 16-byte loads (8 channels) by the last threads
  constexpr int kLoaders = SEG * D / 8;
  constexpr int kLoad0 = kThreads - kLoaders;
  static_assert(kLoad0 >= 0, "one 16-byte load per loader thread");
  auto fetch = [&](int a0, int n) {
    const int li = threadIdx.x - kLoad0;
    const int lt = li / (D / 8), lc = li % (D / 8);
    u32x4 v = {0u, 0u, 0u, 0u};
    if (li >= 0 && lt < n)
      v = *reinterpret_cast<const u32x4*>(xg + ((int64_t)b * N + pixel_of(a0 + lt)) * Dt + (int64_t)h * D + lc * 8);
    return v;
  };
  auto stage = [&](const u32x4& v, int a0, int n) {
    const int li = threadIdx.x - kLoad0;
    if (li >= 0) {
      const int lt = li / (D / 8), lc = li % (D / 8);
      if (lt < 16 * TT) *reinterpret_cast<u32x4*>(Xs + lt * XLD + lc * 8) = v;
    }
    for (int t = threadIdx.x; t < 16 * TT; t += kThreads) pixs[t] = t < n ? pixel_of(a0 + t) : 0;
  };
  // the segment after the one at a0 (chunk [s0, s1)): start and length, length 0 past the end
  auto next_seg = [&](int a0, int s1, int& an, int& nn) {
    if (a0 + SEG < s1) {
      an = a0 + SEG;
      nn = min(SEG, s1 - an);
    } else {
      an = s1;
      nn = s1 < N ? min(SEG, min(C, N - s1)) : 0;
    }
  };
  u32x4 pf;
  {
    const int n0 = min(SEG, min(C, N));
    stage(fetch(0, n0), 0, n0);
    int an, nn;
    next_seg(0, min(C, N), an, nn);
    pf = fetch(an, nn);
  }
  lds_barrier();

  V Sh, Sl;  // hi/lo split of the chunk-start state (constant over the chunk)
  for (int s0 = 0; s0 < N; s0 += C) {
    const int s1 = min(s0 + C, N);
    Ops::split(St, Sh, Sl);
#pragma unroll
    for (int n = 0; n < NT; ++n) Acc[n] = (RW == 1 || u == 0) ? St[n] : f32x4{0.f, 0.f, 0.f, 0.f};
    if (kTwoShares) {
#pragma unroll
      for (int n = 0; n < NT; ++n) Acc2[kTwoShares ? n : 0] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    for (int a0 = s0; a0 < s1; a0 += SEG) {
      const int ns = min(SEG, s1 - a0);   // tokens in this segment
      // Every segment runs TT token tiles, the launch's maximum: tokens from ns on are
      // padding (no key, no write, unit retention), so a shorter segment costs the work of a
      // full one, and every tile loop below has a compile-time trip count (straight-line
      // code whose LDS reads the compiler can issue ahead of their uses)
      constexpr int TS = TT;
      const bool first = a0 == s0;
      const bool last = a0 + SEG >= s1;
      // lane indices re-derived through an opaque copy each segment: the address arithmetic
      // built on them is recomputed per segment instead of being hoisted out of the loops
      // and held in registers across every phase
      int lid = threadIdx.x;
      asm volatile("" : "+v"(lid));
      const int lane = lid & 63, c16 = lid & 15, g = (lid >> 4) & 3;

      // ---- A: projections P[t][row] = x_t . S_b[row] for the k, v, q and gate rows ----
      if (m >= NT && !(has_q && m >= 3 * NT)) {
#pragma unroll
        for (int tau = 0; tau < TMAX; ++tau) {
          if (tau >= TS) break;
          if (RW > 1 && tau % RW != u) continue;
          const V xa = Ops::row(Xs + (16 * tau + c16) * XLD, g);
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
          acc = Ops::mma(xa, Sl, acc);
          acc = Ops::mma(xa, Sh, acc);
#pragma unroll
          for (int i = 0; i < 4; ++i) Pj[(16 * tau + 4 * g + i) * PLD + 16 * m + c16 - D] = acc[i];
        }
      }
      if (m == 0) {  // gate rows: lanes c16 < 2 carry m_eta, m_alpha, the others zero
        f32x4 tv[NT];
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          const f32x4 z = {0.f, 0.f, 0.f, 0.f};
          tv[n] = c16 < 2 ? *reinterpret_cast<const f32x4*>(Tb[cur] + c16 * D + 16 * n + 4 * g) : z;
        }
        V th, tl;
        Ops::split(tv, th, tl);
#pragma unroll
        for (int tau = 0; tau < TMAX; ++tau) {
          if (tau >= TS) break;
          if (RW > 1 && tau % RW != u) continue;
          const V xa = Ops::row(Xs + (16 * tau + c16) * XLD, g);
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
          acc = Ops::mma(xa, tl, acc);
          acc = Ops::mma(xa, th, acc);
          if (c16 < 2) {
#pragma unroll
            for (int i = 0; i < 4; ++i) Pj[(16 * tau + 4 * g + i) * PLD + 3 * D + c16] = acc[i];
          }
        }
      }
      lds_barrier();

      // ---- B: normalisation; 16 lanes (a DPP row) per token, each holding D / 16 components:
      // normalised k and q, delta = k - v, and the token's scalars for the step control
      {
        constexpr int CPL = D / 16;
        for (int t = 4 * w + g; t < 16 * TS; t += 4 * NW) {
          const bool live = t < ns;
          const float* pt = Pj + t * PLD + c16 * CPL;
          float kr[CPL], vr[CPL], qr[CPL];
          float kk = 0.f, qq = 0.f;
#pragma unroll
          for (int e = 0; e < CPL; ++e) {
            kr[e] = pt[e];
            vr[e] = pt[D + e];
            if (!has_q) {
              qr[e] = pt[2 * D + e];
            } else {
              const int64_t qi = ((int64_t)b * N + pixs[t]) * Dt + (int64_t)h * D + c16 * CPL + e;
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
          const float kk2 = kk_all * kinv * kinv;  // |k|^2 of the normalised key
          dd = row16_sum(dd);
          if (c16 == 0) {
            Sc[t] = kk2;
            Sc[16 * TT + t] = dd;
            Sc[32 * TT + t] = pt[3 * D];
            Sc[48 * TT + t] = pt[3 * D + 1];
          }
          if constexpr (CPL >= 2) {
            // consecutive components in pairs: one 8-byte store per fp32 row and one 4-byte
            // store per bf16 row (only the transposed key copy stays 2-byte)
            typedef float f32x2v __attribute__((ext_vector_type(2)));
#pragma unroll
            for (int e = 0; e < CPL; e += 2) {
              const int col = c16 * CPL + e;
              // padding tokens have x = 0: k and delta are exactly zero; only queries read
              // from the map need the mask
              const bool qlive = live || !has_q;
              const float k0 = kn[e], k1 = kn[e + 1];
              const float q0 = qlive ? qn[e] : 0.f, q1 = qlive ? qn[e + 1] : 0.f;
              Ks[col * KSLD + t] = k0;
              Ks[(col + 1) * KSLD + t] = k1;
              Dls[col * KSLD + t] = dl[e];
              Dls[(col + 1) * KSLD + t] = dl[e + 1];
              unsigned kh, kl, qh, ql;
              split_pair(k0, k1, kh, kl);
              split_pair(q0, q1, qh, ql);
              *reinterpret_cast<unsigned*>(KH + t * XLD + col) = kh;
              *reinterpret_cast<unsigned*>(KL + t * XLD + col) = kl;
              *reinterpret_cast<unsigned*>(QH + t * XLD + col) = qh;
              *reinterpret_cast<unsigned*>(QL + t * XLD + col) = ql;
              KtH[col * KTLD + t] = (unsigned short)kh;
              KtH[(col + 1) * KTLD + t] = (unsigned short)(kh >> 16);
              KtL[col * KTLD + t] = (unsigned short)kl;
              KtL[(col + 1) * KTLD + t] = (unsigned short)(kl >> 16);
            }
          } else {
            const int col = c16;
            const float k0 = kn[0], q0 = (live || !has_q) ? qn[0] : 0.f;
            Ks[col * KSLD + t] = k0;
            Dls[col * KSLD + t] = dl[0];
            const __bf16 khv = (__bf16)k0, qhv = (__bf16)q0;
            const __bf16 klv = (__bf16)(k0 - (float)khv), qlv = (__bf16)(q0 - (float)qhv);
            const unsigned short khb = __builtin_bit_cast(unsigned short, khv);
            const unsigned short klb = __builtin_bit_cast(unsigned short, klv);
            KH[t * XLD + col] = khb;
            KL[t * XLD + col] = klb;
            QH[t * XLD + col] = __builtin_bit_cast(unsigned short, qhv);
            QL[t * XLD + col] = __builtin_bit_cast(unsigned short, qlv);
            KtH[col * KTLD + t] = khb;
            KtL[col * KTLD + t] = klb;
          }
        }
      }
      lds_barrier();

      // ---- B2: the executed step (Eq. 19-20) and the retention products, one token per lane
      // on wave 0 (a DPP row is a 16-token tile); the other waves form their token Gram tiles
      // G'[4g+i][c] = k_{16J+4g+i} . k_{16I+c} for tile pairs (I >= J), q = I (I + 1) / 2 + J,
      // dealt round robin to the "pair waves" (rank pw): waves 1 .. NW-1, or, in the 8-wave
      // launches, the waves that hold no M_mem rows, which then read out during C1 (measured:
      // faster there, slower in the 16-wave launches)
      const int npairs = v_nodgd ? 0 : TS * (TS + 1) / 2;
      constexpr bool kReadC1 = RW == 1 && NW == 8;
      constexpr int kPairWaves = kReadC1 ? MT - NT : NW - 1;
      const int pw = kReadC1 ? (m >= NT ? m - NT : -1) : w - 1;
      constexpr int kMaxPairsPerWave = (TMAX * (TMAX + 1) / 2 + kPairWaves - 1) / kPairWaves;
      f32x4 gram[kMaxPairsPerWave];
      if (w == 0) {
#pragma unroll
        for (int ps = 0; ps < (TMAX + 3) / 4; ++ps) {
          const int t = 64 * ps + lane, tile = 4 * ps + g;
          const bool live = t < ns;
          float alpha = 1.f, step = 0.f;
          if (tile < TS) {
            StepFlags sf;
            step = executed_step(Sc[t], Sc[16 * TT + t], Sc[32 * TT + t], Sc[48 * TT + t], gp, &alpha, &sf);
            if (v_counts && live) {
              atomicAdd(&cnt_lds[0], 1u);
              atomicAdd(&cnt_lds[1], (unsigned)(sf.bits & 1));
              atomicAdd(&cnt_lds[2], (unsigned)((sf.bits >> 1) & 1));
            }
            if (v_steps && live) v_steps[(((int64_t)b * 4 + r) * p.nh + h) * ((int64_t)p.H * p.W) + pixs[t]] = step;
            if (!live) {
              alpha = 1.f;
              step = 0.f;
            }
            alph[t] = alpha;
            stp[t] = step;
          }
          // exclusive prefix and suffix products of alpha within the tile (lanes past the
          // row ends count as 1), and the tile's total from its last lane
          const int one = __builtin_bit_cast(int, 1.f);
          const float a_prev = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(one, __builtin_bit_cast(int, alpha), 0x111, 0xF, 0xF, false));
          const float a_next = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(one, __builtin_bit_cast(int, alpha), 0x101, 0xF, 0xF, false));
          const float pre = row16_prefix_prod(a_prev);
          const float suf = row16_suffix_prod(a_next);
          if (tile < TS) {
            pre_ex[t] = pre;
            suf_ex[t] = suf;
            if (c16 == 15) Tt[tile] = pre * alpha;
          }
        }
      } else {
#pragma unroll
        for (int k = 0; k < kMaxPairsPerWave; ++k) {
          const int q = pw + k * kPairWaves;
          if (pw < 0 || q >= npairs) break;
          int I = 0;
          while ((I + 1) * (I + 2) / 2 <= q) ++I;
          const int J = q - I * (I + 1) / 2;
          const V ah = Ops::row(KH + (16 * J + c16) * XLD, g), al = Ops::row(KL + (16 * J + c16) * XLD, g);
          const V bh = Ops::row(KH + (16 * I + c16) * XLD, g), bl = Ops::row(KL + (16 * I + c16) * XLD, g);
          gram[k] = Ops::mma3(ah, al, bh, bl, f32x4{0.f, 0.f, 0.f, 0.f});
        }
      }
      lds_barrier();

      // per-tile totals: the segment's retention and the products between tiles
      float tot[TMAX];
#pragma unroll
      for (int j = 0; j < TMAX; ++j) tot[j] = j < TS ? Tt[j] : 1.f;
      auto tiles_prod = [&](int lo, int hi) {
        float q = 1.f;
#pragma unroll
        for (int j = 0; j < TMAX; ++j)
          if (j >= lo && j < hi) q *= tot[j];
        return q;
      };
      const float cseg = tiles_prod(0, TS);
      // per-token retention factors for the solve and the carry
      if (w == 0) {
        for (int t = lane; t < 16 * TS; t += 64) {
          const int tile = t >> 4;
          P0s[t] = tiles_prod(0, tile) * pre_ex[t];
          Sfs[t] = suf_ex[t] * tiles_prod(tile + 1, TS);
        }
      }

      // ---- C1: the L tiles (negated, in the A layout, hi/lo) and the diagonal inverses on
      // the pair waves; the readout on the M_mem waves ----
      if (pw >= 0) {
#pragma unroll
        for (int k = 0; k < kMaxPairsPerWave; ++k) {
          const int q = pw + k * kPairWaves;
          if (q >= npairs) break;
          int I = 0;
          while ((I + 1) * (I + 2) / 2 <= q) ++I;
          const int J = q - I * (I + 1) / 2;
          const f32x4 gr = gram[k];
          const float st_t = stp[16 * I + c16];  // step of this lane's row t = 16 I + c
          f32x4 lv;                              // L[t = 16I + c][j = 16J + 4g + i]
          if (I > J) {
            const float rowf = st_t * pre_ex[16 * I + c16] * tiles_prod(J + 1, I);
#pragma unroll
            for (int i = 0; i < 4; ++i) lv[i] = rowf * suf_ex[16 * J + 4 * g + i] * gr[i];
            bf16x4 hi, lo;
            split4(-lv, hi, lo);
            const u32x2 h2 = __builtin_bit_cast(u32x2, hi), l2 = __builtin_bit_cast(u32x2, lo);
            Lt[q * 64 + lane] = u32x4{h2[0], h2[1], l2[0], l2[1]};
          } else {
            // P(j+1, t) within the tile: prefix over lanes of alpha_{s-1} for s >= j + 2
            const int tt = 16 * I + c16;
            const float a_prev = c16 >= 1 ? alph[tt - 1] : 1.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int j = 4 * g + i;
              const float pjt = row16_prefix_prod(c16 >= j + 2 ? a_prev : 1.f);
              lv[i] = j < c16 ? st_t * pjt * gr[i] : 0.f;
            }
            // T = (I + L)^-1 by forward substitution: a quad of lanes per column of T, quad
            // lane qd holding rows qd, qd + 4, qd + 8, qd + 12; L copied so that one 16-byte
            // read gives a lane its four coefficients of column j
            float* const LTw = LTs + J * (16 * LTLD);
            __builtin_amdgcn_s_setprio(2);  // the inverses end the phase: let them issue first
#pragma unroll
            for (int i = 0; i < 4; ++i) LTw[(4 * g + i) * LTLD + 4 * (c16 & 3) + (c16 >> 2)] = lv[i];
            const int col = lane >> 2, qd = lane & 3;
            float uu[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) uu[i] = (4 * i + qd == col) ? 1.f : 0.f;
            // coefficient rows are read kPf steps ahead of their use, so that the steps wait
            // on one another rather than on LDS (all of them at d = 32, whose launches are
            // latency-bound; four elsewhere, within the register budget)
            constexpr int kPf = D == 32 ? 15 : 4;
            f32x4 cfs[kPf];
#pragma unroll
            for (int j = 0; j < kPf; ++j) cfs[j] = *reinterpret_cast<const f32x4*>(LTw + j * LTLD + 4 * qd);
#pragma unroll
            for (int j = 0; j < 15; ++j) {
              const f32x4 cf = cfs[j % kPf];
              if (j + kPf < 15) cfs[j % kPf] = *reinterpret_cast<const f32x4*>(LTw + (j + kPf) * LTLD + 4 * qd);
              const float uj = quad_bcast(uu[j >> 2], j & 3);
              // (L is zero on and above its diagonal: rows t <= j subtract an exact zero)
#pragma unroll
              for (int i = j >> 2; i < 4; ++i) uu[i] = fmaf(-cf[i], uj, uu[i]);
            }
            // back through LDS into the A layout: lane (g, c) takes T[c][4g + i]
#pragma unroll
            for (int i = 0; i < 4; ++i) LTw[(4 * i + qd) * LTLD + col] = uu[i];
            const f32x4 tv = *reinterpret_cast<const f32x4*>(LTw + c16 * LTLD + 4 * g);
            bf16x4 hi, lo;
            split4(tv, hi, lo);
            const u32x2 h2 = __builtin_bit_cast(u32x2, hi), l2 = __builtin_bit_cast(u32x2, lo);
            Lt[q * 64 + lane] = u32x4{h2[0], h2[1], l2[0], l2[1]};
            __builtin_amdgcn_s_setprio(0);
          }
        }
      }
      // readout y_t = M_mem,b q_t for this wave's 16 rows of M_mem (the M_mem waves)
      auto readout = [&]() {
        const int64_t c = (int64_t)h * D + 16 * m + c16;
        const float skip_c = has_skip ? static_cast<const float*>(vptr[0])[c] : 0.f;
        const float scale_c = has_scales ? static_cast<const float*>(vptr[1])[(int64_t)r * Dt + c] : 1.f;
#pragma unroll
        for (int tau = 0; tau < TMAX; ++tau) {
          if (tau >= TS) break;
          if (RW > 1 && tau % RW != u) continue;
          const V qh = Ops::row(QH + (16 * tau + c16) * XLD, g), ql = Ops::row(QL + (16 * tau + c16) * XLD, g);
          const f32x4 y = Ops::mma3(qh, ql, Sh, Sl, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int t = 16 * tau + 4 * g + i;
            if (t < ns) {
              float yv = y[i];
              if (has_skip) yv = fmaf(skip_c, __uint_as_float((unsigned)Xs[t * XLD + 16 * m + c16] << 16), yv);
              if (has_scales) yv *= scale_c;
              dst[((int64_t)b * N + pixs[t]) * Dt + c] = yv;
            }
          }
        }
      };
      if (kReadC1 && m < NT) readout();
      lds_barrier();

      // ---- C2: the write vectors (solve waves) -------------------------------------------
      if (w >= SW0) {
        __builtin_amdgcn_s_setprio(3);  // the segment's critical path
        const int n = w - SW0;          // this wave's 16 columns of W
        f32x4 R[TMAX];
        // G_s k_t on the matrix cores for a later segment of the chunk (G_s = I otherwise)
        const bool gk_mfma = multi && !first && !v_nodgd;
        V gh, gl;
        if (gk_mfma) {
          f32x4 gv[NT];
#pragma unroll
          for (int e = 0; e < NT; ++e) gv[e] = *reinterpret_cast<const f32x4*>(Gs + (16 * n + c16) * LD + 16 * e + 4 * g);
          Ops::split(gv, gh, gl);
        }
        // (the wave-uniform choice is taken once, outside the loops, so that each form is
        // straight-line code)
        if (gk_mfma) {
#pragma unroll
          for (int tau = 0; tau < TMAX; ++tau) {
            if (tau >= TS) break;
            const V kh = Ops::row(KH + (16 * tau + c16) * XLD, g), kl = Ops::row(KL + (16 * tau + c16) * XLD, g);
            const f32x4 gk = Ops::mma3(kh, kl, gh, gl, f32x4{0.f, 0.f, 0.f, 0.f});
            const int t0 = 16 * tau + 4 * g;
            const f32x4 st4 = *reinterpret_cast<const f32x4*>(stp + t0), p04 = *reinterpret_cast<const f32x4*>(P0s + t0);
            const f32x4 dv = *reinterpret_cast<const f32x4*>(Dls + (16 * n + c16) * KSLD + t0);
#pragma unroll
            for (int i = 0; i < 4; ++i) R[tau][i] = -st4[i] * fmaf(p04[i], gk[i], dv[i]);
          }
        } else {
#pragma unroll
          for (int tau = 0; tau < TMAX; ++tau) {
            if (tau >= TS) break;
            const int t0 = 16 * tau + 4 * g;
            const f32x4 st4 = *reinterpret_cast<const f32x4*>(stp + t0), p04 = *reinterpret_cast<const f32x4*>(P0s + t0);
            const f32x4 kv = *reinterpret_cast<const f32x4*>(Ks + (16 * n + c16) * KSLD + t0);
            const f32x4 dv = *reinterpret_cast<const f32x4*>(Dls + (16 * n + c16) * KSLD + t0);
#pragma unroll
            for (int i = 0; i < 4; ++i) R[tau][i] = -st4[i] * fmaf(p04[i], v_nodgd ? 0.f : kv[i], dv[i]);
          }
        }
        // W_J = T_JJ R_J, then R_I -= L_IJ W_J for the later tiles; W_J replaces R_J
        if (!v_nodgd) {
          // the tiles on the dependent chain (T_JJ and L_{J+1,J}) are read a step ahead
          const u32x4 zq = {0u, 0u, 0u, 0u};
          u32x4 tq_n = Lt[lane];
          u32x4 lq_n = TS > 1 ? Lt[64 + lane] : zq;
#pragma unroll
          for (int J = 0; J < TMAX; ++J) {
            if (J >= TS) break;
            const u32x4 tq = tq_n, lq1 = lq_n;
            if (J + 1 < TS) tq_n = Lt[((J + 1) * (J + 2) / 2 + J + 1) * 64 + lane];
            if (J + 2 < TS) lq_n = Lt[((J + 2) * (J + 3) / 2 + J + 1) * 64 + lane];
            bf16x4 rh, rl;
            split4(R[J], rh, rl);
            const bf16x4 th = __builtin_bit_cast(bf16x4, u32x2{tq[0], tq[1]});
            const bf16x4 tl = __builtin_bit_cast(bf16x4, u32x2{tq[2], tq[3]});
            R[J] = mma16x3(th, tl, rh, rl, f32x4{0.f, 0.f, 0.f, 0.f});
            bf16x4 wh, wl;
            split4(R[J], wh, wl);
#pragma unroll
            for (int I = J + 1; I < TMAX; ++I) {
              if (I >= TS) break;
              const u32x4 lq = I == J + 1 ? lq1 : Lt[(I * (I + 1) / 2 + J) * 64 + lane];
              R[I] = mma16x3(__builtin_bit_cast(bf16x4, u32x2{lq[0], lq[1]}),
                             __builtin_bit_cast(bf16x4, u32x2{lq[2], lq[3]}), wh, wl, R[I]);
            }
          }
        }
        // Ub_t = P(t+1, n) w_t, token-major hi/lo for the carry
#pragma unroll
        for (int J = 0; J < TMAX; ++J) {
          if (J >= TS) break;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int t = 16 * J + 4 * g + i;
            const float ub = Sfs[t] * R[J][i];
            const __bf16 uh = (__bf16)ub;
            UbH[t * XLD + 16 * n + c16] = __builtin_bit_cast(unsigned short, uh);
            UbL[t * XLD + 16 * n + c16] = __builtin_bit_cast(unsigned short, (__bf16)(ub - (float)uh));
          }
        }
        __builtin_amdgcn_s_setprio(0);
      } else if (!kReadC1 && m < NT) {
        readout();
      }
      lds_barrier();

      // ---- D: carry  S_b G_e = cseg (S_b G_s) + (S_b Ub^T) K, per token tile ----------
      if (!my_tile_frozen) {
        // this wave's token tiles: tau = u (mod RW)
        f32x4 acc[NT], acc2[kTwoShares ? NT : 1];
#pragma unroll
        for (int n = 0; n < NT; ++n) acc[n] = Acc[n] * cseg;
        if (kTwoShares) {
#pragma unroll
          for (int n = 0; n < NT; ++n) acc2[kTwoShares ? n : 0] = Acc2[kTwoShares ? n : 0] * cseg;
        }
#pragma unroll
        for (int tau = 0; tau < TMAX; ++tau) {
          if (tau >= TS) break;
          if (RW > 1 && tau % RW != u) continue;
          f32x4* const share = (kTwoShares && (tau & 1)) ? acc2 : acc;
          // Z^T[t][row] = Ub_t . S_b[row]
          const V uh = Ops::row(UbH + (16 * tau + c16) * XLD, g), ul = Ops::row(UbL + (16 * tau + c16) * XLD, g);
          const f32x4 z = Ops::mma3(uh, ul, Sh, Sl, f32x4{0.f, 0.f, 0.f, 0.f});
          bf16x4 zh, zl;
          split4(z, zh, zl);
#pragma unroll
          for (int n = 0; n < NT; ++n) {
            const bf16x4 kh = __builtin_bit_cast(bf16x4, *reinterpret_cast<const u32x2*>(KtH + (16 * n + c16) * KTLD + 16 * tau + 4 * g));
            const bf16x4 kl = __builtin_bit_cast(bf16x4, *reinterpret_cast<const u32x2*>(KtL + (16 * n + c16) * KTLD + 16 * tau + 4 * g));
            share[n] = mma16x3(kh, kl, zh, zl, share[n]);
          }
        }
#pragma unroll
        for (int n = 0; n < NT; ++n) Acc[n] = acc[n];
        if (kTwoShares) {
#pragma unroll
          for (int n = 0; n < NT; ++n) Acc2[kTwoShares ? n : 0] = acc2[kTwoShares ? n : 0];
        }
      }
      // gate rows: the M_mem waves each update column tile w (rows m_eta, m_alpha in lanes
      // c16 < 2 of the accumulator layout)
      if (w < NT && !gates_frozen) {
        const float* run = first ? Tb[cur] : Tb[cur ^ 1];
        f32x4 tv[NT];
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          const f32x4 zz = {0.f, 0.f, 0.f, 0.f};
          tv[n] = c16 < 2 ? *reinterpret_cast<const f32x4*>(Tb[cur] + c16 * D + 16 * n + 4 * g) : zz;
        }
        V th, tl;
        Ops::split(tv, th, tl);
        const f32x4 zz = {0.f, 0.f, 0.f, 0.f};
        f32x4 acc = c16 < 2 ? *reinterpret_cast<const f32x4*>(run + c16 * D + 16 * w + 4 * g) : zz;
        acc *= cseg;
        // even and odd token tiles accumulate apart (two independent product chains), then
        // add in that order
        f32x4 acc_odd = zz;
#pragma unroll
        for (int tau = 0; tau < TMAX; ++tau) {
          if (tau >= TS) break;
          const V uh = Ops::row(UbH + (16 * tau + c16) * XLD, g), ul = Ops::row(UbL + (16 * tau + c16) * XLD, g);
          const f32x4 z = Ops::mma3(uh, ul, th, tl, f32x4{0.f, 0.f, 0.f, 0.f});
          bf16x4 zh, zl;
          split4(z, zh, zl);
          const bf16x4 kh = __builtin_bit_cast(bf16x4, *reinterpret_cast<const u32x2*>(KtH + (16 * w + c16) * KTLD + 16 * tau + 4 * g));
          const bf16x4 kl = __builtin_bit_cast(bf16x4, *reinterpret_cast<const u32x2*>(KtL + (16 * w + c16) * KTLD + 16 * tau + 4 * g));
          if (tau & 1) {
            acc_odd = mma16x3(kh, kl, zh, zl, acc_odd);
          } else {
            acc = mma16x3(kh, kl, zh, zl, acc);
          }
        }
        acc += acc_odd;
        // (every wave read the running rows before the barrier above; only this wave
        // writes its column tile)
        if (c16 < 2) *reinterpret_cast<f32x4*>(Tb[cur ^ 1] + c16 * D + 16 * w + 4 * g) = acc;
      }
      // gain of the chunk so far, for the next segment: G <- cseg G + Ub^T K, tiles of 16 x 16
      // dealt from wave NT on, after the waves that carry the gate rows above
      if (multi && !last && !v_nodgd) {
        // (at d = 32 with 16 waves the four tiles go to waves 2, 3, 6 and 7: SIMDs 2 and 3,
        // whose matrix cores do not also carry the gate rows, so the four SIMDs end the carry
        // with equal product counts)
        const int tile0 = (NT == 2 && NW == 16) ? (((w & 3) >= 2 && w < 8) ? (w & 1) + 2 * (w >> 2) : NT * NT)
                                                : (w + NW - NT) % NW;
        for (int tile = tile0; tile < NT * NT; tile += NW) {
          const int ti = tile / NT, tn = tile % NT;
          f32x4 acc;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int gi = 16 * ti + 4 * g + e, gn = 16 * tn + c16;
            acc[e] = first ? (gi == gn ? cseg : 0.f) : cseg * Gs[gi * LD + gn];
          }
          f32x4 acc_odd = {0.f, 0.f, 0.f, 0.f};  // odd token tiles, added at the end
#pragma unroll
          for (int tau = 0; tau < TMAX; ++tau) {
            if (tau >= TS) break;
            // G[16 ti + 4 g + e][16 tn + c] += sum_t Ub[t][16 ti + 4 g + e] K[t][16 tn + c]:
            // A = Ub^T (lane (g, c) supplies row 16 ti + c at tokens 16 tau + 4 g + e, four
            // scattered bf16 reads), B = K (the transposed copy, one 8-byte read)
            unsigned short ah[4], al[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              ah[e] = UbH[(16 * tau + 4 * g + e) * XLD + 16 * ti + c16];
              al[e] = UbL[(16 * tau + 4 * g + e) * XLD + 16 * ti + c16];
            }
            const u32x2 ah2 = {(unsigned)ah[0] | ((unsigned)ah[1] << 16), (unsigned)ah[2] | ((unsigned)ah[3] << 16)};
            const u32x2 al2 = {(unsigned)al[0] | ((unsigned)al[1] << 16), (unsigned)al[2] | ((unsigned)al[3] << 16)};
            const bf16x4 kh = __builtin_bit_cast(bf16x4, *reinterpret_cast<const u32x2*>(KtH + (16 * tn + c16) * KTLD + 16 * tau + 4 * g));
            const bf16x4 kl = __builtin_bit_cast(bf16x4, *reinterpret_cast<const u32x2*>(KtL + (16 * tn + c16) * KTLD + 16 * tau + 4 * g));
            if (tau & 1) {
              acc_odd = mma16x3(__builtin_bit_cast(bf16x4, ah2), __builtin_bit_cast(bf16x4, al2), kh, kl, acc_odd);
            } else {
              acc = mma16x3(__builtin_bit_cast(bf16x4, ah2), __builtin_bit_cast(bf16x4, al2), kh, kl, acc);
            }
          }
          acc += acc_odd;
#pragma unroll
          for (int e = 0; e < 4; ++e) Gs[(16 * ti + 4 * g + e) * LD + 16 * tn + c16] = acc[e];
        }
      }
      // stage the next segment's tokens and request the one after
      {
        int an, nn;
        next_seg(a0, s1, an, nn);
        if (nn > 0) {
          stage(pf, an, nn);
          const int s1n = an == s1 ? min(s1 + C, N) : s1;
          int an2, nn2;
          next_seg(an, s1n, an2, nn2);
          pf = fetch(an2, nn2);
        }
      }
      lds_barrier();
    }
    if (RW > 1) {
      // the two waves of a row tile carried the token tiles of either parity: the state is
      // the sum of their shares, added in the same order by both
      f32x4* const xch = reinterpret_cast<f32x4*>(lds + Lo.xch);
      const int ln = threadIdx.x & 63;
#pragma unroll
      for (int n = 0; n < NT; ++n) xch[((m * RW + u) * NT + n) * 64 + ln] = Acc[n];
      lds_barrier();
#pragma unroll
      for (int n = 0; n < NT; ++n) Acc[n] = xch[((m * RW + 0) * NT + n) * 64 + ln] + xch[((m * RW + 1) * NT + n) * 64 + ln];
    }
    if (kTwoShares) {
#pragma unroll
      for (int n = 0; n < NT; ++n) Acc[n] = Acc[n] + Acc2[kTwoShares ? n : 0];
    }
#pragma unroll
    for (int n = 0; n < NT; ++n) St[n] = Acc[n];
    if (!gates_frozen) cur ^= 1;  // frozen gate rows stay in the chunk-start copy
  }

  if (p.final_mem) {
    float* fin = p.final_mem + (((int64_t)b * 4 + r) * nh + h) * SS;
    const int row = 16 * m + c16;
#pragma unroll
    for (int n = 0; n < NT; ++n) *reinterpret_cast<f32x4*>(fin + row * D + 16 * n + 4 * g) = St[n];
    for (int i = threadIdx.x; i < 2 * D; i += kThreads) fin[TR * D + i] = Tb[cur][i];
  }
  if (v_counts && threadIdx.x < 3) atomicAdd(&v_counts[threadIdx.x], (unsigned long long)cnt_lds[threadIdx.x]);
}

// longest chunk (clipped to the sequence) over the selected routes
int longest_chunk(const ChainParams& p) {
  int cmax = 0;
  for (int s = 0; s < p.n_sel; ++s) {
    const int r = p.route_of_slot[s];
    const int C = p.chunk > 0 ? p.chunk : (r < 2 ? p.W : p.H);
    cmax = std::max(cmax, std::min(C, p.H * p.W));
  }
  return cmax;
}

// LDS bytes and the segment shape of a launch: TT token tiles per segment, and whether some
// chunk spans more than one segment (the gain is then carried between segments)
ChunkLds launch_lds(const ChainParams& p, int d, int seg, bool exchange, int& TT, int& multi) {
  const int cmax = longest_chunk(p);
  TT = (std::min(cmax, seg) + 15) / 16;
  multi = cmax > seg ? 1 : 0;
  if (d == 16) return chunk_lds<16>(TT, multi != 0, exchange);
  if (d == 32) return chunk_lds<32>(TT, multi != 0, exchange);
  return chunk_lds<64>(TT, multi != 0, exchange);
}

constexpr int kChunkLdsMax = 150 * 1024;  // dynamic LDS of one workgroup, at most

template <int D, int SEG, int NW, int TT, int VAR>
hipError_t launch_tt(const ChainParams& p, int multi, int lds_bytes, hipStream_t stream) {
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&chain_chunk_kernel<D, SEG, NW, TT, VAR>),
      hipFuncAttributeMaxDynamicSharedMemorySize, kChunkLdsMax);
  if (attr != hipSuccess) return attr;
  const dim3 grid((unsigned)((int64_t)p.n_sel * p.B * p.nh)), block(64 * NW);
  hipLaunchKernelGGL((chain_chunk_kernel<D, SEG, NW, TT, VAR>), grid, block, lds_bytes, stream, p, multi);
  return hipGetLastError();
}

template <int D, int SEG, int NW, int VAR>
hipError_t launch_cfg(const ChainParams& p, hipStream_t stream) {
  int TT = 0, multi = 0;
  const ChunkLds L = launch_lds(p, D, SEG, NW > D / 4, TT, multi);
  constexpr int TM = SEG / 16;
  switch (TT) {
    case 1: return launch_tt<D, SEG, NW, 1, VAR>(p, multi, L.total, stream);
    case 2: return launch_tt<D, SEG, NW, (TM >= 2 ? 2 : 1), VAR>(p, multi, L.total, stream);
    case 3: return launch_tt<D, SEG, NW, (TM >= 3 ? 3 : 1), VAR>(p, multi, L.total, stream);
    case 4: return launch_tt<D, SEG, NW, (TM >= 4 ? 4 : 1), VAR>(p, multi, L.total, stream);
  }
  return hipErrorInvalidValue;
}

template <int D, int SEG, int NW>
hipError_t launch_v(const ChainParams& p, hipStream_t stream) {
  if (!needs_variants(p)) return launch_cfg<D, SEG, NW, 0>(p, stream);
  const bool block_only = !(p.counts || p.frozen || p.no_dgd || p.injection || p.spectral || p.steps);
  return block_only ? launch_cfg<D, SEG, NW, 2>(p, stream) : launch_cfg<D, SEG, NW, 1>(p, stream);
}

// Segment length of a launch: one 16-token tile at d = 16 when every chunk fits in it (fewer
// registers, more chains per CU), 32 tokens at d = 64 (LDS), else 64 tokens
int segment_of(const ChainParams& p, int d) {
  if (d == 64) return 32;
  return (d == 16 && longest_chunk(p) <= 16) ? 16 : 64;
}

}  // namespace

// Waves per chain at d = 32: two per state-row tile when the chains leave CUs idle (the
// chain's latency bounds the call), one per row tile otherwise (more chains per CU)
int waves_of_d32(const ChainParams& p) {
  return (int64_t)p.n_sel * p.B * p.nh <= 256 ? 16 : 8;
}

bool chunk_path_supported(const ChainParams& p, int d) {
  if (!p.x_bf16 || p.mem_chunk > 0 || p.readout) return false;
  if (d != 16 && d != 32 && d != 64) return false;
  // chunks that fit one 16-token block at d = 32 and 64: the register-resident block
  // kernel is faster there
  if (d == 32 && longest_chunk(p) <= 16) return false;
  if (d == 64 && longest_chunk(p) <= 16) return false;
  int TT = 0, multi = 0;
  return launch_lds(p, d, segment_of(p, d), d == 32, TT, multi).total <= kChunkLdsMax;
}

hipError_t launch_chain_chunk(const ChainParams& p, int d, hipStream_t stream) {
  if (d == 16) {
    return segment_of(p, d) == 16 ? launch_v<16, 16, 4>(p, stream) : launch_v<16, 64, 4>(p, stream);
  }
  if (d == 32) return waves_of_d32(p) == 16 ? launch_v<32, 64, 16>(p, stream) : launch_v<32, 64, 8>(p, stream);
  if (d == 64) return launch_v<64, 32, 16>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace hope
