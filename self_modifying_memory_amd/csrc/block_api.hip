// Host side of the C ABI declared in include/hope_block.h: one VisionHOPE block
// ("VisionHOPE: Visual Backbones as Self-Modifying Learning Systems", Sec. 2.3 Eq. 27 and
// App. B.5) as a fixed sequence of launches on the caller's stream: the conditional
// positional encoding, LayerNorm, the input projection, the gated depthwise branch, the
// query projection, the four-direction operator, the local positional branch, the output
// projection with the residual, LayerNorm, and the FFN with its residual.
#include <string.h>

#include "../../include/hope_block.h"
#include "block_kernels.h"
#include "scan_api.h"

hope_status_t hope_status_of(hipError_t e);

namespace {

constexpr float kLnEps = 1e-5f;

size_t align256(size_t b) { return (b + 255) / 256 * 256; }

bool aligned16(const void* p) { return p && (reinterpret_cast<uintptr_t>(p) % 16) == 0; }

struct BlockLayout {
  size_t r, a, u, z, q, y, y2, h, op, total;  // byte offsets
};

bool sizes_ok(int32_t B, int32_t H, int32_t W, int32_t D, int32_t Dm, int32_t n_heads,
              int32_t ffn_dim, int32_t chunk) {
  if (B <= 0 || H <= 0 || W <= 0 || D <= 0 || Dm <= 0 || n_heads <= 0 || ffn_dim <= 0 || chunk < 0)
    return false;
  if (D % 16 || Dm % 16 || ffn_dim % 16 || Dm % n_heads) return false;
  if (D > 1024 || Dm > 1024 || ffn_dim > 16384) return false;
  const int32_t cmax = D > Dm ? D : Dm;
  // (64-bit throughout: each factor is below 2^31, so no product of two overflows)
  if ((int64_t)B * H > ((int64_t)1 << 31) || (int64_t)B * H * W > ((int64_t)1 << 31)) return false;
  if ((int64_t)B * H * (((int64_t)W + 3) / 4) * (cmax / 4) >= (int64_t)1 << 31) return false;  // stencil indexing
  return true;
}

hope_fmap_t z_map(const void* data, int32_t B, int32_t H, int32_t W, int32_t D, int32_t n_heads) {
  hope_fmap_t m;
  m.data = data;
  m.dtype = HOPE_BF16;
  m.B = B;
  m.H = H;
  m.W = W;
  m.D = D;
  m.n_heads = n_heads;
  return m;
}

BlockLayout layout(int32_t B, int32_t H, int32_t W, int32_t D, int32_t Dm, int32_t n_heads,
                   int32_t ffn_dim, int32_t chunk) {
  const size_t M = (size_t)B * H * W;
  BlockLayout L{};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += align256(bytes);
    return at;
  };
  L.r = take(M * D * 4);
  L.a = take(M * D * 2);
  L.u = take(M * Dm * 4);
  L.z = take(M * Dm * 2);
  L.q = take(M * Dm * 4);
  L.y = take(M * Dm * 4);
  L.y2 = take(M * Dm * 2);
  L.h = take(M * (size_t)ffn_dim * 2);
  const hope_fmap_t zm = z_map(reinterpret_cast<const void*>(256), B, H, W, Dm, n_heads);
  L.op = take(hope_scan2d_workspace_size(&zm, HOPE_DIR_ALL, chunk, nullptr));
  L.total = o;
  return L;
}

}  // namespace

extern "C" {

size_t hope_block_workspace_size(int32_t B, int32_t H, int32_t W, int32_t D, int32_t D_m,
                                 int32_t n_heads, int32_t ffn_dim, int32_t chunk) {
  if (!sizes_ok(B, H, W, D, D_m, n_heads, ffn_dim, chunk)) return 0;
  return layout(B, H, W, D, D_m, n_heads, ffn_dim, chunk).total;
}

hope_status_t hope_block_forward(const float* x, int32_t B, int32_t H, int32_t W, int32_t D,
                                 int32_t D_m, int32_t n_heads, int32_t ffn_dim, int32_t chunk,
                                 const hope_block_weights_t* wt, float* out, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
  if (!sizes_ok(B, H, W, D, D_m, n_heads, ffn_dim, chunk) || !wt) return HOPE_ERR_INVALID_ARG;
  const int d = D_m / n_heads;
  const void* ptrs[] = {x, out, wt->cpe_w, wt->cpe_b, wt->ln1_g, wt->ln1_b, wt->w_in, wt->b_in,
                        wt->dw_w, wt->dw_b, wt->w_q, wt->init_memories, wt->route_scales,
                        wt->skip, wt->lpe_w, wt->lpe_b, wt->w_out, wt->b_out, wt->ln2_g,
                        wt->ln2_b, wt->w1, wt->b1, wt->w2, wt->b2};
  for (const void* p : ptrs)
    if (!aligned16(p)) return HOPE_ERR_INVALID_ARG;
  const size_t M = (size_t)B * H * W;
  const uintptr_t xo = reinterpret_cast<uintptr_t>(x), oo = reinterpret_cast<uintptr_t>(out);
  if (xo < oo + M * D * 4 && oo < xo + M * D * 4) return HOPE_ERR_INVALID_ARG;  // aliasing
  if (d != 16 && d != 32 && d != 64) return HOPE_ERR_UNSUPPORTED;
  const BlockLayout L = layout(B, H, W, D, D_m, n_heads, ffn_dim, chunk);
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) % 256) || workspace_bytes < L.total)
    return HOPE_ERR_WORKSPACE;
  const uintptr_t wo = reinterpret_cast<uintptr_t>(workspace);
  if ((xo < wo + L.total && wo < xo + M * D * 4) || (oo < wo + L.total && wo < oo + M * D * 4))
    return HOPE_ERR_INVALID_ARG;

  char* ws = static_cast<char*>(workspace);
  float* r = reinterpret_cast<float*>(ws + L.r);
  uint16_t* a = reinterpret_cast<uint16_t*>(ws + L.a);
  float* u = reinterpret_cast<float*>(ws + L.u);
  uint16_t* z = reinterpret_cast<uint16_t*>(ws + L.z);
  float* q = reinterpret_cast<float*>(ws + L.q);
  float* y = reinterpret_cast<float*>(ws + L.y);
  uint16_t* y2 = reinterpret_cast<uint16_t*>(ws + L.y2);
  uint16_t* h = reinterpret_cast<uint16_t*>(ws + L.h);
  const int Mi = (int)M;

  hope_scan2d_opts_t o;
  hope_scan2d_default_opts(&o);
  o.stream = stream;
  o.workspace = ws + L.op;
  o.workspace_bytes = L.total - L.op;
  o.route_scales = wt->route_scales;
  o.skip = wt->skip;
  o.queries = q;
  o.queries_dtype = HOPE_F32;
  const hope_fmap_t zm = z_map(z, B, H, W, D_m, n_heads);

  hipError_t e;
  // x1 = x + CPE(x); a = LN1(x1); r = x1 + b_out
  if (D % 128 == 0) {  // one fused pass: x1 stays on chip
    if ((e = hope::launch_cpe_layernorm(x, wt->cpe_w, wt->cpe_b, wt->ln1_g, wt->ln1_b, wt->b_out, a, r, B,
                                        H, W, D, kLnEps, stream)))
      return hope_status_of(e);
  } else {  // x1 into r, then LayerNorm with r += b_out in place
    if ((e = hope::launch_cpe(x, wt->cpe_w, wt->cpe_b, r, B, H, W, D, stream))) return hope_status_of(e);
    if ((e = hope::launch_layernorm(r, wt->ln1_g, wt->ln1_b, a, wt->b_out, r, M, D, kLnEps, stream)))
      return hope_status_of(e);
  }
  // u = a W_in^T + b_in (D -> D_m); z = u + SiLU(DW(u)); q = z W_q^T
  if ((e = hope::launch_gemm_bf16(hope::kEpiF32, a, wt->w_in, Mi, D_m, D, wt->b_in, nullptr, u, stream)))
    return hope_status_of(e);
  if ((e = hope::launch_dwconv_gated(u, wt->dw_w, wt->dw_b, z, B, H, W, D_m, stream))) return hope_status_of(e);
  if ((e = hope::launch_gemm_bf16(hope::kEpiF32, z, wt->w_q, Mi, D_m, D_m, nullptr, nullptr, q, stream)))
    return hope_status_of(e);
  // y = VH(z; q, skip, scales); y2 = y + LPE(z)
  // (the operator's route sum, in slot order, is fused into the local positional branch)
  hope::RoutePlanes rp;
  const hope_status_t st = hope::scan_forward(&zm, wt->init_memories, HOPE_DIR_ALL, chunk, y, &o, &rp);
  if (st != HOPE_OK) return st;
  if ((e = hope::launch_dwconv_lpe(z, y, rp.planes, rp.stride, rp.n, wt->lpe_w, wt->lpe_b, y2, B, H, W,
                                   D_m, stream)))
    return hope_status_of(e);
  // x' = r + y2 W_out^T (D_m -> D; b_out already in r); a = LN2(x'); out = x' + b2
  if ((e = hope::launch_gemm_bf16(hope::kEpiResidualF32, y2, wt->w_out, Mi, D, D_m, nullptr, r, r, stream)))
    return hope_status_of(e);
  if ((e = hope::launch_layernorm(r, wt->ln2_g, wt->ln2_b, a, wt->b2, out, M, D, kLnEps, stream)))
    return hope_status_of(e);
  // h = GELU(a W_1^T + b_1); out = out + h W_2^T
  if ((e = hope::launch_gemm_bf16(hope::kEpiGeluBf16, a, wt->w1, Mi, ffn_dim, D, wt->b1, nullptr, h, stream)))
    return hope_status_of(e);
  if ((e = hope::launch_gemm_bf16(hope::kEpiResidualF32, h, wt->w2, Mi, D, ffn_dim, nullptr, out, out, stream)))
    return hope_status_of(e);
  return HOPE_OK;
}

}  // extern "C"
