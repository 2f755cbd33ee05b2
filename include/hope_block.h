/*
 * hope_block.h -- C ABI of one VisionHOPE block around the four-direction scan, MI355X (gfx950).
 *
 * The operation ("VisionHOPE: Visual Backbones as Self-Modifying Learning Systems",
 * Sec. 2.3 Eq. 27 and App. B.5), inference form, channels-last x[B][H][W][D]; the operator
 * runs at the inner width D_m (Sec. 2.3: Proj_in maps D to D_m, Proj_out maps back; App. C.3
 * gives the evaluated models D_m = D / 2 with n_heads = D / 32 heads of 16):
 *   x1  = x + CPE(x)                      CPE: 3x3 depthwise convolution over D (App. B.5)
 *   u   = LN1(x1) W_in^T + b_in           pre-normalisation, input projection D -> D_m
 *   z   = u + SiLU(DW(u))                 the gated depthwise-convolutional residual branch
 *   q   = z W_q^T                         the outer D_m x D_m query projection shared by
 *                                         the routes
 *   y   = VH(z; q, skip, scales) + LPE(z) the operator (hope_scan2d.h, with its channel-wise
 *                                         skip and direction scales, Eq. 26) plus the
 *                                         depthwise local positional branch on z
 *   x'  = x1 + y W_out^T + b_out          output projection D_m -> D, first residual
 *   out = x' + GELU(LN2(x') W_1^T + b_1) W_2^T + b_2     FFN branch, second residual
 * Where the pages leave the form open this library takes: 3x3 depthwise convolutions with
 * zero padding and a bias; the gated branch u + SiLU(DW(u)); LayerNorm with eps 1e-5 and
 * an affine map; GELU in its erf form; W_q without bias.
 *
 * Precision: the residual stream, the LayerNorm and depthwise arithmetic and every matrix
 * product's accumulation are fp32; the operands of the five projections (LN outputs, z, the
 * operator branch, the FFN hidden layer, and the weights) are bf16.  z enters the operator
 * as bf16 and q as fp32.
 *
 * Conventions: as in hope_scan2d.h (device pointers owned by the caller, nothing
 * allocated, work only enqueued on the stream, arguments validated before anything is
 * enqueued).  Every pointer is 16-byte aligned.  D, D_m and ffn_dim are multiples of 16
 * (D and ffn_dim at most 1024 and 16384), D_m / n_heads is 16, 32 or 64 (the pages use
 * D_m = D / 2, n_heads = D / 32, ffn_dim = 4 D).
 */
#ifndef HOPE_BLOCK_H
#define HOPE_BLOCK_H

#include "hope_scan2d.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Weights of one block.  Linear weights are bf16 bit patterns, [out][in] row-major
 * (y = x W^T + b); depthwise weights are fp32 [3][3][C] (row offset, column offset,
 * channel); vectors fp32.  S(d) = 4 d^2 + 2 d with d = D_m / n_heads. */
typedef struct {
  const float* cpe_w;          /* [3][3][D] */
  const float* cpe_b;          /* [D] */
  const float* ln1_g;          /* [D] */
  const float* ln1_b;          /* [D] */
  const uint16_t* w_in;        /* [D_m][D] */
  const float* b_in;           /* [D_m] */
  const float* dw_w;           /* [3][3][D_m], the gated branch */
  const float* dw_b;           /* [D_m] */
  const uint16_t* w_q;         /* [D_m][D_m] */
  const float* init_memories;  /* [4][n_heads][S(d)], as for hope_scan2d_forward */
  const float* route_scales;   /* [4][D_m] */
  const float* skip;           /* [D_m] */
  const float* lpe_w;          /* [3][3][D_m], the local positional branch */
  const float* lpe_b;          /* [D_m] */
  const uint16_t* w_out;       /* [D][D_m] */
  const float* b_out;          /* [D] */
  const float* ln2_g;          /* [D] */
  const float* ln2_b;          /* [D] */
  const uint16_t* w1;          /* [ffn_dim][D] */
  const float* b1;             /* [ffn_dim] */
  const uint16_t* w2;          /* [D][ffn_dim] */
  const float* b2;             /* [D] */
} hope_block_weights_t;

/* Bytes of device scratch hope_block_forward needs for these sizes (0 on invalid sizes). */
size_t hope_block_workspace_size(int32_t B, int32_t H, int32_t W, int32_t D, int32_t D_m,
                                 int32_t n_heads, int32_t ffn_dim, int32_t chunk);

/*
 * hope_block_forward -- one block on x (fp32 [B][H][W][D]) into out (fp32, same shape; may
 * not alias x).  D_m: the operator's width, split into n_heads heads.  chunk: the
 * operator's chunk length (0 = aligned, Eq. 25).  workspace: device scratch of at least
 * hope_block_workspace_size() bytes, 256-byte aligned; its contents are not kept.  The
 * weights are only read; they must not overlap out or the workspace (the aliasing check
 * covers x, out and the workspace only).  Returns HOPE_ERR_INVALID_ARG for bad sizes, null
 * or misaligned pointers or aliasing, HOPE_ERR_UNSUPPORTED for a head dimension other than
 * 16/32/64, HOPE_ERR_WORKSPACE for a short workspace, HOPE_ERR_HIP when a launch fails.
 */
hope_status_t hope_block_forward(const float* x, int32_t B, int32_t H, int32_t W, int32_t D,
                                 int32_t D_m, int32_t n_heads, int32_t ffn_dim, int32_t chunk,
                                 const hope_block_weights_t* weights, float* out,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* HOPE_BLOCK_H */
