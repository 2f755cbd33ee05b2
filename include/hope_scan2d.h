/*
 * hope_scan2d.h -- C ABI of the four-direction Hope memory scan on MI355X (gfx950).
 *
 * The operation (page titles cited, then section / equation):
 *   "VisionHOPE: Visual Backbones as Self-Modifying Learning Systems" (VisionHOPE)
 *     Sec. 2.3 Eq. 24-26: serialise the feature map along four routes
 *       (row-major, its reversal, column-major, its reversal), run one
 *       self-referential memory per route and head, restore and sum;
 *     Sec. 2.3 Eq. 25: chunks span one row (row routes) or one column
 *       (column routes);
 *     Sec. 2.1.3 Eq. 15-16: per chunk, k, v, q, eta, alpha and the readout
 *       y = M_mem q are generated from the memories frozen at the chunk start;
 *     Sec. 2.2 Definition 1, Eq. 19-20 and App. B.3: the executed step
 *       (soft injection cap, spectral clamp, finite-precision safeguards);
 *     Sec. 2.1.2 Eq. 13 / App. B.4 Eq. 45-46: every memory is updated by the
 *       same right-multiplicative gain of the chunk.
 *   "Nested Learning: The Illusion of Deep Learning Architectures" part 12,
 *     Eq. 94-96: the update set {k, v, q, eta, alpha, memory}; this library
 *     keeps q as a sixth coupled memory M_q, q = n(M_q x).
 *   "VMamba: Visual State Space Model" (explainer): the exact scan orders and
 *     the restore-then-sum merge (no averaging).
 *
 * Conventions shared by every entry point
 *   - All data pointers are DEVICE pointers owned by the caller.  The library
 *     keeps no pointer after a call returns and never allocates device memory.
 *   - Every call only enqueues work on the given stream (0 = default stream) and
 *     returns; results are ready when the stream is synchronised.
 *   - Every argument is validated before anything is enqueued: a call that
 *     returns an error has written nothing.
 *   - Feature maps are channels-last and contiguous: x[B][H][W][D], the flat
 *     pixel index is h * W + w.  Heads are contiguous channel slices of width
 *     d = D / n_heads; d must be 16, 32 or 64.
 *   - Route index r: 0 = row-major forward, 1 = its full reversal, 2 = column-major
 *     forward (flatten of the spatial transpose), 3 = its full reversal.
 *   - Per (route, head) state: S(d) = 4 d^2 + 2 d floats, the concatenation of
 *     M_mem, M_k, M_v, M_q (each d x d, row-major, applied as M @ x), m_eta and
 *     m_alpha (each 1 x d).
 *   - Thread safety: reentrant; no mutable global state.
 */
#ifndef HOPE_SCAN2D_H
#define HOPE_SCAN2D_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  HOPE_OK = 0,
  HOPE_ERR_INVALID_ARG = -1,  /* malformed shape, null or misaligned pointer, aliasing, bad flag */
  HOPE_ERR_UNSUPPORTED = -2,  /* well-formed but not implemented (head dimension not 16/32/64) */
  HOPE_ERR_WORKSPACE = -3,    /* workspace missing or smaller than hope_scan2d_workspace_size() */
  HOPE_ERR_HIP = -4           /* a HIP launch failed; hope_last_hip_error() tells which */
} hope_status_t;

typedef enum { HOPE_F32 = 0, HOPE_BF16 = 1 } hope_dtype_t;

enum {
  HOPE_DIR_ROW_FWD = 1u, /* route 0 */
  HOPE_DIR_ROW_REV = 2u, /* route 1 */
  HOPE_DIR_COL_FWD = 4u, /* route 2 */
  HOPE_DIR_COL_REV = 8u, /* route 3 */
  HOPE_DIR_ALL = 15u
};

typedef enum {
  HOPE_ETA_SIGMOID = 0,  /* eta = eta_scale * sigmoid(s)  (synthetic workloads: eta_scale = 1) */
  HOPE_ETA_SOFTPLUS = 1  /* eta = eta_scale * softplus(s) (VisionHOPE App. C.1 Eq. 53, gamma = 0.025) */
} hope_eta_map_t;

/* A feature map.  data: device pointer to x[B][H][W][D], 16-byte aligned;
 * dtype: hope_dtype_t (F32 or BF16). */
typedef struct {
  const void* data;
  int32_t dtype;
  int32_t B, H, W, D, n_heads;
} hope_fmap_t;

/* Which memory the readout y_t = M_mem q_t uses inside a chunk.
 *   BOUNDARY: the memory frozen at the chunk start, M_mem,b ("VisionHOPE: Visual
 *             Backbones as Self-Modifying Learning Systems", Sec. 2.1.3 Eq. 16).
 *   RUNNING:  the memory after the chunk's earlier tokens, M_mem,b G_{t-1} ("Nested
 *             Learning: The Illusion of Deep Learning Architectures", Eq. 94, which reads
 *             M_memory,t-1; the gain G of VisionHOPE App. B.4 Prop. 2).  q_t and every
 *             other projection still come from the chunk-start memories.  Equal to
 *             BOUNDARY when every chunk is one token. */
typedef enum { HOPE_READOUT_BOUNDARY = 0, HOPE_READOUT_RUNNING = 1 } hope_readout_t;

/* Step-control variants ("VisionHOPE", Sec. 3.5 ablations).
 *   INJECTION_SOFT  the soft injection cap of Eq. 19;  HARD  min(eta, eta_inj) at the same
 *   limit;  NONE  no injection control.
 *   SPECTRAL_CLAMP  min(eta_bar, eta_spec) of Eq. 20;  SOFT  eta_spec (1 - exp(-eta_bar /
 *   eta_spec)), a smooth map to the same limit;  NONE  no spectral control. */
typedef enum { HOPE_INJECTION_SOFT = 0, HOPE_INJECTION_HARD = 1, HOPE_INJECTION_NONE = 2 } hope_injection_t;
typedef enum { HOPE_SPECTRAL_CLAMP = 0, HOPE_SPECTRAL_SOFT = 1, HOPE_SPECTRAL_NONE = 2 } hope_spectral_t;

/* Memories held fixed within the image (Sec. 3.5: without adaptive K/V, without adaptive
 * dynamics); the content memory always evolves. */
typedef enum { HOPE_FREEZE_KV = 1, HOPE_FREEZE_DYNAMICS = 2, HOPE_FREEZE_Q = 4 } hope_freeze_t;

/* Options of hope_scan2d_forward.  Start from hope_scan2d_default_opts(). */
typedef struct {
  hipStream_t stream;        /* stream to enqueue on; 0 = default stream */
  float* final_memories;     /* NULL, or device [B][4][n_heads][S(d)] fp32: state after the
                                last chunk of every (image, route, head); rows of unselected
                                routes are left untouched */
  void* workspace;           /* device scratch of at least workspace_bytes, 256-byte aligned */
  size_t workspace_bytes;
  int32_t eta_map;           /* hope_eta_map_t; default HOPE_ETA_SIGMOID */
  float eta_scale;           /* default 1.0 */
  float alpha_bias;          /* alpha = sigmoid(s + alpha_bias); default 4.0 */
  float eps;                 /* stabiliser of the key / query normalisation (App. C.1) and the
                                epsilon of the soft injection cap (Eq. 19); default 1e-6 */
  int32_t init_per_image;    /* 0: init is [4][n_heads][S]; 1: [B][4][n_heads][S] (resume) */
  int32_t out_dtype;         /* hope_dtype_t of out: HOPE_F32 (default) or HOPE_BF16; a bf16
                                out holds the fp32 route sum rounded once to nearest even */
  hipEvent_t scan_begin;     /* NULL, or an event recorded on the stream just before the scan
                                kernel is enqueued (profiling) */
  hipEvent_t scan_end;       /* NULL, or an event recorded just after it, before the route sum;
                                the pair times the scan kernel alone.  Both or neither. */
  int32_t readout;           /* hope_readout_t; default HOPE_READOUT_BOUNDARY */
  int32_t reserved;          /* must be 0 */
  /* Variants of "VisionHOPE: Visual Backbones as Self-Modifying Learning Systems"
   * (Sec. 2.3 Eq. 26, App. B.5 and the Sec. 3.5 ablations).  Defaults reproduce the
   * operator above. */
  const float* route_scales; /* NULL (unit scales), or device [4][D] fp32: the channel-wise
                                direction scales lambda_r of Eq. 26, indexed by route */
  const float* skip;         /* NULL, or device [D] fp32: a channel-wise skip added to every
                                route's reads before its scale, Y_r = reads_r + skip * Z_r */
  unsigned long long* counts;/* NULL, or device [3] uint64, 8-byte aligned, accumulated (not
                                cleared): live token updates; tokens whose raw eta exceeds the
                                injection limit; tokens whose eta_bar exceeds the spectral limit
                                (decided in fp32) */
  int32_t injection;         /* hope_injection_t; default HOPE_INJECTION_SOFT */
  int32_t spectral;          /* hope_spectral_t; default HOPE_SPECTRAL_CLAMP */
  uint32_t frozen;           /* OR of hope_freeze_t: memories held fixed within the image */
  int32_t no_dgd;            /* 1: drop the key-dependent correction -eta M k k^T of the
                                update (the DGD ablation), keeping signal, retention and step */
  int32_t shared_init;       /* 1: init_memories is [n_heads][S], shared by all routes (the
                                trajectories stay separate); excludes init_per_image */
  int32_t queries_dtype;     /* hope_dtype_t of queries (ignored when queries is NULL) */
  const void* queries;       /* NULL, or device [B][H][W][D] of queries_dtype: queries from the
                                fixed outer D x D projection of App. B.5 (Eq. 14), computed
                                once per image and shared by all routes; q_t is the route-
                                ordered head slice, normalised within the head, and M_q takes
                                no part (it is left at its initial value) */
  int32_t mem_chunk;         /* 0 (default): one chunk length for all six memories.  > 0: the
                                working memory M_mem keeps its boundary state over chunks of
                                this many tokens ("Nested Learning", two chunk sizes, one for
                                the working memory and one for the projection memories): its
                                boundary readout and its self-generated targets use M_mem at
                                the start of the token's mem_chunk-chunk, while k, v, q, eta and
                                alpha come from the other memories at the start of its chunk-
                                chunk.  Runs on the fp32 chain kernel.  < 0: invalid */
  float* step_map;           /* NULL, or device [B][4][n_heads][H][W] fp32, 4-byte aligned: the
                                executed step eta_tilde (Sec. 2.2 Eq. 20, or the selected
                                ablation control) of every token of a selected route, written
                                at the token's pixel; entries of unselected routes are left
                                untouched.  The per-pixel step maps that the Sec. 3.5 analysis
                                of the step controls inspects.  Must not overlap out, x,
                                init_memories, final_memories, counts or the workspace. */
} hope_scan2d_opts_t;

/* Fill *opts with the defaults listed above (no stream, no final state, no workspace). */
void hope_scan2d_default_opts(hope_scan2d_opts_t* opts);

/*
 * hope_scan2d_forward -- the four-direction scan (VisionHOPE Sec. 2.3 Eq. 24-26
 * with unit direction scales; recurrence of Sec. 2.1.3 Eq. 15-16 with the
 * executed step of Sec. 2.2 Eq. 19-20 and the shared gain of App. B.4 Eq. 46).
 *
 *   x              feature map (see hope_fmap_t).
 *   init_memories  device fp32, [4][n_heads][S(d)] (or [B][4][n_heads][S(d)] when
 *                  opts->init_per_image): the initial state of every route and head;
 *                  rows of unselected routes are not read.
 *   dirs           bit set of routes (HOPE_DIR_*), 1..15.  Unselected routes add
 *                  nothing to out.
 *   chunk          chunk length; 0 = aligned (W on row routes, H on column routes,
 *                  Eq. 25).  A chunk length that does not divide H*W leaves a
 *                  shorter last chunk.
 *   out            device [B][H][W][D] of opts->out_dtype (fp32 by default, or bf16),
 *                  16-byte aligned, overwritten with the sum over selected routes of
 *                  each route's readout restored to its pixel, added in fp32 in the
 *                  fixed order route 0, 1, 2, 3 (then rounded once for a bf16 out).
 *   opts           NULL = defaults.  With two or more routes selected, or a bf16 out,
 *                  a workspace is required (hope_scan2d_workspace_size).
 * Errors: HOPE_ERR_INVALID_ARG for null / misaligned pointers, non-positive sizes,
 * D not divisible by n_heads, dirs outside 1..15, chunk < 0, dtype or out_dtype not
 * F32/BF16,
 * out overlapping x, init_memories, final_memories or the workspace;
 * HOPE_ERR_UNSUPPORTED for d not in {16, 32, 64}; HOPE_ERR_WORKSPACE when the
 * workspace is missing or too small; HOPE_ERR_HIP when a launch fails.
 * Results are deterministic: the same inputs give bit-identical outputs.
 */
hope_status_t hope_scan2d_forward(const hope_fmap_t* x, const float* init_memories,
                                  uint32_t dirs, int32_t chunk, void* out,
                                  const hope_scan2d_opts_t* opts);

/* Size of the device array that serves hope_scan2d_forward_noalloc as its route-plane
 * scratch: 64 MiB, one array per GPU the library runs on, held until the process ends. */
#define HOPE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * hope_scan2d_forward_noalloc -- hope_scan2d_forward for callers that cannot allocate device
 * memory or pass a workspace: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same arguments, results (bit for bit) and checks, except:
 *   - opts->workspace must be NULL and opts->workspace_bytes 0 (else HOPE_ERR_INVALID_ARG):
 *     the route planes live in the library's own device array of
 *     HOPE_NOALLOC_SCRATCH_BYTES bytes.  The batch is processed in consecutive slices of
 *     whole images whose planes fit in it (one slice when none is needed: one route with
 *     an fp32 out).  HOPE_ERR_WORKSPACE when one image's planes do not fit:
 *     (popcount(dirs) - 1) * H * W * D * 4 bytes for an fp32 out, popcount(dirs) * ... for
 *     a bf16 out, above HOPE_NOALLOC_SCRATCH_BYTES.
 *   - opts->scan_begin / scan_end, when given, bracket every slice's scan kernel together
 *     (with the route sums of the slices before the last).
 *   - The array is per GPU (the current device) and shared by every call on that GPU: calls
 *     that overlap in time on one GPU (other streams, other host threads) race on it and
 *     must be serialised by the caller.  It keeps the last call's contents; every element
 *     a call reads it has written first.
 * Calls no allocating routine (no hipMalloc, no hipFree).  The stream must belong to the
 * current device.
 */
hope_status_t hope_scan2d_forward_noalloc(const hope_fmap_t* x, const float* init_memories,
                                          uint32_t dirs, int32_t chunk, void* out,
                                          const hope_scan2d_opts_t* opts);

/* Bytes of workspace hope_scan2d_forward needs for this call with these options (NULL =
 * defaults): one fp32 plane of the map per selected route beyond the first, or per
 * selected route for a bf16 out; 0 when none is needed, and 0 for arguments that
 * hope_scan2d_forward would reject. */
size_t hope_scan2d_workspace_size(const hope_fmap_t* x, uint32_t dirs, int32_t chunk,
                                  const hope_scan2d_opts_t* opts);

/*
 * hope_scan2d_backward -- gradients of a scalar loss L(out) of hope_scan2d_forward with
 * respect to the feature map and the initial memories: the outer gradients through the
 * explicit, differentiable memory trajectory ("VisionHOPE: Visual Backbones as
 * Self-Modifying Learning Systems", Sec. 1; forward as in Sec. 2.1.3 Eq. 15-16, Sec. 2.2
 * Eq. 19-20, App. B.4 Eq. 46).  The forward is recomputed inside the call (chunk-boundary
 * states are checkpointed in the workspace); nothing from a forward call is needed.
 *
 *   x, init_memories, dirs, chunk   as for hope_scan2d_forward.
 *   grad_out       device fp32 [B][H][W][D], dL/dout, 16-byte aligned.
 *   grad_x         device fp32 [B][H][W][D], 16-byte aligned, overwritten with dL/dx
 *                  (for a bf16 map: the gradient with respect to the bf16 values).
 *   grad_init      device fp32 shaped like init_memories ([4][n_heads][S(d)], or
 *                  [B][4][n_heads][S(d)] with init_per_image), overwritten with
 *                  dL/dinit; rows of unselected routes are set to zero.
 *   opts           NULL = defaults.  Honoured: stream, workspace, eta_map, eta_scale,
 *                  alpha_bias, eps, init_per_image, and at d = 32 readout (boundary or
 *                  running).  A workspace is always required
 *                  (hope_scan2d_backward_workspace_size).
 * Where the step of Eq. 20 is not differentiable: min(eta_bar, eta_spec) follows
 * eta_bar when eta_bar <= eta_spec; no derivative through the |k|^2 floor or the one-ulp
 * rounding of eta_spec; eta_bar = 0 (eta = 0 or eta_inj = 0) has derivative zero.
 * Errors: as hope_scan2d_forward for the shared arguments; HOPE_ERR_INVALID_ARG when
 * grad_out, grad_x or grad_init is null, misaligned or overlaps another argument;
 * HOPE_ERR_UNSUPPORTED for d not in {16, 32, 64}, a chunk (after clipping to H*W)
 * longer than 128 tokens at d = 16 or 32 tokens at d = 64 (d = 32 takes any chunk
 * length), or any option outside the honoured set away
 * from its default (the running readout at d = 16 or 64, variants, two chunk sizes,
 * final_memories, bf16 out); HOPE_ERR_WORKSPACE; HOPE_ERR_HIP.  Deterministic: per-route map gradients and
 * per-image state gradients are summed in a fixed order.
 */
hope_status_t hope_scan2d_backward(const hope_fmap_t* x, const float* init_memories,
                                   uint32_t dirs, int32_t chunk, const float* grad_out,
                                   float* grad_x, float* grad_init,
                                   const hope_scan2d_opts_t* opts);

/* Bytes of workspace hope_scan2d_backward needs: the map-gradient planes of the routes
 * beyond the first, plus per chain the state adjoint and the forward records (at d = 32
 * the product of the earlier chunks' gains and, per 16-token block of each chunk, its end
 * gain, its token vectors and gates; otherwise every chunk-boundary state and one chunk's
 * gain trajectory);
 * 0 for arguments it would reject. */
size_t hope_scan2d_backward_workspace_size(const hope_fmap_t* x, uint32_t dirs, int32_t chunk,
                                           const hope_scan2d_opts_t* opts);

/* Name of the scan kernel hope_scan2d_forward launches for these arguments (opts NULL =
 * defaults; only the shape, dtype, routes, chunk and option flags are read, no pointer is
 * dereferenced), e.g. "chain_mfma_kernel"; "" for arguments it would reject.  A static
 * string.  For profiling: it names the kernel a trace of the call shows. */
const char* hope_scan2d_kernel_name(const hope_fmap_t* x, uint32_t dirs, int32_t chunk,
                                    const hope_scan2d_opts_t* opts);

/* Static, human-readable name of a status code. */
const char* hope_status_string(hope_status_t status);

/* The hipError_t behind the last HOPE_ERR_HIP returned on this thread (0 if none). */
int hope_last_hip_error(void);

/*
 * Test and measurement exports of the two permutations on their own.
 *
 * hope_debug_cross_scan -- routes[slot][b][t][c] = x[b][p_r(t)][c] for every
 * selected route r, slots numbered in increasing r ("VMamba: Visual State Space
 * Model", the four scan orders; VisionHOPE Eq. 24).  routes has the dtype of x and
 * popcount(dirs) * B * H * W * D elements; it must not overlap x.  Bit-exact copy.
 */
hope_status_t hope_debug_cross_scan(const hope_fmap_t* x, uint32_t dirs, void* routes,
                                    hipStream_t stream);

/*
 * hope_debug_cross_merge -- out[b][p][c] = sum over selected routes, in increasing r,
 * of routes[slot][b][t][c] at p = p_r(t) (the restore-then-sum merge of VisionHOPE
 * Eq. 26 with unit scales).  routes: dtype F32 or BF16 (widened to fp32 before the
 * adds), popcount(dirs) * B * H * W * D elements; out: fp32 [B][H][W][D], not
 * overlapping routes.
 */
hope_status_t hope_debug_cross_merge(const void* routes, int32_t dtype, int32_t B, int32_t H,
                                     int32_t W, int32_t D, uint32_t dirs, float* out,
                                     hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* HOPE_SCAN2D_H */
