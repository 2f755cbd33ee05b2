// Host side of the C ABI declared in include/hope_scan2d.h: argument validation
// (all of it before anything is enqueued), workspace accounting and kernel dispatch.
#include <algorithm>
#include <mutex>
#include <math.h>
#include <string.h>

#include "../../include/hope_scan2d.h"
#include "kernels.h"
#include "scan_api.h"

namespace {

thread_local int g_last_hip_error = 0;

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

bool overlaps(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

Range range_of(const void* p, size_t bytes) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return {lo, lo + bytes};
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int popcount4(uint32_t dirs) {
  int n = 0;
  for (int r = 0; r < 4; ++r) n += (dirs >> r) & 1u;
  return n;
}

int slots_of(uint32_t dirs, int* route_of_slot) {
  int n = 0;
  for (int r = 0; r < 4; ++r)
    if ((dirs >> r) & 1u) route_of_slot[n++] = r;
  return n;
}

// Workspace layout: fp32 route planes of one map each, each padded to 256 bytes: one per
// selected route beyond the first (route 0 writes an fp32 out directly), or one per
// selected route when out is bf16 (the route sum then rounds once, in its own pass).
int64_t plane_stride_elems(int64_t n_elem) { return (n_elem + 63) / 64 * 64; }

hope_status_t check_fmap(const hope_fmap_t* x) {
  if (!x || !x->data) return HOPE_ERR_INVALID_ARG;
  if (x->dtype != HOPE_F32 && x->dtype != HOPE_BF16) return HOPE_ERR_INVALID_ARG;
  if (x->B <= 0 || x->H <= 0 || x->W <= 0 || x->D <= 0 || x->n_heads <= 0)
    return HOPE_ERR_INVALID_ARG;
  if (x->D % x->n_heads) return HOPE_ERR_INVALID_ARG;
  if ((int64_t)x->H * x->W > INT32_MAX) return HOPE_ERR_INVALID_ARG;
  if ((int64_t)x->B * x->H * x->W > INT64_MAX / 8 / x->D) return HOPE_ERR_INVALID_ARG;
  if (!aligned(x->data, 16)) return HOPE_ERR_INVALID_ARG;
  return HOPE_OK;
}

hope_status_t check_opts(const hope_scan2d_opts_t* o) {
  if (o->eta_map != HOPE_ETA_SIGMOID && o->eta_map != HOPE_ETA_SOFTPLUS)
    return HOPE_ERR_INVALID_ARG;
  if (!isfinite(o->eta_scale) || o->eta_scale < 0.f) return HOPE_ERR_INVALID_ARG;
  if (!isfinite(o->alpha_bias)) return HOPE_ERR_INVALID_ARG;
  if (!isfinite(o->eps) || o->eps < 0.f) return HOPE_ERR_INVALID_ARG;
  if (o->init_per_image != 0 && o->init_per_image != 1) return HOPE_ERR_INVALID_ARG;
  if (o->out_dtype != HOPE_F32 && o->out_dtype != HOPE_BF16) return HOPE_ERR_INVALID_ARG;
  if ((o->scan_begin == nullptr) != (o->scan_end == nullptr)) return HOPE_ERR_INVALID_ARG;
  if (o->readout != HOPE_READOUT_BOUNDARY && o->readout != HOPE_READOUT_RUNNING)
    return HOPE_ERR_INVALID_ARG;
  if (o->reserved != 0) return HOPE_ERR_INVALID_ARG;
  if (o->queries && o->queries_dtype != HOPE_F32 && o->queries_dtype != HOPE_BF16) return HOPE_ERR_INVALID_ARG;
  if (o->queries && !aligned(o->queries, 16)) return HOPE_ERR_INVALID_ARG;
  if (o->injection < HOPE_INJECTION_SOFT || o->injection > HOPE_INJECTION_NONE) return HOPE_ERR_INVALID_ARG;
  if (o->spectral < HOPE_SPECTRAL_CLAMP || o->spectral > HOPE_SPECTRAL_NONE) return HOPE_ERR_INVALID_ARG;
  if (o->frozen & ~7u) return HOPE_ERR_INVALID_ARG;
  if (o->mem_chunk < 0) return HOPE_ERR_INVALID_ARG;
  if (o->no_dgd != 0 && o->no_dgd != 1) return HOPE_ERR_INVALID_ARG;
  if (o->shared_init != 0 && o->shared_init != 1) return HOPE_ERR_INVALID_ARG;
  if (o->shared_init && o->init_per_image) return HOPE_ERR_INVALID_ARG;
  if (o->route_scales && !aligned(o->route_scales, 4)) return HOPE_ERR_INVALID_ARG;
  if (o->skip && !aligned(o->skip, 4)) return HOPE_ERR_INVALID_ARG;
  if (o->counts && !aligned(o->counts, 8)) return HOPE_ERR_INVALID_ARG;
  if (o->final_memories && !aligned(o->final_memories, 16)) return HOPE_ERR_INVALID_ARG;
  if (o->workspace && !aligned(o->workspace, 256)) return HOPE_ERR_INVALID_ARG;
  return HOPE_OK;
}

int planes_for(uint32_t dirs, int32_t out_dtype) {
  const int n_sel = popcount4(dirs);
  return out_dtype == HOPE_BF16 ? n_sel : n_sel - 1;
}

size_t workspace_bytes_for(const hope_fmap_t* x, uint32_t dirs, int32_t out_dtype) {
  const int n_planes = planes_for(dirs, out_dtype);
  if (n_planes <= 0) return 0;
  const int64_t n_elem = (int64_t)x->B * x->H * x->W * x->D;
  return (size_t)n_planes * (size_t)plane_stride_elems(n_elem) * sizeof(float);
}

hope_status_t hip_status(hipError_t e) {
  if (e == hipSuccess) return HOPE_OK;
  g_last_hip_error = (int)e;
  return HOPE_ERR_HIP;
}

}  // namespace

// The status of a HIP result for the entry points of other translation units (records the
// error for hope_last_hip_error, as the entry points here do).
hope_status_t hope_status_of(hipError_t e) { return hip_status(e); }

namespace {

// Backward workspace: map-gradient planes of the selected routes beyond the first, then
// chain_floats per chain (n_sel * B * n_heads chains, in launch order).
struct BackLayout {
  int n_sel;
  int64_t plane_stride, planes_floats, chain_floats, nck, cmax;
};

BackLayout backward_layout(const hope_fmap_t* x, uint32_t dirs, int32_t chunk) {
  BackLayout L{};
  int route_of_slot[4];
  L.n_sel = slots_of(dirs, route_of_slot);
  const int d = x->D / x->n_heads;
  const int64_t N = (int64_t)x->H * x->W;
  for (int s = 0; s < L.n_sel; ++s) {
    const int r = route_of_slot[s];
    const int64_t C = chunk > 0 ? chunk : (r < 2 ? x->W : x->H);
    L.nck = std::max<int64_t>(L.nck, (N + C - 1) / C);
    L.cmax = std::max<int64_t>(L.cmax, std::min<int64_t>(C, N));
  }
  const int64_t SS = 4LL * d * d + 2LL * d;
  L.chain_floats = d == 32 ? hope::backward_wy32_chain_floats(L.nck, L.cmax)
                           : ((L.nck + 1) * SS + L.cmax * d * d + 63) / 64 * 64;
  L.plane_stride = plane_stride_elems((int64_t)x->B * x->H * x->W * x->D);
  L.planes_floats = (int64_t)(L.n_sel - 1) * L.plane_stride;
  return L;
}

size_t backward_workspace_bytes(const hope_fmap_t* x, const BackLayout& L) {
  const int64_t chains = (int64_t)L.n_sel * x->B * x->n_heads;
  return (size_t)(L.planes_floats + chains * L.chain_floats) * sizeof(float);
}

// options the backward pass honours: everything else must be at its default
bool backward_opts_supported(const hope_scan2d_opts_t& o) {
  return (o.readout == HOPE_READOUT_BOUNDARY || o.readout == HOPE_READOUT_RUNNING) && !o.route_scales && !o.skip && !o.counts &&
         o.injection == HOPE_INJECTION_SOFT && o.spectral == HOPE_SPECTRAL_CLAMP && o.frozen == 0 &&
         o.no_dgd == 0 && o.shared_init == 0 && !o.queries && o.mem_chunk == 0 && !o.final_memories &&
         o.out_dtype == HOPE_F32;
}

}  // namespace

namespace hope {

// bf16 maps: the chunk-parallel kernel at d = 16 and 32 (boundary readout, one chunk
// length), the register-resident block kernel for the rest of d = 32 and for d = 64 with
// chunks of at most 16 tokens; everything else on the fp32 kernel
ScanPath select_scan_path(const ChainParams& p, int d) {
  if (chunk_path_supported(p, d)) return kPathChunk;
  return mfma_path_supported(p, d) ? kPathMfma : kPathChain;
}

const char* scan_path_kernel(ScanPath path) {
  switch (path) {
    case kPathChunk: return "chain_chunk_kernel";
    case kPathMfma: return "chain_mfma_kernel";
    case kPathChain: return "chain_kernel";
  }
  return "";
}

hipError_t launch_scan(const ChainParams& p, int d, hipStream_t s) {
  switch (select_scan_path(p, d)) {
    case kPathChunk: return launch_chain_chunk(p, d, s);
    case kPathMfma: return launch_chain_mfma(p, d, s);
    case kPathChain: return launch_chain(p, d, s);
  }
  return hipErrorInvalidValue;
}

// Every check of hope_scan2d_forward (the workspace's only with check_workspace) and the
// kernel parameters of the call, without the route planes (attach_planes).
hope_status_t plan_forward(const hope_fmap_t* x, const float* init_memories, uint32_t dirs,
                           int32_t chunk, void* out, const hope_scan2d_opts_t& o, bool check_workspace,
                           ChainParams& p, int& d) {
  hope_status_t st = check_fmap(x);
  if (st != HOPE_OK) return st;
  if ((st = check_opts(&o)) != HOPE_OK) return st;
  if (!init_memories || !out) return HOPE_ERR_INVALID_ARG;
  if (!aligned(init_memories, 16) || !aligned(out, 16)) return HOPE_ERR_INVALID_ARG;
  if (dirs == 0 || dirs > 15 || chunk < 0) return HOPE_ERR_INVALID_ARG;

  d = x->D / x->n_heads;
  const int64_t n_elem = (int64_t)x->B * x->H * x->W * x->D;
  const size_t x_bytes = (size_t)n_elem * (x->dtype == HOPE_BF16 ? 2 : 4);
  const bool out_bf16 = o.out_dtype == HOPE_BF16;
  const size_t out_bytes = (size_t)n_elem * (out_bf16 ? 2 : 4);
  const size_t state_floats = (size_t)4 * d * d + 2 * (size_t)d;
  const size_t init_bytes = (o.init_per_image ? (size_t)x->B : 1) * (o.shared_init ? 1 : 4) *
                            (size_t)x->n_heads * state_floats * sizeof(float);
  const size_t final_bytes = (size_t)x->B * 4 * x->n_heads * state_floats * sizeof(float);
  const size_t ws_need = workspace_bytes_for(x, dirs, o.out_dtype);

  const Range r_out = range_of(out, out_bytes);
  if (overlaps(r_out, range_of(x->data, x_bytes))) return HOPE_ERR_INVALID_ARG;
  if (overlaps(r_out, range_of(init_memories, init_bytes))) return HOPE_ERR_INVALID_ARG;
  if (o.route_scales && overlaps(r_out, range_of(o.route_scales, 4 * (size_t)x->D * sizeof(float))))
    return HOPE_ERR_INVALID_ARG;
  if (o.skip && overlaps(r_out, range_of(o.skip, (size_t)x->D * sizeof(float)))) return HOPE_ERR_INVALID_ARG;
  if (o.queries &&
      overlaps(r_out, range_of(o.queries, (size_t)n_elem * (o.queries_dtype == HOPE_BF16 ? 2 : 4))))
    return HOPE_ERR_INVALID_ARG;
  if (o.counts) {
    const Range r_cnt = range_of(o.counts, 3 * sizeof(unsigned long long));
    if (overlaps(r_out, r_cnt) || overlaps(r_cnt, range_of(x->data, x_bytes)) ||
        overlaps(r_cnt, range_of(init_memories, init_bytes)))
      return HOPE_ERR_INVALID_ARG;
    if (o.workspace && o.workspace_bytes && overlaps(r_cnt, range_of(o.workspace, o.workspace_bytes)))
      return HOPE_ERR_INVALID_ARG;
  }
  if (o.final_memories) {
    const Range r_fin = range_of(o.final_memories, final_bytes);
    if (overlaps(r_out, r_fin) || overlaps(r_fin, range_of(x->data, x_bytes)) ||
        overlaps(r_fin, range_of(init_memories, init_bytes)))
      return HOPE_ERR_INVALID_ARG;
  }
  if (o.workspace && o.workspace_bytes) {
    const Range r_ws = range_of(o.workspace, o.workspace_bytes);
    if (overlaps(r_out, r_ws) || overlaps(r_ws, range_of(x->data, x_bytes)) ||
        overlaps(r_ws, range_of(init_memories, init_bytes)))
      return HOPE_ERR_INVALID_ARG;
    if (o.final_memories && overlaps(r_ws, range_of(o.final_memories, final_bytes)))
      return HOPE_ERR_INVALID_ARG;
  }
  if (o.step_map) {
    const size_t steps_bytes = (size_t)x->B * 4 * x->n_heads * x->H * x->W * sizeof(float);
    const Range r_st = range_of(o.step_map, steps_bytes);
    if (!aligned(o.step_map, 4) || overlaps(r_out, r_st) || overlaps(r_st, range_of(x->data, x_bytes)) ||
        overlaps(r_st, range_of(init_memories, init_bytes)))
      return HOPE_ERR_INVALID_ARG;
    if (o.workspace && o.workspace_bytes && overlaps(r_st, range_of(o.workspace, o.workspace_bytes)))
      return HOPE_ERR_INVALID_ARG;
    if (o.final_memories && overlaps(r_st, range_of(o.final_memories, final_bytes)))
      return HOPE_ERR_INVALID_ARG;
    if (o.counts && overlaps(r_st, range_of(o.counts, 3 * sizeof(unsigned long long))))
      return HOPE_ERR_INVALID_ARG;
  }
  if (d != 16 && d != 32 && d != 64) return HOPE_ERR_UNSUPPORTED;
  if (check_workspace && ws_need > 0 && (!o.workspace || o.workspace_bytes < ws_need)) return HOPE_ERR_WORKSPACE;

  memset(&p, 0, sizeof(p));
  p.x = x->data;
  p.init = init_memories;
  p.final_mem = o.final_memories;
  p.x_bf16 = x->dtype == HOPE_BF16;
  p.B = x->B;
  p.H = x->H;
  p.W = x->W;
  p.D = x->D;
  p.nh = x->n_heads;
  p.n_sel = slots_of(dirs, p.route_of_slot);
  p.chunk = chunk;
  p.init_per_image = o.init_per_image;
  p.eta_map = o.eta_map;
  p.eta_scale = o.eta_scale;
  p.alpha_bias = o.alpha_bias;
  p.eps = o.eps;
  p.readout = o.readout;
  p.route_scales = o.route_scales;
  p.skip = o.skip;
  p.counts = o.counts;
  p.injection = o.injection;
  p.spectral = o.spectral;
  p.frozen = o.frozen;
  p.no_dgd = o.no_dgd;
  p.shared_init = o.shared_init;
  p.queries = o.queries;
  p.queries_bf16 = o.queries_dtype == HOPE_BF16;
  p.mem_chunk = o.mem_chunk;
  p.steps = o.step_map;
  if ((int64_t)p.n_sel * p.B * p.nh > INT32_MAX) return HOPE_ERR_INVALID_ARG;

  return HOPE_OK;
}

// Route planes of a planned call: with a bf16 out every route writes an fp32 plane (the
// route sum rounds once); with an fp32 out route slot 0 writes out and the others planes.
void attach_planes(ChainParams& p, void* out, float* planes, bool out_bf16) {
  p.plane_stride = plane_stride_elems((int64_t)p.B * p.H * p.W * p.D);
  if (out_bf16) {
    p.out = planes;
    p.planes = planes + p.plane_stride;
  } else {
    p.out = static_cast<float*>(out);
    p.planes = planes;
  }
}

// The scan kernel of a planned call with its planes (bracketed by the events when given),
// then the route sum (left to the caller through defer for an fp32 out when defer is given).
hope_status_t enqueue_forward(const ChainParams& p, int d, void* out, bool out_bf16, hipStream_t s,
                              hipEvent_t begin, hipEvent_t end, RoutePlanes* defer) {
  const int64_t n_elem = (int64_t)p.B * p.H * p.W * p.D;
  hope_status_t st;
  if (begin && (st = hip_status(hipEventRecord(begin, s))) != HOPE_OK) return st;
  if ((st = hip_status(launch_scan(p, d, s))) != HOPE_OK) return st;
  if (end && (st = hip_status(hipEventRecord(end, s))) != HOPE_OK) return st;
  if (out_bf16)
    return hip_status(hope::launch_plane_sum_bf16(static_cast<unsigned short*>(out), p.out,
                                                  p.plane_stride, p.n_sel, n_elem, s));
  if (p.n_sel == 1) return st;
  if (defer) {  // the caller adds the planes to out
    defer->planes = p.planes;
    defer->stride = p.plane_stride;
    defer->n = p.n_sel - 1;
    return st;
  }
  return hip_status(
      hope::launch_plane_sum(static_cast<float*>(out), p.planes, p.plane_stride, p.n_sel - 1, n_elem, s));
}

hope_status_t scan_forward(const hope_fmap_t* x, const float* init_memories, uint32_t dirs,
                           int32_t chunk, void* out, const hope_scan2d_opts_t* opts,
                           RoutePlanes* defer) {
  if (defer) *defer = RoutePlanes{nullptr, 0, 0};
  hope_scan2d_opts_t o;
  if (opts) {
    o = *opts;
  } else {
    hope_scan2d_default_opts(&o);
  }
  ChainParams p;
  int d = 0;
  const hope_status_t st = plan_forward(x, init_memories, dirs, chunk, out, o, true, p, d);
  if (st != HOPE_OK) return st;
  const bool out_bf16 = o.out_dtype == HOPE_BF16;
  attach_planes(p, out, static_cast<float*>(o.workspace), out_bf16);
  return enqueue_forward(p, d, out, out_bf16, o.stream, o.scan_begin, o.scan_end, defer);
}

// Images per launch of the no-allocation forward: the most whose route planes fit in
// scratch_floats (all of them when no plane is needed); 0 when one image's do not.
int32_t images_per_slice(const hope_fmap_t* x, uint32_t dirs, int32_t out_dtype, int64_t scratch_floats) {
  const int n_planes = planes_for(dirs, out_dtype);
  if (n_planes <= 0) return x->B;
  const int64_t per_image = (int64_t)x->H * x->W * x->D;
  const int64_t cap = scratch_floats / n_planes;  // floats per plane, padding included
  int64_t b = std::min<int64_t>(cap / per_image, x->B);
  while (b > 0 && plane_stride_elems(b * per_image) > cap) --b;
  return (int32_t)b;
}

}  // namespace hope

// ---- the entry point that allocates nothing ---------------------------------------------
// Route planes in a file-scope device array of fixed size: each GPU the library runs on holds
// its own copy until the process ends.  In host code the array's name is not a device
// address: host code uses only the address hipGetSymbolAddress returns on each device.
constexpr size_t kScratchBytes = HOPE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices] = {};

// The scratch array's device address on the current device, looked up once per device
// (with that device current) and kept.
hipError_t scratch_of_current_device(float** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* addr = nullptr;
    e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = static_cast<float*>(addr);
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

void hope_scan2d_default_opts(hope_scan2d_opts_t* opts) {
  if (!opts) return;
  memset(opts, 0, sizeof(*opts));
  opts->eta_map = HOPE_ETA_SIGMOID;
  opts->eta_scale = 1.0f;
  opts->alpha_bias = 4.0f;
  opts->eps = 1e-6f;
}

size_t hope_scan2d_workspace_size(const hope_fmap_t* x, uint32_t dirs, int32_t chunk,
                                  const hope_scan2d_opts_t* opts) {
  if (check_fmap(x) != HOPE_OK || dirs == 0 || dirs > 15 || chunk < 0) return 0;
  const int32_t out_dtype = opts ? opts->out_dtype : HOPE_F32;
  if (out_dtype != HOPE_F32 && out_dtype != HOPE_BF16) return 0;
  return workspace_bytes_for(x, dirs, out_dtype);
}

hope_status_t hope_scan2d_forward(const hope_fmap_t* x, const float* init_memories,
                                  uint32_t dirs, int32_t chunk, void* out,
                                  const hope_scan2d_opts_t* opts) {
  return hope::scan_forward(x, init_memories, dirs, chunk, out, opts, nullptr);
}

hope_status_t hope_scan2d_forward_noalloc(const hope_fmap_t* x, const float* init_memories,
                                          uint32_t dirs, int32_t chunk, void* out,
                                          const hope_scan2d_opts_t* opts) {
  hope_scan2d_opts_t o;
  if (opts) {
    o = *opts;
  } else {
    hope_scan2d_default_opts(&o);
  }
  if (o.workspace || o.workspace_bytes) return HOPE_ERR_INVALID_ARG;  // the scratch array serves
  hope::ChainParams p;
  int d = 0;
  hope_status_t st = hope::plan_forward(x, init_memories, dirs, chunk, out, o, false, p, d);
  if (st != HOPE_OK) return st;
  const int64_t scratch_floats = (int64_t)(kScratchBytes / sizeof(float));
  const int32_t per_slice = hope::images_per_slice(x, dirs, o.out_dtype, scratch_floats);
  if (per_slice <= 0) return HOPE_ERR_WORKSPACE;  // one image's route planes exceed the scratch
  float* planes = nullptr;
  if ((st = hip_status(scratch_of_current_device(&planes))) != HOPE_OK) return st;

  // whole images per launch: every per-image pointer moves by the slice's first image
  const bool out_bf16 = o.out_dtype == HOPE_BF16;
  const int64_t map_elems = (int64_t)x->H * x->W * x->D;
  const int64_t state_floats = 4LL * d * d + 2LL * d;
  const int64_t per_image_state = 4LL * x->n_heads * state_floats;
  hipStream_t s = o.stream;
  if (o.scan_begin && (st = hip_status(hipEventRecord(o.scan_begin, s))) != HOPE_OK) return st;
  for (int32_t b0 = 0; b0 < x->B; b0 += per_slice) {
    const int32_t nb = std::min(per_slice, x->B - b0);
    hope::ChainParams q = p;
    q.B = nb;
    q.x = static_cast<const char*>(p.x) + b0 * map_elems * (p.x_bf16 ? 2 : 4);
    if (p.init_per_image) q.init = p.init + b0 * per_image_state;
    if (p.final_mem) q.final_mem = p.final_mem + b0 * per_image_state;
    if (p.steps) q.steps = p.steps + b0 * 4LL * x->n_heads * x->H * x->W;
    if (p.queries) q.queries = static_cast<const char*>(p.queries) + b0 * map_elems * (p.queries_bf16 ? 2 : 4);
    void* out_b = static_cast<char*>(out) + b0 * map_elems * (out_bf16 ? 2 : 4);
    hope::attach_planes(q, out_b, planes, out_bf16);
    const bool last = b0 + nb >= x->B;
    st = hope::enqueue_forward(q, d, out_b, out_bf16, s, nullptr, last ? o.scan_end : nullptr, nullptr);
    if (st != HOPE_OK) return st;
  }
  return HOPE_OK;
}

size_t hope_scan2d_backward_workspace_size(const hope_fmap_t* x, uint32_t dirs, int32_t chunk,
                                           const hope_scan2d_opts_t* opts) {
  (void)opts;
  if (check_fmap(x) != HOPE_OK || dirs == 0 || dirs > 15 || chunk < 0) return 0;
  return backward_workspace_bytes(x, backward_layout(x, dirs, chunk));
}

hope_status_t hope_scan2d_backward(const hope_fmap_t* x, const float* init_memories,
                                   uint32_t dirs, int32_t chunk, const float* grad_out,
                                   float* grad_x, float* grad_init,
                                   const hope_scan2d_opts_t* opts) {
  hope_scan2d_opts_t o;
  if (opts) {
    o = *opts;
  } else {
    hope_scan2d_default_opts(&o);
  }
  hope_status_t st = check_fmap(x);
  if (st != HOPE_OK) return st;
  if ((st = check_opts(&o)) != HOPE_OK) return st;
  if (!init_memories || !grad_out || !grad_x || !grad_init) return HOPE_ERR_INVALID_ARG;
  if (!aligned(init_memories, 16) || !aligned(grad_out, 16) || !aligned(grad_x, 16) || !aligned(grad_init, 16))
    return HOPE_ERR_INVALID_ARG;
  if (dirs == 0 || dirs > 15 || chunk < 0) return HOPE_ERR_INVALID_ARG;

  const int d = x->D / x->n_heads;
  const int64_t n_elem = (int64_t)x->B * x->H * x->W * x->D;
  const size_t x_bytes = (size_t)n_elem * (x->dtype == HOPE_BF16 ? 2 : 4);
  const size_t map_bytes = (size_t)n_elem * sizeof(float);
  const size_t state_floats = (size_t)4 * d * d + 2 * (size_t)d;
  const size_t init_bytes = (o.init_per_image ? (size_t)x->B : 1) * 4 * (size_t)x->n_heads * state_floats * sizeof(float);
  const Range r_gx = range_of(grad_x, map_bytes), r_gi = range_of(grad_init, init_bytes);
  const Range r_go = range_of(grad_out, map_bytes), r_x = range_of(x->data, x_bytes);
  const Range r_init = range_of(init_memories, init_bytes);
  if (overlaps(r_gx, r_x) || overlaps(r_gx, r_init) || overlaps(r_gx, r_go) || overlaps(r_gx, r_gi) ||
      overlaps(r_gi, r_x) || overlaps(r_gi, r_init) || overlaps(r_gi, r_go))
    return HOPE_ERR_INVALID_ARG;
  if (!backward_opts_supported(o)) return HOPE_ERR_UNSUPPORTED;
  if (d != 16 && d != 32 && d != 64) return HOPE_ERR_UNSUPPORTED;
  if (o.readout == HOPE_READOUT_RUNNING && d != 32) return HOPE_ERR_UNSUPPORTED;
  const BackLayout L = backward_layout(x, dirs, chunk);
  if (d != 32 && L.cmax > hope::backward_max_chunk(d)) return HOPE_ERR_UNSUPPORTED;
  const size_t ws_need = backward_workspace_bytes(x, L);
  if (!o.workspace || o.workspace_bytes < ws_need) return HOPE_ERR_WORKSPACE;
  const Range r_ws = range_of(o.workspace, o.workspace_bytes);
  if (overlaps(r_ws, r_gx) || overlaps(r_ws, r_gi) || overlaps(r_ws, r_go) || overlaps(r_ws, r_x) ||
      overlaps(r_ws, r_init))
    return HOPE_ERR_INVALID_ARG;
  if ((int64_t)L.n_sel * x->B * x->n_heads > INT32_MAX) return HOPE_ERR_INVALID_ARG;

  hope::BackParams p;
  memset(&p, 0, sizeof(p));
  p.x = x->data;
  p.init = init_memories;
  p.grad_out = grad_out;
  p.grad_x = grad_x;
  p.planes = static_cast<float*>(o.workspace);
  p.chain_ws = static_cast<float*>(o.workspace) + L.planes_floats;
  p.plane_stride = L.plane_stride;
  p.chain_floats = L.chain_floats;
  p.nck = L.nck;
  p.x_bf16 = x->dtype == HOPE_BF16;
  p.B = x->B;
  p.H = x->H;
  p.W = x->W;
  p.D = x->D;
  p.nh = x->n_heads;
  p.n_sel = slots_of(dirs, p.route_of_slot);
  p.chunk = chunk;
  p.init_per_image = o.init_per_image;
  p.eta_map = o.eta_map;
  p.eta_scale = o.eta_scale;
  p.alpha_bias = o.alpha_bias;
  p.eps = o.eps;
  p.readout = o.readout == HOPE_READOUT_RUNNING ? 1 : 0;

  hipStream_t s = o.stream;
  st = hip_status(hope::launch_chain_backward(p, d, grad_init, s));
  if (st != HOPE_OK || p.n_sel == 1) return st;
  return hip_status(hope::launch_plane_sum(grad_x, p.planes, p.plane_stride, p.n_sel - 1, n_elem, s));
}

const char* hope_scan2d_kernel_name(const hope_fmap_t* x, uint32_t dirs, int32_t chunk,
                                    const hope_scan2d_opts_t* opts) {
  hope_scan2d_opts_t o;
  if (opts) {
    o = *opts;
  } else {
    hope_scan2d_default_opts(&o);
  }
  if (check_fmap(x) != HOPE_OK || check_opts(&o) != HOPE_OK) return "";
  if (dirs == 0 || dirs > 15 || chunk < 0) return "";
  const int d = x->D / x->n_heads;
  if (d != 16 && d != 32 && d != 64) return "";
  hope::ChainParams p;
  memset(&p, 0, sizeof(p));
  p.x_bf16 = x->dtype == HOPE_BF16;
  p.B = x->B;
  p.H = x->H;
  p.W = x->W;
  p.D = x->D;
  p.nh = x->n_heads;
  p.n_sel = slots_of(dirs, p.route_of_slot);
  p.chunk = chunk;
  p.readout = o.readout;
  p.route_scales = o.route_scales;
  p.skip = o.skip;
  p.counts = o.counts;
  p.injection = o.injection;
  p.spectral = o.spectral;
  p.frozen = o.frozen;
  p.no_dgd = o.no_dgd;
  p.shared_init = o.shared_init;
  p.queries = o.queries;
  p.mem_chunk = o.mem_chunk;
  p.steps = o.step_map;
  return hope::scan_path_kernel(hope::select_scan_path(p, d));
}

const char* hope_status_string(hope_status_t status) {
  switch (status) {
    case HOPE_OK: return "HOPE_OK";
    case HOPE_ERR_INVALID_ARG: return "HOPE_ERR_INVALID_ARG";
    case HOPE_ERR_UNSUPPORTED: return "HOPE_ERR_UNSUPPORTED";
    case HOPE_ERR_WORKSPACE: return "HOPE_ERR_WORKSPACE";
    case HOPE_ERR_HIP: return "HOPE_ERR_HIP";
  }
  return "HOPE_ERR_UNKNOWN";
}

int hope_last_hip_error(void) { return g_last_hip_error; }

hope_status_t hope_debug_cross_scan(const hope_fmap_t* x, uint32_t dirs, void* routes,
                                    hipStream_t stream) {
  hope_status_t st = check_fmap(x);
  if (st != HOPE_OK) return st;
  if (!routes || !aligned(routes, 16) || dirs == 0 || dirs > 15) return HOPE_ERR_INVALID_ARG;
  int route_of_slot[4];
  const int n_sel = slots_of(dirs, route_of_slot);
  const int eb = x->dtype == HOPE_BF16 ? 2 : 4;
  const size_t n_elem = (size_t)x->B * x->H * x->W * x->D;
  if (overlaps(range_of(routes, n_elem * n_sel * eb), range_of(x->data, n_elem * eb)))
    return HOPE_ERR_INVALID_ARG;
  return hip_status(hope::launch_cross_scan(x->data, eb, x->B, x->H, x->W, x->D, route_of_slot,
                                            n_sel, routes, stream));
}

hope_status_t hope_debug_cross_merge(const void* routes, int32_t dtype, int32_t B, int32_t H,
                                     int32_t W, int32_t D, uint32_t dirs, float* out,
                                     hipStream_t stream) {
  if (!routes || !out || !aligned(routes, 16) || !aligned(out, 16)) return HOPE_ERR_INVALID_ARG;
  if (dtype != HOPE_F32 && dtype != HOPE_BF16) return HOPE_ERR_INVALID_ARG;
  if (B <= 0 || H <= 0 || W <= 0 || D <= 0 || dirs == 0 || dirs > 15) return HOPE_ERR_INVALID_ARG;
  if ((int64_t)H * W > INT32_MAX) return HOPE_ERR_INVALID_ARG;
  int route_of_slot[4];
  const int n_sel = slots_of(dirs, route_of_slot);
  const int eb = dtype == HOPE_BF16 ? 2 : 4;
  const size_t n_elem = (size_t)B * H * W * D;
  if (overlaps(range_of(routes, n_elem * n_sel * eb), range_of(out, n_elem * sizeof(float))))
    return HOPE_ERR_INVALID_ARG;
  return hip_status(hope::launch_cross_merge(routes, dtype == HOPE_BF16, B, H, W, D, route_of_slot,
                                             n_sel, out, stream));
}

}  // extern "C"
