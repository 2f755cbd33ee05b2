// Internal entry of the scan forward (api.hip) for callers inside the library.
#pragma once

#include <stdint.h>

#include "../../include/hope_scan2d.h"

namespace hope {

// Route planes left unsummed: out holds the first selected route's result and planes
// [k * stride, k * stride + n_elem) for k < n the others, in slot order; the route sum is
// out + planes[0] + ... + planes[n - 1], added left to right.
struct RoutePlanes {
  const float* planes;
  int64_t stride;
  int n;
};

// hope_scan2d_forward with the same checks and results; with defer non-null and fp32 out,
// the final route sum is left to the caller (defer receives the planes, in the workspace).
hope_status_t scan_forward(const hope_fmap_t* x, const float* init_memories, uint32_t dirs,
                           int32_t chunk, void* out, const hope_scan2d_opts_t* opts,
                           RoutePlanes* defer);

}  // namespace hope
