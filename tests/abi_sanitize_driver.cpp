// Host-side driver of the C ABI's argument checking, built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the library's host code (tests/test_abi_sanitized.py).
// Every call here is rejected before anything is enqueued, so no GPU is touched; the device
// pointers are fake addresses that the library never dereferences.  Exit status 0 when every
// call returns the expected status.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "hope_block.h"
#include "hope_scan2d.h"

static int failures = 0;

#define EXPECT(call, want)                                                                  \
  do {                                                                                      \
    const int got_ = (int)(call);                                                           \
    if (got_ != (int)(want)) {                                                              \
      fprintf(stderr, "line %d: %s returned %d, expected %d\n", __LINE__, #call, got_, (int)(want)); \
      ++failures;                                                                           \
    }                                                                                       \
  } while (0)

static void* fake(uint64_t gib) { return reinterpret_cast<void*>((uint64_t(1) << 40) + (gib << 30)); }

static hope_fmap_t fmap(int B, int H, int W, int D, int nh, hope_dtype_t dt = HOPE_F32, void* data = fake(0)) {
  hope_fmap_t x;
  x.data = data;
  x.dtype = dt;
  x.B = B;
  x.H = H;
  x.W = W;
  x.D = D;
  x.n_heads = nh;
  return x;
}

static hope_scan2d_opts_t defaults() {
  hope_scan2d_opts_t o;
  hope_scan2d_default_opts(&o);
  return o;
}

int main() {
  const float* init = static_cast<const float*>(fake(1));
  void* out = fake(2);
  hope_fmap_t x = fmap(2, 4, 5, 32, 1);
  hope_scan2d_opts_t o = defaults();

  // shapes
  const int bad[][5] = {{0, 4, 5, 32, 1}, {2, 0, 5, 32, 1}, {2, 4, 0, 32, 1}, {2, 4, 5, 0, 1},
                        {2, 4, 5, 32, 0}, {2, 4, 5, 32, 3}, {-1, 4, 5, 32, 1}};
  for (const auto& s : bad) {
    hope_fmap_t y = fmap(s[0], s[1], s[2], s[3], s[4]);
    EXPECT(hope_scan2d_forward(&y, init, 15, 0, out, nullptr), HOPE_ERR_INVALID_ARG);
    EXPECT(hope_scan2d_workspace_size(&y, 15, 0, nullptr), 0);
    EXPECT(hope_scan2d_backward_workspace_size(&y, 15, 0, nullptr), 0);
  }
  hope_fmap_t d8 = fmap(2, 4, 5, 8, 1);
  EXPECT(hope_scan2d_forward(&d8, init, 15, 0, out, nullptr), HOPE_ERR_UNSUPPORTED);
  // sizes near the integer limits: rejected, no overflow in the checks
  hope_fmap_t huge = fmap(0x7fffffff, 0x7fffffff, 0x7fffffff, 0x7fffffc0, 1);
  EXPECT(hope_scan2d_forward(&huge, init, 15, 0, out, nullptr), HOPE_ERR_INVALID_ARG);
  EXPECT(hope_scan2d_workspace_size(&huge, 15, 0, nullptr), 0);
  EXPECT(hope_scan2d_backward_workspace_size(&huge, 15, 0, nullptr), 0);
  hope_fmap_t wide = fmap(1, 46341, 46341, 16, 1);  // H * W above 2^31
  EXPECT(hope_scan2d_forward(&wide, init, 15, 0, out, nullptr), HOPE_ERR_INVALID_ARG);

  // arguments
  EXPECT(hope_scan2d_forward(nullptr, init, 15, 0, out, nullptr), HOPE_ERR_INVALID_ARG);
  EXPECT(hope_scan2d_forward(&x, nullptr, 15, 0, out, nullptr), HOPE_ERR_INVALID_ARG);
  EXPECT(hope_scan2d_forward(&x, init, 15, 0, nullptr, nullptr), HOPE_ERR_INVALID_ARG);
  EXPECT(hope_scan2d_forward(&x, init, 0, 0, out, nullptr), HOPE_ERR_INVALID_ARG);
  EXPECT(hope_scan2d_forward(&x, init, 16, 0, out, nullptr), HOPE_ERR_INVALID_ARG);
  EXPECT(hope_scan2d_forward(&x, init, 15, -1, out, nullptr), HOPE_ERR_INVALID_ARG);
  EXPECT(hope_scan2d_forward(&x, init, 15, 0, static_cast<char*>(out) + 4, nullptr), HOPE_ERR_INVALID_ARG);
  EXPECT(hope_scan2d_forward(&x, init, 15, 0, fake(0), nullptr), HOPE_ERR_INVALID_ARG);  // out over x
  hope_fmap_t xm = fmap(2, 4, 5, 32, 1, HOPE_F32, static_cast<char*>(fake(0)) + 8);
  EXPECT(hope_scan2d_forward(&xm, init, 15, 0, out, nullptr), HOPE_ERR_INVALID_ARG);
  // option flags
  const int32_t bad_flag = 7;
  o = defaults(); o.eta_map = static_cast<hope_eta_map_t>(bad_flag);
  EXPECT(hope_scan2d_forward(&x, init, 15, 0, out, &o), HOPE_ERR_INVALID_ARG);
  o = defaults(); o.eta_scale = -1.f;
  EXPECT(hope_scan2d_forward(&x, init, 15, 0, out, &o), HOPE_ERR_INVALID_ARG);
  o = defaults(); o.readout = bad_flag;
  EXPECT(hope_scan2d_forward(&x, init, 15, 0, out, &o), HOPE_ERR_INVALID_ARG);
  o = defaults(); o.frozen = 8u;
  EXPECT(hope_scan2d_forward(&x, init, 15, 0, out, &o), HOPE_ERR_INVALID_ARG);
  o = defaults(); o.shared_init = 1; o.init_per_image = 1;
  EXPECT(hope_scan2d_forward(&x, init, 15, 0, out, &o), HOPE_ERR_INVALID_ARG);
  o = defaults(); o.mem_chunk = -2;
  EXPECT(hope_scan2d_forward(&x, init, 15, 0, out, &o), HOPE_ERR_INVALID_ARG);
  o = defaults(); o.reserved = 1;
  EXPECT(hope_scan2d_forward(&x, init, 15, 0, out, &o), HOPE_ERR_INVALID_ARG);
  // workspace
  const size_t ws = hope_scan2d_workspace_size(&x, 15, 0, nullptr);
  if (ws != 3 * (((size_t)2 * 4 * 5 * 32 + 63) / 64 * 64) * 4) {
    fprintf(stderr, "workspace size %zu\n", ws);
    ++failures;
  }
  EXPECT(hope_scan2d_forward(&x, init, 15, 0, out, nullptr), HOPE_ERR_WORKSPACE);
  o = defaults(); o.workspace = fake(4); o.workspace_bytes = ws - 4;
  EXPECT(hope_scan2d_forward(&x, init, 15, 0, out, &o), HOPE_ERR_WORKSPACE);
  o = defaults(); o.workspace = out; o.workspace_bytes = ws;  // workspace over out
  EXPECT(hope_scan2d_forward(&x, init, 15, 0, out, &o), HOPE_ERR_INVALID_ARG);
  o = defaults(); o.workspace = static_cast<char*>(fake(4)) + 16; o.workspace_bytes = ws;
  EXPECT(hope_scan2d_forward(&x, init, 15, 0, out, &o), HOPE_ERR_INVALID_ARG);

  // backward
  float* gx = static_cast<float*>(fake(5));
  float* gi = static_cast<float*>(fake(6));
  const float* go = static_cast<const float*>(fake(7));
  const size_t bws = hope_scan2d_backward_workspace_size(&x, 15, 0, nullptr);
  EXPECT(hope_scan2d_backward(&x, init, 15, 0, go, gx, gi, nullptr), HOPE_ERR_WORKSPACE);
  o = defaults(); o.workspace = fake(8); o.workspace_bytes = bws;
  EXPECT(hope_scan2d_backward(&x, init, 15, 0, nullptr, gx, gi, &o), HOPE_ERR_INVALID_ARG);
  EXPECT(hope_scan2d_backward(&x, init, 15, 0, go, static_cast<float*>(fake(0)), gi, &o), HOPE_ERR_INVALID_ARG);
  hope_fmap_t x16 = fmap(2, 4, 5, 32, 2);  // d = 16: the running readout is honoured at d = 32 only
  o = defaults(); o.workspace = fake(8); o.workspace_bytes = hope_scan2d_backward_workspace_size(&x16, 15, 0, nullptr);
  o.readout = HOPE_READOUT_RUNNING;
  EXPECT(hope_scan2d_backward(&x16, init, 15, 0, go, gx, gi, &o), HOPE_ERR_UNSUPPORTED);
  hope_fmap_t rows200 = fmap(1, 2, 200, 16, 1);  // d = 16: rows of 200 > 128
  o = defaults(); o.workspace = fake(8); o.workspace_bytes = hope_scan2d_backward_workspace_size(&rows200, 1, 0, nullptr);
  EXPECT(hope_scan2d_backward(&rows200, init, 1, 0, go, gx, gi, &o), HOPE_ERR_UNSUPPORTED);

  // the entry point that allocates nothing
  o = defaults(); o.workspace = fake(4); o.workspace_bytes = 1 << 20;
  EXPECT(hope_scan2d_forward_noalloc(&x, init, 15, 0, out, &o), HOPE_ERR_INVALID_ARG);
  EXPECT(hope_scan2d_forward_noalloc(&x, init, 0, 0, out, nullptr), HOPE_ERR_INVALID_ARG);
  EXPECT(hope_scan2d_forward_noalloc(&d8, init, 15, 0, out, nullptr), HOPE_ERR_UNSUPPORTED);
  hope_fmap_t big = fmap(1, 256, 256, 128, 2);
  EXPECT(hope_scan2d_forward_noalloc(&big, static_cast<const float*>(fake(32)), 15, 0, fake(64), nullptr),
         HOPE_ERR_WORKSPACE);

  // kernel names
  hope_fmap_t s3 = fmap(128, 14, 14, 384, 6, HOPE_BF16);
  if (strcmp(hope_scan2d_kernel_name(&s3, 15, 0, nullptr), "chain_mfma_kernel") != 0) ++failures;
  hope_fmap_t s1 = fmap(16, 56, 56, 96, 3, HOPE_BF16);
  if (strcmp(hope_scan2d_kernel_name(&s1, 15, 0, nullptr), "chain_chunk_kernel") != 0) ++failures;
  if (strcmp(hope_scan2d_kernel_name(&d8, 15, 0, nullptr), "") != 0) ++failures;

  // permutation exports
  EXPECT(hope_debug_cross_scan(&x, 0, fake(3), nullptr), HOPE_ERR_INVALID_ARG);
  EXPECT(hope_debug_cross_merge(fake(3), 3, 2, 4, 5, 32, 15, static_cast<float*>(fake(2)), nullptr),
         HOPE_ERR_INVALID_ARG);

  // the block
  EXPECT(hope_block_workspace_size(2, 14, 14, 100, 48, 3, 400, 0), 0);
  EXPECT(hope_block_workspace_size(0x7fffffff, 0x7fffffff, 0x7fffffff, 1024, 1024, 16, 16384, 0), 0);
  if (hope_block_workspace_size(2, 14, 14, 384, 192, 12, 1536, 0) == 0) ++failures;
  hope_block_weights_t wt;
  memset(&wt, 0, sizeof(wt));
  EXPECT(hope_block_forward(static_cast<const float*>(fake(0)), 1, 4, 4, 128, 64, 2, 512, 0, &wt,
                            static_cast<float*>(fake(1)), fake(2), 1 << 30, nullptr),
         HOPE_ERR_INVALID_ARG);

  if (strcmp(hope_status_string(HOPE_ERR_WORKSPACE), "HOPE_ERR_WORKSPACE") != 0) ++failures;
  if (failures) fprintf(stderr, "%d failures\n", failures);
  else printf("all argument checks as expected\n");
  return failures ? 1 : 0;
}
