"""Host-side checks of the C ABI: the library loads, exports every declared symbol,
its structs have the C layout, and every validation error returns before anything
is enqueued.  No test here launches a kernel; the device pointers passed to the
rejected calls are never dereferenced (validation is pure pointer arithmetic).
"""
import ctypes
import os
import shutil
import subprocess

import pytest

from self_modifying_memory_amd import _native as N

FAKE = 1 << 40          # 256-byte aligned address, never dereferenced


@pytest.fixture(scope="module")
def lib():
    return N.load_library()


def fmap(B=2, H=4, W=5, D=32, nh=1, dtype=N.HOPE_F32, data=FAKE):
    return N.hope_fmap_t(data, dtype, B, H, W, D, nh)


def opts(lib, **kw):
    o = N.hope_scan2d_opts_t()
    lib.hope_scan2d_default_opts(ctypes.byref(o))
    for k, v in kw.items():
        setattr(o, k, v)
    return o


def call(lib, x, init=FAKE + (1 << 30), dirs=15, chunk=0, out=FAKE + (2 << 30), o=None):
    return lib.hope_scan2d_forward(ctypes.byref(x), init, dirs, chunk, out,
                                   ctypes.byref(o) if o is not None else None)


def test_every_declared_function_is_exported(lib):
    names = N.header_functions()
    assert "hope_scan2d_forward" in names and "hope_scan2d_backward" in names
    assert "hope_block_forward" in names and "hope_block_workspace_size" in names and len(names) == 13
    for n in names:
        assert hasattr(lib, n), n


def test_struct_layout_matches_c():
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    src = r"""
#include <stdio.h>
#include <stddef.h>
#include "hope_scan2d.h"
int main(void) {
  printf("%zu %zu %zu %zu %zu %zu %zu %zu %zu %zu %zu %zu %zu %zu %zu %zu %zu %zu\n", sizeof(hope_fmap_t), sizeof(hope_scan2d_opts_t),
         offsetof(hope_fmap_t, dtype), offsetof(hope_fmap_t, n_heads),
         offsetof(hope_scan2d_opts_t, final_memories), offsetof(hope_scan2d_opts_t, workspace_bytes),
         offsetof(hope_scan2d_opts_t, eta_map), offsetof(hope_scan2d_opts_t, eta_scale),
         offsetof(hope_scan2d_opts_t, eps), offsetof(hope_scan2d_opts_t, init_per_image),
         offsetof(hope_scan2d_opts_t, out_dtype), offsetof(hope_scan2d_opts_t, scan_begin),
         offsetof(hope_scan2d_opts_t, scan_end), offsetof(hope_scan2d_opts_t, readout),
         offsetof(hope_scan2d_opts_t, reserved), offsetof(hope_scan2d_opts_t, queries),
         offsetof(hope_scan2d_opts_t, mem_chunk), offsetof(hope_scan2d_opts_t, step_map));
  return 0;
}
"""
    tmp = os.path.join(os.environ.get("TMPDIR", "/tmp"), f"hope_abi_{os.getpid()}")
    os.makedirs(tmp, exist_ok=True)
    with open(os.path.join(tmp, "abi.c"), "w") as f:
        f.write(src)
    exe = os.path.join(tmp, "abi")
    inc = os.path.dirname(N.HEADER_PATH)
    res = subprocess.run([gcc, "-D__HIP_PLATFORM_AMD__", "-I", inc, "-I", "/opt/rocm/include",
                          os.path.join(tmp, "abi.c"), "-o", exe], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    vals = [int(v) for v in subprocess.run([exe], capture_output=True, text=True).stdout.split()]
    F, O = N.hope_fmap_t, N.hope_scan2d_opts_t
    want = [ctypes.sizeof(F), ctypes.sizeof(O), F.dtype.offset, F.n_heads.offset,
            O.final_memories.offset, O.workspace_bytes.offset, O.eta_map.offset, O.eta_scale.offset,
            O.eps.offset, O.init_per_image.offset, O.out_dtype.offset, O.scan_begin.offset,
            O.scan_end.offset, O.readout.offset, O.reserved.offset, O.queries.offset,
            O.mem_chunk.offset, O.step_map.offset]
    assert vals == want


def test_default_opts_and_status_strings(lib):
    o = opts(lib)
    assert (o.eta_map, o.eta_scale, o.alpha_bias, o.init_per_image) == (0, 1.0, 4.0, 0)
    assert abs(o.eps - 1e-6) < 1e-12 and o.final_memories is None and o.workspace is None
    assert o.scan_begin is None and o.scan_end is None and o.readout == N.HOPE_READOUT_BOUNDARY
    for code, name in [(0, b"HOPE_OK"), (-1, b"HOPE_ERR_INVALID_ARG"), (-2, b"HOPE_ERR_UNSUPPORTED"),
                       (-3, b"HOPE_ERR_WORKSPACE"), (-4, b"HOPE_ERR_HIP")]:
        assert lib.hope_status_string(code) == name
    assert lib.hope_last_hip_error() == 0


def test_workspace_size(lib):
    x = fmap(B=2, H=4, W=5, D=32)
    n = 2 * 4 * 5 * 32
    plane = (n + 63) // 64 * 64 * 4
    cnt = 0  # no counters: the route sum is a separate streaming pass
    assert lib.hope_scan2d_workspace_size(ctypes.byref(x), 15, 0, None) == cnt + 3 * plane
    assert lib.hope_scan2d_workspace_size(ctypes.byref(x), 5, 0, None) == cnt + plane
    assert lib.hope_scan2d_workspace_size(ctypes.byref(x), 4, 0, None) == 0
    assert lib.hope_scan2d_workspace_size(ctypes.byref(fmap(B=0)), 15, 0, None) == 0
    assert lib.hope_scan2d_workspace_size(ctypes.byref(x), 0, 0, None) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), N.HOPE_ERR_INVALID_ARG),
    (dict(H=-1), N.HOPE_ERR_INVALID_ARG),
    (dict(W=0), N.HOPE_ERR_INVALID_ARG),
    (dict(D=33), N.HOPE_ERR_INVALID_ARG),            # not a multiple of n_heads (33 % 2)
    (dict(dtype=7), N.HOPE_ERR_INVALID_ARG),
    (dict(data=0), N.HOPE_ERR_INVALID_ARG),
    (dict(data=FAKE + 8), N.HOPE_ERR_INVALID_ARG),    # misaligned
    (dict(D=16, nh=2), N.HOPE_ERR_UNSUPPORTED),       # d = 8
    (dict(D=96, nh=1), N.HOPE_ERR_UNSUPPORTED),       # d = 96
])
def test_shape_errors(lib, kw, code):
    base = dict(B=2, H=4, W=5, D=32, nh=2)
    base.update(kw)
    x = fmap(**base)
    assert call(lib, x, o=opts(lib)) == code


def test_argument_errors(lib):
    x = fmap()
    o = opts(lib)
    assert call(lib, x, dirs=0, o=o) == N.HOPE_ERR_INVALID_ARG
    assert call(lib, x, dirs=16, o=o) == N.HOPE_ERR_INVALID_ARG
    assert call(lib, x, chunk=-1, o=o) == N.HOPE_ERR_INVALID_ARG
    assert call(lib, x, init=0, o=o) == N.HOPE_ERR_INVALID_ARG
    assert call(lib, x, out=0, o=o) == N.HOPE_ERR_INVALID_ARG
    assert call(lib, x, out=FAKE + (2 << 30) + 4, o=o) == N.HOPE_ERR_INVALID_ARG
    # out overlapping x / init
    assert call(lib, x, out=FAKE + 256, o=o) == N.HOPE_ERR_INVALID_ARG
    assert call(lib, x, out=FAKE + (1 << 30), o=o) == N.HOPE_ERR_INVALID_ARG
    for k, v in [("eta_map", 2), ("eta_scale", -1.0), ("eta_scale", float("nan")),
                 ("alpha_bias", float("inf")), ("eps", -1e-6), ("init_per_image", 2), ("out_dtype", 2),
                 ("scan_begin", FAKE), ("scan_end", FAKE),  # the event pair is both or neither
                 ("readout", 2), ("reserved", 1), ("injection", 3), ("spectral", -1),
                 ("queries", FAKE + (3 << 30) + 8),
                 ("frozen", 8), ("no_dgd", 2), ("shared_init", 2), ("counts", FAKE + (3 << 30) + 4),
                 ("skip", FAKE + (3 << 30) + 2), ("step_map", FAKE + (3 << 30) + 2),
                 ("step_map", FAKE + (2 << 30) + 64)]:  # misaligned; overlapping out
        assert call(lib, x, o=opts(lib, **{k: v})) == N.HOPE_ERR_INVALID_ARG, k
    # final memories overlapping out, misaligned workspace
    assert call(lib, x, o=opts(lib, final_memories=FAKE + (2 << 30))) == N.HOPE_ERR_INVALID_ARG
    assert call(lib, x, o=opts(lib, workspace=FAKE + (3 << 30) + 16,
                               workspace_bytes=1 << 20)) == N.HOPE_ERR_INVALID_ARG


def test_workspace_errors(lib):
    x = fmap()
    need = lib.hope_scan2d_workspace_size(ctypes.byref(x), 15, 0, None)
    assert call(lib, x, o=opts(lib)) == N.HOPE_ERR_WORKSPACE
    assert call(lib, x, o=None) == N.HOPE_ERR_WORKSPACE
    small = opts(lib, workspace=FAKE + (3 << 30), workspace_bytes=need - 4)
    assert call(lib, x, o=small) == N.HOPE_ERR_WORKSPACE
    overlap = opts(lib, workspace=FAKE + (2 << 30), workspace_bytes=need)
    assert call(lib, x, o=overlap) == N.HOPE_ERR_INVALID_ARG


def test_workspace_size_counts_route_planes(lib):
    x = fmap(B=2, H=4, W=5, D=32)
    plane = 2 * 4 * 5 * 32 * 4  # one fp32 map, already a multiple of 256 bytes
    bf = opts(lib, out_dtype=N.HOPE_BF16)
    for dirs, n_sel in [(1, 1), (5, 2), (15, 4)]:
        assert lib.hope_scan2d_workspace_size(ctypes.byref(x), dirs, 0, None) == (n_sel - 1) * plane
        assert lib.hope_scan2d_workspace_size(ctypes.byref(x), dirs, 0, ctypes.byref(bf)) == n_sel * plane
    # a single route with a bf16 out still needs its fp32 plane
    assert call(lib, x, dirs=1, o=bf) == N.HOPE_ERR_WORKSPACE
    assert lib.hope_scan2d_workspace_size(ctypes.byref(x), 15, 0, ctypes.byref(opts(lib, out_dtype=5))) == 0


def test_debug_export_errors(lib):
    x = fmap()
    assert lib.hope_debug_cross_scan(ctypes.byref(x), 0, FAKE + (2 << 30), None) == N.HOPE_ERR_INVALID_ARG
    assert lib.hope_debug_cross_scan(ctypes.byref(x), 15, FAKE + 64, None) == N.HOPE_ERR_INVALID_ARG
    assert lib.hope_debug_cross_scan(ctypes.byref(fmap(B=0)), 15, FAKE + (2 << 30), None) == N.HOPE_ERR_INVALID_ARG
    assert lib.hope_debug_cross_merge(FAKE, 3, 2, 4, 5, 32, 15, FAKE + (2 << 30), None) == N.HOPE_ERR_INVALID_ARG
    assert lib.hope_debug_cross_merge(FAKE, 0, 2, 4, 5, 32, 15, FAKE + 64, None) == N.HOPE_ERR_INVALID_ARG
    assert lib.hope_debug_cross_merge(FAKE, 0, 2, 0, 5, 32, 15, FAKE + (2 << 30), None) == N.HOPE_ERR_INVALID_ARG


def test_variant_option_errors(lib):
    x = fmap()
    ws = lib.hope_scan2d_workspace_size(ctypes.byref(x), 15, 0, None)
    base = dict(workspace=FAKE + (3 << 30), workspace_bytes=ws)
    # a negative working-memory chunk length
    assert call(lib, x, o=opts(lib, mem_chunk=-1, **base)) == N.HOPE_ERR_INVALID_ARG
    # shared and per-image initial states exclude each other
    assert call(lib, x, o=opts(lib, shared_init=1, init_per_image=1, **base)) == N.HOPE_ERR_INVALID_ARG
    # scales / skip / counters overlapping out
    out = FAKE + (2 << 30)
    for k in ("route_scales", "skip", "counts"):
        assert call(lib, x, o=opts(lib, **{k: out}, **base)) == N.HOPE_ERR_INVALID_ARG, k
    # counters overlapping the workspace
    assert call(lib, x, o=opts(lib, counts=FAKE + (3 << 30) + 64, **base)) == N.HOPE_ERR_INVALID_ARG


def bcall(lib, x, init=FAKE + (1 << 30), dirs=15, chunk=0, gout=FAKE + (2 << 30),
          gx=FAKE + (4 << 30), gi=FAKE + (5 << 30), o=None):
    return lib.hope_scan2d_backward(ctypes.byref(x), init, dirs, chunk, gout, gx, gi,
                                    ctypes.byref(o) if o is not None else None)


def test_backward_workspace_size(lib):
    n_elem = 2 * 4 * 5 * 32
    plane = (n_elem + 63) // 64 * 64
    # d = 16 (token-serial kernel), S = 1056, N = 20: aligned chunks are rows of 5 (4 chunks)
    # and columns of 4 (5 chunks) -> 5 + 1 state records and one chunk's gain trajectory
    x16 = fmap(B=2, H=4, W=5, D=32, nh=2)
    per_chain = ((5 + 1) * 1056 + 5 * 16 * 16 + 63) // 64 * 64
    want = (3 * plane + 4 * 2 * 2 * per_chain) * 4
    assert lib.hope_scan2d_backward_workspace_size(ctypes.byref(x16), 15, 0, None) == want
    # d = 32 (blocked kernel), S = 4160: the state adjoint, then per chunk P_c (1024) and a
    # record per 16-token block (its end gain, six 16 x 32 token arrays, 8 x 16 scalars:
    # 4224); one block per 5-token chunk, 5 chunks at most
    blk = 1024 + 6 * 16 * 32 + 8 * 16
    x = fmap(B=2, H=4, W=5, D=32, nh=1)
    per_chain = (4160 + 5 * (1024 + blk) + 63) // 64 * 64
    want = (3 * plane + 4 * 2 * 1 * per_chain) * 4
    assert lib.hope_scan2d_backward_workspace_size(ctypes.byref(x), 15, 0, None) == want
    # route 0 alone: no planes, two chains of 4 row chunks of 5 tokens
    assert lib.hope_scan2d_backward_workspace_size(ctypes.byref(x), 1, 0, None) == \
        (2 * ((4160 + 4 * (1024 + blk) + 63) // 64 * 64)) * 4
    # rows of 200 tokens at d = 32: one chunk per row, 13 blocks each
    big = fmap(B=1, H=2, W=200, D=32, nh=1)
    assert lib.hope_scan2d_backward_workspace_size(ctypes.byref(big), 1, 0, None) == \
        ((4160 + 2 * (1024 + 13 * blk) + 63) // 64 * 64) * 4
    assert lib.hope_scan2d_backward_workspace_size(ctypes.byref(x), 0, 0, None) == 0
    assert lib.hope_scan2d_backward_workspace_size(ctypes.byref(x), 15, -1, None) == 0


def test_backward_argument_errors(lib):
    x = fmap()
    ws = lib.hope_scan2d_backward_workspace_size(ctypes.byref(x), 15, 0, None)
    base = dict(workspace=FAKE + (8 << 30), workspace_bytes=ws)
    o = opts(lib, **base)
    assert bcall(lib, x, gout=0, o=o) == N.HOPE_ERR_INVALID_ARG
    assert bcall(lib, x, gx=0, o=o) == N.HOPE_ERR_INVALID_ARG
    assert bcall(lib, x, gi=0, o=o) == N.HOPE_ERR_INVALID_ARG
    assert bcall(lib, x, gx=FAKE + 8, o=o) == N.HOPE_ERR_INVALID_ARG      # misaligned
    assert bcall(lib, x, gx=FAKE, o=o) == N.HOPE_ERR_INVALID_ARG          # grad_x over x
    assert bcall(lib, x, gi=FAKE + (2 << 30), o=o) == N.HOPE_ERR_INVALID_ARG  # grad_init over grad_out
    assert bcall(lib, x, dirs=0, o=o) == N.HOPE_ERR_INVALID_ARG
    # a workspace is always needed
    assert bcall(lib, x, o=opts(lib)) == N.HOPE_ERR_WORKSPACE
    assert bcall(lib, x, o=opts(lib, workspace=FAKE + (8 << 30), workspace_bytes=ws - 4)) == N.HOPE_ERR_WORKSPACE
    # options outside the honoured set
    for kw in (dict(no_dgd=1), dict(mem_chunk=3),
               dict(injection=1), dict(spectral=2), dict(frozen=1), dict(final_memories=FAKE + (6 << 30)),
               dict(out_dtype=N.HOPE_BF16)):
        assert bcall(lib, x, o=opts(lib, **kw, **base)) == N.HOPE_ERR_UNSUPPORTED, kw
    # the running readout is honoured at d = 32 only
    x16 = fmap(D=32, nh=2)
    ws16 = lib.hope_scan2d_backward_workspace_size(ctypes.byref(x16), 15, 0, None)
    assert bcall(lib, x16, o=opts(lib, readout=N.HOPE_READOUT_RUNNING, workspace=FAKE + (8 << 30),
                                  workspace_bytes=ws16)) == N.HOPE_ERR_UNSUPPORTED
    # head dimension and chunk length limits
    assert bcall(lib, fmap(D=8, nh=1), o=o) == N.HOPE_ERR_UNSUPPORTED
    big = fmap(B=1, H=2, W=200, D=16, nh=1)
    wsb = lib.hope_scan2d_backward_workspace_size(ctypes.byref(big), 1, 0, None)
    assert bcall(lib, big, dirs=1, o=opts(lib, workspace=FAKE + (8 << 30), workspace_bytes=wsb)) == \
        N.HOPE_ERR_UNSUPPORTED                                            # d = 16: rows of 200 > 128
    d64 = fmap(B=1, H=4, W=40, D=64, nh=1)
    wsd = lib.hope_scan2d_backward_workspace_size(ctypes.byref(d64), 1, 0, None)
    assert bcall(lib, d64, dirs=1, o=opts(lib, workspace=FAKE + (8 << 30), workspace_bytes=wsd)) == \
        N.HOPE_ERR_UNSUPPORTED                                            # d = 64: rows of 40 > 32


def test_block_weights_layout_matches_c():
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    src = r"""
#include <stdio.h>
#include <stddef.h>
#include "hope_block.h"
int main(void) {
  printf("%zu %zu %zu %zu\n", sizeof(hope_block_weights_t), offsetof(hope_block_weights_t, w_q),
         offsetof(hope_block_weights_t, init_memories), offsetof(hope_block_weights_t, b2));
  return 0;
}
"""
    import subprocess, tempfile, os
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "t.c")
        open(c, "w").write(src)
        exe = os.path.join(d, "t")
        inc = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
        r = subprocess.run([gcc, c, "-o", exe, "-I", inc,
                            "-I", "/opt/rocm/include", "-D__HIP_PLATFORM_AMD__"], capture_output=True, text=True)
        if r.returncode:
            pytest.skip("cannot compile the layout probe: " + r.stderr[:200])
        got = [int(v) for v in subprocess.run([exe], capture_output=True, text=True).stdout.split()]
    S = N.hope_block_weights_t
    assert got == [ctypes.sizeof(S), S.w_q.offset, S.init_memories.offset, S.b2.offset]


def test_block_workspace_size_and_errors(lib):
    #                                   B, H,  W,  D,   D_m, nh, ffn,  chunk
    assert lib.hope_block_workspace_size(2, 14, 14, 384, 192, 12, 1536, 0) > 0   # the pages' evaluated form
    assert lib.hope_block_workspace_size(2, 14, 14, 96, 48, 3, 384, 0) > 0
    assert lib.hope_block_workspace_size(2, 14, 14, 384, 384, 6, 1536, 0) > 0
    assert lib.hope_block_workspace_size(2, 14, 14, 100, 48, 3, 400, 0) == 0   # D % 16
    assert lib.hope_block_workspace_size(2, 14, 14, 96, 40, 2, 384, 0) == 0    # D_m % 16
    assert lib.hope_block_workspace_size(2, 14, 14, 128, 128, 3, 512, 0) == 0  # D_m % n_heads
    assert lib.hope_block_workspace_size(2, 14, 14, 128, 64, 2, 500, 0) == 0   # ffn_dim % 16
    assert lib.hope_block_workspace_size(2, 14, 14, 2048, 64, 2, 512, 0) == 0  # D > 1024
    assert lib.hope_block_workspace_size(0, 14, 14, 128, 64, 2, 512, 0) == 0
    assert lib.hope_block_workspace_size(2, 14, 14, 128, 0, 2, 512, 0) == 0
    w = N.hope_block_weights_t()
    # null weights: rejected before anything is enqueued (no device needed)
    assert lib.hope_block_forward(FAKE, 1, 4, 4, 128, 64, 2, 512, 0, ctypes.byref(w), FAKE + (1 << 30),
                                  FAKE + (2 << 30), 1 << 30, None) == N.HOPE_ERR_INVALID_ARG
    for name in N.BLOCK_WEIGHT_FIELDS:
        setattr(w, name, FAKE + (3 << 30))
    # a head dimension of 128 is well formed but not supported
    assert lib.hope_block_forward(FAKE, 1, 4, 4, 128, 128, 1, 512, 0, ctypes.byref(w), FAKE + (1 << 30),
                                  FAKE + (2 << 30), 1 << 30, None) == N.HOPE_ERR_UNSUPPORTED
    # x and out alias
    assert lib.hope_block_forward(FAKE, 1, 4, 4, 128, 64, 2, 512, 0, ctypes.byref(w), FAKE,
                                  FAKE + (2 << 30), 1 << 30, None) == N.HOPE_ERR_INVALID_ARG
    # short workspace
    assert lib.hope_block_forward(FAKE, 1, 4, 4, 128, 64, 2, 512, 0, ctypes.byref(w), FAKE + (1 << 30),
                                  FAKE + (2 << 30), 256, None) == N.HOPE_ERR_WORKSPACE


def test_noalloc_entry_errors(lib):
    # the entry point that allocates nothing: every check before anything is enqueued (no
    # device is touched for these: the scratch array is looked up only after them)
    x = fmap(B=2, H=4, W=5, D=32, nh=1)
    assert lib.hope_scan2d_forward_noalloc(ctypes.byref(x), FAKE + (1 << 30), 15, 0, FAKE + (2 << 30),
                                           ctypes.byref(opts(lib, workspace=FAKE + (4 << 30),
                                                             workspace_bytes=1 << 20))) == N.HOPE_ERR_INVALID_ARG
    assert lib.hope_scan2d_forward_noalloc(ctypes.byref(x), FAKE + (1 << 30), 0, 0, FAKE + (2 << 30),
                                           None) == N.HOPE_ERR_INVALID_ARG
    assert lib.hope_scan2d_forward_noalloc(ctypes.byref(fmap(D=8, nh=1)), FAKE + (1 << 30), 15, 0,
                                           FAKE + (2 << 30), None) == N.HOPE_ERR_UNSUPPORTED
    # one image's three fp32 route planes (256 x 256 x 128 x 4 bytes each) exceed the 64 MiB
    big = fmap(B=1, H=256, W=256, D=128, nh=2, data=FAKE)
    assert 3 * 256 * 256 * 128 * 4 > N.HOPE_NOALLOC_SCRATCH_BYTES
    assert lib.hope_scan2d_forward_noalloc(ctypes.byref(big), FAKE + (1 << 33), 15, 0, FAKE + (1 << 34),
                                           None) == N.HOPE_ERR_WORKSPACE
    # header constant and binding agree
    text = open(N.HEADER_PATH).read()
    assert "#define HOPE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)" in text


def test_kernel_name_query(lib):
    def name(x, dirs=15, chunk=0, o=None):
        return lib.hope_scan2d_kernel_name(ctypes.byref(x), dirs, chunk,
                                           ctypes.byref(o) if o is not None else None).decode()
    assert name(fmap(B=128, H=14, W=14, D=384, nh=6, dtype=N.HOPE_BF16)) == "chain_mfma_kernel"
    assert name(fmap(B=1, H=8, W=8, D=16, nh=1, dtype=N.HOPE_F32)) == "chain_kernel"
    assert name(fmap(D=8, nh=1)) == ""                       # d = 8: rejected by the forward
    assert name(fmap(), dirs=0) == ""
