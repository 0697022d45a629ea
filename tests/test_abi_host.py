"""C-ABI library on the host (no GPU): it loads, exports every function the
header declares, and its host-only paths (status strings, sizes, planning,
argument checks) behave as documented.  No call here reaches a kernel."""
import ctypes
import os
import re

import pytest

from w4_gemm_gated_amd import _binding

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(REPO, "include", "spear_w4ec.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_binding.LIB_PATH),
                                reason="libspear_w4ec.so not built (run __graft_entry__.build())")


@pytest.fixture(scope="module")
def lib():
    return _binding.load()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(spear_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = header_functions()
    for required in ("spear_w4ec_linear", "spear_pack_w4", "spear_dispatch_plan"):
        assert required in names
    assert set(names) == set(_binding.EXPORTS)


def test_library_exports_every_declared_function(lib):
    for name in header_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_status_strings_and_version(lib):
    assert lib.spear_abi_version() == 3
    for code, name in _binding.STATUS_NAMES.items():
        assert lib.spear_status_str(code).decode().startswith(name)
    assert lib.spear_status_str(99).decode() == "SPEAR_ERR_UNKNOWN"


def test_service_entry_points_check_arguments(lib):
    out = ctypes.c_uint32(0)
    buf = ctypes.create_string_buffer(64)
    # spear_take_error: null pointers, a workspace smaller than the header
    assert lib.spear_take_error(None, 1 << 20, ctypes.byref(out), None) == 1
    assert lib.spear_take_error(buf, 1 << 20, None, None) == 1
    assert lib.spear_take_error(buf, 1024, ctypes.byref(out), None) == 5
    # spear_debug_stream_read: shapes and alignment, before any launch
    assert lib.spear_debug_stream_read(None, 64, 1, buf, None) == 1
    assert lib.spear_debug_stream_read(buf, 0, 1, buf, None) == 2
    assert lib.spear_debug_stream_read(buf, 24, 1, buf, None) == 2
    assert lib.spear_debug_stream_read(buf, 64, 0, buf, None) == 2
    # spear_debug_mfma_rate: arguments, before any device query or launch
    fl = ctypes.c_double(0.0)
    assert lib.spear_debug_mfma_rate(0, 1, 10, None, None, ctypes.byref(fl)) == 1
    assert lib.spear_debug_mfma_rate(0, 1, 10, buf, None, None) == 1
    assert lib.spear_debug_mfma_rate(2, 1, 10, buf, None, ctypes.byref(fl)) == 8
    assert lib.spear_debug_mfma_rate(0, 3, 10, buf, None, ctypes.byref(fl)) == 8
    assert lib.spear_debug_mfma_rate(1, 4, 0, buf, None, ctypes.byref(fl)) == 8
    # the debug knobs take any value and return nothing
    lib.spear_debug_set_spin_limit(0)
    lib.spear_debug_set_spin_limit(-1)
    lib.spear_debug_fail_waits(0)


def test_packed_bytes(lib):
    out = ctypes.c_size_t(0)
    assert lib.spear_packed_bytes(4096, 4096, ctypes.byref(out)) == 0 and out.value == 4096 * 4096 // 2
    assert lib.spear_packed_bytes(136, 20, ctypes.byref(out)) == 0 and out.value == 256 * 32 // 2
    assert lib.spear_packed_bytes(12, 20, ctypes.byref(out)) == 2
    assert lib.spear_packed_bytes(0, 20, ctypes.byref(out)) == 2
    assert lib.spear_packed_bytes(8, 0, ctypes.byref(out)) == 2
    assert lib.spear_packed_bytes(8, 8, None) == 1


def plan(lib, M, K, N, r, variant=0, cus=256, bias=0.0, tau=0.0):
    d = _binding.LinearDesc(M, K, N, r, bias, tau, variant, cus)
    p = _binding.Plan()
    st = lib.spear_dispatch_plan(ctypes.byref(d), ctypes.byref(p))
    return st, p


def test_dispatch_rules(lib):
    st, p = plan(lib, 16, 4096, 4096, 32)
    assert st == 0 and p.variant == 1 and p.kernel == 0
    # 128 x 448 tiles: auto takes split (the eight-wave tile kernel); forced
    # fused, about 128 EC workgroups (32 row tiles x 4 K slices) lead the
    # grid, then the 16 x 32 tiles
    st, p = plan(lib, 2048, 4096, 14336, 64)
    assert st == 0 and p.variant == 2 and p.kernel == 1 and p.workspace_bytes > 0
    assert p.grid == 16 * 32 and p.tile_m == 128 and p.tile_n == 448
    st, p = plan(lib, 2048, 4096, 14336, 64, variant=1)
    assert st == 0 and p.variant == 1 and p.kernel == 1 and p.workspace_bytes > 0
    assert p.producers == 32 * 4 and p.grid == 128 + 16 * 32 and p.tile_m == 128 and p.tile_n == 448
    # N in whole 224-column tiles but not 448: 256 x 224; otherwise 256 x 256
    st, p = plan(lib, 3100, 264, 3360, 0)
    assert st == 0 and p.tile_m == 256 and p.tile_n == 224 and p.split_k == 1
    st, p = plan(lib, 4096, 512, 4000, 0)
    assert st == 0 and p.tile_m == 256 and p.tile_n == 256 and p.split_k == 1
    st, p = plan(lib, 2048, 4096, 14336, 64, variant=2)
    assert st == 0 and p.variant == 2 and p.kernel == 1 and p.grid == 8 * 64
    # EC workgroups are padded to a multiple of 8 (the GEMM tiles keep their
    # XCD order): 1 row tile x 14 K slices -> 16
    st, p = plan(lib, 64, 14336, 4096, 64)
    assert st == 0 and p.variant == 1 and p.producers == 14 and p.grid == 16 + 32 * p.split_k
    # 128 x 256 tiles at mid-size M: fused, also when its EC workgroups
    # overflow the CUs; the K split fills about one workgroup per CU
    st, p = plan(lib, 512, 4096, 14336, 64)
    assert st == 0 and p.variant == 1 and p.tile_m == 128 and p.tile_n == 256 and p.grid > 256
    st, p = plan(lib, 512, 14336, 4096, 64)
    assert st == 0 and p.variant == 1 and p.tile_m == 128 and p.tile_n == 256 and p.grid > 256
    st, p = plan(lib, 512, 14336, 4096, 64, variant=2)
    assert st == 0 and p.variant == 2 and p.tile_n == 256 and p.split_k == 4 and p.grid == 4 * 16 * 4
    st, p = plan(lib, 256, 2048, 8192, 32)
    assert st == 0 and p.variant == 1 and p.tile_m == 64
    st, p = plan(lib, 16, 4096, 4096, 32)
    # fused, A of 256 KiB: the EC producer workgroups, then the GEMM tiles
    # (128 tiles of two 16-column panels, two K ranges); P goes over through
    # the workspace
    assert p.variant == 1 and p.ec_local == 0 and p.producers == 8 and p.grid == 256 + 8
    # two 16-column panels and two K splits per workgroup (same count)
    assert p.split_k == 2 and p.tile_n == 32
    assert p.workspace_bytes > 0
    # fused, local EC: one K range and an A of at most 64 KiB (128 KiB with
    # rank <= 32 and M <= 4), so every GEMM workgroup computes the projection
    # itself; no producers, no workspace
    st, p = plan(lib, 4, 2048, 4096, 32)
    assert st == 0 and p.ec_local == 1 and p.producers == 0 and p.grid == 256 and p.workspace_bytes == 0
    st, p = plan(lib, 16, 1024, 4096, 32)
    assert st == 0 and p.ec_local == 1 and p.producers == 0
    st, p = plan(lib, 1, 512, 14336, 64)
    assert st == 0 and p.ec_local == 1 and p.split_k == 1
    # 128 KiB with 16 rows, or with rank 64: the hand-off
    st, p = plan(lib, 16, 2048, 4096, 32)
    assert st == 0 and p.ec_local == 0 and p.producers > 0
    st, p = plan(lib, 1, 1024, 14336, 64)
    assert st == 0 and p.ec_local == 0 and p.producers > 0
    st, p = plan(lib, 16, 4096, 14336, 64)
    assert st == 0 and p.ec_local == 0 and p.producers > 0       # A of 512 KiB: hand-off
    # fused with a K split: producer workgroups lead the grid
    st, p = plan(lib, 1, 14336, 4096, 64)
    assert st == 0 and p.variant == 1 and p.ec_local == 0 and p.split_k == 7 and p.producers == 56
    assert p.grid == 56 + 64 * 7 and p.workspace_bytes > 0
    st, p = plan(lib, 1, 8192, 4096, 64)
    assert st == 0 and p.ec_local == 0 and p.producers > 0      # A of 1 MiB: hand-off
    st, p = plan(lib, 16, 512, 512, 16)
    assert st == 0 and p.ec_local == 0 and p.split_k > 1 and p.producers > 0
    st, p = plan(lib, 4, 4096, 4096, 30)
    assert st == 0 and p.variant == 2     # fused needs rank % 4 == 0: auto takes split
    st, p = plan(lib, 4, 4096, 4096, 30, variant=1)
    assert st == 3
    st, p = plan(lib, 40000, 60000, 4096, 16)
    assert st == 3                        # X above 2^31 - 1 bytes for the tiled kernel
    st, p = plan(lib, 16, 4096, 4096, 0)
    assert st == 0 and p.variant == 3 and p.producers == 0
    st, p = plan(lib, 16, 4096, 4096, 32, variant=2)
    assert st == 0 and p.variant == 2
    st, p = plan(lib, 64, 4096, 4096, 30, variant=1)
    assert st == 3                        # fused (skinny or tiled) needs rank % 4 == 0
    st, p = plan(lib, 64, 4096, 4096, 30)
    assert st == 0 and p.variant == 2
    st, p = plan(lib, 2048, 4096, 14336, 32, variant=3)
    assert st == 0 and p.variant == 3 and p.split_k == 1 and p.workspace_bytes == 0
    # mid-size M: 64-row tiles with K split over workgroups (partials in the workspace)
    st, p = plan(lib, 64, 4096, 4096, 32, variant=3)
    assert st == 0 and p.variant == 3 and p.tile_m == 64 and p.split_k > 1 and p.workspace_bytes > 0
    st, p = plan(lib, 0, 512, 512, 16)
    assert st == 0
    assert p.abi_version == 3 and p.layout_id == 2 and p.cus == 256


def test_dispatch_is_deterministic(lib):
    a = plan(lib, 512, 14336, 4096, 64)[1].as_dict()
    b = plan(lib, 512, 14336, 4096, 64)[1].as_dict()
    assert a == b


@pytest.mark.parametrize("M,K,N,r,code", [
    (-1, 512, 512, 16, 2), (16, 12, 512, 16, 2), (16, 0, 512, 16, 2), (16, 512, 0, 16, 2),
    (16, 512, 512, -1, 2), (16, 512, 512, 257, 2),
])
def test_dispatch_rejects_bad_shapes(lib, M, K, N, r, code):
    assert plan(lib, M, K, N, r)[0] == code


def test_dispatch_limits_of_the_kernels(lib):
    """Shapes the kernels cannot run are UNSUPPORTED, never a plan of zero
    workgroups: the decode kernel takes K up to 64 splits of 32 chunks of 128,
    and a launch stays within 2^30 workgroups."""
    st, p = plan(lib, 16, 262144, 512, 0)
    assert st == 0 and p.kernel == 0 and p.grid >= 1
    assert plan(lib, 16, 262144 + 128, 512, 0)[0] == 3
    assert plan(lib, 1, 1 << 24, 16, 0)[0] == 3
    assert plan(lib, 1 << 24, 8, 1 << 24, 0)[0] == 3
    nb = ctypes.c_size_t(0)
    assert lib.spear_ec_init_workspace_bytes(2147483640, 2147483647, 32, ctypes.byref(nb)) == 3
    assert lib.spear_ec_init_workspace_bytes(8, 1, 1, ctypes.byref(nb)) == 3     # l = 0 < rank
    assert lib.spear_ec_init_workspace_bytes(4096, 4096, 32, ctypes.byref(nb)) == 0
    assert nb.value >= 4096 * 4096 * 4


def test_dispatch_rejects_bad_arguments(lib):
    assert plan(lib, 16, 512, 512, 16, variant=7)[0] == 8
    assert plan(lib, 16, 512, 512, 16, bias=float("nan"))[0] == 8
    assert plan(lib, 16, 512, 512, 16, tau=1.5)[0] == 8
    assert plan(lib, 16, 512, 512, 16, tau=float("inf"))[0] == 8
    assert lib.spear_dispatch_plan(None, None) == 1


def test_linear_checks_before_launch(lib):
    """Every one of these returns an error before anything is enqueued."""
    st, p = plan(lib, 16, 512, 512, 16)
    d = _binding.LinearDesc(16, 512, 512, 16, 0.0, 0.0, 0, 256)
    fake = ctypes.c_void_p(0x1000)          # never dereferenced: checks fail first
    odd = ctypes.c_void_p(0x1002)
    null = ctypes.c_void_p(0)
    ws = p.workspace_bytes
    call = lambda *a: lib.spear_w4ec_linear(ctypes.byref(d), ctypes.byref(p), *a)  # noqa: E731
    assert call(null, fake, fake, fake, fake, fake, fake, fake, ws, null) == 1
    assert call(fake, fake, fake, null, fake, fake, fake, fake, ws, null) == 1
    assert call(fake, fake, fake, fake, fake, fake, fake, fake, ws - 1, null) == 5
    assert call(odd, fake, fake, fake, fake, fake, fake, fake, ws, null) == 4
    assert call(fake, odd, fake, fake, fake, fake, fake, fake, ws, null) == 4
    assert call(fake, fake, fake, fake, fake, fake, fake, odd, ws, null) == 4
    # a plan for another shape is rejected
    st2, p2 = plan(lib, 32, 512, 512, 16)
    assert lib.spear_w4ec_linear(ctypes.byref(d), ctypes.byref(p2), fake, fake, fake, fake, fake, fake,
                                 fake, fake, ws, null) == 6
    bad = _binding.Plan.from_buffer_copy(p)
    bad.grid += 1
    assert lib.spear_w4ec_linear(ctypes.byref(d), ctypes.byref(bad), fake, fake, fake, fake, fake, fake,
                                 fake, fake, ws, null) == 6
    bad = _binding.Plan.from_buffer_copy(p)
    bad.abi_version = 7
    assert lib.spear_w4ec_linear(ctypes.byref(d), ctypes.byref(bad), fake, fake, fake, fake, fake, fake,
                                 fake, fake, ws, null) == 6
    # M = 0 is a no-op that succeeds without touching any pointer
    d0 = _binding.LinearDesc(0, 512, 512, 16, 0.0, 0.0, 0, 256)
    st0, p0 = plan(lib, 0, 512, 512, 16)
    assert lib.spear_w4ec_linear(ctypes.byref(d0), ctypes.byref(p0), null, null, null, null, null, null,
                                 null, null, 0, null) == 0


def test_pack_and_unpack_checks(lib):
    fake = ctypes.c_void_p(0x1000)
    null = ctypes.c_void_p(0)
    assert lib.spear_pack_w4(null, 512, 512, fake, fake, null) == 1
    assert lib.spear_pack_w4(fake, 500, 512, fake, fake, null) == 2
    assert lib.spear_pack_w4(fake, 512, 512, ctypes.c_void_p(0x1004), fake, null) == 4
    assert lib.spear_debug_unpack_w4(null, 512, 512, fake, null) == 1
    assert lib.spear_debug_unpack_w4(fake, 8, 0, fake, null) == 2


def test_ec_project_checks(lib):
    fake = ctypes.c_void_p(0x1000)
    null = ctypes.c_void_p(0)
    nb = ctypes.c_size_t(0)
    assert lib.spear_ec_workspace_bytes(16, 512, 16, ctypes.byref(nb)) == 0 and nb.value > 0
    assert lib.spear_ec_workspace_bytes(16, 512, 0, ctypes.byref(nb)) == 2
    assert lib.spear_ec_project(16, 512, 16, fake, fake, fake, 0.0, 0.0, fake, fake, fake, 0, null) == 5
    assert lib.spear_ec_project(16, 512, 16, null, fake, fake, 0.0, 0.0, fake, fake, fake, nb.value, null) == 1
    assert lib.spear_ec_project(16, 512, 16, fake, fake, fake, float("nan"), 0.0, fake, fake, fake,
                                nb.value, null) == 8


def test_group_scales_descriptor_and_pack_checks(lib):
    """Group-wise scales: only groups of 128 (others UNSUPPORTED); the plan
    carries the group size; the grouped pack checks its arguments before any
    launch (a group size other than 128, shapes, alignment)."""
    d = _binding.LinearDesc(16, 4096, 4096, 32, 0.0, 0.0, 0, 256, 128)
    p = _binding.Plan()
    assert lib.spear_dispatch_plan(ctypes.byref(d), ctypes.byref(p)) == 0
    assert p.group_size == 128 and p.variant == 1 and p.kernel == 0
    d = _binding.LinearDesc(2048, 4096, 14336, 64, 0.0, 0.0, 0, 256, 128)
    assert lib.spear_dispatch_plan(ctypes.byref(d), ctypes.byref(p)) == 0
    assert p.group_size == 128 and p.kernel == 1
    for bad in (64, 32, 1, -1, 256):
        d = _binding.LinearDesc(16, 4096, 4096, 32, 0.0, 0.0, 0, 256, bad)
        assert lib.spear_dispatch_plan(ctypes.byref(d), ctypes.byref(p)) == 3
    buf = ctypes.create_string_buffer(1024)
    assert lib.spear_pack_w4_grouped(None, 128, 16, 128, buf, buf, None) == 1
    assert lib.spear_pack_w4_grouped(buf, 12, 16, 128, buf, buf, None) == 2
    assert lib.spear_pack_w4_grouped(buf, 128, 16, 64, buf, buf, None) == 3
