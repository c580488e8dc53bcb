"""Host-side tests (no GPU): the C-ABI library loads and exports every symbol
the public header declares, and the launch planner's residency and fallback
rules hold for made-up device properties.

The fake-device planner tests stand in for the low-shared-memory fallback
test that the PR #54110 page says was added and then dropped: instead of
mocking a device they call the pure planning function with chosen CU counts
and occupancies.
"""

from __future__ import annotations

import ctypes
import os
import re

import pytest

import row_radix_top_amd as rrt
from row_radix_top_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "topk_ragged.h")


def header_functions() -> list[str]:
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(topk_ragged\w*)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = binding.load()
    names = header_functions()
    assert len(names) >= 10, names
    assert set(names) == set(binding.EXPORTED), "binding and header disagree"
    for n in names:
        assert hasattr(lib, n), n
    assert binding.version() >= 100


def test_library_carries_gfx950_code():
    blob = open(binding.LIB_PATH, "rb").read()
    assert b"gfx950" in blob


def test_plan_single_path_for_short_rows():
    p = rrt.plan_for_props(256, 3, 3, 64, 32768, 2048)
    assert p["path"] == rrt.PATH_SINGLE and p["workspace_bytes"] == 0
    assert p["grid"] == 64 and p["headroom"] == 0 and p["kmax"] == 2048
    # At the threshold exactly: still one workgroup per row (strict ">").
    p = rrt.plan_for_props(256, 3, 3, 2, 32768, 1024)
    assert p["path"] == rrt.PATH_SINGLE
    # Rows up to 65536 elements stay on one workgroup each, whatever their count.
    for stride in (32769, 40000, 65536):
        p = rrt.plan_for_props(256, 3, 3, 2, stride, 1024)
        assert p["path"] == rrt.PATH_SINGLE, (stride, p)
    p = rrt.plan_for_props(256, 3, 3, 2, 65537, 1024)
    assert p["path"] == rrt.PATH_MULTI and p["wg_per_row"] >= 4
    # Fewer than four workgroups per row are not worth it: one workgroup per row.
    p = rrt.plan_for_props(256, 3, 3, 200, 131072, 1024)
    assert p["path"] == rrt.PATH_SINGLE and p["fell_back"] == 0
    # Unless the caller asks for it.
    p = rrt.plan_for_props(256, 3, 3, 2, 40000, 1024, force_path=2)
    assert p["path"] == rrt.PATH_MULTI and p["wg_per_row"] >= 2


def test_plan_many_long_rows_use_persistent_single_path():
    p = rrt.plan_for_props(256, 3, 3, 4096, 65536, 2048)
    assert p["path"] == rrt.PATH_SINGLE
    assert p["grid"] == 768 == p["resident_cap"]
    p = rrt.plan_for_props(256, 3, 3, 4096, 65536, 2048, max_grid=100)
    assert p["grid"] == 100
    assert p["workspace_bytes"] == 256
    p = rrt.plan_for_props(256, 3, 3, 768, 65536, 2048)
    assert p["grid"] == 768 and p["workspace_bytes"] == 0


@pytest.mark.parametrize("cus,occ", [(256, 1), (256, 2), (256, 3), (256, 4), (80, 2), (4, 1), (1, 1)])
@pytest.mark.parametrize("rows,stride", [(16, 131072), (64, 65536), (1, 1 << 20), (3, 40000), (300, 65536)])
def test_plan_multi_is_always_coresident(cus, occ, rows, stride):
    p = rrt.plan_for_props(cus, occ, occ, rows, stride, 2048)
    cap = cus * occ
    if p["path"] == rrt.PATH_MULTI:
        headroom = cus if occ > 1 else 1
        assert p["headroom"] == headroom
        assert p["grid"] == rows * p["wg_per_row"]
        assert p["grid"] <= cap - headroom, p
        assert stride > 65536 and p["wg_per_row"] >= 4
        assert p["chunk"] % 2048 == 0
        assert (p["wg_per_row"] - 1) * p["chunk"] < stride <= p["wg_per_row"] * p["chunk"]
        assert p["workspace_bytes"] > 0
    else:
        assert p["path"] == rrt.PATH_SINGLE
        # A ticket counter in the workspace header hands out rows past the grid.
        assert p["workspace_bytes"] == (256 if rows > p["grid"] else 0)
        assert p["grid"] <= cap


def test_plan_forced_multi_that_cannot_be_resident_falls_back():
    # 64 rows x 16 workgroups cannot be resident on 8 CUs with occupancy 1.
    p = rrt.plan_for_props(8, 1, 1, 64, 65536, 2048, force_path=2, force_wg_per_row=16)
    assert p["path"] == rrt.PATH_SINGLE and p["fell_back"] == 1 and p["grid"] == 8
    assert p["workspace_bytes"] == 256  # 64 rows on 8 workgroups: ticket counter
    p = rrt.plan_for_props(256, 2, 2, 4, 65536, 2048, force_path=2, force_wg_per_row=4)
    assert p["path"] == rrt.PATH_MULTI and p["wg_per_row"] == 4


def test_plan_headroom_only_when_there_is_room():
    # One CU, occupancy 1: no room for headroom plus a group -> no headroom,
    # and a group of 2 cannot be resident -> single path.
    p = rrt.plan_for_props(1, 1, 1, 1, 131072, 2048)
    assert p["path"] == rrt.PATH_SINGLE
    # Four slots less one of headroom leave a group of 3: below the minimum group.
    p = rrt.plan_for_props(4, 1, 1, 1, 131072, 2048)
    assert p["path"] == rrt.PATH_SINGLE
    p = rrt.plan_for_props(8, 1, 1, 1, 131072, 2048)
    assert p["path"] == rrt.PATH_MULTI and p["headroom"] == 1 and 4 <= p["grid"] <= 7


def test_plan_single_when_multi_kernel_cannot_run():
    p = rrt.plan_for_props(256, 2, 0, 4, 131072, 2048)
    assert p["path"] == rrt.PATH_SINGLE


def test_plan_index_width_and_vec():
    for K in (1, 256, 1000, 2048):
        assert rrt.plan_for_props(256, 2, 2, 4, 8192, K)["kmax"] == 2048
    # 16-bit candidate indices when every row index fits them, on both paths:
    # the workgroup that merges a row's chunks holds row indices.
    assert rrt.plan_for_props(256, 3, 3, 4096, 65536, 2048)["idx16"] == 1
    assert rrt.plan_for_props(256, 3, 3, 4096, 65537, 2048)["idx16"] == 0
    p = rrt.plan_for_props(256, 3, 3, 16, 131072, 2048)
    assert p["path"] == rrt.PATH_MULTI and p["chunk"] <= 65536 and p["idx16"] == 0
    p = rrt.plan_for_props(256, 3, 3, 16, 65536, 2048, force_path=2)
    assert p["path"] == rrt.PATH_MULTI and p["idx16"] == 1
    p = rrt.plan_for_props(256, 3, 3, 2, 1 << 20, 2048, force_path=2, force_wg_per_row=8)
    assert p["chunk"] > 65536 and p["idx16"] == 0
    assert rrt.plan_for_props(256, 3, 3, 4, 131072, 2048, force_path=1)["idx16"] == 0
    assert rrt.plan_for_props(256, 2, 2, 4, 8192, 64, vec_allowed=2)["vec"] == 2
    assert rrt.plan_for_props(256, 2, 2, 4, 8192, 64, vec_allowed=4, force_vec=1)["vec"] == 1
    with pytest.raises(rrt.TopKError):
        rrt.plan_for_props(256, 2, 2, 4, 8192, 64, vec_allowed=2, force_vec=4)


def test_plan_rejects_bad_arguments():
    with pytest.raises(rrt.TopKError) as e:
        rrt.plan_for_props(256, 2, 2, 4, 8192, 0)
    assert e.value.code == -2
    with pytest.raises(rrt.TopKError) as e:
        rrt.plan_for_props(256, 2, 2, 4, 8192, 4097)
    assert e.value.code == -2 and "4097" in str(e.value)
    with pytest.raises(rrt.TopKError) as e:
        rrt.plan_for_props(256, 2, 2, -1, 8192, 10)
    assert e.value.code == -1
    with pytest.raises(rrt.TopKError):
        rrt.plan_for_props(256, 2, 2, 4, 0, 10)
    with pytest.raises(rrt.TopKError):
        rrt.plan_for_props(256, 2, 2, 4, 100000, 10, force_path=2, force_chunk=6)
    p = rrt.plan_for_props(256, 2, 2, 0, 8192, 10)
    assert p["path"] == rrt.PATH_NONE


def test_launch_argument_errors_need_no_gpu():
    # Argument checks happen before any HIP call.
    lib = binding.load()
    out = ctypes.c_void_p(256)
    assert lib.topk_ragged(None, 10, None, -1, 1, 4, None, None, None) == -1
    assert lib.topk_ragged(None, 10, None, 4, 3, 4, None, None, None) == -1  # 4 % 3 != 0
    assert lib.topk_ragged(None, 10, None, 4, 0, 4, None, None, None) == -1
    assert lib.topk_ragged(None, 10, None, 0, 1, 4, None, None, None) == 0   # no-op
    assert lib.topk_ragged(ctypes.c_void_p(256), 10, ctypes.c_void_p(256), 4, 1, 0, out, None, None) == -2
    assert "K=0" in binding.last_error()
    assert lib.topk_ragged(None, 10, ctypes.c_void_p(256), 4, 1, 4, out, None, None) == -1
    assert lib.topk_ragged(ctypes.c_void_p(256), 10, ctypes.c_void_p(256), 4, 1, 4, ctypes.c_void_p(258),
                           None, None) == -1


def test_plan_forced_group_sizes_are_kept():
    for G in (1, 2, 3, 5, 7, 16, 31, 32):
        p = rrt.plan_for_props(256, 3, 3, 16, 131072, 2048, force_path=2, force_wg_per_row=G)
        assert p["path"] == rrt.PATH_MULTI and p["wg_per_row"] == G, (G, p)
        assert p["chunk"] % 4 == 0
    # 16 x 64 = 1024 workgroups exceed 768 slots less 256 of headroom.
    p = rrt.plan_for_props(256, 3, 3, 16, 131072, 2048, force_path=2, force_wg_per_row=64)
    assert p["path"] == rrt.PATH_SINGLE and p["fell_back"] == 1


def test_plan_ticket_workspace():
    # One workgroup per row: no workspace while every row has its own
    # workgroup, a 256-byte header (the row ticket) once rows outnumber the grid.
    p = rrt.plan_for_props(256, 4, 4, 1024, 32768, 2048)
    assert p["path"] == rrt.PATH_SINGLE and p["grid"] == 1024 and p["workspace_bytes"] == 0
    p = rrt.plan_for_props(256, 4, 4, 1025, 32768, 2048)
    assert p["grid"] == 1024 and p["workspace_bytes"] == 256
    p = rrt.plan_for_props(256, 4, 4, 64, 32768, 2048, max_grid=7)
    assert p["grid"] == 7 and p["workspace_bytes"] == 256
    # The row-splitting overrides of earlier versions are gone.
    for bad in ("split_rows", "split_g", "split_chunk"):
        with pytest.raises(TypeError):
            rrt.plan_for_props(256, 4, 4, 8, 65536, 2048, **{bad: 4})


def test_plan_occupancy_cap():
    # A device that keeps one workgroup per CU: one slot of headroom, and
    # every row group must fit the remaining 255 slots.
    p = rrt.plan_for_props(256, 3, 3, 16, 131072, 2048, max_occupancy=1)
    assert p["path"] == rrt.PATH_MULTI and p["resident_cap"] == 256 and p["headroom"] == 1
    assert p["grid"] <= 255 and p["wg_per_row"] >= 4
    assert p["grid"] == 16 * p["wg_per_row"]
    # The one-workgroup path's persistent grid shrinks with it.
    p = rrt.plan_for_props(256, 4, 4, 4096, 65536, 2048, max_occupancy=1)
    assert p["path"] == rrt.PATH_SINGLE and p["grid"] == 256 and p["resident_cap"] == 256
    # A forced group that no longer fits falls back to one workgroup per row.
    p = rrt.plan_for_props(256, 3, 3, 16, 131072, 2048, max_occupancy=1, force_path=2, force_wg_per_row=16)
    assert p["path"] == rrt.PATH_SINGLE and p["fell_back"] == 1
    # Too many rows for four workgroups each: one per row.
    p = rrt.plan_for_props(256, 3, 3, 100, 131072, 2048, max_occupancy=1)
    assert p["path"] == rrt.PATH_SINGLE and p["fell_back"] == 0
    # Occupancy 2: a CU's worth of headroom.
    p = rrt.plan_for_props(256, 3, 3, 16, 131072, 2048, max_occupancy=2)
    assert p["path"] == rrt.PATH_MULTI and p["resident_cap"] == 512 and p["headroom"] == 256
    assert p["grid"] <= 256
    # A cap above the device's changes nothing.
    assert rrt.plan_for_props(256, 3, 3, 16, 131072, 2048, max_occupancy=8) == \
        rrt.plan_for_props(256, 3, 3, 16, 131072, 2048)
    with pytest.raises(rrt.TopKError):
        rrt.plan_for_props(256, 3, 3, 16, 131072, 2048, max_occupancy=-1)


def test_plan_large_k_layout():
    # K above 2048 takes the large layout: kmax 4096, more LDS per workgroup.
    small = rrt.plan_for_props(256, 4, 4, 64, 32768, 2048)
    big = rrt.plan_for_props(256, 2, 2, 64, 32768, 2049)
    assert small["kmax"] == 2048 and big["kmax"] == 4096
    assert big["lds_bytes"] > small["lds_bytes"]
    assert rrt.plan_for_props(256, 2, 2, 64, 32768, 4096)["kmax"] == 4096
    # Forcing 32-bit indices changes the index width only.
    p = rrt.plan_for_props(256, 2, 2, 64, 32768, 3000, force_idx32=1)
    assert p["idx16"] == 0 and p["kmax"] == 4096
    assert rrt.plan_for_props(256, 2, 2, 64, 32768, 3000)["idx16"] == 1
    # Cooperative lists size with the layout's capacity.
    ws = [rrt.plan_for_props(256, 2, 2, 8, 131072, k, force_path=2, force_wg_per_row=4)["workspace_bytes"]
          for k in (2048, 4096)]
    assert ws[1] - ws[0] == 8 * 4 * 4 * (7168 - 5120)


# ---------------------------------------------------------------------------
# Workgroup width
# ---------------------------------------------------------------------------

WIDE = dict(occupancy_w512=(2, 2, 2, 2), occupancy_w1024=(1, 1, 1, 1))


def test_plan_block_width_auto():
    # Few long rows that speculate with the 512-thread sample: 512 threads.
    p = rrt.plan_for_props(256, 3, 3, 64, 32768, 2048, occupancy_single16=4, **WIDE)
    assert p["path"] == rrt.PATH_SINGLE and p["block"] == 512 and p["grid"] == 64
    p = rrt.plan_for_props(256, 3, 3, 64, 65536, 2048, occupancy_single16=4, **WIDE)
    assert p["block"] == 512 and p["lds_bytes"] > 0
    # 4 x 8192 at K = 512: the 512-thread sample (8192) would be the whole
    # row, no speculation there, so 256 threads.
    p = rrt.plan_for_props(256, 3, 3, 4, 8192, 512, occupancy_single16=4, **WIDE)
    assert p["block"] == 256
    # A batch that fills the GPU stays on 256 threads.
    p = rrt.plan_for_props(256, 3, 3, 4096, 65536, 2048, occupancy_single16=4, **WIDE)
    assert p["block"] == 256 and p["grid"] == 1024
    # More rows than 512-thread slots: 256.
    p = rrt.plan_for_props(256, 3, 3, 600, 32768, 2048, occupancy_single16=4, **WIDE)
    assert p["block"] == 256
    # No wide instance on the device (zeros): 256.
    p = rrt.plan_for_props(256, 3, 3, 64, 32768, 2048, occupancy_single16=4)
    assert p["block"] == 256


def test_plan_block_width_forced():
    for b in (256, 512, 1024):
        p = rrt.plan_for_props(256, 3, 3, 64, 32768, 2048, force_block=b, **WIDE)
        assert p["block"] == b and p["path"] == rrt.PATH_SINGLE
        p = rrt.plan_for_props(256, 3, 3, 16, 131072, 2048, force_block=b, force_path=2, **WIDE)
        assert p["block"] == b and p["path"] == rrt.PATH_MULTI
        # Chunks of the multi path are whole tiles of this width.
        assert p["chunk"] % (b * 8) == 0
    with pytest.raises(rrt.TopKError):
        rrt.plan_for_props(256, 3, 3, 64, 32768, 2048, force_block=384, **WIDE)
    # A forced width the device cannot keep resident is an error, not a silent change.
    with pytest.raises(rrt.TopKError):
        rrt.plan_for_props(256, 3, 3, 64, 32768, 2048, force_block=1024)


def test_ctypes_mirrors_match_the_header():
    # The binding's ctypes structs must list the header's fields in order,
    # with the same widths: a mismatch would make the library read or write
    # past the caller's struct.
    import ctypes
    import os
    import re
    from row_radix_top_amd import binding
    hdr = open(os.path.join(os.path.dirname(__file__), "..", "include", "topk_ragged.h")).read()
    hdr = re.sub(r"/\*.*?\*/", "", hdr, flags=re.S)
    widths = {"int32_t": 4, "uint32_t": 4, "int64_t": 8, "uint64_t": 8}
    for cname, cls in (("topk_plan", binding.Plan), ("topk_overrides", binding.Overrides),
                       ("topk_device_props", binding.DeviceProps)):
        body = re.search(r"typedef struct \{([^{}]*)\}\s*" + cname + ";", hdr).group(1)
        fields = []
        for decl in body.split(";"):
            decl = decl.strip()
            if not decl:
                continue
            m = re.fullmatch(r"(\w+)\s+(\w+)(?:\[(\d+)\])?", decl)
            assert m, (cname, decl)
            fields.append((m.group(2), widths[m.group(1)] * int(m.group(3) or 1)))
        mirror = [(name, ctypes.sizeof(t)) for name, t in cls._fields_]
        assert mirror == fields, (cname, mirror, fields)


def test_counter_hash_ignores_comments_only():
    """The key of a stored counter reading follows the sources' code: a
    comment or whitespace edit keeps it, any code edit changes it, and
    comment markers inside string literals are code."""
    import bench
    a = 'int x = 1; // one\n/* two\n   lines */ const char* s = "a // b /* c */";\n'
    b = 'int x = 1;   /* other words */\nconst char* s = "a // b /* c */"; // trailing\n'
    c = 'int x = 2; const char* s = "a // b /* c */";'
    assert bench.code_of(a) == bench.code_of(b) == 'int x = 1; const char* s = "a // b /* c */";'
    assert bench.code_of(c) != bench.code_of(a)
    assert bench.code_of("char q = '\\''; // x") == "char q = '\\'';"
    assert len(bench.kernel_source_hash()) == 64


def test_wide_plans_load_one_element_per_lane():
    """fp32 rows on 512- (or 1024-) thread workgroups load one element per
    lane unless a width is forced; 256-thread plans keep the widest load the
    alignment allows, and bf16 plans keep theirs."""
    w512 = (2, 2, 2, 2)
    # 64 rows fitting the CUs at the 512-thread occupancy, long enough to go wave by wave.
    p = rrt.plan_for_props(256, 4, 4, 64, 32768, 2048, occupancy_w512=w512)
    assert p["block"] == 512 and p["vec"] == 1
    p = rrt.plan_for_props(256, 4, 4, 64, 32768, 2048, occupancy_w512=w512, force_vec=4)
    assert p["block"] == 512 and p["vec"] == 4
    p = rrt.plan_for_props(256, 4, 4, 64, 32768, 2048, vec_allowed=2, occupancy_w512=w512, force_vec=2)
    assert p["vec"] == 2
    # Cooperative long rows on 512 threads.
    p = rrt.plan_for_props(256, 3, 3, 16, 131072, 2048, occupancy_w512=w512)
    assert p["path"] == rrt.PATH_MULTI and p["block"] == 512 and p["vec"] == 1
    # A batch that fills the GPU stays on 256 threads and wide loads.
    p = rrt.plan_for_props(256, 4, 4, 4096, 65536, 2048, occupancy_w512=w512)
    assert p["block"] == 256 and p["vec"] == 4
    # bf16 (8-element loads allowed) keeps its width on wide workgroups.
    p = rrt.plan_for_props(256, 4, 4, 64, 32768, 2048, vec_allowed=8, occupancy_w512=w512)
    assert p["block"] == 512 and p["vec"] == 8
