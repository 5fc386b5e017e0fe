"""Host-side tests of the C-ABI library (no GPU, no compute calls).

- the shared library loads and exports every function include/exact_row_top.h
  declares;
- argument validation returns the documented status codes without touching a
  device;
- launch planning picks the tiers the design states for the five workloads.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "exact_row_top.h")

ert = pytest.importorskip("exact_row_top_amd")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(topk_\w+)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = _declared_functions()
    for required in ("topk_decode", "topk_prefill", "topk_workspace_bytes",
                     "topk_workspace_init", "topk_strerror"):
        assert required in names


def test_library_exports_every_declared_symbol():
    lib = ert.load_library()
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_strerror_covers_codes():
    for code in range(6):
        assert ert.strerror(code)
    assert "unknown" in ert.strerror(99)


P16 = 1 << 20  # a fake, 16-byte aligned "device" address (never dereferenced)


def _validate(mode=0, logits=P16, stride=4096, e1=P16, e2=P16, rows=4, k=512, idx=P16,
              ws=None, ws_bytes=0, max_len=0):
    return ert.load_library().topk_validate(mode, logits, stride, e1, e2, rows, k, idx, ws,
                                            ws_bytes, max_len)


def test_validate_ok():
    assert _validate() == 0
    assert _validate(mode=1) == 0
    assert _validate(rows=0, logits=None, e1=None, e2=None, idx=None) == 0  # empty is a no-op


@pytest.mark.parametrize("k", [0, 1, 256, 511, 513, 2047, 4096, -512])
def test_validate_rejects_k(k):
    assert _validate(k=k) == ert.TOPK_EINVAL


def test_validate_rejects_nulls_and_counts():
    assert _validate(rows=-1) == ert.TOPK_EINVAL
    assert _validate(logits=None) == ert.TOPK_EINVAL
    assert _validate(e1=None) == ert.TOPK_EINVAL
    assert _validate(idx=None) == ert.TOPK_EINVAL
    assert _validate(mode=1, e2=None) == ert.TOPK_EINVAL
    assert _validate(mode=0, e2=None) == 0  # decode has no second extent
    assert _validate(stride=0) == ert.TOPK_EINVAL
    assert _validate(mode=2) == ert.TOPK_EINVAL
    assert _validate(max_len=-1) == ert.TOPK_EINVAL


def test_validate_layout():
    assert _validate(logits=P16 + 4) == ert.TOPK_ELAYOUT  # float aligned, not float4 aligned
    assert _validate(logits=P16 + 8) == ert.TOPK_ELAYOUT
    assert _validate(stride=4098) == ert.TOPK_ELAYOUT
    assert _validate(stride=4099) == ert.TOPK_ELAYOUT
    assert _validate(idx=P16 + 2) == ert.TOPK_ELAYOUT
    assert _validate(e1=P16 + 1) == ert.TOPK_ELAYOUT
    assert _validate(mode=1, e2=P16 + 3) == ert.TOPK_ELAYOUT


def test_validate_workspace_size():
    need = ert.workspace_bytes(64, 131072, 2048)
    assert need > 0
    assert _validate(stride=131072, rows=64, k=2048, ws=P16, ws_bytes=need) == 0
    assert _validate(stride=131072, rows=64, k=2048, ws=P16, ws_bytes=need - 1) == ert.TOPK_EWORKSPACE
    # the split tier moves its counts as 16-byte words
    assert _validate(stride=131072, rows=64, k=2048, ws=P16 + 8, ws_bytes=need) == ert.TOPK_ELAYOUT
    # a plan without the split tier takes no workspace, aligned or not
    assert _validate(stride=4096, rows=4096, k=512, ws=P16 + 8, ws_bytes=need) == 0


def test_workspace_layout():
    lay = ert.workspace_layout()
    assert lay["header_bytes"] == 256 and lay["slots"] == 256
    assert lay["slot_fixed_bytes"] % 256 == 0
    assert lay["data_offset"] == lay["header_bytes"] + lay["slots"] * lay["slot_fixed_bytes"]
    assert lay["slice_bytes"] == 2 * 2048       # one 16-bit suffix count per bin
    assert lay["list_bytes"] >= 8 * 2048        # the crossing bin's members, (key, index)
    p = ert.plan_query(64, 131072, 2048)
    per_slot = p["wgs_per_row"] * lay["slice_bytes"] + lay["list_bytes"]
    assert ert.workspace_bytes(64, 131072, 2048) >= lay["data_offset"] + 64 * per_slot


def test_workspace_bytes():
    assert ert.workspace_bytes(4096, 16640, 1024) == 0      # one workgroup per row
    assert ert.workspace_bytes(0, 4096, 512) == 0
    assert ert.workspace_bytes(4, 4096, 513) == 0             # invalid k
    a = ert.workspace_bytes(8, 262144, 2048)
    b = ert.workspace_bytes(64, 131072, 2048)
    assert 0 < a < b


def test_plans_for_the_workloads():
    # many short-to-mid rows: one workgroup per row, whole window resident
    p = ert.plan_query(4096, 16640, 1024)
    assert p["wgs_per_row"] == 1 and p["quads_per_thread"] * p["block"] * 4 >= 16640 + 6
    # few long rows: split, the row's parts cover the whole stride
    for rows, stride, k in ((64, 131072, 2048), (1, 131072, 512), (8, 131072, 512),
                            (8, 262144, 2048)):
        p = ert.plan_query(rows, stride, k)
        assert p["wgs_per_row"] > 1 and p["block"] in (256, 512)
        assert p["wgs_per_row"] * p["quads_per_thread"] * p["block"] >= (stride + 6) // 4
        assert p["cap"] == 2048
    # few rows of 262144: parts of about 2048 float4 groups in the 512-thread
    # shape, no more than the compute units of the row's XCD (32)
    for rows, k in ((1, 2048), (7, 512), (2, 1024)):
        p = ert.plan_query(rows, 262144, k)
        assert p["wgs_per_row"] == 32 and p["block"] == 512
        assert 32 * p["quads_per_thread"] * p["block"] >= (262144 + 6) // 4
    # the longest row a plan holds needs all 64 parts of the largest shape
    p = ert.plan_query(1, 64 * 9 * 512 * 4 - 16, 512)
    assert p["wgs_per_row"] == 64 and p["block"] == 512 and p["quads_per_thread"] == 9
    # rows that already fill the chip keep the fewest parts the shape allows
    assert ert.plan_query(64, 131072, 2048)["wgs_per_row"] == 8
    # capacity bounds rows per launch (co-resident split workgroups)
    p = ert.plan_query(64, 131072, 2048, cu_count=16, wgs_per_cu=2)
    assert p["rows_per_launch"] * p["wgs_per_row"] <= 32 and p["launches"] > 1


def test_plan_forced_tiers():
    p = ert.plan_query(8, 16384, 512, force_wgs_per_row=1)
    assert p["wgs_per_row"] == 1
    p = ert.plan_query(8, 16384, 512, force_wgs_per_row=4)
    assert p["wgs_per_row"] == 4
    with pytest.raises(ert.TopKError):
        ert.plan_query(8, 131072, 512, force_wgs_per_row=1)   # row does not fit one workgroup
    with pytest.raises(ert.TopKError):
        ert.plan_query(8, 4096, 512, force_wgs_per_row=65)
    with pytest.raises(ert.TopKError):
        ert.plan_query(1, 64 * 9 * 512 * 4 + 64, 512)         # longer than the largest plan


def test_output_options_and_varlen_validation():
    lib = ert.load_library()
    # bad next_n / compression ratio, unknown flag bits, misaligned values: all
    # rejected on the host before any device work
    assert lib.topk_decode_varlen(P16, 4096, P16, 4, 0, 1, 512, P16, None, 0, None, 0,
                                  None) == ert.TOPK_EINVAL
    assert lib.topk_decode_varlen(P16, 4096, P16, 4, 2, 0, 512, P16, None, 0, None, 0,
                                  None) == ert.TOPK_EINVAL
    assert lib.topk_decode_varlen(P16, 4096, P16, 4, 2, 4, 513, P16, None, 0, None, 0,
                                  None) == ert.TOPK_EINVAL
    assert lib.topk_decode_v(P16, 4096, P16, 4, 512, P16, None, 4, None, 0, None) == ert.TOPK_EINVAL
    assert lib.topk_decode_v(P16, 4096, P16, 4, 512, P16, P16 + 2, 0, None, 0,
                             None) == ert.TOPK_ELAYOUT
    assert lib.topk_prefill_v(P16, 4096, P16, P16, 4, 512, P16, None, 8, 0, None, 0,
                              None) == ert.TOPK_EINVAL
    # hints: a stride below k, a misaligned hint array, hints on the prefill
    # form -- all rejected on the host
    assert lib.topk_decode_hinted(P16, 4096, P16, P16, 511, 4, 512, P16, None, 0, None, 0,
                                  None) == ert.TOPK_EINVAL
    assert lib.topk_decode_hinted(P16, 4096, P16, P16 + 2, 512, 4, 512, P16, None, 0, None, 0,
                                  None) == ert.TOPK_ELAYOUT
    assert lib.topk_decode_varlen_hinted(P16, 4096, P16, P16, 100, 4, 2, 4, 1024, P16, None, 0,
                                         None, 0, None) == ert.TOPK_EINVAL
    o = ert._Options(0, 0, None, None, 0, P16, 512)
    assert lib.topk_prefill_ex(P16, 4096, P16, P16, 4, 512, P16, 0, None, 0, None,
                               ctypes.pointer(o)) == ert.TOPK_EINVAL
    # block-skip: bmax stride below ceil(row_stride / 32), a forced pass
    # without maxima, maxima on the prefill form, a misaligned bmax
    assert lib.topk_decode_blockskip(P16, 4096, P16, P16, 127, 4, 512, P16, None, 0, None, 0,
                                     None) == ert.TOPK_EINVAL
    assert lib.topk_decode_blockskip(P16, 4096, P16, None, 128, 4, 512, P16, None, 0, None, 0,
                                     None) == ert.TOPK_EINVAL
    assert lib.topk_decode_blockskip(P16, 4096, P16, P16 + 2, 128, 4, 512, P16, None, 0, None, 0,
                                     None) == ert.TOPK_ELAYOUT
    o = ert._Options(0, 0, None, None, 0, None, 0, P16, 128, 0)
    assert lib.topk_prefill_ex(P16, 4096, P16, P16, 4, 512, P16, 0, None, 0, None,
                               ctypes.pointer(o)) == ert.TOPK_EINVAL
    o = ert._Options(0, 0, None, None, 0, None, 0, None, 0, 1)
    assert lib.topk_decode_ex(P16, 4096, P16, 4, 512, P16, None, 0, None,
                              ctypes.pointer(o)) == ert.TOPK_EINVAL
    o = ert._Options(0, 0, None, None, 0, None, 0, P16, 128, 3)
    assert lib.topk_decode_ex(P16, 4096, P16, 4, 512, P16, None, 0, None,
                              ctypes.pointer(o)) == ert.TOPK_EINVAL
    # the streaming pass (blockskip=2): decode forms only, rows of at most
    # 8192 blocks of 32
    o = ert._Options(0, 0, None, None, 0, None, 0, None, 0, 2)
    assert lib.topk_prefill_ex(P16, 4096, P16, P16, 4, 512, P16, 0, None, 0, None,
                               ctypes.pointer(o)) == ert.TOPK_EINVAL
    assert lib.topk_decode_ex(P16, 8192 * 32 + 4, P16, 4, 512, P16, None, 0, None,
                              ctypes.pointer(o)) == ert.TOPK_EINVAL
    assert lib.topk_block_max(P16, 4096, 4, P16, 127, None) == ert.TOPK_EINVAL
    assert lib.topk_block_max(P16, 0, 4, P16, 128, None) == ert.TOPK_EINVAL
    assert lib.topk_block_max(None, 4096, 0, None, 0, None) == 0
    # empty batches are a no-op for every form
    assert lib.topk_decode_varlen(None, 4096, None, 0, 2, 4, 512, None, None, 0, None, 0,
                                  None) == 0
    assert lib.topk_decode_varlen_hinted(None, 4096, None, None, 0, 0, 2, 4, 512, None, None, 0,
                                         None, 0, None) == 0
    assert _validate(stride=1 << 30) == ert.TOPK_EINVAL


def test_status_rejects_bad_output_without_a_device():
    lib = ert.load_library()
    assert lib.topk_status(None, None) == ert.TOPK_EINVAL
    assert lib.topk_status(P16 + 2, None) == ert.TOPK_ELAYOUT


def test_options_reject_negative_barrier_spins():
    # validated on the host before any device query
    o = ert._Options(0, 0, None, None, 0, None, 0, None, 0, 0, -1)
    lib = ert.load_library()
    rc = lib.topk_decode_ex(P16, 4096, P16, 4, 512, P16, None, 0, None, ctypes.pointer(o))
    assert rc == ert.TOPK_EINVAL


def test_read_floor_validates_on_the_host():
    lib = ert.load_library()
    assert lib.topk_read_floor(2, P16, 4096, P16, P16, 4, 512, P16, None) == ert.TOPK_EINVAL
    assert lib.topk_read_floor(0, P16, 4096, P16, None, 4, 100, P16, None) == ert.TOPK_EINVAL
    assert lib.topk_read_floor(0, P16 + 4, 4096, P16, None, 4, 512, P16, None) == ert.TOPK_ELAYOUT
    assert lib.topk_read_floor(1, P16, 4096, P16, P16, 0, 512, None, None) == 0  # empty
