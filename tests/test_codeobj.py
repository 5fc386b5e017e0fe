"""The built library's gfx950 code objects, read on the host (no GPU).

Every kernel must keep its state in registers and LDS: a private (scratch)
segment means the compiler moved something -- typically a row's resident
scores indexed at a computed position -- to per-lane memory, where every
access is a memory round trip behind the row's own load waits.  Vector
register spills are checked the same way (scalar registers that spill go to
lanes of a vector register, not to memory, and are allowed), and the
17-group one-workgroup kernels must fit the 96-VGPR budget of five waves per
SIMD that their launch shape assumes.
The code objects are read from the library's clang offload bundles with
llvm-readelf's metadata notes.
"""
import os
import re
import shutil
import struct
import subprocess
import tempfile

import pytest

from exact_row_top_amd import LIB_PATH

READELF = next((p for p in ("/opt/rocm/llvm/bin/llvm-readelf", shutil.which("llvm-readelf"))
                if p and os.path.exists(p)), None)
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"


def _code_objects(path):
    data = open(path, "rb").read()
    for m in re.finditer(re.escape(MAGIC), data):
        s = m.start()
        (n,) = struct.unpack_from("<Q", data, s + len(MAGIC))
        p = s + len(MAGIC) + 8
        for _ in range(n):
            off, size, idl = struct.unpack_from("<QQQ", data, p)
            p += 24
            tid = data[p:p + idl].decode()
            p += idl
            if "gfx950" in tid and size:
                yield tid, data[s + off:s + off + size]


def _kernels(path):
    """(name, metadata dict) for every kernel of every gfx950 code object."""
    out = []
    for _, co in _code_objects(path):
        with tempfile.NamedTemporaryFile(suffix=".co", delete=False) as f:
            f.write(co)
            fn = f.name
        try:
            notes = subprocess.run([READELF, "--notes", fn], capture_output=True, text=True,
                                   check=True).stdout
        finally:
            os.unlink(fn)
        # one block per kernel in the metadata's kernel list
        for block in re.split(r"\n\s+- \.agpr_count:", notes)[1:]:
            meta = dict(re.findall(r"\.(\w+):\s+(\S+)", block))
            out.append((meta.get("name", "?"), meta))
    return out


pytestmark = pytest.mark.skipif(
    not os.path.exists(LIB_PATH) or READELF is None,
    reason="needs the built library and llvm-readelf")


def test_every_kernel_without_scratch_or_spills():
    ks = _kernels(LIB_PATH)
    assert len(ks) >= 30, f"expected the library's kernels, found {len(ks)}"
    bad = [(n, m.get("private_segment_fixed_size"), m.get("vgpr_spill_count")) for n, m in ks
           if int(m.get("private_segment_fixed_size", 0)) != 0
           or int(m.get("vgpr_spill_count", 0)) != 0]
    assert not bad, f"kernels with scratch or spills: {bad}"


def test_resident_row_kernels_fit_five_waves():
    ks = [(n, m) for n, m in _kernels(LIB_PATH) if "gvr_topk_kernel" in n and "Li17ELi256ELb0" in n]
    assert len(ks) == 3, [n for n, _ in ks]
    for n, m in ks:
        assert int(m["vgpr_count"]) <= 96, (n, m["vgpr_count"])
