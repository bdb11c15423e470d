"""Every kernel of the built library runs without scratch memory: no vector registers spilled
and no arrays in private memory.  Read from the library's own gfx950 code objects: the
section .hip_fatbin holds one offload bundle per source file; each bundle's gfx950 entry is
an ELF whose AMDGPU metadata note lists, per kernel, .private_segment_fixed_size and
.vgpr_spill_count.  (Scalar registers spilled go to vector register lanes, not to memory.)"""
import os
import re
import struct
import subprocess
import tempfile

import pytest

import chunked_linear_attention_segment_amd as mc

LLVM = "/opt/rocm/llvm/bin"
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"


def _code_objects(fatbin: bytes):
    """The gfx950 entries of the concatenated offload bundles."""
    pos = fatbin.find(MAGIC)
    while pos >= 0:
        n = struct.unpack_from("<Q", fatbin, pos + len(MAGIC))[0]
        p = pos + len(MAGIC) + 8
        for _ in range(n):
            off, size, tlen = struct.unpack_from("<QQQ", fatbin, p)
            triple = fatbin[p + 24:p + 24 + tlen].decode()
            p += 24 + tlen
            if "gfx950" in triple:
                yield fatbin[pos + off:pos + off + size]
        pos = fatbin.find(MAGIC, pos + 1)


def _kernels(obj: bytes):
    with tempfile.NamedTemporaryFile(suffix=".co") as f:
        f.write(obj)
        f.flush()
        notes = subprocess.run([os.path.join(LLVM, "llvm-readelf"), "--notes", f.name],
                               capture_output=True, text=True, check=True).stdout
    for block in notes.split("\n  - ")[1:]:  # one YAML list item per kernel
        name = re.search(r"\.name:\s+(\S+)", block)
        if not name:
            continue
        field = lambda k: int(re.search(r"\." + k + r":\s+(\d+)", block).group(1))
        yield name.group(1), field("private_segment_fixed_size"), field("vgpr_spill_count")


def test_no_kernel_uses_scratch():
    if not os.path.exists(mc.LIB_PATH) or not os.path.exists(os.path.join(LLVM, "llvm-readelf")):
        pytest.skip("library or llvm tools missing")
    with tempfile.TemporaryDirectory() as td:
        fb = os.path.join(td, "fatbin")
        subprocess.run([os.path.join(LLVM, "llvm-objcopy"), "--dump-section=.hip_fatbin=" + fb,
                        mc.LIB_PATH, os.path.join(td, "copy.so")], check=True)
        data = open(fb, "rb").read()
    kernels = [k for obj in _code_objects(data) for k in _kernels(obj)]
    assert len(kernels) > 100  # every source file's kernels were read
    bad = [k for k in kernels if k[1] or k[2]]
    assert not bad, bad
