"""Register spills of the built kernels (CPU only: reads the code-object
metadata of ``libtileattn.so`` with ``llvm-readelf``, runs nothing).

Every kernel holds its working set in registers: no kernel may use
scratch memory, so that a change that spills fails on the CPU."""

import os
import re
import shutil
import struct
import subprocess

import pytest

import tiled_attention_tileattn_amd as ta

READELF = next((p for p in ("/opt/rocm/llvm/bin/llvm-readelf", shutil.which("llvm-readelf") or "")
                if p and os.path.exists(p)), None)
BUNDLE_MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"

def _code_objects(path):
    """The gfx950 code objects of every offload bundle in the library's
    .hip_fatbin section (one bundle per compiled source)."""
    data = open(path, "rb").read()
    objs = []
    start = data.find(BUNDLE_MAGIC)
    while start >= 0:
        (entries,) = struct.unpack_from("<Q", data, start + 24)
        p = start + 32
        for _ in range(entries):
            off, size, tlen = struct.unpack_from("<QQQ", data, p)
            p += 24
            triple = data[p:p + tlen].decode()
            p += tlen
            if triple.endswith("gfx950"):
                objs.append(data[start + off:start + off + size])
        start = data.find(BUNDLE_MAGIC, start + 1)
    return objs


def _kernel_scratch(tmp_path):
    lib = ta.binding.LIB_PATH
    assert os.path.exists(lib), "libtileattn.so is not built"
    out = {}
    for i, obj in enumerate(_code_objects(lib)):
        f = tmp_path / f"co{i}.o"
        f.write_bytes(obj)
        notes = subprocess.run([READELF, "--notes", str(f)], capture_output=True, text=True, check=True).stdout
        for block in notes.split("  - .agpr_count")[1:]:
            name = re.search(r"\.name:\s+(\S+)", block).group(1)
            scratch = int(re.search(r"\.private_segment_fixed_size:\s+(\d+)", block).group(1))
            out[name] = scratch
    return out


@pytest.mark.skipif(READELF is None, reason="llvm-readelf (ROCm) not found")
def test_no_kernel_spills(tmp_path):
    scratch = _kernel_scratch(tmp_path)
    assert any("attn_fwd_16_kernel" in n for n in scratch) and any("attn_fwd_f32_kernel" in n for n in scratch)
    for name, bytes_per_lane in scratch.items():
        assert bytes_per_lane == 0, f"{name}: {bytes_per_lane} B/lane of scratch"
