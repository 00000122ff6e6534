"""Resource checks on the kernels of the built library (CPU only).

The device code objects of ``libwq.so`` (built here from this repository's
sources) are extracted with the ROCm LLVM tools and their kernel metadata is
read: no kernel may use scratch memory or spill registers.  A spill turns a
bandwidth-bound kernel into a much slower one with no change in its results
(the eight-tile gate/up pair once spilled 228 bytes per lane and ran 2.4x
slower), so parity tests alone do not catch it.
"""

import os
import re
import shutil
import subprocess

import pytest

import bit_quantized_linear_int4_amd as wq

LLVM = "/opt/rocm/llvm/bin"
TOOLS = [os.path.join(LLVM, t) for t in ("llvm-objcopy", "clang-offload-bundler", "llvm-readelf")]
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"

pytestmark = pytest.mark.skipif(
    not os.path.exists(wq.library_path()) or not all(os.path.exists(t) for t in TOOLS),
    reason="libwq.so or the ROCm LLVM tools are missing")


def kernel_metadata(tmp_path):
    fatbin = tmp_path / "fatbin.bin"
    subprocess.run([TOOLS[0], f"--dump-section=.hip_fatbin={fatbin}", wq.library_path(),
                    str(tmp_path / "stripped.so")], check=True, capture_output=True)
    data = fatbin.read_bytes()
    starts = [m.start() for m in re.finditer(re.escape(MAGIC), data)]
    kernels = {}
    for i, s in enumerate(starts):
        chunk = tmp_path / f"bundle{i}.bin"
        chunk.write_bytes(data[s:starts[i + 1] if i + 1 < len(starts) else len(data)])
        co = tmp_path / f"bundle{i}.co"
        subprocess.run([TOOLS[1], "--unbundle", "--type=o", f"--input={chunk}",
                        "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", f"--output={co}"],
                       check=True, capture_output=True)
        notes = subprocess.run([TOOLS[2], "--notes", str(co)], check=True, capture_output=True,
                               text=True).stdout
        name = None
        for line in notes.splitlines():
            line = line.strip()
            if line.startswith(".name:"):
                name = line.split(":", 1)[1].strip()
                kernels.setdefault(name, {})
            elif name and ":" in line and line.split(":", 1)[0] in (
                    ".private_segment_fixed_size", ".vgpr_spill_count", ".sgpr_spill_count",
                    ".vgpr_count"):
                k, v = line.split(":", 1)
                kernels[name][k[1:]] = int(v)
    return kernels


def test_no_kernel_uses_scratch_or_spills(tmp_path):
    kernels = kernel_metadata(tmp_path)
    # every family of the library is present
    for fam in ("stream_kernel", "gemm_i4_kernel", "gemm_kernel", "quant_int4_kernel",
                "pack_nf4_kernel", "int8_gemm_kernel", "permute_cols_kernel", "dequant_kernel"):
        assert any(fam in k for k in kernels), fam
    bad = {k: v for k, v in kernels.items()
           if v.get("private_segment_fixed_size", 0) or v.get("vgpr_spill_count", 0)
           or v.get("sgpr_spill_count", 0)}
    assert not bad, f"{len(bad)} kernels use scratch or spill, e.g. {sorted(bad)[:3]}"
