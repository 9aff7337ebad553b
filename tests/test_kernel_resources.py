"""Register budget of the built kernels, read from the AMDGPU metadata of libmifa.so's own device
code: no kernel spills vector registers or uses scratch memory, and the forward kernels stay within the 256 vector
registers per lane that two waves per SIMD leave each wave, the d = 64 ones within the 168 of three
(the launch shapes assume it)."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "io_aware_softmax_mifa_amd", "libmifa.so")
LLVM = "/opt/rocm/llvm/bin"

pytestmark = pytest.mark.skipif(
    not os.path.exists(LIB) or not os.path.exists(os.path.join(LLVM, "clang-offload-bundler")),
    reason="libmifa.so or the ROCm LLVM tools missing")


def kernel_metadata(tmp_path):
    fat, co = str(tmp_path / "fatbin.bin"), str(tmp_path / "dev.co")
    subprocess.run([os.path.join(LLVM, "llvm-objcopy"), f"--dump-section=.hip_fatbin={fat}", LIB,
                    str(tmp_path / "copy.so")], check=True, capture_output=True)
    # one offload bundle per translation unit, back to back in the section
    data = open(fat, "rb").read()
    magic = b"__CLANG_OFFLOAD_BUNDLE__"
    starts = [m.start() for m in re.finditer(re.escape(magic), data)]
    assert starts and starts[0] == 0, "no offload bundle in .hip_fatbin"
    notes = ""
    for i, a in enumerate(starts):
        part = str(tmp_path / f"bundle{i}.bin")
        with open(part, "wb") as f:
            f.write(data[a:starts[i + 1] if i + 1 < len(starts) else len(data)])
        subprocess.run([os.path.join(LLVM, "clang-offload-bundler"), "--unbundle", "--type=o", f"--input={part}",
                        "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", f"--output={co}"], check=True,
                       capture_output=True)
        notes += subprocess.run([os.path.join(LLVM, "llvm-readelf"), "--notes", co], check=True,
                                capture_output=True, text=True).stdout
    kernels, cur = {}, None
    for line in notes.splitlines():
        m = re.match(r"\s*\.name:\s+(\S+)", line)
        if m:
            cur = kernels.setdefault(m.group(1), {})
            continue
        m = re.match(r"\s*\.(private_segment_fixed_size|vgpr_count|agpr_count|vgpr_spill_count|sgpr_spill_count):\s+(\d+)",
                     line)
        if m and cur is not None:
            cur[m.group(1)] = int(m.group(2))
    return kernels


def test_no_spills_and_forward_register_budget(tmp_path):
    if shutil.which(os.path.join(LLVM, "llvm-readelf")) is None:
        pytest.skip("llvm-readelf missing")
    ks = kernel_metadata(tmp_path)
    fwd = [n for n in ks if "mifa_fwd_kernel" in n]
    assert len(fwd) == 16, sorted(ks)  # d 64|128 x causal|not x three shapes, + two paired causal
    for part in ("dq_kernel", "dkdv_kernel", "row_dot_kernel", "softmax_resident", "softmax_stream",
                 "merge_splits", "clock_probe_kernel"):
        assert any(part in n for n in ks), part
    for name, m in ks.items():
        assert m.get("private_segment_fixed_size") == 0, (name, m)
        # (SGPR spills go to VGPR lanes, not to memory; a few in the softmax kernels are harmless)
        assert m.get("vgpr_spill_count", 0) == 0, (name, m)
    for name in fwd:
        assert ks[name]["vgpr_count"] <= 256, (name, ks[name])
        if "CfgILi64E" in name:  # d = 64: three waves per SIMD (512 / 3, in granules of 8)
            assert ks[name]["vgpr_count"] <= 168, (name, ks[name])
