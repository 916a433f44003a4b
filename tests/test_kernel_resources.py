"""Every kernel keeps its working set in registers and LDS: no scratch
(private segment) memory, no register spills, no dynamic stack.

Compiles each HIP source for gfx950 to device assembly with the library's own
flags and reads the code-object metadata.  Scratch use would turn the
register arrays of the unrolled loops into memory traffic (it happened once,
when lambdas were left to the inliner) and would make the "allocates nothing"
promise of the C ABI depend on the runtime's scratch reservation.
"""
import os
import re
import shutil
import subprocess
import tempfile

import pytest

from weight_quantized_decode_block_amd import build as hip_build

HIP_SOURCES = [s for s in hip_build.SOURCES if s.endswith(".hip")]


def _hipcc():
    h = hip_build.hipcc()
    return h if (os.path.exists(h) or shutil.which(h)) else None


@pytest.fixture(scope="module")
def kernel_metadata():
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    flags = [f for f in hip_build.HIPCC_FLAGS if f not in ("-fPIC", "-shared")]
    out = {}
    with tempfile.TemporaryDirectory() as tmp:
        procs = {}
        for src in HIP_SOURCES:
            asm = os.path.join(tmp, src + ".s")
            cmd = [hipcc, *flags, "-I", os.path.join(hip_build.ROOT, "include"), "-x", "hip",
                   "--cuda-device-only", "-S", os.path.join(hip_build.CSRC, src), "-o", asm]
            procs[src] = (subprocess.Popen(cmd, stdout=subprocess.DEVNULL, stderr=subprocess.PIPE), asm)
        for src, (p, asm) in procs.items():
            _, err = p.communicate(timeout=600)
            assert p.returncode == 0, err.decode()[-2000:]
            text = open(asm).read()
            meta = text[text.index("amdhsa.kernels"):]
            kernels = []
            for block in re.split(r"\n\s+- \.", meta):
                name = re.search(r"\.name:\s+(\S+)", block)
                if not name or ".kd" in name.group(1):
                    continue
                fields = dict(re.findall(r"\.(private_segment_fixed_size|vgpr_spill_count|sgpr_spill_count|"
                                         r"uses_dynamic_stack|vgpr_count):\s+(\S+)", block))
                if "vgpr_count" in fields:
                    kernels.append((name.group(1), fields))
            out[src] = kernels
    return out


@pytest.mark.parametrize("src", HIP_SOURCES)
def test_no_scratch_no_spills(kernel_metadata, src):
    kernels = kernel_metadata[src]
    assert kernels, f"no kernels found in {src}"
    for name, f in kernels:
        assert f.get("private_segment_fixed_size") == "0", (name, f)
        assert f.get("vgpr_spill_count") == "0", (name, f)
        assert f.get("uses_dynamic_stack", "false") == "false", (name, f)
        assert int(f["vgpr_count"]) <= 256, (name, f)
