"""The built library's gfx950 code: every kernel runs without scratch memory.

A kernel that spills registers, or calls a function that saves registers,
writes to and reads from scratch memory in HBM -- traffic and latency that no
parity test sees.  The chained step's staging call once did (8 callee-saved
registers per call: 4.4 MB more written per 1.5B step), so this reads each
kernel's metadata from the code objects in libq4stream.so (extracted with
llvm-objdump, read with llvm-readelf; no GPU needed).
"""
import os
import re
import shutil
import subprocess

import pytest

from q4_weight_streaming_amd import _lib as q

LLVM = "/opt/rocm/llvm/bin"


def kernel_metadata(tmp_path):
    objdump, readelf = os.path.join(LLVM, "llvm-objdump"), os.path.join(LLVM, "llvm-readelf")
    if not (os.path.exists(objdump) and os.path.exists(readelf)):
        pytest.skip("llvm-objdump / llvm-readelf not found")
    if not os.path.exists(q.LIB_PATH):
        pytest.skip("libq4stream.so is not built")
    lib = tmp_path / "lib.so"
    shutil.copy(q.LIB_PATH, lib)
    subprocess.run([objdump, "--offloading", str(lib)], cwd=tmp_path, check=True, capture_output=True)
    kernels = {}
    for f in sorted(tmp_path.iterdir()):
        if "gfx950" not in f.name or f.stat().st_size == 0:
            continue
        notes = subprocess.run([readelf, "--notes", str(f)], check=True, capture_output=True, text=True).stdout
        # one kernel entry per ".name:" line; its fields follow until the next entry
        for entry in re.split(r"\n\s*- \.", notes)[1:]:
            m = re.search(r"\.name:\s+(\S+)", entry)
            if not m:
                continue
            fields = dict(re.findall(r"\.(private_segment_fixed_size|vgpr_spill_count|sgpr_count|vgpr_count):\s+(\d+)",
                                     entry))
            if "private_segment_fixed_size" in fields:
                kernels[m.group(1)] = {k: int(v) for k, v in fields.items()}
    return kernels


def test_no_kernel_uses_scratch(tmp_path):
    kernels = kernel_metadata(tmp_path)
    names = " ".join(kernels)
    for k in ("k_sweep_fused", "k_sweep_split", "k_chain", "k_gemv_q8_split", "k_attn_partial", "k_quantize"):
        assert k in names, f"{k} not found among the code objects' kernels"
    assert len(kernels) >= 40
    bad = {k: v for k, v in kernels.items() if v["private_segment_fixed_size"] or v.get("vgpr_spill_count", 0)}
    assert not bad, f"kernels with scratch memory or register spills: {bad}"
