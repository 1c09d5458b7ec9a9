"""Host-side check of the built library's gfx950 code object (no GPU needed):
every kernel runs without a private (scratch) segment and spills no vector
register. The chained kernel holds its accumulators, fragments and ring
addresses in nearly the whole register file, so an edit that pushes it over
shows up here instead of as a slower step."""
import os
import re
import shutil
import subprocess

import pytest

import muon_newton_schulz_04_amd as mu

LLVM = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "llvm", "bin")


def kernel_metadata(lib_path, workdir):
    """Per-kernel metadata of every gfx950 code object in the library's
    offload bundles: name -> {field: int}."""
    objdump, readelf = os.path.join(LLVM, "llvm-objdump"), os.path.join(LLVM, "llvm-readelf")
    if not (os.path.exists(objdump) and os.path.exists(readelf)):
        pytest.skip("ROCm LLVM tools not found")
    # the bundles are written next to the input file: work on a copy
    copy = os.path.join(workdir, "lib.so")
    shutil.copyfile(lib_path, copy)
    subprocess.run([objdump, "--offloading", copy], check=True, cwd=workdir,
                   stdout=subprocess.DEVNULL, stderr=subprocess.PIPE)
    objs = sorted(f for f in os.listdir(workdir) if f.endswith("--gfx950"))
    assert objs, "no gfx950 code object in the library"
    kernels = {}
    for o in objs:
        notes = subprocess.run([readelf, "--notes", os.path.join(workdir, o)], check=True,
                               stdout=subprocess.PIPE, text=True).stdout
        cur = None
        for line in notes.splitlines():
            m = re.match(r"\s*(?:- )?\.name:\s+(\S+)", line)
            if m:
                cur = kernels.setdefault(m.group(1), {})
                continue
            m = re.match(r"\s*\.(private_segment_fixed_size|vgpr_count|vgpr_spill_count|agpr_count):\s+(\d+)", line)
            if m and cur is not None:
                cur[m.group(1)] = int(m.group(2))
    return kernels


def test_no_kernel_uses_scratch_or_spills_vector_registers(tmp_path):
    if not os.path.exists(mu.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    ks = kernel_metadata(mu.LIB_PATH, str(tmp_path))
    names = " ".join(ks)
    for k in ("chain16_kernel", "gemm16_kernel", "gemm32_kernel", "momentum_x0_kernel", "adam_kernel"):
        assert k in names, f"{k} missing from the code object"
    for name, md in ks.items():
        assert "private_segment_fixed_size" in md and "vgpr_spill_count" in md, name
        assert md["private_segment_fixed_size"] == 0, (name, md)
        assert md["vgpr_spill_count"] == 0, (name, md)
        assert md["vgpr_count"] <= 512, (name, md)
