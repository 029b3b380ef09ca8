"""The built library's gfx950 code objects (read from its own .hip_fatbin section with the ROCm LLVM tools): every
kernel instance runs without private (scratch) memory and without register spills to memory (only the SGPR-capped
Phase A instances spill SGPRs, into VGPR lanes). This covers the instances that
no plan selects directly (the unaligned-row twins of the direct-to-LDS kernel, picked at launch), which the GPU test
of sdm_gx_kernel_attrs cannot reach. CPU only: nothing is loaded on a device."""

import os
import subprocess

import pytest

from deterministic_fp32_gemm_amd._build import LIB_PATH

LLVM = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "llvm", "bin")
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"


def kernel_notes(tmp_path):
    objcopy, bundler, readelf = (os.path.join(LLVM, t) for t in ("llvm-objcopy", "clang-offload-bundler", "llvm-readelf"))
    if not (os.path.exists(LIB_PATH) and all(map(os.path.exists, (objcopy, bundler, readelf)))):
        pytest.skip("library not built or ROCm LLVM tools missing")
    fat = tmp_path / "fatbin.bin"
    subprocess.run([objcopy, f"--dump-section=.hip_fatbin={fat}", LIB_PATH], check=True)
    data = fat.read_bytes()
    starts, i = [], data.find(MAGIC)
    while i >= 0:
        starts.append(i)
        i = data.find(MAGIC, i + 1)
    notes = []
    for k, a in enumerate(starts):
        b = starts[k + 1] if k + 1 < len(starts) else len(data)
        part, co = tmp_path / f"b{k}.bin", tmp_path / f"b{k}.co"
        part.write_bytes(data[a:b])
        subprocess.run([bundler, "--type=o", f"--input={part}", "--targets=hipv4-amdgcn-amd-amdhsa--gfx950",
                        f"--output={co}", "--unbundle"], check=True)
        notes.append(subprocess.run([readelf, "--notes", str(co)], check=True, capture_output=True, text=True).stdout)
    return notes


def kernels(note: str):
    """(name, {field: value}) for every kernel in a code object's metadata note (keys are sorted, so the fields
    checked here, all after .name, belong to the kernel named last)."""
    out, cur = [], None
    for line in note.splitlines():
        s = line.strip().lstrip("- ").strip()
        if s.startswith(".name:") and "gx_" in s:
            cur = {}
            out.append((s.split(":", 1)[1].strip(), cur))
        elif cur is not None and s.startswith(".") and ":" in s:
            key, val = s.split(":", 1)
            cur.setdefault(key, val.strip())
    return out


def test_every_kernel_instance_has_no_scratch_and_no_spills(tmp_path):
    found = [kv for note in kernel_notes(tmp_path) for kv in kernels(note)]
    names = [n for n, _ in found]
    assert sum("gx_chain_kernel" in n for n in names) == 134
    assert sum("gx_mfma_kernel" in n for n in names) == 28
    assert sum("gx_mfma_dma_kernel" in n for n in names) == 64
    assert sum("gx_pa2_kernel" in n for n in names) == 6
    assert sum("gx_pa2_staged_kernel" in n for n in names) == 6
    for name, f in found:
        assert f.get(".private_segment_fixed_size") == "0", name
        assert f.get(".vgpr_spill_count") == "0", name
        if "gx_pa2_staged_kernel" in name:
            # capped at 80 SGPRs so that a SIMD holds 8 wavefronts: the rest spill to VGPR lanes (no memory), and the
            # VGPRs stay within the 64 that 8 wavefronts per SIMD allow
            assert int(f[".sgpr_count"]) <= 80 and int(f[".vgpr_count"]) <= 64, name
        else:
            assert f.get(".sgpr_spill_count") == "0", name
