"""Register and LDS use of the hot kernels, read from the built library's gfx950 code objects
(CPU only: no kernel runs).

Several kernels depend on the compiler keeping their working set in registers: the
independent-wavefront forward kernel (the Mamba-1.4B layer), its split modes (the million-token
config), its four-wavefront workgroups (the Mamba-130M layer), the chunked MFMA kernel,
the decode kernels. A compiler or source change that makes them spill shows up here as scratch
use, before any timing does. Kernels with a known, small spill are held to it.

The code objects are taken from the library's .hip_fatbin section (one offload bundle per
translation unit) with the LLVM tools of the ROCm install; their AMDGPU metadata note lists, per
kernel, its VGPRs, spilled VGPRs, scratch bytes per lane and LDS bytes.
"""
import os
import re
import shutil
import subprocess
import tempfile

import pytest

import selective_state_space_24_amd as ssm

LLVM = "/opt/rocm/llvm/bin"
TOOLS = ("llvm-objcopy", "clang-offload-bundler", "llvm-readelf")


def _kernel_metadata():
    yaml = pytest.importorskip("yaml")
    for t in TOOLS:
        if not os.path.exists(os.path.join(LLVM, t)):
            pytest.skip(f"{t} not found under {LLVM}")
    if not os.path.exists(ssm.LIB_PATH):
        pytest.skip("library not built")
    tmp = tempfile.mkdtemp()
    try:
        fb = os.path.join(tmp, "fatbin.bin")
        subprocess.run([os.path.join(LLVM, "llvm-objcopy"), f"--dump-section=.hip_fatbin={fb}",
                        ssm.LIB_PATH, os.path.join(tmp, "copy.so")], check=True)
        data = open(fb, "rb").read()
        magic = b"__CLANG_OFFLOAD_BUNDLE__"
        starts = [m.start() for m in re.finditer(re.escape(magic), data)] + [len(data)]
        kernels = {}
        for i in range(len(starts) - 1):
            part = os.path.join(tmp, f"b{i}.bin")
            co = os.path.join(tmp, f"b{i}.co")
            with open(part, "wb") as f:
                f.write(data[starts[i]:starts[i + 1]])
            subprocess.run([os.path.join(LLVM, "clang-offload-bundler"), "--type=o",
                            "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", f"--input={part}",
                            f"--output={co}", "--unbundle"], check=True)
            notes = subprocess.run([os.path.join(LLVM, "llvm-readelf"), "--notes", co],
                                   capture_output=True, text=True, check=True).stdout
            doc = notes[notes.index("---"):notes.index("\n...") + 4]
            for k in yaml.safe_load(doc)["amdhsa.kernels"]:
                kernels[k[".name"]] = {"vgpr": k[".vgpr_count"],
                                       "spill": k.get(".vgpr_spill_count", 0),
                                       "scratch": k[".private_segment_fixed_size"],
                                       "lds": k[".group_segment_fixed_size"]}
        return kernels
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


@pytest.fixture(scope="module")
def kernels():
    return _kernel_metadata()


def _one(kernels, fragment):
    hits = [n for n in kernels if fragment in n]
    assert len(hits) == 1, f"{fragment}: {len(hits)} kernels match"
    return kernels[hits[0]]


# (mangled-name fragment, what it is, largest spill allowed in VGPRs, largest LDS in bytes)
HOT = [
    ("scan_fwd_wave_kernelItLb0ELb1ELb0ELi0ELi8E",
     "independent-wavefront forward, bf16, gate (Mamba-1.4B layer)", 0, 160 * 1024),
    ("scan_fwd_wave_kernelItLb0ELb0ELb0ELi1ELi8E",
     "its segment-summary mode (splits into shorter segments)", 0, 160 * 1024),
    ("scan_fwd_wave_kernelItLb0ELb1ELb0ELi3ELi8E",
     "its zero-start output pass of a split, gate (million-token config)", 0, 160 * 1024),
    ("scan_fwd_wave_kernelItLb0ELb1ELb0ELi4ELi8E",
     "its correcting pass of a split, gate (million-token config)", 0, 160 * 1024),
    ("scan_fwd_wave_kernelItLb0ELb0ELb0ELi2ELi8E",
     "its checkpoint mode (backward of the Mamba-1.4B layer)", 11, 160 * 1024),
    ("scan_fwd_wave_kernelItLb0ELb1ELb0ELi0ELi4E",
     "independent-wavefront forward in four-wavefront workgroups, gate (Mamba-130M layer)", 0,
     160 * 1024),
    ("ssd_fwd_kernelILi128ELb1E", "chunked MFMA form, N 128, gate (scalar-decay heads)", 0,
     160 * 1024),
    ("decode_vec_kernelItLi16ELb0ELb1E", "decode step, bf16, N 16, gate", 0, 0),
    ("bwd_kernelItLi4ELb1E", "backward reverse kernel, bf16, N <= 16, gate", 0, 80 * 1024),
    ("scan_complex_kernelItLi2ELi8ELb1E", "complex-A forward, bf16, N <= 16, gate", 0, 64 * 1024),
    ("scan_complex_kernelIfLi4ELi8ELb1E", "complex-A forward, fp32, N <= 32, gate", 0, 64 * 1024),
    ("bwd_wide_kernelItLi16ELi8ELi4ELb1ELb0ELb1E",
     "backward reverse kernel, one A per head, N 128, gate", 57, 160 * 1024),
]


@pytest.mark.parametrize("frag,what,max_spill,max_lds", HOT, ids=[h[0] for h in HOT])
def test_hot_kernel_registers(kernels, frag, what, max_spill, max_lds):
    k = _one(kernels, frag)
    assert k["vgpr"] <= 512, what
    assert k["spill"] <= max_spill, f"{what}: {k['spill']} VGPRs spilled ({k['scratch']} B/lane)"
    if max_spill == 0:
        assert k["scratch"] == 0, f"{what}: {k['scratch']} bytes of scratch per lane"
    assert k["lds"] <= max_lds, f"{what}: {k['lds']} bytes of LDS"


def test_lds_budgets_allow_the_planned_occupancy(kernels):
    """The occupancy the kernels are designed for: two backward workgroups per CU
    would need at most 80 KB each; the kernels that run one per CU fit 160 KB."""
    assert _one(kernels, "bwd_kernelItLi4ELb1E")["lds"] <= 80 * 1024  # two per CU
    for frag, *_ in HOT:
        assert _one(kernels, frag)["lds"] <= 160 * 1024
