"""Register budget of the layer's kernels (host-only: hipcc cross-compiles).

Each kernel's speed rests on how many of its waves a SIMD can hold: the
direct-load projection kernel overlaps the loads of one workgroup with the
MFMAs of the other only at two waves per SIMD, and the skinny decode kernel
keeps more weight loads in flight at three. A few extra live registers in a
shared helper can halve that without any test of results noticing, so this
test compiles each source with the compiler's resource report, using the
library's own flags, and checks every kernel's occupancy against the level
its launch shape was measured at, and that no kernel spills.
"""
import os
import re
import shutil
import subprocess

import pytest

from lora_mixture_experts_amd import build as B

# minimum waves per SIMD, by kernel name prefix (demangled form)
MIN_OCCUPANCY = {
    # one wave per tile (the library's choice); the 2- and 4-wave variants
    # are tuning options; the paired-run variants (last argument true) run
    # only grids of at most two waves per SIMD
    "k_gemm_skinny<true, 4, 2, 1, false>": 3,
    "k_gemm_skinny<false, 4, 2, 1, false>": 3,
    "k_gemm_skinny<true, 4, 2, 2, false>": 2,
    "k_gemm_skinny<true, 4, 2, 4, false>": 2,
    "k_gemm_skinny<false, 4, 2, 2, false>": 2,
    "k_gemm_skinny<false, 4, 2, 4, false>": 2,
    "k_gemm_skinny<true, 4, 2, 1, true>": 2,
    "k_gemm_skinny<false, 4, 2, 1, true>": 2,
    "k_gemm_skinny<true, 4, 2, 2, true>": 2,
    "k_gemm_skinny<true, 4, 2, 4, true>": 2,
    "k_gemm_skinny<false, 4, 2, 2, true>": 2,
    "k_gemm_skinny<false, 4, 2, 4, true>": 2,
    # the 8-fragment gate_up form: one wave per SIMD, for grids of fewer
    # tiles than SIMDs (a tuning option)
    "k_gemm_skinny<true, 8, 2, 1, false>": 1,
    "k_gemm_skinny<true, 8, 2, 1, true>": 1,
    "k_gemm_tiled<32, 128, 1, 4, true>": 4,
    "k_gemm_tiled<32, 128, 1, 4, false>": 4,
    "k_gemm_tiled<64, 128, 2, 2, true>": 3,
    "k_gemm_tiled<64, 128, 2, 2, false>": 3,
    "k_gemm_dma<128, 192, 2, 2, 2, true>": 2,
    "k_gemm_dma<128, 192, 2, 2, 2, false>": 2,
    "k_gemm_dma<256, 256, 2, 4, 2, true>": 2,
    "k_gemm_dma<256, 256, 2, 4, 2, false>": 2,
}
# one fragment per wave group (16-row LoRA blocks), and the groups of 2 or 4
# fragments that share one load of the LoRA A chunk (larger blocks)
MIN_OCCUPANCY_SHRINK = {"k_shrink<1, 1>": 6, "k_shrink<2, 1>": 5, "k_shrink<4, 1>": 3, "k_shrink<8, 1>": 2,
                        "k_shrink<1, 4>": 3, "k_shrink<2, 4>": 2, "k_shrink<4, 2>": 2}


def _demangle(names):
    cxxfilt = shutil.which("c++filt") or shutil.which("llvm-cxxfilt")
    if not cxxfilt:
        return {n: n for n in names}
    out = subprocess.run([cxxfilt], input="\n".join(names), capture_output=True, text=True).stdout.split("\n")
    return dict(zip(names, out))


def resource_report(src):
    """{demangled kernel: (occupancy, vgpr spills, sgpr spills)} for one source."""
    cmd = [B.HIPCC, *B.FLAGS, "-c", os.path.join(B.CSRC, src), "-o", os.devnull,
           "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    rep, cur = {}, None
    for line in r.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = m.group(1)
            rep[cur] = {}
            continue
        m = re.search(r"remark:\s+([A-Za-z ]+?)(?: \[[^\]]*\])?: (\d+)", line)
        if m and cur:
            rep[cur][m.group(1).strip()] = int(m.group(2))
    names = _demangle(list(rep))
    return {re.sub(r"^void ", "", names[k].split("(")[0]).replace("moelora::", ""): v for k, v in rep.items()}


@pytest.fixture(scope="module")
def reports():
    if not os.path.exists(B.HIPCC):
        pytest.skip("hipcc not available")
    return {src: resource_report(src) for src in B.SOURCES}


def test_no_kernel_spills(reports):
    for src, rep in reports.items():
        for name, v in rep.items():
            assert v.get("VGPRs Spill", 0) == 0 and v.get("SGPRs Spill", 0) == 0, (src, name, v)


def test_projection_kernels_keep_their_occupancy(reports):
    rep = reports["grouped_gemm.hip"]
    for name, want in MIN_OCCUPANCY.items():
        hits = [v for k, v in rep.items() if k.startswith(name)]
        assert hits, f"{name} not found among {sorted(rep)}"
        for v in hits:
            got = v.get("Occupancy")  # waves per SIMD
            assert got is not None and got >= want, (name, v)


def test_shrink_kernels_keep_their_occupancy(reports):
    rep = reports["lora_shrink.hip"]
    for name, want in MIN_OCCUPANCY_SHRINK.items():
        hits = [v for k, v in rep.items() if k.startswith(name)]
        assert hits, f"{name} not found among {sorted(rep)}"
        for v in hits:
            assert v.get("Occupancy", 0) >= want, (name, v)
