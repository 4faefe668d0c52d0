"""Register budget of the kernels, checked at compile time (no GPU needed).

The decode GEMV kernels are designed so that a whole decode step's grid is
resident at once (8 waves per SIMD, at most 64 VGPRs), and the prefill GEMM
kernels for 2 workgroups per CU.  A kernel that spills to scratch memory runs
markedly slower on this chip, so no kernel may use scratch.  The compiler's
resource-usage remarks give VGPRs, scratch bytes per lane and occupancy for
every kernel of a source file.
"""
import glob
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "bit_moe_expert_nvfp4_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# kernel name fragment -> occupancy (waves per SIMD) the kernel is designed for
OCCUPANCY = {
    "fc1_decode_kernel": 8,
    "fc2_decode_kernel": 8,
    "fc1_prefill_kernel": 2,
    "fc2_prefill_kernel": 2,
    "fc1_prefill_delta_kernel": 2,
    "fc2_prefill_delta_kernel": 2,
}


def _resource_usage(src):
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "--cuda-device-only", "-c", src, "-o", os.devnull, "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    kernels, cur = {}, None
    for line in r.stderr.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = kernels.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+(VGPRs|ScratchSize \[bytes/lane\]|Occupancy \[waves/SIMD\]): (\d+)", line)
        if m and cur is not None:
            cur[m.group(1).split()[0]] = int(m.group(2))
    return kernels


_HAVE_HIPCC = bool(shutil.which(HIPCC)) or os.path.exists(HIPCC)


@pytest.fixture(scope="module")
def usage():
    out = {}
    for src in sorted(glob.glob(os.path.join(CSRC, "*.hip"))):
        out.update(_resource_usage(src))
    return out


@pytest.mark.skipif(not _HAVE_HIPCC, reason="hipcc not available")
def test_no_kernel_uses_scratch(usage):
    assert usage, "no kernel remarks parsed"
    spilled = {n: r.get("ScratchSize") for n, r in usage.items() if r.get("ScratchSize") != 0}
    assert not spilled, f"kernels using scratch (bytes per lane): {spilled}"


@pytest.mark.skipif(not _HAVE_HIPCC, reason="hipcc not available")
@pytest.mark.parametrize("frag,waves", sorted(OCCUPANCY.items()))
def test_hot_kernels_keep_their_occupancy(usage, frag, waves):
    # match the exact kernel name (fc1_prefill_kernel must not match fc1_prefill_delta_kernel); a
    # template's every instantiation counts
    hits = [n for n in usage if re.search(rf"\d{frag}[EI]", n)]
    assert hits, f"{frag}: not found"
    for h in hits:
        assert usage[h].get("Occupancy", 0) >= waves, f"{h}: occupancy {usage[h]}"


@pytest.mark.skipif(not _HAVE_HIPCC, reason="hipcc not available")
def test_m0_written_only_by_the_lds_dma_asm():
    """The prefill pipeline's inline asm sets m0 (the LDS destination of
    global_load_lds_dwordx4) and lists it as clobbered.  m0 is a reserved
    register the compiler does not preserve across such asm, so no other
    instruction of these kernels may read or write it: every m0 access in the
    generated code must be the asm's own s_mov_b32 m0 directly followed by its
    LDS-DMA load (global_load_lds_dword or _dwordx4)."""
    src = os.path.join(CSRC, "moe_prefill.hip")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "--cuda-device-only", "-S", src, "-o", "-"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l.strip() for l in r.stdout.splitlines()]
    code = [l for l in lines if l and not l.startswith((";", ".", "//")) and not l.endswith(":")]
    writes = 0
    for i, l in enumerate(code):
        if re.search(r"\bm0\b", l):
            assert l.startswith("s_mov_b32 m0,"), f"m0 used outside the LDS-DMA asm: {l}"
            assert i + 1 < len(code) and code[i + 1].startswith("global_load_lds_dword"), \
                f"m0 write not followed by its LDS-DMA load: {l} / {code[i + 1] if i + 1 < len(code) else ''}"
            writes += 1
    assert writes > 0, "no LDS-DMA loads found"
