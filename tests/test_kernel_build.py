"""Resource checks of the gfx950 copy kernel, from the compiler's own kernel
descriptors and resource-usage remarks (hipcc cross-compiles on a machine
without a GPU): no kernel variant may use scratch memory (a stack frame or a
spilled kernel argument turns the copy into a scratch-bound one), and each keeps
eight waves per SIMD."""
import os
import re
import subprocess

import pytest

from dtensor_layout_movement_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def kernel_meta(tmp_path_factory):
    out = tmp_path_factory.mktemp("isa") / "reshard.s"
    flags = [f for f in B.HIP_FLAGS if f not in ("-fPIC", "-Wall")]
    cmd = [B.hipcc(), *flags, "--cuda-device-only", "-S", "-Rpass-analysis=kernel-resource-usage",
           "-I", B.INCLUDE, "-I", B.CSRC, os.path.join(B.CSRC, "kernel.hip"), "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    text = out.read_text()
    kernels = {}
    occupancy = {}
    name = None
    for line in res.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
        m = re.search(r"Occupancy \[waves/SIMD\]: (\d+)", line)
        if m and name:
            occupancy[name] = int(m.group(1))
    for block in re.findall(r"\n  - \.agpr_count:.*?(?=\n  - \.agpr_count:|\namdhsa\.|\n\s*\.end_amdgpu_metadata)", text, re.S):
        name = re.search(r"\.name:\s+(\S+)", block).group(1)
        kernels[name] = {
            "private": int(re.search(r"\.private_segment_fixed_size:\s+(\d+)", block).group(1)),
            "vgpr": int(re.search(r"\.vgpr_count:\s+(\d+)", block).group(1)),
            "occupancy": occupancy.get(name),
            "lds": int(re.search(r"\.group_segment_fixed_size:\s+(\d+)", block).group(1)),
        }
    return kernels


def test_every_variant_is_compiled(kernel_meta):
    names = [n for n in kernel_meta if "reshard_copy_kernel" in n]
    # two pointer placements x eleven variants (16-byte items, destination
    # chunks, aligned destination chunks, copy modes, quad row bands, 2-byte-run
    # bands, gather-rows bands, Partial sums, narrow bands of dword segments,
    # narrow bands of any segments, all modes)
    assert len(names) == 22, sorted(kernel_meta)


def test_no_scratch(kernel_meta):
    for name, meta in kernel_meta.items():
        assert meta["private"] == 0, (name, meta)


def test_lds_only_in_the_window_variants(kernel_meta):
    """Only the all-modes variant allocates LDS statically (its 16 KiB window;
    the narrow-band variants take theirs as dynamic LDS at launch): a private
    array the compiler moved to LDS (an index it could not resolve) shows up
    here."""
    for name, meta in kernel_meta.items():
        want = 16384 if re.search(r"reshard_copy_kernelILb[01]ELi3E", name) else 0
        assert meta["lds"] == want, (name, meta)


def test_eight_waves_per_simd(kernel_meta):
    for name, meta in kernel_meta.items():
        assert meta["occupancy"] == 8 and meta["vgpr"] <= 64, (name, meta)
