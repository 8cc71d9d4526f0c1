"""Register and scratch budgets of the gfx950 kernels, read from the code
object metadata of a device-only compile of the library's sources (CPU only:
hipcc cross-compiles, nothing runs).

Occupancy is designed, not incidental: the persistent expert kernel runs four
256-thread blocks per CU and the prefill kernels two 512-thread blocks per
CU, both at four waves per SIMD, which needs at most 128 VGPRs (arch + acc)
per wave. A spill would put per-lane scratch traffic in the hot loops and
make the runtime reserve scratch memory behind the caller's back.
"""
import os
import re
import shutil
import subprocess

import pytest

from bit_quantized_moe_block_amd import build as BLD

CSRC = os.path.join(os.path.dirname(BLD.__file__), "csrc")


@pytest.fixture(scope="module")
def kernel_meta(tmp_path_factory):
    if not os.path.exists(BLD.HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / "kernels.s"
    flags = [f for f in BLD.FLAGS if f not in ("-shared", "-fPIC")]
    cmd = [BLD.HIPCC] + flags + ["--cuda-device-only", "-S", os.path.join(CSRC, "kernels.hip"),
                                 "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    text = out.read_text()
    meta = {}
    for blk in re.findall(r"(\.agpr_count:.*?\.wavefront_size:\s+\d+)", text, re.S):
        name = re.search(r"\.name:\s+(\S+)", blk).group(1)
        get = lambda key: int(re.search(key + r":\s+(\d+)", blk).group(1))
        meta[name] = dict(vgpr=get(r"\.vgpr_count"), agpr=get(r"\.agpr_count"),
                          spill=get(r"\.vgpr_spill_count"),
                          private=get(r"\.private_segment_fixed_size"))
    assert meta, "no kernel metadata in the device assembly"
    return meta


def test_no_kernel_spills_or_uses_scratch(kernel_meta):
    for name, m in kernel_meta.items():
        assert m["spill"] == 0 and m["private"] == 0, (name, m)


@pytest.mark.parametrize("kind", ["expert_kernel", "prefill_kernel"])
def test_four_waves_per_simd_fit(kernel_meta, kind):
    found = [(n, m) for n, m in kernel_meta.items() if kind in n]
    assert found, kind
    for name, m in found:
        assert m["vgpr"] + m["agpr"] <= 128, (name, m)


def test_dynamic_lds_arrays_are_16_byte_aligned():
    """The dynamic LDS array starts right after the kernel's static LDS,
    rounded up to the array's declared alignment. MFMA operands are read
    and staged with 16-byte LDS accesses, which need 16-byte aligned
    addresses: with the element type's 2-byte alignment the array started
    12 bytes in and every such access was split."""
    src = open(os.path.join(CSRC, "kernels.hip")).read()
    decls = re.findall(r"extern __shared__[^;]*;", src)
    assert decls
    for d in decls:
        if "uint32_t" in d:  # 4-byte accesses only (route bucketing)
            continue
        assert "__align__(16)" in d, d
