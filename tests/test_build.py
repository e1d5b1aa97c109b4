"""Build checks that need no GPU: the compiler's resource report for the device code. A
register spill in the GEMM main loops (scratch memory per lane) would cost far more than any
change that caused it, so every kernel must compile without scratch."""
import shutil

import pytest

from bit_block_scaled_quantize_amd import build


@pytest.fixture(scope="module")
def usage():
    if not (shutil.which("hipcc") or __import__("os").path.exists("/opt/rocm/bin/hipcc")):
        pytest.skip("hipcc not available")
    return build.resource_usage()


def test_no_kernel_spills(usage):
    assert usage, "no kernels reported"
    spills = {k: v for k, v in usage.items() if v.get("scratch", 0) > 0}
    assert not spills, f"kernels using scratch (register spills): {spills}"


def test_gemm_kernels_present(usage):
    names = " ".join(usage)
    for k in ("k_gemm_big", "k_grouped_gemm_big", "k_grouped_gemm_k_big", "k_encode_1x16", "k_rht"):
        assert k in names, k
