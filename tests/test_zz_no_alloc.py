"""GPU test of nvfp4_quantize_noalloc (the quantize entry point that allocates nothing and keeps
its amax partials in the library's static per-device array): through the C ABI, its codes,
scales and tensor scales equal nvfp4_quantize's (with a caller workspace) bit for bit, on two
calls in a row where the second is smaller. The segmented case gives the first call larger
maxima than the second, so stale contents of the shared array would show."""
import numpy as np
import pytest
import torch

import bit_block_scaled_quantize_amd as nv
import workloads
from helpers import assert_quant_equal, host, log, to_device_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _pair(x, **kw):
    """(noalloc result, nvfp4_quantize result) as host triples, transposed ones too."""
    q_n, qt_n = nv.quantize_noalloc(x, **kw)
    q_w, qt_w = nv.quantize(x, **kw)
    res = [(host(q_n), host(q_w))]
    if qt_n is not None:
        res.append((host(qt_n), host(qt_w)))
    return res


CASES = [
    ("1x16 sr", dict(block="1x16", rounding="sr", seed=7, offset=3), (1024, 2048), (96, 512)),
    ("16x16 + transposed", dict(block="16x16", rounding="rn", emit_transposed=True), (512, 1024), (64, 256)),
    ("1x16 rn", dict(block="1x16", rounding="rn"), (4096, 4096), (16, 64)),
]


@pytest.mark.parametrize("name,kw,big,small", CASES, ids=[c[0] for c in CASES])
def test_noalloc_equals_quantize_two_calls(name, kw, big, small):
    for i, shape in enumerate((big, small)):
        log(f"noalloc {name} call {i} {shape}")
        bits = workloads.with_outliers_bf16(shape, 700 + i + shape[0])
        for got, want in _pair(to_device_bf16(bits), **kw):
            assert_quant_equal(got, want, f"noalloc {name} call {i}")


def test_noalloc_segments_two_calls():
    """Per-expert tensor scales from atomic maxima in the shared array: the first call's
    experts have maxima ~1000x the second's."""
    for i, (rows, scale, seg) in enumerate((
            (640, 1000.0, [0, 128, 128, 400, 640]),
            (160, 1.0, [0, 16, 96, 160]))):
        log(f"noalloc segments call {i}")
        x = workloads.bf16_bits_to_f32(workloads.with_outliers_bf16((rows, 256), 710 + i)) * np.float32(scale)
        bits = workloads.f32_to_bf16_bits(x)
        segd = torch.from_numpy(np.array(seg, np.int64)).cuda()
        for kw in (dict(block="1x16", rounding="sr", seed=1), dict(block="16x16", rounding="rn")):
            for got, want in _pair(to_device_bf16(bits), segments=segd, **kw):
                assert_quant_equal(got, want, f"noalloc segments call {i} {kw['block']}")


def test_noalloc_rejects_too_many_segments():
    x = to_device_bf16(workloads.normal_bf16((16, 32), 720))
    seg = torch.zeros((16386,), dtype=torch.int64, device="cuda")
    seg[-1] = 16
    with pytest.raises(nv.NVFP4Error, match="at most 16384 segments"):
        nv.quantize_noalloc(x, segments=seg)
