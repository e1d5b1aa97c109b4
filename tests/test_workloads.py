"""The seeded input generators (CPU only)."""
import numpy as np
import torch

import workloads


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(2)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 1e3,
                        np.float32([1.0, -2.5, 3.0e38, 1e-40])])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(workloads.f32_to_bf16_bits(x), ref)
    back = workloads.bf16_bits_to_f32(ref)
    assert np.array_equal(back, torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_generators_are_deterministic_and_shaped():
    a, w = workloads.tiny()
    a2, _ = workloads.tiny()
    assert a.shape == (256, 256) and w.shape == (256, 256) and np.array_equal(a, a2)
    f = workloads.bf16_bits_to_f32(a)
    assert (np.abs(f) > 10).sum() >= 50           # ~65 outliers scaled by 50


def test_moe_routing_statistics():
    off = workloads.moe_routing()
    cnt = np.diff(off)
    assert off[-1] == 16384 * 6 and cnt.min() > 0 and cnt.max() == 13452


def test_padded_token_layout():
    off = np.array([0, 37, 37, 167, 231], np.int64)
    pad = workloads.pad_offsets(off, 64)
    assert list(pad) == [0, 64, 64, 256, 320]
    bits = np.arange(231 * 3, dtype=np.uint16).reshape(231, 3)
    out = workloads.scatter_rows(bits, off, pad)
    assert out.shape == (320, 3)
    assert np.array_equal(out[0:37], bits[0:37]) and np.all(out[37:64] == 0)
    assert np.array_equal(out[64:194], bits[37:167]) and np.all(out[194:256] == 0)
    assert np.array_equal(out[256:320], bits[167:231])
