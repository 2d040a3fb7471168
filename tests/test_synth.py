"""The seeded generator gives the same bits on the host (NumPy) and through
PyTorch integer ops, and its values have the intended N(0,1)-like moments."""
import numpy as np
import torch

import synth


def test_numpy_and_torch_forms_agree():
    for stream, off in [(1, 0), (2, 12345), (1 << 20, 7)]:
        a = synth.normal_bf16_bits(3, stream, (4096,), offset=off)
        b = synth.normal_bf16_torch_tensor(3, stream, (4096,), "cpu", offset=off)
        assert np.array_equal(a, b.view(torch.int16).numpy().view(np.uint16))


def test_slices_are_reproducible():
    full = synth.normal_bf16_bits(0, 1, (1000,))
    part = synth.normal_f32(0, 1, np.arange(500, 600))
    assert np.array_equal(full[500:600], synth.f32_to_bf16_bits(part))


def test_rounding_is_nearest_even():
    x = np.array([1.0, 1.00390625, 1.01171875, -2.5, 3.0e-3], dtype=np.float32)
    got = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)


def test_moments():
    x = synth.bf16_bits_to_f64(synth.normal_bf16_bits(0, 9, (1 << 18,)))
    assert abs(x.mean()) < 0.01
    assert abs(x.std() - 1) < 0.01
    assert abs(np.mean(x ** 4) - 2.9) < 0.1     # Irwin-Hall(12): kurtosis 3 - 0.1


def test_e4m3_codes_numpy_and_torch_agree():
    import torch
    idx = np.arange(0, 200000, 7, dtype=np.int64)
    a = synth.e4m3_codes(5, 33, idx)
    b = synth.e4m3_codes_torch(5, 33, torch.from_numpy(idx)).numpy()
    assert np.array_equal(a, b)
    mag = a & 0x7F
    assert mag.min() >= 0x20 and mag.max() <= 0x47 and 0.4 < (a >> 7).mean() < 0.6
