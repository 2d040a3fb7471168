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


def test_block_inputs_are_scaled_draws_with_host_bits():
    """The decoder-block inputs: each weight is the stream's N(0,1) bf16 draw
    times its scale, rounded to bf16 (nearest-even) from the fp32 product;
    the same bits on the CPU form as the numpy form gives."""
    import torch
    from synth.device import block_device_setup
    from synth.workloads import Block, Layer, S_X, S_W_QKVG, S_RES_GATE, S_POST_NORM
    layer = Layer(hq=4, hkv=2, d=16, window=8, theta=10000.0, scale=3.87)
    for spark in (True, False):
        cfg = Block("tiny", layer, 64, spark, 2, 5, seed=3)
        s = block_device_setup(cfg, device="cpu")
        assert np.array_equal(s["x"].view(torch.int16).numpy().view(np.uint16),
                              synth.normal_bf16_bits(3, S_X, (2, 5, 64)))
        n = (2 * 4 + 2 * 2) * 16
        raw = synth.bf16_bits_to_f32(synth.normal_bf16_bits(3, S_W_QKVG, (n, 64)))
        want = synth.f32_to_bf16_bits(raw * np.float32(64 ** -0.5))
        assert np.array_equal(s["w_qkvg"].view(torch.int16).numpy().view(np.uint16), want)
        if spark:
            assert s["post_norm"] is None and s["residual_gate"].dtype == torch.float32
            g = synth.bf16_bits_to_f32(synth.normal_bf16_bits(3, S_RES_GATE, (64,))) * np.float32(0.5)
            assert np.array_equal(s["residual_gate"].numpy(), g)
        else:
            assert s["residual_gate"] is None
            p = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(synth.normal_bf16_bits(3, S_POST_NORM, (64,)))
                                       * np.float32(0.1))
            assert np.array_equal(s["post_norm"].view(torch.int16).numpy().view(np.uint16), p)


def test_sign_draws_agree_and_have_unit_mean_square():
    import torch
    idx = np.arange(5, 5 + 64 * 300, dtype=np.int64)
    a = synth.sign_bf16_bits(0, 77, idx)
    b = synth.sign_bf16_torch(0, 77, torch.from_numpy(idx)).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(a, b)
    v = synth.bf16_bits_to_f64(a).reshape(300, 64)
    assert set(np.unique(v)) == {-1.0, 1.0}
    assert np.all(np.mean(v * v, axis=1) == 1.0)          # every cached key row: mean square exactly 1
    assert abs(np.mean(v)) < 0.05


def test_cached_keys_are_unit_rms_rows():
    from synth.device import cache_values_host
    k = cache_values_host(0, 3, 1, 16, "k", 100, 400, 64)
    assert np.all(np.mean(k * k, axis=1) == 1.0)
    v = cache_values_host(0, 3, 1, 16, "v", 100, 400, 64)
    assert 0.8 < np.mean(v * v) < 1.2
