"""The shared seeded input generator: fixed check values, determinism, NaN poison."""
import numpy as np

import workloads


def test_varlen_lengths_check_values():
    rng = np.random.Generator(np.random.PCG64(45))
    lens = workloads.draw_seq_lens(workloads.CONFIGS[3], rng)
    assert list(lens[:3]) == [15187, 9609, 12124]
    assert lens.min() == 1211 and lens.max() == 15814 and int(lens.sum()) == 575004


def test_named_config_shapes_and_bytes():
    want_tokens = [1024, 32768, 131072, 575004, 190388]
    for i, cfg in enumerate(workloads.CONFIGS):
        rng = np.random.Generator(np.random.PCG64(42 + i))
        lens = workloads.draw_seq_lens(cfg, rng)
        assert int(lens.sum()) == want_tokens[i]
        assert cfg.Hq % cfg.Hkv == 0


def test_deterministic_and_poisoned():
    cfg = workloads.custom_config(2, 4, 2, 16, 40)
    a = workloads.make_inputs(cfg, 7, seq_lens=(40, 9))
    b = workloads.make_inputs(cfg, 7, seq_lens=(40, 9))
    for name in ("q", "k", "v"):
        assert np.array_equal(getattr(a, name), getattr(b, name))
    assert np.all(a.k[1, :, 9:] == workloads.BF16_QNAN) and np.all(a.v[1, :, 9:] == workloads.BF16_QNAN)
    assert not np.any(a.k[1, :, :9] == workloads.BF16_QNAN)
    c = workloads.make_inputs(cfg, 8, seq_lens=(40, 9))
    assert not np.array_equal(a.k, c.k)


def test_k_multiplier_is_exact():
    cfg = workloads.custom_config(1, 2, 1, 8, 12)
    cfg4 = workloads.custom_config(1, 2, 1, 8, 12, k_mult=4.0)
    a = workloads.make_inputs(cfg, 3)
    b = workloads.make_inputs(cfg4, 3)
    np.testing.assert_array_equal(workloads.bf16_bits_to_f32(b.k), 4 * workloads.bf16_bits_to_f32(a.k))
    assert np.array_equal(a.v, b.v) and np.array_equal(a.q, b.q)


def test_int4_generator_codes_scales_and_poison():
    cfg = workloads.custom_config(2, 4, 2, 32, 40)
    a = workloads.make_int4_inputs(cfg, 11, seq_lens=(40, 9))
    b = workloads.make_int4_inputs(cfg, 11, seq_lens=(40, 9))
    for name in ("q", "k", "v", "k_scale", "v_scale"):
        assert np.array_equal(getattr(a, name), getattr(b, name), equal_nan=name.endswith("scale"))
    assert a.k.shape == (2, 2, 40, 16) and a.k_scale.shape == (2, 2, 40)
    # rows past the valid ones: code byte 0x88 and a NaN scale; valid scales finite and positive
    assert np.all(a.k[1, :, 9:] == 0x88) and np.all(np.isnan(a.v_scale[1, :, 9:]))
    assert np.all(a.k_scale[0] > 0) and np.all(np.isfinite(a.k_scale[1, :, :9]))
    # every nibble value occurs among the valid codes
    lo = a.k[0] & 15
    hi = a.k[0] >> 4
    assert set(np.unique(np.concatenate([lo.ravel(), hi.ravel()]))) == set(range(16))
    # the same q stream as the bf16 inputs of the same seed
    assert np.array_equal(a.q, workloads.make_inputs(cfg, 11, seq_lens=(40, 9)).q)
    assert a.kv_bytes == (40 + 9) * 2 * (16 + 4) * 2
