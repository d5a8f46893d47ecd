"""CPU checks of the seeded input generator (shared by both sides, no method arithmetic)."""
import numpy as np

import synth
from synth import workloads as W


def test_splitmix64_matches_published_outputs():
    # SplitMix64 seeded with 0: the first two outputs of the reference generator
    outs = synth._mix64(np.array([0x9E3779B97F4A7C15, (2 * 0x9E3779B97F4A7C15) % 2**64], dtype=np.uint64))
    assert int(outs[0]) == 0xE220A8397B1DCDAF
    assert int(outs[1]) == 0x6E789E6AA1B965F4


def test_normal_table_is_the_standard_normal_quantile():
    t = synth.normal_table()
    assert t.dtype == np.float32 and t.shape == (65536,)
    np.testing.assert_array_equal(t, -t[::-1])            # symmetric
    assert abs(float(t.mean())) < 1e-6
    assert abs(float(t.std()) - 1.0) < 1e-4
    assert np.all(np.diff(t) > 0)
    assert abs(float(t[32767]) - (-1.9123e-05)) < 1e-7  # Phi^-1(32767.5 / 65536)


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, -2.5, 3.14159265], dtype=np.float32)
    b = synth.f32_to_bf16_bits(x)
    back = synth.bf16_bits_to_f32(b)
    np.testing.assert_array_equal(back[:4], np.array([1.0, 1.0, 1.0 + 2**-6, -2.5], dtype=np.float32))
    assert abs(float(back[4]) - 3.140625) < 1e-7


def test_e4m3_encoding_is_nearest_even_and_saturating():
    import torch
    x = np.array([1.0, 1.0625, 1.1875, 1.125, -3.5, 448.0, 449.0, 1000.0, -1e6, 0.0, -0.0,
                  2.0 ** -10, 3 * 2.0 ** -10, 2.0 ** -6, 0.015625 * 0.999], dtype=np.float32)
    c = synth.f32_to_e4m3(x)
    # 1.0625 lies halfway between 1.0 (mantissa 0) and 1.125 (1): even -> 1.0;
    # 1.1875 halfway between 1.125 (1) and 1.25 (2): even -> 1.25
    assert list(c[:5]) == [0x38, 0x38, 0x3A, 0x39, 0xC6]
    assert list(c[5:9]) == [0x7E, 0x7E, 0x7E, 0xFE]          # saturation at +-448
    assert c[9] == 0x00 and c[10] == 0x80                    # signed zeros
    assert c[11] == 0x00 and c[12] == 0x02                   # subnormal ties to even
    assert c[13] == 0x08 and c[14] == 0x08                   # rounds up into the smallest normal
    # inside the finite range the encoding is torch's round-to-nearest-even conversion
    rng = np.random.default_rng(5)
    v = np.concatenate([rng.standard_normal(100000) * 20, rng.standard_normal(100000) * 0.02]).astype(np.float32)
    v = v[np.abs(v) < 448]
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(synth.f32_to_e4m3(v), ref)


def test_generation_is_deterministic_and_seed_dependent():
    a = synth.TensorSpec((1, 2, 50, 8), 7, synth.TID_Q)
    b = synth.TensorSpec((1, 2, 50, 8), 8, synth.TID_Q)
    np.testing.assert_array_equal(synth.host_tensor(a), synth.host_tensor(a))
    assert not np.array_equal(synth.host_tensor(a), synth.host_tensor(b))
    c = synth.TensorSpec((1, 2, 50, 8), 7, synth.TID_K)
    assert not np.array_equal(synth.host_tensor(a), synth.host_tensor(c))


def test_structured_index_inputs_follow_the_recipe():
    wl = W.small("s", S=1, T=256, N=1024, H=8, Hkv=2, d=64, dI=64, k=4, structure="band_sink_needles")
    sp = wl.specs()
    qI = synth.bf16_bits_to_f32(synth.host_tensor(sp["q_idx"]))
    kI = synth.bf16_bits_to_f32(synth.host_tensor(sp["k_idx"]))
    assert np.all(qI[..., 0] == 1.0)                                   # boost channel
    mask = wl.boost_mask()
    assert mask[0, 0, 0] == 1 and mask.sum(axis=-1).max() == 1 + 7    # sink + needles (nb - 1 = 7)
    base = synth.TensorSpec(sp["k_idx"].shape, wl.seed, synth.TID_KI)
    raw = synth.values_at(base, np.arange(int(np.prod(base.shape)))).reshape(base.shape)
    boosted = np.repeat(mask.astype(bool), 128, axis=-1)[..., : wl.N]
    expect0 = np.where(boosted, raw[..., 0] + np.float32(24.0), raw[..., 0])
    np.testing.assert_array_equal(kI[..., 0], synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(expect0)))
    # rotary band: q.k over dims 1..16 is 3 * sum_i cos(theta_i * (p - j)); 24 at distance 0
    band_q = qI[0, 0, :, 1:17].astype(np.float64)
    band_k = kI[0, 0, :, 1:17].astype(np.float64)
    p = wl.N - wl.T + 10
    dot0 = band_q[10] @ band_k[p]
    assert abs(dot0 - 24.0) < 0.2
    far = band_q[10] @ band_k[p - 600]
    assert abs(far) < 24.0


def test_needles_are_distinct_and_in_range():
    nd = synth.needle_blocks(123, 3, 4, 50, 8)
    for s in range(3):
        for g in range(4):
            v = nd[s, g]
            assert len(set(v.tolist())) == 8 and v.min() >= 1 and v.max() <= 49


def test_workloads_match_the_configured_shapes():
    assert (W.C1.T, W.C1.N, W.C1.H, W.C1.Hkv, W.C1.d, W.C1.dI, W.C1.k) == (32768, 32768, 64, 8, 128, 64, 16)
    assert (W.C2.T, W.C2.nb) == (131072, 1024)
    assert (W.C3.S, W.C3.T, W.C3.N, W.C3.nb) == (16, 1, 1 << 20, 8192)
    assert (W.C4.T, W.C4.N, W.C4.N - W.C4.T) == (8192, 1 << 20, 1040384)
    rows = W.C4.sampled_rows(64, always=[0, 127, 128, 8191])
    assert len(rows) == 64 and {0, 127, 128, 8191} <= set(rows.tolist())
