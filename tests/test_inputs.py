"""Pins for the seeded input module: bf16 rounding and the workload recipes."""
import numpy as np
import pytest
import torch

import hyena_inputs as hi


def _f(bits):
    return np.array([bits], dtype=np.uint32).view(np.float32)


def test_bf16_rne_ties_and_boundaries():
    one = 0x3F800000
    # exactly halfway between 1 and 1+2^-7: ties to even (1.0)
    assert hi.bf16_bits_rne(_f(one | 0x8000))[0] == 0x3F80
    # halfway between 1+2^-7 and 1+2^-6: ties to even (1+2^-6)
    assert hi.bf16_bits_rne(_f(one | 0x18000))[0] == 0x3F82
    # just above / below halfway
    assert hi.bf16_bits_rne(_f(one | 0x8001))[0] == 0x3F81
    assert hi.bf16_bits_rne(_f(one | 0x7FFF))[0] == 0x3F80
    # rounding that carries into the exponent
    assert hi.bf16_bits_rne(_f(0x3FFFFFFF))[0] == 0x4000
    # signs, zero, infinities
    assert hi.bf16_bits_rne(np.array([-0.0], np.float32))[0] == 0x8000
    assert hi.bf16_bits_rne(np.array([np.inf], np.float32))[0] == 0x7F80
    assert hi.bf16_bits_rne(np.array([-np.inf], np.float32))[0] == 0xFF80
    assert np.isnan(hi.bf16_bits_to_f32(hi.bf16_bits_rne(np.array([np.nan], np.float32))))[0]


def test_bf16_matches_torch_conversion():
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 100000),
                        rng.standard_normal(1000).astype(np.float32)]).astype(np.float32)
    ours = hi.bf16_bits_rne(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, theirs)
    np.testing.assert_array_equal(hi.bf16_bits_to_f32(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_workloads_table():
    assert [w.order for w in hi.WORKLOADS] == [2, 2, 3, 2, 2, 2, 2, 2, 2, 2]
    assert [w.mode for w in hi.WORKLOADS] == ["causal"] * 4 + ["linear", "circular", "circular", "linear", "causal", "causal"]
    assert [w.filter for w in hi.WORKLOADS] == ["exp"] * 7 + ["film", "exp", "exp"]
    assert [w.d_model for w in hi.WORKLOADS] == [0] * 8 + [768, 0]
    assert [w.decode_block for w in hi.WORKLOADS] == [0] * 9 + [256]
    assert hi.WORKLOADS[1].tokens_channels == 4 * 768 * 8192
    assert hi.WORKLOADS[3].dims == (1 << 20,)
    assert hi.WORKLOADS[4].support == 127 ** 3
    assert hi.WORKLOADS[5].support == 8192 and hi.WORKLOADS[6].support == 64 ** 3


def test_draws_are_seeded_and_shaped():
    w = hi.WORKLOADS[0]
    v1, xs1 = hi.draw_activations(w)
    v2, xs2 = hi.draw_activations(w)
    assert v1.shape == (1, 16, 1024) and v1.dtype == np.float32 and len(xs1) == 2
    np.testing.assert_array_equal(v1, v2)
    np.testing.assert_array_equal(xs1[1], xs2[1])
    assert abs(v1.std() - 1) < 0.05
    p = hi.draw_filter_params(w)
    assert len(p) == 2 and p[0]["W1"].shape == (64, 64) and p[0]["W2"].shape == (16, 64)
    assert np.all(p[1]["alpha"] >= 0.3) and np.all(p[1]["alpha"] < 3.0)
    bound = np.sqrt(6 / (64 + 16))
    assert np.max(np.abs(p[0]["W2"])) <= bound


def test_bf16_workload_values_are_representable():
    w = hi.WORKLOADS[1].with_(B=1, D=4, dims=(256,))
    v, xs = hi.draw_activations(w)
    np.testing.assert_array_equal(hi.bf16_bits_to_f32(hi.bf16_bits_rne(v)), v)


def test_dna_activations_take_four_values_per_channel():
    w = hi.WORKLOADS[3].with_(D=8, dims=(4096,))
    v, xs = hi.draw_activations(w)
    for a in [v] + xs:
        for d in range(8):
            assert len(np.unique(a[0, d])) <= 4
    # the three streams come from different embedding columns
    assert not np.array_equal(v, xs[0])


def test_film_draws_are_seeded_and_shaped():
    w = hi.WORKLOADS[7]
    p1, p2 = hi.draw_film_params(w), hi.draw_film_params(w)
    assert len(p1) == 2
    for k in p1[0]:
        np.testing.assert_array_equal(p1[0][k], p2[0][k])
        assert p1[0][k].dtype == np.float32
    assert p1[0]["A1"].shape == (64, 3) and p1[0]["G2"].shape == (64, 128) and p1[0]["A3"].shape == (128, 64)
    assert sorted(set(p1[0]["omega0"].tolist())) == list(hi.FILM_OMEGA0_BLOCKS)
    assert np.all(p1[1]["sigma"] >= 0.2) and np.all(p1[1]["sigma"] < 0.8)
    assert not np.array_equal(p1[0]["A2"], p1[1]["A2"])
    r = hi.draw_registers(w)
    assert r.shape == (2, 8, 128) and r.dtype == np.float32
    np.testing.assert_array_equal(r, hi.draw_registers(w))


def test_projection_draws():
    w = hi.WORKLOADS[8].with_(B=2, dims=(256,))
    x, W, b = hi.draw_projection(w)
    assert x.shape == (2, 256, 768) and W.shape == (3 * 768, 768) and b.shape == (3 * 768,)
    np.testing.assert_array_equal(hi.bf16_bits_to_f32(hi.bf16_bits_rne(x)), x)
    np.testing.assert_array_equal(hi.bf16_bits_to_f32(hi.bf16_bits_rne(W)), W)
    x2, W2, _ = hi.draw_projection(w)
    np.testing.assert_array_equal(x, x2)
    assert np.max(np.abs(W)) <= np.sqrt(6.0 / (4 * 768)) and not np.any(b)
