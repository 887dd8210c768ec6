"""Input generator: RoPE properties, bf16 rounding, determinism, config shapes."""
import numpy as np
import pytest

from learned_kv_cache_02_amd import configs, synth


def test_rope_preserves_norm_and_is_relative():
    rng = np.random.default_rng(0)
    d = 128
    x = rng.standard_normal((5, d))
    y = rng.standard_normal((5, d))
    pos = np.array([0, 7, 1000, 61440, 1048575])
    rx = synth.rope(x, pos, 1e6)
    np.testing.assert_allclose(np.linalg.norm(rx, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
    np.testing.assert_allclose(synth.rope(x, np.zeros(5), 1e4), x, atol=0)
    # <RoPE(x, m), RoPE(y, n)> depends only on m - n
    for shift in (0, 3, 123456):
        a = np.sum(synth.rope(x[:1], [10 + shift], 5e5) * synth.rope(y[:1], [4 + shift], 5e5))
        b = np.sum(synth.rope(x[:1], [6], 5e5) * synth.rope(y[:1], [0], 5e5))
        assert abs(a - b) < 1e-9


def test_bf16_round_to_nearest_even():
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1.0 + 2 ** -9, 65504.0],
                    dtype=np.float64)
    bits = synth.to_bf16_bits(vals)
    # 1+2^-8 is a tie -> even (0x3F80); 1+3*2^-8 is a tie -> even (0x3F82)
    assert list(bits) == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x3F80, 0x4780]
    np.testing.assert_array_equal(synth.bf16_bits_to_f32(bits)[:4], [1.0, 1.0, 1.015625, -2.5])


def test_generation_is_deterministic_and_chunk_independent():
    a = synth.normal((1, 2, 3), 40000, 8)
    b = synth.normal((1, 2, 3), 40000, 8)
    np.testing.assert_array_equal(a, b)
    # the first chunk does not depend on how many rows follow it
    c = synth.normal((1, 2, 3), 100, 8)
    np.testing.assert_array_equal(a[:100], c)
    assert abs(a.mean()) < 0.01 and abs(a.std() - 1) < 0.01


def test_config_shapes_and_capacity():
    c2 = configs.C2
    assert c2.G == 4 and c2.R == 1 and c2.local_len(0) == 513 and c2.q_offset(0) == 512
    assert c2.mlps[0].params(128) == 1567105
    assert abs(c2.rho(c2.mlps[0].params(128)) - 0.09963) < 1e-4
    c3 = configs.C3
    assert c3.R == 16384 and c3.R * c3.G == 114688 and c3.T_cap == 1024
    assert c3.mlps[1].params(128) == 2639489
    c4 = configs.C4
    assert c4.mlps[0].params(128) == 3364737 and c4.local_len(127) == 384
    c5 = configs.C5
    assert 2 * c5.kv_pairs * c5.d == 2684416
    assert abs(c5.rho(2 * c5.kv_pairs * c5.d) - 0.01) < 1e-5


def test_small_config_tensors():
    c1 = configs.C1
    K, V = synth.doc_kv(c1)
    assert K.shape == (1, 512, 64) and K.dtype == np.float32
    Kl, Vl = synth.local_kv(c1)
    assert Kl.shape == (1, 1, 16, 64)
    q = synth.queries(c1)
    assert q.shape == (16, 2, 64)
    P = synth.mlp_params(c1)
    assert P["W1"].shape == (1, 256, 64) and P["ws2"].shape == (1, 256) and P["bs2"].shape == (1,)
    np.testing.assert_allclose(P["W1"].std(), 64 ** -0.5, rtol=0.05)
    np.testing.assert_allclose(P["W2t"].std(), 256 ** -0.5, rtol=0.05)
    # document keys are RoPE'd at 0..n-1: key 0 is unrotated
    raw = synth.normal((c1.seed, 0, synth.T_DOC_K, 0), 512, 64)
    np.testing.assert_array_equal(K[0, 0], raw[0].astype(np.float32))


def test_layer_capacity_allocation_table10():
    """App. C.1 / Table 10: groups of 9, 6, 12 and 1 layers with multipliers
    (1, 2, 5, 2); the layer-weighted mean multiplier is 83/28, and the normalised
    factors keep the total capacity of the uniform allocation."""
    from learned_kv_cache_02_amd import configs
    f = configs.layer_capacity_factors()
    assert len(f) == 28
    assert abs(f[0] - 28 / 83) < 1e-15 and abs(f[20] - 5 * 28 / 83) < 1e-15 and abs(f[27] - 2 * 28 / 83) < 1e-15
    assert abs(sum(f) - 28) < 1e-12
    assert [f[i] / f[0] for i in (0, 8, 9, 14, 15, 26, 27)] == pytest.approx([1, 1, 2, 2, 5, 5, 2])
    g = configs.layer_capacity_factors(mult=configs.TABLE11_MULT)
    assert abs(sum(g) - 28) < 1e-12 and abs(g[27] / g[0] - 12) < 1e-12


def test_widths_for_budget_recover_the_workload_module():
    """The 4B layer's 4608/2944 module: its parameter count and score share give
    back its widths."""
    from learned_kv_cache_02_amd import configs
    m = configs.C2.mlps[0]
    P = m.params(128)
    score = 2944 * (128 + 2) + 1
    assert configs.mlp_widths_for_budget(P, 128, score / P) == (4608, 2944)
    shapes = configs.allocated_mlps(configs.C3, 0.10, score / P)
    tot = sum(s.params(128) for s in shapes)
    assert abs(tot / (28 * 0.10 * 2 * configs.C3.n * 128) - 1) < 0.01      # rounding to multiples of 64
    assert shapes[20].Ht > shapes[10].Ht > shapes[0].Ht
