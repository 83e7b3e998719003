"""Checks of the seeded input generators (no method arithmetic here)."""
import numpy as np
import pytest
import torch

import synth


def test_seeds_reproducible_and_chunks_independent():
    cfg = synth.test_config("q_proj_7b")
    np.testing.assert_array_equal(synth.weights(cfg), synth.weights(cfg))
    full = synth.x_all(cfg, threads=3)
    for c in reversed(range(cfg.n_chunks)):
        t0, t1 = cfg.chunk_range(c)
        np.testing.assert_array_equal(synth.x_chunk(cfg, c), full[t0:t1])
    assert full.shape == (cfg.n_tokens, cfg.d_in)


def test_bf16_cast_is_round_to_nearest_even():
    r = np.random.default_rng(5)
    x = np.concatenate([r.standard_normal(10000).astype(np.float32) * 10,
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8,
                                  3.0e38, 1e-40, 0.0, -0.0], dtype=np.float32)])
    ours = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(synth.bf16_bits_to_f32(ours),
                                  torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_outlier_counts_and_channel_factors():
    want = {"tiny": 2, "q_proj_7b": 20, "down_proj_7b": 110, "up_proj_70b": 25, "moe_w1_8x7b": 20}
    for name, k in want.items():
        cfg = synth.CONFIGS[name]
        oc = synth.outlier_channels(cfg)
        assert len(oc) == k and len(set(oc.tolist())) == k
        f = synth.channel_factor(cfg)
        if cfg.chan_std_loguniform is None:
            assert np.all(f[oc] == np.float32(cfg.outlier_mult))
            assert np.sum(f != 1.0) == k
    f3 = synth.channel_factor(synth.CONFIGS["down_proj_7b"])
    base = np.delete(f3, synth.outlier_channels(synth.CONFIGS["down_proj_7b"]))
    assert 0.1 <= base.min() and base.max() <= 10.0


def test_zipf_top2_marginals():
    cfg = synth.CONFIGS["moe_w1_8x7b"]
    p = synth.expert_popularity(cfg)
    np.testing.assert_allclose(p, [.429, .187, .115, .081, .062, .050, .042, .035], atol=6e-4)
    counts = np.array([len(ix) for ix in synth.routing(cfg)])
    assert counts.sum() == 2 * cfg.n_tokens
    # P(e among the first two draws without replacement) = p_e + sum_j p_j p_e / (1 - p_j)
    marg = np.array([p[e] + sum(p[j] * p[e] / (1 - p[j]) for j in range(8) if j != e)
                     for e in range(8)])
    np.testing.assert_allclose(marg, [.706, .404, .260, .187, .145, .117, .098, .083], atol=2e-3)
    n = cfg.n_tokens
    sigma = np.sqrt(n * marg * (1 - marg))
    assert np.all(np.abs(counts - n * marg) < 5 * sigma)


def test_small_moe_variant_tops_up_cold_experts():
    cfg = synth.test_config("moe_w1_8x7b")
    idx = synth.routing(cfg)
    assert min(len(i) for i in idx) == 128
    assert sum(len(i) > 128 for i in idx) >= 3
    for ix in idx:
        assert np.all(np.diff(ix) > 0) and ix.min() >= 0 and ix.max() < cfg.n_tokens
