"""The seeded input generator: Dirichlet skew model ("Decoding the Skew" II-D,
III-A) and the fp8 block quantiser.  CPU only."""
import numpy as np
import pytest
import scipy.stats

import synth


def test_dirichlet_moments():
    rng = np.random.default_rng(0)
    for N, a in ((8, 0.5), (128, 1.0), (64, 10.0), (256, 0.05)):
        P = np.stack([synth.dirichlet_shares(rng, a, N) for _ in range(4000)])
        np.testing.assert_allclose(P.sum(axis=1), 1.0, atol=1e-12)
        assert abs(P.mean() - 1.0 / N) < 1e-12
        var = (N - 1) / (N * N * (N * a + 1))
        # sample variance of one coordinate pooled over coordinates
        assert abs(P.var(axis=0).mean() / var - 1.0) < 0.08, (N, a)
        # E[sum p^2] = (a + 1) / (N a + 1)
        s2 = (P * P).sum(axis=1).mean()
        assert abs(s2 / ((a + 1) / (N * a + 1)) - 1.0) < 0.08, (N, a)


def test_eff_exp_range():
    assert synth.eff_exp([5, 5, 5, 5]) == 4.0   # N under uniform routing
    assert synth.eff_exp([0, 9, 0, 0]) == 1.0   # 1 when one expert takes all
    assert synth.eff_exp([3, 6, 9]) == synth.eff_exp([30, 60, 90])  # scale-invariant


def test_gumbel_first_pick_frequencies_are_p(oracle_lib):
    """argmax(log p + Gumbel) ~ Categorical(p): the first pick's frequencies."""
    rng = np.random.default_rng(1)
    p = synth.dirichlet_shares(rng, 1.0, 8)
    B = 40000
    lg = (np.log(p)[None, :] + synth.gumbel(rng, (B, 8))).astype(np.float32)
    ids, _ = oracle_lib.route_topk(lg, 1)
    obs = np.bincount(ids[:, 0], minlength=8)
    chi = scipy.stats.chisquare(obs, p * B)
    assert chi.pvalue > 1e-4


def test_large_alpha_near_uniform_counts(oracle_lib):
    """alpha -> infinity: counts of k-subsets drawn without replacement are close to
    uniform; their eff_exp approaches E / (1 + (E - k)/(T k))."""
    E, k, T = 128, 8, 4096
    rng = np.random.default_rng(2)
    lg, p = synth.routing_logits(synth.SHAPES["qwen3"], T, 1e6, rng)
    assert np.abs(p * E - 1).max() < 0.02
    ids, _ = oracle_lib.route_topk(lg, k)
    cnt = oracle_lib.counts(ids, 0, E)
    assert cnt.sum() == T * k
    chi = scipy.stats.chisquare(cnt, np.full(E, T * k / E))
    assert chi.pvalue > 1e-4
    closed = E / (1 + (E - k) / (T * k))
    assert abs(synth.eff_exp(cnt) / closed - 1) < 0.01


def test_small_alpha_skews():
    rng = np.random.default_rng(3)
    eff = [synth.eff_exp(synth.dirichlet_shares(rng, a, 128)) for a in (0.05, 10.0)]
    assert eff[0] < 20 < 100 < eff[1]


def test_fp8_quantiser_block_scale():
    rng = np.random.default_rng(4)
    w = (rng.standard_normal((256, 384)) * 0.02).astype(np.float32)
    q, s = synth.quantize_fp8_blocks(w)
    assert q.dtype == np.uint8 and s.shape == (2, 3)
    amax = np.abs(w.reshape(2, 128, 3, 128)).max(axis=(1, 3))
    np.testing.assert_allclose(s, amax / 448.0, rtol=1e-7)
    # the largest magnitude of each block encodes as +-448 (code 0x7E / 0xFE)
    blk = q.reshape(2, 128, 3, 128)
    for i in range(2):
        for j in range(3):
            assert ((blk[i, :, j, :] & 0x7F) == 0x7E).any()


def test_layer_seeds_are_deterministic():
    a = synth.make_layer("tiny", 64, None, 0)
    b = synth.make_layer("tiny", 64, None, 0)
    np.testing.assert_array_equal(a.logits, b.logits)
    np.testing.assert_array_equal(a.x, b.x)
    np.testing.assert_array_equal(a.w2, b.w2)
    c = synth.make_layer("tiny", 64, None, 1)
    assert not np.array_equal(a.logits, c.logits)


def test_ddist_alpha_hits_its_target():
    """The searched alpha gives mean effective experts n / X on fresh draws."""
    rng = np.random.default_rng(11)
    for n, x in ((8, 2.0), (128, 4.0), (256, 16.0)):
        a = synth.ddist_alpha(x, n, samples=64, iters=40, seed=1)
        v = np.mean([synth.eff_exp(synth.dirichlet_shares(rng, a, n)) for _ in range(400)])
        assert abs(v / (n / x) - 1) < 0.05, (n, x, a, v)


def test_ddist_alpha_against_the_second_moment():
    """For Dir(a 1_n), E[sum p_i^2] = (a + 1) / (n a + 1); with many experts the
    mean of 1 / sum p^2 is close to its reciprocal, so the alpha found for ddist:X
    is close to the closed-form root of (n a + 1) / (a + 1) = n / X."""
    n, x = 256, 4.0
    t = n / x
    a_closed = (t - 1) / (n - t)
    a = synth.ddist_alpha(x, n, samples=64, iters=40, seed=2)
    assert abs(a / a_closed - 1) < 0.08, (a, a_closed)


def test_ddist_alpha_is_monotone_and_bounded():
    a = [synth.ddist_alpha(x, 64, samples=32, iters=40, seed=3) for x in (1.0, 2.0, 8.0, 32.0)]
    assert a[0] > 1e5  # X = 1: no draw reaches n, the search runs to the top of the range
    assert a[0] > a[1] > a[2] > a[3] > 1e-6
    with pytest.raises(ValueError):
        synth.ddist_alpha(0.5, 64)
