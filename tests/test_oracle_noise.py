"""Pins the oracle's noise levels and corruption to what the pages fix.

LLaDA-8B-MDLM-LoRA card, Training table, "Objective" row: one t ~ U(0,1) for
each sequence, and every token is masked with probability
p = (1 - 1e-3) t + 1e-3.  diffusiongemma card, "Finetuning notes": uniformly
drawn vocabulary ids, each example with its own rate t ~ U(eps, 1), and no
mask token.

These tests check distributions and special cases, not the formulas' text:
  * t is uniform on [0, 1) (Kolmogorov-Smirnov);
  * p covers exactly [eps, 1), and eps = 1 corrupts every token;
  * per-document corrupted counts follow Binomial(L, p): standardised
    residuals have mean 0 and variance 1, and the corrupted fraction
    regresses on p with slope 1 and intercept 0;
  * uniform-noise replacement ids are uniform over [0, rand_vocab) (chi^2);
  * absorbing noise writes the mask id exactly where a token is corrupted.
"""

import numpy as np
import pytest
from scipy import stats

from oracle import corrupt, noise_levels, NOISE_ABSORB, NOISE_UNIFORM


def test_t_is_uniform_on_unit_interval():
    t, p, thr = noise_levels(seed=11, eps=1e-3, n_docs=20000)
    assert t.min() >= 0.0 and t.max() < 1.0
    res = stats.kstest(t, "uniform")
    assert res.pvalue > 1e-3
    # every t lies on the 24-bit grid
    assert np.all(t * 2.0**24 == np.floor(t * 2.0**24))


@pytest.mark.parametrize("eps", [1e-3, 0.25, 0.9])
def test_p_spans_eps_to_one(eps):
    t, p, thr = noise_levels(seed=3, eps=eps, n_docs=50000)
    assert p.min() >= eps and p.max() < 1.0
    # p is uniform on [eps, 1): its quantiles follow the affine map of U(0,1)
    res = stats.kstest((p - eps) / (1.0 - eps), "uniform")
    assert res.pvalue > 1e-3
    # thresholds count the 24-bit grid points below p
    assert np.all(thr >= 1) and np.all(thr <= 2**24)
    assert np.all((thr - 1) < p * 2.0**24) and np.all(thr >= p * 2.0**24)


def test_eps_one_corrupts_every_token():
    lengths = [5, 0, 17, 33]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    x0 = np.arange(cu[-1], dtype=np.int32) % 50
    xt, corrupted, p_doc, counts = corrupt(x0, cu, seed=5, eps=1.0,
                                           noise=NOISE_ABSORB, mask_id=99,
                                           rand_vocab=100)
    assert np.all(p_doc == 1.0)
    assert corrupted.all() and np.all(xt == 99)
    assert list(counts) == lengths


def test_counts_follow_binomial_in_p():
    n_docs, L = 6000, 64
    cu = (np.arange(n_docs + 1) * L).astype(np.int32)
    x0 = np.zeros(n_docs * L, dtype=np.int32)
    _, corrupted, p, counts = corrupt(x0, cu, seed=1234, eps=1e-3,
                                      noise=NOISE_ABSORB, mask_id=1,
                                      rand_vocab=2)
    counts = counts.astype(np.float64)
    var = L * p * (1 - p)
    z = (counts - L * p) / np.sqrt(var)
    assert abs(z.mean()) < 4.0 / np.sqrt(n_docs)
    assert abs(z.var() - 1.0) < 0.1
    fit = stats.linregress(p, counts / L)
    assert abs(fit.slope - 1.0) < 5 * fit.stderr
    assert abs(fit.intercept) < 5 * fit.intercept_stderr


def test_uniform_replacement_ids_are_uniform():
    V = 16
    n = 64000
    cu = np.array([0, n], dtype=np.int32)
    x0 = np.zeros(n, dtype=np.int32)
    xt, corrupted, p, counts = corrupt(x0, cu, seed=77, eps=1.0,
                                       noise=NOISE_UNIFORM, mask_id=-1,
                                       rand_vocab=V)
    assert corrupted.all()
    hist = np.bincount(xt, minlength=V)
    assert hist.shape[0] == V
    res = stats.chisquare(hist)
    assert res.pvalue > 1e-3
    # a replacement equal to the clean token still counts as corrupted
    assert np.any(xt == x0) and counts[0] == n


def test_uniform_noise_keeps_clean_tokens_where_not_selected():
    rng = np.random.default_rng(0)
    lengths = rng.integers(1, 200, size=40)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    x0 = rng.integers(0, 1000, size=cu[-1]).astype(np.int32)
    xt, corrupted, p, counts = corrupt(x0, cu, seed=9, eps=1e-3,
                                       noise=NOISE_UNIFORM, mask_id=-1,
                                       rand_vocab=1000)
    keep = corrupted == 0
    assert np.array_equal(xt[keep], x0[keep])
    assert xt.min() >= 0 and xt.max() < 1000
    for b in range(len(lengths)):
        assert counts[b] == corrupted[cu[b]:cu[b + 1]].sum()


def test_absorbing_writes_mask_exactly_at_corrupted():
    rng = np.random.default_rng(1)
    lengths = rng.integers(0, 300, size=30)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    x0 = rng.integers(0, 500, size=cu[-1]).astype(np.int32)
    xt, corrupted, p, counts = corrupt(x0, cu, seed=2, eps=1e-3,
                                       noise=NOISE_ABSORB, mask_id=500,
                                       rand_vocab=501)
    assert np.array_equal(xt == 500, corrupted.astype(bool))
    assert np.array_equal(xt[corrupted == 0], x0[corrupted == 0])
    assert counts.sum() == corrupted.sum()


def test_decision_depends_only_on_seed_index_and_threshold():
    """Each document draws its own t; a token's decision depends on its global
    index and its document's threshold only (documents stay isolated)."""
    x0 = np.zeros(300, dtype=np.int32)
    cu_a = np.array([0, 100, 300], dtype=np.int32)
    cu_b = np.array([0, 100, 150, 300], dtype=np.int32)
    _, ca, pa, _ = corrupt(x0, cu_a, seed=4, eps=1e-3, noise=NOISE_ABSORB,
                           mask_id=1, rand_vocab=2)
    _, cb, pb, _ = corrupt(x0, cu_b, seed=4, eps=1e-3, noise=NOISE_ABSORB,
                           mask_id=1, rand_vocab=2)
    assert pa[0] == pb[0] and pa[1] == pb[1]
    assert np.array_equal(ca[:150], cb[:150])
    # a different seed gives a different draw
    _, cc, pc, _ = corrupt(x0, cu_a, seed=5, eps=1e-3, noise=NOISE_ABSORB,
                           mask_id=1, rand_vocab=2)
    assert not np.array_equal(pa, pc)
