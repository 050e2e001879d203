"""Pins of the oracle's corrective mixture (corrupt_mixture,
compact_corrective) against what holds independently of the reading taken
for its options: the reductions to absorbing and uniform noise and to the
MDLM row list, the mixture's frequency and its independence from the
corruption decision, a vectorised brute force of the row list, the
clean-token weighting against torch's cross-entropy, and the whole loss at
any weight as the straight line through its pinned ends."""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import (ALIGNED, SHIFTED, NOISE_ABSORB, NOISE_UNIFORM, CODE_CLEAN, CODE_MASKED,
                    CODE_REPLACED, compact, compact_corrective, corrupt, corrupt_mixture,
                    head_ce)


def _stream(seed, n_docs=40, max_len=300, V=5000):
    rng = np.random.default_rng(seed)
    lengths = rng.integers(1, max_len + 1, size=n_docs)
    lengths[rng.random(n_docs) < 0.2] = 0
    cu = np.zeros(n_docs + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    x0 = rng.integers(0, V - 1, size=int(cu[-1])).astype(np.int32)
    return x0, cu, V


def test_mixture_zero_is_absorbing_noise():
    x0, cu, V = _stream(1)
    xt, codes, p, counts = corrupt_mixture(x0, cu, 77, 0.2, 0.0, V - 1, V)
    xa, ca, pa, na = corrupt(x0, cu, 77, 0.2, NOISE_ABSORB, V - 1, V)
    assert np.array_equal(xt, xa) and np.array_equal(codes, ca)
    assert np.array_equal(p.view(np.uint64), pa.view(np.uint64))
    assert np.array_equal(counts, na)


def test_mixture_one_is_uniform_noise():
    x0, cu, V = _stream(2)
    xt, codes, p, counts = corrupt_mixture(x0, cu, 78, 0.2, 1.0, V - 1, V)
    xu, cu_, pu, nu = corrupt(x0, cu, 78, 0.2, NOISE_UNIFORM, V - 1, V)
    assert np.array_equal(xt, xu)
    assert np.array_equal(codes, cu_.astype(np.uint8) * CODE_REPLACED)
    assert np.array_equal(counts, nu)


@pytest.mark.parametrize("m", [0.1, 0.5, 0.9])
def test_mixture_frequency_and_independence(m):
    # one long document per noise level: low and high p
    n = 1 << 16
    x0 = np.zeros(2 * n, dtype=np.int32)
    cu = np.array([0, n, 2 * n], dtype=np.int32)
    xt, codes, p, counts = corrupt_mixture(x0, cu, 99, 0.05, m, 7, 1000)
    for b in range(2):
        c = codes[cu[b]:cu[b + 1]]
        k = int((c != CODE_CLEAN).sum())
        r = int((c == CODE_REPLACED).sum())
        sd = np.sqrt(k * m * (1 - m))
        assert abs(r - k * m) < 4 * sd + 1, (b, k, r)
    # the masked / replaced choice does not depend on the noise level: tokens
    # corrupted under two rates get the same kind of corruption
    _, codes2, _, _ = corrupt_mixture(x0, cu, 99, 0.6, m, 7, 1000)
    both = (codes != CODE_CLEAN) & (codes2 != CODE_CLEAN)
    assert both.sum() > 1000 and np.array_equal(codes[both], codes2[both])
    assert np.all(xt[codes == CODE_MASKED] == 7)


@pytest.mark.parametrize("align", [ALIGNED, SHIFTED])
def test_zero_weights_give_the_mdlm_row_list(align):
    x0, cu, V = _stream(3)
    _, codes, p, _ = corrupt_mixture(x0, cu, 5, 0.3, 0.0, V - 1, V)
    got = compact_corrective(codes, x0, cu, p, align, 0.0, 0.0)
    want = compact(codes, x0, cu, p, align)
    for a, b in zip(got, want):
        assert np.array_equal(a, b)
    # with replaced tokens and unit noise weight: the MDLM list of all
    # corrupted tokens, as uniform noise would score them
    _, codes, p, _ = corrupt_mixture(x0, cu, 5, 0.3, 0.5, V - 1, V)
    got = compact_corrective(codes, x0, cu, p, align, 1.0, 0.0)
    want = compact(codes != 0, x0, cu, p, align)
    for a, b in zip(got, want):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("align", [ALIGNED, SHIFTED])
@pytest.mark.parametrize("a,c", [(0.5, 0.0), (0.0, 0.3), (2.0, 0.25)])
def test_row_list_brute_force(align, a, c):
    x0, cu, V = _stream(4)
    _, codes, p, _ = corrupt_mixture(x0, cu, 6, 0.4, 0.3, V - 1, V)
    rows, tgt, w = compact_corrective(codes, x0, cu, p, align, a, c)
    n = x0.shape[0]
    doc = np.searchsorted(cu, np.arange(n), side="right") - 1
    keep = (codes != CODE_CLEAN) | (c != 0.0)
    if align == SHIFTED:
        keep &= np.arange(n) != cu[doc]
    g = np.flatnonzero(keep)
    k = codes[g]
    want_w = np.where(k == CODE_MASKED, 1.0 / (p[doc[g]] * n),
                      np.where(k == CODE_REPLACED, a / (p[doc[g]] * n), c / n))
    assert np.array_equal(rows, g - 1 if align == SHIFTED else g)
    assert np.array_equal(tgt, x0[g])
    assert np.allclose(w, want_w, rtol=1e-15, atol=0)


def test_clean_weight_is_mean_ce_over_all_tokens():
    # nothing corrupted: the loss is clean_token_wt times the mean CE over
    # every token (aligned), which torch computes independently
    rng = np.random.default_rng(8)
    n, H, V = 300, 32, 50
    h = rng.standard_normal((n, H))
    W = rng.standard_normal((V, H)) * 0.3
    x0 = rng.integers(0, V, size=n).astype(np.int32)
    cu = np.array([0, 120, 300], dtype=np.int32)
    codes = np.zeros(n, dtype=np.uint8)
    p = np.array([0.5, 0.25])
    rows, tgt, w = compact_corrective(codes, x0, cu, p, ALIGNED, 1.0, 0.7)
    loss, _, _ = head_ce(h, W, rows, tgt, w)
    z = torch.from_numpy(h) @ torch.from_numpy(W).T
    want = 0.7 * F.cross_entropy(z, torch.from_numpy(x0).long()).item()
    assert abs(loss - want) <= 1e-12 * abs(want)


@pytest.mark.parametrize("align", [ALIGNED, SHIFTED])
def test_weights_interpolate_between_their_pinned_ends(align):
    # The ends are pinned above: noise_token_wt 0 gives the MDLM list of the
    # masked tokens, 1 the MDLM list of every corrupted token (as uniform
    # noise scores it), and clean_token_wt scales the mean CE over the clean
    # tokens.  A weight enters the loss as a factor of its rows' CE, so the
    # whole loss (row list, then head + CE) at any other weight is the
    # straight line through those ends; a weight applied twice, squared, or
    # to the wrong rows leaves it.
    x0, cu, V = _stream(5, n_docs=12, max_len=120, V=300)
    rng = np.random.default_rng(11)
    n, H = x0.shape[0], 16
    h = rng.standard_normal((n, H))
    W = rng.standard_normal((V, H)) * 0.3
    _, codes, p, _ = corrupt_mixture(x0, cu, 9, 0.4, 0.3, V - 1, V)
    assert (codes == CODE_MASKED).sum() > 50 and (codes == CODE_REPLACED).sum() > 20

    def loss(a, c=0.0):
        rows, tgt, w = compact_corrective(codes, x0, cu, p, align, a, c)
        return head_ce(h, W, rows, tgt, w)[0]

    l0, l1, lc = loss(0.0), loss(1.0), loss(0.0, 1.0)
    assert l1 > l0 > 0 and lc > l0
    for a in (0.25, 0.5, 2.0, 3.7):
        want = (1.0 - a) * l0 + a * l1
        assert abs(loss(a) - want) <= 1e-12 * (1.0 + abs(a)) * l1
    for c in (0.3, 0.7):
        want = (1.0 - c) * l0 + c * lc
        assert abs(loss(0.0, c) - want) <= 1e-12 * lc
