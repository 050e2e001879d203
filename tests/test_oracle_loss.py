"""Pins the oracle's compaction and weighted head + CE to independent facts.

  * compaction against a vectorised brute force (np.flatnonzero);
  * CE = log V exactly when every logit is equal (hidden = 0), with and
    without the softcap;
  * the closed-form gradient at hidden = 0: w * (mean_v W_v - W_tgt);
  * central finite differences of the loss (aligned and shifted, softcap on
    and off) -- the guard the LLaDA card's note on a fused-CE gradient issue
    calls for;
  * with eps = 1 every token is scored with weight 1/N, so the loss is
    torch's mean cross-entropy (aligned) or the next-token CE summed over
    non-first tokens / N (shifted); gradients from torch autograd;
  * rows that are not scored do not influence the loss and get zero gradient;
  * the 1/p weighting is unbiased: the mean loss over many seeds equals the
    eps = 1 loss (LLaDA card, Training table, "Objective" row).
"""

import numpy as np
import pytest
import torch

from oracle import (corrupt, compact, head_ce, head_ce_rows, mdlm_loss,
                    NOISE_ABSORB, NOISE_UNIFORM, ALIGNED, SHIFTED)


def _case(seed, n_docs=5, max_len=40, H=16, V=64, hs=1.0, ws=0.5):
    rng = np.random.default_rng(seed)
    lengths = rng.integers(0, max_len + 1, size=n_docs)
    lengths[0] = max(lengths[0], 2)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    n = int(cu[-1])
    x0 = rng.integers(0, V - 1, size=n).astype(np.int32)
    hidden = rng.standard_normal((n, H)) * hs
    W = rng.standard_normal((V, H)) * ws
    return cu, x0, hidden, W


@pytest.mark.parametrize("align", [ALIGNED, SHIFTED])
def test_compact_matches_bruteforce(align):
    cu, x0, _, _ = _case(3, n_docs=30, max_len=50)
    xt, corrupted, p, counts = corrupt(x0, cu, seed=8, eps=1e-3,
                                       noise=NOISE_ABSORB, mask_id=63,
                                       rand_vocab=64)
    rows, tgt, w = compact(corrupted, x0, cu, p, align)
    n = x0.shape[0]
    doc = np.searchsorted(cu[1:], np.arange(n), side="right")
    sel = corrupted.astype(bool)
    if align == SHIFTED:
        sel &= np.arange(n) != cu[doc]
    g = np.flatnonzero(sel)
    exp_rows = g - (1 if align == SHIFTED else 0)
    assert np.array_equal(rows, exp_rows)
    assert np.array_equal(tgt, x0[g])
    assert np.array_equal(w, 1.0 / (p[doc[g]] * n))
    starts_hit = sum(int(corrupted[cu[b]]) for b in range(len(cu) - 1)
                     if cu[b + 1] > cu[b])
    expect_m = counts.sum() - (starts_hit if align == SHIFTED else 0)
    assert rows.shape[0] == expect_m


@pytest.mark.parametrize("softcap", [0.0, 30.0, 2.0])
def test_ce_is_log_v_for_equal_logits(softcap):
    cu, x0, hidden, W = _case(5, V=97)
    hidden[:] = 0.0
    rows = np.arange(x0.shape[0])
    ce, lse = head_ce_rows(hidden, W, rows, x0, softcap=softcap, chunk=10)
    assert np.allclose(ce, np.log(97.0), rtol=0, atol=1e-13)
    w = np.full(rows.shape[0], 0.37)
    loss, _, _ = head_ce(hidden, W, rows, x0, w, softcap=softcap,
                         want_grad=False)
    assert abs(loss - np.log(97.0) * w.sum()) < 1e-11


@pytest.mark.parametrize("softcap", [0.0, 30.0])
def test_gradient_closed_form_at_zero_hidden(softcap):
    cu, x0, hidden, W = _case(6, V=50, H=12)
    hidden[:] = 0.0
    rng = np.random.default_rng(0)
    rows = np.sort(rng.choice(x0.shape[0], size=20, replace=False))
    tgt = x0[rows]
    w = rng.random(20) + 0.1
    _, _, dh = head_ce(hidden, W, rows, tgt, w, softcap=softcap, chunk=7)
    expect = w[:, None] * (W.mean(axis=0)[None, :] - W[tgt])
    assert np.allclose(dh[rows], expect, rtol=1e-12, atol=1e-14)
    other = np.setdiff1d(np.arange(x0.shape[0]), rows)
    assert np.all(dh[other] == 0.0)


@pytest.mark.parametrize("align", [ALIGNED, SHIFTED])
@pytest.mark.parametrize("softcap", [0.0, 1.5])
def test_gradient_matches_finite_differences(align, softcap):
    cu, x0, hidden, W = _case(11 + align, n_docs=3, max_len=12, H=6, V=20,
                              hs=1.0, ws=1.0)
    xt, corrupted, p, _ = corrupt(x0, cu, seed=21, eps=0.3,
                                  noise=NOISE_ABSORB, mask_id=19, rand_vocab=20)
    rows, tgt, w = compact(corrupted, x0, cu, p, align)
    assert rows.size > 0
    loss, _, dh = head_ce(hidden, W, rows, tgt, w, softcap=softcap, chunk=7)
    h = 1e-5
    fd = np.zeros_like(hidden)
    for i in range(hidden.shape[0]):
        for k in range(hidden.shape[1]):
            hp = hidden.copy()
            hp[i, k] += h
            hm = hidden.copy()
            hm[i, k] -= h
            lp, _, _ = head_ce(hp, W, rows, tgt, w, softcap, want_grad=False)
            lm, _, _ = head_ce(hm, W, rows, tgt, w, softcap, want_grad=False)
            fd[i, k] = (lp - lm) / (2 * h)
    err = np.linalg.norm(fd - dh) / np.linalg.norm(dh)
    assert err < 1e-6


def _torch_head_loss(hidden, W, x0, cu, align, softcap):
    h = torch.tensor(hidden, dtype=torch.float64, requires_grad=True)
    Wt = torch.tensor(W, dtype=torch.float64)
    z = h @ Wt.T
    if softcap > 0:
        z = softcap * torch.tanh(z / softcap)
    n = x0.shape[0]
    tg = torch.tensor(x0, dtype=torch.long)
    if align == ALIGNED:
        loss = torch.nn.functional.cross_entropy(z, tg, reduction="mean")
    else:
        terms = []
        for b in range(len(cu) - 1):
            lo, hi = int(cu[b]), int(cu[b + 1])
            if hi - lo >= 2:
                terms.append(torch.nn.functional.cross_entropy(
                    z[lo:hi - 1], tg[lo + 1:hi], reduction="sum"))
        loss = torch.stack(terms).sum() / n
    loss.backward()
    return float(loss.detach()), h.grad.numpy()


@pytest.mark.parametrize("align", [ALIGNED, SHIFTED])
@pytest.mark.parametrize("softcap", [0.0, 30.0])
def test_eps_one_equals_torch_cross_entropy(align, softcap):
    cu, x0, hidden, W = _case(17, n_docs=6, max_len=30, H=24, V=300, hs=1.0,
                              ws=0.3)
    out = mdlm_loss(x0, cu, hidden, W, seed=1, eps=1.0, noise=NOISE_ABSORB,
                    mask_id=299, rand_vocab=300, align=align, softcap=softcap,
                    chunk=64)
    ref_loss, ref_grad = _torch_head_loss(hidden, W, x0, cu, align, softcap)
    assert abs(out["loss"] - ref_loss) <= 1e-12 * abs(ref_loss)
    assert np.allclose(out["d_hidden"], ref_grad, rtol=1e-10, atol=1e-15)


@pytest.mark.parametrize("noise", [NOISE_ABSORB, NOISE_UNIFORM])
def test_unscored_rows_have_no_influence(noise):
    cu, x0, hidden, W = _case(23, n_docs=4, max_len=40)
    base = mdlm_loss(x0, cu, hidden, W, seed=3, eps=1e-3, noise=noise,
                     mask_id=63, rand_vocab=64, align=ALIGNED)
    unscored = np.flatnonzero(base["corrupted"] == 0)
    assert unscored.size > 0
    h2 = hidden.copy()
    h2[unscored] += np.random.default_rng(1).standard_normal(
        (unscored.size, hidden.shape[1])) * 10.0
    pert = mdlm_loss(x0, cu, h2, W, seed=3, eps=1e-3, noise=noise,
                     mask_id=63, rand_vocab=64, align=ALIGNED)
    assert pert["loss"] == base["loss"]
    assert np.all(base["d_hidden"][unscored] == 0.0)


def test_empty_selection_gives_zero_loss_and_gradient():
    cu, x0, hidden, W = _case(2)
    loss, ce, dh = head_ce(hidden, W, np.zeros(0, np.int64),
                           np.zeros(0, np.int64), np.zeros(0))
    assert loss == 0.0 and ce.size == 0 and np.all(dh == 0.0)


def test_inverse_p_weighting_is_unbiased():
    """E over noise draws of sum_{corrupted} CE/p / N equals sum_all CE / N,
    because each token is corrupted with probability p (up to the 2^-24
    grid, a relative bias below 2^-24 / eps)."""
    rng = np.random.default_rng(0)
    n_docs, L, H, V = 32, 32, 8, 40
    cu = (np.arange(n_docs + 1) * L).astype(np.int32)
    x0 = rng.integers(0, V - 1, size=n_docs * L).astype(np.int32)
    hidden = rng.standard_normal((n_docs * L, H))
    W = rng.standard_normal((V, H)) * 0.7
    full = mdlm_loss(x0, cu, hidden, W, seed=0, eps=1.0, noise=NOISE_ABSORB,
                     mask_id=V - 1, rand_vocab=V, align=ALIGNED,
                     want_grad=False)["loss"]
    losses = []
    for s in range(400):
        losses.append(mdlm_loss(x0, cu, hidden, W, seed=1000 + s, eps=0.05,
                                noise=NOISE_ABSORB, mask_id=V - 1,
                                rand_vocab=V, align=ALIGNED,
                                want_grad=False)["loss"])
    losses = np.array(losses)
    se = losses.std(ddof=1) / np.sqrt(losses.size)
    assert abs(losses.mean() - full) < 4 * se
    # the pin has teeth: weighting by 1/(1-p) or leaving the loss unweighted
    # would move the mean by many standard errors
    assert se < 0.02 * full
