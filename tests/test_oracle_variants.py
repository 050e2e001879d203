"""Pins the oracle's loss variants (row lists beyond the masked-token rows,
other weightings, the head-weight gradient) to independent facts.

  * the row selection against a vectorised brute force, for every
    combination of corruption mask, eligibility mask and alignment; with a
    mask, no eligibility mask and 1/(p N) weights it is ``compact``;
  * the encoder AR term: every-token shifted rows with mean weights give
    lambda * torch's mean next-token cross-entropy, gradients from autograd;
  * the mean weighting is torch's mean CE over the scored rows;
  * the clipped example-mean weighting against an explicit per-document loop
    over torch's per-row CE (clip active, documents without scored rows);
  * the head-weight gradient against central finite differences and its
    closed form at W = 0.
"""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import (corrupt, compact, compact_rows, head_ce, head_ce_weight_grad,
                    NOISE_ABSORB, ALIGNED, SHIFTED, WEIGHT_INV_P, WEIGHT_MEAN,
                    WEIGHT_EXAMPLE_MEAN_CLIPPED)


def _case(seed, n_docs=6, max_len=30, H=8, V=40, hs=1.0, ws=0.5):
    rng = np.random.default_rng(seed)
    lengths = rng.integers(0, max_len + 1, size=n_docs)
    lengths[0] = max(lengths[0], 3)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    n = int(cu[-1])
    x0 = rng.integers(0, V, size=n).astype(np.int32)
    hidden = rng.standard_normal((n, H)) * hs
    W = rng.standard_normal((V, H)) * ws
    return rng, cu, x0, hidden, W


@pytest.mark.parametrize("align", [ALIGNED, SHIFTED])
@pytest.mark.parametrize("use_mask", [False, True])
@pytest.mark.parametrize("use_elig", [False, True])
def test_row_selection_bruteforce(align, use_mask, use_elig):
    rng, cu, x0, _, _ = _case(1, n_docs=20)
    n = x0.shape[0]
    mask = rng.random(n) < 0.4 if use_mask else None
    elig = rng.random(n) < 0.7 if use_elig else None
    p = rng.uniform(0.05, 1.0, size=cu.shape[0] - 1)
    rows, tgt, w = compact_rows(x0, cu, align, mask, elig, p, WEIGHT_INV_P)
    doc = np.searchsorted(cu[1:], np.arange(n), side="right")
    sel = np.ones(n, dtype=bool)
    if mask is not None:
        sel &= mask
    if elig is not None:
        sel &= elig
    if align == SHIFTED:
        sel &= np.arange(n) != cu[doc]
    g = np.flatnonzero(sel)
    assert np.array_equal(rows, g - (1 if align == SHIFTED else 0))
    assert np.array_equal(tgt, x0[g])
    assert np.array_equal(w, 1.0 / (p[doc[g]] * n))
    if use_mask and not use_elig:
        r2, t2, w2 = compact(mask, x0, cu, p, align)
        assert np.array_equal(rows, r2) and np.array_equal(tgt, t2) and np.array_equal(w, w2)


def _torch_logits(h, W, softcap):
    z = h @ W.T
    return softcap * torch.tanh(z / softcap) if softcap > 0 else z


@pytest.mark.parametrize("softcap", [0.0, 3.0])
def test_encoder_ar_term_is_lambda_times_next_token_ce(softcap):
    _, cu, x0, hidden, W = _case(2)
    lam = 0.37
    rows, tgt, w = compact_rows(x0, cu, SHIFTED, weighting=WEIGHT_MEAN, scale=lam)
    loss, _, d_hidden = head_ce(hidden, W, rows, tgt, w, softcap)
    # independent: per document, positions 0..L-2 predict tokens 1..L-1
    th = torch.tensor(hidden, dtype=torch.float64, requires_grad=True)
    tw = torch.tensor(W, dtype=torch.float64)
    zs, ts = [], []
    for b in range(cu.shape[0] - 1):
        a, e = int(cu[b]), int(cu[b + 1])
        if e - a >= 2:
            zs.append(_torch_logits(th[a:e - 1], tw, softcap))
            ts.append(torch.tensor(x0[a + 1:e], dtype=torch.int64))
    ref = lam * F.cross_entropy(torch.cat(zs), torch.cat(ts))
    ref.backward()
    ref = float(ref.detach())
    assert rows.shape[0] == sum(max(int(cu[b + 1] - cu[b]) - 1, 0) for b in range(cu.shape[0] - 1))
    assert loss == pytest.approx(ref, rel=1e-12)
    assert np.allclose(d_hidden, th.grad.numpy(), rtol=1e-10, atol=1e-13)


def test_mean_weighting_is_mean_ce_over_scored_rows():
    _, cu, x0, hidden, W = _case(3, n_docs=8)
    _, corrupted, p, _ = corrupt(x0, cu, 5, 1e-3, NOISE_ABSORB, 39, 40)
    rows, tgt, w = compact_rows(x0, cu, ALIGNED, corrupted, None, p, WEIGHT_MEAN, 1.0)
    loss, _, _ = head_ce(hidden, W, rows, tgt, w)
    z = torch.tensor(hidden[rows]) @ torch.tensor(W).T
    ref = F.cross_entropy(z, torch.tensor(tgt))
    assert loss == pytest.approx(float(ref), rel=1e-12)


def test_example_mean_clipped_against_a_per_document_loop():
    rng, cu, x0, hidden, W = _case(4, n_docs=6, max_len=25)
    n = x0.shape[0]
    nd = cu.shape[0] - 1
    p = np.array([0.5, 0.95, 0.2, 0.99, 0.7, 0.3])[:nd]   # 0.95 and 0.99 hit the clip
    clip, scale = 10.0, 1.3
    mask = rng.random(n) < 0.5
    mask[cu[2]:cu[3]] = False                             # a document with no scored row
    rows, tgt, w = compact_rows(x0, cu, SHIFTED, mask, None, p,
                                WEIGHT_EXAMPLE_MEAN_CLIPPED, scale, clip)
    loss, _, _ = head_ce(hidden, W, rows, tgt, w)
    per_doc = []
    for b in range(nd):
        gs = [g for g in range(cu[b] + 1, cu[b + 1]) if mask[g]]
        if not gs:
            continue
        z = torch.tensor(hidden[[g - 1 for g in gs]]) @ torch.tensor(W).T
        ce = F.cross_entropy(z, torch.tensor(x0[gs], dtype=torch.int64), reduction="none")
        per_doc.append(min(1.0 / (1.0 - p[b]), clip) * float(ce.mean()))
    ref = scale * sum(per_doc) / len(per_doc)
    assert loss == pytest.approx(ref, rel=1e-12)
    # the weights of a document sum to scale * min(1/(1-p), clip) / B
    doc = np.searchsorted(cu[1:], rows + 1, side="right")
    B = len(per_doc)
    for b in set(doc.tolist()):
        assert w[doc == b].sum() == pytest.approx(scale * min(1 / (1 - p[b]), clip) / B,
                                                  rel=1e-12)


def test_example_mean_without_a_clip_is_the_plain_inverse_one_minus_rate():
    # no clip argument: nothing is capped, each document's weights sum to
    # scale / ((1 - p_b) B), written out here per document
    rng, cu, x0, hidden, W = _case(7, n_docs=4, max_len=20)
    nd = cu.shape[0] - 1
    p = np.array([0.25, 0.5, 0.9, 0.6])[:nd]
    mask = rng.random(x0.shape[0]) < 0.6
    rows, tgt, w = compact_rows(x0, cu, ALIGNED, mask, None, p, WEIGHT_EXAMPLE_MEAN_CLIPPED, 2.0)
    doc = np.searchsorted(cu[1:], rows, side="right")
    B = len(set(doc.tolist()))
    for b in set(doc.tolist()):
        assert w[doc == b].sum() == pytest.approx(2.0 / ((1.0 - p[b]) * B), rel=1e-12)


@pytest.mark.parametrize("softcap", [0.0, 2.0])
def test_head_weight_gradient_finite_differences(softcap):
    rng, cu, x0, hidden, W = _case(5, n_docs=2, max_len=6, H=3, V=7)
    n = x0.shape[0]
    rows = np.arange(n)
    w = rng.uniform(0.1, 1.0, size=n)
    dW = head_ce_weight_grad(hidden, W, rows, x0, w, softcap)
    h = 1e-6
    for v in range(W.shape[0]):
        for k in range(W.shape[1]):
            Wp, Wm = W.copy(), W.copy()
            Wp[v, k] += h
            Wm[v, k] -= h
            lp, _, _ = head_ce(hidden, Wp, rows, x0, w, softcap, want_grad=False)
            lm, _, _ = head_ce(hidden, Wm, rows, x0, w, softcap, want_grad=False)
            assert dW[v, k] == pytest.approx((lp - lm) / (2 * h), rel=1e-5, abs=1e-8)


@pytest.mark.parametrize("softcap", [0.0, 2.0])
def test_head_weight_gradient_selected_rows_equal_the_full_gradient(softcap):
    # the v_rows form (a repeated index, the targets' rows, others) against
    # the full gradient, which finite differences and the closed form pin
    rng, cu, x0, hidden, W = _case(8, n_docs=3, max_len=12, H=6, V=13)
    rows = np.arange(0, x0.shape[0], 2)
    tgt = x0[rows]
    w = rng.uniform(0.1, 1.0, size=rows.shape[0])
    full = head_ce_weight_grad(hidden, W, rows, tgt, w, softcap)
    pick = np.array([int(tgt[0]), 0, 12, int(tgt[0]), 5, int(tgt[-1])])
    part = head_ce_weight_grad(hidden, W, rows, tgt, w, softcap, v_rows=pick)
    assert np.allclose(part, full[pick], rtol=1e-12, atol=1e-15)


def test_head_weight_gradient_closed_form_at_zero_head():
    # W = 0: every logit is 0, softmax is uniform 1/V, so
    # dW_v = sum_j w_j (1/V - [v = tgt_j]) h_j
    rng, cu, x0, hidden, W = _case(6, H=5, V=11)
    n = x0.shape[0]
    rows = np.arange(0, n, 2)
    tgt = x0[rows]
    w = rng.uniform(0.1, 1.0, size=rows.shape[0])
    W0 = np.zeros_like(W)
    dW = head_ce_weight_grad(hidden, W0, rows, tgt, w)
    V = W.shape[0]
    want = np.zeros_like(W)
    for j, r in enumerate(rows):
        for v in range(V):
            want[v] += w[j] * ((1.0 / V) - (1.0 if v == tgt[j] else 0.0)) * hidden[r]
    assert np.allclose(dW, want, rtol=1e-12, atol=1e-14)
