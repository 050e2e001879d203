"""The oracle's pins have teeth: each test plants one plausible mistake in the
oracle (on the CPU, through monkeypatch, for the duration of the test only)
and checks that a pin written for it fails.

Mistakes planted: a Philox multiplier, the token-to-word layout, the noise
level's affine map and its 24-bit scale, the shifted row index, the 1/p
weight, the softcap derivative, the target column, the gradient's sign, a
log-sum-exp that misses a vocabulary chunk, and in the variants the
example-mean divisor, the eligibility position, the mean's denominator and
the weight in the head-weight gradient, and in the corrective mixture the
masked and replaced weights swapped, the replace decision inverted or drawn
from the corruption word, the clean weight taken over the clean tokens, the
noise weight squared, and the clean weight leaking onto the replaced rows.
"""

import math

import numpy as np
import pytest

import oracle
import oracle.mdlm as M
import oracle.philox as P
import test_oracle_loss as TL
import test_oracle_noise as TN
import test_oracle_philox as TP
from test_oracle_philox import rocrand_ref  # noqa: F401  (the fixture)
import test_oracle_variants as TV
import test_oracle_corrective as TC

_MODULES = (M, oracle, TL, TN, TP, TV)


def _patch(monkeypatch, name, fn):
    """Replace `name` wherever the oracle and the pin modules bound it."""
    for mod in _MODULES:
        if hasattr(mod, name):
            monkeypatch.setattr(mod, name, fn)


def _fails(pin, *args, **kw):
    with pytest.raises(AssertionError):
        pin(*args, **kw)


def test_philox_multiplier(monkeypatch, request):
    monkeypatch.setattr(P, "PHILOX_M1", P.PHILOX_M0)
    _fails(TP.test_philox_matches_rocrand_random_counters, request.getfixturevalue("rocrand_ref"))


def test_token_word_layout(monkeypatch, request):
    orig = M.token_words

    def bad(seed, n_tokens, tag, start=0):
        # word (g >> 2) & 3 instead of g & 3
        k0, k1 = M._key(seed)
        g = np.arange(start, start + n_tokens, dtype=np.uint64)
        q = g >> np.uint64(2)
        words = np.stack(P.philox4x32_10(q & 0xFFFFFFFF, q >> 32, 0, tag, k0, k1), axis=1)
        return words[np.arange(n_tokens), ((g >> np.uint64(2)) & np.uint64(3)).astype(np.int64)]
    assert orig is not None
    monkeypatch.setattr(M, "token_words", bad)
    _fails(TP.test_token_words_match_rocrand, request.getfixturevalue("rocrand_ref"), 1)


def test_noise_level_missing_scale(monkeypatch):
    orig = M.noise_levels

    def bad(seed, eps, n_docs):
        t, p, thr = orig(seed, eps, n_docs)
        p = float(eps) + t                       # (1 - eps) dropped
        return t, p, np.ceil(p * float(1 << 24)).astype(np.int64)
    _patch(monkeypatch, "noise_levels", bad)
    _fails(TN.test_p_spans_eps_to_one, 0.1)


def test_noise_level_wrong_grid(monkeypatch):
    orig = M.noise_levels

    def bad(seed, eps, n_docs):
        t, p, thr = orig(seed, eps, n_docs)
        t = np.minimum(t * 2.0, 1.0 - 2.0**-24)  # 23-bit scale
        p = float(eps) + (1.0 - float(eps)) * t
        return t, p, np.ceil(p * float(1 << 24)).astype(np.int64)
    _patch(monkeypatch, "noise_levels", bad)
    _fails(TN.test_t_is_uniform_on_unit_interval)


def test_shifted_row_off_by_one(monkeypatch):
    orig = M.compact

    def bad(corrupted, x0, cu_seqlens, p_doc, align):
        rows, tgt, w = orig(corrupted, x0, cu_seqlens, p_doc, align)
        return (rows + 1 if align == M.SHIFTED else rows), tgt, w
    _patch(monkeypatch, "compact", bad)
    _fails(TL.test_compact_matches_bruteforce, M.SHIFTED)


def test_weight_p_instead_of_inverse(monkeypatch):
    orig = M.compact

    def bad(corrupted, x0, cu_seqlens, p_doc, align):
        rows, tgt, w = orig(corrupted, x0, cu_seqlens, p_doc, align)
        n = np.asarray(x0).shape[0]
        return rows, tgt, 1.0 / (w * n * n)      # p / N instead of 1 / (p N)
    _patch(monkeypatch, "compact", bad)
    _fails(TL.test_compact_matches_bruteforce, M.ALIGNED)


def test_softcap_derivative_dropped(monkeypatch):
    orig = M._capped_logits

    def bad(rows_h, w_chunk, softcap):
        z, d = orig(rows_h, w_chunk, softcap)
        return z, np.ones_like(d)
    monkeypatch.setattr(M, "_capped_logits", bad)
    _fails(TL.test_gradient_matches_finite_differences, M.ALIGNED, 1.5)


def test_target_column_off_by_one(monkeypatch):
    orig = M.head_ce_rows

    def bad(hidden, W, row_idx, tgt, softcap=0.0, chunk=8192):
        V = np.asarray(W).shape[0]
        return orig(hidden, W, row_idx, (np.asarray(tgt) + 1) % V, softcap, chunk)
    _patch(monkeypatch, "head_ce_rows", bad)
    _fails(TL.test_eps_one_equals_torch_cross_entropy, M.ALIGNED, 0.0)


def test_gradient_sign(monkeypatch):
    orig = M.head_ce

    def bad(*a, **kw):
        loss, ce, dh = orig(*a, **kw)
        return loss, ce, (None if dh is None else -dh)
    _patch(monkeypatch, "head_ce", bad)
    _fails(TL.test_gradient_closed_form_at_zero_hidden, 0.0)


def test_log_sum_exp_missing_a_chunk(monkeypatch):
    orig_lse = M.logsumexp
    calls = {"n": 0}

    def bad(x, axis=None):
        # the per-chunk log-sum-exps are combined without the last chunk
        if isinstance(x, np.ndarray) and x.ndim == 2 and axis == 1 and x.shape[1] > 1 \
                and calls.get("combine"):
            return orig_lse(x[:, :-1], axis=1)
        return orig_lse(x, axis=axis)
    orig_rows = M.head_ce_rows

    def rows_wrapper(*a, **kw):
        calls["combine"] = True
        try:
            return orig_rows(*a, **kw)
        finally:
            calls["combine"] = False
    monkeypatch.setattr(M, "logsumexp", bad)
    _patch(monkeypatch, "head_ce_rows", rows_wrapper)
    _fails(TL.test_ce_is_log_v_for_equal_logits, 0.0)


def test_example_mean_divides_by_document_length(monkeypatch):
    orig = M.compact_rows

    def bad(x0, cu_seqlens, align, corrupted=None, eligible=None, p_doc=None,
            weighting=M.WEIGHT_INV_P, scale=1.0, clip=None):
        rows, tgt, w = orig(x0, cu_seqlens, align, corrupted, eligible, p_doc, weighting, scale,
                            clip)
        if weighting != M.WEIGHT_EXAMPLE_MEAN_CLIPPED or rows.size == 0:
            return rows, tgt, w
        cu = np.asarray(cu_seqlens, dtype=np.int64)
        g = rows + (1 if align == M.SHIFTED else 0)
        doc = np.searchsorted(cu[1:], g, side="right")
        nb = np.bincount(doc, minlength=cu.shape[0] - 1)
        length = np.diff(cu)
        return rows, tgt, w * nb[doc] / length[doc]
    _patch(monkeypatch, "compact_rows", bad)
    _fails(TV.test_example_mean_clipped_against_a_per_document_loop)


def test_eligibility_on_the_row_token(monkeypatch):
    orig = M.compact_rows

    def bad(x0, cu_seqlens, align, corrupted=None, eligible=None, p_doc=None,
            weighting=M.WEIGHT_INV_P, scale=1.0, clip=None):
        if eligible is not None and align == M.SHIFTED:
            eligible = np.roll(np.asarray(eligible), 1)   # tests g - 1 instead of g
        return orig(x0, cu_seqlens, align, corrupted, eligible, p_doc, weighting, scale, clip)
    _patch(monkeypatch, "compact_rows", bad)
    _fails(TV.test_row_selection_bruteforce, M.SHIFTED, True, True)


def test_mean_weight_over_all_tokens(monkeypatch):
    orig = M.compact_rows

    def bad(x0, cu_seqlens, align, corrupted=None, eligible=None, p_doc=None,
            weighting=M.WEIGHT_INV_P, scale=1.0, clip=None):
        rows, tgt, w = orig(x0, cu_seqlens, align, corrupted, eligible, p_doc, weighting, scale,
                            clip)
        if weighting == M.WEIGHT_MEAN:
            w = np.full(rows.shape[0], scale / float(np.asarray(x0).shape[0]))
        return rows, tgt, w
    _patch(monkeypatch, "compact_rows", bad)
    _fails(TV.test_mean_weighting_is_mean_ce_over_scored_rows)


def test_head_weight_gradient_without_row_weights(monkeypatch):
    orig = M.head_ce_weight_grad

    def bad(hidden, W, row_idx, tgt, w, softcap=0.0, chunk=8192):
        return orig(hidden, W, row_idx, tgt, np.ones_like(np.asarray(w, dtype=np.float64)),
                    softcap, chunk)
    _patch(monkeypatch, "head_ce_weight_grad", bad)
    _fails(TV.test_head_weight_gradient_finite_differences, 0.0)


# ---- corrective mixture ---------------------------------------------------


def _patch_c(monkeypatch, name, fn):
    for mod in (M, oracle, TC):
        if hasattr(mod, name):
            monkeypatch.setattr(mod, name, fn)


def test_corrective_weights_swapped(monkeypatch):
    orig = M.compact_corrective

    def bad(codes, x0, cu_seqlens, p_doc, align, a, c):
        codes = np.asarray(codes)
        swapped = np.where(codes == M.CODE_MASKED, M.CODE_REPLACED,
                           np.where(codes == M.CODE_REPLACED, M.CODE_MASKED, codes))
        return orig(swapped.astype(np.uint8), x0, cu_seqlens, p_doc, align, a, c)
    _patch_c(monkeypatch, "compact_corrective", bad)
    _fails(TC.test_row_list_brute_force, M.ALIGNED, 0.5, 0.0)


def test_mixture_decision_inverted(monkeypatch):
    orig = M.corrupt_mixture

    def bad(x0, cu_seqlens, seed, eps, mixture_prob, mask_id, rand_vocab):
        return orig(x0, cu_seqlens, seed, eps, 1.0 - mixture_prob, mask_id, rand_vocab)
    _patch_c(monkeypatch, "corrupt_mixture", bad)
    _fails(TC.test_mixture_zero_is_absorbing_noise)


def test_mixture_decision_from_the_corruption_word(monkeypatch):
    monkeypatch.setattr(M, "TAG_MIX", M.TAG_BERNOULLI)
    _fails(TC.test_mixture_frequency_and_independence, 0.1)


def test_clean_weight_over_clean_tokens(monkeypatch):
    orig = M.compact_corrective

    def bad(codes, x0, cu_seqlens, p_doc, align, a, c):
        rows, tgt, w = orig(codes, x0, cu_seqlens, p_doc, align, a, c)
        codes = np.asarray(codes)
        g = rows + 1 if align == M.SHIFTED else rows
        clean = codes[g] == M.CODE_CLEAN
        n, n_clean = codes.shape[0], max(int((codes == M.CODE_CLEAN).sum()), 1)
        return rows, tgt, np.where(clean, w * n / n_clean, w)
    _patch_c(monkeypatch, "compact_corrective", bad)
    _fails(TC.test_row_list_brute_force, M.ALIGNED, 2.0, 0.25)


def test_replaced_weight_squared(monkeypatch):
    # noise_token_wt applied as its square: equal at the pinned ends 0 and 1,
    # wrong in between; the interpolation pin (which does not restate the
    # weight formula) catches it
    orig = M.compact_corrective

    def bad(codes, x0, cu_seqlens, p_doc, align, a, c):
        return orig(codes, x0, cu_seqlens, p_doc, align, a * a, c)
    _patch_c(monkeypatch, "compact_corrective", bad)
    _fails(TC.test_weights_interpolate_between_their_pinned_ends, M.ALIGNED)


def test_clean_weight_on_replaced_rows_too(monkeypatch):
    # clean_token_wt added to the replaced rows as well: the clean end (c = 1)
    # moves with it, but the line through the ends does not hold
    orig = M.compact_corrective

    def bad(codes, x0, cu_seqlens, p_doc, align, a, c):
        rows, tgt, w = orig(codes, x0, cu_seqlens, p_doc, align, a, c)
        codes = np.asarray(codes)
        g = rows + 1 if align == M.SHIFTED else rows
        rep = codes[g] == M.CODE_REPLACED
        return rows, tgt, np.where(rep, w + c * c / codes.shape[0], w)
    _patch_c(monkeypatch, "compact_corrective", bad)
    _fails(TC.test_weights_interpolate_between_their_pinned_ends, M.SHIFTED)
