"""fp64 reference for corruption, compaction and the fused head + CE loss.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).  Each function follows
the definition on the pages, step by step, in float64.  Where the pages are
silent the reading taken is stated next to the step.

Pages cited:
  [LLaDA]  LLaDA-8B-MDLM-LoRA model card, "Training" table ("Objective",
           "Batch", "Precision" rows) and the paragraph after it.
  [Gemma]  diffusiongemma-26B-A4B-it-ALWAYS-THINK, "Finetuning notes".
  [Axolotl] Native diffusion language-model training: the model table,
           "Start with Nemotron 3B", "Packed training", "Attention backends",
           "Adapters, merging and inference", "Batching".
"""

import numpy as np
from scipy.special import logsumexp

from .philox import philox4x32_10

NOISE_ABSORB = 0
NOISE_UNIFORM = 1
ALIGNED = 0
SHIFTED = 1

# Stream tags carried in the last counter word: one independent stream per
# kind of draw, so no two draws ever share a counter.
TAG_DOC_T = 0      # per-document noise level t
TAG_BERNOULLI = 1  # per-token keep/corrupt decision
TAG_REPLACE = 2    # per-token replacement id under uniform noise
TAG_MIX = 3        # per-token choice between mask and replacement (mixture)

# Codes of the corrective mixture's corruption mask.
CODE_CLEAN = 0
CODE_MASKED = 1
CODE_REPLACED = 2

_TWO24 = float(1 << 24)


def _key(seed):
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    return seed & 0xFFFFFFFF, seed >> 32


def noise_levels(seed, eps, n_docs):
    """Per-document noise level t_b, corruption probability p_b and threshold.

    [LLaDA] Objective row: one t ~ U(0,1) for each sequence, masking
    probability p = (1 - 1e-3) t + 1e-3.  [Gemma] Finetuning notes: each
    example draws its own rate t ~ U(eps, 1) -- the same affine map with general eps, so both noise modes
    share this step.

    Reading taken: t is the top 24 bits of Philox word 0 at counter
    (b, 0, 0, TAG_DOC_T), scaled by 2^-24, so t lies on the grid
    {0, 2^-24, ..., 1 - 2^-24}.  p is evaluated in IEEE fp64 in the order
    (1 - eps), times t, plus eps (each step rounded).  The integer threshold
    thr = ceil(p * 2^24) is exact (power-of-two scaling) and turns the test
    "u < p" for a 24-bit uniform u = u24 * 2^-24 into "u24 < thr".

    Returns (t, p, thr): float64[B], float64[B], int64[B].
    """
    k0, k1 = _key(seed)
    b = np.arange(n_docs, dtype=np.uint64)
    r0, _, _, _ = philox4x32_10(b & 0xFFFFFFFF, b >> 32, 0, TAG_DOC_T, k0, k1)
    u24 = (r0 >> np.uint32(8)).astype(np.float64)
    t = u24 / _TWO24
    one_minus_eps = 1.0 - float(eps)
    p = float(eps) + one_minus_eps * t
    thr = np.ceil(p * _TWO24).astype(np.int64)
    return t, p, thr


def token_words(seed, n_tokens, tag, start=0):
    """Philox word for each token index g in [start, start + n_tokens): word
    (g & 3) of the call at counter (g >> 2 low 32 bits, g >> 2 high 32 bits,
    0, tag)."""
    k0, k1 = _key(seed)
    g = np.arange(start, start + n_tokens, dtype=np.uint64)
    q = g >> np.uint64(2)
    words = np.stack(philox4x32_10(q & 0xFFFFFFFF, q >> 32, 0, tag, k0, k1), axis=1)
    return words[np.arange(n_tokens), (g & np.uint64(3)).astype(np.int64)]


def corrupt(x0, cu_seqlens, seed, eps, noise, mask_id, rand_vocab):
    """Corrupt a packed token stream, one noise level per document.

    [LLaDA] Objective row: absorbing corruption; each token of a sequence is
    masked with probability p (read here as independent Bernoulli(p) draws,
    no forced minimum count).  [Axolotl] "Start with Nemotron 3B": masked
    tokens become the mask id (100 there).  [Gemma] Finetuning notes: under
    uniform noise a corrupted position takes a uniform-random vocabulary id
    (no mask token).  [Axolotl] "Packed training": documents in one packed
    stream stay isolated, so each document draws its own t.

    Readings taken: the decision for token g is (word1(g) >> 8) < thr_b with
    word1 from stream TAG_BERNOULLI; the replacement id is
    floor(word2(g) * rand_vocab / 2^32) with word2 from stream TAG_REPLACE
    (multiply-shift; a draw equal to x0 still counts as corrupted).

    x0: int[N]; cu_seqlens: int[B+1] with cu[0] = 0, cu[B] = N, nondecreasing.
    Returns (xt int32[N], corrupted uint8[N], p_doc float64[B],
    doc_counts int32[B]).
    """
    x0 = np.asarray(x0, dtype=np.int64)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    n = x0.shape[0]
    n_docs = cu.shape[0] - 1
    assert cu[0] == 0 and cu[-1] == n
    _, p, thr = noise_levels(seed, eps, n_docs)
    w1 = token_words(seed, n, TAG_BERNOULLI).astype(np.int64)
    if noise == NOISE_UNIFORM:
        w2 = token_words(seed, n, TAG_REPLACE).astype(np.uint64)
    xt = x0.copy()
    corrupted = np.zeros(n, dtype=np.uint8)
    doc_counts = np.zeros(n_docs, dtype=np.int32)
    for b in range(n_docs):
        lo, hi = cu[b], cu[b + 1]
        sel = (w1[lo:hi] >> 8) < thr[b]
        corrupted[lo:hi] = sel
        doc_counts[b] = int(sel.sum())
        if noise == NOISE_ABSORB:
            xt[lo:hi][sel] = mask_id
        else:
            ids = (w2[lo:hi] * np.uint64(rand_vocab)) >> np.uint64(32)
            xt[lo:hi][sel] = ids[sel].astype(np.int64)
    return xt.astype(np.int32), corrupted, p, doc_counts


def compact(corrupted, x0, cu_seqlens, p_doc, align):
    """List the scored rows in ascending token order, with targets and weights.

    [LLaDA] Objective row: the loss is the CE of each masked token, scaled
    by 1/p.  [Axolotl] model table: Nemotron uses aligned
    logits (the hidden state at position g predicts token g), Dream uses
    shifted logits (position g-1 predicts token g).

    Readings taken:
      * aligned: every corrupted g gives (row g, target x0[g]);
      * shifted: every corrupted g except a document's first token gives
        (row g-1, target x0[g]); a document start has no predecessor inside
        its own document ("Packed training": documents stay isolated);
      * weight w = 1 / (p_b * N) with N the total number of tokens in the
        call (the sum of CE/p over masked tokens, over all tokens),
        evaluated in fp64.

    Returns (row_idx int64[M], tgt int64[M], w float64[M]).  The weight the
    library stores is fp32; ``np.float32(w)`` is its exact expected value.
    """
    corrupted = np.asarray(corrupted).astype(bool)
    x0 = np.asarray(x0, dtype=np.int64)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    p_doc = np.asarray(p_doc, dtype=np.float64)
    n = x0.shape[0]
    rows, tgts, ws = [], [], []
    for b in range(cu.shape[0] - 1):
        for g in range(cu[b], cu[b + 1]):
            if not corrupted[g]:
                continue
            if align == SHIFTED:
                if g == cu[b]:
                    continue
                rows.append(g - 1)
            else:
                rows.append(g)
            tgts.append(x0[g])
            ws.append(1.0 / (p_doc[b] * float(n)))
    return (np.asarray(rows, dtype=np.int64), np.asarray(tgts, dtype=np.int64),
            np.asarray(ws, dtype=np.float64))


def corrupt_mixture(x0, cu_seqlens, seed, eps, mixture_prob, mask_id, rand_vocab):
    """Corruption of the corrective mixture: absorbing corruption in which a
    share of the corrupted tokens takes a uniform-random id instead of the
    mask token.

    [LLaDA] Training table, Objective row: the MDLM arm sets mixture_prob,
    noise_token_wt and clean_token_wt to 0 and is then "absorbing corruption
    only"; the corrective arm (paragraph before the table) differs from it in
    mixture_prob and noise_token_wt.  The pages give no formula.  Reading
    taken (parity unpinned beyond the reductions below): a token is
    corrupted exactly as under absorbing noise (same noise level, same
    Bernoulli words); a corrupted token is replaced by a uniform-random id
    (the uniform-noise draw of ``corrupt``) with probability mixture_prob,
    decided by (word3(g) >> 8) < ceil(mixture_prob * 2^24) with word3 from
    stream TAG_MIX, and masked otherwise.  mixture_prob = 0 is absorbing
    corruption; mixture_prob = 1 replaces every corrupted token with the id
    uniform noise would give it.

    Returns (xt int32[N], codes uint8[N] (CODE_CLEAN / CODE_MASKED /
    CODE_REPLACED), p_doc float64[B], doc_counts int32[B] (corrupted tokens
    of either kind)).
    """
    x0 = np.asarray(x0, dtype=np.int64)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    n = x0.shape[0]
    n_docs = cu.shape[0] - 1
    assert cu[0] == 0 and cu[-1] == n
    assert 0.0 <= mixture_prob <= 1.0
    _, p, thr = noise_levels(seed, eps, n_docs)
    thr_mix = int(np.ceil(float(mixture_prob) * _TWO24))
    w1 = token_words(seed, n, TAG_BERNOULLI).astype(np.int64)
    w2 = token_words(seed, n, TAG_REPLACE).astype(np.uint64)
    w3 = token_words(seed, n, TAG_MIX).astype(np.int64)
    xt = x0.copy()
    codes = np.zeros(n, dtype=np.uint8)
    doc_counts = np.zeros(n_docs, dtype=np.int32)
    for b in range(n_docs):
        for g in range(cu[b], cu[b + 1]):
            if (w1[g] >> 8) >= thr[b]:
                continue
            doc_counts[b] += 1
            if (w3[g] >> 8) < thr_mix:
                codes[g] = CODE_REPLACED
                xt[g] = int((int(w2[g]) * int(rand_vocab)) >> 32)
            else:
                codes[g] = CODE_MASKED
                xt[g] = mask_id
    return xt.astype(np.int32), codes, p, doc_counts


def compact_corrective(codes, x0, cu_seqlens, p_doc, align, noise_token_wt, clean_token_wt):
    """Scored rows of the corrective mixture's loss, in ascending token order.

    [LLaDA] Training table, Objective row: the option names noise_token_wt
    and clean_token_wt; with both 0 the loss is the MDLM one (the CE of
    each masked token, scaled by 1/p).  Reading taken (pinned at the ends,
    zero weights, noise weight 1 and the clean weight alone, by reductions,
    and in between by the loss being linear in each weight): every position
    predicts its
    clean token; a masked token keeps the weight 1 / (p_b N), a replaced
    token gets noise_token_wt / (p_b N) and, when clean_token_wt is not 0,
    every uncorrupted token gets clean_token_wt / N.  Rows are the corrupted
    tokens of either kind (a replaced token is listed even at weight 0) and,
    when clean_token_wt is not 0, every other token; alignment as in
    ``compact``.  Weights in fp64, stored by the library as fp32.

    Returns (row_idx int64[M], tgt int64[M], w float64[M]).
    """
    codes = np.asarray(codes, dtype=np.int64)
    x0 = np.asarray(x0, dtype=np.int64)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    p_doc = np.asarray(p_doc, dtype=np.float64)
    n = x0.shape[0]
    rows, tgts, ws = [], [], []
    for b in range(cu.shape[0] - 1):
        for g in range(cu[b], cu[b + 1]):
            c = codes[g]
            if c == CODE_CLEAN and clean_token_wt == 0.0:
                continue
            if align == SHIFTED:
                if g == cu[b]:
                    continue
                rows.append(g - 1)
            else:
                rows.append(g)
            tgts.append(x0[g])
            if c == CODE_MASKED:
                ws.append(1.0 / (p_doc[b] * float(n)))
            elif c == CODE_REPLACED:
                ws.append(float(noise_token_wt) / (p_doc[b] * float(n)))
            else:
                ws.append(float(clean_token_wt) / float(n))
    return (np.asarray(rows, dtype=np.int64), np.asarray(tgts, dtype=np.int64),
            np.asarray(ws, dtype=np.float64))


WEIGHT_INV_P = 0           # 1 / (p_b N), the LLaDA objective
WEIGHT_MEAN = 1            # 1 / M: unweighted mean over the scored rows
WEIGHT_EXAMPLE_MEAN_CLIPPED = 2  # min(1 / (1 - p_b), clip), example mean


def compact_rows(x0, cu_seqlens, align, corrupted=None, eligible=None, p_doc=None,
                 weighting=WEIGHT_INV_P, scale=1.0, clip=float("inf")):
    """Scored rows, targets and weights for the loss variants.

    A token g of document b is scored when it is corrupted (every token when
    ``corrupted`` is None), eligible for the loss (every token when
    ``eligible`` is None) and, with shifted logits, not the document's first
    token.  It gives (row g or g-1, target x0[g]) as in ``compact``.

    Weights (fp64, rounded once to fp32 by the library):
      * WEIGHT_INV_P: scale / (p_b N), N the call's token count ([LLaDA]
        Objective row, as in ``compact``).
      * WEIGHT_MEAN: scale / M, M the number of scored rows.  With
        corrupted=None, shifted logits and scale = lambda this is
        lambda * (the left-to-right next-token CE of the clean sequence), the
        encoder AR term of [Gemma] Finetuning notes; with a mask it is the
        unweighted mean CE over the corrupted tokens.
      * WEIGHT_EXAMPLE_MEAN_CLIPPED: scale * min(1 / (1 - p_b), clip) /
        (n_b * B): the per-example mean of the scored CE weighted by the
        clipped inverse of one minus the example's rate, averaged over the B
        examples that have at least one scored row ([Axolotl] objective
        options: inv_one_minus_t with example_mean, capped by
        rhine_weight_clip).  The example's corruption rate p_b plays the
        role of t: under uniform noise the rate is drawn directly as
        t ~ U(eps, 1) ([Gemma] Finetuning notes).
        Order of evaluation: a = 1 / (1 - p_b); a = min(a, clip);
        w = scale * a / (n_b * B).  The default clip, +inf, caps nothing
        (as the library's weight_clip = +inf does).

    Eligibility ([Axolotl] "Packed training": tokens outside the loss, such
    as prompt tokens, are excluded) applies to the target token g.

    Returns (row_idx int64[M], tgt int64[M], w float64[M]).
    """
    x0 = np.asarray(x0, dtype=np.int64)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    n = x0.shape[0]
    rows, tgts, docs = [], [], []
    for b in range(cu.shape[0] - 1):
        for g in range(cu[b], cu[b + 1]):
            if corrupted is not None and not corrupted[g]:
                continue
            if eligible is not None and not eligible[g]:
                continue
            if align == SHIFTED:
                if g == cu[b]:
                    continue
                rows.append(g - 1)
            else:
                rows.append(g)
            tgts.append(x0[g])
            docs.append(b)
    m = len(rows)
    ws = []
    if weighting == WEIGHT_INV_P:
        p_doc = np.asarray(p_doc, dtype=np.float64)
        ws = [scale / (p_doc[b] * float(n)) for b in docs]
    elif weighting == WEIGHT_MEAN:
        ws = [scale / float(m) for _ in docs]
    elif weighting == WEIGHT_EXAMPLE_MEAN_CLIPPED:
        p_doc = np.asarray(p_doc, dtype=np.float64)
        per_doc = {}
        for b in docs:
            per_doc[b] = per_doc.get(b, 0) + 1
        n_examples = float(len(per_doc))
        for b in docs:
            a = 1.0 / (1.0 - p_doc[b])
            a = min(a, clip)
            ws.append(scale * a / (float(per_doc[b]) * n_examples))
    else:
        raise ValueError(f"unknown weighting {weighting}")
    return (np.asarray(rows, dtype=np.int64), np.asarray(tgts, dtype=np.int64),
            np.asarray(ws, dtype=np.float64))


def _capped_logits(rows_h, w_chunk, softcap):
    """Logits of the plain linear head, z = h W^T (no bias: [Axolotl]
    "Adapters, merging and inference": the output head is a bare linear map),
    then the tanh softcap c*tanh(z/c) applied once when c > 0 ([Gemma]
    Finetuning notes: the forward already softcaps; do not apply it twice).
    Returns (capped logits, d capped / d z)."""
    z = rows_h @ w_chunk.T
    if softcap > 0.0:
        th = np.tanh(z / softcap)
        return softcap * th, 1.0 - th * th
    return z, np.ones_like(z)


def head_ce_rows(hidden, W, row_idx, tgt, softcap=0.0, chunk=8192):
    """Per-row cross-entropy of hidden[row_idx] through the head W against tgt.

    CE_j = logsumexp_v(zhat_jv) - zhat_j,tgt_j over the full vocabulary.
    The vocabulary is processed in chunks only to bound memory; the
    log-sum-exp of the whole row is the log-sum-exp of the chunk values.

    Returns (ce float64[M], lse float64[M]).
    """
    rows_h = np.asarray(hidden)[np.asarray(row_idx, dtype=np.int64)].astype(np.float64)
    tgt = np.asarray(tgt, dtype=np.int64)
    W = np.asarray(W)
    m = rows_h.shape[0]
    v_total = W.shape[0]
    chunk_lse = []
    z_tgt = np.zeros(m, dtype=np.float64)
    for v0 in range(0, v_total, chunk):
        v1 = min(v0 + chunk, v_total)
        zc, _ = _capped_logits(rows_h, W[v0:v1].astype(np.float64), softcap)
        chunk_lse.append(logsumexp(zc, axis=1))
        hit = (tgt >= v0) & (tgt < v1)
        z_tgt[hit] = zc[np.flatnonzero(hit), tgt[hit] - v0]
    if m == 0:
        return np.zeros(0), np.zeros(0)
    lse = logsumexp(np.stack(chunk_lse, axis=1), axis=1)
    return lse - z_tgt, lse


def head_ce(hidden, W, row_idx, tgt, w, softcap=0.0, want_grad=True, chunk=8192):
    """Weighted CE loss and its gradient with respect to every hidden row.

    loss = sum_j w_j * CE_j.
    d loss / d h_row_j = w_j * ((softmax(zhat_j) - onehot(tgt_j)) * zhat'_j) W
    where zhat' is the softcap's derivative (1 without a cap).  The head is
    frozen ([LLaDA] LoRA row: embeddings and output layer frozen), so no
    gradient for W is formed.  Rows of hidden that are not scored get an
    exact zero gradient.

    Returns (loss float64, ce float64[M], d_hidden float64[N,H] or None).
    """
    hidden = np.asarray(hidden)
    row_idx = np.asarray(row_idx, dtype=np.int64)
    tgt = np.asarray(tgt, dtype=np.int64)
    w = np.asarray(w, dtype=np.float64)
    ce, lse = head_ce_rows(hidden, W, row_idx, tgt, softcap, chunk)
    loss = float(np.sum(w * ce)) if ce.size else 0.0
    if not want_grad:
        return loss, ce, None
    d_hidden = np.zeros(hidden.shape, dtype=np.float64)
    if row_idx.size == 0:
        return loss, ce, d_hidden
    rows_h = hidden[row_idx].astype(np.float64)
    d_rows = np.zeros_like(rows_h)
    W = np.asarray(W)
    for v0 in range(0, W.shape[0], chunk):
        v1 = min(v0 + chunk, W.shape[0])
        wc = W[v0:v1].astype(np.float64)
        zc, dcap = _capped_logits(rows_h, wc, softcap)
        prob = np.exp(zc - lse[:, None])
        hit = np.flatnonzero((tgt >= v0) & (tgt < v1))
        prob[hit, tgt[hit] - v0] -= 1.0
        d_rows += (w[:, None] * prob * dcap) @ wc
    d_hidden[row_idx] = d_rows
    return loss, ce, d_hidden


def head_ce_weight_grad(hidden, W, row_idx, tgt, w, softcap=0.0, chunk=8192, v_rows=None):
    """Gradient of loss = sum_j w_j CE_j with respect to the head W, for a
    head that is trained (the frozen-head case of [LLaDA] forms none):
        dW_v = sum_j w_j (softmax(zhat_j)_v - [v = tgt_j]) zhat'_jv h_row_j.
    Returns float64[V, H]; with ``v_rows`` (vocabulary indices) only those
    rows, float64[len(v_rows), H], from the same formula (the softmax still
    normalised over the whole vocabulary)."""
    hidden = np.asarray(hidden)
    row_idx = np.asarray(row_idx, dtype=np.int64)
    tgt = np.asarray(tgt, dtype=np.int64)
    w = np.asarray(w, dtype=np.float64)
    W = np.asarray(W)
    if v_rows is not None:
        v_rows = np.asarray(v_rows, dtype=np.int64)
        if row_idx.size == 0:
            return np.zeros((v_rows.shape[0], W.shape[1]), dtype=np.float64)
        _, lse = head_ce_rows(hidden, W, row_idx, tgt, softcap, chunk)
        rows_h = hidden[row_idx].astype(np.float64)
        zc, dcap = _capped_logits(rows_h, W[v_rows].astype(np.float64), softcap)
        prob = np.exp(zc - lse[:, None])
        prob -= (tgt[:, None] == v_rows[None, :]).astype(np.float64)
        return (w[:, None] * prob * dcap).T @ rows_h
    dW = np.zeros(W.shape, dtype=np.float64)
    if row_idx.size == 0:
        return dW
    _, lse = head_ce_rows(hidden, W, row_idx, tgt, softcap, chunk)
    rows_h = hidden[row_idx].astype(np.float64)
    for v0 in range(0, W.shape[0], chunk):
        v1 = min(v0 + chunk, W.shape[0])
        zc, dcap = _capped_logits(rows_h, W[v0:v1].astype(np.float64), softcap)
        prob = np.exp(zc - lse[:, None])
        hit = np.flatnonzero((tgt >= v0) & (tgt < v1))
        prob[hit, tgt[hit] - v0] -= 1.0
        dW[v0:v1] = (w[:, None] * prob * dcap).T @ rows_h
    return dW


def mdlm_loss(x0, cu_seqlens, hidden, W, seed, eps, noise, mask_id, rand_vocab,
              align, softcap=0.0, want_grad=True, chunk=8192):
    """The whole path: corrupt, list scored rows, weighted head + CE.

    The model forward that would turn xt into hidden states lies outside this
    path; ``hidden`` is given.  Returns a dict of every intermediate.
    """
    xt, corrupted, p_doc, doc_counts = corrupt(
        x0, cu_seqlens, seed, eps, noise, mask_id, rand_vocab)
    row_idx, tgt, w = compact(corrupted, x0, cu_seqlens, p_doc, align)
    loss, ce, d_hidden = head_ce(hidden, W, row_idx, tgt, w, softcap,
                                 want_grad, chunk)
    return dict(xt=xt, corrupted=corrupted, p_doc=p_doc, doc_counts=doc_counts,
                row_idx=row_idx, tgt=tgt, w=w, loss=loss, ce=ce,
                d_hidden=d_hidden)
