"""GPU parity of corruption and compaction: bit-exact against the oracle.

Integer outputs (xt, corrupted, doc_counts, row_idx, tgt, n_rows) must be
identical; p_doc is fp64 and must be identical bit for bit (same operation
order, no fused multiply-add); w is fp32(1/(p N)) and must be identical.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle.mdlm import token_words
import workloads as WL
from uniform_noise_diffusion_amd import binding as B
from uniform_noise_diffusion_amd.pipeline import MdlmLossStep

from gpu_common import DEV, dev_tokens, host

pytestmark = pytest.mark.gpu


def _case(seed, n_docs, max_len, empty=False, V=1000):
    rng = np.random.default_rng(seed)
    lengths = rng.integers(1, max_len + 1, size=n_docs)
    if empty:
        lengths[rng.random(n_docs) < 0.3] = 0
    cu = np.zeros(n_docs + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    x0 = rng.integers(0, V - 1, size=int(cu[-1])).astype(np.int32)
    return x0, cu


def _gpu_corrupt_compact(x0, cu, seed, eps, noise, mask_id, rand_vocab, align):
    n, nd = x0.shape[0], cu.shape[0] - 1
    step = MdlmLossStep(n, nd, 64, 64, device=DEV, head_workspace_bytes=0, want_grad=False)
    tx0 = torch.from_numpy(x0).to(DEV)
    tcu = torch.from_numpy(cu).to(DEV)
    step.corrupt(tx0, tcu, seed, eps, noise, mask_id, rand_vocab)
    step.compact(tx0, tcu, align)
    torch.cuda.synchronize()
    m = int(host(step.n_rows)[0])
    return dict(xt=host(step.xt), corrupted=host(step.corrupted), p_doc=host(step.p_doc),
                doc_counts=host(step.doc_counts), n_rows=m, row_idx=host(step.row_idx)[:m],
                tgt=host(step.tgt)[:m], w=host(step.w)[:m])


def _check(x0, cu, seed, eps, noise, mask_id, rand_vocab, align):
    g = _gpu_corrupt_compact(x0, cu, seed, eps, noise, mask_id, rand_vocab, align)
    xt, corrupted, p, counts = oracle.corrupt(x0, cu, seed, eps, noise, mask_id, rand_vocab)
    assert np.array_equal(g["xt"], xt)
    assert np.array_equal(g["corrupted"], corrupted)
    assert np.array_equal(g["p_doc"].view(np.uint64), p.view(np.uint64))
    assert np.array_equal(g["doc_counts"], counts)
    rows, tgt, w = oracle.compact(corrupted, x0, cu, p, align)
    assert g["n_rows"] == rows.shape[0]
    assert np.array_equal(g["row_idx"], rows)
    assert np.array_equal(g["tgt"], tgt)
    assert np.array_equal(g["w"].view(np.uint32), w.astype(np.float32).view(np.uint32))
    return g


@pytest.mark.parametrize("noise", [oracle.NOISE_ABSORB, oracle.NOISE_UNIFORM])
@pytest.mark.parametrize("align", [oracle.ALIGNED, oracle.SHIFTED])
@pytest.mark.parametrize("seed,n_docs,max_len,empty", [
    (1, 1, 7, False),        # a single tiny document, N not a multiple of 4
    (2, 40, 300, True),      # empty documents, several compaction tiles
    (3, 7, 3000, False),     # documents spanning block boundaries
    (4, 600, 20, True),      # many short documents per block
    (5, 5000, 2, True),      # more documents per 4096-token block than it caches
    (10, 2000, 2, True),     # one block, more documents than it caches
    (11, 1024, 4, False),    # one block holding exactly as many documents as it caches
])
def test_corrupt_compact_bit_exact_small(noise, align, seed, n_docs, max_len, empty):
    x0, cu = _case(seed, n_docs, max_len, empty)
    _check(x0, cu, seed * 7919 + 13, 1e-3, noise, 999, 1000, align)


@pytest.mark.parametrize("eps", [1.0, 0.5, 1e-6])
def test_corrupt_eps_extremes(eps):
    x0, cu = _case(9, 20, 500)
    g = _check(x0, cu, 2**63 + 12345, eps, oracle.NOISE_ABSORB, 999, 1000, oracle.ALIGNED)
    if eps == 1.0:
        assert g["corrupted"].all()


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("align", [oracle.ALIGNED, oracle.SHIFTED])
def test_corrupt_compact_bit_exact_workloads(k, align):
    wl = WL.make_workload(k)
    inp = WL.generate(wl, with_hidden=False, with_head=False)
    for seed in (wl.seed, 1, 2, 3):
        _check(inp.x0, inp.cu_seqlens, seed, wl.eps, wl.noise, wl.mask_id, wl.rand_vocab, align)


@pytest.mark.parametrize("align", [oracle.ALIGNED, oracle.SHIFTED])
def test_compaction_across_scan_groups(align):
    """1,025 full tiles and a ragged one (two groups of the offset scan), with
    lognormal documents of mean 296 plus a run of 3-token documents: every
    output is compared with the oracle."""
    rng = np.random.default_rng(31)
    n = 1025 * 4096 + 1234
    cu = WL.lognormal_stream_offsets(77, 296, n)
    short = np.arange(cu[100], cu[100] + 3 * 400, 3)
    cu = np.unique(np.concatenate([cu, short])).astype(np.int32)
    x0 = rng.integers(0, 126000, size=n).astype(np.int32)
    _check(x0, cu, 4242, 1e-3, oracle.NOISE_ABSORB, 126336, 126464, align)


def test_empty_stream():
    x0 = np.zeros(0, dtype=np.int32)
    cu = np.zeros(2, dtype=np.int32)
    g = _gpu_corrupt_compact(x0, cu, 5, 1e-3, 0, 1, 2, oracle.ALIGNED)
    assert g["n_rows"] == 0
    _, _, p, counts = oracle.corrupt(x0, cu, 5, 1e-3, 0, 1, 2)
    assert np.array_equal(g["p_doc"].view(np.uint64), p.view(np.uint64))
    assert g["doc_counts"][0] == 0


def test_shifted_single_token_documents_score_nothing():
    cu = np.arange(0, 301, dtype=np.int32)
    x0 = np.arange(300, dtype=np.int32) % 50
    g = _gpu_corrupt_compact(x0, cu, 3, 1.0, 0, 99, 100, oracle.SHIFTED)
    assert g["n_rows"] == 0 and g["corrupted"].all()


def test_repeat_is_deterministic():
    x0, cu = _case(11, 50, 400, True)
    a = _gpu_corrupt_compact(x0, cu, 77, 1e-3, 1, 0, 1000, oracle.SHIFTED)
    b = _gpu_corrupt_compact(x0, cu, 77, 1e-3, 1, 0, 1000, oracle.SHIFTED)
    for key in a:
        assert np.array_equal(np.asarray(a[key]), np.asarray(b[key])), key


def test_large_stream_sampled():
    """2^27 tokens in 32,768 documents of 4,096 (the bandwidth shape): the
    full corruption mask is checked against the oracle on sampled documents
    and the compaction by its invariants plus sampled rows."""
    n_docs, L = 32768, 4096
    n = n_docs * L
    cu = torch.arange(0, n + 1, L, dtype=torch.int32, device=DEV)
    x0 = torch.randint(0, 126336, (n,), dtype=torch.int32,
                       generator=torch.Generator().manual_seed(0)).to(DEV)
    step = MdlmLossStep(n, n_docs, 64, 64, device=DEV, head_workspace_bytes=0,
                        want_grad=False)
    step.corrupt(x0, cu, 42, 1e-3, oracle.NOISE_ABSORB, 126336, 126464)
    step.compact(x0, cu, oracle.ALIGNED)
    torch.cuda.synchronize()
    counts = host(step.doc_counts)
    m = int(host(step.n_rows)[0])
    assert m == int(counts.astype(np.int64).sum())
    # the oracle on sampled documents: the draw of document b depends only on
    # (seed, b, absolute token index), so a document is checked in place
    rng = np.random.default_rng(1)
    x0h = host(x0)
    corr = host(step.corrupted)
    xt = host(step.xt)
    _, p_all, thr_all = oracle.noise_levels(42, 1e-3, n_docs)
    assert np.array_equal(host(step.p_doc).view(np.uint64), p_all.view(np.uint64))
    for b in rng.choice(n_docs, size=6, replace=False):
        lo, hi = b * L, (b + 1) * L
        wsub = token_words(42, L, oracle.mdlm.TAG_BERNOULLI, start=lo)
        exp = ((wsub >> 8) < thr_all[b]).astype(np.uint8)
        assert np.array_equal(corr[lo:hi], exp)
        assert np.array_equal(xt[lo:hi], np.where(exp == 1, 126336, x0h[lo:hi]))
    # compaction: rows ascending, exactly the corrupted positions
    rows = host(step.row_idx)[:m]
    assert np.array_equal(rows, np.flatnonzero(corr))
    tg = host(step.tgt)[:m]
    assert np.array_equal(tg, x0h[rows])
    w = host(step.w)[:m]
    doc = rows // L
    assert np.array_equal(w.view(np.uint32),
                          (1.0 / (p_all[doc] * float(n))).astype(np.float32).view(np.uint32))


@pytest.mark.parametrize("align", [oracle.ALIGNED, oracle.SHIFTED])
def test_maximum_stream_sampled(align):
    """The largest stream the ABI accepts: 2^31 - 1 tokens (documents of 4,096,
    the last one 4,095 long).  p is compared in full; the corruption on
    sampled documents including the last ones, whose token indices are the
    largest; the compaction by invariants checked on the device (rows are the
    scored positions in order, targets gathered from x0, weights
    1 / (p N))."""
    L = 4096
    n = 2**31 - 1
    n_docs = -(-n // L)
    cu = torch.arange(0, n_docs + 1, dtype=torch.int64, device=DEV) * L
    cu[-1] = n
    cu = cu.to(torch.int32)
    g = torch.Generator(device=DEV).manual_seed(3)
    x0 = torch.randint(0, 126336, (n,), dtype=torch.int32, device=DEV, generator=g)
    step = MdlmLossStep(n, n_docs, 64, 64, device=DEV, head_workspace_bytes=0,
                        want_grad=False)
    seed = 2**63 + 7
    step.corrupt(x0, cu, seed, 1e-3, oracle.NOISE_ABSORB, 126336, 126464)
    step.compact(x0, cu, align)
    torch.cuda.synchronize()
    _, p_all, thr_all = oracle.noise_levels(seed, 1e-3, n_docs)
    assert np.array_equal(host(step.p_doc).view(np.uint64), p_all.view(np.uint64))
    for b in [0, 1, n_docs // 2, n_docs - 2, n_docs - 1]:
        lo, hi = b * L, min((b + 1) * L, n)
        wsub = token_words(seed, hi - lo, oracle.mdlm.TAG_BERNOULLI, start=lo)
        exp = ((wsub >> 8) < thr_all[b]).astype(np.uint8)
        assert np.array_equal(host(step.corrupted[lo:hi]), exp), b
        assert np.array_equal(host(step.xt[lo:hi]),
                              np.where(exp == 1, 126336, host(x0[lo:hi]))), b
        assert int(host(step.doc_counts[b:b + 1])[0]) == int(exp.sum())
    # compaction invariants on the device
    m = int(host(step.n_rows)[0])
    scored = step.corrupted.bool()
    if align == oracle.SHIFTED:
        scored[cu[:-1].long()] = False
    pos = torch.nonzero(scored).flatten()
    assert m == pos.numel()
    rows = step.row_idx[:m].long()
    assert torch.equal(rows, pos - (1 if align == oracle.SHIFTED else 0))
    assert torch.equal(step.tgt[:m], x0[pos])
    p_dev = torch.from_numpy(p_all).to(DEV)
    want_w = (1.0 / (p_dev[pos // L] * float(n))).to(torch.float32)
    assert torch.equal(step.w[:m].view(torch.int32), want_w.view(torch.int32))


@pytest.mark.parametrize("fill", ["zeros", "minus_one", "int_max", "random_docs", "other_layout"])
def test_corruption_ignores_stale_xt(fill):
    """The corruption call keeps per-block document hints in xt before it
    writes the tokens there; whatever xt holds on entry must not change the
    result.  xt is pre-filled with values that are out of range, in range but
    wrong, or the output of an earlier call with another document layout."""
    rng = np.random.default_rng(8)
    n = 40 * 4096 + 123
    cu = WL.lognormal_stream_offsets(12, 296, n).astype(np.int32)
    x0 = rng.integers(0, 999, size=n).astype(np.int32)
    nd = cu.shape[0] - 1
    step = MdlmLossStep(n, max(nd, 41), 64, 64, device=DEV, head_workspace_bytes=0,
                        want_grad=False)
    tx0 = torch.from_numpy(x0).to(DEV)
    if fill == "other_layout":
        cu_other = np.minimum(np.arange(0, n + 4096, 4096), n).astype(np.int32)
        cu_other = np.unique(cu_other)
        B_other = cu_other.shape[0] - 1
        p_other = torch.empty(B_other, dtype=torch.float64, device=DEV)
        c_other = torch.empty(B_other, dtype=torch.int32, device=DEV)
        from uniform_noise_diffusion_amd import binding as Bn
        Bn.mdlm_corrupt(tx0, torch.from_numpy(cu_other).to(DEV), 1, 1e-3, 0, 999, 1000,
                        step.xt, step.corrupted, p_other, c_other)
    else:
        val = {"zeros": 0, "minus_one": -1, "int_max": 2**31 - 1}.get(fill)
        if val is None:
            step.xt.copy_(torch.from_numpy(rng.integers(0, nd, size=n).astype(np.int32)))
        else:
            step.xt.fill_(val)
    p_doc = torch.empty(nd, dtype=torch.float64, device=DEV)
    counts = torch.empty(nd, dtype=torch.int32, device=DEV)
    from uniform_noise_diffusion_amd import binding as Bn
    Bn.mdlm_corrupt(tx0, torch.from_numpy(cu).to(DEV), 99, 1e-3, 0, 999, 1000, step.xt,
                    step.corrupted, p_doc, counts)
    torch.cuda.synchronize()
    xt, corrupted, p, cnt = oracle.corrupt(x0, cu, 99, 1e-3, 0, 999, 1000)
    assert np.array_equal(host(step.xt), xt)
    assert np.array_equal(host(step.corrupted), corrupted)
    assert np.array_equal(host(counts), cnt)


@pytest.mark.parametrize("align", [oracle.ALIGNED, oracle.SHIFTED])
def test_long_documents(align):
    """Documents spanning more blocks than the per-document hints cover
    (the blocks past them search for their documents), among enough short
    ones that the mean length selects the hints."""
    lengths = ([300_000] + [5] * 1500 + [4096 * 70] + [17] * 500 + [0] * 10
               + [4096 * 64 + 1] + [3] * 3000)
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    rng = np.random.default_rng(9)
    x0 = rng.integers(0, 999, size=int(cu[-1])).astype(np.int32)
    for noise in (oracle.NOISE_ABSORB, oracle.NOISE_UNIFORM):
        _check(x0, cu, 1234 + noise, 0.3, noise, 999, 1000, align)


def _offset_view(n, dtype, fill=None):
    """A device tensor of n elements that starts one element into its
    allocation, so that its address is not 16-byte aligned."""
    base = torch.empty(n + 1, dtype=dtype, device=DEV)
    if fill is not None:
        base.fill_(fill)
    return base[1:]


@pytest.mark.parametrize("noise", [oracle.NOISE_ABSORB, oracle.NOISE_UNIFORM])
@pytest.mark.parametrize("align", [oracle.ALIGNED, oracle.SHIFTED])
@pytest.mark.parametrize("mean_len", [30, 5000])
def test_unaligned_buffers(noise, align, mean_len):
    """Token, mask and row buffers that are not 16-byte (the mask: not
    4-byte) aligned take the kernels' scalar paths; results as the oracle's."""
    from uniform_noise_diffusion_amd import binding as Bn
    rng = np.random.default_rng(13 + mean_len)
    n = 3 * 4096 + 777
    cu = WL.lognormal_stream_offsets(14 + mean_len, mean_len, n).astype(np.int32)
    nd = cu.shape[0] - 1
    x0 = rng.integers(0, 999, size=n).astype(np.int32)
    tx0 = _offset_view(n, torch.int32)
    tx0.copy_(torch.from_numpy(x0))
    tcu = torch.from_numpy(cu).to(DEV)
    xt = _offset_view(n, torch.int32)
    corr = _offset_view(n, torch.uint8)
    p_doc = torch.empty(nd, dtype=torch.float64, device=DEV)
    counts = torch.empty(nd, dtype=torch.int32, device=DEV)
    Bn.mdlm_corrupt(tx0, tcu, 321, 1e-3, noise, 999, 1000, xt, corr, p_doc, counts)
    rows = _offset_view(n, torch.int32)
    tgt = _offset_view(n, torch.int32)
    w = _offset_view(n, torch.float32)
    n_rows = torch.empty(1, dtype=torch.int32, device=DEV)
    ws = torch.empty(Bn.mdlm_compact_workspace_bytes(n), dtype=torch.uint8, device=DEV)
    Bn.mdlm_compact_masked(corr, tx0, tcu, p_doc, align, rows, tgt, w, n_rows, ws)
    torch.cuda.synchronize()
    e_xt, e_corr, e_p, e_cnt = oracle.corrupt(x0, cu, 321, 1e-3, noise, 999, 1000)
    assert np.array_equal(host(xt), e_xt)
    assert np.array_equal(host(corr), e_corr)
    assert np.array_equal(host(counts), e_cnt)
    e_rows, e_tgt, e_w = oracle.compact(e_corr, x0, cu, e_p, align)
    m = int(host(n_rows)[0])
    assert m == e_rows.shape[0]
    assert np.array_equal(host(rows)[:m], e_rows)
    assert np.array_equal(host(tgt)[:m], e_tgt)
    assert np.array_equal(host(w)[:m].view(np.uint32), e_w.astype(np.float32).view(np.uint32))
    # the corrective pair on the same unaligned buffers
    Bn.mdlm_corrupt_mixture(tx0, tcu, 322, 1e-3, 0.4, 999, 1000, xt, corr, p_doc, counts)
    Bn.mdlm_compact_corrective(corr, tx0, tcu, p_doc, align, 0.5, 0.2, rows, tgt, w, n_rows, ws)
    torch.cuda.synchronize()
    e_xt, e_codes, e_p, e_cnt = oracle.corrupt_mixture(x0, cu, 322, 1e-3, 0.4, 999, 1000)
    assert np.array_equal(host(xt), e_xt)
    assert np.array_equal(host(corr), e_codes)
    e_rows, e_tgt, e_w = oracle.compact_corrective(e_codes, x0, cu, e_p, align, 0.5, 0.2)
    m = int(host(n_rows)[0])
    assert m == e_rows.shape[0]
    assert np.array_equal(host(rows)[:m], e_rows)
    assert np.array_equal(host(tgt)[:m], e_tgt)
    assert np.array_equal(host(w)[:m].view(np.uint32), e_w.astype(np.float32).view(np.uint32))


@pytest.mark.parametrize("weighting", [oracle.WEIGHT_MEAN, oracle.WEIGHT_EXAMPLE_MEAN_CLIPPED])
def test_unaligned_row_masks(weighting):
    """mdlm_compact_rows with corruption and eligibility masks that are not
    4-byte aligned (the per-document count of the example mean included)."""
    from uniform_noise_diffusion_amd import binding as Bn
    rng = np.random.default_rng(17)
    n = 2 * 4096 + 333
    cu = WL.lognormal_stream_offsets(18, 200, n).astype(np.int32)
    nd = cu.shape[0] - 1
    x0 = rng.integers(0, 999, size=n).astype(np.int32)
    corr_h = (rng.random(n) < 0.5).astype(np.uint8)
    elig_h = (rng.random(n) < 0.8).astype(np.uint8)
    p_h = rng.uniform(0.01, 1.0, size=nd)
    tx0 = torch.from_numpy(x0).to(DEV)
    tcu = torch.from_numpy(cu).to(DEV)
    corr = _offset_view(n, torch.uint8)
    corr.copy_(torch.from_numpy(corr_h))
    elig = _offset_view(n, torch.uint8)
    elig.copy_(torch.from_numpy(elig_h))
    p_doc = torch.from_numpy(p_h).to(DEV)
    rows = torch.empty(n, dtype=torch.int32, device=DEV)
    tgt = torch.empty(n, dtype=torch.int32, device=DEV)
    w = torch.empty(n, dtype=torch.float32, device=DEV)
    n_rows = torch.empty(1, dtype=torch.int32, device=DEV)
    ws = torch.empty(Bn.mdlm_compact_rows_workspace_bytes(n, nd, weighting), dtype=torch.uint8,
                     device=DEV)
    for align in (oracle.ALIGNED, oracle.SHIFTED):
        Bn.mdlm_compact_rows(corr, elig, tx0, tcu, p_doc, align, weighting, 1.5, 4.0, rows, tgt,
                             w, n_rows, ws)
        torch.cuda.synchronize()
        e_rows, e_tgt, e_w = oracle.compact_rows(x0, cu, align, corr_h, elig_h, p_h, weighting,
                                                 1.5, 4.0)
        m = int(host(n_rows)[0])
        assert m == e_rows.shape[0]
        assert np.array_equal(host(rows)[:m], e_rows)
        assert np.array_equal(host(tgt)[:m], e_tgt)
        assert np.array_equal(host(w)[:m].view(np.uint32),
                              e_w.astype(np.float32).view(np.uint32))
