"""GPU parity of the corrective mixture (mdlm_corrupt_mixture and
mdlm_compact_corrective) against the oracle: tokens, codes, p, counts, rows,
targets and fp32 weights bit-exact; the loss through the fused head against
the oracle's loss (1e-3 relative) and gradient (1e-2 relative L2)."""

import numpy as np
import pytest
import torch

import oracle
import workloads as WL
from uniform_noise_diffusion_amd.pipeline import MdlmLossStep

from gpu_common import DEV, host

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


def _run(x0, cu, seed, eps, mix, align, a, c, mask_id=999, rand_vocab=1000):
    n, nd = x0.shape[0], cu.shape[0] - 1
    step = MdlmLossStep(n, nd, 64, 64, device=DEV, head_workspace_bytes=0, want_grad=False)
    tx0, tcu = torch.from_numpy(x0).to(DEV), torch.from_numpy(cu).to(DEV)
    step.corrupt_mixture(tx0, tcu, seed, eps, mix, mask_id, rand_vocab)
    step.compact_corrective(tx0, tcu, align, a, c)
    torch.cuda.synchronize()
    m = int(host(step.n_rows)[0])
    return dict(xt=host(step.xt), codes=host(step.corrupted), p_doc=host(step.p_doc),
                doc_counts=host(step.doc_counts), n_rows=m, row_idx=host(step.row_idx)[:m],
                tgt=host(step.tgt)[:m], w=host(step.w)[:m])


def _check(x0, cu, seed, eps, mix, align, a, c, mask_id=999, rand_vocab=1000):
    g = _run(x0, cu, seed, eps, mix, align, a, c, mask_id, rand_vocab)
    xt, codes, p, counts = oracle.corrupt_mixture(x0, cu, seed, eps, mix, mask_id, rand_vocab)
    assert np.array_equal(g["xt"], xt)
    assert np.array_equal(g["codes"], codes)
    assert np.array_equal(g["p_doc"].view(np.uint64), p.view(np.uint64))
    assert np.array_equal(g["doc_counts"], counts)
    rows, tgt, w = oracle.compact_corrective(codes, x0, cu, p, align, a, c)
    assert g["n_rows"] == rows.shape[0]
    assert np.array_equal(g["row_idx"], rows)
    assert np.array_equal(g["tgt"], tgt)
    assert np.array_equal(g["w"].view(np.uint32), w.astype(np.float32).view(np.uint32))
    return g


WEIGHTS = [(0.0, 0.0), (0.5, 0.0), (1.0, 0.0), (0.3, 0.7), (2.0, -0.5)]


@pytest.mark.parametrize("a,c", WEIGHTS)
@pytest.mark.parametrize("align", [oracle.ALIGNED, oracle.SHIFTED])
@pytest.mark.parametrize("seed,n_docs,max_len,empty", [
    (1, 1, 7, False),        # one tiny document, N not a multiple of 4
    (2, 40, 300, True),      # empty documents, several compaction tiles
    (3, 7, 3000, False),     # documents spanning block boundaries
    (4, 600, 20, True),      # many short documents per block
    (5, 5000, 2, True),      # more documents per 4096-token block than it caches
    (6, 3000, 9, False),     # about 800 documents per block: cached by the masked
                             # form, not by the code-weight form
])
def test_corrective_bit_exact_small(a, c, align, seed, n_docs, max_len, empty):
    x0, cu = _case(seed, n_docs, max_len, empty)
    _check(x0, cu, seed * 104729 + 5, 1e-3, 0.3, align, a, c)


@pytest.mark.parametrize("mix", [0.0, 1e-7, 0.5, 1.0])
def test_mixture_extremes(mix):
    """mixture_prob 0 is absorbing corruption (mdlm_corrupt's output with the
    same codes); 1 replaces every corrupted token with the uniform-noise id."""
    x0, cu = _case(9, 30, 700)
    g = _check(x0, cu, 2**63 + 99, 1e-3, mix, oracle.ALIGNED, 0.5, 0.0)
    if mix in (0.0, 1.0):
        step = MdlmLossStep(x0.shape[0], cu.shape[0] - 1, 64, 64, device=DEV,
                            head_workspace_bytes=0, want_grad=False)
        tx0, tcu = torch.from_numpy(x0).to(DEV), torch.from_numpy(cu).to(DEV)
        noise = oracle.NOISE_ABSORB if mix == 0.0 else oracle.NOISE_UNIFORM
        step.corrupt(tx0, tcu, 2**63 + 99, 1e-3, noise, 999, 1000)
        torch.cuda.synchronize()
        corr = host(step.corrupted)
        assert np.array_equal(g["codes"], corr * (1 if mix == 0.0 else 2))
        assert np.array_equal(g["xt"], host(step.xt))
        assert np.array_equal(g["doc_counts"], host(step.doc_counts))


@pytest.mark.parametrize("k", [1, 2, 4])
@pytest.mark.parametrize("align", [oracle.ALIGNED, oracle.SHIFTED])
def test_corrective_bit_exact_workloads(k, align):
    wl = WL.make_workload(k)
    inp = WL.generate(wl, with_hidden=False, with_head=False)
    for seed, (a, c) in zip((wl.seed, 1, 2), WEIGHTS[1:]):
        _check(inp.x0, inp.cu_seqlens, seed, wl.eps, 0.25, align, a, c, wl.mask_id,
               wl.rand_vocab)


@pytest.mark.parametrize("align", [oracle.ALIGNED, oracle.SHIFTED])
@pytest.mark.parametrize("a,c", [(0.5, 0.0), (0.5, 0.2)])
def test_corrective_across_scan_groups(align, a, c):
    """1,025 full tiles and a ragged one, lognormal documents of mean 296."""
    rng = np.random.default_rng(41)
    n = 1025 * 4096 + 777
    cu = WL.lognormal_stream_offsets(78, 296, n).astype(np.int32)
    x0 = rng.integers(0, 126000, size=n).astype(np.int32)
    _check(x0, cu, 5151, 1e-3, 0.2, align, a, c, 126336, 126464)


def test_empty_stream():
    x0 = np.zeros(0, dtype=np.int32)
    cu = np.zeros(2, dtype=np.int32)
    g = _run(x0, cu, 5, 1e-3, 0.5, oracle.ALIGNED, 0.5, 0.5)
    assert g["n_rows"] == 0
    assert g["doc_counts"][0] == 0


@pytest.mark.parametrize("softcap", [0.0, 30.0])
def test_corrective_loss_through_the_fused_head(softcap):
    """The corrective rows through the fused bf16 head, against the oracle's
    loss and gradient on the oracle's rows."""
    case = WL.small_case(23, n_docs=6, max_len=300, H=128, V=1000, dtype="bf16",
                         softcap=softcap)
    x0, cu = case.x0, case.cu_seqlens
    n = x0.shape[0]
    seed, eps, mix, a, c = 321, 1e-3, 0.3, 0.6, 0.1
    step = MdlmLossStep(n, cu.shape[0] - 1, 128, 1000, dtype=torch.bfloat16, device=DEV)
    tx0, tcu = torch.from_numpy(x0).to(DEV), torch.from_numpy(cu).to(DEV)
    h = torch.from_numpy(case.hidden_bits.view(np.int16)).to(DEV).view(torch.bfloat16)
    W = torch.from_numpy(case.W_bits.view(np.int16)).to(DEV).view(torch.bfloat16)
    step.corrupt_mixture(tx0, tcu, seed, eps, mix, 999, 1000)
    step.compact_corrective(tx0, tcu, oracle.SHIFTED, a, c)
    step.head_ce(h, W, softcap)
    torch.cuda.synchronize()
    _, codes, p, _ = oracle.corrupt_mixture(x0, cu, seed, eps, mix, 999, 1000)
    rows, tgt, w = oracle.compact_corrective(codes, x0, cu, p, oracle.SHIFTED, a, c)
    loss, _, dh = oracle.head_ce(case.hidden, case.W, rows, tgt, w.astype(np.float32), softcap)
    got = float(host(step.loss)[0])
    assert abs(got - loss) <= 1e-3 * abs(loss)
    gd = host(step.d_hidden.float())
    assert np.linalg.norm(gd - dh) <= 1e-2 * np.linalg.norm(dh)


def test_large_stream_sampled():
    """2^27 tokens in documents of 4,096: counts and row total on the device,
    codes against the oracle's draws on sampled documents, rows and weights
    by their definition."""
    n_docs, L = 32768, 4096
    n = n_docs * L
    cu = torch.arange(0, n + 1, L, dtype=torch.int32, device=DEV)
    g = torch.Generator(device=DEV).manual_seed(4)
    x0 = torch.randint(0, 126336, (n,), dtype=torch.int32, device=DEV, generator=g)
    step = MdlmLossStep(n, n_docs, 64, 64, device=DEV, head_workspace_bytes=0,
                        want_grad=False)
    seed, a, mix = 77, 0.5, 0.25
    step.corrupt_mixture(x0, cu, seed, 1e-3, mix, 126336, 126464)
    step.compact_corrective(x0, cu, oracle.ALIGNED, a, 0.0)
    torch.cuda.synchronize()
    _, p_all, thr_all = oracle.noise_levels(seed, 1e-3, n_docs)
    assert np.array_equal(host(step.p_doc).view(np.uint64), p_all.view(np.uint64))
    codes = step.corrupted
    m = int(host(step.n_rows)[0])
    assert m == int(host(step.doc_counts).astype(np.int64).sum())
    thr_mix = int(np.ceil(mix * 2.0**24))
    for b in [0, 1, n_docs // 3, n_docs - 1]:
        lo, hi = b * L, (b + 1) * L
        w1 = oracle.mdlm.token_words(seed, L, oracle.mdlm.TAG_BERNOULLI, start=lo)
        w3 = oracle.mdlm.token_words(seed, L, oracle.mdlm.TAG_MIX, start=lo)
        corr = (w1 >> 8) < thr_all[b]
        want = np.where(corr, np.where((w3 >> 8) < thr_mix, 2, 1), 0).astype(np.uint8)
        assert np.array_equal(host(codes[lo:hi]), want), b
    pos = torch.nonzero(codes).flatten()
    assert torch.equal(step.row_idx[:m].long(), pos)
    assert torch.equal(step.tgt[:m], x0[pos])
    p_dev = torch.from_numpy(p_all).to(DEV)
    cp = codes[pos].to(torch.float64)
    scale = torch.where(cp == 1, torch.ones_like(cp), torch.full_like(cp, a))
    want_w = (scale / (p_dev[pos // L] * float(n))).to(torch.float32)
    assert torch.equal(step.w[:m].view(torch.int32), want_w.view(torch.int32))
