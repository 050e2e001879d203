"""GPU parity of mdlm_compact_rows (the loss variants' row lists) against the
oracle: rows, targets and fp32 weights bit-exact; the encoder AR term through
the fused head against the oracle's loss and gradient."""

import numpy as np
import pytest
import torch

import oracle
import workloads as WL
from uniform_noise_diffusion_amd import binding as B
from uniform_noise_diffusion_amd.pipeline import MdlmLossStep

from gpu_common import DEV, host

pytestmark = pytest.mark.gpu

MODES = [oracle.WEIGHT_INV_P, oracle.WEIGHT_MEAN, oracle.WEIGHT_EXAMPLE_MEAN_CLIPPED]


def _docs(seed, n_docs, max_len, empty=True):
    rng = np.random.default_rng(seed)
    lengths = rng.integers(1, max_len + 1, size=n_docs)
    if empty:
        lengths[rng.random(n_docs) < 0.2] = 0
    cu = np.zeros(n_docs + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    x0 = rng.integers(0, 999, size=int(cu[-1])).astype(np.int32)
    return rng, x0, cu


def _gpu_rows(x0, cu, align, weighting, scale, clip, use_mask, elig, seed=17, eps=1e-3,
              noise=0):
    n, nd = x0.shape[0], cu.shape[0] - 1
    step = MdlmLossStep(n, nd, 64, 64, device=DEV, head_workspace_bytes=0, want_grad=False)
    tx0, tcu = torch.from_numpy(x0).to(DEV), torch.from_numpy(cu).to(DEV)
    step.corrupt(tx0, tcu, seed, eps, noise, 999, 1000)
    te = None if elig is None else torch.from_numpy(elig.astype(np.uint8)).to(DEV)
    step.compact_rows(tx0, tcu, align, weighting, scale, clip,
                      corrupted=True if use_mask else None, eligible=te)
    torch.cuda.synchronize()
    m = int(host(step.n_rows)[0])
    return (host(step.corrupted), host(step.p_doc), m, host(step.row_idx)[:m],
            host(step.tgt)[:m], host(step.w)[:m])


def _check(x0, cu, align, weighting, scale, clip, use_mask, elig, **kw):
    corrupted, p, m, rows, tgt, w = _gpu_rows(x0, cu, align, weighting, scale, clip, use_mask,
                                              elig, **kw)
    r, t, ww = oracle.compact_rows(x0, cu, align, corrupted if use_mask else None, elig, p,
                                   weighting, scale, clip)
    assert m == r.shape[0]
    assert np.array_equal(rows, r)
    assert np.array_equal(tgt, t)
    assert np.array_equal(w.view(np.uint32), ww.astype(np.float32).view(np.uint32))
    return m


@pytest.mark.parametrize("weighting", MODES)
@pytest.mark.parametrize("align", [oracle.ALIGNED, oracle.SHIFTED])
@pytest.mark.parametrize("use_mask,use_elig", [(True, False), (False, False), (True, True),
                                               (False, True)])
@pytest.mark.parametrize("seed,n_docs,max_len", [(1, 1, 9), (2, 40, 300), (3, 600, 20),
                                                 (4, 7, 3000)])
def test_rows_bit_exact_small(weighting, align, use_mask, use_elig, seed, n_docs, max_len):
    rng, x0, cu = _docs(seed, n_docs, max_len)
    elig = (rng.random(x0.shape[0]) < 0.8) if use_elig else None
    _check(x0, cu, align, weighting, 0.7, 3.0, use_mask, elig, seed=seed + 100)


@pytest.mark.parametrize("weighting", MODES)
@pytest.mark.parametrize("k", [3, 5])
def test_rows_bit_exact_workloads(weighting, k):
    wl = WL.make_workload(k)
    inp = WL.generate(wl, with_hidden=False, with_head=False)
    for use_mask in (True, False):
        _check(inp.x0, inp.cu_seqlens, wl.align, weighting, 1.0, 8.0, use_mask, None,
               seed=3, eps=wl.eps, noise=wl.noise)


def test_causal_rows_across_scan_groups():
    """Every-token shifted rows over 1,025 tiles plus a ragged one (two
    groups of the offset scan) with lognormal documents."""
    rng = np.random.default_rng(9)
    n = 1025 * 4096 + 77
    cu = WL.lognormal_stream_offsets(5, 296, n).astype(np.int32)
    x0 = rng.integers(0, 126000, size=n).astype(np.int32)
    m = _check(x0, cu, oracle.SHIFTED, oracle.WEIGHT_MEAN, 0.5, 1.0, False, None)
    assert m == n - (cu.shape[0] - 1)


def test_no_eligible_token_gives_no_rows():
    rng, x0, cu = _docs(5, 30, 100)
    elig = np.zeros(x0.shape[0], dtype=bool)
    for weighting in MODES:
        assert _check(x0, cu, oracle.ALIGNED, weighting, 1.0, 2.0, True, elig) == 0


def test_clip_infinity_and_full_rate():
    # eps = 1: every rate is 1, so 1/(1-p) = inf and the clip decides
    rng, x0, cu = _docs(6, 12, 200, empty=False)
    _check(x0, cu, oracle.ALIGNED, oracle.WEIGHT_EXAMPLE_MEAN_CLIPPED, 1.0, 5.0, True, None,
           eps=1.0)
    _check(x0, cu, oracle.SHIFTED, oracle.WEIGHT_EXAMPLE_MEAN_CLIPPED, 2.0, float("inf"), True,
           None, eps=0.3)


@pytest.mark.parametrize("softcap", [0.0, 30.0])
def test_encoder_ar_term_through_the_fused_head(softcap):
    """total = diffusion CE + lambda * AR CE, AR term alone: every-token
    shifted rows with mean weights through the fused bf16 head, against the
    oracle's loss (1e-3 relative) and gradient (1e-2 relative L2)."""
    case = WL.small_case(21, n_docs=5, max_len=300, H=128, V=1000, dtype="bf16",
                         softcap=softcap)
    x0, cu = case.x0, case.cu_seqlens
    n = x0.shape[0]
    lam = 0.25
    step = MdlmLossStep(n, cu.shape[0] - 1, 128, 1000, dtype=torch.bfloat16, device=DEV)
    tx0, tcu = torch.from_numpy(x0).to(DEV), torch.from_numpy(cu).to(DEV)
    h = torch.from_numpy(case.hidden_bits.view(np.int16)).to(DEV).view(torch.bfloat16)
    W = torch.from_numpy(case.W_bits.view(np.int16)).to(DEV).view(torch.bfloat16)
    step.compact_rows(tx0, tcu, oracle.SHIFTED, B.MDLM_WEIGHT_MEAN, lam, corrupted=None)
    step.head_ce(h, W, softcap)
    torch.cuda.synchronize()
    rows, tgt, w = oracle.compact_rows(x0, cu, oracle.SHIFTED, weighting=oracle.WEIGHT_MEAN,
                                       scale=lam)
    loss, _, dh = oracle.head_ce(case.hidden, case.W, rows, tgt, w.astype(np.float32), softcap)
    got = float(host(step.loss)[0])
    assert abs(got - loss) <= 1e-3 * abs(loss)
    gd = host(step.d_hidden.float())
    assert np.linalg.norm(gd - dh) <= 1e-2 * np.linalg.norm(dh)
