"""Seeded random sweeps of the whole path against the oracle.

Each case draws its own shape and options from a fixed seed: document
layouts (empty and one-token documents included), both noise modes, both
alignments, eps, hidden sizes that are multiples of 64, vocabularies from a
handful of entries to a few thousand (ragged 256-wide tiles), softcap on or
off, and head workspaces from the minimum (256-wide vocabulary chunks,
logits recomputed) through intermediate sizes to the preferred one (the
forward pass's stash).  The bar is the one of the dedicated tests:
corruption and row lists bit for bit, loss 1e-3 relative, d_hidden and dW
1e-2 relative L2.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as WL
from uniform_noise_diffusion_amd import binding as B

from gpu_common import DEV, d_hidden_host, dev_float, dev_tokens, host, rel_l2, run_step
from test_gpu_corrupt_compact import _check
from test_gpu_dw import _oracle_rows, _run

pytestmark = pytest.mark.gpu


def _layout(rng, max_tokens):
    n_docs = int(rng.integers(1, 200))
    max_len = int(rng.integers(1, max(2, max_tokens // n_docs)))
    lengths = rng.integers(1, max_len + 1, size=n_docs)
    lengths[rng.random(n_docs) < rng.choice([0.0, 0.2])] = 0
    lengths[rng.random(n_docs) < 0.05] = 1
    cu = np.zeros(n_docs + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    return cu


@pytest.mark.parametrize("case", range(32))
def test_random_corruption_and_row_lists(case):
    rng = np.random.default_rng(1000 + case)
    cu = _layout(rng, 40000)
    V = int(rng.integers(2, 200000))
    x0 = rng.integers(0, V, size=int(cu[-1])).astype(np.int32)
    eps = float(rng.choice([1e-3, rng.random(), 1.0]))
    noise = int(rng.integers(0, 2))
    align = int(rng.integers(0, 2))
    seed = int(rng.integers(0, 2**63))
    _check(x0, cu, seed, eps, noise, int(rng.integers(0, V)), V, align)


@pytest.mark.parametrize("case", range(24))
def test_random_head(case):
    rng = np.random.default_rng(2000 + case)
    H = 64 * int(rng.integers(1, 9))
    V = int(rng.choice([int(rng.integers(1, 300)), int(rng.integers(300, 4000))]))
    softcap = float(rng.choice([0.0, 30.0, 4.0]))
    noise = int(rng.integers(0, 2))
    align = int(rng.integers(0, 2))
    inp = WL.small_case(3000 + case, n_docs=int(rng.integers(1, 8)),
                        max_len=int(rng.integers(20, 600)), H=H, V=max(V, 2),
                        noise=noise, align=align, softcap=softcap)
    n = inp.wl.n_tokens
    lo = B.mdlm_head_ce_workspace_min_bytes(n, H, inp.wl.V, B.MDLM_BF16)
    hi = B.mdlm_head_ce_workspace_bytes(n, H, inp.wl.V, B.MDLM_BF16)
    ws = int(rng.choice([lo, (lo + hi) // 2, hi]))
    eps = float(rng.choice([1e-3, 0.3, 1.0]))
    seed = int(rng.integers(0, 2**40))
    params = dict(seed=seed, eps=eps, align=align, softcap=softcap, noise=noise)
    s = run_step(inp, head_workspace_bytes=ws, **params)
    wl = inp.wl
    xt, corrupted, p, _ = oracle.corrupt(inp.x0, inp.cu_seqlens, seed, eps, noise, wl.mask_id,
                                         wl.rand_vocab)
    rows, tgt, w = oracle.compact(corrupted, inp.x0, inp.cu_seqlens, p, align)
    m = int(host(s.n_rows)[0])
    assert m == rows.shape[0]
    g_dh = d_hidden_host(s)
    if m == 0:
        assert float(host(s.loss)[0]) == 0.0 and np.all(g_dh == 0)
        return
    loss, ce, dh = oracle.head_ce(inp.hidden, inp.W, rows, tgt, w, softcap)
    assert abs(float(host(s.loss)[0]) - loss) <= 1e-3 * abs(loss)
    assert rel_l2(g_dh, dh) < 1e-2
    unscored = np.setdiff1d(np.arange(n), rows)
    assert np.all(g_dh[unscored] == 0.0)


@pytest.mark.parametrize("case", range(8))
def test_random_head_weight_gradient(case):
    rng = np.random.default_rng(4000 + case)
    H = 64 * int(rng.integers(1, 6))
    V = int(rng.integers(2, 2500))
    softcap = float(rng.choice([0.0, 30.0]))
    align = int(rng.integers(0, 2))
    inp = WL.small_case(5000 + case, n_docs=int(rng.integers(1, 6)),
                        max_len=int(rng.integers(50, 500)), H=H, V=V, softcap=softcap)
    min_ws = bool(rng.integers(0, 2))
    step, m, loss, row_ce, dh, dW = _run(inp, 11 + case, 0.5, align, softcap, min_ws=min_ws)
    rows, tgt, w = _oracle_rows(inp, 11 + case, 0.5, align)
    assert m == rows.shape[0]
    if m == 0:
        return
    want = oracle.head_ce_weight_grad(inp.hidden, inp.W, rows, tgt, w.astype(np.float32),
                                      softcap)
    assert rel_l2(host(dW), want) < 1e-2


@pytest.mark.parametrize("case", range(16))
def test_random_corrective_mixture(case):
    """Random layouts, mixture shares and token weights through
    mdlm_corrupt_mixture and mdlm_compact_corrective, bit for bit."""
    from test_gpu_corrective import _check as _check_corrective
    rng = np.random.default_rng(4000 + case)
    cu = _layout(rng, 40000)
    V = int(rng.integers(2, 200000))
    x0 = rng.integers(0, V, size=int(cu[-1])).astype(np.int32)
    eps = float(rng.choice([1e-3, rng.random(), 1.0]))
    mix = float(rng.choice([0.0, rng.random(), 1.0]))
    a = float(rng.choice([0.0, rng.random(), 1.0]))
    c = float(rng.choice([0.0, 0.0, rng.random()]))
    align = int(rng.integers(0, 2))
    seed = int(rng.integers(0, 2**63))
    _check_corrective(x0, cu, seed, eps, mix, align, a, c, int(rng.integers(0, V)), V)
