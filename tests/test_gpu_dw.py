"""GPU parity of the head-weight gradient (mdlm_fused_head_ce_fwd_bwd_dw).

Small and multi-tile cases compare dW with the oracle's fp64 gradient (1e-2
relative L2, the d_hidden bar; both products take bf16-rounded per-logit
factors).  The call's loss, row CE and d_hidden must be bit-identical to those
of mdlm_fused_head_ce_fwd_bwd.  At full size (llada8b-1x4096) 640 vocabulary
rows of dW -- the targets of scored rows, the vocabulary's first and last
rows and a random sample -- are compared with the oracle's, which forms
exactly those rows (after its full log-sum-exp pass), each row on its own
within 1e-2 relative L2; and two identities that hold at any size are
checked, to within the bf16 rounding of those factors:
<dW, W> = <d_hidden, hidden> (both equal sum_jv G_jv z_jv) and, with no
softcap, sum_v dW_v = 0 (each row's softmax minus one-hot sums to zero).
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as WL
from uniform_noise_diffusion_amd import binding as B
from uniform_noise_diffusion_amd.pipeline import MdlmLossStep

from gpu_common import DEV, dev_float, dev_tokens, far_row_case, host, rel_l2

pytestmark = pytest.mark.gpu

DW_RTOL = 1e-2


def _run(inp, seed, eps, align, softcap, min_ws=False, want_dh=True):
    """corrupt + compact, then the plain call and the dW call on the same rows."""
    wl = inp.wl
    x0, cu = dev_tokens(inp)
    h, W = dev_float(inp)
    step = MdlmLossStep(wl.n_tokens, wl.n_docs, wl.H, wl.V, dtype=torch.bfloat16, device=DEV)
    step.corrupt(x0, cu, seed, eps, wl.noise, wl.mask_id, wl.rand_vocab)
    step.compact(x0, cu, align)
    step.head_ce(h, W, softcap)
    n = wl.n_tokens
    ws_fn = (B.mdlm_head_ce_dw_workspace_min_bytes if min_ws
             else B.mdlm_head_ce_dw_workspace_bytes)
    ws = torch.empty(ws_fn(n, wl.H, wl.V), dtype=torch.uint8, device=DEV)
    dW = torch.full((wl.V, wl.H), float("nan"), dtype=torch.float32, device=DEV)
    loss = torch.empty(1, dtype=torch.float32, device=DEV)
    row_ce = torch.empty(n, dtype=torch.float32, device=DEV)
    dh = torch.empty_like(h) if want_dh else None
    B.mdlm_fused_head_ce_fwd_bwd_dw(h, W, step.row_idx, step.tgt, step.w, step.n_rows, n,
                                    softcap, loss, row_ce, dh, dW, ws)
    torch.cuda.synchronize()
    m = int(host(step.n_rows)[0])
    return step, m, loss, row_ce, dh, dW


def _oracle_rows(inp, seed, eps, align):
    wl = inp.wl
    _, corrupted, p, _ = oracle.corrupt(inp.x0, inp.cu_seqlens, seed, eps, wl.noise,
                                        wl.mask_id, wl.rand_vocab)
    return oracle.compact(corrupted, inp.x0, inp.cu_seqlens, p, align)


@pytest.mark.parametrize("H,V", [(64, 1000), (192, 300), (320, 2600), (256, 4096)])
@pytest.mark.parametrize("align", [oracle.ALIGNED, oracle.SHIFTED])
@pytest.mark.parametrize("softcap", [0.0, 30.0])
def test_dw_small_tiles_and_ragged_tails(H, V, align, softcap):
    # ~300-700 scored rows (K = rows: several 64-row steps, ragged); V with a
    # ragged 256-wide tile; H a multiple of 64 but not always of 256
    inp = WL.small_case(H + V + 7, n_docs=6, max_len=250, H=H, V=V, softcap=softcap)
    step, m, loss, row_ce, dh, dW = _run(inp, 5, 0.6, align, softcap)
    # the same loss, row CE and d_hidden as the plain call, bit for bit
    assert host(loss)[0] == host(step.loss)[0]
    assert np.array_equal(host(row_ce)[:m], host(step.row_ce)[:m])
    assert torch.equal(dh, step.d_hidden)
    rows, tgt, w = _oracle_rows(inp, 5, 0.6, align)
    assert m == rows.shape[0] and m > 64
    want = oracle.head_ce_weight_grad(inp.hidden, inp.W, rows, tgt, w.astype(np.float32), softcap)
    assert rel_l2(host(dW), want) < DW_RTOL


@pytest.mark.parametrize("want_dh", [True, False])
def test_dw_with_rows_far_from_their_target(want_dh):
    # rows whose largest logit is ~100 nats above the target's: the forward
    # pass keeps them relative to their half-tile maxima (see the head tests)
    inp, _ = far_row_case(43, H=192, V=2000, beta=100.0, philox_seed=3, eps=0.5,
                          align=oracle.ALIGNED)
    step, m, loss, row_ce, dh, dW = _run(inp, 3, 0.5, oracle.ALIGNED, 0.0, want_dh=want_dh)
    assert host(loss)[0] == host(step.loss)[0]
    if want_dh:
        assert torch.equal(dh, step.d_hidden)
    rows, tgt, w = _oracle_rows(inp, 3, 0.5, oracle.ALIGNED)
    assert m == rows.shape[0]
    want = oracle.head_ce_weight_grad(inp.hidden, inp.W, rows, tgt, w.astype(np.float32))
    assert rel_l2(host(dW), want) < DW_RTOL


def test_dw_with_the_minimal_workspace_and_no_d_hidden():
    # 256-wide vocabulary chunks: dW rows of every chunk are written
    inp = WL.small_case(77, n_docs=4, max_len=300, H=128, V=1300)
    step, m, loss, row_ce, dh, dW = _run(inp, 9, 0.5, oracle.SHIFTED, 0.0, min_ws=True,
                                         want_dh=False)
    assert dh is None and host(loss)[0] == host(step.loss)[0]
    rows, tgt, w = _oracle_rows(inp, 9, 0.5, oracle.SHIFTED)
    want = oracle.head_ce_weight_grad(inp.hidden, inp.W, rows, tgt, w.astype(np.float32))
    assert rel_l2(host(dW), want) < DW_RTOL


def test_dw_is_zero_without_scored_rows():
    # eps tiny and one short document: with this seed no token is corrupted
    inp = WL.small_case(3, n_docs=1, max_len=3, H=64, V=500)
    for seed in range(200):
        _, corrupted, _, _ = oracle.corrupt(inp.x0, inp.cu_seqlens, seed, 1e-6, 0,
                                            inp.wl.mask_id, inp.wl.rand_vocab)
        if not corrupted.any():
            break
    step, m, loss, row_ce, dh, dW = _run(inp, seed, 1e-6, oracle.ALIGNED, 0.0)
    assert m == 0 and host(loss)[0] == 0.0
    assert torch.count_nonzero(dW) == 0


def test_dw_full_size_sampled_vocabulary_rows():
    inp = WL.generate(WL.make_workload(2))
    wl = inp.wl
    print(f"full-size dW, workload {wl.name}", flush=True)
    step, m, loss, row_ce, dh, dW = _run(inp, 0, wl.eps, wl.align, wl.softcap)
    rows, tgt, w = _oracle_rows(inp, 0, wl.eps, wl.align)
    assert rows.shape[0] == m and m > 0
    rng = np.random.default_rng(2)
    pick = np.unique(np.concatenate([
        rng.choice(np.unique(tgt), size=min(256, np.unique(tgt).shape[0]), replace=False),
        rng.choice(wl.V, size=380, replace=False), [0, 1, wl.V - 2, wl.V - 1]]))
    want = oracle.head_ce_weight_grad(inp.hidden, inp.W, rows, tgt, w.astype(np.float32),
                                      wl.softcap, v_rows=pick)
    got = host(dW[torch.from_numpy(pick).to(DEV)]).astype(np.float64)
    assert rel_l2(got, want) < DW_RTOL
    row_err = np.linalg.norm(got - want, axis=1) / np.linalg.norm(want, axis=1)
    print(f"  {pick.shape[0]} vocabulary rows: rel-L2 {rel_l2(got, want):.2e}, "
          f"worst row {row_err.max():.2e}", flush=True)
    assert row_err.max() < DW_RTOL, (int(pick[row_err.argmax()]), float(row_err.max()))


@pytest.mark.parametrize("k", [2, 5])
def test_dw_full_size_identities(k):
    """llada8b-1x4096 (V=126,464, H=4,096) and diffusiongemma-canvas-8x1024
    (V=262,144, H=2,816, softcap 30) at full size."""
    inp = WL.generate(WL.make_workload(k))
    wl = inp.wl
    step, m, loss, row_ce, dh, dW = _run(inp, 0, wl.eps, wl.align, wl.softcap)
    assert m > 0 and torch.isfinite(dW).all()
    h, W = dev_float(inp)
    lhs = float((dW.double() * W.double()).sum())
    rhs = float((dh.double() * h.double()).sum())
    assert abs(lhs - rhs) <= 2e-3 * max(abs(lhs), abs(rhs))
    if wl.softcap == 0.0:
        col = dW.double().sum(dim=0)
        assert float(col.norm()) <= 1e-2 * float(dW.double().norm())
    # the most frequent target's row of dW: its rows contribute -w_j h_j each,
    # every other term is w_j p_jv h_j with p_jv ~ 1/V, so the row points
    # along -sum_j w_j h_j over the rows with that target (rows, targets and
    # weights from the oracle's own corruption and compaction)
    rows, tgt, w = _oracle_rows(inp, 0, wl.eps, wl.align)
    assert rows.shape[0] == m
    v = int(np.bincount(tgt).argmax())
    sel = tgt == v
    ref = -(w[sel, None] * inp.hidden[rows[sel]].astype(np.float64)).sum(0)
    got = host(dW[v]).astype(np.float64)
    cos = float(got @ ref / (np.linalg.norm(got) * np.linalg.norm(ref)))
    assert cos > 0.9
