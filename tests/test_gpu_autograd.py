"""GPU parity of the autograd wrapper (uniform_noise_diffusion_amd.autograd)
and of mdlm_scale, the call its backward makes.

The loss must equal the oracle's within 1e-3 relative and the gradient that
reaches `hidden` must be the upstream gradient times the oracle's d_hidden
within 1e-2 relative L2 (upstream gradients other than 1: a scale, a sum
with a second loss term, autograd.grad with explicit grad_outputs, a
backward repeated through a retained graph).  mdlm_scale itself is compared
bit for bit with torch's fp32 product rounded once to the output dtype.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as WL
from uniform_noise_diffusion_amd import binding as B
from uniform_noise_diffusion_amd.autograd import masked_diffusion_loss
from uniform_noise_diffusion_amd.pipeline import MdlmLossStep

from gpu_common import DEV, dev_float, dev_tokens, host, rel_l2

pytestmark = pytest.mark.gpu


def _rows(inp, seed, eps, align):
    """The library's row list for a seeded corruption (the oracle's, bit for
    bit, as the corruption tests establish) and the oracle's own."""
    wl = inp.wl
    x0, cu = dev_tokens(inp)
    step = MdlmLossStep(wl.n_tokens, wl.n_docs, wl.H, wl.V, dtype=torch.bfloat16, device=DEV,
                        head_workspace_bytes=0, want_grad=False)
    step.corrupt(x0, cu, seed, eps, wl.noise, wl.mask_id, wl.rand_vocab)
    step.compact(x0, cu, align)
    _, corrupted, p, _ = oracle.corrupt(inp.x0, inp.cu_seqlens, seed, eps, wl.noise,
                                        wl.mask_id, wl.rand_vocab)
    rows, tgt, w = oracle.compact(corrupted, inp.x0, inp.cu_seqlens, p, align)
    torch.cuda.synchronize()
    assert int(host(step.n_rows)[0]) == rows.shape[0]
    return step, (rows, tgt, w)


def _leaf(inp):
    h, W = dev_float(inp)
    return h.clone().requires_grad_(True), W


@pytest.mark.parametrize("upstream", [1.0, 3.7, -0.25])
@pytest.mark.parametrize("softcap", [0.0, 30.0])
def test_backward_scales_by_the_upstream_gradient(upstream, softcap):
    inp = WL.small_case(5, n_docs=4, max_len=300, H=128, V=1500, softcap=softcap)
    step, (rows, tgt, w) = _rows(inp, 3, 0.5, oracle.ALIGNED)
    h, W = _leaf(inp)
    loss = masked_diffusion_loss(h, W, step.row_idx, step.tgt, step.w, step.n_rows,
                                 softcap=softcap)
    (loss * upstream).backward()
    o_loss, _, o_dh = oracle.head_ce(inp.hidden, inp.W, rows, tgt, w, softcap)
    assert loss.dim() == 0
    assert abs(float(loss.detach()) - o_loss) <= 1e-3 * abs(o_loss)
    g = h.grad.float().cpu().numpy()
    assert rel_l2(g, upstream * o_dh) < 1e-2
    unscored = np.setdiff1d(np.arange(inp.wl.n_tokens), rows)
    assert np.all(g[unscored] == 0.0)


def test_sum_of_two_loss_terms_and_autograd_grad():
    # a diffusion term (masked rows, aligned) plus lambda times an every-token
    # causal term on the same hidden states: the gradient is the sum
    inp = WL.small_case(8, n_docs=3, max_len=250, H=64, V=900)
    wl = inp.wl
    step, (rows, tgt, w) = _rows(inp, 11, 0.4, oracle.ALIGNED)
    x0, cu = dev_tokens(inp)
    ar = MdlmLossStep(wl.n_tokens, wl.n_docs, wl.H, wl.V, dtype=torch.bfloat16, device=DEV,
                      head_workspace_bytes=0, want_grad=False)
    ar.compact_rows(x0, cu, oracle.SHIFTED, B.MDLM_WEIGHT_MEAN, 1.0, corrupted=None)
    h, W = _leaf(inp)
    lam = 0.3
    total = (masked_diffusion_loss(h, W, step.row_idx, step.tgt, step.w, step.n_rows) +
             lam * masked_diffusion_loss(h, W, ar.row_idx, ar.tgt, ar.w, ar.n_rows))
    (gh,) = torch.autograd.grad(total, h, grad_outputs=torch.tensor(-2.5, device=DEV))
    r2, t2, w2 = oracle.compact_rows(inp.x0, inp.cu_seqlens, oracle.SHIFTED,
                                     weighting=oracle.WEIGHT_MEAN)
    l1, _, d1 = oracle.head_ce(inp.hidden, inp.W, rows, tgt, w)
    l2, _, d2 = oracle.head_ce(inp.hidden, inp.W, r2, t2, w2)
    assert abs(float(total.detach()) - (l1 + lam * l2)) <= 1e-3 * abs(l1 + lam * l2)
    assert rel_l2(gh.float().cpu().numpy(), -2.5 * (d1 + lam * d2)) < 1e-2


def test_backward_through_a_retained_graph_twice():
    inp = WL.small_case(9, n_docs=2, max_len=200, H=64, V=700)
    step, (rows, tgt, w) = _rows(inp, 4, 0.6, oracle.SHIFTED)
    h, W = _leaf(inp)
    loss = masked_diffusion_loss(h, W, step.row_idx, step.tgt, step.w, step.n_rows)
    (2.0 * loss).backward(retain_graph=True)
    first = h.grad.clone()
    (2.0 * loss).backward()
    # the second backward adds the same gradient again (nothing scaled twice)
    assert torch.equal(h.grad.float(), 2.0 * first.float())
    _, _, o_dh = oracle.head_ce(inp.hidden, inp.W, rows, tgt, w)
    assert rel_l2(first.float().cpu().numpy(), 2.0 * o_dh) < 1e-2


def test_no_gradient_wanted_and_frozen_head_required():
    inp = WL.small_case(10, n_docs=2, max_len=100, H=64, V=300)
    step, (rows, tgt, w) = _rows(inp, 5, 0.7, oracle.ALIGNED)
    h, W = dev_float(inp)
    with torch.no_grad():
        loss = masked_diffusion_loss(h, W, step.row_idx, step.tgt, step.w, step.n_rows)
    o_loss, _, _ = oracle.head_ce(inp.hidden, inp.W, rows, tgt, w, want_grad=False)
    assert abs(float(loss) - o_loss) <= 1e-3 * abs(o_loss)
    with pytest.raises(ValueError, match="frozen head"):
        masked_diffusion_loss(h.clone().requires_grad_(True), W.clone().requires_grad_(True),
                              step.row_idx, step.tgt, step.w, step.n_rows)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("n", [0, 1, 7, 8, 4096 * 4096 + 3])
def test_scale_matches_torch_bit_for_bit(dtype, n):
    g = torch.Generator(device=DEV).manual_seed(n)
    x = torch.randn(n, generator=g, device=DEV).to(dtype)
    for s in (1.0, -3.3, 0.0):
        scale = torch.tensor([s], dtype=torch.float32, device=DEV)
        y = torch.empty_like(x)
        B.mdlm_scale(x, y, scale)
        want = (x.float() * s).to(dtype)
        assert torch.equal(y.view(torch.int16 if dtype == torch.bfloat16 else torch.int32),
                           want.view(torch.int16 if dtype == torch.bfloat16 else torch.int32))
    # in place
    scale = torch.tensor([0.5], dtype=torch.float32, device=DEV)
    want = (x.float() * 0.5).to(dtype)
    B.mdlm_scale(x, x, scale)
    assert torch.equal(x.float(), want.float())
