"""The fused head + CE call as a torch.autograd.Function.

LLaDA-8B-MDLM-LoRA card, Training table, "Objective" row: the masked-
diffusion loss is what the trainer backpropagates through (with the output
layer frozen, "LoRA" row).  `masked_diffusion_loss` returns that loss as a
0-dim tensor whose gradient flows into `hidden`, so it can sit inside any
larger expression (a sum with other loss terms, a scale by an accumulation
factor) before `.backward()`.

Marshalling only: the forward is one mdlm_fused_head_ce_fwd_bwd call, which
forms d_hidden for an upstream gradient of 1 along with the loss; the
backward is one mdlm_scale call, d_hidden times the upstream gradient, read
on the device (no host synchronisation).  The head W must be frozen
(requires_grad False); the head-weight gradient is available through
binding.mdlm_fused_head_ce_fwd_bwd_dw.
"""

import torch

from . import binding as B


class FusedHeadCE(torch.autograd.Function):
    """loss = sum_j w_j CE_j over the scored rows (see include/mdlm.h,
    mdlm_fused_head_ce_fwd_bwd); the gradient with respect to `hidden`."""

    @staticmethod
    def forward(ctx, hidden, W, row_idx, tgt, w, n_rows, max_rows, softcap, workspace):
        if W.requires_grad:
            raise ValueError("masked_diffusion_loss takes a frozen head (W.requires_grad "
                             "False); use mdlm_fused_head_ce_fwd_bwd_dw for a trained head")
        want = ctx.needs_input_grad[0]
        n_tokens, H = hidden.shape
        V = W.shape[0]
        if workspace is None:
            need = B.mdlm_head_ce_workspace_bytes(max_rows, H, V, B.dtype_code(hidden))
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=hidden.device)
        loss = torch.empty(1, dtype=torch.float32, device=hidden.device)
        d_hidden = torch.empty_like(hidden) if want else None
        B.mdlm_fused_head_ce_fwd_bwd(hidden, W, row_idx, tgt, w, n_rows, max_rows, softcap,
                                     loss, None, d_hidden, workspace)
        ctx.save_for_backward(d_hidden)
        return loss.view(())

    @staticmethod
    def backward(ctx, grad_loss):
        (d_hidden,) = ctx.saved_tensors
        if d_hidden is None:
            return (None,) * 9
        g = grad_loss.reshape(1)
        if g.dtype != torch.float32:
            g = g.float()
        out = torch.empty_like(d_hidden)
        B.mdlm_scale(d_hidden, out, g.contiguous())
        return (out,) + (None,) * 8


def masked_diffusion_loss(hidden, W, row_idx, tgt, w, n_rows, max_rows=None, softcap=0.0,
                          workspace=None):
    """The weighted CE of the scored rows (row list from mdlm_compact_masked
    or its variants) through the frozen head W, differentiable in `hidden`.

    hidden: [n_tokens, H] bf16 or float32 (contiguous, on the device);
    W: [V, H] of the same dtype; row_idx, tgt, w, n_rows: the row list;
    max_rows: host bound on *n_rows (default n_tokens); workspace: optional
    uint8 device tensor (default: the preferred size, allocated per call).
    Returns a 0-dim float32 tensor."""
    if max_rows is None:
        max_rows = hidden.shape[0]
    return FusedHeadCE.apply(hidden, W, row_idx, tgt, w, n_rows, int(max_rows), float(softcap),
                             workspace)
