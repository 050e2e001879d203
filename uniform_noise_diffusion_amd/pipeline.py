"""Buffers for one training step of the loss path, and the three calls.

Plumbing only: torch allocates the device buffers once; each step enqueues
mdlm_corrupt, mdlm_compact_masked and mdlm_fused_head_ce_fwd_bwd on one
stream with no host synchronisation (the number of scored rows stays on the
device).  The hidden states would come from the model's forward on `xt`; here
they are an input.
"""

import torch

from . import binding as B


class MdlmLossStep:
    """Owns every buffer the three calls write for a stream of `n_tokens`
    tokens in `n_docs` documents, hidden size H and vocabulary V."""

    def __init__(self, n_tokens, n_docs, H, V, dtype=torch.bfloat16, device="cuda",
                 head_workspace_bytes=None, want_grad=True):
        self.n_tokens, self.n_docs, self.H, self.V = n_tokens, n_docs, H, V
        self.dtype = dtype
        dev = torch.device(device)
        i32 = dict(dtype=torch.int32, device=dev)
        self.xt = torch.empty(n_tokens, **i32)
        self.corrupted = torch.empty(n_tokens, dtype=torch.uint8, device=dev)
        self.p_doc = torch.empty(n_docs, dtype=torch.float64, device=dev)
        self.doc_counts = torch.empty(n_docs, **i32)
        self.row_idx = torch.empty(max(n_tokens, 1), **i32)
        self.tgt = torch.empty(max(n_tokens, 1), **i32)
        self.w = torch.empty(max(n_tokens, 1), dtype=torch.float32, device=dev)
        self.n_rows = torch.empty(1, **i32)
        self.compact_ws = torch.empty(max(B.mdlm_compact_workspace_bytes(n_tokens), 1),
                                      dtype=torch.uint8, device=dev)
        self.rows_ws = None
        self.loss = torch.empty(1, dtype=torch.float32, device=dev)
        self.row_ce = torch.empty(max(n_tokens, 1), dtype=torch.float32, device=dev)
        self.d_hidden = (torch.empty((n_tokens, H), dtype=dtype, device=dev)
                         if want_grad else None)
        code = B.dtype_code(torch.empty(0, dtype=dtype))
        if head_workspace_bytes is None:
            head_workspace_bytes = B.mdlm_head_ce_workspace_bytes(n_tokens, H, V, code)
        self.head_ws = torch.empty(max(head_workspace_bytes, 1), dtype=torch.uint8, device=dev)

    def corrupt(self, x0, cu_seqlens, seed, eps, noise, mask_id, rand_vocab, stream=None):
        B.mdlm_corrupt(x0, cu_seqlens, seed, eps, noise, mask_id, rand_vocab, self.xt,
                       self.corrupted, self.p_doc, self.doc_counts, stream)

    def compact(self, x0, cu_seqlens, align, stream=None):
        B.mdlm_compact_masked(self.corrupted, x0, cu_seqlens, self.p_doc, align, self.row_idx,
                              self.tgt, self.w, self.n_rows, self.compact_ws, stream)

    def corrupt_mixture(self, x0, cu_seqlens, seed, eps, mixture_prob, mask_id, rand_vocab,
                        stream=None):
        """mdlm_corrupt_mixture: `corrupted` then holds the codes (0 clean,
        1 masked, 2 replaced)."""
        B.mdlm_corrupt_mixture(x0, cu_seqlens, seed, eps, mixture_prob, mask_id, rand_vocab,
                               self.xt, self.corrupted, self.p_doc, self.doc_counts, stream)

    def compact_corrective(self, x0, cu_seqlens, align, noise_token_wt, clean_token_wt,
                           stream=None):
        """mdlm_compact_corrective over the codes of the last corrupt_mixture()."""
        B.mdlm_compact_corrective(self.corrupted, x0, cu_seqlens, self.p_doc, align,
                                  noise_token_wt, clean_token_wt, self.row_idx, self.tgt,
                                  self.w, self.n_rows, self.compact_ws, stream)

    def compact_rows(self, x0, cu_seqlens, align, weighting, weight_scale=1.0,
                     weight_clip=float("inf"), corrupted=True, eligible=None, stream=None):
        """mdlm_compact_rows into this step's row buffers: `corrupted` True uses
        the mask of the last corrupt() call, None scores every token;
        `eligible` is an optional uint8 mask."""
        need = B.mdlm_compact_rows_workspace_bytes(self.n_tokens, self.n_docs, weighting)
        if self.rows_ws is None or self.rows_ws.numel() < need:
            self.rows_ws = torch.empty(max(need, 1), dtype=torch.uint8, device=self.xt.device)
        mask = self.corrupted if corrupted is True else corrupted
        B.mdlm_compact_rows(mask, eligible, x0, cu_seqlens, self.p_doc, align, weighting,
                            weight_scale, weight_clip, self.row_idx, self.tgt, self.w,
                            self.n_rows, self.rows_ws, stream)

    def head_ce(self, hidden, W, softcap, stream=None, want_grad=True, row_ce=True):
        B.mdlm_fused_head_ce_fwd_bwd(hidden, W, self.row_idx, self.tgt, self.w, self.n_rows,
                                     self.n_tokens, softcap, self.loss,
                                     self.row_ce if row_ce else None,
                                     self.d_hidden if want_grad else None, self.head_ws,
                                     stream)

    def step(self, x0, cu_seqlens, hidden, W, seed, eps, noise, mask_id, rand_vocab, align,
             softcap, stream=None, want_grad=True, row_ce=True):
        self.corrupt(x0, cu_seqlens, seed, eps, noise, mask_id, rand_vocab, stream)
        self.compact(x0, cu_seqlens, align, stream)
        self.head_ce(hidden, W, softcap, stream, want_grad, row_ce)
