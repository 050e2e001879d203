"""The three calls launch kernels only (no memset, no allocation, no host
synchronisation), so a whole step can be captured in a HIP graph.  The
captured step is replayed several times, with new hidden states written by
eager work between replays, and every replay must match an eager step on the
same inputs bit for bit."""

import numpy as np
import pytest
import torch

import workloads as WL

from gpu_common import DEV, dev_float, dev_tokens, host
from uniform_noise_diffusion_amd.pipeline import MdlmLossStep

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n_docs,max_len", [(1, 3000), (7, 900)])
def test_captured_step_replays_match_eager(n_docs, max_len):
    inp = WL.small_case(41 + n_docs, n_docs=n_docs, max_len=max_len, H=256, V=2600,
                        softcap=30.0)
    wl = inp.wl
    x0, cu = dev_tokens(inp)
    h, W = dev_float(inp)
    args = (wl.seed, wl.eps, wl.noise, wl.mask_id, wl.rand_vocab, wl.align, wl.softcap)
    step = MdlmLossStep(wl.n_tokens, wl.n_docs, wl.H, wl.V, dtype=torch.bfloat16, device=DEV)
    ref = MdlmLossStep(wl.n_tokens, wl.n_docs, wl.H, wl.V, dtype=torch.bfloat16, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step.step(x0, cu, h, W, *args)  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step.step(x0, cu, h, W, *args)
    gen = torch.Generator(device=DEV).manual_seed(0)
    for r in range(4):
        # new hidden states, written by eager work between replays
        h.copy_((torch.randn(h.shape, device=DEV, generator=gen) * (1 + r)).to(h.dtype))
        graph.replay()
        torch.cuda.synchronize()
        ref.step(x0, cu, h, W, *args)
        torch.cuda.synchronize()
        m = int(host(step.n_rows)[0])
        assert m == int(host(ref.n_rows)[0]) and m > 0
        assert np.array_equal(host(step.row_idx)[:m], host(ref.row_idx)[:m])
        assert np.array_equal(host(step.loss).view(np.uint32), host(ref.loss).view(np.uint32)), r
        assert np.array_equal(host(step.d_hidden.view(torch.int16)),
                              host(ref.d_hidden.view(torch.int16))), r
