"""Every call runs on the stream it is given.  A whole step on a side stream
(default priority) gives bit for bit what it gives on the default stream, and
two steps with their own buffers on two streams at once give what each gives
alone (the library holds no state shared between calls)."""

import numpy as np
import pytest
import torch

import workloads as WL

from gpu_common import DEV, dev_float, dev_tokens, host, run_step
from uniform_noise_diffusion_amd.pipeline import MdlmLossStep

pytestmark = pytest.mark.gpu


def _outputs(step):
    m = int(host(step.n_rows)[0])
    return dict(xt=host(step.xt), corrupted=host(step.corrupted), p=host(step.p_doc),
                counts=host(step.doc_counts), rows=host(step.row_idx)[:m],
                tgt=host(step.tgt)[:m], w=host(step.w)[:m], loss=host(step.loss),
                dh=host(step.d_hidden.view(torch.int16)))


def _same(a, b):
    for k in a:
        assert np.array_equal(np.asarray(a[k]).view(np.uint8), np.asarray(b[k]).view(np.uint8)), k


def _step_on(inp, stream, seed):
    wl = inp.wl
    x0, cu = dev_tokens(inp)
    h, W = dev_float(inp)
    step = MdlmLossStep(wl.n_tokens, wl.n_docs, wl.H, wl.V, dtype=torch.bfloat16, device=DEV)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        step.step(x0, cu, h, W, seed, wl.eps, wl.noise, wl.mask_id, wl.rand_vocab, wl.align,
                  wl.softcap, stream=stream)
    return step


def test_side_stream_matches_default_stream():
    inp = WL.small_case(31, n_docs=6, max_len=700, H=256, V=3000, softcap=30.0)
    ref = _outputs(run_step(inp, seed=5))
    side = torch.cuda.Stream()
    step = _step_on(inp, side, 5)
    side.synchronize()
    _same(ref, _outputs(step))


def test_two_streams_at_once():
    a = WL.small_case(32, n_docs=5, max_len=900, H=320, V=2500)
    b = WL.small_case(33, n_docs=9, max_len=400, H=192, V=4100, noise=WL.NOISE_UNIFORM,
                      align=WL.SHIFTED)
    ref_a = _outputs(run_step(a, seed=7))
    ref_b = _outputs(run_step(b, seed=8))
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for _ in range(3):
        sa = _step_on(a, s1, 7)
        sb = _step_on(b, s2, 8)
        s1.synchronize()
        s2.synchronize()
        _same(ref_a, _outputs(sa))
        _same(ref_b, _outputs(sb))
