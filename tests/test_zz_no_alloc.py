"""GPU test of mdlm_compact_masked_noalloc, the compaction that takes no
workspace (its scratch is a device array inside the library), against
mdlm_compact_masked with a caller workspace: rows, targets, weight bits and
the row count bit for bit, on two calls in a row through the C ABI, the
second on a smaller stream (the array keeps the first call's contents), and
a stream past the array's limit refused on the host.
"""

import ctypes

import numpy as np
import pytest
import torch

import workloads as WL
from uniform_noise_diffusion_amd import binding as B

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _lib():
    lib = B.load()
    f = lib.mdlm_compact_masked_noalloc
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    f.argtypes = [vp, vp, i64, vp, i32, vp, i32, vp, vp, vp, vp, vp]
    f.restype = ctypes.c_int
    return lib


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def _stream(n, mean, seed):
    """A corrupted stream of n tokens in lognormal documents of the given mean
    length: tokens, offsets, corruption mask and noise levels (from
    mdlm_corrupt)."""
    cu = torch.from_numpy(WL.lognormal_stream_offsets(seed, mean, n).astype(np.int32)).to(DEV)
    g = torch.Generator(device=DEV).manual_seed(seed)
    x0 = torch.randint(0, 126336, (n,), dtype=torch.int32, device=DEV, generator=g)
    nd = cu.numel() - 1
    xt = torch.empty_like(x0)
    corrupted = torch.empty(n, dtype=torch.uint8, device=DEV)
    p = torch.empty(nd, dtype=torch.float64, device=DEV)
    counts = torch.empty(nd, dtype=torch.int32, device=DEV)
    B.mdlm_corrupt(x0, cu, seed, 1e-3, B.MDLM_NOISE_ABSORB, 126336, 126464, xt, corrupted, p,
                   counts)
    return x0, cu, corrupted, p


def _outputs(n):
    i32 = dict(dtype=torch.int32, device=DEV)
    return (torch.full((n,), -1, **i32), torch.full((n,), -1, **i32),
            torch.full((n,), float("nan"), dtype=torch.float32, device=DEV),
            torch.full((1,), -1, **i32))


@pytest.mark.parametrize("align", [B.MDLM_ALIGNED, B.MDLM_SHIFTED])
def test_noalloc_matches_the_workspace_call_twice(align):
    lib = _lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for n, mean, seed in ((1 << 22, 296, 5), (30_001, 512, 6)):
        x0, cu, corrupted, p = _stream(n, mean, seed)
        nd = cu.numel() - 1
        r0, t0, w0, m0 = _outputs(n)
        ws = torch.empty(B.mdlm_compact_workspace_bytes(n), dtype=torch.uint8, device=DEV)
        B.mdlm_compact_masked(corrupted, x0, cu, p, align, r0, t0, w0, m0, ws)
        r1, t1, w1, m1 = _outputs(n)
        rc = lib.mdlm_compact_masked_noalloc(_p(corrupted), _p(x0), n, _p(cu), nd, _p(p), align,
                                             _p(r1), _p(t1), _p(w1), _p(m1), stream)
        assert rc == B.MDLM_OK, B.mdlm_last_error()
        torch.cuda.synchronize()
        m = int(m0.item())
        assert m > 0 and int(m1.item()) == m
        assert torch.equal(r0[:m], r1[:m]) and torch.equal(t0[:m], t1[:m])
        assert torch.equal(w0[:m].view(torch.int32), w1[:m].view(torch.int32))
        # nothing written past the row count
        assert torch.all(r1[m:] == -1)


def test_noalloc_refuses_streams_past_its_scratch():
    lib = _lib()
    n = (1 << 28) + 1
    # every pointer null: the size check comes first and nothing is launched
    rc = lib.mdlm_compact_masked_noalloc(None, None, n, None, 1, None, 0, None, None, None, None,
                                         None)
    assert rc == B.MDLM_EUNSUPPORTED
    assert "exceeds" in B.mdlm_last_error()
