"""GPU parity of mdlm_corrupt_compact (corruption and the row list in one
call, the compaction sized by the corruption's per-tile counts) against the
oracle: every output bit for bit (xt, corrupted, p_doc's
fp64 bits, doc_counts, n_rows, row_idx, tgt, w's fp32 bits), on the layouts
the two-call tests use (tiny and empty documents, documents spanning tiles,
more documents per tile than it caches, one-tile streams, many tiles), on the
named workloads, with a reused workspace, on unaligned buffers and without
the mask output.  At 2^27 tokens (the bandwidth shape: documents of 4,096
and lognormal documents of mean 296) the fused call is compared bit for bit
with the two-call path, which the other tests pin to the oracle.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as WL
from uniform_noise_diffusion_amd import binding as B
from uniform_noise_diffusion_amd.pipeline import MdlmLossStep

from gpu_common import DEV, host

pytestmark = pytest.mark.gpu

i32 = dict(dtype=torch.int32, device=DEV)


def _case(seed, n_docs, max_len, empty=False, V=1000):
    rng = np.random.default_rng(seed)
    lengths = rng.integers(1, max_len + 1, size=n_docs)
    if empty:
        lengths[rng.random(n_docs) < 0.3] = 0
    cu = np.zeros(n_docs + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    x0 = rng.integers(0, V - 1, size=int(cu[-1])).astype(np.int32)
    return x0, cu


class Out:
    """Output buffers of one fused call, filled with sentinels; `offset`
    shifts every buffer off its allocation's alignment (the scalar paths)."""

    def __init__(self, n, nd, offset=0, mask=True):
        def buf(k, dtype, fill):
            return torch.full((k + offset,), fill, dtype=dtype, device=DEV)[offset:]
        self.xt = buf(n, torch.int32, -5)
        self.corrupted = buf(n, torch.uint8, 7) if mask else None
        self.p_doc = torch.full((nd,), -1.0, dtype=torch.float64, device=DEV)
        self.doc_counts = torch.full((nd,), -9, **i32)
        self.row_idx = buf(max(n, 1), torch.int32, -3)
        self.tgt = buf(max(n, 1), torch.int32, -3)
        self.w = buf(max(n, 1), torch.float32, float("nan"))
        self.n_rows = torch.full((1,), -7, **i32)


def _fused(x0, cu, seed, eps, noise, mask_id, rand_vocab, align, out=None, ws=None, offset=0,
           mask=True):
    n, nd = x0.shape[0], cu.shape[0] - 1
    tx0 = torch.full((n + offset,), 0, **i32)[offset:]
    tx0.copy_(torch.from_numpy(x0))
    tcu = torch.from_numpy(cu).to(DEV)
    out = out or Out(n, nd, offset, mask)
    if ws is None:
        ws = torch.empty(max(B.mdlm_corrupt_compact_workspace_bytes(n), 1), dtype=torch.uint8,
                         device=DEV)
    B.mdlm_corrupt_compact(tx0, tcu, seed, eps, noise, mask_id, rand_vocab, align, out.xt,
                           out.corrupted, out.p_doc, out.doc_counts, out.row_idx, out.tgt, out.w,
                           out.n_rows, ws)
    torch.cuda.synchronize()
    return out


def _check(x0, cu, seed, eps, noise, mask_id, rand_vocab, align, **kw):
    o = _fused(x0, cu, seed, eps, noise, mask_id, rand_vocab, align, **kw)
    xt, corrupted, p, counts = oracle.corrupt(x0, cu, seed, eps, noise, mask_id, rand_vocab)
    assert np.array_equal(host(o.xt), xt)
    if o.corrupted is not None:
        assert np.array_equal(host(o.corrupted), corrupted)
    assert np.array_equal(host(o.p_doc).view(np.uint64), p.view(np.uint64))
    assert np.array_equal(host(o.doc_counts), counts)
    rows, tgt, w = oracle.compact(corrupted, x0, cu, p, align)
    m = int(host(o.n_rows)[0])
    assert m == rows.shape[0]
    assert np.array_equal(host(o.row_idx)[:m], rows)
    assert np.array_equal(host(o.tgt)[:m], tgt)
    assert np.array_equal(host(o.w)[:m].view(np.uint32), w.astype(np.float32).view(np.uint32))
    # nothing written past the list
    assert np.all(host(o.row_idx)[m:] == -3)
    return o


@pytest.mark.parametrize("noise", [oracle.NOISE_ABSORB, oracle.NOISE_UNIFORM])
@pytest.mark.parametrize("align", [oracle.ALIGNED, oracle.SHIFTED])
@pytest.mark.parametrize("seed,n_docs,max_len,empty", [
    (1, 1, 7, False),        # a single tiny document, N not a multiple of 4
    (2, 40, 300, True),      # empty documents, several tiles
    (3, 7, 3000, False),     # documents spanning tile boundaries
    (4, 600, 20, True),      # many short documents per tile
    (5, 5000, 2, True),      # more documents per 4096-token tile than it caches
    (10, 2000, 2, True),     # one tile, more documents than it caches
    (11, 512, 8, False),     # one tile holding exactly as many documents as it caches
    (12, 300, 600, False),   # tens of tiles, documents of a few hundred tokens
])
def test_fused_bit_exact_small(noise, align, seed, n_docs, max_len, empty):
    x0, cu = _case(seed, n_docs, max_len, empty)
    _check(x0, cu, seed * 7919 + 13, 1e-3, noise, 999, 1000, align)


@pytest.mark.parametrize("eps", [1.0, 0.5, 1e-6])
def test_fused_eps_extremes(eps):
    x0, cu = _case(9, 20, 500)
    o = _check(x0, cu, 2**63 + 12345, eps, oracle.NOISE_ABSORB, 999, 1000, oracle.SHIFTED)
    if eps == 1.0:
        assert np.all(host(o.corrupted) == 1)


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("align", [oracle.ALIGNED, oracle.SHIFTED])
def test_fused_bit_exact_workloads(k, align):
    wl = WL.make_workload(k)
    inp = WL.generate(wl, with_hidden=False, with_head=False)
    for seed in (wl.seed, 1, 2):
        _check(inp.x0, inp.cu_seqlens, seed, wl.eps, wl.noise, wl.mask_id, wl.rand_vocab, align)


def test_fused_reused_workspace_and_buffers():
    """Three calls in a row on one workspace and one set of outputs, the
    stream shrinking and growing: the tile counts of each call start clean."""
    x_big, cu_big = _case(21, 400, 900)
    x_small, cu_small = _case(22, 30, 700)
    n = x_big.shape[0]
    ws = torch.empty(B.mdlm_corrupt_compact_workspace_bytes(n), dtype=torch.uint8, device=DEV)
    for (x0, cu, seed) in ((x_big, cu_big, 1), (x_small, cu_small, 2), (x_big, cu_big, 3)):
        _check(x0, cu, seed, 1e-3, oracle.NOISE_ABSORB, 999, 1000, oracle.ALIGNED, ws=ws)


@pytest.mark.parametrize("offset", [1, 3])
def test_fused_unaligned_buffers_and_no_mask(offset):
    x0, cu = _case(23, 60, 400, empty=True)
    _check(x0, cu, 77, 1e-3, oracle.NOISE_UNIFORM, 999, 1000, oracle.SHIFTED, offset=offset)
    _check(x0, cu, 78, 1e-3, oracle.NOISE_ABSORB, 999, 1000, oracle.ALIGNED, mask=False)


def test_fused_empty_stream():
    x0 = np.zeros(0, dtype=np.int32)
    cu = np.zeros(3, dtype=np.int32)
    o = _fused(x0, cu, 5, 1e-3, 0, 1, 2, oracle.ALIGNED)
    assert int(host(o.n_rows)[0]) == 0
    _, _, p, counts = oracle.corrupt(x0, cu, 5, 1e-3, 0, 1, 2)
    assert np.array_equal(host(o.p_doc).view(np.uint64), p.view(np.uint64))
    assert np.all(host(o.doc_counts) == 0)


def _two_call(x0, cu, seed, align):
    n, nd = x0.numel(), cu.numel() - 1
    s = MdlmLossStep(n, nd, 64, 64, device=DEV, head_workspace_bytes=0, want_grad=False)
    s.corrupt(x0, cu, seed, 1e-3, oracle.NOISE_ABSORB, 126336, 126464)
    s.compact(x0, cu, align)
    return s


@pytest.mark.parametrize("layout", ["docs4096", "lognormal296"])
def test_fused_equals_two_calls_at_bandwidth_size(layout):
    n = 1 << 27
    if layout == "docs4096":
        cu = torch.arange(0, n + 1, 4096, dtype=torch.int32, device=DEV)
    else:
        cu = torch.from_numpy(
            WL.lognormal_stream_offsets(5296, 296, n).astype(np.int32)).to(DEV)
    print(f"2^27 tokens, {layout}: {cu.numel() - 1} documents", flush=True)
    g = torch.Generator(device=DEV).manual_seed(0)
    x0 = torch.randint(0, 126336, (n,), dtype=torch.int32, device=DEV, generator=g)
    nd = cu.numel() - 1
    ws = torch.empty(B.mdlm_corrupt_compact_workspace_bytes(n), dtype=torch.uint8, device=DEV)
    for seed, align in ((11, oracle.ALIGNED), (12, oracle.SHIFTED)):
        ref = _two_call(x0, cu, seed, align)
        o = Out(n, nd)
        B.mdlm_corrupt_compact(x0, cu, seed, 1e-3, oracle.NOISE_ABSORB, 126336, 126464, align,
                               o.xt, o.corrupted, o.p_doc, o.doc_counts, o.row_idx, o.tgt, o.w,
                               o.n_rows, ws)
        torch.cuda.synchronize()
        m = int(ref.n_rows.item())
        assert int(o.n_rows.item()) == m and m > 0
        assert torch.equal(o.xt, ref.xt) and torch.equal(o.corrupted, ref.corrupted)
        assert torch.equal(o.p_doc.view(torch.int64), ref.p_doc.view(torch.int64))
        assert torch.equal(o.doc_counts, ref.doc_counts)
        assert torch.equal(o.row_idx[:m], ref.row_idx[:m])
        assert torch.equal(o.tgt[:m], ref.tgt[:m])
        assert torch.equal(o.w[:m].view(torch.int32), ref.w[:m].view(torch.int32))
        del ref, o


def _random_layout(rng, max_tokens):
    n_docs = int(rng.integers(1, 300))
    max_len = int(rng.integers(1, max(2, max_tokens // n_docs)))
    lengths = rng.integers(1, max_len + 1, size=n_docs)
    lengths[rng.random(n_docs) < rng.choice([0.0, 0.2])] = 0
    lengths[rng.random(n_docs) < 0.05] = 1
    cu = np.zeros(n_docs + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    return cu


@pytest.mark.parametrize("case", range(24))
def test_fused_random_sweep(case):
    """Seeded random layouts (empty and one-token documents, one to tens of
    tiles), both noise modes and alignments, eps from 1e-3 to 1, with and
    without the mask output: bit for bit against the oracle."""
    rng = np.random.default_rng(5000 + case)
    cu = _random_layout(rng, 60000)
    V = int(rng.integers(2, 200000))
    x0 = rng.integers(0, V, size=int(cu[-1])).astype(np.int32)
    eps = float(rng.choice([1e-3, rng.random(), 1.0]))
    noise = int(rng.integers(0, 2))
    align = int(rng.integers(0, 2))
    seed = int(rng.integers(0, 2**63))
    mask = bool(rng.integers(0, 2))
    _check(x0, cu, seed, eps, noise, int(rng.integers(0, V)), V, align, mask=mask)


@pytest.mark.parametrize("align", [oracle.ALIGNED, oracle.SHIFTED])
def test_fused_documents_on_tile_boundaries(align):
    """Every document starts on a 4096-token tile boundary and every token is
    corrupted (eps = 1): with shifted rows each tile's count loses exactly
    its first token."""
    cu = np.arange(0, 4096 * 9 + 1, 4096, dtype=np.int32)
    cu = np.concatenate([cu, [cu[-1] + 100]]).astype(np.int32)  # a ragged last tile
    x0 = np.random.default_rng(7).integers(0, 999, size=int(cu[-1])).astype(np.int32)
    o = _check(x0, cu, 99, 1.0, oracle.NOISE_ABSORB, 999, 1000, align)
    n = int(cu[-1])
    assert int(host(o.n_rows)[0]) == (n - (cu.shape[0] - 1) if align == oracle.SHIFTED else n)
