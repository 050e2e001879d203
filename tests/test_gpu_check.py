"""GPU tests of the device-side precondition checks and of checking mode.

Every invalid input here is built on the host and only ever read by the
check kernels: in checking mode a call whose inputs fail returns
MDLM_EINVAL before enqueueing its own work (its outputs keep the sentinel
values written beforehand), so no kernel of the loss path sees them.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as WL
from uniform_noise_diffusion_amd import binding as B
from uniform_noise_diffusion_amd.pipeline import MdlmLossStep

from gpu_common import DEV, dev_float, dev_tokens, host, run_step

pytestmark = pytest.mark.gpu

i32 = dict(dtype=torch.int32, device=DEV)


def _status():
    return torch.zeros(1, **i32)


def _offsets_bits(cu, n):
    st = _status()
    B.mdlm_check_offsets(torch.tensor(cu, **i32), n, st)
    torch.cuda.synchronize()
    return int(st.item())


def test_offsets():
    assert _offsets_bits([0, 5, 5, 9], 9) == 0
    assert _offsets_bits([0], 0) == 0
    assert _offsets_bits([1, 5, 9], 9) == B.MDLM_CHECK_OFFSETS      # not from 0
    assert _offsets_bits([0, 5, 8], 9) == B.MDLM_CHECK_OFFSETS      # not to n
    assert _offsets_bits([0, 6, 5, 9], 9) == B.MDLM_CHECK_OFFSETS   # decreasing
    assert _offsets_bits([0, -1, 9], 9) == B.MDLM_CHECK_OFFSETS     # negative
    # a long valid stream, and one bad entry deep inside it
    cu = np.arange(0, 4096 * 3000 + 1, 4096).astype(np.int32)
    assert _offsets_bits(cu, int(cu[-1])) == 0
    cu[2500] = cu[2499] - 1
    assert _offsets_bits(cu, int(cu[-1])) == B.MDLM_CHECK_OFFSETS


def test_probs():
    st = _status()
    B.mdlm_check_probs(torch.tensor([1e-3, 0.5, 1.0], dtype=torch.float64, device=DEV), st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    for bad in (0.0, -0.1, 1.5, float("nan")):
        st = _status()
        B.mdlm_check_probs(torch.tensor([0.5, bad], dtype=torch.float64, device=DEV), st)
        torch.cuda.synchronize()
        assert int(st.item()) == B.MDLM_CHECK_PROB, bad


def _rows_bits(rows, tgt, w, n_rows, max_rows, n_tokens, V):
    st = _status()
    t = lambda a, dt: None if a is None else torch.tensor(a, dtype=dt, device=DEV)  # noqa: E731
    B.mdlm_check_rows(t(rows, torch.int32), t(tgt, torch.int32), t(w, torch.float32),
                      torch.tensor([n_rows], **i32), max_rows, n_tokens, V, st)
    torch.cuda.synchronize()
    return int(st.item())


def test_rows():
    ok = dict(rows=[0, 3, 9], tgt=[1, 0, 6], w=[0.5, 0.25, 1.0], n_rows=3, max_rows=3,
              n_tokens=10, V=7)
    assert _rows_bits(**ok) == 0
    assert _rows_bits(**{**ok, "n_rows": 4}) == B.MDLM_CHECK_ROW_COUNT
    assert _rows_bits(**{**ok, "n_rows": -1}) == B.MDLM_CHECK_ROW_COUNT
    assert _rows_bits(**{**ok, "rows": [0, 10, 9]}) == B.MDLM_CHECK_ROW_INDEX
    assert _rows_bits(**{**ok, "tgt": [1, 7, 6]}) == B.MDLM_CHECK_TARGET
    assert _rows_bits(**{**ok, "tgt": [-1, 0, 6]}) == B.MDLM_CHECK_TARGET
    assert _rows_bits(**{**ok, "w": [0.5, float("inf"), 1.0]}) == B.MDLM_CHECK_WEIGHT
    # entries past the device count are not rows: not checked
    assert _rows_bits(**{**ok, "n_rows": 2, "tgt": [1, 0, 99]}) == 0
    # tgt and w optional; several violations at once
    assert _rows_bits(**{**ok, "tgt": None, "w": None}) == 0
    assert _rows_bits(**{**ok, "rows": [-4, 3, 9], "tgt": [1, 0, 7]}) == (
        B.MDLM_CHECK_ROW_INDEX | B.MDLM_CHECK_TARGET)


@pytest.fixture
def checking():
    prev = B.mdlm_set_checking(True)
    yield
    B.mdlm_set_checking(prev)


def test_checking_mode_passes_valid_inputs_unchanged(checking):
    inp = WL.small_case(21, n_docs=4, max_len=300, H=128, V=1000, softcap=30.0)
    a = run_step(inp, seed=3, eps=0.5)
    B.mdlm_set_checking(False)
    b = run_step(inp, seed=3, eps=0.5)
    m = int(host(a.n_rows)[0])
    assert m == int(host(b.n_rows)[0]) and m > 0
    for name in ("xt", "corrupted", "loss"):
        assert np.array_equal(host(getattr(a, name)), host(getattr(b, name))), name
    for name in ("row_idx", "tgt", "w"):
        assert np.array_equal(host(getattr(a, name))[:m], host(getattr(b, name))[:m]), name
    assert torch.equal(a.d_hidden, b.d_hidden)


def test_checking_mode_refuses_bad_offsets_before_any_work(checking):
    inp = WL.small_case(22, n_docs=4, max_len=100, H=64, V=500)
    wl = inp.wl
    x0, _ = dev_tokens(inp)
    bad = inp.cu_seqlens.copy()
    bad[2] = bad[1] - 1                       # decreasing offsets
    cu = torch.from_numpy(bad).to(DEV)
    step = MdlmLossStep(wl.n_tokens, wl.n_docs, wl.H, wl.V, device=DEV, head_workspace_bytes=0,
                        want_grad=False)
    step.xt.fill_(-7)
    step.corrupted.fill_(9)
    with pytest.raises(B.MdlmError, match="cu_seqlens") as e:
        step.corrupt(x0, cu, 1, 0.5, wl.noise, wl.mask_id, wl.rand_vocab)
    assert e.value.code == B.MDLM_EINVAL
    torch.cuda.synchronize()
    assert torch.all(step.xt == -7) and torch.all(step.corrupted == 9)
    step.n_rows.fill_(-3)
    with pytest.raises(B.MdlmError, match="cu_seqlens"):
        step.compact(x0, cu, oracle.ALIGNED)
    torch.cuda.synchronize()
    assert int(step.n_rows.item()) == -3


def test_checking_mode_refuses_bad_row_lists_before_any_work(checking):
    inp = WL.small_case(23, n_docs=3, max_len=150, H=64, V=400)
    wl = inp.wl
    h, W = dev_float(inp)
    n = wl.n_tokens
    rows = torch.arange(0, n, 3, dtype=torch.int32, device=DEV)
    m = rows.numel()
    tgt = torch.zeros(m, **i32)
    tgt[m // 2] = wl.V                           # a target past the vocabulary
    w = torch.full((m,), 0.01, dtype=torch.float32, device=DEV)
    n_rows = torch.tensor([m], **i32)
    loss = torch.full((1,), 5.0, device=DEV)
    dh = torch.full_like(h, 2.0)
    ws = torch.empty(B.mdlm_head_ce_workspace_bytes(m, wl.H, wl.V, B.MDLM_BF16),
                     dtype=torch.uint8, device=DEV)
    with pytest.raises(B.MdlmError, match="tgt"):
        B.mdlm_fused_head_ce_fwd_bwd(h, W, rows, tgt, w, n_rows, m, 0.0, loss, None, dh, ws)
    torch.cuda.synchronize()
    assert float(loss.item()) == 5.0 and torch.all(dh == 2.0)
    tgt[m // 2] = 3
    n_rows.fill_(m + 1)                          # more rows than max_rows
    with pytest.raises(B.MdlmError, match="n_rows"):
        B.mdlm_fused_head_ce_fwd_bwd(h, W, rows, tgt, w, n_rows, m, 0.0, loss, None, dh, ws)
    torch.cuda.synchronize()
    assert float(loss.item()) == 5.0
    # repaired, the same call runs
    n_rows.fill_(m)
    B.mdlm_fused_head_ce_fwd_bwd(h, W, rows, tgt, w, n_rows, m, 0.0, loss, None, dh, ws)
    torch.cuda.synchronize()
    assert np.isfinite(float(loss.item())) and float(loss.item()) != 5.0


def test_checking_mode_refuses_stream_capture(checking):
    inp = WL.small_case(24, n_docs=2, max_len=80, H=64, V=300)
    wl = inp.wl
    x0, cu = dev_tokens(inp)
    step = MdlmLossStep(wl.n_tokens, wl.n_docs, wl.H, wl.V, device=DEV, head_workspace_bytes=0,
                        want_grad=False)
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    err = None
    with torch.cuda.graph(g, stream=s):
        try:
            step.corrupt(x0, cu, 1, 0.5, wl.noise, wl.mask_id, wl.rand_vocab)
        except B.MdlmError as e:  # (caught inside, so that the capture ends normally)
            err = e
    assert err is not None and err.code == B.MDLM_EINVAL and "capture" in str(err)
