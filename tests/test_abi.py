"""Host-side checks of the C ABI: no GPU needed.

The library must load, export every function include/mdlm.h declares, size
its workspaces, and reject bad arguments on the host (returning a status and
a message) before enqueueing anything.  Every rejected call below passes null
data pointers, so nothing could run even if a check were missing.
"""

import ctypes
import os
import re

import pytest

from uniform_noise_diffusion_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mdlm.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mdlm_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.skip("libmdlm.so not built")
    return B.load()


def test_header_declares_the_three_entry_points():
    names = declared_functions()
    for n in ("mdlm_corrupt", "mdlm_compact_masked", "mdlm_fused_head_ce_fwd_bwd",
              "mdlm_head_ce_workspace_bytes", "mdlm_last_error"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 8
    for n in names:
        assert hasattr(lib, n), n
    assert set(B.EXPORTED) == set(names)


def test_version(lib):
    assert B.mdlm_version() >> 16 == 1


def compact_ws(n):
    # three 32-bit words per 4096-token tile, one per group of 1024 tiles
    tiles = -(-n // 4096)
    return 4 * (3 * tiles + -(-tiles // 1024))


def test_compact_workspace_sizes(lib):
    assert B.mdlm_compact_workspace_bytes(0) == 0
    assert B.mdlm_compact_workspace_bytes(1) == 16
    assert B.mdlm_compact_workspace_bytes(4096) == 16
    assert B.mdlm_compact_workspace_bytes(4097) == 28
    assert B.mdlm_compact_workspace_bytes(1024 * 4096) == 4 * (3 * 1024 + 1)
    assert B.mdlm_compact_workspace_bytes(1024 * 4096 + 1) == 4 * (3 * 1025 + 2)
    assert B.mdlm_compact_workspace_bytes(1 << 27) == compact_ws(1 << 27) == 4 * (3 * 32768 + 32)


def test_head_workspace_sizes(lib):
    for dt in (B.MDLM_BF16, B.MDLM_F32):
        lo = B.mdlm_head_ce_workspace_min_bytes(4096, 4096, 126464, dt)
        hi = B.mdlm_head_ce_workspace_bytes(4096, 4096, 126464, dt)
        assert 0 < lo <= hi
    assert B.mdlm_head_ce_workspace_bytes(-1, 64, 64, B.MDLM_BF16) == 0
    assert B.mdlm_head_ce_workspace_bytes(8, 0, 64, B.MDLM_BF16) == 0
    assert B.mdlm_head_ce_workspace_bytes(8, 64, 64, 7) == 0
    # the bf16 gradient chunk grows with the workspace but never beyond V
    small = B.mdlm_head_ce_workspace_bytes(16, 64, 1000, B.MDLM_BF16)
    assert small == B.mdlm_head_ce_workspace_bytes(16, 64, 1024, B.MDLM_BF16)


NULL = None


def corrupt_call(lib, **kw):
    a = dict(x0=NULL, n=16, cu=NULL, n_docs=1, seed=0, eps=1e-3, noise=0, mask_id=1,
             rand_vocab=2, xt=NULL, corrupted=NULL, p_doc=NULL, counts=NULL, stream=NULL)
    a.update(kw)
    return lib.mdlm_corrupt(a["x0"], a["n"], a["cu"], a["n_docs"], a["seed"], a["eps"],
                            a["noise"], a["mask_id"], a["rand_vocab"], a["xt"],
                            a["corrupted"], a["p_doc"], a["counts"], a["stream"])


@pytest.mark.parametrize("kw,code,msg", [
    (dict(n=-1), B.MDLM_EINVAL, "n_tokens < 0"),
    (dict(n=1 << 31), B.MDLM_EUNSUPPORTED, "below 2^31"),
    (dict(n_docs=-2), B.MDLM_EINVAL, "n_docs < 0"),
    (dict(n_docs=0), B.MDLM_EINVAL, "n_docs = 0"),
    (dict(eps=0.0), B.MDLM_EINVAL, "eps"),
    (dict(eps=1.5), B.MDLM_EINVAL, "eps"),
    (dict(eps=float("nan")), B.MDLM_EINVAL, "eps"),
    (dict(noise=5), B.MDLM_EINVAL, "noise"),
    (dict(noise=1, rand_vocab=0), B.MDLM_EINVAL, "rand_vocab"),
    (dict(), B.MDLM_EINVAL, "null token pointer"),
])
def test_corrupt_rejects_bad_arguments(lib, kw, code, msg):
    assert corrupt_call(lib, **kw) == code
    assert msg in B.mdlm_last_error()


def compact_call(lib, **kw):
    a = dict(corrupted=NULL, x0=NULL, n=16, cu=NULL, n_docs=1, p_doc=NULL, align=0,
             row_idx=NULL, tgt=NULL, w=NULL, n_rows=NULL, ws=NULL, ws_bytes=0, stream=NULL)
    a.update(kw)
    return lib.mdlm_compact_masked(a["corrupted"], a["x0"], a["n"], a["cu"], a["n_docs"],
                                   a["p_doc"], a["align"], a["row_idx"], a["tgt"], a["w"],
                                   a["n_rows"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code,msg", [
    (dict(n=-3), B.MDLM_EINVAL, "n_tokens < 0"),
    (dict(n_docs=0), B.MDLM_EINVAL, "n_docs"),
    (dict(align=2), B.MDLM_EINVAL, "alignment"),
    (dict(), B.MDLM_EINVAL, "null n_rows"),
])
def test_compact_rejects_bad_arguments(lib, kw, code, msg):
    assert compact_call(lib, **kw) == code
    assert msg in B.mdlm_last_error()


def head_call(lib, **kw):
    a = dict(hidden=NULL, W=NULL, dtype=B.MDLM_BF16, n=64, H=128, V=1000, row_idx=NULL,
             tgt=NULL, w=NULL, n_rows=NULL, max_rows=32, softcap=0.0, loss=NULL, row_ce=NULL,
             d_hidden=NULL, ws=NULL, ws_bytes=0, stream=NULL)
    a.update(kw)
    return lib.mdlm_fused_head_ce_fwd_bwd(
        a["hidden"], a["W"], a["dtype"], a["n"], a["H"], a["V"], a["row_idx"], a["tgt"],
        a["w"], a["n_rows"], a["max_rows"], a["softcap"], a["loss"], a["row_ce"],
        a["d_hidden"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code,msg", [
    (dict(dtype=3), B.MDLM_EINVAL, "dtype"),
    (dict(H=0), B.MDLM_EINVAL, "bad sizes"),
    (dict(V=-1), B.MDLM_EINVAL, "bad sizes"),
    (dict(max_rows=65), B.MDLM_EINVAL, "max_rows"),
    (dict(max_rows=-1), B.MDLM_EINVAL, "max_rows"),
    (dict(H=96), B.MDLM_EUNSUPPORTED, "multiple of 64"),
    (dict(n=1 << 19, H=4096, max_rows=8), B.MDLM_EUNSUPPORTED, "below 4 GiB"),
    (dict(V=1 << 19, H=4096), B.MDLM_EUNSUPPORTED, "below 4 GiB"),
    (dict(softcap=-1.0), B.MDLM_EINVAL, "softcap"),
    (dict(softcap=float("inf")), B.MDLM_EINVAL, "softcap"),
    (dict(), B.MDLM_EINVAL, "null loss"),
])
def test_head_rejects_bad_arguments(lib, kw, code, msg):
    assert head_call(lib, **kw) == code
    assert msg in B.mdlm_last_error()


def test_head_rejects_missing_or_small_workspace(lib):
    # the inputs are non-null placeholders that are never dereferenced: the
    # workspace check fails first and nothing is enqueued
    fake = ctypes.c_void_p(1 << 20)
    kw = dict(hidden=fake, W=fake, row_idx=fake, tgt=fake, w=fake, n_rows=fake, loss=fake)
    assert head_call(lib, **kw) == B.MDLM_EWORKSPACE
    assert "workspace" in B.mdlm_last_error()
    need = B.mdlm_head_ce_workspace_min_bytes(32, 128, 1000, B.MDLM_BF16)
    assert head_call(lib, ws=fake, ws_bytes=need - 1, **kw) == B.MDLM_EWORKSPACE
    # a misaligned input is rejected before the workspace is looked at
    odd = ctypes.c_void_p((1 << 20) + 2)
    kw2 = dict(kw, hidden=odd)
    assert head_call(lib, **kw2) == B.MDLM_EINVAL
    assert "16-byte aligned" in B.mdlm_last_error()
    kw3 = dict(kw, d_hidden=ctypes.c_void_p((1 << 20) + 8))
    assert head_call(lib, **kw3) == B.MDLM_EINVAL
    assert "d_hidden must be 16-byte aligned" in B.mdlm_last_error()


def test_compact_rejects_small_workspace(lib):
    # placeholders are never dereferenced: the workspace check fails first
    fake = ctypes.c_void_p(1 << 20)
    n = 1 << 20
    need = B.mdlm_compact_workspace_bytes(n)
    assert need == compact_ws(n)
    kw = dict(corrupted=fake, x0=fake, cu=fake, p_doc=fake, row_idx=fake, tgt=fake, w=fake,
              n_rows=fake, n=n)
    assert compact_call(lib, **kw) == B.MDLM_EWORKSPACE
    assert compact_call(lib, ws=fake, ws_bytes=need - 1, **kw) == B.MDLM_EWORKSPACE
    assert "workspace" in B.mdlm_last_error()


def mixture_call(lib, **kw):
    a = dict(x0=NULL, n=16, cu=NULL, n_docs=1, seed=0, eps=1e-3, mix=0.5, mask_id=1,
             rand_vocab=2, xt=NULL, codes=NULL, p_doc=NULL, counts=NULL, stream=NULL)
    a.update(kw)
    return lib.mdlm_corrupt_mixture(a["x0"], a["n"], a["cu"], a["n_docs"], a["seed"],
                                    a["eps"], a["mix"], a["mask_id"], a["rand_vocab"],
                                    a["xt"], a["codes"], a["p_doc"], a["counts"], a["stream"])


@pytest.mark.parametrize("kw,code,msg", [
    (dict(n=-1), B.MDLM_EINVAL, "n_tokens < 0"),
    (dict(n=1 << 31), B.MDLM_EUNSUPPORTED, "below 2^31"),
    (dict(n_docs=0), B.MDLM_EINVAL, "n_docs = 0"),
    (dict(eps=0.0), B.MDLM_EINVAL, "eps"),
    (dict(mix=-0.1), B.MDLM_EINVAL, "mixture_prob"),
    (dict(mix=1.5), B.MDLM_EINVAL, "mixture_prob"),
    (dict(mix=float("nan")), B.MDLM_EINVAL, "mixture_prob"),
    (dict(rand_vocab=0), B.MDLM_EINVAL, "rand_vocab"),
    (dict(), B.MDLM_EINVAL, "null token pointer"),
])
def test_corrupt_mixture_rejects_bad_arguments(lib, kw, code, msg):
    assert mixture_call(lib, **kw) == code
    assert msg in B.mdlm_last_error()


def corrective_call(lib, **kw):
    a = dict(codes=NULL, x0=NULL, n=16, cu=NULL, n_docs=1, p_doc=NULL, align=0, a=0.5, c=0.0,
             row_idx=NULL, tgt=NULL, w=NULL, n_rows=NULL, ws=NULL, ws_bytes=0, stream=NULL)
    a.update(kw)
    return lib.mdlm_compact_corrective(a["codes"], a["x0"], a["n"], a["cu"], a["n_docs"],
                                       a["p_doc"], a["align"], a["a"], a["c"], a["row_idx"],
                                       a["tgt"], a["w"], a["n_rows"], a["ws"], a["ws_bytes"],
                                       a["stream"])


@pytest.mark.parametrize("kw,code,msg", [
    (dict(n=-1), B.MDLM_EINVAL, "n_tokens < 0"),
    (dict(n=1 << 31), B.MDLM_EUNSUPPORTED, "below 2^31"),
    (dict(n_docs=0), B.MDLM_EINVAL, "n_docs"),
    (dict(align=2), B.MDLM_EINVAL, "alignment"),
    (dict(a=float("nan")), B.MDLM_EINVAL, "finite"),
    (dict(c=float("inf")), B.MDLM_EINVAL, "finite"),
    (dict(), B.MDLM_EINVAL, "null n_rows"),
])
def test_compact_corrective_rejects_bad_arguments(lib, kw, code, msg):
    assert corrective_call(lib, **kw) == code
    assert msg in B.mdlm_last_error()


def test_compact_corrective_pointer_and_workspace_checks(lib):
    fake = ctypes.c_void_p(1 << 20)
    n = 1 << 20
    kw = dict(x0=fake, cu=fake, row_idx=fake, tgt=fake, w=fake, n_rows=fake, n=n)
    assert corrective_call(lib, p_doc=fake, **kw) == B.MDLM_EINVAL   # no codes
    assert "null pointer" in B.mdlm_last_error()
    assert corrective_call(lib, codes=fake, **kw) == B.MDLM_EINVAL   # no p_doc
    need = B.mdlm_compact_workspace_bytes(n)
    assert corrective_call(lib, codes=fake, p_doc=fake, ws=fake, ws_bytes=need - 1,
                           **kw) == B.MDLM_EWORKSPACE
    odd = ctypes.c_void_p((1 << 20) + 2)
    assert corrective_call(lib, codes=fake, p_doc=fake, ws=odd, ws_bytes=need,
                           **kw) == B.MDLM_EINVAL
    assert "4-byte aligned" in B.mdlm_last_error()


def rows_call(lib, **kw):
    a = dict(corrupted=NULL, eligible=NULL, x0=NULL, n=16, cu=NULL, n_docs=1, p_doc=NULL,
             align=0, weighting=1, scale=1.0, clip=10.0, row_idx=NULL, tgt=NULL, w=NULL,
             n_rows=NULL, ws=NULL, ws_bytes=0, stream=NULL)
    a.update(kw)
    return lib.mdlm_compact_rows(a["corrupted"], a["eligible"], a["x0"], a["n"], a["cu"],
                                 a["n_docs"], a["p_doc"], a["align"], a["weighting"],
                                 a["scale"], a["clip"], a["row_idx"], a["tgt"], a["w"],
                                 a["n_rows"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code,msg", [
    (dict(n=-1), B.MDLM_EINVAL, "n_tokens < 0"),
    (dict(n_docs=0), B.MDLM_EINVAL, "n_docs"),
    (dict(align=3), B.MDLM_EINVAL, "alignment"),
    (dict(weighting=3), B.MDLM_EINVAL, "weighting"),
    (dict(weighting=-1), B.MDLM_EINVAL, "weighting"),
    (dict(scale=float("nan")), B.MDLM_EINVAL, "weight_scale"),
    (dict(scale=float("inf")), B.MDLM_EINVAL, "weight_scale"),
    (dict(weighting=2, clip=0.0), B.MDLM_EINVAL, "weight_clip"),
    (dict(weighting=2, clip=float("nan")), B.MDLM_EINVAL, "weight_clip"),
    (dict(), B.MDLM_EINVAL, "null n_rows"),
])
def test_compact_rows_rejects_bad_arguments(lib, kw, code, msg):
    assert rows_call(lib, **kw) == code
    assert msg in B.mdlm_last_error()


def test_compact_rows_pointer_and_workspace_checks(lib):
    fake = ctypes.c_void_p(1 << 20)
    n = 1 << 20
    kw = dict(x0=fake, cu=fake, row_idx=fake, tgt=fake, w=fake, n_rows=fake, n=n, n_docs=9)
    # the mean weighting needs no p_doc and no mask; others need p_doc
    assert rows_call(lib, **kw) == B.MDLM_EWORKSPACE
    assert rows_call(lib, weighting=0, **kw) == B.MDLM_EINVAL
    assert "null pointer" in B.mdlm_last_error()
    # weights per document (mean, example mean); rows per document + 1 (example mean)
    need = B.mdlm_compact_rows_workspace_bytes(n, 9, 2)
    assert need == compact_ws(n) + 4 * (9 + 9 + 1)
    assert B.mdlm_compact_rows_workspace_bytes(n, 9, 1) == compact_ws(n) + 4 * 9
    assert B.mdlm_compact_rows_workspace_bytes(n, 9, 0) == compact_ws(n)
    assert B.mdlm_compact_rows_workspace_bytes(n, 9, 7) == 0
    assert B.mdlm_compact_rows_workspace_bytes(n, -1, 1) == 0
    assert rows_call(lib, weighting=2, p_doc=fake, ws=fake, ws_bytes=need - 1,
                     **kw) == B.MDLM_EWORKSPACE
    odd = ctypes.c_void_p((1 << 20) + 2)
    assert rows_call(lib, weighting=2, p_doc=fake, ws=odd, ws_bytes=need, **kw) == B.MDLM_EINVAL
    assert "4-byte aligned" in B.mdlm_last_error()


def test_error_is_cleared_by_next_call(lib):
    assert corrupt_call(lib, eps=0.0) == B.MDLM_EINVAL
    assert B.mdlm_last_error() != ""
    assert B.mdlm_compact_workspace_bytes(5) > 0
    # size queries do not touch the error slot; a failing call overwrites it
    assert compact_call(lib, align=9) == B.MDLM_EINVAL
    assert "alignment" in B.mdlm_last_error()


def test_probe_library_exports_its_header():
    from uniform_noise_diffusion_amd import probe
    if not os.path.exists(probe.PROBE_LIB_PATH):
        pytest.skip("libmdlm_probe.so not built")
    text = open(os.path.join(ROOT, "include", "mdlm_probe.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = sorted(set(re.findall(r"\b(mdlm_\w+)\s*\(", text)))
    assert set(names) == set(probe.EXPORTED)
    lib = probe.load()
    for n in names:
        assert hasattr(lib, n), n
    for m in re.finditer(r"\b(mdlm_\w+)\s*\(([^)]*)\)\s*;", text):
        n_params = len([q for q in m.group(2).split(",") if q.strip()])
        assert len(getattr(lib, m.group(1)).argtypes) == n_params, m.group(1)
    # invalid launch shapes are refused before anything is enqueued
    assert lib.mdlm_probe_mfma(None, 0, 1, None) != 0
    assert lib.mdlm_probe_mfma(None, 1, 0, None) != 0
    assert lib.mdlm_probe_copy(None, None, 0, None) == 0


def test_dw_entry_point_checks(lib):
    fake = ctypes.c_void_p(1 << 20)
    a = dict(hidden=fake, W=fake, n=64, H=128, V=1000, row_idx=fake, tgt=fake, w=fake,
             n_rows=fake, max_rows=32, softcap=0.0, loss=fake, row_ce=None, d_hidden=None,
             dW=fake, ws=None, ws_bytes=0)

    def call(**kw):
        b = dict(a)
        b.update(kw)
        return lib.mdlm_fused_head_ce_fwd_bwd_dw(
            b["hidden"], b["W"], b["n"], b["H"], b["V"], b["row_idx"], b["tgt"], b["w"],
            b["n_rows"], b["max_rows"], b["softcap"], b["loss"], b["row_ce"], b["d_hidden"],
            b["dW"], b["ws"], b["ws_bytes"], None)

    assert call(dW=None) == B.MDLM_EINVAL and "null dW" in B.mdlm_last_error()
    assert call(dW=ctypes.c_void_p((1 << 20) + 4)) == B.MDLM_EINVAL
    assert "dW must be 16-byte aligned" in B.mdlm_last_error()
    assert call(H=96) == B.MDLM_EUNSUPPORTED
    assert call() == B.MDLM_EWORKSPACE
    need = B.mdlm_head_ce_dw_workspace_min_bytes(32, 128, 1000)
    # the gathered rows (32 x 128 bf16) on top of the plain call's workspace
    assert need >= B.mdlm_head_ce_workspace_min_bytes(32, 128, 1000, B.MDLM_BF16) + 32 * 128 * 2
    assert call(ws=fake, ws_bytes=need - 1) == B.MDLM_EWORKSPACE
    assert (B.mdlm_head_ce_dw_workspace_bytes(32, 128, 1000) >= need > 0)
    assert B.mdlm_head_ce_dw_workspace_bytes(-1, 128, 1000) == 0


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setattr(B, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        B.load()


def declared_prototypes():
    """name -> number of parameters, from the header's prototypes."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    out = {}
    for m in re.finditer(r"\b(mdlm_\w+)\s*\(([^)]*)\)\s*;", text):
        params = [p.strip() for p in m.group(2).split(",") if p.strip()]
        if params == ["void"]:
            params = []
        out[m.group(1)] = len(params)
    return out


def test_binding_signatures_match_the_header(lib):
    """Every ctypes declaration in the binding takes as many arguments as the
    header's prototype (a miscounted binding would shift every argument)."""
    protos = declared_prototypes()
    assert set(protos) == set(B.EXPORTED)
    for name, n in protos.items():
        fn = getattr(lib, name)
        assert fn.argtypes is not None, name
        assert len(fn.argtypes) == n, (name, len(fn.argtypes), n)


@pytest.mark.parametrize("args,code,msg", [
    ((NULL, NULL, 5, 16, NULL, NULL), B.MDLM_EINVAL, "dtype"),
    ((NULL, NULL, B.MDLM_BF16, -1, NULL, NULL), B.MDLM_EINVAL, "n < 0"),
    ((NULL, NULL, B.MDLM_BF16, 16, NULL, NULL), B.MDLM_EINVAL, "null pointer"),
])
def test_scale_rejects_bad_arguments(lib, args, code, msg):
    assert lib.mdlm_scale(*args, NULL) == code
    assert msg in B.mdlm_last_error()
    # nothing to scale: accepted without touching a pointer
    assert lib.mdlm_scale(NULL, NULL, B.MDLM_F32, 0, NULL, NULL) == B.MDLM_OK


def test_check_calls_reject_bad_arguments(lib):
    assert lib.mdlm_check_offsets(NULL, -1, 10, NULL, NULL) == B.MDLM_EINVAL
    assert lib.mdlm_check_offsets(NULL, 2, 10, NULL, NULL) == B.MDLM_EINVAL
    assert "null pointer" in B.mdlm_last_error()
    assert lib.mdlm_check_probs(NULL, -1, NULL, NULL) == B.MDLM_EINVAL
    assert lib.mdlm_check_probs(NULL, 3, NULL, NULL) == B.MDLM_EINVAL
    assert lib.mdlm_check_rows(NULL, NULL, NULL, NULL, -1, 10, 5, NULL, NULL) == B.MDLM_EINVAL
    assert lib.mdlm_check_rows(NULL, NULL, NULL, NULL, 4, 10, 5, NULL, NULL) == B.MDLM_EINVAL
    assert "null pointer" in B.mdlm_last_error()


def test_checking_mode_switch_and_host_checks_first(lib):
    prev = B.mdlm_set_checking(True)
    try:
        assert B.mdlm_set_checking(True) is True
        # host-side checks still come first: null pointers are rejected before
        # any device check could be enqueued
        assert corrupt_call(lib) == B.MDLM_EINVAL
        assert "null token pointer" in B.mdlm_last_error()
        assert head_call(lib) == B.MDLM_EINVAL
    finally:
        B.mdlm_set_checking(prev)
    assert B.mdlm_set_checking(prev) is prev
