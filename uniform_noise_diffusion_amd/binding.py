"""ctypes binding of libmdlm.so (include/mdlm.h).

Argument marshalling only: every computation runs in the HIP library.  The
functions keep the C names and take torch tensors for device memory; the
stream is torch's current stream unless one is given.  A non-zero status from
the library raises MdlmError carrying mdlm_last_error().  If the library has
not been built the first call raises; nothing falls back to another
implementation.
"""

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmdlm.so")

MDLM_OK = 0
MDLM_EINVAL = 1
MDLM_EUNSUPPORTED = 2
MDLM_EWORKSPACE = 3
MDLM_EHIP = 4
MDLM_NOISE_ABSORB = 0
MDLM_NOISE_UNIFORM = 1
MDLM_ALIGNED = 0
MDLM_SHIFTED = 1
MDLM_F32 = 0
MDLM_BF16 = 1
MDLM_WEIGHT_INV_P = 0
MDLM_WEIGHT_MEAN = 1
MDLM_WEIGHT_EXAMPLE_MEAN_CLIPPED = 2
MDLM_CODE_CLEAN = 0
MDLM_CODE_MASKED = 1
MDLM_CODE_REPLACED = 2
MDLM_CHECK_OFFSETS = 1
MDLM_CHECK_ROW_COUNT = 2
MDLM_CHECK_ROW_INDEX = 4
MDLM_CHECK_TARGET = 8
MDLM_CHECK_WEIGHT = 16
MDLM_CHECK_PROB = 32

EXPORTED = (
    "mdlm_corrupt",
    "mdlm_corrupt_mixture",
    "mdlm_corrupt_compact_workspace_bytes",
    "mdlm_corrupt_compact",
    "mdlm_compact_workspace_bytes",
    "mdlm_compact_masked",
    "mdlm_compact_masked_noalloc",
    "mdlm_compact_corrective",
    "mdlm_compact_rows_workspace_bytes",
    "mdlm_compact_rows",
    "mdlm_head_ce_workspace_bytes",
    "mdlm_head_ce_workspace_min_bytes",
    "mdlm_fused_head_ce_fwd_bwd",
    "mdlm_head_ce_dw_workspace_bytes",
    "mdlm_head_ce_dw_workspace_min_bytes",
    "mdlm_fused_head_ce_fwd_bwd_dw",
    "mdlm_scale",
    "mdlm_check_offsets",
    "mdlm_check_probs",
    "mdlm_check_rows",
    "mdlm_set_checking",
    "mdlm_last_error",
    "mdlm_version",
)

_lib = None


class MdlmError(RuntimeError):
    def __init__(self, code, message):
        super().__init__(f"[mdlm status {code}] {message}")
        self.code = code


def load():
    """Load libmdlm.so once and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with "
            "`python -m uniform_noise_diffusion_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, u64, f32, f64, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                       ctypes.c_uint64, ctypes.c_float, ctypes.c_double,
                                       ctypes.c_size_t)
    lib.mdlm_corrupt.argtypes = [vp, i64, vp, i32, u64, f64, i32, i32, i32, vp, vp, vp, vp, vp]
    lib.mdlm_corrupt.restype = ctypes.c_int
    lib.mdlm_corrupt_mixture.argtypes = [vp, i64, vp, i32, u64, f64, f64, i32, i32, vp, vp, vp,
                                         vp, vp]
    lib.mdlm_corrupt_mixture.restype = ctypes.c_int
    lib.mdlm_corrupt_compact_workspace_bytes.argtypes = [i64]
    lib.mdlm_corrupt_compact_workspace_bytes.restype = sz
    lib.mdlm_corrupt_compact.argtypes = [vp, i64, vp, i32, u64, f64, i32, i32, i32, i32, vp, vp,
                                         vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.mdlm_corrupt_compact.restype = ctypes.c_int
    lib.mdlm_compact_workspace_bytes.argtypes = [i64]
    lib.mdlm_compact_workspace_bytes.restype = sz
    lib.mdlm_compact_masked.argtypes = [vp, vp, i64, vp, i32, vp, i32, vp, vp, vp, vp, vp, sz, vp]
    lib.mdlm_compact_masked.restype = ctypes.c_int
    lib.mdlm_compact_masked_noalloc.argtypes = [vp, vp, i64, vp, i32, vp, i32, vp, vp, vp, vp,
                                                vp]
    lib.mdlm_compact_masked_noalloc.restype = ctypes.c_int
    lib.mdlm_compact_corrective.argtypes = [vp, vp, i64, vp, i32, vp, i32, f64, f64, vp, vp, vp,
                                            vp, vp, sz, vp]
    lib.mdlm_compact_corrective.restype = ctypes.c_int
    lib.mdlm_compact_rows_workspace_bytes.argtypes = [i64, i32, i32]
    lib.mdlm_compact_rows_workspace_bytes.restype = sz
    lib.mdlm_compact_rows.argtypes = [vp, vp, vp, i64, vp, i32, vp, i32, i32, f64, f64, vp, vp,
                                      vp, vp, vp, sz, vp]
    lib.mdlm_compact_rows.restype = ctypes.c_int
    lib.mdlm_head_ce_workspace_bytes.argtypes = [i64, i32, i32, i32]
    lib.mdlm_head_ce_workspace_bytes.restype = sz
    lib.mdlm_head_ce_workspace_min_bytes.argtypes = [i64, i32, i32, i32]
    lib.mdlm_head_ce_workspace_min_bytes.restype = sz
    lib.mdlm_fused_head_ce_fwd_bwd.argtypes = [vp, vp, i32, i64, i32, i32, vp, vp, vp, vp, i64,
                                               f32, vp, vp, vp, vp, sz, vp]
    lib.mdlm_fused_head_ce_fwd_bwd.restype = ctypes.c_int
    lib.mdlm_head_ce_dw_workspace_bytes.argtypes = [i64, i32, i32]
    lib.mdlm_head_ce_dw_workspace_bytes.restype = sz
    lib.mdlm_head_ce_dw_workspace_min_bytes.argtypes = [i64, i32, i32]
    lib.mdlm_head_ce_dw_workspace_min_bytes.restype = sz
    lib.mdlm_fused_head_ce_fwd_bwd_dw.argtypes = [vp, vp, i64, i32, i32, vp, vp, vp, vp, i64,
                                                  f32, vp, vp, vp, vp, vp, sz, vp]
    lib.mdlm_fused_head_ce_fwd_bwd_dw.restype = ctypes.c_int
    lib.mdlm_scale.argtypes = [vp, vp, i32, i64, vp, vp]
    lib.mdlm_scale.restype = ctypes.c_int
    lib.mdlm_check_offsets.argtypes = [vp, i32, i64, vp, vp]
    lib.mdlm_check_offsets.restype = ctypes.c_int
    lib.mdlm_check_probs.argtypes = [vp, i32, vp, vp]
    lib.mdlm_check_probs.restype = ctypes.c_int
    lib.mdlm_check_rows.argtypes = [vp, vp, vp, vp, i64, i64, i32, vp, vp]
    lib.mdlm_check_rows.restype = ctypes.c_int
    lib.mdlm_set_checking.argtypes = [ctypes.c_int]
    lib.mdlm_set_checking.restype = ctypes.c_int
    lib.mdlm_last_error.argtypes = []
    lib.mdlm_last_error.restype = ctypes.c_char_p
    lib.mdlm_version.argtypes = []
    lib.mdlm_version.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(code):
    if code != MDLM_OK:
        raise MdlmError(code, load().mdlm_last_error().decode())


def _need(t, dtype, name):
    if t is None:
        return
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name}: expected a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous tensor")


def mdlm_last_error():
    return load().mdlm_last_error().decode()


def mdlm_version():
    return load().mdlm_version()


def mdlm_corrupt(x0, cu_seqlens, seed, eps, noise, mask_id, rand_vocab, xt, corrupted,
                 p_doc, doc_counts, stream=None):
    """See mdlm_corrupt in include/mdlm.h."""
    _need(x0, torch.int32, "x0")
    _need(cu_seqlens, torch.int32, "cu_seqlens")
    _need(xt, torch.int32, "xt")
    _need(corrupted, torch.uint8, "corrupted")
    _need(p_doc, torch.float64, "p_doc")
    _need(doc_counts, torch.int32, "doc_counts")
    n_docs = cu_seqlens.numel() - 1
    _check(load().mdlm_corrupt(_ptr(x0), x0.numel(), _ptr(cu_seqlens), n_docs,
                               int(seed) & 0xFFFFFFFFFFFFFFFF, float(eps), int(noise),
                               int(mask_id), int(rand_vocab), _ptr(xt), _ptr(corrupted),
                               _ptr(p_doc), _ptr(doc_counts), _stream(stream)))


def mdlm_corrupt_mixture(x0, cu_seqlens, seed, eps, mixture_prob, mask_id, rand_vocab, xt,
                         codes, p_doc, doc_counts, stream=None):
    """See mdlm_corrupt_mixture in include/mdlm.h."""
    _need(x0, torch.int32, "x0")
    _need(cu_seqlens, torch.int32, "cu_seqlens")
    _need(xt, torch.int32, "xt")
    _need(codes, torch.uint8, "codes")
    _need(p_doc, torch.float64, "p_doc")
    _need(doc_counts, torch.int32, "doc_counts")
    n_docs = cu_seqlens.numel() - 1
    _check(load().mdlm_corrupt_mixture(_ptr(x0), x0.numel(), _ptr(cu_seqlens), n_docs,
                                       int(seed) & 0xFFFFFFFFFFFFFFFF, float(eps),
                                       float(mixture_prob), int(mask_id), int(rand_vocab),
                                       _ptr(xt), _ptr(codes), _ptr(p_doc), _ptr(doc_counts),
                                       _stream(stream)))


def mdlm_corrupt_compact_workspace_bytes(n_tokens):
    return load().mdlm_corrupt_compact_workspace_bytes(int(n_tokens))


def mdlm_corrupt_compact(x0, cu_seqlens, seed, eps, noise, mask_id, rand_vocab, align, xt,
                         corrupted, p_doc, doc_counts, row_idx, tgt, w, n_rows, workspace,
                         stream=None):
    """See mdlm_corrupt_compact in include/mdlm.h.  `corrupted` may be None;
    `workspace` is a uint8 tensor."""
    _need(x0, torch.int32, "x0")
    _need(cu_seqlens, torch.int32, "cu_seqlens")
    _need(xt, torch.int32, "xt")
    _need(corrupted, torch.uint8, "corrupted")
    _need(p_doc, torch.float64, "p_doc")
    _need(doc_counts, torch.int32, "doc_counts")
    _need(row_idx, torch.int32, "row_idx")
    _need(tgt, torch.int32, "tgt")
    _need(w, torch.float32, "w")
    _need(n_rows, torch.int32, "n_rows")
    _need(workspace, torch.uint8, "workspace")
    ws_bytes = 0 if workspace is None else workspace.numel()
    _check(load().mdlm_corrupt_compact(
        _ptr(x0), x0.numel(), _ptr(cu_seqlens), cu_seqlens.numel() - 1,
        int(seed) & 0xFFFFFFFFFFFFFFFF, float(eps), int(noise), int(mask_id), int(rand_vocab),
        int(align), _ptr(xt), _ptr(corrupted), _ptr(p_doc), _ptr(doc_counts), _ptr(row_idx),
        _ptr(tgt), _ptr(w), _ptr(n_rows), _ptr(workspace), ws_bytes, _stream(stream)))


def mdlm_compact_workspace_bytes(n_tokens):
    return load().mdlm_compact_workspace_bytes(int(n_tokens))


def mdlm_compact_masked(corrupted, x0, cu_seqlens, p_doc, align, row_idx, tgt, w, n_rows,
                        workspace, stream=None):
    """See mdlm_compact_masked in include/mdlm.h.  `workspace` is a uint8 tensor."""
    _need(corrupted, torch.uint8, "corrupted")
    _need(x0, torch.int32, "x0")
    _need(cu_seqlens, torch.int32, "cu_seqlens")
    _need(p_doc, torch.float64, "p_doc")
    _need(row_idx, torch.int32, "row_idx")
    _need(tgt, torch.int32, "tgt")
    _need(w, torch.float32, "w")
    _need(n_rows, torch.int32, "n_rows")
    _need(workspace, torch.uint8, "workspace")
    ws_bytes = 0 if workspace is None else workspace.numel()
    _check(load().mdlm_compact_masked(_ptr(corrupted), _ptr(x0), x0.numel(), _ptr(cu_seqlens),
                                      cu_seqlens.numel() - 1, _ptr(p_doc), int(align),
                                      _ptr(row_idx), _ptr(tgt), _ptr(w), _ptr(n_rows),
                                      _ptr(workspace), ws_bytes, _stream(stream)))


def mdlm_compact_masked_noalloc(corrupted, x0, cu_seqlens, p_doc, align, row_idx, tgt, w,
                                n_rows, stream=None):
    """See mdlm_compact_masked_noalloc in include/mdlm.h (no workspace)."""
    _need(corrupted, torch.uint8, "corrupted")
    _need(x0, torch.int32, "x0")
    _need(cu_seqlens, torch.int32, "cu_seqlens")
    _need(p_doc, torch.float64, "p_doc")
    _need(row_idx, torch.int32, "row_idx")
    _need(tgt, torch.int32, "tgt")
    _need(w, torch.float32, "w")
    _need(n_rows, torch.int32, "n_rows")
    _check(load().mdlm_compact_masked_noalloc(
        _ptr(corrupted), _ptr(x0), x0.numel(), _ptr(cu_seqlens), cu_seqlens.numel() - 1,
        _ptr(p_doc), int(align), _ptr(row_idx), _ptr(tgt), _ptr(w), _ptr(n_rows),
        _stream(stream)))


def mdlm_compact_corrective(codes, x0, cu_seqlens, p_doc, align, noise_token_wt,
                            clean_token_wt, row_idx, tgt, w, n_rows, workspace, stream=None):
    """See mdlm_compact_corrective in include/mdlm.h.  `workspace` is a uint8
    tensor of mdlm_compact_workspace_bytes(n_tokens) bytes."""
    _need(codes, torch.uint8, "codes")
    _need(x0, torch.int32, "x0")
    _need(cu_seqlens, torch.int32, "cu_seqlens")
    _need(p_doc, torch.float64, "p_doc")
    _need(row_idx, torch.int32, "row_idx")
    _need(tgt, torch.int32, "tgt")
    _need(w, torch.float32, "w")
    _need(n_rows, torch.int32, "n_rows")
    _need(workspace, torch.uint8, "workspace")
    ws_bytes = 0 if workspace is None else workspace.numel()
    _check(load().mdlm_compact_corrective(
        _ptr(codes), _ptr(x0), x0.numel(), _ptr(cu_seqlens), cu_seqlens.numel() - 1,
        _ptr(p_doc), int(align), float(noise_token_wt), float(clean_token_wt), _ptr(row_idx),
        _ptr(tgt), _ptr(w), _ptr(n_rows), _ptr(workspace), ws_bytes, _stream(stream)))


def mdlm_compact_rows_workspace_bytes(n_tokens, n_docs, weighting):
    return load().mdlm_compact_rows_workspace_bytes(int(n_tokens), int(n_docs), int(weighting))


def mdlm_compact_rows(corrupted, eligible, x0, cu_seqlens, p_doc, align, weighting,
                      weight_scale, weight_clip, row_idx, tgt, w, n_rows, workspace,
                      stream=None):
    """See mdlm_compact_rows in include/mdlm.h.  `corrupted`, `eligible` and
    `p_doc` may be None; `workspace` is a uint8 tensor."""
    _need(corrupted, torch.uint8, "corrupted")
    _need(eligible, torch.uint8, "eligible")
    _need(x0, torch.int32, "x0")
    _need(cu_seqlens, torch.int32, "cu_seqlens")
    _need(p_doc, torch.float64, "p_doc")
    _need(row_idx, torch.int32, "row_idx")
    _need(tgt, torch.int32, "tgt")
    _need(w, torch.float32, "w")
    _need(n_rows, torch.int32, "n_rows")
    _need(workspace, torch.uint8, "workspace")
    ws_bytes = 0 if workspace is None else workspace.numel()
    _check(load().mdlm_compact_rows(
        _ptr(corrupted), _ptr(eligible), _ptr(x0), x0.numel(), _ptr(cu_seqlens),
        cu_seqlens.numel() - 1, _ptr(p_doc), int(align), int(weighting), float(weight_scale),
        float(weight_clip), _ptr(row_idx), _ptr(tgt), _ptr(w), _ptr(n_rows), _ptr(workspace),
        ws_bytes, _stream(stream)))


def dtype_code(t):
    if t.dtype == torch.bfloat16:
        return MDLM_BF16
    if t.dtype == torch.float32:
        return MDLM_F32
    raise TypeError(f"unsupported element type {t.dtype}")


def mdlm_head_ce_workspace_bytes(max_rows, H, V, dtype):
    return load().mdlm_head_ce_workspace_bytes(int(max_rows), int(H), int(V), int(dtype))


def mdlm_head_ce_workspace_min_bytes(max_rows, H, V, dtype):
    return load().mdlm_head_ce_workspace_min_bytes(int(max_rows), int(H), int(V), int(dtype))


def mdlm_fused_head_ce_fwd_bwd(hidden, W, row_idx, tgt, w, n_rows, max_rows, softcap, loss,
                               row_ce, d_hidden, workspace, stream=None):
    """See mdlm_fused_head_ce_fwd_bwd in include/mdlm.h.  `d_hidden` and
    `row_ce` may be None; `workspace` is a uint8 tensor."""
    dt = dtype_code(hidden)
    _need(hidden, hidden.dtype, "hidden")
    _need(W, hidden.dtype, "W")
    _need(row_idx, torch.int32, "row_idx")
    _need(tgt, torch.int32, "tgt")
    _need(w, torch.float32, "w")
    _need(n_rows, torch.int32, "n_rows")
    _need(loss, torch.float32, "loss")
    _need(row_ce, torch.float32, "row_ce")
    _need(d_hidden, hidden.dtype, "d_hidden")
    _need(workspace, torch.uint8, "workspace")
    n_tokens, H = hidden.shape
    V = W.shape[0]
    if W.shape[1] != H:
        raise ValueError("W must be [V, H] with the hidden size of `hidden`")
    if d_hidden is not None and tuple(d_hidden.shape) != tuple(hidden.shape):
        raise ValueError("d_hidden must have the shape of hidden")
    ws_bytes = 0 if workspace is None else workspace.numel()
    _check(load().mdlm_fused_head_ce_fwd_bwd(
        _ptr(hidden), _ptr(W), dt, n_tokens, H, V, _ptr(row_idx), _ptr(tgt), _ptr(w),
        _ptr(n_rows), int(max_rows), float(softcap), _ptr(loss), _ptr(row_ce), _ptr(d_hidden),
        _ptr(workspace), ws_bytes, _stream(stream)))


def mdlm_head_ce_dw_workspace_bytes(max_rows, H, V):
    return load().mdlm_head_ce_dw_workspace_bytes(int(max_rows), int(H), int(V))


def mdlm_head_ce_dw_workspace_min_bytes(max_rows, H, V):
    return load().mdlm_head_ce_dw_workspace_min_bytes(int(max_rows), int(H), int(V))


def mdlm_fused_head_ce_fwd_bwd_dw(hidden, W, row_idx, tgt, w, n_rows, max_rows, softcap, loss,
                                  row_ce, d_hidden, dW, workspace, stream=None):
    """See mdlm_fused_head_ce_fwd_bwd_dw in include/mdlm.h (bf16 only).
    `d_hidden` and `row_ce` may be None; `dW` is a float32 [V, H] tensor."""
    if hidden.dtype != torch.bfloat16:
        raise TypeError("mdlm_fused_head_ce_fwd_bwd_dw takes bf16 hidden and W")
    _need(hidden, torch.bfloat16, "hidden")
    _need(W, torch.bfloat16, "W")
    _need(row_idx, torch.int32, "row_idx")
    _need(tgt, torch.int32, "tgt")
    _need(w, torch.float32, "w")
    _need(n_rows, torch.int32, "n_rows")
    _need(loss, torch.float32, "loss")
    _need(row_ce, torch.float32, "row_ce")
    _need(d_hidden, torch.bfloat16, "d_hidden")
    _need(dW, torch.float32, "dW")
    _need(workspace, torch.uint8, "workspace")
    n_tokens, H = hidden.shape
    V = W.shape[0]
    if W.shape[1] != H or dW is None or tuple(dW.shape) != (V, H):
        raise ValueError("W and dW must be [V, H] with the hidden size of `hidden`")
    if d_hidden is not None and tuple(d_hidden.shape) != tuple(hidden.shape):
        raise ValueError("d_hidden must have the shape of hidden")
    ws_bytes = 0 if workspace is None else workspace.numel()
    _check(load().mdlm_fused_head_ce_fwd_bwd_dw(
        _ptr(hidden), _ptr(W), n_tokens, H, V, _ptr(row_idx), _ptr(tgt), _ptr(w), _ptr(n_rows),
        int(max_rows), float(softcap), _ptr(loss), _ptr(row_ce), _ptr(d_hidden), _ptr(dW),
        _ptr(workspace), ws_bytes, _stream(stream)))


def mdlm_scale(x, y, scale, stream=None):
    """See mdlm_scale in include/mdlm.h: y = scale * x for bf16 or float32
    tensors of one size (y may be x); `scale` a one-element float32 device
    tensor."""
    dt = dtype_code(x)
    _need(x, x.dtype, "x")
    _need(y, x.dtype, "y")
    _need(scale, torch.float32, "scale")
    if y.numel() != x.numel():
        raise ValueError("x and y must have as many entries")
    _check(load().mdlm_scale(_ptr(x), _ptr(y), dt, x.numel(), _ptr(scale), _stream(stream)))


def mdlm_check_offsets(cu_seqlens, n_tokens, status, stream=None):
    """See mdlm_check_offsets in include/mdlm.h: ORs violation bits into the
    one-element int32 device tensor `status`."""
    _need(cu_seqlens, torch.int32, "cu_seqlens")
    _need(status, torch.int32, "status")
    _check(load().mdlm_check_offsets(_ptr(cu_seqlens), cu_seqlens.numel() - 1, int(n_tokens),
                                     _ptr(status), _stream(stream)))


def mdlm_check_probs(p_doc, status, stream=None):
    """See mdlm_check_probs in include/mdlm.h."""
    _need(p_doc, torch.float64, "p_doc")
    _need(status, torch.int32, "status")
    _check(load().mdlm_check_probs(_ptr(p_doc), p_doc.numel(), _ptr(status), _stream(stream)))


def mdlm_check_rows(row_idx, tgt, w, n_rows, max_rows, n_tokens, V, status, stream=None):
    """See mdlm_check_rows in include/mdlm.h; `tgt` and `w` may be None."""
    _need(row_idx, torch.int32, "row_idx")
    _need(tgt, torch.int32, "tgt")
    _need(w, torch.float32, "w")
    _need(n_rows, torch.int32, "n_rows")
    _need(status, torch.int32, "status")
    _check(load().mdlm_check_rows(_ptr(row_idx), _ptr(tgt), _ptr(w), _ptr(n_rows),
                                  int(max_rows), int(n_tokens), int(V), _ptr(status),
                                  _stream(stream)))


def mdlm_set_checking(enable):
    """See mdlm_set_checking in include/mdlm.h; returns the previous setting."""
    return bool(load().mdlm_set_checking(1 if enable else 0))
