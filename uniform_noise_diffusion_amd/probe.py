"""ctypes binding of libmdlm_probe.so (include/mdlm_probe.h): the streaming
copy and the MFMA issue loop that give the achievable peaks the loss path is
measured against.  Argument marshalling only; raises if the library has not
been built."""

import ctypes
import os

import torch

PROBE_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmdlm_probe.so")
EXPORTED = ("mdlm_probe_copy", "mdlm_probe_mfma")
MFMA_FLOPS = 32 * 32 * 16 * 2   # one v_mfma_f32_32x32x16_bf16
MFMA_CHAINS = 8                 # MFMAs per wave per iteration
MFMA_WAVES = 8                  # waves per workgroup

_lib = None


def load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(PROBE_LIB_PATH):
        raise RuntimeError(f"{PROBE_LIB_PATH} is missing: build it with "
                           "`python -m uniform_noise_diffusion_amd.build`")
    lib = ctypes.CDLL(PROBE_LIB_PATH)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.mdlm_probe_copy.argtypes = [vp, vp, i64, vp]
    lib.mdlm_probe_copy.restype = ctypes.c_int
    lib.mdlm_probe_mfma.argtypes = [vp, i32, i32, vp]
    lib.mdlm_probe_mfma.restype = ctypes.c_int
    _lib = lib
    return lib


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def copy(src, dst, stream=None):
    """dst <- src for two contiguous 16-byte-aligned device tensors of the
    same byte size (a multiple of 16)."""
    nb = src.numel() * src.element_size()
    assert src.is_cuda and dst.is_cuda and src.is_contiguous() and dst.is_contiguous()
    assert dst.numel() * dst.element_size() == nb and nb % 16 == 0
    assert src.data_ptr() % 16 == 0 and dst.data_ptr() % 16 == 0
    rc = load().mdlm_probe_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()),
                                nb // 16, _stream(stream))
    if rc != 0:
        raise RuntimeError(f"mdlm_probe_copy: HIP error {rc}")


def mfma(out, blocks, iters, stream=None):
    """MFMA issue loop; out: float32 device tensor of at least blocks * 8
    elements.  Returns the flops executed."""
    assert out.is_cuda and out.dtype == torch.float32 and out.numel() >= blocks * MFMA_WAVES
    rc = load().mdlm_probe_mfma(ctypes.c_void_p(out.data_ptr()), blocks, iters, _stream(stream))
    if rc != 0:
        raise RuntimeError(f"mdlm_probe_mfma: HIP error {rc}")
    return blocks * MFMA_WAVES * iters * MFMA_CHAINS * MFMA_FLOPS
