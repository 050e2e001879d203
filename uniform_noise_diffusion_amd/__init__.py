"""Masked-diffusion LM loss on AMD MI355X (gfx950).

The HIP library libmdlm.so (C ABI in include/mdlm.h) implements per-document
noise levels, corruption, ordered compaction of scored rows and the fused
frozen-head + cross-entropy forward and backward.  `binding` exposes its
entry points under the same names; `pipeline` owns the buffers of one step;
`autograd` wraps the fused call as a differentiable loss.
"""

from .binding import (  # noqa: F401
    MdlmError,
    MDLM_OK, MDLM_EINVAL, MDLM_EUNSUPPORTED, MDLM_EWORKSPACE, MDLM_EHIP,
    MDLM_NOISE_ABSORB, MDLM_NOISE_UNIFORM, MDLM_ALIGNED, MDLM_SHIFTED,
    MDLM_F32, MDLM_BF16, MDLM_CODE_CLEAN, MDLM_CODE_MASKED, MDLM_CODE_REPLACED,
    mdlm_corrupt, mdlm_corrupt_mixture, mdlm_compact_workspace_bytes, mdlm_compact_masked,
    mdlm_compact_corrective,
    mdlm_head_ce_workspace_bytes, mdlm_head_ce_workspace_min_bytes,
    mdlm_fused_head_ce_fwd_bwd, mdlm_last_error, mdlm_version,
)
from .pipeline import MdlmLossStep  # noqa: F401
from .autograd import FusedHeadCE, masked_diffusion_loss  # noqa: F401
