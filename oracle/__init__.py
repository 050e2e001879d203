"""Plain fp64 CPU oracle for the masked-diffusion loss path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product package may import, call,
link or execute anything under this directory; only the test-suite, the smoke
check in ``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` use it.

The oracle is written from the pages' definitions and shares no code with the
HIP library (no common helpers, tables or constants).  It is deliberately slow
and obvious: numpy in float64, one library matmul per V-chunk, no fusion.

Sources for what is computed:
  * LLaDA-8B-MDLM-LoRA model card, "Training" table, "Objective" row:
    t ~ U(0,1) per sequence, mask probability p = (1-1e-3) t + 1e-3,
    cross-entropy on masked tokens divided by p.
  * diffusiongemma-26B-A4B-it-ALWAYS-THINK, "Finetuning notes": corrupt
    positions with uniform-random vocabulary ids at a per-example rate
    t ~ U(eps, 1), no mask token; the logit softcap is applied exactly once.
  * Native diffusion language-model training (Axolotl docs): model table
    (aligned vs shifted logits; inverse-time weighted CE), "Packed training"
    (documents stay isolated; padding is excluded from loss) and
    "Adapters, merging and inference" (full-vocabulary CE from hidden states
    through a plain linear output head, aligned targets).
  * LLaDA-8B-MDLM-LoRA model card, "Training" table, "Objective" row: the
    corrective mixture's option names (mixture_prob, noise_token_wt,
    clean_token_wt), all 0 for the MDLM objective.  No formula is given:
    ``corrupt_mixture`` and ``compact_corrective`` take a stated reading and
    are pinned only through their reductions (mixture 0 = absorbing noise,
    mixture 1 = the uniform-noise ids, zero weights = the MDLM row list) and
    the mixture's frequency; beyond those, parity unpinned.
"""

from .philox import philox4x32_10  # noqa: F401
from .mdlm import (  # noqa: F401
    NOISE_ABSORB,
    NOISE_UNIFORM,
    ALIGNED,
    SHIFTED,
    noise_levels,
    corrupt,
    compact,
    compact_rows,
    corrupt_mixture,
    compact_corrective,
    CODE_CLEAN,
    CODE_MASKED,
    CODE_REPLACED,
    WEIGHT_INV_P,
    WEIGHT_MEAN,
    WEIGHT_EXAMPLE_MEAN_CLIPPED,
    head_ce,
    head_ce_weight_grad,
    head_ce_rows,
    mdlm_loss,
)
