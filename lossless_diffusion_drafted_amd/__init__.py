"""MI355X-native hot path of Uno (Psi-Spec) block draft-and-verify decoding.

The compute lives in libuno.so (hand-written HIP kernels for gfx950 behind the C
ABI in include/uno.h); this package only marshals torch tensors into it.
"""

from ._lib import (FLAG_OVERFLOW, FLAG_Q_ZERO, FLAG_RES_ZERO, FLAG_TIE_ACCEPT,  # noqa: F401
                   FLAG_TIE_ICDF, FLAG_TIE_MASK, FLAG_TIE_TOPP_P, FLAG_TIE_TOPP_Q,
                   LIB_PATH, UnoError, load)
from .ops import (PROJECTIONS, Model, sampling_params, uno_ar_step, uno_decode_step,  # noqa: F401
                  uno_draft_sample, uno_forward, uno_gated_lora_linear, uno_gated_lora_linear_bwd,
                  uno_tv_loss_fwd_bwd, uno_verify_block, uno_verify_block_noalloc)

__all__ = ["uno_verify_block", "uno_verify_block_noalloc", "uno_draft_sample", "uno_tv_loss_fwd_bwd",
           "uno_gated_lora_linear", "uno_gated_lora_linear_bwd", "uno_forward", "uno_decode_step", "uno_ar_step",
           "Model", "PROJECTIONS", "sampling_params", "load", "UnoError", "LIB_PATH"]
