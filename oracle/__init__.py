"""CPU oracle of the Uno (Psi-Spec) block draft-and-verify hot path.

TEST INFRASTRUCTURE ONLY. Only the tests, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this package. The product library
never imports, links or calls it, and it shares no code with the HIP kernels:
both sides read only the seeded inputs produced by ``workloads``.

Every function is plain fp64 numpy written from the pages' statement of the
method (page titles and sections are cited in each module), pinned by the
``-m "not gpu"`` tests to closed forms, exact rational enumeration, library
routines and invariants.
"""

from .philox import noise_token, philox4x64_10, slot_uniforms, word_to_uniform  # noqa: F401
from .sampling import (  # noqa: F401
    EVENT_Q_ZERO, EVENT_RES_ZERO, NEAR_TIE, TIE_ACCEPT, TIE_ICDF, TIE_MASK,
    TIE_TOPP_P, TIE_TOPP_Q, decode_logits, draft_sample, expected_accept_len,
    filter_logits, inverse_cdf, verify_block,
)
from .tv import tv_loss_fwd_bwd  # noqa: F401
from .gated_lora import bf16_bits_to_f64, gated_lora_linear, gated_lora_linear_bwd, lora_delta  # noqa: F401
from . import step  # noqa: F401
