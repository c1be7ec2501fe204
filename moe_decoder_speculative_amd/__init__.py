"""MI355X (gfx950) library for one speculative verification step of a
mixture-of-experts decoder: RMSNorm, top-k softmax router, routed + shared
SwiGLU experts, combine, LM-head greedy pick and longest-prefix acceptance,
all in hand-written HIP kernels behind a C ABI (include/moe_verify.h).

`binding` is the ctypes layer (same names as the C functions); `model` builds
contexts and device tensors from seeded synthetic weights; `synth` draws the
seeded inputs.
"""
from .binding import (  # noqa: F401
    MOE_DTYPE_BF16, MOE_DTYPE_F32, MoeVerifyAux, MoeVerifyConfig, MoeVerifyError, MoeVerifyWeights,
    load_library, make_aux, moe_block_forward, moe_verify_destroy, moe_verify_init,
    moe_verify_last_error, moe_verify_set_stage_events, moe_verify_step, moe_verify_step_ex,
)
