"""MI355X (gfx950) fused weight-gradient + optimizer step (FORGE) behind a C ABI.

The kernels live in libforge.so (optimizer_gemm_amd/csrc, declared in
include/forge.h); this package only builds and binds them.
"""
from .forge import (  # noqa: F401
    OPTIMIZERS, SLOTS, ForgeError, default_hyper, dgrad, describe, lib, make_hyper, new_states,
    optimizer_step, rand16, sr_bf16, status_str, step_scalars, version, wgrad, wgrad_step, wgrad_unfused,
    wgrad_unfused_noalloc, wgrad_step_group, MAX_GROUP,
    dyn_value, dyn_encode, mfma_peak,
)
