"""CPU oracle for the fused weight-gradient + optimizer step (test infrastructure).

This package is the plain, slow, float64 statement of what the fused path
computes. It exists only to check the HIP path: the tests, the smoke check and
the CPU-baseline leg of the benchmark may import it; the product path never
does, and the product never falls back to it. It shares no code with the HIP
library (no kernels, headers, constants, tables or helpers). Its inputs come
from the seeded generators in ``synth`` or from the caller.

Sources are the FORGE explainer pages ("FORGE: Fused On-Register Gradient
Elimination for Memory-Efficient LLM Training", technical summary, §2 Method).
The pages give no equations, RNG, rounding rule or quantiser; where they are
silent the readings used here are stated in each function.

Parity status of each function (what pins it independently of itself):
  gemm.wgrad / gemm.dgrad       brute force with math.fsum; one-hot closed forms
  optim.update (7 of 8)         torch.optim float64 cross-check + closed forms
  optim.update("lion")          closed forms only (no library implementation here)
  rounding.splitmix64           published SplitMix64 output sequence
  rounding.sr_bf16              counting identity + value-based SR definition
  q8.*                          codec invariants; block-64 < block-2048 error
  step.wgrad_step               composition of the above; tile-wise == full
End-to-end values of the method have no printed worked example on the pages.
"""
from . import gemm, optim, rounding, q8, step  # noqa: F401
