// Fused weight-gradient + optimizer kernels on bf16 / fp32 operands for two of the
// optimizers (one translation unit per pair, so the library builds in parallel).
#include "forge_gemm_kernel.h"

namespace forge {
FORGE_INST_BF16(FORGE_SGD_MOMENTUM)
FORGE_INST_BF16(FORGE_LION)
}  // namespace forge
