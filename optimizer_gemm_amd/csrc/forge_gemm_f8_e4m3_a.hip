// FP8-operand kernels (X in E4M3, dY in E4M3): fused weight-gradient + optimizer
// step for four of the optimizers, and the float32 dW store.
#include "forge_gemm_kernel.h"

namespace forge {
FORGE_INST_F8(FORGE_ADAMW, 0)
FORGE_INST_F8(FORGE_SGD, 0)
FORGE_INST_F8(FORGE_SGD_MOMENTUM, 0)
FORGE_INST_F8(FORGE_LION, 0)
template hipError_t wgrad_store_f8<0>(const GArgs&, hipStream_t);
}  // namespace forge
