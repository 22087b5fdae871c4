// FP8-operand kernels (X in E4M3, dY in E4M3): fused weight-gradient + optimizer
// step for four of the optimizers.
#include "forge_gemm_kernel.h"

namespace forge {
FORGE_INST_F8(FORGE_RMSPROP, 0)
FORGE_INST_F8(FORGE_ADAGRAD, 0)
FORGE_INST_F8(FORGE_NADAM, 0)
FORGE_INST_F8(FORGE_RADAM, 0)

}  // namespace forge
