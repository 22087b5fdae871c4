// FP8-operand kernels (X in E4M3, dY in E5M2): fused weight-gradient + optimizer
// step for four of the optimizers.
#include "forge_gemm_kernel.h"

namespace forge {
FORGE_INST_F8(FORGE_RMSPROP, 1)
FORGE_INST_F8(FORGE_ADAGRAD, 1)
FORGE_INST_F8(FORGE_NADAM, 1)
FORGE_INST_F8(FORGE_RADAM, 1)

}  // namespace forge
