// Kernel instances for one input type and B layout (all tile configurations,
// all three output types).
#include "configs.hpp"

GEMM_RELU_DEFINE_LAUNCHER(launcher_bf16_nt, DT_BF16, true)
