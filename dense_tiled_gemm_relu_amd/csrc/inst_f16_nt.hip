// Kernel instances for one input type and B layout (all tile configurations,
// all three output types).
#include "configs.hpp"

GEMM_RELU_DEFINE_LAUNCHER(launcher_f16_nt, DT_F16, true)
