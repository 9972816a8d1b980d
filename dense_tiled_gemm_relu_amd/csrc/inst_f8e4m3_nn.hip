// Kernel instances for one 8-bit input type and B layout (the configurations
// plan selection uses, all three output types).
#include "configs.hpp"

GEMM_RELU_DEFINE_LAUNCHER_FP8(launcher_f8e4m3_nn, DT_F8E4M3, false)
