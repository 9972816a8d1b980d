// Kernel instances for one block-scaled (MX) element format, B stored (N,K)
// (the two-stage direct configurations, all three output types).
#include "configs.hpp"

GEMM_RELU_DEFINE_LAUNCHER_MX(launcher_mx_e4m3, DT_MX_E4M3)
