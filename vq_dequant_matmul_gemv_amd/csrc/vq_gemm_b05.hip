// vq_gemm_b05.hip -- MFMA GEMM kernels for 5-bit codes (K = 32); see vq_gemm_impl.h.
#include "vq_gemm_impl.h"

namespace vqmi {
VQMI_GEMM_UNIT(5)
}  // namespace vqmi
