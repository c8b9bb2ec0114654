// vq_gemm_b12.hip -- MFMA GEMM kernels for 12-bit codes (K = 4096); see vq_gemm_impl.h.
#include "vq_gemm_impl.h"

namespace vqmi {
VQMI_GEMM_UNIT(12)
}  // namespace vqmi
