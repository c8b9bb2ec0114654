// vq_gemm_b06.hip -- MFMA GEMM kernels for 6-bit codes (K = 64); see vq_gemm_impl.h.
#include "vq_gemm_impl.h"

namespace vqmi {
VQMI_GEMM_UNIT(6)
}  // namespace vqmi
