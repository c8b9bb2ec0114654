// vq_gemm_b11.hip -- MFMA GEMM kernels for 11-bit codes (K = 2048); see vq_gemm_impl.h.
#include "vq_gemm_impl.h"

namespace vqmi {
VQMI_GEMM_UNIT(11)
}  // namespace vqmi
