// vq_gemm_b04.hip -- MFMA GEMM kernels for 4-bit codes (K = 16); see vq_gemm_impl.h.
#include "vq_gemm_impl.h"

namespace vqmi {
VQMI_GEMM_UNIT(4)
}  // namespace vqmi
