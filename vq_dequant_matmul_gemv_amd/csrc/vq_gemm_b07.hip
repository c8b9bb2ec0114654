// vq_gemm_b07.hip -- MFMA GEMM kernels for 7-bit codes (K = 128); see vq_gemm_impl.h.
#include "vq_gemm_impl.h"

namespace vqmi {
VQMI_GEMM_UNIT(7)
}  // namespace vqmi
