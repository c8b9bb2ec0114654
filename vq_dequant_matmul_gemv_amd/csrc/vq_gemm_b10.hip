// vq_gemm_b10.hip -- MFMA GEMM kernels for 10-bit codes (K = 1024); see vq_gemm_impl.h.
#include "vq_gemm_impl.h"

namespace vqmi {
VQMI_GEMM_UNIT(10)
}  // namespace vqmi
