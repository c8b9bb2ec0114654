// vq_gemm_b09.hip -- MFMA GEMM kernels for 9-bit codes (K = 512); see vq_gemm_impl.h.
#include "vq_gemm_impl.h"

namespace vqmi {
VQMI_GEMM_UNIT(9)
}  // namespace vqmi
