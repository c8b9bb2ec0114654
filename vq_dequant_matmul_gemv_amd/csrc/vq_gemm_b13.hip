// vq_gemm_b13.hip -- MFMA GEMM kernels for 13-bit codes (K = 8192); see vq_gemm_impl.h.
#include "vq_gemm_impl.h"

namespace vqmi {
VQMI_GEMM_UNIT(13)
}  // namespace vqmi
