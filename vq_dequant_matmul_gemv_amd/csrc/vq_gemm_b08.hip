// vq_gemm_b08.hip -- MFMA GEMM kernels for 8-bit codes (K = 256); see vq_gemm_impl.h.
#include "vq_gemm_impl.h"

namespace vqmi {
VQMI_GEMM_UNIT(8)
}  // namespace vqmi
