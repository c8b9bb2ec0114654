// vq_gemm_b14.hip -- MFMA GEMM kernels for 14-bit codes (K = 16384); see vq_gemm_impl.h.
#include "vq_gemm_impl.h"

namespace vqmi {
VQMI_GEMM_UNIT(14)
}  // namespace vqmi
