// vq_gemv_b10.hip -- GEMV and dequant kernels for 10-bit codes (K = 1024); see vq_gemv_impl.h.
#include "vq_gemv_impl.h"

namespace vqmi {
VQMI_GEMV_UNIT(10)
}  // namespace vqmi
