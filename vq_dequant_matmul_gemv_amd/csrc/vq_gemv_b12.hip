// vq_gemv_b12.hip -- GEMV and dequant kernels for 12-bit codes (K = 4096); see vq_gemv_impl.h.
#include "vq_gemv_impl.h"

namespace vqmi {
VQMI_GEMV_UNIT(12)
}  // namespace vqmi
