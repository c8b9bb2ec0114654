// vq_gemv_b05.hip -- GEMV and dequant kernels for 5-bit codes (K = 32); see vq_gemv_impl.h.
#include "vq_gemv_impl.h"

namespace vqmi {
VQMI_GEMV_UNIT(5)
}  // namespace vqmi
