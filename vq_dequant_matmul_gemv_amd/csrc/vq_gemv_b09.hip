// vq_gemv_b09.hip -- GEMV and dequant kernels for 9-bit codes (K = 512); see vq_gemv_impl.h.
#include "vq_gemv_impl.h"

namespace vqmi {
VQMI_GEMV_UNIT(9)
}  // namespace vqmi
