// vq_gemv_b13.hip -- GEMV and dequant kernels for 13-bit codes (K = 8192); see vq_gemv_impl.h.
#include "vq_gemv_impl.h"

namespace vqmi {
VQMI_GEMV_UNIT(13)
}  // namespace vqmi
