// vq_gemv_b08.hip -- GEMV and dequant kernels for 8-bit codes (K = 256); see vq_gemv_impl.h.
#include "vq_gemv_impl.h"

namespace vqmi {
VQMI_GEMV_UNIT(8)
}  // namespace vqmi
