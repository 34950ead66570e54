// Q8_0 matvec kernel instances with 8-column lane rows (m_tile 1..4).
#include "q8_gemv_kernel.h"

namespace q8 {

GemvKernel gemv_kernel_v8(int m_tile) { return pick_m_tile<8>(m_tile); }

}  // namespace q8
