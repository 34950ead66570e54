// Q8_0 matvec kernel instances with 2-column lane rows (m_tile 1..8).
#include "q8_gemv_kernel.h"

namespace q8 {

GemvKernel gemv_kernel_v2(int m_tile) { return pick_m_tile<2>(m_tile); }

}  // namespace q8
