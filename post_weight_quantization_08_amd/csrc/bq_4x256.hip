// Block quantizer kernels of one workgroup shape (see block_quant.h).
#include "block_quant.h"

namespace gq {

void launch_bq_4x256(const QArgs& a, int g, int64_t batch, hipStream_t st) { launch_bq_g<4, 256>(a, g, batch, st); }

}  // namespace gq
