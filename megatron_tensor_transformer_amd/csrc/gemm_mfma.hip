// Prefill projections on bf16 MFMA (gfx950). Placeholder until the MFMA GEMM
// lands: reports no supported shape, so every projection takes the GEMV path.
#include "kernels.h"

namespace tpk {

bool gemm_supported(int, int, int, int) { return false; }

hipError_t gemm_launch(const GemmArgs&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace tpk
