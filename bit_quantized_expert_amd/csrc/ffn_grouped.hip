// Grouped-GEMM expert FFN for prefill (placeholder until the MFMA kernel
// lands): reports "not supported" so callers select the GEMV path.
#include "common.h"
#include "launch.h"

namespace moe {

hipError_t launch_ffn_grouped(const FfnArgs&, int, int64_t, hipStream_t) { return hipErrorNotSupported; }

}  // namespace moe
