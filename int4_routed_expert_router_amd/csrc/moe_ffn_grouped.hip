// Batched grouped-GEMM family (matrix cores) - placeholder until written.
#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {
hipError_t launch_gateup_grouped(int, const FfnArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_down_grouped(const FfnArgs&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace moe
