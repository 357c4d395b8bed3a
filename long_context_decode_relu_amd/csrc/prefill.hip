// Chunked ReLU^2 prefill on the matrix cores (placeholder until the kernel lands).
#include "kernels.h"

namespace ssa {
size_t prefill_ws_bytes(int, int, int, int, int) { return 0; }
hipError_t launch_prefill(const PrefillArgs&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace ssa
