// Top-k + recent selection (placeholder until the radix-select kernel lands).
#include "kernels.h"

namespace ssa {
size_t select_ws_bytes(int, int, int, int) { return 0; }
hipError_t launch_select(const SelectArgs&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace ssa
