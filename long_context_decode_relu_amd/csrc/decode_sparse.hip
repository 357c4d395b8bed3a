// Sparse-layer gather-softmax decode (placeholder until the kernel lands).
#include "kernels.h"

namespace ssa {
size_t decode_sparse_ws_bytes(int, int, int, int, int) { return 0; }
hipError_t launch_decode_sparse(const DecodeSparseArgs&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace ssa
