// Fused read-once verification path (not yet enabled).
#include "verify_internal.hpp"

namespace specv {
size_t fused_workspace_bytes(int, int, int, int) { return 0; }
bool fused_supported(int, int, int, int) { return false; }
hipError_t fused_launch(const VerifyArgs&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace specv
