// Chunked prefill (placeholder until the kernels land).
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
size_t prefill_workspace_bytes(int, int, int, int, int) { return 0; }
hipError_t launch_prefill(PrefillArgs &, void *, hipStream_t) { return hipErrorNotSupported; }
}  // namespace kda
