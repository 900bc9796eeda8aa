// prefill.hip -- chunked KDA prefill (not yet built: every request is
// reported as unsupported).
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

bool prefill_supported(int, int, int) { return false; }

size_t prefill_workspace_bytes(int32_t N, int32_t, int64_t, int, int) {
    return (static_cast<size_t>(N) * sizeof(SeqWork) + 255) / 256 * 256;
}

hipError_t launch_prefill(int, int, int, const PrefillParams&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace kda
