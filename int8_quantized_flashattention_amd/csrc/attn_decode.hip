// Split-KV decode kernel: not built yet; the schedule never selects it.
#include "attn_internal.h"

namespace attn {
hipError_t launch_decode(const FwdArgs&, int, hipStream_t) { return hipErrorNotSupported; }
}  // namespace attn
