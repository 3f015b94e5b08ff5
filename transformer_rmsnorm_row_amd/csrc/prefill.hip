// bf16 MFMA prefill kernel (placeholder until the tiled MFMA kernel lands).
#include "device_common.h"
#include "launch.h"

namespace qkv {

bool prefill_supports(int, int, int, int, int) { return false; }

hipError_t launch_prefill(const ForwardArgs&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace qkv
