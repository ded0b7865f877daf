// placeholder, replaced below
#include <hip/hip_runtime.h>
#include "attn_internal.h"
namespace attn {
bool prefill_supported(int D) { return false; }
hipError_t launch_prefill(const PrefillArgs&, hipStream_t) { return hipErrorInvalidValue; }
}
