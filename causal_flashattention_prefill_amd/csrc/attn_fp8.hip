// Causal forward attention, FP8 e4m3fn inputs (placeholder until the FP8
// kernel lands: reports "not supported").
#include "device_common.h"
#include "zyfa_internal.h"

namespace zyfa {
hipError_t launch_attn_fp8(const AttnArgs&, int, bool, int, hipStream_t) { return hipErrorNotSupported; }
}  // namespace zyfa
