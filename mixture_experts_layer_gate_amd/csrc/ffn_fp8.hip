// Grouped SwiGLU expert FFN with fp8 (E4M3) operands: placeholder until the
// MFMA fp8 kernels land; the call reports "not supported".
#include "common.h"
#include "launch.h"

namespace moe {

hipError_t launch_ffn_fp8_gate_up(const FfnArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_ffn_fp8_down(const FfnArgs&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace moe
