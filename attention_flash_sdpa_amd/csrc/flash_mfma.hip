// bf16 MFMA flash-attention kernels for gfx950 (placeholder until built).
#include "common.h"

namespace sdpa {
bool flash_mfma_supports(const FwdParams&) { return false; }
hipError_t launch_flash_mfma(const FwdParams&, hipStream_t) { return hipErrorInvalidDeviceFunction; }
}  // namespace sdpa
