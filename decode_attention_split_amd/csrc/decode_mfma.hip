// decode_mfma.hip -- matrix-core split-KV decode for the K = V global geometry.
// (Filled in after the vector path is measured.)
#include "ga_device.h"
#include "ga_internal.h"

namespace ga {

bool decode_mfma_supported(int, int, bool) { return false; }
int decode_mfma_keys_per_iter() { return 64; }
hipError_t decode_mfma_launch(const DecodeArgs&, hipStream_t) { return hipErrorInvalidValue; }

}  // namespace ga
