// decode_valu_d256.hip -- the vector split-KV decode kernels for head_dim 256.
#include "decode_valu_impl.h"

namespace ga {
template hipError_t valu_launch_d<256>(const DecodeArgs&, bool, hipStream_t);
}  // namespace ga
