// decode_valu_d512.hip -- the vector split-KV decode kernels for head_dim 512.
#include "decode_valu_impl.h"

namespace ga {
template hipError_t valu_launch_d<512>(const DecodeArgs&, bool, hipStream_t);
}  // namespace ga
