// decode_valu_d128.hip -- the vector split-KV decode kernels for head_dim 128.
#include "decode_valu_impl.h"

namespace ga {
template hipError_t valu_launch_d<128>(const DecodeArgs&, bool, hipStream_t);
}  // namespace ga
