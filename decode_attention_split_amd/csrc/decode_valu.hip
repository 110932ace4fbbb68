// decode_valu.hip -- dispatch of the vector split-KV decode by head dim.  The kernels
// are instantiated in decode_valu_d128.hip, decode_valu_d256.hip and decode_valu_d512.hip
// (one head dim each, so they compile in parallel); see decode_valu_impl.h.
#include "decode_valu_impl.h"

namespace ga {

extern template hipError_t valu_launch_d<128>(const DecodeArgs&, bool, hipStream_t);
extern template hipError_t valu_launch_d<256>(const DecodeArgs&, bool, hipStream_t);
extern template hipError_t valu_launch_d<512>(const DecodeArgs&, bool, hipStream_t);

bool decode_valu_supported(int D, int G) {
  return (D == 128 || D == 256 || D == 512) && (G == 1 || G == 2 || G == 4 || G == 8 || G == 16);
}

hipError_t decode_valu_launch(const DecodeArgs& a, bool k_eq_v, hipStream_t stream) {
  if (a.D == 128) return valu_launch_d<128>(a, k_eq_v, stream);
  if (a.D == 256) return valu_launch_d<256>(a, k_eq_v, stream);
  if (a.D == 512) return valu_launch_d<512>(a, k_eq_v, stream);
  return hipErrorInvalidValue;
}

}  // namespace ga
