// qknorm_launch.cpp -- launch dispatch on the element type.
#include "qknorm_launch.h"

#include "qknorm.h"

namespace qkn {

hipError_t launch(const Variant& v, const Args& a, dim3 grid, unsigned lds_bytes, hipStream_t stream) {
  switch (v.dtype) {
    case QKNORM_F32: return launch_f32(v, a, grid, lds_bytes, stream);
    case QKNORM_BF16: return launch_bf16(v, a, grid, lds_bytes, stream);
    case QKNORM_FP8_E4M3: return launch_fp8(v, a, grid, lds_bytes, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qkn
