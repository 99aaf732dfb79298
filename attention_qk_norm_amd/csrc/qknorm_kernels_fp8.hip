// qknorm_kernels_fp8.hip -- the FP8 E4M3 instantiation of the gfx950 kernels.
#include "qknorm_kernels.h"

namespace qkn {

hipError_t launch_fp8(const Variant& v, const Args& a, dim3 grid, unsigned lds_bytes, hipStream_t stream) {
  return launch_dtype<FP8>(v, a, grid, lds_bytes, stream);
}

}  // namespace qkn
