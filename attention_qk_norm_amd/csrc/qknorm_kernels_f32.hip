// qknorm_kernels_f32.hip -- the binary32 instantiation of the gfx950 kernels.
#include "qknorm_kernels.h"

namespace qkn {

hipError_t launch_f32(const Variant& v, const Args& a, dim3 grid, unsigned lds_bytes, hipStream_t stream) {
  return launch_dtype<F32>(v, a, grid, lds_bytes, stream);
}

}  // namespace qkn
