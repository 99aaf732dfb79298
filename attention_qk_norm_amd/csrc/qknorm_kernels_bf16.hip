// qknorm_kernels_bf16.hip -- the bfloat16 instantiation of the gfx950 kernels.
#include "qknorm_kernels.h"

namespace qkn {

hipError_t launch_bf16(const Variant& v, const Args& a, dim3 grid, unsigned lds_bytes, hipStream_t stream) {
  return launch_dtype<BF16>(v, a, grid, lds_bytes, stream);
}

}  // namespace qkn
