// pa_kernels_bf16.hip -- the decode and merge kernels for bf16 inputs.
#include "pa_kernels.h"

namespace pa_detail {
template hipError_t launch_decode<PA_DTYPE_BF16>(const Params &, int, int, int, int, hipStream_t);
template hipError_t launch_merge<PA_DTYPE_BF16>(const MergeParams &, int, hipStream_t);
}  // namespace pa_detail
