// pa_kernels_f32.hip -- the decode and merge kernels for fp32 inputs.
#include "pa_kernels.h"

namespace pa_detail {
template hipError_t launch_decode<PA_DTYPE_F32>(const Params &, int, int, int, int, hipStream_t);
template hipError_t launch_merge<PA_DTYPE_F32>(const MergeParams &, int, hipStream_t);
}  // namespace pa_detail
