// qk_split.hip -- the two passes of the across-heads norm when the heads of a
// segment are split over ranks ("Kernel reference: qkv_cte", Design section
// 1): QK_SUMSQ is step a (each token's sum of squares over this rank's heads,
// per segment) and QK_APPLY is step c (gamma and RoPE with the inverse RMS of
// step b, computed from the ranks' added sums and the whole segment's channel
// count). The addition itself (an all-reduce of 4 bytes per token and segment)
// belongs to the caller.
#include "qk_kernel.h"

namespace qknr {

hipError_t qk_launch_split(const QkParams &p, int elem_type, int vec, int J, int mode, hipStream_t stream) {
    if (mode == QK_SUMSQ) return qk_launch_mode<QK_SUMSQ>(p, elem_type, vec, J, stream);
    if (mode == QK_APPLY) return qk_launch_mode<QK_APPLY>(p, elem_type, vec, J, stream);
    return hipErrorInvalidValue;
}

}  // namespace qknr
