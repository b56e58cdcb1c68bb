// qk_per_head.hip -- the per-head form of the QK kernel: one RMS per (token,
// head) over head_dim channels with one [head_dim] gamma shared by every head,
// the upstream qk-norm that the "Kernel reference: qkv_cte" page contrasts with
// its across-heads norm ("Upstream behavior", Design section 1), followed by the
// same rotate-half RoPE (Design section 2).
#include "qk_kernel.h"

namespace qknr {

hipError_t qk_launch_per_head(const QkParams &p, int elem_type, int vec, int J, hipStream_t stream) {
    return qk_launch_mode<QK_PER_HEAD>(p, elem_type, vec, J, stream);
}

}  // namespace qknr
