// qk_across_heads.hip -- the across-heads form of the QK kernel (one RMS per
// token over the whole Q segment and the whole K segment; "Kernel reference:
// qkv_cte", Design sections 1-2, all heads on one GPU). The lane-geometry
// planner shared by every form and the dispatcher over the forms are in
// plan.cpp.
#include "qk_kernel.h"

namespace qknr {

hipError_t qk_launch_across(const QkParams &p, int elem_type, int vec, int J, hipStream_t stream) {
    return qk_launch_mode<QK_ACROSS>(p, elem_type, vec, J, stream);
}

}  // namespace qknr
