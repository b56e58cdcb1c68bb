// qk_across_heads.hip -- the across-heads form of the QK kernel (one RMS per
// token over the whole Q segment and the whole K segment; "Kernel reference:
// qkv_cte", Design sections 1-2, all heads on one GPU), the lane-geometry
// planner shared by every form, and the dispatcher over the forms.
#include "qk_kernel.h"

namespace qknr {

hipError_t qk_launch_across(const QkParams &p, int elem_type, int vec, int J, hipStream_t stream) {
    return qk_launch_mode<QK_ACROSS>(p, elem_type, vec, J, stream);
}

static int round_up_j(int j) {
    if (j <= 6) return j;
    if (j <= 8) return 8;
    return -1;
}

int qk_plan(QkParams &p, int vec) {
    const int half = p.head_dim / 2;
    if (half % vec) return -1;
    const int kc = half / vec;
    if (kc > 64) return -1;
    const int hpw = 64 / kc;
    const int heads = p.n_q > p.n_k ? p.n_q : p.n_k;
    for (int W = 1; W <= 4; W *= 2) {
        const int J = round_up_j((heads + hpw * W - 1) / (hpw * W));
        if (J > 0) {
            p.half = half;
            p.chunks_per_half = kc;
            p.heads_per_step = hpw;
            p.waves_per_unit = W;
            return J;
        }
    }
    return -1;
}

hipError_t qk_launch(QkParams &p, int elem_type, int vec, int mode, hipStream_t stream) {
    const int J = qk_plan(p, vec);
    if (J < 0) return hipErrorInvalidValue;
    if (p.tokens == 0) return hipSuccess;
    switch (mode) {
    case QK_ACROSS: return qk_launch_across(p, elem_type, vec, J, stream);
    case QK_PER_HEAD: return qk_launch_per_head(p, elem_type, vec, J, stream);
    case QK_SUMSQ:
    case QK_APPLY: return qk_launch_split(p, elem_type, vec, J, mode, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace qknr
