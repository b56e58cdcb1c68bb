// kv_rmsnorm_rope_cache.hip -- the bf16 instantiations of the
// KvRmsNormRopeCache kernel. The kernel itself (and its design notes) is in
// kv_kernel.h; the launch planner and dispatcher in plan.cpp; the f16
// instantiations in kv_rmsnorm_rope_cache_f16.hip (compiled in parallel).
#include "kv_kernel.h"

namespace qknr {

hipError_t kv_launch_bf16(const KvParams &p, int vec, bool v2, int ca, int cb, hipStream_t stream) {
    return launch_elem<bf16_t>(p, vec, v2, ca, cb, stream);
}

}  // namespace qknr
