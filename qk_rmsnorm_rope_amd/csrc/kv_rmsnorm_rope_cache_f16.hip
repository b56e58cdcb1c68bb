// kv_rmsnorm_rope_cache_f16.hip -- the f16 instantiations of the
// KvRmsNormRopeCache kernel (kv_kernel.h), in a translation unit of their own
// so that the two element types compile in parallel.
#include "kv_kernel.h"

namespace qknr {

hipError_t kv_launch_f16(const KvParams &p, int vec, bool v2, int ca, int cb, hipStream_t stream) {
    return launch_elem<f16_t>(p, vec, v2, ca, cb, stream);
}

}  // namespace qknr
