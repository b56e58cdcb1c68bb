// permute.hip -- the offline lane conversion of an interleaved-pair RoPE
// checkpoint to the rotate-half layout that the QK kernels implement
// ("Kernel reference: qkv_cte", Design section 2 and "Adapting this kernel":
// the caller permutes the Q/K weights, bias, gamma and the cos/sin caches once,
// so the kernels never see the interleaved form).
//
// Along one axis of a tensor viewed as [outer, axis_len, inner], each of
// n_heads blocks of head_dim indices starting at `first` is permuted so that
// rotate-half lane j holds interleaved lane 2j (j < d/2) or 2(j - d/2) + 1
// (j >= d/2); `inverse` maps back. Every other index is copied unchanged.
//
// A gather copy, run once per checkpoint: each thread moves one `U`-sized
// piece of one index's inner block (the largest of 16/8/4/2/1 bytes that
// divides the block and both pointers), grid-stride over the whole tensor.
#include "launch.h"

namespace qknr {

namespace {

struct alignas(16) U16 {
    uint32_t w[4];
};

template <typename U>
__global__ __launch_bounds__(256) void permute_kernel(PermuteParams p) {
    const U *src = reinterpret_cast<const U *>(p.src);
    U *dst = reinterpret_cast<U *>(p.dst);
    const uint64_t total = p.outer * p.axis_len * p.units_per_index;
    const uint64_t block_end = p.first + p.n_heads * p.head_dim;
    const uint64_t half = p.head_dim / 2;
    for (uint64_t i = (uint64_t)blockIdx.x * 256u + threadIdx.x; i < total; i += (uint64_t)gridDim.x * 256u) {
        const uint64_t u = i % p.units_per_index;
        const uint64_t rest = i / p.units_per_index;
        const uint64_t l = rest % p.axis_len;
        const uint64_t o = rest / p.axis_len;
        uint64_t sl = l;
        if (l >= p.first && l < block_end) {
            const uint64_t off = l - p.first;
            const uint64_t h = off / p.head_dim;
            const uint64_t j = off - h * p.head_dim;
            uint64_t from;
            if (!p.inverse) from = j < half ? 2 * j : 2 * (j - half) + 1;   // rotate-half lane j <- interleaved
            else from = (j & 1) ? half + j / 2 : j / 2;                     // interleaved lane j <- rotate-half
            sl = p.first + h * p.head_dim + from;
        }
        dst[(o * p.axis_len + l) * p.units_per_index + u] = src[(o * p.axis_len + sl) * p.units_per_index + u];
    }
}

template <typename U>
hipError_t launch(const PermuteParams &p, hipStream_t stream) {
    const uint64_t total = p.outer * p.axis_len * p.units_per_index;
    if (total == 0) return hipSuccess;
    uint64_t blocks = (total + 255) / 256;
    if (blocks > 8192) blocks = 8192;     // 32 blocks per CU, then grid-stride
    hipLaunchKernelGGL(permute_kernel<U>, dim3((uint32_t)blocks), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t permute_launch(const PermuteParams &p, int unit, hipStream_t stream) {
    switch (unit) {
    case 1: return launch<uint8_t>(p, stream);
    case 2: return launch<uint16_t>(p, stream);
    case 4: return launch<uint32_t>(p, stream);
    case 8: return launch<uint64_t>(p, stream);
    case 16: return launch<U16>(p, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace qknr
