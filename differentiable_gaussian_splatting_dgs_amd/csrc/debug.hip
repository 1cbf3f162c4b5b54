// Debug check: the number of NaN and infinite values in a float32 array.
//
// Method source: Gaussian Splatting backward CUDA page (lshu.cn), section 6:
// its troubleshooting table traces NaN to invalid math (for instance the range
// of exp's argument).  A caller in debug mode counts the non-finite values of
// the inputs and outputs of each call to find where they first appear.
#include "gs_internal.h"

namespace gs {
namespace {

constexpr int kNfThreads = 256;
constexpr int kNfMaxBlocks = 1024;  // one atomic per block on one address

__global__ void k_zero_count(unsigned long long* out) { *out = 0ull; }

__global__ __launch_bounds__(kNfThreads) void k_count_nonfinite(const float* __restrict__ x, size_t count,
                                                                 unsigned long long* out) {
    __shared__ uint32_t s_w[kNfThreads / 64];
    uint32_t c = 0;
    const size_t stride = (size_t)gridDim.x * kNfThreads;
    for (size_t i = (size_t)blockIdx.x * kNfThreads + threadIdx.x; i < count; i += stride) {
        // exponent all ones: infinity or NaN
        c += ((__float_as_uint(x[i]) & 0x7f800000u) == 0x7f800000u) ? 1u : 0u;
    }
    for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o, 64);
    if ((threadIdx.x & 63) == 0) s_w[threadIdx.x >> 6] = c;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t t = 0;
        for (int w = 0; w < kNfThreads / 64; ++w) t += s_w[w];
        if (t) atomicAdd(out, (unsigned long long)t);
    }
}

}  // namespace
}  // namespace gs

using namespace gs;

extern "C" int gs_count_nonfinite(const float* x, int64_t count, int64_t* out, void* stream) {
    if (count < 0 || !out || (count > 0 && !x)) return GS_EINVAL;
    auto* o = reinterpret_cast<unsigned long long*>(out);
    hipLaunchKernelGGL(k_zero_count, dim3(1), dim3(1), 0, as_stream(stream), o);
    if (count > 0) {
        const size_t blocks = std::min<size_t>(((size_t)count + kNfThreads - 1) / kNfThreads, kNfMaxBlocks);
        hipLaunchKernelGGL(k_count_nonfinite, dim3((unsigned)blocks), dim3(kNfThreads), 0, as_stream(stream), x,
                           (size_t)count, o);
    }
    return launch_status();
}
