// Measurement helpers: the two kernels whose rates are the measured
// denominators of a roofline on this GPU, one per binding resource.
//
//  - k_stream_copy: a 16-byte-per-lane copy, grid-stride, non-temporal both
//    ways, so every byte crosses HBM once in each direction;
//  - k_fma_loop: eight independent fp32 FMA chains per lane, the instruction a
//    vector fp32 peak counts, 64 FMAs per loop iteration (a branch every 8 FMAs
//    costs a third of the rate), with one store per lane at the end.
//
// Neither computes anything of the method; they exist so a benchmark can
// quote achieved bandwidth and flop rates against what the chip delivers as
// well as against its published figures.
#include "gs_internal.h"
#include "gs_measure.h"

namespace gs {
namespace {

typedef float v4f_t __attribute__((ext_vector_type(4)));

constexpr int kCopyThreads = 256;
constexpr int kFmaThreads = 256;
constexpr int kFmaChains = 8;
constexpr int kFmaRounds = 8;  // rounds of the chains per loop iteration

__global__ __launch_bounds__(kCopyThreads) void k_stream_copy(const v4f_t* __restrict__ src,
                                                              v4f_t* __restrict__ dst, size_t n4) {
    const size_t stride = (size_t)gridDim.x * kCopyThreads;
    size_t i = (size_t)blockIdx.x * kCopyThreads + threadIdx.x;
    // four loads in flight per lane before the stores
    for (; i + 3 * stride < n4; i += 4 * stride) {
        v4f_t v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < 4; ++u) __builtin_nontemporal_store(v[u], dst + i + u * stride);
    }
    for (; i < n4; i += stride) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

__global__ __launch_bounds__(kFmaThreads) void k_fma_loop(float* out, int32_t iters, float a, float b) {
    // a and b are copied into VGPRs: with a scalar-register operand an fp32 VALU
    // instruction issues at about half the rate on gfx950
    asm volatile("" : "+v"(a), "+v"(b));
    float f[kFmaChains];
#pragma unroll
    for (int c = 0; c < kFmaChains; ++c) f[c] = (float)(threadIdx.x + c);
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int r = 0; r < kFmaRounds; ++r)
#pragma unroll
            for (int c = 0; c < kFmaChains; ++c) f[c] = __builtin_fmaf(f[c], a, b);
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < kFmaChains; ++c) s += f[c];
    out[(size_t)blockIdx.x * kFmaThreads + threadIdx.x] = s;
}

}  // namespace
}  // namespace gs

using namespace gs;

extern "C" int gs_stream_copy(const float* src, float* dst, int64_t count, void* stream) {
    if (count < 0 || (count > 0 && (!src || !dst)) || (count & 3)) return GS_EINVAL;
    if (count == 0) return GS_OK;
    if (!aligned16(src) || !aligned16(dst)) return GS_EALIGN;
    const size_t n4 = (size_t)count / 4;
    const size_t blocks = std::min<size_t>((n4 + kCopyThreads - 1) / kCopyThreads, (size_t)256 * 32);
    hipLaunchKernelGGL(k_stream_copy, dim3((unsigned)blocks), dim3(kCopyThreads), 0, as_stream(stream),
                       reinterpret_cast<const v4f_t*>(src), reinterpret_cast<v4f_t*>(dst), n4);
    return launch_status();
}

extern "C" int gs_fma_loop(int32_t blocks, int32_t iters, float a, float b, float* out, void* stream) {
    if (blocks <= 0 || iters < 0 || !out) return GS_EINVAL;
    hipLaunchKernelGGL(k_fma_loop, dim3(blocks), dim3(kFmaThreads), 0, as_stream(stream), out, iters, a, b);
    return launch_status();
}
