// Training-step tail: image loss, densification statistic, Adam.
//
// Method source: 3DGS training notes (huajishe): E.1 (the training loop:
// render, image loss, backpropagate, accumulate the position-gradient
// statistic, Adam update), C.2 (Adam with per-parameter learning rates),
// D.1 (the densification statistic is the accumulated position gradient),
// D.4 (quaternions are renormalised after the update).  Adam itself follows
// Kingma and Ba (2015), which the notes cite.
#include "gs_internal.h"

namespace gs {
namespace {

constexpr int kLossBlocks = GS_LOSS_PARTIALS;

// Pass 1: each block writes the sum of its grid-stride share to partial[block].
__global__ __launch_bounds__(256) void k_loss(int mode, int64_t count, const float* pred, const float* target,
                                              float* grad, double* partial) {
    __shared__ double s_part[4];
    double acc = 0.0;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride) {
        const float r = pred[i] - target[i];
        if (mode == 1) {
            acc += (double)fabsf(r);
            grad[i] = r > 0.f ? 1.f : (r < 0.f ? -1.f : 0.f);
        } else {
            acc += (double)r * (double)r;
            grad[i] = 2.f * r;
        }
    }
    for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) s_part[wave] = acc;
    __syncthreads();
    if (threadIdx.x == 0) partial[blockIdx.x] = (s_part[0] + s_part[1]) + (s_part[2] + s_part[3]);
}

// Pass 2: one block adds the partials in a fixed order (deterministic).
__global__ __launch_bounds__(256) void k_loss_sum(const double* partial, int nparts, double* loss) {
    __shared__ double s_part[4];
    double acc = 0.0;
    for (int i = threadIdx.x; i < nparts; i += blockDim.x) acc += partial[i];
    for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) s_part[wave] = acc;
    __syncthreads();
    if (threadIdx.x == 0) *loss = (s_part[0] + s_part[1]) + (s_part[2] + s_part[3]);
}

__global__ __launch_bounds__(256) void k_densify(int32_t n, const int32_t* tt, const float* grad2d, float* accum,
                                                 int32_t* count) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n || tt[i] <= 0) return;
    const float2 d = *reinterpret_cast<const float2*>(grad2d + (size_t)i * GS_GRAD2D_STRIDE);
    accum[i] += sqrtf(d.x * d.x + d.y * d.y);
    count[i] += 1;
}

struct AdamArgs {
    gs_adam_group g[GS_ADAM_MAX_GROUPS];
    int64_t first_block[GS_ADAM_MAX_GROUPS + 1];
    int32_t n_groups;
    float b1, b2, eps, inv_c1, inv_sqrt_c2;
};

constexpr int kAdamThreads = 256;
constexpr int kAdamIPT = 4;

__device__ __forceinline__ void adam_one(float& p, float g, float& m, float& v, float lr, const AdamArgs& a) {
    m = a.b1 * m + (1.f - a.b1) * g;
    v = a.b2 * v + (1.f - a.b2) * g * g;
    // the same arithmetic as the fused tail's update: hardware square root and reciprocal
    const float denom = __builtin_amdgcn_sqrtf(v) * a.inv_sqrt_c2 + a.eps;
    p -= lr * (m * a.inv_c1) * __builtin_amdgcn_rcpf(denom);
}

__global__ __launch_bounds__(kAdamThreads) void k_adam(AdamArgs a) {
    int gi = 0;
    while (gi + 1 < a.n_groups && (int64_t)blockIdx.x >= a.first_block[gi + 1]) ++gi;
    const gs_adam_group& G = a.g[gi];
    const int64_t local = (int64_t)blockIdx.x - a.first_block[gi];
    const int ncol = G.col_end - G.col_begin;
    if (G.normalize_rows) {
        // one thread per row: update the row, then renormalise it
        const int64_t row = local * kAdamThreads + threadIdx.x;
        if (row >= G.rows) return;
        const int64_t base = row * G.row_len;
        float ss = 0.f;
        for (int c = 0; c < G.row_len; ++c) {
            float p = G.param[base + c], m = G.exp_avg[base + c], v = G.exp_avg_sq[base + c];
            adam_one(p, G.grad[base + c], m, v, G.lr, a);
            G.exp_avg[base + c] = m;
            G.exp_avg_sq[base + c] = v;
            G.param[base + c] = p;
            ss += p * p;
        }
        const float inv = 1.f / sqrtf(ss);
        for (int c = 0; c < G.row_len; ++c) G.param[base + c] *= inv;
        return;
    }
    const int64_t total = G.rows * ncol;
    const int64_t e0 = local * (kAdamThreads * kAdamIPT) + threadIdx.x;
#pragma unroll
    for (int k = 0; k < kAdamIPT; ++k) {
        const int64_t e = e0 + (int64_t)k * kAdamThreads;
        if (e >= total) return;
        const int64_t row = ncol == G.row_len ? 0 : e / ncol;
        const int64_t idx = ncol == G.row_len ? e : row * G.row_len + G.col_begin + (e - row * ncol);
        float p = G.param[idx], m = G.exp_avg[idx], v = G.exp_avg_sq[idx];
        adam_one(p, G.grad[idx], m, v, G.lr, a);
        G.param[idx] = p;
        G.exp_avg[idx] = m;
        G.exp_avg_sq[idx] = v;
    }
}

}  // namespace
}  // namespace gs

using namespace gs;

extern "C" int gs_image_loss(int32_t mode, int64_t count, const float* pred, const float* target, float* dL_dpred,
                             double* loss_dev, void* stream) {
    if ((mode != 1 && mode != 2) || count < 0 || !loss_dev) return GS_EINVAL;
    if (count > 0 && (!pred || !target || !dL_dpred)) return GS_EINVAL;
    hipStream_t s = as_stream(stream);
    int64_t blocks = (count + 255) / 256;
    if (blocks > kLossBlocks) blocks = kLossBlocks;
    if (blocks < 1) blocks = 1;
    if (count > 0)
        hipLaunchKernelGGL(k_loss, dim3((unsigned)blocks), dim3(256), 0, s, mode, count, pred, target, dL_dpred,
                           loss_dev + 1);
    hipLaunchKernelGGL(k_loss_sum, dim3(1), dim3(256), 0, s, loss_dev + 1, count > 0 ? (int)blocks : 0, loss_dev);
    return launch_status();
}

extern "C" int gs_densify_accum(int32_t n, const int32_t* tiles_touched, const float* grad2d, float* accum,
                                int32_t* count, void* stream) {
    if (n < 0) return GS_EINVAL;
    if (n == 0) return GS_OK;
    if (!tiles_touched || !grad2d || !accum || !count) return GS_EINVAL;
    if (!aligned16(grad2d)) return GS_EALIGN;
    hipLaunchKernelGGL(k_densify, dim3((n + 255) / 256), dim3(256), 0, as_stream(stream), n, tiles_touched, grad2d,
                       accum, count);
    return launch_status();
}

extern "C" int gs_adam_step(int32_t n_groups, const gs_adam_group* groups, float beta1, float beta2, float eps,
                            int32_t step, void* stream) {
    if (n_groups < 0 || n_groups > GS_ADAM_MAX_GROUPS || step < 1 || (n_groups > 0 && !groups)) return GS_EINVAL;
    AdamArgs a{};
    a.n_groups = n_groups;
    a.b1 = beta1; a.b2 = beta2; a.eps = eps;
    a.inv_c1 = (float)(1.0 / (1.0 - pow((double)beta1, step)));
    a.inv_sqrt_c2 = (float)(1.0 / sqrt(1.0 - pow((double)beta2, step)));
    int64_t blocks = 0;
    for (int i = 0; i < n_groups; ++i) {
        const gs_adam_group& G = groups[i];
        if (G.rows < 0 || G.row_len <= 0 || G.col_begin < 0 || G.col_end > G.row_len || G.col_begin >= G.col_end)
            return GS_EINVAL;
        if (G.rows > 0 && (!G.param || !G.grad || !G.exp_avg || !G.exp_avg_sq)) return GS_EINVAL;
        if (G.normalize_rows && (G.col_begin != 0 || G.col_end != G.row_len)) return GS_EINVAL;
        a.g[i] = G;
        a.first_block[i] = blocks;
        const int64_t work = G.normalize_rows ? G.rows : G.rows * (G.col_end - G.col_begin);
        const int64_t per = G.normalize_rows ? kAdamThreads : kAdamThreads * kAdamIPT;
        blocks += (work + per - 1) / per;
    }
    a.first_block[n_groups] = blocks;
    if (blocks == 0) return GS_OK;
    if (blocks > 0x7fffffff) return GS_ECAPACITY;
    hipLaunchKernelGGL(k_adam, dim3((unsigned)blocks), dim3(kAdamThreads), 0, as_stream(stream), a);
    return launch_status();
}
