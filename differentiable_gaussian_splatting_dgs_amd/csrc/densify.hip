// Densification, pruning and opacity reset.
//
// Method source: 3DGS training notes (huajishe): D.1 (Gaussians whose
// accumulated position gradient is large are densified; a split replaces one
// Gaussian by two smaller ones), D.2 (split along the long axis when Sigma is
// anisotropic, i.e. its eigenvalue ratio is large; clone to a slightly offset
// copy when it is isotropic), D.3 (remove Gaussians of low opacity), E.1
// steps 4-6 (densify and prune every 100 iterations; scale every opacity by
// 0.3 every 3000).  The numbers the notes leave out arrive in
// gs_densify_params.
//
// gs_densify is out of place and keeps the input order: Gaussian i is
// replaced by 0, 1 or 2 consecutive output rows.  Three passes:
//   1. k_dens_count: each Gaussian's action; output rows per partition of
//      kPart Gaussians.
//   2. k_dens_offsets: each Gaussian's first output row (its partition's
//      offset is the sum of the earlier partitions' totals, a few thousand
//      L2-resident words); the last partition writes the row count and the
//      overflow flag.
//   3. k_dens_write<K>: a block of kWriteBlock Gaussians owns one contiguous
//      run of output rows.  Each thread records where its Gaussian's rows
//      come from (and, for a split or a clone, the displacement along the
//      long axis); then the block writes every array over the run with
//      coalesced accesses, streaming the float4-wide ones (the quaternion and
//      the SH coefficients with their moments: 3 x 52 of the 177 floats per
//      row at degree 3) past the caches.
#include "gs_internal.h"

namespace gs {
namespace {

constexpr int kThreads = 256;
constexpr int kIPT = 4;
constexpr int kPart = kThreads * kIPT;  // Gaussians per offset partition
constexpr int kWriteBlock = 256;        // Gaussians per write block
constexpr uint32_t kFresh = 1u << 31;   // output row with zero Adam moments

enum Action : uint8_t { kRemoved = 0, kKept = 1, kCloned = 2, kSplit = 3 };

struct DensArgs {
    int32_t n;
    uint32_t parts;
    uint64_t cap;
    float grad_threshold, prune_logit, split_log_gap, split_shrink, split_offset, clone_offset;
    const float* in[5];   // means, log_scales, quats, opacity_logits, sh
    const float* min[10]; // exp_avg x5, exp_avg_sq x5, or all null
    const float* accum;
    const int32_t* count;
    float* out[5];
    float* mout[10];
    float* oaccum;        // may be null
    int32_t* ocount;      // may be null
    uint8_t* act;         // [n] workspace
    uint8_t* act_user;    // [n] or null
    uint32_t* part;       // [parts] output rows per partition
    uint32_t* off;        // [n] first output row
    uint32_t* n_out;
    uint32_t* overflow;
};

__device__ inline uint32_t rows_of(uint32_t act) { return act == kRemoved ? 0u : (act == kKept ? 1u : 2u); }

// The decisions are exact comparisons of the float32 inputs (widened to
// double where a quotient or a difference is involved), so they do not
// depend on rounding order.
__device__ inline uint32_t action_of(const DensArgs& a, int64_t i) {
    const float* ls = a.in[1] + 3 * i;
    const float l0 = ls[0], l1 = ls[1], l2 = ls[2];
    float lmax = l0, lmin = l0;
    if (l1 > lmax) lmax = l1;
    if (l2 > lmax) lmax = l2;
    if (l1 < lmin) lmin = l1;
    if (l2 < lmin) lmin = l2;
    const int32_t c = a.count[i];
    const bool dens = c > 0 && (double)a.accum[i] / (double)c >= (double)a.grad_threshold;
    if (a.in[3][i] < a.prune_logit) return kRemoved;
    if (!dens) return kKept;
    return (double)lmax - (double)lmin >= (double)a.split_log_gap ? kSplit : kCloned;
}

// Block-wide exclusive sum over kThreads threads; returns this thread's prefix and the total.
__device__ inline uint32_t block_excl_sum(uint32_t v, uint32_t* s_wsum, uint32_t& total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t x = v;
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    __syncthreads();
    if (lane == 63) s_wsum[wave] = x;
    __syncthreads();
    uint32_t add = 0;
    total = 0;
    for (int w = 0; w < kThreads / 64; ++w) {
        if (w < wave) add += s_wsum[w];
        total += s_wsum[w];
    }
    return x - v + add;
}

// 1. actions and rows per partition
__global__ __launch_bounds__(kThreads) void k_dens_count(DensArgs a) {
    __shared__ uint32_t s_wsum[kThreads / 64];
    const int64_t j0 = (int64_t)blockIdx.x * kPart + (int64_t)threadIdx.x * kIPT;
    uint32_t rows = 0;
#pragma unroll
    for (int k = 0; k < kIPT; ++k) {
        const int64_t j = j0 + k;
        if (j < a.n) {
            const uint32_t act = action_of(a, j);
            a.act[j] = (uint8_t)act;
            if (a.act_user) a.act_user[j] = (uint8_t)act;
            rows += rows_of(act);
        }
    }
    uint32_t total;
    block_excl_sum(rows, s_wsum, total);
    if (threadIdx.x == 0) a.part[blockIdx.x] = total;
}

// 2. first output row of every Gaussian; the last partition writes the row count
__global__ __launch_bounds__(kThreads) void k_dens_offsets(DensArgs a) {
    __shared__ uint32_t s_wsum[kThreads / 64];
    uint32_t before = 0;
    for (uint32_t i = threadIdx.x; i < blockIdx.x; i += kThreads) before += a.part[i];
    uint32_t pbase;
    block_excl_sum(before, s_wsum, pbase);
    const int64_t j0 = (int64_t)blockIdx.x * kPart + (int64_t)threadIdx.x * kIPT;
    uint32_t r[kIPT], sum = 0;
#pragma unroll
    for (int k = 0; k < kIPT; ++k) {
        r[k] = j0 + k < a.n ? rows_of(a.act[j0 + k]) : 0u;
        sum += r[k];
    }
    uint32_t total;
    uint32_t o = pbase + block_excl_sum(sum, s_wsum, total);
#pragma unroll
    for (int k = 0; k < kIPT; ++k) {
        if (j0 + k < a.n) a.off[j0 + k] = o;
        o += r[k];
    }
    if (blockIdx.x == gridDim.x - 1 && threadIdx.x == 0) {
        const uint32_t rows = pbase + total;
        *a.n_out = rows;
        *a.overflow = (uint64_t)rows > a.cap ? 1u : 0u;
    }
}

// Column `axis` of the rotation of the unit quaternion q / |q| (w, x, y, z):
// the Gaussian's axis in world coordinates.
__device__ inline void rot_column(const float4 q4, int axis, float e[3]) {
    const float nrm = sqrtf(q4.x * q4.x + q4.y * q4.y + q4.z * q4.z + q4.w * q4.w);
    const float w = q4.x / nrm, x = q4.y / nrm, y = q4.z / nrm, z = q4.w / nrm;
    if (axis == 0) {
        e[0] = 1.f - 2.f * (y * y + z * z); e[1] = 2.f * (x * y + w * z); e[2] = 2.f * (x * z - w * y);
    } else if (axis == 1) {
        e[0] = 2.f * (x * y - w * z); e[1] = 1.f - 2.f * (x * x + z * z); e[2] = 2.f * (y * z + w * x);
    } else {
        e[0] = 2.f * (x * z + w * y); e[1] = 2.f * (y * z - w * x); e[2] = 1.f - 2.f * (x * x + y * y);
    }
}

typedef float v4f __attribute__((ext_vector_type(4)));
// Streaming (non-temporal) float4 access: every byte is read or written once.
__device__ __forceinline__ float4 nt_ld4(const float4* p) {
    const v4f v = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(p));
    return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void nt_st4(float4 v, float4* p) {
    v4f w;
    w.x = v.x; w.y = v.y; w.z = v.z; w.w = v.w;
    __builtin_nontemporal_store(w, reinterpret_cast<v4f*>(p));
}

// Per output row of a write block: its source Gaussian (| kFresh for a copy
// or a child), the displacement of its mean and the shift of its log-scales.
struct RowInfo {
    uint32_t src[2 * kWriteBlock];
    float disp[2 * kWriteBlock][3];
    float shift[2 * kWriteBlock];
};

// The block's rows [obase, obase + nrows) of one array of W floats per row,
// from the source rows.  MODE 0: copy; 1: copy, zero for fresh rows (Adam
// moments); 2: add the row's mean displacement; 3: subtract the row's
// log-scale shift; 4: zero (the statistic).  Writes are contiguous and
// coalesced; reads follow the source rows, which are consecutive too.
template <int W, int MODE, typename T>
__device__ inline void copy_rows(const T* src, T* dst, uint32_t obase, uint32_t nrows, const RowInfo& ri) {
    if constexpr (W % 4 == 0 && MODE <= 1 && sizeof(T) == 4) {
        constexpr int W4 = W / 4;
        const float4* s4 = reinterpret_cast<const float4*>(src);
        float4* d4 = reinterpret_cast<float4*>(dst) + (uint64_t)obase * W4;
        for (uint32_t e = threadIdx.x; e < nrows * W4; e += kWriteBlock) {
            const uint32_t r = e / W4, c = e - r * W4;
            const uint32_t sv = ri.src[r];
            const bool z = MODE == 1 && (sv & kFresh);
            nt_st4(z ? make_float4(0.f, 0.f, 0.f, 0.f) : nt_ld4(s4 + (uint64_t)(sv & ~kFresh) * W4 + c), d4 + e);
        }
    } else {
        T* d = dst + (uint64_t)obase * W;
        for (uint32_t e = threadIdx.x; e < nrows * W; e += kWriteBlock) {
            const uint32_t r = e / W, c = e - r * W;
            const uint32_t sv = ri.src[r];
            T v = T(0);
            if (MODE != 4) v = src[(uint64_t)(sv & ~kFresh) * W + c];
            if (MODE == 1 && (sv & kFresh)) v = T(0);
            if constexpr (MODE == 2) v += ri.disp[r][c];
            if constexpr (MODE == 3) v -= ri.shift[r];
            d[e] = v;
        }
    }
}

// 3. the outputs of kWriteBlock consecutive Gaussians.  K = SH coefficients.
// Each thread records its Gaussian's output rows in RowInfo (a split or a
// clone also computes the long axis and its displacement); the block then
// writes every array over its contiguous run of output rows.
template <int K>
__global__ __launch_bounds__(kWriteBlock) void k_dens_write(DensArgs a) {
    __shared__ RowInfo ri;
    if (*a.overflow) return;  // uniform: nothing is written past the capacity
    const int64_t g0 = (int64_t)blockIdx.x * kWriteBlock;
    const int64_t g = g0 + threadIdx.x;
    const int64_t glast = min((int64_t)a.n, g0 + kWriteBlock) - 1;
    const uint32_t obase = a.off[g0];
    const uint32_t nrows = a.off[glast] + rows_of(a.act[glast]) - obase;  // <= 2 kWriteBlock
    if (g < a.n) {
        const uint32_t act = a.act[g];
        const uint32_t o = a.off[g] - obase;
        const uint32_t nr = rows_of(act);
        // x + (-0) == x for every x, so an undisplaced mean is copied bit for bit
        float d[2][3] = {{-0.f, -0.f, -0.f}, {-0.f, -0.f, -0.f}};
        if (act == kCloned || act == kSplit) {
            const float* ls = a.in[1] + 3 * g;
            const float l[3] = {ls[0], ls[1], ls[2]};
            int axis = 0;
            if (l[1] > l[axis]) axis = 1;
            if (l[2] > l[axis]) axis = 2;
            float e[3];
            rot_column(reinterpret_cast<const float4*>(a.in[2])[g], axis, e);
            const float smax = expf(l[axis]);
            if (act == kCloned) {
                const float dd = a.clone_offset * smax;
#pragma unroll
                for (int c = 0; c < 3; ++c) d[1][c] = dd * e[c];
            } else {
                const float dd = a.split_offset * smax;
#pragma unroll
                for (int c = 0; c < 3; ++c) {
                    d[0][c] = dd * e[c];
                    d[1][c] = -(dd * e[c]);
                }
            }
        }
        for (uint32_t r = 0; r < nr; ++r) {
            const bool fresh = act == kSplit || r == 1;  // a child or the copy
            ri.src[o + r] = (uint32_t)g | (fresh ? kFresh : 0u);
#pragma unroll
            for (int c = 0; c < 3; ++c) ri.disp[o + r][c] = d[r][c];
            ri.shift[o + r] = act == kSplit ? a.split_shrink : 0.f;
        }
    }
    __syncthreads();
    copy_rows<3, 2>(a.in[0], a.out[0], obase, nrows, ri);
    copy_rows<3, 3>(a.in[1], a.out[1], obase, nrows, ri);
    copy_rows<4, 0>(a.in[2], a.out[2], obase, nrows, ri);
    copy_rows<1, 0>(a.in[3], a.out[3], obase, nrows, ri);
    copy_rows<3 * K, 0>(a.in[4], a.out[4], obase, nrows, ri);
    if (a.min[0]) {
#pragma unroll
        for (int mv = 0; mv < 2; ++mv) {
            copy_rows<3, 1>(a.min[5 * mv + 0], a.mout[5 * mv + 0], obase, nrows, ri);
            copy_rows<3, 1>(a.min[5 * mv + 1], a.mout[5 * mv + 1], obase, nrows, ri);
            copy_rows<4, 1>(a.min[5 * mv + 2], a.mout[5 * mv + 2], obase, nrows, ri);
            copy_rows<1, 1>(a.min[5 * mv + 3], a.mout[5 * mv + 3], obase, nrows, ri);
            copy_rows<3 * K, 1>(a.min[5 * mv + 4], a.mout[5 * mv + 4], obase, nrows, ri);
        }
    }
    if (a.oaccum) {
        copy_rows<1, 4>(a.oaccum, a.oaccum, obase, nrows, ri);
        copy_rows<1, 4>(a.ocount, a.ocount, obase, nrows, ri);
    }
}

// No Gaussians: no rows, no overflow.
__global__ void k_dens_empty(uint32_t* n_out, uint32_t* overflow) {
    *n_out = 0u;
    *overflow = 0u;
}

// Opacity reset: sigma <- factor sigma, as a logit, computed stably:
// log sigma(x) = -softplus(-x), new logit = log(factor sigma) - log1p(-factor sigma).
__global__ __launch_bounds__(256) void k_opacity_reset(int32_t n, float factor, float log_factor, float* logit,
                                                       float* m, float* v) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const float x = logit[i];
    const float log_sig = -(fmaxf(-x, 0.f) + log1pf(expf(-fabsf(x))));
    const float s = factor * expf(log_sig);
    logit[i] = log_factor + log_sig - log1pf(-s);
    if (m) m[i] = 0.f;
    if (v) v[i] = 0.f;
}

struct DensLayout {
    size_t part, off, act, total;
    uint32_t parts;
};

inline size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }

inline DensLayout dens_layout(int32_t n) {
    DensLayout L;
    L.parts = (uint32_t)((n + kPart - 1) / kPart);
    size_t o = 0;
    L.part = o; o = up256(o + (size_t)L.parts * 4);
    L.off = o; o = up256(o + (size_t)n * 4);
    L.act = o; o = up256(o + (size_t)n);
    L.total = o;
    return L;
}

template <int K>
void launch_write(int32_t n, const DensArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(k_dens_write<K>, dim3((n + kWriteBlock - 1) / kWriteBlock), dim3(kWriteBlock), 0, s, a);
}

}  // namespace
}  // namespace gs

using namespace gs;

extern "C" int gs_densify_workspace_size(int32_t n, size_t* bytes) {
    if (n < 0 || !bytes) return GS_EINVAL;
    *bytes = dens_layout(n).total;
    return GS_OK;
}

extern "C" int gs_densify(const gs_densify_params* dp, int32_t n, int32_t sh_degree, const gs_gaussian_set* in,
                          int64_t capacity, const gs_gaussian_set* out, uint32_t* n_out_dev,
                          uint32_t* overflow_dev, uint8_t* action, void* workspace, size_t workspace_bytes,
                          void* stream) {
    if (!dp || !in || !out || n < 0 || capacity < 0 || sh_degree < 0 || sh_degree > GS_MAX_SH_DEGREE ||
        !n_out_dev || !overflow_dev || (n > 0 && !workspace))
        return GS_EINVAL;
    const DensLayout L = dens_layout(n);
    if (workspace_bytes < L.total) return GS_EWORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) & 255u) return GS_EALIGN;  // (NULL passes when n == 0)
    const int K = (sh_degree + 1) * (sh_degree + 1);
    DensArgs a;
    a.n = n; a.parts = L.parts; a.cap = (uint64_t)capacity;
    a.grad_threshold = dp->grad_threshold; a.prune_logit = dp->prune_logit; a.split_log_gap = dp->split_log_gap;
    a.split_shrink = dp->split_shrink; a.split_offset = dp->split_offset; a.clone_offset = dp->clone_offset;
    const float* ip[5] = {in->means, in->log_scales, in->quats, in->opacity_logits, in->sh};
    float* op[5] = {out->means, out->log_scales, out->quats, out->opacity_logits, out->sh};
    int in_mom = 0, out_mom = 0;
    for (int g = 0; g < 5; ++g) {
        a.in[g] = ip[g]; a.out[g] = op[g];
        a.min[g] = in->exp_avg[g]; a.min[5 + g] = in->exp_avg_sq[g];
        a.mout[g] = out->exp_avg[g]; a.mout[5 + g] = out->exp_avg_sq[g];
    }
    for (int k = 0; k < 10; ++k) {
        in_mom += a.min[k] != nullptr;
        out_mom += a.mout[k] != nullptr;
    }
    // all ten moments or none on each side; they must agree when anything can be written
    if ((in_mom != 0 && in_mom != 10) || (out_mom != 0 && out_mom != 10)) return GS_EINVAL;
    if (capacity > 0 && out_mom != in_mom) return GS_EINVAL;
    if (out_mom == 0)
        for (int k = 0; k < 10; ++k) a.min[k] = nullptr;  // the kernels carry moments only when both sides have them
    a.accum = in->densify_accum; a.count = in->densify_count;
    a.oaccum = out->densify_accum; a.ocount = out->densify_count;
    if (n > 0 && (!a.accum || !a.count)) return GS_EINVAL;
    if (capacity > 0 && (a.oaccum == nullptr) != (a.ocount == nullptr)) return GS_EINVAL;
    if (a.ocount == nullptr) a.oaccum = nullptr;
    if (n > 0) {
        for (int g = 0; g < 5; ++g)
            if (!ip[g]) return GS_EINVAL;
        if (!aligned16(in->quats) || !aligned16(in->sh)) return GS_EALIGN;
        if (in_mom && (!aligned16(in->exp_avg[2]) || !aligned16(in->exp_avg_sq[2]) || !aligned16(in->exp_avg[4]) ||
                       !aligned16(in->exp_avg_sq[4])))
            return GS_EALIGN;
    }
    if (capacity > 0) {
        for (int g = 0; g < 5; ++g)
            if (!op[g]) return GS_EINVAL;
        if (!aligned16(out->quats) || !aligned16(out->sh)) return GS_EALIGN;
        if (out_mom && (!aligned16(out->exp_avg[2]) || !aligned16(out->exp_avg_sq[2]) ||
                        !aligned16(out->exp_avg[4]) || !aligned16(out->exp_avg_sq[4])))
            return GS_EALIGN;
    }
    char* ws = static_cast<char*>(workspace);
    a.part = reinterpret_cast<uint32_t*>(ws + L.part);
    a.off = reinterpret_cast<uint32_t*>(ws + L.off);
    a.act = reinterpret_cast<uint8_t*>(ws + L.act);
    a.act_user = action;
    a.n_out = n_out_dev; a.overflow = overflow_dev;
    hipStream_t s = as_stream(stream);
    if (n == 0) {
        hipLaunchKernelGGL(k_dens_empty, dim3(1), dim3(1), 0, s, n_out_dev, overflow_dev);
        return launch_status();
    }
    hipLaunchKernelGGL(k_dens_count, dim3(L.parts), dim3(kThreads), 0, s, a);
    hipLaunchKernelGGL(k_dens_offsets, dim3(L.parts), dim3(kThreads), 0, s, a);
    switch (K) {
        case 1: launch_write<1>(n, a, s); break;
        case 4: launch_write<4>(n, a, s); break;
        case 9: launch_write<9>(n, a, s); break;
        default: launch_write<16>(n, a, s); break;
    }
    return launch_status();
}

extern "C" int gs_opacity_reset(int32_t n, float factor, float* opacity_logits, float* exp_avg, float* exp_avg_sq,
                                void* stream) {
    if (n < 0 || !(factor > 0.f && factor <= 1.f)) return GS_EINVAL;
    if (n == 0) return GS_OK;
    if (!opacity_logits) return GS_EINVAL;
    hipLaunchKernelGGL(k_opacity_reset, dim3((n + 255) / 256), dim3(256), 0, as_stream(stream), n, factor,
                       logf(factor), opacity_logits, exp_avg, exp_avg_sq);
    return launch_status();
}
