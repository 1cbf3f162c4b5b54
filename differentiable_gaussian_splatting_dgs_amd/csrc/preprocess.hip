// Per-Gaussian projection: camera-space centre, EWA 2D covariance, conic,
// tile rectangle and view-dependent SH colour.  One thread per Gaussian,
// computed in float64 (cheap on CDNA4: the kernel is HBM-bound) so the
// integer tile rectangle and the float32 sort key are correctly rounded
// values of the exact projection.
//
// Method sources: Gaussian Splatting backward CUDA page (lshu.cn), section 4
// (the forward chain this kernel computes is the one its backward inverts:
// view transform, perspective Jacobian, Sigma = R S S^T R^T, SH basis);
// 3DGS training notes (huajishe), section E.3 (project, then cull against
// tiles with an axis-aligned bounding box).
#include "gs_internal.h"

namespace gs {
namespace {

struct PreArgs {
    CamArgs cams[GS_MAX_VIEWS];  // views of one size; outputs are [views, n, ...]
    int32_t views;
    double near_z, alpha_min, dilation;
    int32_t n;
    const float* means;
    const float* log_scales;
    const float* quats;
    const float* opac;
    const float* sh;
    float* splats;
    float* depth;
    int16_t* rect;
    int32_t* tiles_touched;
    uint8_t* clamp;
    float* cjac;  // optional [views, n, 9]: d colour_c / d dir_j before the clamp, row-major by c
    bool h16;     // splats holds 16-bit records (GS_SPLAT16_STRIDE floats each)
};

// Two floats as one word of binary16 values, lo in the low half; each is the
// binary16 number nearest to the float (ties to even, the hardware conversion).
__device__ __forceinline__ uint32_t pack_h2(float lo, float hi) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)lo) |
           ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)hi) << 16);
}

// Real spherical harmonics with the Condon-Shortley phase as polynomials of
// the unit direction: Y[l*l + l + m].  Constants are the normalisations
// sqrt((2l+1)/(4 pi) (l-m)!/(l+m)!) times sqrt(2) for m != 0, folded with
// the Legendre polynomial coefficients.
template <int DEG>
__device__ inline void sh_eval(double x, double y, double z, double* Y) {
    Y[0] = 0.28209479177387814;
    if (DEG >= 1) {
        Y[1] = -0.48860251190291992 * y;
        Y[2] = 0.48860251190291992 * z;
        Y[3] = -0.48860251190291992 * x;
    }
    if (DEG >= 2) {
        const double xx = x * x, yy = y * y, zz = z * z;
        Y[4] = 1.0925484305920792 * x * y;
        Y[5] = -1.0925484305920792 * y * z;
        Y[6] = 0.31539156525252005 * (2.0 * zz - xx - yy);
        Y[7] = -1.0925484305920792 * x * z;
        Y[8] = 0.54627421529603959 * (xx - yy);
        if (DEG >= 3) {
            Y[9] = -0.59004358992664352 * y * (3.0 * xx - yy);
            Y[10] = 2.8906114426405538 * x * y * z;
            Y[11] = -0.45704579946446572 * y * (4.0 * zz - xx - yy);
            Y[12] = 0.37317633259011540 * z * (2.0 * zz - 3.0 * xx - 3.0 * yy);
            Y[13] = -0.45704579946446572 * x * (4.0 * zz - xx - yy);
            Y[14] = 1.4453057213202769 * z * (xx - yy);
            Y[15] = -0.59004358992664352 * x * (xx - 3.0 * yy);
        }
    }
}

constexpr int kPreBlock = 256;  // Gaussians (= threads) per block

// Gaussian i's SH row (3 (DEG+1)^2 consecutive floats), as 16-byte loads when the
// row length and the pointer allow (VEC): neighbouring lanes' rows are adjacent,
// so the lines a wave touches are fetched once and served from the cache for
// its remaining loads.
template <int DEG, bool VEC>
__device__ __forceinline__ void load_sh(const float* sh, int i, float* shv) {
    constexpr int J = 3 * (DEG + 1) * (DEG + 1);
    if constexpr (VEC) {
        static_assert(J % 4 == 0, "vector SH loads need a row length that is a multiple of 4");
        const float4* src = reinterpret_cast<const float4*>(sh + (size_t)i * J);
#pragma unroll
        for (int k = 0; k < J / 4; ++k) {
            const float4 v = src[k];
            shv[4 * k] = v.x; shv[4 * k + 1] = v.y; shv[4 * k + 2] = v.z; shv[4 * k + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int k = 0; k < J; ++k) shv[k] = sh[(size_t)i * J + k];
    }
}

// Colour max(0, sum_k sh_k Y_k(dir) + 0.5) with dir the unit vector from the
// camera centre -R^T t to the mean; cm gets bit c when channel c was clamped.
template <int DEG>
__device__ __forceinline__ void shade(const CamArgs& c, double mx, double my, double mz, const float* shv,
                                      double rgb[3], uint8_t& cm, double dir[3]) {
    constexpr int K = (DEG + 1) * (DEG + 1);
    const double cpx = -(c.R[0] * c.t[0] + c.R[3] * c.t[1] + c.R[6] * c.t[2]);
    const double cpy = -(c.R[1] * c.t[0] + c.R[4] * c.t[1] + c.R[7] * c.t[2]);
    const double cpz = -(c.R[2] * c.t[0] + c.R[5] * c.t[1] + c.R[8] * c.t[2]);
    double dx = mx - cpx, dy = my - cpy, dz = mz - cpz;
    const double dinv = 1.0 / sqrt(dx * dx + dy * dy + dz * dz);
    dx *= dinv; dy *= dinv; dz *= dinv;
    dir[0] = dx; dir[1] = dy; dir[2] = dz;
    double Y[16];
    sh_eval<DEG>(dx, dy, dz, Y);
    rgb[0] = rgb[1] = rgb[2] = 0.5;
#pragma unroll
    for (int k = 0; k < K; ++k) {
        rgb[0] += Y[k] * (double)shv[3 * k];
        rgb[1] += Y[k] * (double)shv[3 * k + 1];
        rgb[2] += Y[k] * (double)shv[3 * k + 2];
    }
    cm = 0;
    for (int ch = 0; ch < 3; ++ch)
        if (rgb[ch] < 0.0) { cm |= (uint8_t)(1u << ch); rgb[ch] = 0.0; }
}

// One thread per Gaussian: projection, tile rectangle and the SH colour, for
// each view in turn (the parameters are read once; the view-free parts --
// opacity, M = R S -- are computed once).  CJ: also the colour's gradient with
// respect to the view direction (a.cjac).  H16: 16-bit splat records (the
// float32 mean, then the conic factor, opacity and colour in binary16).
template <int DEG, bool VEC, bool CJ, bool H16>
__global__ __launch_bounds__(kPreBlock) void k_preprocess(PreArgs a) {
    constexpr int J = 3 * (DEG + 1) * (DEG + 1);
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= a.n) return;
    float shv[J];
    load_sh<DEG, VEC>(a.sh, i, shv);

    const float4 z4 = make_float4(0.f, 0.f, 0.f, 0.f);
    auto cull = [&](size_t o) {
        if constexpr (H16) {
            uint2* sp = reinterpret_cast<uint2*>(a.splats + o * GS_SPLAT16_STRIDE);
            sp[0] = sp[1] = sp[2] = make_uint2(0u, 0u);
        } else {
            float4* sp = reinterpret_cast<float4*>(a.splats + o * GS_SPLAT_STRIDE);
            sp[0] = z4; sp[1] = z4; sp[2] = z4;
        }
        if constexpr (CJ)
            for (int k = 0; k < 9; ++k) a.cjac[9 * o + k] = 0.f;
        a.clamp[o] = 0;
        a.depth[o] = 0.f;
        reinterpret_cast<uint2*>(a.rect)[o] = make_uint2(0u, 0u);
        a.tiles_touched[o] = 0;
    };

    const double mx = a.means[3 * i], my = a.means[3 * i + 1], mz = a.means[3 * i + 2];
    // opacity
    const double sigma = 1.0 / (1.0 + exp(-(double)a.opac[i]));
    if (sigma < a.alpha_min) {
        for (int view = 0; view < a.views; ++view) cull((size_t)view * a.n + i);
        return;
    }
    // rotation of the normalised quaternion (w, x, y, z), M = R S
    const float4 qf = reinterpret_cast<const float4*>(a.quats)[i];
    double qw = qf.x, qx = qf.y, qy = qf.z, qz = qf.w;
    const double qinv = 1.0 / sqrt(qw * qw + qx * qx + qy * qy + qz * qz);
    qw *= qinv; qx *= qinv; qy *= qinv; qz *= qinv;
    const double s0 = exp((double)a.log_scales[3 * i]);
    const double s1 = exp((double)a.log_scales[3 * i + 1]);
    const double s2 = exp((double)a.log_scales[3 * i + 2]);
    double M[9];
    M[0] = (1.0 - 2.0 * (qy * qy + qz * qz)) * s0;
    M[1] = 2.0 * (qx * qy - qw * qz) * s1;
    M[2] = 2.0 * (qx * qz + qw * qy) * s2;
    M[3] = 2.0 * (qx * qy + qw * qz) * s0;
    M[4] = (1.0 - 2.0 * (qx * qx + qz * qz)) * s1;
    M[5] = 2.0 * (qy * qz - qw * qx) * s2;
    M[6] = 2.0 * (qx * qz - qw * qy) * s0;
    M[7] = 2.0 * (qy * qz + qw * qx) * s1;
    M[8] = (1.0 - 2.0 * (qx * qx + qy * qy)) * s2;
    // alpha >= alpha_min ellipse: d^T conic d <= k2 = 2 ln(sigma / alpha_min)
    const double k2 = 2.0 * log(sigma / a.alpha_min);

    for (int view = 0; view < a.views; ++view) {
        const size_t o = (size_t)view * a.n + i;
        const CamArgs& c = a.cams[view];
        const double tx = c.R[0] * mx + c.R[1] * my + c.R[2] * mz + c.t[0];
        const double ty = c.R[3] * mx + c.R[4] * my + c.R[5] * mz + c.t[1];
        const double tz = c.R[6] * mx + c.R[7] * my + c.R[8] * mz + c.t[2];
        if (!(tz > a.near_z)) { cull(o); continue; }

        // T = J R_view (2x3), J the pinhole Jacobian at t; W = T M, cov2d = W W^T + dilation I
        const double iz = 1.0 / tz;
        const double j00 = c.fx * iz, j02 = -c.fx * tx * iz * iz;
        const double j11 = c.fy * iz, j12 = -c.fy * ty * iz * iz;
        double T0[3], T1[3];
        for (int k = 0; k < 3; ++k) {
            T0[k] = j00 * c.R[k] + j02 * c.R[6 + k];
            T1[k] = j11 * c.R[3 + k] + j12 * c.R[6 + k];
        }
        double W0[3], W1[3];
        for (int k = 0; k < 3; ++k) {
            W0[k] = T0[0] * M[k] + T0[1] * M[3 + k] + T0[2] * M[6 + k];
            W1[k] = T1[0] * M[k] + T1[1] * M[3 + k] + T1[2] * M[6 + k];
        }
        const double ca = W0[0] * W0[0] + W0[1] * W0[1] + W0[2] * W0[2] + a.dilation;
        const double cb = W0[0] * W1[0] + W0[1] * W1[1] + W0[2] * W1[2];
        const double cc = W1[0] * W1[0] + W1[1] * W1[1] + W1[2] * W1[2] + a.dilation;
        const double det = ca * cc - cb * cb;
        if (!(det > 0.0)) { cull(o); continue; }

        const double u = c.fx * tx * iz + c.cx;
        const double v = c.fy * ty * iz + c.cy;

        // bounding box of the alpha >= alpha_min ellipse: half-widths sqrt(k2 ca), sqrt(k2 cc)
        const double ex = sqrt(k2 * ca), ey = sqrt(k2 * cc);
        double xl = ceil(u - ex - 0.5), xh = floor(u + ex - 0.5);
        double yl = ceil(v - ey - 0.5), yh = floor(v + ey - 0.5);
        xl = fmax(xl, 0.0); yl = fmax(yl, 0.0);
        xh = fmin(xh, (double)(c.width - 1)); yh = fmin(yh, (double)(c.height - 1));
        int tx0 = 0, ty0 = 0, tx1 = 0, ty1 = 0, touched = 0;
        if (xl <= xh && yl <= yh) {
            tx0 = (int)xl / kTile; tx1 = (int)xh / kTile + 1;
            ty0 = (int)yl / kTile; ty1 = (int)yh / kTile + 1;
            touched = (tx1 - tx0) * (ty1 - ty0);
        }

        // colour: max(0, sum sh Y(dir) + 0.5), dir from the camera centre
        double rgb[3], dir[3];
        uint8_t cm = 0;
        shade<DEG>(c, mx, my, mz, shv, rgb, cm, dir);
        if constexpr (CJ) {
            // the colour's gradient with respect to the direction, for the 2D -> 3D backward
            // (computed in float32 from the float32 coefficients, as that backward would)
            float* jo = a.cjac + 9 * o;
#pragma unroll
            for (int ch = 0; ch < 3; ++ch) {
                float w[16];
#pragma unroll
                for (int k = 0; k < (DEG + 1) * (DEG + 1); ++k) w[k] = shv[3 * k + ch];
                float gx, gy, gz;
                sh_grad<DEG>((float)dir[0], (float)dir[1], (float)dir[2], w, gx, gy, gz);
                jo[3 * ch] = gx; jo[3 * ch + 1] = gy; jo[3 * ch + 2] = gz;
            }
        }

        // Cholesky factor of the conic, scaled so that G = exp2(-|L^T d|^2):
        // conic = [[cc, -cb], [-cb, ca]] / det = L L^T with
        // L00 = sqrt(cc / det), L10 = -cb / sqrt(cc det), L11 = 1 / sqrt(cc).
        const double sc = 0.84932180028801907;  // sqrt(log2(e) / 2)
        const double l00 = sqrt(cc / det) * sc;
        const double l10 = -cb / sqrt(cc * det) * sc;
        const double l11 = sc / sqrt(cc);

        const float uf = (float)u, vf = (float)v;
        if constexpr (H16) {
            // binary16 of the float32 value: the record is the float32 one, rounded.  Without
            // contraction the two roundings stay two (with it they may be folded into one
            // double -> binary16 rounding, which differs near binary16 ties).
#pragma clang fp contract(off)
            uint2* sp = reinterpret_cast<uint2*>(a.splats + o * GS_SPLAT16_STRIDE);
            sp[0] = make_uint2(__float_as_uint(uf), __float_as_uint(vf));
            sp[1] = make_uint2(pack_h2((float)l00, (float)l10), pack_h2((float)l11, (float)sigma));
            sp[2] = make_uint2(pack_h2((float)rgb[0], (float)rgb[1]), pack_h2((float)rgb[2], 0.f));
        } else {
            float4* sp = reinterpret_cast<float4*>(a.splats + o * GS_SPLAT_STRIDE);
            sp[0] = make_float4(uf, vf, (float)(u - (double)uf), (float)(v - (double)vf));
            sp[1] = make_float4((float)l00, (float)l10, (float)l11, (float)sigma);
            sp[2] = make_float4((float)rgb[0], (float)rgb[1], (float)rgb[2], 0.f);
        }
        a.clamp[o] = cm;
        a.depth[o] = (float)tz;
        const uint32_t r0 = (uint32_t)(uint16_t)tx0 | ((uint32_t)(uint16_t)ty0 << 16);
        const uint32_t r1 = (uint32_t)(uint16_t)tx1 | ((uint32_t)(uint16_t)ty1 << 16);
        reinterpret_cast<uint2*>(a.rect)[o] = make_uint2(r0, r1);
        a.tiles_touched[o] = touched;
    }
}

}  // namespace
}  // namespace gs

using namespace gs;

namespace gs {
namespace {

template <int DEG, bool VEC, bool H16>
void launch_pre_rec(dim3 grid, dim3 block, hipStream_t s, const PreArgs& a) {
    if (a.cjac)
        hipLaunchKernelGGL((k_preprocess<DEG, VEC, true, H16>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((k_preprocess<DEG, VEC, false, H16>), grid, block, 0, s, a);
}

template <int DEG, bool VEC>
void launch_pre(dim3 grid, dim3 block, hipStream_t s, const PreArgs& a) {
    if (a.h16)
        launch_pre_rec<DEG, VEC, true>(grid, block, s, a);
    else
        launch_pre_rec<DEG, VEC, false>(grid, block, s, a);
}

int preprocess_impl(const gs_camera* cams, int32_t views, const gs_settings* set, int32_t n,
                    int32_t sh_degree, const float* means, const float* log_scales, const float* quats,
                    const float* opacity_logits, const float* sh, float* splats, float* depth, int16_t* rect,
                    int32_t* tiles_touched, uint8_t* clamp_mask, float* cjac, void* stream, bool h16 = false) {
    if (!views_ok(cams, views) || n < 0 || sh_degree < 0 || sh_degree > GS_MAX_SH_DEGREE) return GS_EINVAL;
    if ((int64_t)views * n > (int64_t)INT32_MAX) return GS_ECAPACITY;
    if (!set) return GS_EINVAL;
    if (n == 0) return GS_OK;
    if (!means || !splats || !log_scales || !quats || !opacity_logits || !depth || !rect || !tiles_touched || !sh ||
        !clamp_mask)
        return GS_EINVAL;
    if (!(h16 ? aligned8(splats) : aligned16(splats)) || !aligned16(quats) || !aligned16(rect)) return GS_EALIGN;
    PreArgs a{};
    for (int v = 0; v < views; ++v) a.cams[v] = cam_args(cams + v);
    a.views = views;
    a.near_z = set->near_z; a.alpha_min = set->alpha_min; a.dilation = set->dilation;
    a.n = n;
    a.means = means; a.log_scales = log_scales; a.quats = quats; a.opac = opacity_logits; a.sh = sh;
    a.splats = splats; a.depth = depth; a.rect = rect; a.tiles_touched = tiles_touched; a.clamp = clamp_mask;
    a.cjac = cjac;
    a.h16 = h16;
    const dim3 grid((n + kPreBlock - 1) / kPreBlock), block(kPreBlock);
    hipStream_t s = as_stream(stream);
    const bool vec = aligned16(sh);
    switch (sh_degree) {
        case 0: launch_pre<0, false>(grid, block, s, a); break;
        case 1: vec ? launch_pre<1, true>(grid, block, s, a) : launch_pre<1, false>(grid, block, s, a); break;
        case 2: launch_pre<2, false>(grid, block, s, a); break;
        default: vec ? launch_pre<3, true>(grid, block, s, a) : launch_pre<3, false>(grid, block, s, a); break;
    }
    return launch_status();
}

}  // namespace
}  // namespace gs

extern "C" int gs_preprocess(const gs_camera* cam, const gs_settings* set, int32_t n, int32_t sh_degree,
                             const float* means, const float* log_scales, const float* quats,
                             const float* opacity_logits, const float* sh, float* splats, float* depth,
                             int16_t* rect, int32_t* tiles_touched, uint8_t* clamp_mask, void* stream) {
    return preprocess_impl(cam, 1, set, n, sh_degree, means, log_scales, quats, opacity_logits, sh,
                           splats, depth, rect, tiles_touched, clamp_mask, nullptr, stream);
}

extern "C" int gs_preprocess_colorjac(const gs_camera* cam, const gs_settings* set, int32_t n, int32_t sh_degree,
                                      const float* means, const float* log_scales, const float* quats,
                                      const float* opacity_logits, const float* sh, float* splats, float* depth,
                                      int16_t* rect, int32_t* tiles_touched, uint8_t* clamp_mask, float* colorjac,
                                      void* stream) {
    if (!colorjac && n > 0) return GS_EINVAL;
    return preprocess_impl(cam, 1, set, n, sh_degree, means, log_scales, quats, opacity_logits, sh,
                           splats, depth, rect, tiles_touched, clamp_mask, colorjac, stream);
}

extern "C" int gs_preprocess_views(const gs_camera* cams, int32_t views, const gs_settings* set, int32_t n,
                                   int32_t sh_degree, const float* means, const float* log_scales,
                                   const float* quats, const float* opacity_logits, const float* sh, float* splats,
                                   float* depth, int16_t* rect, int32_t* tiles_touched, uint8_t* clamp_mask,
                                   void* stream) {
    return preprocess_impl(cams, views, set, n, sh_degree, means, log_scales, quats, opacity_logits, sh,
                           splats, depth, rect, tiles_touched, clamp_mask, nullptr, stream);
}

extern "C" int gs_preprocess_h16(const gs_camera* cam, const gs_settings* set, int32_t n, int32_t sh_degree,
                                 const float* means, const float* log_scales, const float* quats,
                                 const float* opacity_logits, const float* sh, float* splats16, float* depth,
                                 int16_t* rect, int32_t* tiles_touched, uint8_t* clamp_mask, float* colorjac,
                                 void* stream) {
    return preprocess_impl(cam, 1, set, n, sh_degree, means, log_scales, quats, opacity_logits, sh,
                           splats16, depth, rect, tiles_touched, clamp_mask, colorjac, stream, true);
}
