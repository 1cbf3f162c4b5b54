// 2D -> 3D gradients, one thread per Gaussian, float32.
//
// Method source: Gaussian Splatting backward CUDA page (lshu.cn), section 4:
// the 2D-mean gradient goes back through the perspective projection and the
// inverse view transform; the 2D covariance gradient goes to the 3D covariance
// as dSigma = T^T dSigma2D T with T = J R_view; colour gradients reach the SH
// coefficients through the SH basis; Sigma = R S S^T R^T gives the scale and
// rotation gradients by matrix differentials.  3DGS training notes (huajishe),
// D.4: the rotation comes from the normalised quaternion.
//
// The forward chain is recomputed from the parameters (nothing but the 2D
// gradients, tiles_touched and the clamp mask is carried over from the forward).
#include "gs_internal.h"

namespace gs {
namespace {

struct BwdArgs {
    CamArgs cam;
    float dilation;
    int32_t n;
    const float* means;
    const float* log_scales;
    const float* quats;
    const float* opac;
    const float* sh;
    const int32_t* tt;
    const uint8_t* clamp;
    const float* grad2d;
    float* dmeans;
    float* dls;
    float* dquats;
    float* dopac;
    float* dsh;
};

// SH values Y[k] at unit direction (x, y, z) and the gradient of
// sum_k w[k] Y_k with respect to (x, y, z).
template <int DEG>
__device__ __forceinline__ void sh_values(float x, float y, float z, float* Y) {
    Y[0] = 0.28209479177387814f;
    if (DEG >= 1) {
        Y[1] = -0.48860251190291992f * y;
        Y[2] = 0.48860251190291992f * z;
        Y[3] = -0.48860251190291992f * x;
    }
    if (DEG >= 2) {
        const float xx = x * x, yy = y * y, zz = z * z;
        Y[4] = 1.0925484305920792f * x * y;
        Y[5] = -1.0925484305920792f * y * z;
        Y[6] = 0.31539156525252005f * (2.f * zz - xx - yy);
        Y[7] = -1.0925484305920792f * x * z;
        Y[8] = 0.54627421529603959f * (xx - yy);
        if (DEG >= 3) {
            Y[9] = -0.59004358992664352f * y * (3.f * xx - yy);
            Y[10] = 2.8906114426405538f * x * y * z;
            Y[11] = -0.45704579946446572f * y * (4.f * zz - xx - yy);
            Y[12] = 0.37317633259011540f * z * (2.f * zz - 3.f * xx - 3.f * yy);
            Y[13] = -0.45704579946446572f * x * (4.f * zz - xx - yy);
            Y[14] = 1.4453057213202769f * z * (xx - yy);
            Y[15] = -0.59004358992664352f * x * (xx - 3.f * yy);
        }
    }
}

template <int DEG>
__device__ __forceinline__ void sh_grad(float x, float y, float z, const float* w, float& gx, float& gy,
                                        float& gz) {
    gx = gy = gz = 0.f;
    if (DEG >= 1) {
        const float c1 = 0.48860251190291992f;
        gx -= c1 * w[3];
        gy -= c1 * w[1];
        gz += c1 * w[2];
    }
    if (DEG >= 2) {
        const float A = 1.0925484305920792f, B = 0.31539156525252005f, E = 0.54627421529603959f;
        gx += A * y * w[4] - 2.f * B * x * w[6] - A * z * w[7] + 2.f * E * x * w[8];
        gy += A * x * w[4] - A * z * w[5] - 2.f * B * y * w[6] - 2.f * E * y * w[8];
        gz += -A * y * w[5] + 4.f * B * z * w[6] - A * x * w[7];
    }
    if (DEG >= 3) {
        const float P = 0.59004358992664352f, Q = 2.8906114426405538f, R = 0.45704579946446572f;
        const float S = 0.37317633259011540f, U = 1.4453057213202769f;
        const float xx = x * x, yy = y * y, zz = z * z;
        gx += -6.f * P * x * y * w[9] + Q * y * z * w[10] + 2.f * R * x * y * w[11] - 6.f * S * x * z * w[12] -
              R * (4.f * zz - 3.f * xx - yy) * w[13] + 2.f * U * x * z * w[14] - 3.f * P * (xx - yy) * w[15];
        gy += -3.f * P * (xx - yy) * w[9] + Q * x * z * w[10] - R * (4.f * zz - xx - 3.f * yy) * w[11] -
              6.f * S * y * z * w[12] + 2.f * R * x * y * w[13] - 2.f * U * y * z * w[14] + 6.f * P * x * y * w[15];
        gz += Q * x * y * w[10] - 8.f * R * y * z * w[11] + S * (6.f * zz - 3.f * xx - 3.f * yy) * w[12] -
              8.f * R * x * z * w[13] + U * (xx - yy) * w[14];
    }
}

template <int DEG>
__global__ __launch_bounds__(256) void k_preprocess_bwd(BwdArgs a) {
    constexpr int K = (DEG + 1) * (DEG + 1);
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= a.n) return;
    float* dmu = a.dmeans + 3 * (size_t)i;
    float* dls = a.dls + 3 * (size_t)i;
    float4* dq4 = reinterpret_cast<float4*>(a.dquats) + i;
    float* dshi = a.dsh + (size_t)i * K * 3;
    if (a.tt[i] <= 0) {
        dmu[0] = dmu[1] = dmu[2] = 0.f;
        dls[0] = dls[1] = dls[2] = 0.f;
        *dq4 = make_float4(0.f, 0.f, 0.f, 0.f);
        a.dopac[i] = 0.f;
        for (int k = 0; k < 3 * K; ++k) dshi[k] = 0.f;
        return;
    }
    const CamArgs& c = a.cam;
    const float Rv[9] = {(float)c.R[0], (float)c.R[1], (float)c.R[2], (float)c.R[3], (float)c.R[4],
                         (float)c.R[5], (float)c.R[6], (float)c.R[7], (float)c.R[8]};
    const float fx = (float)c.fx, fy = (float)c.fy;
    const float mx = a.means[3 * i], my = a.means[3 * i + 1], mz = a.means[3 * i + 2];
    const float tx = Rv[0] * mx + Rv[1] * my + Rv[2] * mz + (float)c.t[0];
    const float ty = Rv[3] * mx + Rv[4] * my + Rv[5] * mz + (float)c.t[1];
    const float tz = Rv[6] * mx + Rv[7] * my + Rv[8] * mz + (float)c.t[2];

    const float4 g0 = reinterpret_cast<const float4*>(a.grad2d)[3 * (size_t)i];
    const float4 g1 = reinterpret_cast<const float4*>(a.grad2d)[3 * (size_t)i + 1];
    const float4 g2 = reinterpret_cast<const float4*>(a.grad2d)[3 * (size_t)i + 2];
    const float du = g0.x, dv = g0.y, dA = g0.z, dB = g0.w, dC = g1.x, dsig = g1.y;
    float drgb[3] = {g1.z, g1.w, g2.x};

    // opacity
    const float sig = 1.f / (1.f + __expf(-a.opac[i]));
    a.dopac[i] = dsig * sig * (1.f - sig);

    // colour -> SH
    const float cpx = -(float)(c.R[0] * c.t[0] + c.R[3] * c.t[1] + c.R[6] * c.t[2]);
    const float cpy = -(float)(c.R[1] * c.t[0] + c.R[4] * c.t[1] + c.R[7] * c.t[2]);
    const float cpz = -(float)(c.R[2] * c.t[0] + c.R[5] * c.t[1] + c.R[8] * c.t[2]);
    const float vx = mx - cpx, vy = my - cpy, vz = mz - cpz;
    const float vlen = sqrtf(vx * vx + vy * vy + vz * vz);
    const float il = 1.f / vlen;
    const float dx = vx * il, dy = vy * il, dz = vz * il;
    const uint8_t cm = a.clamp[i];
#pragma unroll
    for (int ch = 0; ch < 3; ++ch)
        if ((cm >> ch) & 1u) drgb[ch] = 0.f;
    float Y[16], w[16];
    sh_values<DEG>(dx, dy, dz, Y);
    const float* shi = a.sh + (size_t)i * K * 3;
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const float s0 = shi[3 * k], s1 = shi[3 * k + 1], s2 = shi[3 * k + 2];
        w[k] = drgb[0] * s0 + drgb[1] * s1 + drgb[2] * s2;
        dshi[3 * k] = Y[k] * drgb[0];
        dshi[3 * k + 1] = Y[k] * drgb[1];
        dshi[3 * k + 2] = Y[k] * drgb[2];
    }
    float gdx, gdy, gdz;
    sh_grad<DEG>(dx, dy, dz, w, gdx, gdy, gdz);
    const float dot = dx * gdx + dy * gdy + dz * gdz;
    float dmx = (gdx - dx * dot) * il, dmy = (gdy - dy * dot) * il, dmz = (gdz - dz * dot) * il;

    // rotation and scale: M = R(q/|q|) diag(s)
    const float4 q = reinterpret_cast<const float4*>(a.quats)[i];
    const float qn = sqrtf(q.x * q.x + q.y * q.y + q.z * q.z + q.w * q.w);
    const float iq = 1.f / qn;
    const float qw = q.x * iq, qx = q.y * iq, qy = q.z * iq, qz = q.w * iq;
    const float s[3] = {__expf(a.log_scales[3 * i]), __expf(a.log_scales[3 * i + 1]),
                        __expf(a.log_scales[3 * i + 2])};
    float R[9];
    R[0] = 1.f - 2.f * (qy * qy + qz * qz); R[1] = 2.f * (qx * qy - qw * qz); R[2] = 2.f * (qx * qz + qw * qy);
    R[3] = 2.f * (qx * qy + qw * qz); R[4] = 1.f - 2.f * (qx * qx + qz * qz); R[5] = 2.f * (qy * qz - qw * qx);
    R[6] = 2.f * (qx * qz - qw * qy); R[7] = 2.f * (qy * qz + qw * qx); R[8] = 1.f - 2.f * (qx * qx + qy * qy);
    float M[9];
#pragma unroll
    for (int r = 0; r < 3; ++r)
#pragma unroll
        for (int k = 0; k < 3; ++k) M[3 * r + k] = R[3 * r + k] * s[k];
    float Sig[9];
#pragma unroll
    for (int r = 0; r < 3; ++r)
#pragma unroll
        for (int k = 0; k < 3; ++k) Sig[3 * r + k] = M[3 * r] * M[3 * k] + M[3 * r + 1] * M[3 * k + 1] + M[3 * r + 2] * M[3 * k + 2];

    // T = J R_view
    const float iz = 1.f / tz, iz2 = iz * iz;
    const float j00 = fx * iz, j02 = -fx * tx * iz2, j11 = fy * iz, j12 = -fy * ty * iz2;
    float t0[3], t1[3];
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        t0[k] = j00 * Rv[k] + j02 * Rv[6 + k];
        t1[k] = j11 * Rv[3 + k] + j12 * Rv[6 + k];
    }
    float St0[3], St1[3];
#pragma unroll
    for (int r = 0; r < 3; ++r) {
        St0[r] = Sig[3 * r] * t0[0] + Sig[3 * r + 1] * t0[1] + Sig[3 * r + 2] * t0[2];
        St1[r] = Sig[3 * r] * t1[0] + Sig[3 * r + 1] * t1[1] + Sig[3 * r + 2] * t1[2];
    }
    const float ca = t0[0] * St0[0] + t0[1] * St0[1] + t0[2] * St0[2] + a.dilation;
    const float cb = t0[0] * St1[0] + t0[1] * St1[1] + t0[2] * St1[2];
    const float cc = t1[0] * St1[0] + t1[1] * St1[1] + t1[2] * St1[2] + a.dilation;
    const float D = ca * cc - cb * cb;
    const float iD2 = 1.f / (D * D);
    // conic = [[cc, -cb], [-cb, ca]] / D
    const float da = (-cc * cc * dA + cb * cc * dB - cb * cb * dC) * iD2;
    const float db = (2.f * cb * cc * dA - (ca * cc + cb * cb) * dB + 2.f * ca * cb * dC) * iD2;
    const float dc = (-cb * cb * dA + ca * cb * dB - ca * ca * dC) * iD2;

    // dSigma (symmetric) and dT
    float dS[9];
#pragma unroll
    for (int r = 0; r < 3; ++r)
#pragma unroll
        for (int k = 0; k < 3; ++k)
            dS[3 * r + k] = da * t0[r] * t0[k] + 0.5f * db * (t0[r] * t1[k] + t1[r] * t0[k]) + dc * t1[r] * t1[k];
    float dT0[3], dT1[3];
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        dT0[k] = 2.f * da * St0[k] + db * St1[k];
        dT1[k] = db * St0[k] + 2.f * dc * St1[k];
    }
    // T = J R_view  ->  dJ = dT R_view^T (only the four non-zero entries of J matter)
    const float dJ00 = dT0[0] * Rv[0] + dT0[1] * Rv[1] + dT0[2] * Rv[2];
    const float dJ02 = dT0[0] * Rv[6] + dT0[1] * Rv[7] + dT0[2] * Rv[8];
    const float dJ11 = dT1[0] * Rv[3] + dT1[1] * Rv[4] + dT1[2] * Rv[5];
    const float dJ12 = dT1[0] * Rv[6] + dT1[1] * Rv[7] + dT1[2] * Rv[8];
    const float iz3 = iz2 * iz;
    const float dtx = -fx * iz2 * dJ02 + fx * iz * du;
    const float dty = -fy * iz2 * dJ12 + fy * iz * dv;
    const float dtz = -fx * iz2 * dJ00 + 2.f * fx * tx * iz3 * dJ02 - fy * iz2 * dJ11 + 2.f * fy * ty * iz3 * dJ12 -
                      fx * tx * iz2 * du - fy * ty * iz2 * dv;
    dmx += Rv[0] * dtx + Rv[3] * dty + Rv[6] * dtz;
    dmy += Rv[1] * dtx + Rv[4] * dty + Rv[7] * dtz;
    dmz += Rv[2] * dtx + Rv[5] * dty + Rv[8] * dtz;
    dmu[0] = dmx; dmu[1] = dmy; dmu[2] = dmz;

    // Sigma = M M^T -> dM = 2 dSigma M; M = R S -> dR, ds
    float dM[9];
#pragma unroll
    for (int r = 0; r < 3; ++r)
#pragma unroll
        for (int k = 0; k < 3; ++k)
            dM[3 * r + k] = 2.f * (dS[3 * r] * M[k] + dS[3 * r + 1] * M[3 + k] + dS[3 * r + 2] * M[6 + k]);
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        const float ds = dM[k] * R[k] + dM[3 + k] * R[3 + k] + dM[6 + k] * R[6 + k];
        dls[k] = ds * s[k];
    }
    float dR[9];
#pragma unroll
    for (int r = 0; r < 3; ++r)
#pragma unroll
        for (int k = 0; k < 3; ++k) dR[3 * r + k] = dM[3 * r + k] * s[k];
    const float gw = 2.f * (-qz * dR[1] + qy * dR[2] + qz * dR[3] - qx * dR[5] - qy * dR[6] + qx * dR[7]);
    const float gx = 2.f * (qy * dR[1] + qz * dR[2] + qy * dR[3] - 2.f * qx * dR[4] - qw * dR[5] + qz * dR[6] +
                            qw * dR[7] - 2.f * qx * dR[8]);
    const float gy = 2.f * (-2.f * qy * dR[0] + qx * dR[1] + qw * dR[2] + qx * dR[3] + qz * dR[5] - qw * dR[6] +
                            qz * dR[7] - 2.f * qy * dR[8]);
    const float gz = 2.f * (-2.f * qz * dR[0] - qw * dR[1] + qx * dR[2] + qw * dR[3] - 2.f * qz * dR[4] +
                            qy * dR[5] + qx * dR[6] + qy * dR[7]);
    const float pr = qw * gw + qx * gx + qy * gy + qz * gz;
    *dq4 = make_float4((gw - qw * pr) * iq, (gx - qx * pr) * iq, (gy - qy * pr) * iq, (gz - qz * pr) * iq);
}

}  // namespace
}  // namespace gs

using namespace gs;

extern "C" int gs_preprocess_bwd(const gs_camera* cam, const gs_settings* set, int32_t n, int32_t sh_degree,
                                 const float* means, const float* log_scales, const float* quats,
                                 const float* opacity_logits, const float* sh, const int32_t* tiles_touched,
                                 const uint8_t* clamp_mask, const float* grad2d, float* dmeans,
                                 float* dlog_scales, float* dquats, float* dopacity_logits, float* dsh,
                                 void* stream) {
    if (!camera_ok(cam) || !set || n < 0 || sh_degree < 0 || sh_degree > GS_MAX_SH_DEGREE) return GS_EINVAL;
    if (n == 0) return GS_OK;
    if (!means || !log_scales || !quats || !opacity_logits || !sh || !tiles_touched || !clamp_mask || !grad2d ||
        !dmeans || !dlog_scales || !dquats || !dopacity_logits || !dsh)
        return GS_EINVAL;
    if (!aligned16(quats) || !aligned16(grad2d) || !aligned16(dquats)) return GS_EALIGN;
    BwdArgs a;
    a.cam = cam_args(cam);
    a.dilation = (float)set->dilation;
    a.n = n;
    a.means = means; a.log_scales = log_scales; a.quats = quats; a.opac = opacity_logits; a.sh = sh;
    a.tt = tiles_touched; a.clamp = clamp_mask; a.grad2d = grad2d;
    a.dmeans = dmeans; a.dls = dlog_scales; a.dquats = dquats; a.dopac = dopacity_logits; a.dsh = dsh;
    const dim3 grid((n + 255) / 256), block(256);
    hipStream_t s = as_stream(stream);
    switch (sh_degree) {
        case 0: hipLaunchKernelGGL(k_preprocess_bwd<0>, grid, block, 0, s, a); break;
        case 1: hipLaunchKernelGGL(k_preprocess_bwd<1>, grid, block, 0, s, a); break;
        case 2: hipLaunchKernelGGL(k_preprocess_bwd<2>, grid, block, 0, s, a); break;
        default: hipLaunchKernelGGL(k_preprocess_bwd<3>, grid, block, 0, s, a); break;
    }
    return launch_status();
}
