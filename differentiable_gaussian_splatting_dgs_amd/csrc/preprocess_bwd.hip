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

constexpr int kG = 128;        // Gaussians per block: one per thread in the per-Gaussian phase
constexpr int kThreads = 256;  // threads per block for the staging and element-wise phases

struct AdamHyper {
    float* m[5];  // first moments: means, log_scales, quats, opacity_logits, sh
    float* v[5];  // second moments, same order
    float lr[6];  // means, log_scales, quats, opacity_logits, sh band 0, sh bands >= 1
    float b1, b2, eps, inv_c1, inv_sqrt_c2;
};

struct BwdArgs {
    CamArgs cams[GS_MAX_VIEWS];  // batched views: grad2d, tt, clamp are [views, n, ...]; gradients are summed
    int32_t views;
    float dilation;
    int32_t n;
    float* means;  // read; updated in place by the Adam variant
    float* log_scales;
    float* quats;
    float* opac;
    float* sh;
    const int32_t* tt;
    const uint8_t* clamp;
    const float* grad2d;
    float* dmeans;  // gradient outputs, each optional in the Adam variant
    float* dls;
    float* dquats;
    float* dopac;
    float* dsh;
    float* accum;   // densification statistic, optional
    int32_t* count;
    const float* cjac;  // the CJ variant: [n, 9] d colour_c / d dir_j from the forward preprocess
    AdamHyper adam;
};

// SH values Y[k] at unit direction (x, y, z).
template <int DEG>
__device__ __forceinline__ void sh_values(float x, float y, float z, float* Y) {
    // no contraction: the fused tail and its SH half must round these identically
#pragma clang fp contract(off)
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

// The Adam moments are streamed: read once and written once per step, and not
// touched by anything else in between.  Non-temporal accesses keep them from
// displacing the parameters and the projected data in the L2 and the Infinity
// Cache, which the next step's preprocess reads (measured: preprocess 102 ->
// 78 us, this kernel 288 -> 277 us on the 1M-Gaussian scene).
typedef float v4f __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float nt_ld(const float* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void nt_st(float v, float* p) { __builtin_nontemporal_store(v, p); }
__device__ __forceinline__ float4 nt_ld4(const float* p) {
    const v4f v = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(p));
    return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void nt_st4(float4 v, float* p) {
    v4f w;
    w.x = v.x; w.y = v.y; w.z = v.z; w.w = v.w;
    __builtin_nontemporal_store(w, reinterpret_cast<v4f*>(p));
}

// One Adam update on values already in registers: moments m, v and parameter p.
__device__ __forceinline__ void adam_reg(float& p, float g, float& m, float& v, float lr, const AdamHyper& h) {
    m = h.b1 * m + (1.f - h.b1) * g;
    v = h.b2 * v + (1.f - h.b2) * g * g;
    // hardware square root and reciprocal (1 ulp each) instead of the correctly
    // rounded sequences: a few instructions per element of a memory-bound pass
    p -= lr * (m * h.inv_c1) * __builtin_amdgcn_rcpf(__builtin_amdgcn_sqrtf(v) * h.inv_sqrt_c2 + h.eps);
}

// The per-Gaussian part of the chain: gradients of the mean, log-scales, raw
// quaternion and opacity logit, plus the SH basis and the clamp-masked colour
// gradient the SH coefficients need.  ddir needs the SH coefficients, read
// from the block's LDS copy (coefficient-major, row stride ldg).
// One view's inputs of the chain for one Gaussian: its 2D-gradient record,
// clamp mask and tile count (loaded ahead of use so a view loop can prefetch).
struct ViewIn {
    float4 g0, g1, g2;
    int32_t tt;
    uint8_t cm;
};

__device__ __forceinline__ ViewIn load_view(const BwdArgs& a, size_t iv) {
    ViewIn w;
    w.g0 = reinterpret_cast<const float4*>(a.grad2d)[3 * iv];
    w.g1 = reinterpret_cast<const float4*>(a.grad2d)[3 * iv + 1];
    w.g2 = reinterpret_cast<const float4*>(a.grad2d)[3 * iv + 2];
    w.tt = a.tt[iv];
    w.cm = a.clamp[iv];
    return w;
}

// 1 / x and 1 / sqrt(x) in float64 for a positive, finite x: the hardware
// float64 approximation refined by Newton steps (each doubles the correct bits),
// a few operations where the correctly rounded division is a long sequence.
__device__ __forceinline__ double rcp_f64(double x) {
    double r = __builtin_amdgcn_rcp(x);
    r = r * (2.0 - x * r);
    r = r * (2.0 - x * r);
    return r;
}
__device__ __forceinline__ double rsqrt_f64(double x) {
    double r = __builtin_amdgcn_rsq(x);
    r = r * (1.5 - 0.5 * x * r * r);
    r = r * (1.5 - 0.5 * x * r * r);
    return r;
}

// Gaussian i seen by camera c, with that view's inputs w.  CJ: the colour's
// direction gradient comes from a.cjac instead of the SH coefficients in s_sh.
template <int DEG, bool CJ = false>
__device__ __forceinline__ void chain(const BwdArgs& a, const CamArgs& c, int i, const ViewIn& w, const float* s_sh,
                                      int col, int ldg, float dmu[3], float dls[3], float dq[4], float& dop,
                                      float Y[16], float drgb[3]) {
    constexpr int K = (DEG + 1) * (DEG + 1);
    const float mx = a.means[3 * i], my = a.means[3 * i + 1], mz = a.means[3 * i + 2];

    const float4 g0 = w.g0, g1 = w.g1, g2 = w.g2;
    const float du = g0.x, dv = g0.y, dA = g0.z, dB = g0.w, dC = g1.x, dsig = g1.y;
    drgb[0] = g1.z; drgb[1] = g1.w; drgb[2] = g2.x;

    // opacity: the sigmoid and its derivative in float64, so that a saturated opacity
    // (sigma within 1e-5 of 1) keeps the relative accuracy of sigma (1 - sigma)
    const double sig = 1.0 / (1.0 + exp(-(double)a.opac[i]));
    dop = (float)((double)dsig * (sig * (1.0 - sig)));

    // colour -> SH; the view direction depends on the mean
    const float cpx = -(float)(c.R[0] * c.t[0] + c.R[3] * c.t[1] + c.R[6] * c.t[2]);
    const float cpy = -(float)(c.R[1] * c.t[0] + c.R[4] * c.t[1] + c.R[7] * c.t[2]);
    const float cpz = -(float)(c.R[2] * c.t[0] + c.R[5] * c.t[1] + c.R[8] * c.t[2]);
    const float vx = mx - cpx, vy = my - cpy, vz = mz - cpz;
    const float il = 1.f / sqrtf(vx * vx + vy * vy + vz * vz);
    const float dx = vx * il, dy = vy * il, dz = vz * il;
    const uint8_t cm = w.cm;
#pragma unroll
    for (int ch = 0; ch < 3; ++ch)
        if ((cm >> ch) & 1u) drgb[ch] = 0.f;
    sh_values<DEG>(dx, dy, dz, Y);
    float gdx = 0.f, gdy = 0.f, gdz = 0.f;
    if constexpr (CJ) {
        if constexpr (DEG > 0) {  // the gradient is the drgb-weighted sum of the colour rows
            const float* jr = a.cjac + 9 * (size_t)i;
#pragma unroll
            for (int ch = 0; ch < 3; ++ch) {
                gdx = __builtin_fmaf(drgb[ch], jr[3 * ch], gdx);
                gdy = __builtin_fmaf(drgb[ch], jr[3 * ch + 1], gdy);
                gdz = __builtin_fmaf(drgb[ch], jr[3 * ch + 2], gdz);
            }
        }
    } else {
        float wk[16];
#pragma unroll
        for (int k = 0; k < K; ++k)
            wk[k] = drgb[0] * s_sh[(3 * k) * ldg + col] + drgb[1] * s_sh[(3 * k + 1) * ldg + col] +
                    drgb[2] * s_sh[(3 * k + 2) * ldg + col];
        sh_grad<DEG>(dx, dy, dz, wk, gdx, gdy, gdz);
    }
    const float dot = dx * gdx + dy * gdy + dz * gdz;
    float dmx = (gdx - dx * dot) * il, dmy = (gdy - dy * dot) * il, dmz = (gdz - dz * dot) * il;

    // The geometric part of the chain runs in float64.  Its intermediates span many
    // orders of magnitude for strongly anisotropic Gaussians, and several steps are
    // differences of nearly equal products: the 2D covariance's determinant for a
    // flat Gaussian seen edge-on, and dT = 2 dA Sigma t0 + dB Sigma t1 when Sigma is
    // dominated by one long axis.  float64 runs at the float32 rate per instruction
    // on CDNA4, and this kernel is bound by memory, not by these few hundred operations.
    // rotation and scale: M = R(q/|q|) diag(s)
    const float4 q4 = reinterpret_cast<const float4*>(a.quats)[i];
    const double qn2 = (double)q4.x * q4.x + (double)q4.y * q4.y + (double)q4.z * q4.z + (double)q4.w * q4.w;
    const double iq = rsqrt_f64(qn2);
    const double qw = q4.x * iq, qx = q4.y * iq, qy = q4.z * iq, qz = q4.w * iq;
    // the scales in float64 like the rest of this part: where the scale gradient's two terms
    // cancel, a float32 scale's 2^-24 would be amplified by the cancellation
    const double s[3] = {exp((double)a.log_scales[3 * i]), exp((double)a.log_scales[3 * i + 1]),
                         exp((double)a.log_scales[3 * i + 2])};
    double R[9];
    R[0] = 1.0 - 2.0 * (qy * qy + qz * qz); R[1] = 2.0 * (qx * qy - qw * qz); R[2] = 2.0 * (qx * qz + qw * qy);
    R[3] = 2.0 * (qx * qy + qw * qz); R[4] = 1.0 - 2.0 * (qx * qx + qz * qz); R[5] = 2.0 * (qy * qz - qw * qx);
    R[6] = 2.0 * (qx * qz - qw * qy); R[7] = 2.0 * (qy * qz + qw * qx); R[8] = 1.0 - 2.0 * (qx * qx + qy * qy);
    double M[9];
#pragma unroll
    for (int r = 0; r < 3; ++r)
#pragma unroll
        for (int k = 0; k < 3; ++k) M[3 * r + k] = R[3 * r + k] * s[k];

    // T = J R_view with rows t0, t1; u = M^T t0, v = M^T t1: Sigma t0 = M u, Sigma t1 = M v, and the
    // 2D covariance before dilation is [[u.u, u.v], [u.v, v.v]]
    const double tx = c.R[0] * mx + c.R[1] * my + c.R[2] * mz + c.t[0];
    const double ty = c.R[3] * mx + c.R[4] * my + c.R[5] * mz + c.t[1];
    const double tz = c.R[6] * mx + c.R[7] * my + c.R[8] * mz + c.t[2];
    const double iz = rcp_f64(tz), iz2 = iz * iz, iz3 = iz2 * iz;
    const double j00 = c.fx * iz, j02 = -c.fx * tx * iz2, j11 = c.fy * iz, j12 = -c.fy * ty * iz2;
    double t0[3], t1[3], u[3], v[3];
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        t0[k] = j00 * c.R[k] + j02 * c.R[6 + k];
        t1[k] = j11 * c.R[3 + k] + j12 * c.R[6 + k];
    }
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        u[k] = M[k] * t0[0] + M[3 + k] * t0[1] + M[6 + k] * t0[2];
        v[k] = M[k] * t1[0] + M[3 + k] * t1[1] + M[6 + k] * t1[2];
    }
    const double dil = a.dilation;
    const double ca = u[0] * u[0] + u[1] * u[1] + u[2] * u[2] + dil;
    const double cb = u[0] * v[0] + u[1] * v[1] + u[2] * v[2];
    const double cc = v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + dil;
    const double D = ca * cc - cb * cb;
    const double iD = rcp_f64(D), iD2 = iD * iD;
    // conic = [[cc, -cb], [-cb, ca]] / D  ->  dL/d(2D covariance)
    const double da = (-cc * cc * dA + cb * cc * dB - cb * cb * dC) * iD2;
    const double db = (2.0 * cb * cc * dA - (ca * cc + cb * cb) * dB + 2.0 * ca * cb * dC) * iD2;
    const double dc = (-cb * cb * dA + ca * cb * dB - ca * ca * dC) * iD2;

    // dSigma = da t0 t0^T + db (t0 t1^T + t1 t0^T) / 2 + dc t1 t1^T.  With w0 = 2 da u + db v and
    // w1 = db u + 2 dc v (u = M^T t0, v = M^T t1):
    //   dT = dL/d(t0, t1) = 2 dSigma' -> (M w0, M w1)      (dT0 = 2 da Sigma t0 + db Sigma t1, ...)
    //   dM = 2 dSigma M = t0 w0^T + t1 w1^T                (Sigma = M M^T)
    double w0[3], w1[3], dT0[3], dT1[3];
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        w0[k] = 2.0 * da * u[k] + db * v[k];
        w1[k] = db * u[k] + 2.0 * dc * v[k];
    }
#pragma unroll
    for (int r = 0; r < 3; ++r) {
        dT0[r] = M[3 * r] * w0[0] + M[3 * r + 1] * w0[1] + M[3 * r + 2] * w0[2];
        dT1[r] = M[3 * r] * w1[0] + M[3 * r + 1] * w1[1] + M[3 * r + 2] * w1[2];
    }
    // T = J R_view  ->  dJ = dT R_view^T (only the four non-zero entries of J matter)
    const double dJ00 = dT0[0] * c.R[0] + dT0[1] * c.R[1] + dT0[2] * c.R[2];
    const double dJ02 = dT0[0] * c.R[6] + dT0[1] * c.R[7] + dT0[2] * c.R[8];
    const double dJ11 = dT1[0] * c.R[3] + dT1[1] * c.R[4] + dT1[2] * c.R[5];
    const double dJ12 = dT1[0] * c.R[6] + dT1[1] * c.R[7] + dT1[2] * c.R[8];
    const double dtx = -c.fx * iz2 * dJ02 + c.fx * iz * du;
    const double dty = -c.fy * iz2 * dJ12 + c.fy * iz * dv;
    const double dtz = -c.fx * iz2 * dJ00 + 2.0 * c.fx * tx * iz3 * dJ02 - c.fy * iz2 * dJ11 +
                       2.0 * c.fy * ty * iz3 * dJ12 - c.fx * tx * iz2 * du - c.fy * ty * iz2 * dv;
    dmu[0] = (float)(dmx + c.R[0] * dtx + c.R[3] * dty + c.R[6] * dtz);
    dmu[1] = (float)(dmy + c.R[1] * dtx + c.R[4] * dty + c.R[7] * dtz);
    dmu[2] = (float)(dmz + c.R[2] * dtx + c.R[5] * dty + c.R[8] * dtz);

    // M = R S: dL/ds_k = sum_r dM_rk R_rk and (R^T t0)_k = u_k / s_k, so the log-scale gradient
    // s_k dL/ds_k = w0_k u_k + w1_k v_k; dR_rk = dM_rk s_k
#pragma unroll
    for (int k = 0; k < 3; ++k) dls[k] = (float)(w0[k] * u[k] + w1[k] * v[k]);
    double dR[9];
#pragma unroll
    for (int r = 0; r < 3; ++r)
#pragma unroll
        for (int k = 0; k < 3; ++k) dR[3 * r + k] = (t0[r] * w0[k] + t1[r] * w1[k]) * s[k];
    const double gw = 2.0 * (-qz * dR[1] + qy * dR[2] + qz * dR[3] - qx * dR[5] - qy * dR[6] + qx * dR[7]);
    const double gx = 2.0 * (qy * dR[1] + qz * dR[2] + qy * dR[3] - 2.0 * qx * dR[4] - qw * dR[5] + qz * dR[6] +
                             qw * dR[7] - 2.0 * qx * dR[8]);
    const double gy = 2.0 * (-2.0 * qy * dR[0] + qx * dR[1] + qw * dR[2] + qx * dR[3] + qz * dR[5] - qw * dR[6] +
                             qz * dR[7] - 2.0 * qy * dR[8]);
    const double gz = 2.0 * (-2.0 * qz * dR[0] - qw * dR[1] + qx * dR[2] + qw * dR[3] - 2.0 * qz * dR[4] +
                             qy * dR[5] + qx * dR[6] + qy * dR[7]);
    const double pr = qw * gw + qx * gx + qy * gy + qz * gz;
    dq[0] = (float)((gw - qw * pr) * iq);
    dq[1] = (float)((gx - qx * pr) * iq);
    dq[2] = (float)((gy - qy * pr) * iq);
    dq[3] = (float)((gz - qz * pr) * iq);
}

// Element-wise SH part: the gradient Y_k dL/dc of each coefficient in HBM order
// (coalesced), written out and/or applied with Adam; kChunk elements per thread
// at a time, loads first.  The parameter comes from s_sh (the block's LDS copy)
// when given, else from HBM.
template <int DEG, bool ADAM, bool MV = false>
__device__ __forceinline__ void sh_elements(const BwdArgs& a, const float* s_sh, int LDG, const float* s_y,
                                            const float* s_c, int cnt, size_t base, int t) {
    constexpr int J = 3 * (DEG + 1) * (DEG + 1);
    constexpr int kChunk = 8;
    const AdamHyper& h = a.adam;
    float* const dsh = a.dsh;
    for (int e0 = t; e0 < cnt; e0 += kChunk * kThreads) {
        // Every read of the chunk, from HBM and from LDS, is issued before its first
        // store.  Indices past the end are clamped to the last element (cnt >= 1);
        // their values are never stored.
        float mv[kChunk], vv[kChunk], pv[kChunk], gr[kChunk];
        bool band0[kChunk];
        if (ADAM) {
#pragma unroll
            for (int c = 0; c < kChunk; ++c) {
                const int e = min(e0 + c * kThreads, cnt - 1);
                mv[c] = nt_ld(&h.m[4][base + e]);
                vv[c] = nt_ld(&h.v[4][base + e]);
                pv[c] = s_sh ? 0.f : a.sh[base + e];
            }
        }
#pragma unroll
        for (int c = 0; c < kChunk; ++c) {
            const int e = min(e0 + c * kThreads, cnt - 1);
            const int g = e / J, j = e - g * J;
            const int k = j / 3, ch = j - 3 * k;
            // MV: s_y holds the gradient itself (summed over the views), coefficient-major
            gr[c] = MV ? s_y[j * LDG + g] : s_y[k * LDG + g] * s_c[ch * LDG + g];
            if (ADAM && s_sh) pv[c] = s_sh[j * LDG + g];
            band0[c] = k == 0;
        }
#pragma unroll
        for (int c = 0; c < kChunk; ++c) {
            const int e = e0 + c * kThreads;
            if (e >= cnt) break;
            if (dsh) dsh[base + e] = gr[c];
            if (ADAM) {
                float p = pv[c];
                adam_reg(p, gr[c], mv[c], vv[c], band0[c] ? h.lr[4] : h.lr[5], h);
                a.sh[base + e] = p;
                nt_st(mv[c], &h.m[4][base + e]);
                nt_st(vv[c], &h.v[4][base + e]);
            }
        }
    }
}

// One block of kThreads threads per kG Gaussians.
//  phase 0: the block's SH coefficients, contiguous in HBM, are copied into LDS
//           coefficient-major (row stride kG + 1: conflict-free both ways);
//  phase 1: one thread per Gaussian (the first kG threads) runs the chain, writes or applies (Adam)
//           the mean / scale / quaternion / opacity gradients and the
//           densification statistic, and leaves Y and the colour gradient in LDS;
//  phase 2: the SH gradients Y_k dL/dc, element by element in HBM order, so
//           gradient writes and the Adam read-modify-write are coalesced.
// MV: a batch of a.views views; phase 1 runs the chain once per view in which
// the Gaussian touches a tile and sums the gradients (and the statistic over
// the views), and keeps the summed SH gradient itself in LDS for phase 2.
// CJ (one view, no Adam): the chain takes the colour's direction gradient from
// a.cjac, so phase 0 and the SH coefficients are not needed at all.
template <int DEG, bool ADAM, bool MV = false, bool CJ = false>
__global__ __launch_bounds__(kThreads) void k_grad3d(BwdArgs a) {
    static_assert(!CJ || (!ADAM && !MV), "the colour-Jacobian variant is the one-view gradient pass");
    constexpr int K = (DEG + 1) * (DEG + 1);
    constexpr int J = 3 * K;
    constexpr int LDG = kG + 1;
    __shared__ float s_sh[CJ ? 1 : J * LDG];
    __shared__ float s_y[(MV ? J : K) * LDG];
    __shared__ float s_c[(MV ? 1 : 3) * LDG];
    const int t = threadIdx.x;
    const int g0 = blockIdx.x * kG;
    const int ng = min(kG, a.n - g0);
    const int cnt = ng * J;
    const size_t base = (size_t)g0 * J;

    if constexpr (!CJ) {
        // every load of the thread's share is issued before the first LDS store,
        // so the block waits for one memory latency instead of one per batch
        constexpr int kPer = (J * kG + kThreads - 1) / kThreads;
        // a copy of the thread index the compiler cannot see through, so that it does
        // not keep this phase's index arithmetic alive for the element-wise phase
        int tl = t;
        asm volatile("" : "+v"(tl));
        float r[kPer];
#pragma unroll
        for (int c = 0; c < kPer; ++c)  // clamped (cnt >= 1): no branch around the loads
            r[c] = a.sh[base + min(tl + c * kThreads, cnt - 1)];
#pragma unroll
        for (int c = 0; c < kPer; ++c) {
            const int e = tl + c * kThreads;
            if (e < cnt) {
                const int g = e / J, j = e - g * J;
                s_sh[j * LDG + g] = r[c];
            }
        }
    }
    __syncthreads();

    if (t < ng) {
        const int i = g0 + t;
        // Every global load of this phase is issued before any store: the
        // parameter, moment and statistic arrays do not alias, but the compiler
        // cannot know that and would otherwise serialise each load behind the
        // previous store.
        float pm[3], pl[3], mm[3], vm[3], ml[3], vl[3], po = 0.f, mo = 0.f, vo = 0.f;
        float4 q4 = make_float4(0.f, 0.f, 0.f, 0.f), mq4 = q4, vq4 = q4;
        const AdamHyper& h = a.adam;
        if (ADAM) {
#pragma unroll
            for (int k = 0; k < 3; ++k) {
                pm[k] = a.means[3 * (size_t)i + k]; pl[k] = a.log_scales[3 * (size_t)i + k];
                mm[k] = nt_ld(&h.m[0][3 * (size_t)i + k]); vm[k] = nt_ld(&h.v[0][3 * (size_t)i + k]);
                ml[k] = nt_ld(&h.m[1][3 * (size_t)i + k]); vl[k] = nt_ld(&h.v[1][3 * (size_t)i + k]);
            }
            q4 = reinterpret_cast<const float4*>(a.quats)[i];
            mq4 = nt_ld4(h.m[2] + 4 * (size_t)i);
            vq4 = nt_ld4(h.v[2] + 4 * (size_t)i);
            po = a.opac[i]; mo = nt_ld(&h.m[3][i]); vo = nt_ld(&h.v[3][i]);
        }
        float acc = 0.f;
        int32_t nvis = 0;
        if (a.accum) { acc = a.accum[i]; nvis = a.count[i]; }
        float dmu[3] = {0.f, 0.f, 0.f}, dls[3] = {0.f, 0.f, 0.f}, dq[4] = {0.f, 0.f, 0.f, 0.f}, dop = 0.f;
        float Y[16], drgb[3] = {0.f, 0.f, 0.f};
        if constexpr (MV) {
#pragma unroll
            for (int j = 0; j < J; ++j) s_y[j * LDG + t] = 0.f;
            bool seen = false;
            ViewIn cur = load_view(a, (size_t)i);
            for (int view = 0; view < a.views; ++view) {
                // the next view's loads go out before this view's chain
                ViewIn nxt = cur;
                if (view + 1 < a.views) nxt = load_view(a, (size_t)(view + 1) * a.n + i);
                if (cur.tt <= 0) { cur = nxt; continue; }
                seen = true;
                float vmu[3], vls[3], vq[4], vop;
                chain<DEG>(a, a.cams[view], i, cur, s_sh, t, LDG, vmu, vls, vq, vop, Y, drgb);
#pragma unroll
                for (int k = 0; k < 3; ++k) { dmu[k] += vmu[k]; dls[k] += vls[k]; }
#pragma unroll
                for (int k = 0; k < 4; ++k) dq[k] += vq[k];
                dop += vop;
#pragma unroll
                for (int k = 0; k < K; ++k)
#pragma unroll
                    for (int ch = 0; ch < 3; ++ch) s_y[(3 * k + ch) * LDG + t] += Y[k] * drgb[ch];
                if (a.accum) {
                    acc += sqrtf(cur.g0.x * cur.g0.x + cur.g0.y * cur.g0.y);
                    nvis += 1;
                }
                cur = nxt;
            }
            if (a.accum && seen) {
                a.accum[i] = acc;
                a.count[i] = nvis;
            }
        } else {
            const bool vis = a.tt[i] > 0;
            if (vis) {
                chain<DEG, CJ>(a, a.cams[0], i, load_view(a, (size_t)i), s_sh, t, LDG, dmu, dls, dq, dop, Y, drgb);
                if (a.accum) {
                    const float2 d2 = *reinterpret_cast<const float2*>(a.grad2d + (size_t)i * GS_GRAD2D_STRIDE);
                    a.accum[i] = acc + sqrtf(d2.x * d2.x + d2.y * d2.y);
                    a.count[i] = nvis + 1;
                }
            } else {
#pragma unroll
                for (int k = 0; k < K; ++k) Y[k] = 0.f;
            }
        }
        if constexpr (!MV) {
#pragma unroll
            for (int k = 0; k < K; ++k) s_y[k * LDG + t] = Y[k];
            s_c[t] = drgb[0];
            s_c[LDG + t] = drgb[1];
            s_c[2 * LDG + t] = drgb[2];
        }
        if (a.dmeans) {
            a.dmeans[3 * (size_t)i] = dmu[0]; a.dmeans[3 * (size_t)i + 1] = dmu[1]; a.dmeans[3 * (size_t)i + 2] = dmu[2];
            a.dls[3 * (size_t)i] = dls[0]; a.dls[3 * (size_t)i + 1] = dls[1]; a.dls[3 * (size_t)i + 2] = dls[2];
            reinterpret_cast<float4*>(a.dquats)[i] = make_float4(dq[0], dq[1], dq[2], dq[3]);
            a.dopac[i] = dop;
        }
        if (ADAM) {
            float qv[4] = {q4.x, q4.y, q4.z, q4.w}, mq[4] = {mq4.x, mq4.y, mq4.z, mq4.w};
            float vq[4] = {vq4.x, vq4.y, vq4.z, vq4.w};
#pragma unroll
            for (int k = 0; k < 3; ++k) {
                adam_reg(pm[k], dmu[k], mm[k], vm[k], h.lr[0], h);
                adam_reg(pl[k], dls[k], ml[k], vl[k], h.lr[1], h);
            }
            float ss = 0.f;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                adam_reg(qv[k], dq[k], mq[k], vq[k], h.lr[2], h);
                ss += qv[k] * qv[k];
            }
            const float inv = 1.f / sqrtf(ss);  // renormalise after the update
            adam_reg(po, dop, mo, vo, h.lr[3], h);
#pragma unroll
            for (int k = 0; k < 3; ++k) {
                a.means[3 * (size_t)i + k] = pm[k]; a.log_scales[3 * (size_t)i + k] = pl[k];
                nt_st(mm[k], &h.m[0][3 * (size_t)i + k]); nt_st(vm[k], &h.v[0][3 * (size_t)i + k]);
                nt_st(ml[k], &h.m[1][3 * (size_t)i + k]); nt_st(vl[k], &h.v[1][3 * (size_t)i + k]);
            }
            reinterpret_cast<float4*>(a.quats)[i] = make_float4(qv[0] * inv, qv[1] * inv, qv[2] * inv, qv[3] * inv);
            nt_st4(make_float4(mq[0], mq[1], mq[2], mq[3]), h.m[2] + 4 * (size_t)i);
            nt_st4(make_float4(vq[0], vq[1], vq[2], vq[3]), h.v[2] + 4 * (size_t)i);
            a.opac[i] = po; nt_st(mo, &h.m[3][i]); nt_st(vo, &h.v[3][i]);
        }
    }
    __syncthreads();
    sh_elements<DEG, ADAM, MV>(a, CJ ? nullptr : s_sh, LDG, s_y, s_c, cnt, base, t);
}

template <bool ADAM, bool MV = false, bool CJ = false>
inline void launch_grad3d(int deg, const BwdArgs& a, hipStream_t s) {
    const dim3 grid((a.n + kG - 1) / kG), block(kThreads);
    switch (deg) {
        case 0: hipLaunchKernelGGL((k_grad3d<0, ADAM, MV, CJ>), grid, block, 0, s, a); break;
        case 1: hipLaunchKernelGGL((k_grad3d<1, ADAM, MV, CJ>), grid, block, 0, s, a); break;
        case 2: hipLaunchKernelGGL((k_grad3d<2, ADAM, MV, CJ>), grid, block, 0, s, a); break;
        default: hipLaunchKernelGGL((k_grad3d<3, ADAM, MV, CJ>), grid, block, 0, s, a); break;
    }
}

inline void fill_adam(BwdArgs& a, const gs_adam_state* adam) {
    for (int k = 0; k < 5; ++k) { a.adam.m[k] = adam->exp_avg[k]; a.adam.v[k] = adam->exp_avg_sq[k]; }
    for (int k = 0; k < 6; ++k) a.adam.lr[k] = adam->lr[k];
    a.adam.b1 = adam->beta1; a.adam.b2 = adam->beta2; a.adam.eps = adam->eps;
    a.adam.inv_c1 = (float)(1.0 / (1.0 - pow((double)adam->beta1, adam->step)));
    a.adam.inv_sqrt_c2 = (float)(1.0 / sqrt(1.0 - pow((double)adam->beta2, adam->step)));
}

inline void fill_common(BwdArgs& a, const gs_camera* cams, int32_t views, const gs_settings* set, int32_t n,
                        const float* means, const float* log_scales, const float* quats, const float* opacity_logits,
                        const float* sh, const int32_t* tt, const uint8_t* clamp, const float* grad2d) {
    a = BwdArgs{};
    for (int v = 0; v < views; ++v) a.cams[v] = cam_args(cams + v);
    a.views = views;
    a.dilation = (float)set->dilation;
    a.n = n;
    a.means = const_cast<float*>(means); a.log_scales = const_cast<float*>(log_scales);
    a.quats = const_cast<float*>(quats); a.opac = const_cast<float*>(opacity_logits); a.sh = const_cast<float*>(sh);
    a.tt = tt; a.clamp = clamp; a.grad2d = grad2d;
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
    fill_common(a, cam, 1, set, n, means, log_scales, quats, opacity_logits, sh, tiles_touched, clamp_mask, grad2d);
    a.dmeans = dmeans; a.dls = dlog_scales; a.dquats = dquats; a.dopac = dopacity_logits; a.dsh = dsh;
    launch_grad3d<false>(sh_degree, a, as_stream(stream));
    return launch_status();
}

extern "C" int gs_preprocess_bwd_colorjac(const gs_camera* cam, const gs_settings* set, int32_t n,
                                          int32_t sh_degree, const float* means, const float* log_scales,
                                          const float* quats, const float* opacity_logits, const float* colorjac,
                                          const int32_t* tiles_touched, const uint8_t* clamp_mask,
                                          const float* grad2d, float* dmeans, float* dlog_scales, float* dquats,
                                          float* dopacity_logits, float* dsh, void* stream) {
    if (!camera_ok(cam) || !set || n < 0 || sh_degree < 0 || sh_degree > GS_MAX_SH_DEGREE) return GS_EINVAL;
    if (n == 0) return GS_OK;
    if (!means || !log_scales || !quats || !opacity_logits || !colorjac || !tiles_touched || !clamp_mask ||
        !grad2d || !dmeans || !dlog_scales || !dquats || !dopacity_logits || !dsh)
        return GS_EINVAL;
    if (!aligned16(quats) || !aligned16(grad2d) || !aligned16(dquats)) return GS_EALIGN;
    BwdArgs a;
    fill_common(a, cam, 1, set, n, means, log_scales, quats, opacity_logits, nullptr, tiles_touched, clamp_mask,
                grad2d);
    a.dmeans = dmeans; a.dls = dlog_scales; a.dquats = dquats; a.dopac = dopacity_logits; a.dsh = dsh;
    a.cjac = colorjac;
    launch_grad3d<false, false, true>(sh_degree, a, as_stream(stream));
    return launch_status();
}

extern "C" int gs_preprocess_bwd_adam(const gs_camera* cam, const gs_settings* set, int32_t n, int32_t sh_degree,
                                      float* means, float* log_scales, float* quats, float* opacity_logits,
                                      float* sh, const int32_t* tiles_touched, const uint8_t* clamp_mask,
                                      const float* grad2d, const gs_adam_state* adam, float* densify_accum,
                                      int32_t* densify_count, float* dmeans, float* dlog_scales, float* dquats,
                                      float* dopacity_logits, float* dsh, void* stream) {
    if (!camera_ok(cam) || !set || !adam || n < 0 || sh_degree < 0 || sh_degree > GS_MAX_SH_DEGREE)
        return GS_EINVAL;
    if (adam->step < 1) return GS_EINVAL;
    if (n == 0) return GS_OK;
    if (!means || !log_scales || !quats || !opacity_logits || !sh || !tiles_touched || !clamp_mask || !grad2d)
        return GS_EINVAL;
    for (int k = 0; k < 5; ++k)
        if (!adam->exp_avg[k] || !adam->exp_avg_sq[k]) return GS_EINVAL;
    if ((densify_accum == nullptr) != (densify_count == nullptr)) return GS_EINVAL;
    const bool any_grad = dmeans || dlog_scales || dquats || dopacity_logits;
    if (any_grad && !(dmeans && dlog_scales && dquats && dopacity_logits)) return GS_EINVAL;
    if (!aligned16(quats) || !aligned16(grad2d) || (dquats && !aligned16(dquats))) return GS_EALIGN;
    if (!aligned16(adam->exp_avg[2]) || !aligned16(adam->exp_avg_sq[2])) return GS_EALIGN;
    BwdArgs a;
    fill_common(a, cam, 1, set, n, means, log_scales, quats, opacity_logits, sh, tiles_touched, clamp_mask, grad2d);
    a.dmeans = dmeans; a.dls = dlog_scales; a.dquats = dquats; a.dopac = dopacity_logits; a.dsh = dsh;
    a.accum = densify_accum; a.count = densify_count;
    fill_adam(a, adam);
    launch_grad3d<true>(sh_degree, a, as_stream(stream));
    return launch_status();
}

extern "C" int gs_preprocess_bwd_views(const gs_camera* cams, int32_t views, const gs_settings* set, int32_t n,
                                       int32_t sh_degree, const float* means, const float* log_scales,
                                       const float* quats, const float* opacity_logits, const float* sh,
                                       const int32_t* tiles_touched, const uint8_t* clamp_mask, const float* grad2d,
                                       float* dmeans, float* dlog_scales, float* dquats, float* dopacity_logits,
                                       float* dsh, void* stream) {
    if (!views_ok(cams, views) || !set || n < 0 || sh_degree < 0 || sh_degree > GS_MAX_SH_DEGREE) return GS_EINVAL;
    if ((int64_t)views * n > (int64_t)INT32_MAX) return GS_ECAPACITY;
    if (n == 0) return GS_OK;
    if (!means || !log_scales || !quats || !opacity_logits || !sh || !tiles_touched || !clamp_mask || !grad2d ||
        !dmeans || !dlog_scales || !dquats || !dopacity_logits || !dsh)
        return GS_EINVAL;
    if (!aligned16(quats) || !aligned16(grad2d) || !aligned16(dquats)) return GS_EALIGN;
    BwdArgs a;
    fill_common(a, cams, views, set, n, means, log_scales, quats, opacity_logits, sh, tiles_touched, clamp_mask,
                grad2d);
    a.dmeans = dmeans; a.dls = dlog_scales; a.dquats = dquats; a.dopac = dopacity_logits; a.dsh = dsh;
    launch_grad3d<false, true>(sh_degree, a, as_stream(stream));
    return launch_status();
}

extern "C" int gs_preprocess_bwd_adam_views(const gs_camera* cams, int32_t views, const gs_settings* set,
                                            int32_t n, int32_t sh_degree, float* means, float* log_scales,
                                            float* quats, float* opacity_logits, float* sh,
                                            const int32_t* tiles_touched, const uint8_t* clamp_mask,
                                            const float* grad2d, const gs_adam_state* adam, float* densify_accum,
                                            int32_t* densify_count, float* dmeans, float* dlog_scales,
                                            float* dquats, float* dopacity_logits, float* dsh, void* stream) {
    if (!views_ok(cams, views) || !set || !adam || n < 0 || sh_degree < 0 || sh_degree > GS_MAX_SH_DEGREE)
        return GS_EINVAL;
    if ((int64_t)views * n > (int64_t)INT32_MAX) return GS_ECAPACITY;
    if (adam->step < 1) return GS_EINVAL;
    if (n == 0) return GS_OK;
    if (!means || !log_scales || !quats || !opacity_logits || !sh || !tiles_touched || !clamp_mask || !grad2d)
        return GS_EINVAL;
    for (int k = 0; k < 5; ++k)
        if (!adam->exp_avg[k] || !adam->exp_avg_sq[k]) return GS_EINVAL;
    if ((densify_accum == nullptr) != (densify_count == nullptr)) return GS_EINVAL;
    const bool any_grad = dmeans || dlog_scales || dquats || dopacity_logits;
    if (any_grad && !(dmeans && dlog_scales && dquats && dopacity_logits)) return GS_EINVAL;
    if (!aligned16(quats) || !aligned16(grad2d) || (dquats && !aligned16(dquats))) return GS_EALIGN;
    if (!aligned16(adam->exp_avg[2]) || !aligned16(adam->exp_avg_sq[2])) return GS_EALIGN;
    BwdArgs a;
    fill_common(a, cams, views, set, n, means, log_scales, quats, opacity_logits, sh, tiles_touched, clamp_mask,
                grad2d);
    a.dmeans = dmeans; a.dls = dlog_scales; a.dquats = dquats; a.dopac = dopacity_logits; a.dsh = dsh;
    a.accum = densify_accum; a.count = densify_count;
    fill_adam(a, adam);
    launch_grad3d<true, true>(sh_degree, a, as_stream(stream));
    return launch_status();
}
