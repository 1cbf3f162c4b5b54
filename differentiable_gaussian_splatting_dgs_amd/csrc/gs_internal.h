// Internal helpers of the HIP rasterizer library (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gs.h"

namespace gs {

constexpr int kTile = GS_TILE;                 // 16 x 16 pixel tiles
constexpr int kBlock = kTile * kTile;          // one workgroup per tile: 4 wave64
constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;  // log2(e)

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool aligned8(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 7u) == 0; }

inline int launch_status() { return hipGetLastError() == hipSuccess ? GS_OK : GS_EHIP; }

inline bool camera_ok(const gs_camera* c) {
    return c && c->width > 0 && c->height > 0 && c->width <= 32768 && c->height <= 32768 && c->fx > 0 &&
           c->fy > 0;
}

// views cameras of one image size (the batched entry points take an array).
inline bool views_ok(const gs_camera* cams, int32_t views) {
    if (!cams || views < 1 || views > GS_MAX_VIEWS) return false;
    for (int v = 0; v < views; ++v)
        if (!camera_ok(cams + v) || cams[v].width != cams[0].width || cams[v].height != cams[0].height) return false;
    return true;
}

inline int tiles_x(const gs_camera* c) { return (c->width + kTile - 1) / kTile; }
inline int tiles_y(const gs_camera* c) { return (c->height + kTile - 1) / kTile; }

// Gradient of sum_k w[k] Y_k with respect to the components (x, y, z) of the
// direction, Y the real SH basis of degree DEG taken as polynomials of three free
// variables (Gaussian Splatting backward CUDA page (lshu.cn), section 4: the colour
// gradient reaches the view direction through the SH basis); the projection onto
// the sphere is left to the caller.
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

// Camera and settings as plain kernel arguments.
struct CamArgs {
    double fx, fy, cx, cy;
    double R[9];
    double t[3];
    int32_t width, height;
};

inline CamArgs cam_args(const gs_camera* c) {
    CamArgs a;
    a.fx = c->fx; a.fy = c->fy; a.cx = c->cx; a.cy = c->cy;
    for (int i = 0; i < 9; ++i) a.R[i] = c->R[i];
    for (int i = 0; i < 3; ++i) a.t[i] = c->t[i];
    a.width = c->width; a.height = c->height;
    return a;
}

// Blend-side constants in float32 (the precision the blend decides in).
struct BlendArgs {
    float alpha_min, alpha_max, T_min;
    float bg[3];
    int32_t width, height, tiles_x, tiles_y;  // of one view
    int32_t views;                            // tile t is tile t mod (tiles_x tiles_y) of view t / (tiles_x tiles_y)
};

inline BlendArgs blend_args(const gs_camera* c, const gs_settings* s) {
    BlendArgs b;
    b.alpha_min = (float)s->alpha_min;
    b.alpha_max = (float)s->alpha_max;
    b.T_min = (float)s->T_min;
    for (int i = 0; i < 3; ++i) b.bg[i] = (float)s->bg[i];
    b.width = c->width; b.height = c->height;
    b.views = 1;
    b.tiles_x = tiles_x(c); b.tiles_y = tiles_y(c);
    return b;
}

// Blocks are dealt to the 8 XCDs round robin; give each XCD a contiguous
// band of tiles so neighbouring tiles (which share Gaussians) meet in one L2.
__device__ inline int xcd_tile(int block, int ntiles) {
    const int per = (ntiles + 7) / 8;
    const int xcd = block & 7, slot = block >> 3;
    const int t = xcd * per + slot;
    return t;  // may be >= ntiles for the last XCD; caller checks
}

}  // namespace gs
