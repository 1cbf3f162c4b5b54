/*
 * gs_oracle.c -- CPU oracle for the differentiable tile rasterizer of 3D
 * Gaussian Splatting.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check
 * and the benchmark's CPU-baseline leg may call it; the product path never
 * does.  It shares no code, header or constant with the HIP library.
 *
 * Plain, slow, single-threaded, double precision.  No blocking, fusion or
 * reordering beyond what the method's definition states.
 *
 * Sources (cited by tag and section throughout):
 *  [P1] qqiyuan.cn, "3D Gaussian splatting backward propagation: chain-rule
 *       gradients explained, with pitfalls for beginners" -- the compositing
 *       equation I = sum_i alpha_i c_i prod_{j<i}(1 - alpha_j), and the
 *       central-difference gradient check.
 *  [P3] lshu.cn/news/59090, "CUDA implementation of Gaussian Splatting
 *       backpropagation: from pixel gradients to 3D Gaussian parameter
 *       updates" -- section 1 (architecture: pixel loss -> 2D attribute
 *       gradients -> 3D parameter gradients), section 2 (the recursion
 *       C_i = alpha_i c_i + (1 - alpha_i) C_{i+1}, alpha_i = min(0.99,
 *       sigma_i G_i), and the gradient table dL_dcolors / dL_dopacity /
 *       dL_dmean2D / dL_dconic2D), section 3 (reverse walk from the stored
 *       final transmittance, last contributor), section 4 (2D -> 3D chain:
 *       view transform, projection Jacobian dSigma = J^T dA J, SH basis,
 *       Sigma = R S S^T R^T).
 *  [P4] notes.huajishe.fun, "3DGS training and optimisation" -- C.2 (Adam
 *       with per-parameter learning rates), D.1 (densification statistic:
 *       accumulated position gradient), D.4 (quaternion rotation, renormalise
 *       after update), E.1 (training loop and loss), E.3 (tile rasterization:
 *       AABB cull against tiles, per-tile depth sort, splat in order).
 *
 * Readings where the pages are silent (the same readings the HIP path uses):
 *  - pixel (x, y) is sampled at (x + 0.5, y + 0.5);
 *  - d = pixel - mean2D, power = -0.5 (A dx^2 + C dy^2) - B dx dy with the
 *    conic [[A, B], [B, C]] = inverse of the 2D covariance;
 *  - skip a pair when alpha < alpha_min (1/255); stop a pixel *before*
 *    blending the entry whose T (1 - alpha) would fall below T_min (1e-4);
 *  - the 0.99 clamp has the exact derivative of min(): zero towards sigma
 *    and G when sigma G > 0.99;
 *  - 2D covariance = T Sigma T^T + dilation I, T = J R_view, J the pinhole
 *    Jacobian at the camera-space centre, no guard band;
 *  - cull when t_z <= near_z, sigma < alpha_min or det <= 0;
 *  - tile extent = bounding box of the exact alpha >= alpha_min ellipse,
 *    d^T A d <= 2 ln(sigma / alpha_min), so the tile cull is lossless;
 *  - colour = max(0, sum_lm sh_lm Y_lm(dir) + 0.5) per channel, real
 *    orthonormal SH with the Condon-Shortley phase, dir from the camera
 *    centre to the Gaussian's mean;
 *  - sort key = (tile, float32 depth, Gaussian index).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    double fx, fy, cx, cy;
    int32_t width, height;
    double R[9]; /* world -> camera rotation, row-major */
    double t[3]; /* world -> camera translation */
} orc_camera;

typedef struct {
    double near_z, alpha_min, alpha_max, T_min, dilation;
    double bg[3];
    int32_t tile;
} orc_settings;

/* ------------------------------------------------------------------------- */
/* Real spherical harmonics, degree <= 3, index l*l + l + m.                  */
/* Built from the complex Y_l^m with the Condon-Shortley phase:               */
/*   m < 0: sqrt(2) Im Y_l^|m|,  m = 0: Y_l^0,  m > 0: sqrt(2) Re Y_l^m,      */
/* written as polynomials in the unit direction (x, y, z).  Also returns the */
/* gradient of each polynomial with respect to (x, y, z) when grad != NULL.  */
/* [P3] section 4: colour gradients reach the SH coefficients through the    */
/* SH basis functions.                                                       */
/* ------------------------------------------------------------------------- */
void orc_sh_basis(int deg, const double d[3], double* Y, double* grad /* [K][3] or NULL */)
{
    const double PI = 3.14159265358979323846;
    const double x = d[0], y = d[1], z = d[2];
    double g[16][3];
    memset(g, 0, sizeof g);
    const double c0 = 0.5 * sqrt(1.0 / PI);
    Y[0] = c0;
    if (deg >= 1) {
        const double c1 = sqrt(3.0 / (4.0 * PI));
        Y[1] = -c1 * y;  g[1][1] = -c1;
        Y[2] =  c1 * z;  g[2][2] =  c1;
        Y[3] = -c1 * x;  g[3][0] = -c1;
    }
    if (deg >= 2) {
        const double a = 0.5 * sqrt(15.0 / PI);   /* m = +-2 (xy), +-1 */
        const double b = 0.25 * sqrt(5.0 / PI);   /* m = 0 */
        const double e = 0.25 * sqrt(15.0 / PI);  /* m = 2 (x^2 - y^2) */
        Y[4] =  a * x * y;                  g[4][0] = a * y;  g[4][1] = a * x;
        Y[5] = -a * y * z;                  g[5][1] = -a * z; g[5][2] = -a * y;
        Y[6] =  b * (2 * z * z - x * x - y * y);
        g[6][0] = -2 * b * x; g[6][1] = -2 * b * y; g[6][2] = 4 * b * z;
        Y[7] = -a * x * z;                  g[7][0] = -a * z; g[7][2] = -a * x;
        Y[8] =  e * (x * x - y * y);        g[8][0] = 2 * e * x; g[8][1] = -2 * e * y;
    }
    if (deg >= 3) {
        const double p = 0.25 * sqrt(35.0 / (2.0 * PI));   /* m = +-3 */
        const double q = 0.5 * sqrt(105.0 / PI);           /* m = -2 */
        const double r = 0.25 * sqrt(21.0 / (2.0 * PI));   /* m = +-1 */
        const double s = 0.25 * sqrt(7.0 / PI);            /* m = 0 */
        const double u = 0.25 * sqrt(105.0 / PI);          /* m = 2 */
        /* m = -3: -p y (3x^2 - y^2) */
        Y[9] = -p * y * (3 * x * x - y * y);
        g[9][0] = -p * 6 * x * y; g[9][1] = -p * (3 * x * x - 3 * y * y);
        /* m = -2: q x y z */
        Y[10] = q * x * y * z;
        g[10][0] = q * y * z; g[10][1] = q * x * z; g[10][2] = q * x * y;
        /* m = -1: -r y (4z^2 - x^2 - y^2) */
        Y[11] = -r * y * (4 * z * z - x * x - y * y);
        g[11][0] = -r * y * (-2 * x);
        g[11][1] = -r * (4 * z * z - x * x - 3 * y * y);
        g[11][2] = -r * y * (8 * z);
        /* m = 0: s z (2z^2 - 3x^2 - 3y^2) */
        Y[12] = s * z * (2 * z * z - 3 * x * x - 3 * y * y);
        g[12][0] = s * z * (-6 * x); g[12][1] = s * z * (-6 * y);
        g[12][2] = s * (6 * z * z - 3 * x * x - 3 * y * y);
        /* m = 1: -r x (4z^2 - x^2 - y^2) */
        Y[13] = -r * x * (4 * z * z - x * x - y * y);
        g[13][0] = -r * (4 * z * z - 3 * x * x - y * y);
        g[13][1] = -r * x * (-2 * y);
        g[13][2] = -r * x * (8 * z);
        /* m = 2: u z (x^2 - y^2) */
        Y[14] = u * z * (x * x - y * y);
        g[14][0] = u * z * 2 * x; g[14][1] = -u * z * 2 * y; g[14][2] = u * (x * x - y * y);
        /* m = 3: -p x (x^2 - 3y^2) */
        Y[15] = -p * x * (x * x - 3 * y * y);
        g[15][0] = -p * (3 * x * x - 3 * y * y); g[15][1] = -p * x * (-6 * y);
    }
    if (grad) {
        int K = (deg + 1) * (deg + 1);
        for (int k = 0; k < K; ++k)
            for (int c = 0; c < 3; ++c) grad[3 * k + c] = g[k][c];
    }
}

/* Rotation matrix of the unit quaternion q / |q|, q = (w, x, y, z).  [P4] D.4. */
void orc_quat_to_rot(const double q_in[4], double R[9])
{
    double n = sqrt(q_in[0] * q_in[0] + q_in[1] * q_in[1] + q_in[2] * q_in[2] + q_in[3] * q_in[3]);
    double w = q_in[0] / n, x = q_in[1] / n, y = q_in[2] / n, z = q_in[3] / n;
    R[0] = 1 - 2 * (y * y + z * z); R[1] = 2 * (x * y - w * z);     R[2] = 2 * (x * z + w * y);
    R[3] = 2 * (x * y + w * z);     R[4] = 1 - 2 * (x * x + z * z); R[5] = 2 * (y * z - w * x);
    R[6] = 2 * (x * z - w * y);     R[7] = 2 * (y * z + w * x);     R[8] = 1 - 2 * (x * x + y * y);
}

/* 3D covariance Sigma = R S S^T R^T with S = diag(exp(log_scales)).  [P3] section 4. */
static void cov3d(const double* ls, const double* q, double Sig[9], double M[9], double Rm[9], double s[3])
{
    orc_quat_to_rot(q, Rm);
    for (int j = 0; j < 3; ++j) s[j] = exp(ls[j]);
    for (int i = 0; i < 3; ++i)
        for (int j = 0; j < 3; ++j) M[3 * i + j] = Rm[3 * i + j] * s[j];
    for (int i = 0; i < 3; ++i)
        for (int j = 0; j < 3; ++j) {
            double acc = 0;
            for (int k = 0; k < 3; ++k) acc += M[3 * i + k] * M[3 * j + k];
            Sig[3 * i + j] = acc;
        }
}

/* Everything the projection of one Gaussian produces. */
typedef struct {
    double t[3];      /* camera-space centre */
    double J[6];      /* 2x3 pinhole Jacobian at t */
    double T[6];      /* J R_view */
    double Sig[9], M[9], Rm[9], s[3];
    double cov[3];    /* 2D covariance a, b, c (dilation included) */
    double det;
    double conic[3];  /* A, B, C */
    double u, v;
    double sigma;
    double dir[3], dist;
    double raw[3];    /* colour before the clamp at zero */
    int valid;
} orc_proj;

static int project_one(const orc_camera* cam, const orc_settings* set, int deg,
                       const double* mu, const double* ls, const double* q, double o,
                       const double* sh, orc_proj* P)
{
    memset(P, 0, sizeof *P);
    const double* Rv = cam->R;
    for (int i = 0; i < 3; ++i)
        P->t[i] = Rv[3 * i] * mu[0] + Rv[3 * i + 1] * mu[1] + Rv[3 * i + 2] * mu[2] + cam->t[i];
    if (P->t[2] <= set->near_z) return 0;
    const double tx = P->t[0], ty = P->t[1], tz = P->t[2];
    cov3d(ls, q, P->Sig, P->M, P->Rm, P->s);
    /* J = d(u,v)/dt for u = fx tx/tz + cx, v = fy ty/tz + cy */
    P->J[0] = cam->fx / tz; P->J[1] = 0;              P->J[2] = -cam->fx * tx / (tz * tz);
    P->J[3] = 0;            P->J[4] = cam->fy / tz;   P->J[5] = -cam->fy * ty / (tz * tz);
    for (int r = 0; r < 2; ++r)
        for (int c = 0; c < 3; ++c)
            P->T[3 * r + c] = P->J[3 * r] * Rv[c] + P->J[3 * r + 1] * Rv[3 + c] + P->J[3 * r + 2] * Rv[6 + c];
    /* 2D covariance T Sigma T^T + dilation I */
    double V[2][3];
    for (int r = 0; r < 2; ++r)
        for (int c = 0; c < 3; ++c)
            V[r][c] = P->Sig[3 * c] * P->T[3 * r] + P->Sig[3 * c + 1] * P->T[3 * r + 1] + P->Sig[3 * c + 2] * P->T[3 * r + 2];
    double a = P->T[0] * V[0][0] + P->T[1] * V[0][1] + P->T[2] * V[0][2] + set->dilation;
    double b = P->T[0] * V[1][0] + P->T[1] * V[1][1] + P->T[2] * V[1][2];
    double c = P->T[3] * V[1][0] + P->T[4] * V[1][1] + P->T[5] * V[1][2] + set->dilation;
    P->cov[0] = a; P->cov[1] = b; P->cov[2] = c;
    P->det = a * c - b * b;
    if (!(P->det > 0)) return 0;
    P->conic[0] = c / P->det; P->conic[1] = -b / P->det; P->conic[2] = a / P->det;
    P->sigma = 1.0 / (1.0 + exp(-o));
    if (P->sigma < set->alpha_min) return 0;
    P->u = cam->fx * tx / tz + cam->cx;
    P->v = cam->fy * ty / tz + cam->cy;
    /* colour from SH, [P3] section 4 */
    double campos[3];
    for (int i = 0; i < 3; ++i)
        campos[i] = -(Rv[i] * cam->t[0] + Rv[3 + i] * cam->t[1] + Rv[6 + i] * cam->t[2]);
    double dv[3] = {mu[0] - campos[0], mu[1] - campos[1], mu[2] - campos[2]};
    P->dist = sqrt(dv[0] * dv[0] + dv[1] * dv[1] + dv[2] * dv[2]);
    for (int i = 0; i < 3; ++i) P->dir[i] = dv[i] / P->dist;
    double Y[16];
    orc_sh_basis(deg, P->dir, Y, NULL);
    int K = (deg + 1) * (deg + 1);
    for (int ch = 0; ch < 3; ++ch) {
        double acc = 0;
        for (int k = 0; k < K; ++k) acc += sh[3 * k + ch] * Y[k];
        P->raw[ch] = acc + 0.5;
    }
    P->valid = 1;
    return 1;
}

/*
 * Per-Gaussian projection ([P4] E.3: only Gaussians meeting a tile are
 * projected; [P3] section 1: the forward's per-Gaussian results are reused by
 * the backward).  Outputs for culled Gaussians are zero with tiles_touched 0.
 * rect holds the tile rectangle [x0, x1) x [y0, y1) as x0, y0, x1, y1.
 */
int orc_preprocess(const orc_camera* cam, const orc_settings* set, int N, int deg,
                   const double* means, const double* log_scales, const double* quats,
                   const double* opacity_logits, const double* sh,
                   double* uv, double* depth, double* conic, double* cov2d, double* opacity,
                   double* rgb, unsigned char* clamp, double* ext, int* rect, int* tiles_touched,
                   unsigned char* valid)
{
    const int K = (deg + 1) * (deg + 1);
    const int ts = set->tile;
    for (int i = 0; i < N; ++i) {
        orc_proj P;
        int ok = project_one(cam, set, deg, means + 3 * i, log_scales + 3 * i, quats + 4 * i,
                             opacity_logits[i], sh + 3 * K * i, &P);
        valid[i] = (unsigned char)ok;
        uv[2 * i] = uv[2 * i + 1] = 0; depth[i] = 0; opacity[i] = 0;
        for (int c = 0; c < 3; ++c) { conic[3 * i + c] = 0; cov2d[3 * i + c] = 0; rgb[3 * i + c] = 0; }
        clamp[i] = 0; ext[2 * i] = ext[2 * i + 1] = 0;
        rect[4 * i] = rect[4 * i + 1] = rect[4 * i + 2] = rect[4 * i + 3] = 0;
        tiles_touched[i] = 0;
        if (!ok) continue;
        uv[2 * i] = P.u; uv[2 * i + 1] = P.v;
        depth[i] = P.t[2];
        opacity[i] = P.sigma;
        for (int c = 0; c < 3; ++c) {
            conic[3 * i + c] = P.conic[c];
            cov2d[3 * i + c] = P.cov[c];
            rgb[3 * i + c] = P.raw[c] < 0 ? 0.0 : P.raw[c];
            if (P.raw[c] < 0) clamp[i] |= (unsigned char)(1u << c);
        }
        /* alpha >= alpha_min  <=>  d^T A d <= k2 = 2 ln(sigma / alpha_min);
           the ellipse's bounding box has half-widths sqrt(k2 cov_xx), sqrt(k2 cov_yy). */
        double k2 = 2.0 * log(P.sigma / set->alpha_min);
        double ex = sqrt(k2 * P.cov[0]), ey = sqrt(k2 * P.cov[2]);
        ext[2 * i] = ex; ext[2 * i + 1] = ey;
        /* pixel x is inside iff |x + 0.5 - u| <= ex */
        double xl = ceil(P.u - ex - 0.5), xh = floor(P.u + ex - 0.5);
        double yl = ceil(P.v - ey - 0.5), yh = floor(P.v + ey - 0.5);
        if (xl < 0) xl = 0;
        if (yl < 0) yl = 0;
        if (xh > cam->width - 1) xh = cam->width - 1;
        if (yh > cam->height - 1) yh = cam->height - 1;
        if (xl > xh || yl > yh) continue;
        int x0 = (int)xl / ts, x1 = (int)xh / ts + 1, y0 = (int)yl / ts, y1 = (int)yh / ts + 1;
        rect[4 * i] = x0; rect[4 * i + 1] = y0; rect[4 * i + 2] = x1; rect[4 * i + 3] = y1;
        tiles_touched[i] = (x1 - x0) * (y1 - y0);
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Binning: per tile, the Gaussians whose tile rectangle contains it, ordered */
/* by (depth key, Gaussian index).  [P4] E.3: AABB cull against tiles, then a */
/* depth sort inside each tile.                                               */
/* ------------------------------------------------------------------------- */
static const double* g_sort_depth;

static int cmp_depth_index(const void* pa, const void* pb)
{
    int a = *(const int*)pa, b = *(const int*)pb;
    double da = g_sort_depth[a], db = g_sort_depth[b];
    if (da < db) return -1;
    if (da > db) return 1;
    return (a > b) - (a < b);
}

/* Returns K (number of (tile, Gaussian) pairs); writes at most `cap` list
   entries; ranges[2 t], ranges[2 t + 1] = [begin, end) of tile t. */
int64_t orc_bin(int N, int width, int height, int tile, const int* rect, const int* tiles_touched,
                const double* depth_key, int* point_list, int64_t cap, int64_t* ranges)
{
    const int tx = (width + tile - 1) / tile, ty = (height + tile - 1) / tile;
    const int nt = tx * ty;
    int64_t* count = (int64_t*)calloc((size_t)nt + 1, sizeof(int64_t));
    for (int i = 0; i < N; ++i) {
        if (tiles_touched[i] <= 0) continue;
        for (int y = rect[4 * i + 1]; y < rect[4 * i + 3]; ++y)
            for (int x = rect[4 * i]; x < rect[4 * i + 2]; ++x) count[y * tx + x]++;
    }
    int64_t K = 0;
    for (int t = 0; t < nt; ++t) {
        ranges[2 * t] = K;
        K += count[t];
        ranges[2 * t + 1] = K;
    }
    if (K > cap) { free(count); return K; }
    int64_t* fill = (int64_t*)calloc((size_t)nt, sizeof(int64_t));
    for (int i = 0; i < N; ++i) {
        if (tiles_touched[i] <= 0) continue;
        for (int y = rect[4 * i + 1]; y < rect[4 * i + 3]; ++y)
            for (int x = rect[4 * i]; x < rect[4 * i + 2]; ++x) {
                int t = y * tx + x;
                point_list[ranges[2 * t] + fill[t]++] = i;
            }
    }
    g_sort_depth = depth_key;
    for (int t = 0; t < nt; ++t) {
        int64_t n = ranges[2 * t + 1] - ranges[2 * t];
        if (n > 1) qsort(point_list + ranges[2 * t], (size_t)n, sizeof(int), cmp_depth_index);
    }
    free(fill);
    free(count);
    return K;
}

/* ------------------------------------------------------------------------- */
/* Forward compositing.  [P1] compositing equation; [P3] section 2:           */
/*   alpha = min(alpha_max, sigma G), G = exp(power).                         */
/* Each pixel walks its list front to back.  With global_list != 0 every     */
/* pixel walks ranges[0..1] (all Gaussians): the brute-force mode.           */
/* ------------------------------------------------------------------------- */
typedef struct {
    int idx;          /* Gaussian index */
    double alpha, T;  /* alpha and transmittance before this entry */
    double G, dx, dy;
    int clamped;
} orc_blend;

enum { AMB_SKIP = 1, AMB_STOP = 2, AMB_CLAMP = 4 };

/* Walks one pixel.  Stores blended entries in `out` (if non-NULL).  Returns the
   number blended; *n_contrib = list position of last blended + 1; *evaluated =
   entries evaluated (including the one that stops the pixel); *T_out = final T.
   *hash fingerprints the discrete decisions (which Gaussians blend, which are
   clamped, which one stops the pixel); skipped entries do not enter it. */
static int walk_pixel(const orc_settings* set, double px, double py, const int* list, int64_t len,
                      const double* uv, const double* conic, const double* opacity, const double* rgb,
                      orc_blend* out, double C[3], double* T_out, int* n_contrib, int64_t* evaluated,
                      double* wsum, int* amb, double amb_rel, uint64_t* hash)
{
    double T = 1.0;
    int nb = 0;
    *n_contrib = 0;
    *evaluated = 0;
    *wsum = 0;
    C[0] = C[1] = C[2] = 0;
    uint64_t h = 1469598103934665603ull;
    for (int64_t k = 0; k < len; ++k) {
        int g = list[k];
        (*evaluated)++;
        double dx = px - uv[2 * g], dy = py - uv[2 * g + 1];
        double A = conic[3 * g], B = conic[3 * g + 1], Cc = conic[3 * g + 2];
        double power = -0.5 * (A * dx * dx + Cc * dy * dy) - B * dx * dy;
        double G = exp(power);
        double sG = opacity[g] * G;
        double alpha = sG < set->alpha_max ? sG : set->alpha_max;
        if (fabs(sG - set->alpha_min) <= amb_rel * set->alpha_min) *amb |= AMB_SKIP;
        if (fabs(sG - set->alpha_max) <= amb_rel * set->alpha_max) *amb |= AMB_CLAMP;
        int code;
        if (alpha < set->alpha_min) {
            code = 1;
        } else {
            double Tn = T * (1.0 - alpha);
            if (fabs(Tn - set->T_min) <= amb_rel * set->T_min) *amb |= AMB_STOP;
            if (Tn < set->T_min) {
                code = 2;
                h = (h ^ (uint64_t)(g * 4 + code)) * 1099511628211ull;
                break;
            }
            code = sG > set->alpha_max ? 3 : 0;
            double w = alpha * T;
            for (int c = 0; c < 3; ++c) C[c] += w * rgb[3 * g + c];
            *wsum += w;
            if (out) {
                out[nb].idx = g; out[nb].alpha = alpha; out[nb].T = T; out[nb].G = G;
                out[nb].dx = dx; out[nb].dy = dy; out[nb].clamped = sG > set->alpha_max;
            }
            nb++;
            T = Tn;
            *n_contrib = (int)(k + 1);
        }
        if (code != 1) h = (h ^ (uint64_t)(g * 4 + code)) * 1099511628211ull;
    }
    *T_out = T;
    if (hash) *hash = h;
    return nb;
}

/* counts[0] = P_fwd (evaluated pairs), counts[1] = sum of n_contrib (walked by
   the backward), counts[2] = blended pairs; evaluated_px (optional, [H, W])
   receives each pixel's share of counts[0].  With tile_mask != NULL only the
   pixels of tiles whose mask byte is non-zero are composited (the others are
   left untouched); the backward then equals the full backward for an upstream
   gradient that is zero outside those tiles. */
int orc_render_fwd(const orc_camera* cam, const orc_settings* set, int global_list,
                   const int* point_list, const int64_t* ranges,
                   const double* uv, const double* conic, const double* opacity, const double* rgb,
                   double* image, double* final_T, int* n_contrib, double* wsum,
                   unsigned char* ambiguous, double amb_rel, uint64_t* decision_hash, int64_t* counts,
                   const unsigned char* tile_mask, int64_t* evaluated_px)
{
    const int W = cam->width, H = cam->height, ts = set->tile;
    const int tx = (W + ts - 1) / ts;
    counts[0] = counts[1] = counts[2] = 0;
    for (int y = 0; y < H; ++y)
        for (int x = 0; x < W; ++x) {
            if (tile_mask && !tile_mask[(y / ts) * tx + (x / ts)]) continue;
            int t = global_list ? 0 : (y / ts) * tx + (x / ts);
            int64_t b = ranges[2 * t], e = ranges[2 * t + 1];
            double C[3], T, ws;
            int nc, amb = 0;
            int64_t ev;
            uint64_t h;
            int nb = walk_pixel(set, x + 0.5, y + 0.5, point_list + b, e - b, uv, conic, opacity, rgb,
                                NULL, C, &T, &nc, &ev, &ws, &amb, amb_rel, &h);
            int p = y * W + x;
            for (int c = 0; c < 3; ++c) image[c * W * H + p] = C[c] + T * set->bg[c];
            final_T[p] = T;
            n_contrib[p] = nc;
            if (wsum) wsum[p] = ws;
            if (ambiguous) ambiguous[p] = (unsigned char)amb;
            if (decision_hash) decision_hash[p] = h;
            if (evaluated_px) evaluated_px[p] = ev;
            counts[0] += ev;
            counts[1] += nc;
            counts[2] += nb;
        }
    return 0;
}

/*
 * Backward compositing by explicit reverse recursion ([P3] sections 2-3),
 * with C_{n+1} = background:
 *   dL/dc_k     = T_k alpha_k dL/dpix
 *   dL/dalpha_k = T_k sum_ch dL/dpix_ch (c_k,ch - C_{k+1},ch)
 *   C_k         = alpha_k c_k + (1 - alpha_k) C_{k+1}
 * then alpha = sigma G (unclamped) and G = exp(power) give the opacity,
 * conic and 2D-mean gradients.  The stored alpha_k and T_k are recomputed per
 * pixel by the forward walk, so no division recovers T here.
 */
int orc_render_bwd(const orc_camera* cam, const orc_settings* set, int global_list,
                   const int* point_list, const int64_t* ranges,
                   const double* uv, const double* conic, const double* opacity, const double* rgb,
                   const double* dL_dimage, double* dL_dxy, double* dL_dconic, double* dL_dopacity,
                   double* dL_drgb, int N, const unsigned char* tile_mask, double* abs_sum)
{
    const int W = cam->width, H = cam->height, ts = set->tile;
    const int tx = (W + ts - 1) / ts;
    memset(dL_dxy, 0, sizeof(double) * 2 * (size_t)N);
    memset(dL_dconic, 0, sizeof(double) * 3 * (size_t)N);
    memset(dL_dopacity, 0, sizeof(double) * (size_t)N);
    memset(dL_drgb, 0, sizeof(double) * 3 * (size_t)N);
    if (abs_sum) memset(abs_sum, 0, sizeof(double) * 9 * (size_t)N);
    int64_t maxlen = 0;
    if (global_list) maxlen = ranges[1] - ranges[0];
    else {
        int nt = tx * ((H + ts - 1) / ts);
        for (int t = 0; t < nt; ++t)
            if (ranges[2 * t + 1] - ranges[2 * t] > maxlen) maxlen = ranges[2 * t + 1] - ranges[2 * t];
    }
    orc_blend* st = (orc_blend*)malloc(sizeof(orc_blend) * (size_t)(maxlen + 1));
    for (int y = 0; y < H; ++y)
        for (int x = 0; x < W; ++x) {
            if (tile_mask && !tile_mask[(y / ts) * tx + (x / ts)]) continue;
            int t = global_list ? 0 : (y / ts) * tx + (x / ts);
            int64_t b = ranges[2 * t], e = ranges[2 * t + 1];
            double C[3], T, ws;
            int nc, amb = 0;
            int64_t ev;
            int nb = walk_pixel(set, x + 0.5, y + 0.5, point_list + b, e - b, uv, conic, opacity, rgb,
                                st, C, &T, &nc, &ev, &ws, &amb, 0.0, NULL);
            int p = y * W + x;
            double gp[3] = {dL_dimage[p], dL_dimage[W * H + p], dL_dimage[2 * W * H + p]};
            double Cn[3] = {set->bg[0], set->bg[1], set->bg[2]};
            for (int k = nb - 1; k >= 0; --k) {
                const orc_blend* s = &st[k];
                int g = s->idx;
                const double* c = rgb + 3 * g;
                double dalpha = 0, adalpha = 0;
                for (int ch = 0; ch < 3; ++ch) {
                    dL_drgb[3 * g + ch] += s->T * s->alpha * gp[ch];
                    dalpha += gp[ch] * (c[ch] - Cn[ch]);
                    adalpha += fabs(gp[ch]) * (fabs(c[ch]) + fabs(Cn[ch]));
                    if (abs_sum) abs_sum[9 * g + 6 + ch] += fabs(s->T * s->alpha * gp[ch]);
                }
                dalpha *= s->T;
                adalpha *= s->T;
                for (int ch = 0; ch < 3; ++ch) Cn[ch] = s->alpha * c[ch] + (1.0 - s->alpha) * Cn[ch];
                if (s->clamped) continue;          /* alpha = alpha_max: no dependence on sigma or G */
                dL_dopacity[g] += s->G * dalpha;
                double dG = opacity[g] * dalpha;
                double dpow = s->G * dG;             /* G = exp(power) */
                const double A = conic[3 * g], B = conic[3 * g + 1], Cc = conic[3 * g + 2];
                dL_dconic[3 * g]     += -0.5 * s->dx * s->dx * dpow;
                dL_dconic[3 * g + 1] += -s->dx * s->dy * dpow;
                dL_dconic[3 * g + 2] += -0.5 * s->dy * s->dy * dpow;
                /* d = pixel - mean: d power / d mean = (A dx + B dy, B dx + C dy) */
                dL_dxy[2 * g]     += (A * s->dx + B * s->dy) * dpow;
                dL_dxy[2 * g + 1] += (B * s->dx + Cc * s->dy) * dpow;
                if (abs_sum) {
                    /* the size of each term added above, from |dL/dalpha|'s own terms: a
                       scale for the rounding a float32 evaluation of the same sums carries */
                    const double ap = s->G * opacity[g] * adalpha;  /* |dpow| from |dL/dalpha| */
                    double* a = abs_sum + 9 * g;
                    a[0] += (fabs(A * s->dx) + fabs(B * s->dy)) * ap;
                    a[1] += (fabs(B * s->dx) + fabs(Cc * s->dy)) * ap;
                    a[2] += 0.5 * s->dx * s->dx * ap;
                    a[3] += fabs(s->dx * s->dy) * ap;
                    a[4] += 0.5 * s->dy * s->dy * ap;
                    a[5] += s->G * adalpha;
                }
            }
        }
    free(st);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* 2D -> 3D gradients, [P3] section 4, by the plain chain rule on the steps  */
/* of project_one.  Gaussians with tiles_touched == 0 get zero gradients.    */
/* ------------------------------------------------------------------------- */
int orc_preprocess_bwd(const orc_camera* cam, const orc_settings* set, int N, int deg,
                       const double* means, const double* log_scales, const double* quats,
                       const double* opacity_logits, const double* sh, const int* tiles_touched,
                       const double* dL_dxy, const double* dL_dconic, const double* dL_dopacity,
                       const double* dL_drgb,
                       double* dmeans, double* dlog_scales, double* dquats, double* dopacity_logits,
                       double* dsh)
{
    const int K = (deg + 1) * (deg + 1);
    const double* Rv = cam->R;
    for (int i = 0; i < N; ++i) {
        double* dmu = dmeans + 3 * i;
        double* dls = dlog_scales + 3 * i;
        double* dq = dquats + 4 * i;
        double* dsh_i = dsh + 3 * K * i;
        for (int c = 0; c < 3; ++c) { dmu[c] = 0; dls[c] = 0; }
        for (int c = 0; c < 4; ++c) dq[c] = 0;
        dopacity_logits[i] = 0;
        for (int k = 0; k < 3 * K; ++k) dsh_i[k] = 0;
        if (tiles_touched[i] <= 0) continue;
        orc_proj P;
        if (!project_one(cam, set, deg, means + 3 * i, log_scales + 3 * i, quats + 4 * i,
                         opacity_logits[i], sh + 3 * K * i, &P))
            continue;
        const double tx = P.t[0], ty = P.t[1], tz = P.t[2];

        /* opacity: sigma = sigmoid(logit) */
        dopacity_logits[i] = dL_dopacity[i] * P.sigma * (1.0 - P.sigma);

        /* colour: rgb = max(0, sum sh Y(dir) + 0.5) */
        double Y[16], dY[48];
        orc_sh_basis(deg, P.dir, Y, dY);
        double drgb[3];
        for (int ch = 0; ch < 3; ++ch) drgb[ch] = P.raw[ch] < 0 ? 0.0 : dL_drgb[3 * i + ch];
        double ddir[3] = {0, 0, 0};
        for (int k = 0; k < K; ++k)
            for (int ch = 0; ch < 3; ++ch) {
                dsh_i[3 * k + ch] = Y[k] * drgb[ch];
                for (int a = 0; a < 3; ++a) ddir[a] += drgb[ch] * sh[3 * K * i + 3 * k + ch] * dY[3 * k + a];
            }
        /* dir = v / |v|: dv = (ddir - dir (dir . ddir)) / |v| */
        double dd = P.dir[0] * ddir[0] + P.dir[1] * ddir[1] + P.dir[2] * ddir[2];
        for (int a = 0; a < 3; ++a) dmu[a] += (ddir[a] - P.dir[a] * dd) / P.dist;

        /* conic = inverse of cov2d [[a, b], [b, c]]: A = c/D, B = -b/D, C = a/D, D = ac - b^2 */
        const double a = P.cov[0], b = P.cov[1], c = P.cov[2], D = P.det;
        const double dA = dL_dconic[3 * i], dB = dL_dconic[3 * i + 1], dC = dL_dconic[3 * i + 2];
        const double D2 = D * D;
        double da = (-c * c * dA + b * c * dB - b * b * dC) / D2;
        double db = (2 * b * c * dA - (a * c + b * b) * dB + 2 * a * b * dC) / D2;
        double dc = (-b * b * dA + a * b * dB - a * a * dC) / D2;

        /* a = t0 Sig t0^T + dil, b = t0 Sig t1^T, c = t1 Sig t1^T + dil (t0, t1 rows of T) */
        const double* t0 = P.T;
        const double* t1 = P.T + 3;
        double St0[3], St1[3];
        for (int r = 0; r < 3; ++r) {
            St0[r] = P.Sig[3 * r] * t0[0] + P.Sig[3 * r + 1] * t0[1] + P.Sig[3 * r + 2] * t0[2];
            St1[r] = P.Sig[3 * r] * t1[0] + P.Sig[3 * r + 1] * t1[1] + P.Sig[3 * r + 2] * t1[2];
        }
        double dSig[9]; /* gradient w.r.t. the (symmetric) 3D covariance, symmetrised */
        for (int r = 0; r < 3; ++r)
            for (int s = 0; s < 3; ++s)
                dSig[3 * r + s] = da * t0[r] * t0[s] + 0.5 * db * (t0[r] * t1[s] + t1[r] * t0[s]) + dc * t1[r] * t1[s];
        double dT[6];
        for (int r = 0; r < 3; ++r) {
            dT[r] = 2 * da * St0[r] + db * St1[r];
            dT[3 + r] = db * St0[r] + 2 * dc * St1[r];
        }
        /* T = J Rv  =>  dJ = dT Rv^T */
        double dJ[6];
        for (int r = 0; r < 2; ++r)
            for (int k = 0; k < 3; ++k)
                dJ[3 * r + k] = dT[3 * r] * Rv[3 * k] + dT[3 * r + 1] * Rv[3 * k + 1] + dT[3 * r + 2] * Rv[3 * k + 2];
        const double fx = cam->fx, fy = cam->fy;
        double dt[3] = {0, 0, 0};
        dt[0] += dJ[2] * (-fx / (tz * tz));
        dt[1] += dJ[5] * (-fy / (tz * tz));
        dt[2] += dJ[0] * (-fx / (tz * tz)) + dJ[2] * (2 * fx * tx / (tz * tz * tz))
               + dJ[4] * (-fy / (tz * tz)) + dJ[5] * (2 * fy * ty / (tz * tz * tz));
        /* u = fx tx / tz + cx, v = fy ty / tz + cy */
        const double du = dL_dxy[2 * i], dv = dL_dxy[2 * i + 1];
        dt[0] += du * fx / tz;
        dt[1] += dv * fy / tz;
        dt[2] += -du * fx * tx / (tz * tz) - dv * fy * ty / (tz * tz);
        /* t = Rv mu + tv  =>  dmu += Rv^T dt */
        for (int a2 = 0; a2 < 3; ++a2) dmu[a2] += Rv[a2] * dt[0] + Rv[3 + a2] * dt[1] + Rv[6 + a2] * dt[2];

        /* Sigma = M M^T, M = R S  =>  dM = 2 dSig M */
        double dM[9];
        for (int r = 0; r < 3; ++r)
            for (int s = 0; s < 3; ++s)
                dM[3 * r + s] = 2 * (dSig[3 * r] * P.M[s] + dSig[3 * r + 1] * P.M[3 + s] + dSig[3 * r + 2] * P.M[6 + s]);
        double dR[9];
        for (int r = 0; r < 3; ++r)
            for (int s = 0; s < 3; ++s) dR[3 * r + s] = dM[3 * r + s] * P.s[s];
        for (int s = 0; s < 3; ++s) {
            double ds = dM[s] * P.Rm[s] + dM[3 + s] * P.Rm[3 + s] + dM[6 + s] * P.Rm[6 + s];
            dls[s] = ds * P.s[s]; /* s = exp(log_scale) */
        }
        /* R(qn), qn = q / |q| */
        const double* q = quats + 4 * i;
        double qnorm = sqrt(q[0] * q[0] + q[1] * q[1] + q[2] * q[2] + q[3] * q[3]);
        double w = q[0] / qnorm, x = q[1] / qnorm, y = q[2] / qnorm, z = q[3] / qnorm;
        double dqn[4];
        dqn[0] = 2 * (-z * dR[1] + y * dR[2] + z * dR[3] - x * dR[5] - y * dR[6] + x * dR[7]);
        dqn[1] = 2 * (y * dR[1] + z * dR[2] + y * dR[3] - 2 * x * dR[4] - w * dR[5] + z * dR[6] + w * dR[7] - 2 * x * dR[8]);
        dqn[2] = 2 * (-2 * y * dR[0] + x * dR[1] + w * dR[2] + x * dR[3] + z * dR[5] - w * dR[6] + z * dR[7] - 2 * y * dR[8]);
        dqn[3] = 2 * (-2 * z * dR[0] - w * dR[1] + x * dR[2] + w * dR[3] - 2 * z * dR[4] + y * dR[5] + x * dR[6] + y * dR[7]);
        double qd = w * dqn[0] + x * dqn[1] + y * dqn[2] + z * dqn[3];
        double qn[4] = {w, x, y, z};
        for (int k = 0; k < 4; ++k) dq[k] = (dqn[k] - qn[k] * qd) / qnorm;
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Training-step tail.                                                       */
/* ------------------------------------------------------------------------- */

/* mode 1: L = sum |pred - target|, dL/dpred = sign (sign(0) = 0);
   mode 2: L = sum (pred - target)^2, dL/dpred = 2 (pred - target).
   [P4] E.1 (image reconstruction loss). */
double orc_loss(int mode, int64_t n, const double* pred, const double* target, double* dL_dpred)
{
    double L = 0;
    for (int64_t i = 0; i < n; ++i) {
        double r = pred[i] - target[i];
        if (mode == 1) {
            L += fabs(r);
            dL_dpred[i] = r > 0 ? 1.0 : (r < 0 ? -1.0 : 0.0);
        } else {
            L += r * r;
            dL_dpred[i] = 2.0 * r;
        }
    }
    return L;
}

/* Densification statistic, [P4] D.1 / E.1: per visible Gaussian, accumulate the
   norm of this view's 2D-mean gradient and count the view. */
void orc_densify(int N, const int* tiles_touched, const double* dL_dxy, double* accum, int* count)
{
    for (int i = 0; i < N; ++i) {
        if (tiles_touched[i] <= 0) continue;
        accum[i] += sqrt(dL_dxy[2 * i] * dL_dxy[2 * i] + dL_dxy[2 * i + 1] * dL_dxy[2 * i + 1]);
        count[i] += 1;
    }
}

/* Adam (Kingma and Ba), [P4] C.2: first and second moments with bias correction. */
void orc_adam(int64_t n, double* p, const double* g, double* m, double* v, double lr,
              double b1, double b2, double eps, int step)
{
    double c1 = 1.0 - pow(b1, step), c2 = 1.0 - pow(b2, step);
    for (int64_t i = 0; i < n; ++i) {
        m[i] = b1 * m[i] + (1.0 - b1) * g[i];
        v[i] = b2 * v[i] + (1.0 - b2) * g[i] * g[i];
        double mh = m[i] / c1, vh = v[i] / c2;
        p[i] -= lr * mh / (sqrt(vh) + eps);
    }
}

/* Quaternion renormalisation after the update, [P4] D.4. */
void orc_quat_renorm(int N, double* q)
{
    for (int i = 0; i < N; ++i) {
        double n = sqrt(q[4 * i] * q[4 * i] + q[4 * i + 1] * q[4 * i + 1] + q[4 * i + 2] * q[4 * i + 2] + q[4 * i + 3] * q[4 * i + 3]);
        for (int k = 0; k < 4; ++k) q[4 * i + k] /= n;
    }
}

/*
 * Densification and pruning, [P4] D.1-D.3 and E.1 steps 4-5: every 100
 * iterations, Gaussians whose accumulated position gradient is large are
 * densified -- split in two along the long axis when Sigma is anisotropic
 * (large eigenvalue ratio), cloned to a slightly offset copy when isotropic --
 * and Gaussians of low opacity are removed.  The pages give the rules and
 * leave the numbers out; prm[] carries them:
 *   prm[0] grad_threshold: densify when count > 0 and accum / count >= it;
 *   prm[1] prune_logit:    remove when the opacity logit is below it (the
 *                          outputs would inherit the opacity and go too);
 *   prm[2] split_log_gap:  split (else clone) when the largest minus the
 *                          smallest log-scale is at least it; the eigenvalue
 *                          ratio of Sigma is exp(2 gap);
 *   prm[3] split_shrink:   the children's log-scales are the parent's minus it;
 *   prm[4] split_offset, prm[5] clone_offset: displacements along the long
 *                          axis e (the column of R for the largest scale
 *                          s_max, first on ties), in units of s_max.
 * Each Gaussian is replaced, in index order, by its outputs:
 *   removed: none;  kept: itself;
 *   cloned: itself, then a copy at mean + clone_offset s_max e;
 *   split:  mean + split_offset s_max e, then mean - split_offset s_max e,
 *           both with log-scales minus split_shrink; rotation, opacity and
 *           SH copied.
 * Adam moments (mom_in / mom_out: m of the five groups, then v, or NULL): an
 * original keeps its own, a copy or a child starts at zero.  action[i] is 0
 * removed, 1 kept, 2 cloned, 3 split.  K = SH coefficients per Gaussian.
 * Returns the number of outputs (the arrays hold at least 2 N rows).
 */
int orc_densify_apply(int N, int K, const double* prm, const double* means, const double* log_scales,
                      const double* quats, const double* opacity, const double* sh, const double* accum,
                      const int* count, const double* const* mom_in, double* o_means, double* o_log_scales,
                      double* o_quats, double* o_opacity, double* o_sh, double* const* mom_out,
                      unsigned char* action)
{
    const int width[5] = {3, 3, 4, 1, 3 * K};
    const double* src[5] = {means, log_scales, quats, opacity, sh};
    double* dst[5] = {o_means, o_log_scales, o_quats, o_opacity, o_sh};
    int out = 0;
    for (int i = 0; i < N; ++i) {
        const double* ls = log_scales + 3 * i;
        int densify = count[i] > 0 && accum[i] / (double)count[i] >= prm[0];
        int removed = opacity[i] < prm[1];
        int a = 0; /* the longest axis */
        for (int j = 1; j < 3; ++j)
            if (ls[j] > ls[a]) a = j;
        double lmin = ls[0];
        for (int j = 1; j < 3; ++j)
            if (ls[j] < lmin) lmin = ls[j];
        int split = ls[a] - lmin >= prm[2];
        int act = removed ? 0 : (!densify ? 1 : (split ? 3 : 2));
        action[i] = (unsigned char)act;
        if (act == 0) continue;
        int nout = act == 1 ? 1 : 2;
        /* copy every group, then adjust */
        for (int o = 0; o < nout; ++o) {
            for (int g = 0; g < 5; ++g) {
                for (int c = 0; c < width[g]; ++c) {
                    dst[g][(size_t)(out + o) * width[g] + c] = src[g][(size_t)i * width[g] + c];
                    if (mom_in) {
                        int fresh = act == 3 || o == 1; /* a child or the copy */
                        for (int mv = 0; mv < 2; ++mv)
                            mom_out[5 * mv + g][(size_t)(out + o) * width[g] + c] =
                                fresh ? 0.0 : mom_in[5 * mv + g][(size_t)i * width[g] + c];
                    }
                }
            }
        }
        if (act >= 2) {
            double R[9];
            orc_quat_to_rot(quats + 4 * i, R);
            double smax = exp(ls[a]);
            double e[3] = {R[0 * 3 + a], R[1 * 3 + a], R[2 * 3 + a]};
            if (act == 2) {
                for (int c = 0; c < 3; ++c) o_means[(size_t)(out + 1) * 3 + c] = means[3 * i + c] + prm[5] * smax * e[c];
            } else {
                for (int c = 0; c < 3; ++c) {
                    o_means[(size_t)out * 3 + c] = means[3 * i + c] + prm[4] * smax * e[c];
                    o_means[(size_t)(out + 1) * 3 + c] = means[3 * i + c] - prm[4] * smax * e[c];
                }
                for (int o = 0; o < 2; ++o)
                    for (int c = 0; c < 3; ++c) o_log_scales[(size_t)(out + o) * 3 + c] = ls[c] - prm[3];
            }
        }
        out += nout;
    }
    return out;
}

/* Opacity reset, [P4] E.1 step 6: every 3000 iterations the opacity of every
   Gaussian is scaled by a factor (0.3 on the pages), written back as a logit. */
void orc_opacity_reset(int N, double factor, double* logit)
{
    for (int i = 0; i < N; ++i) {
        double s = 1.0 / (1.0 + exp(-logit[i]));
        double y = factor * s;
        logit[i] = log(y / (1.0 - y));
    }
}

/* ------------------------------------------------------------------------- */
/* 16-bit splat records.  [P3] section 5 stores some intermediate values as   */
/* 16-bit floats to save memory traffic; section 7 runs the rendering path in */
/* FP16 and keeps gradient accumulation in FP32.  The record this models      */
/* keeps the 2D mean in float32 and stores the conic (as its scaled Cholesky  */
/* factor), the opacity and the colour in IEEE 754 binary16.                  */
/* ------------------------------------------------------------------------- */

/* The binary16 number nearest to x, ties to the even significand (IEEE 754
 * binary16: 11-bit significand, exponents -14..15, subnormal spacing 2^-24,
 * largest finite 65504).  |x| >= 65520, the midpoint between 65504 and 2^16,
 * rounds to infinity.  Computed by scaling x to an integer multiple of its
 * binade's spacing, which is exact in double. */
double orc_round_binary16(double x)
{
    if (x != x || x == 0.0) return x;
    double a = fabs(x);
    if (a >= 65520.0) return x > 0 ? INFINITY : -INFINITY;
    int k;
    frexp(a, &k);              /* a = m 2^k, 0.5 <= m < 1: the binade is [2^(k-1), 2^k) */
    int e = k - 1;
    if (e < -14) e = -14;      /* subnormals share the spacing of the lowest binade */
    double s = ldexp(1.0, e - 10);
    double q = a / s;          /* exact: s is a power of two */
    double r = floor(q), f = q - r;
    if (f > 0.5 || (f == 0.5 && fmod(r, 2.0) != 0.0)) r += 1.0;
    double y = r * s;
    return x < 0 ? -y : y;
}

/* A value as the record stores it: the binary16 rounding of its float32
 * rounding (the record is written from the float32 projection). */
static double rec16(double v) { return orc_round_binary16((double)(float)v); }

/*
 * The 2D quantities a blend reads from a 16-bit record, for every Gaussian
 * (zero where valid[i] == 0).  The record holds
 *   u, v              the 2D mean rounded to float32;
 *   L00, L10, L11     the lower Cholesky factor of the conic A = Sigma'^-1
 *                     (Sigma' = [[a, b], [b, c]] the 2D covariance, det =
 *                     a c - b^2) scaled by s = sqrt(log2(e) / 2), so that
 *                     |L^T d|^2 = log2(e) d^T A d / 2:
 *                     L00 = s sqrt(c / det), L10 = -s b / sqrt(c det),
 *                     L11 = s / sqrt(c);
 *   opacity, r, g, b;
 * each of the last seven as rec16 gives it.  Out: uv16 = (u, v); conic16 =
 * the conic that record represents, L L^T / s^2 = (L00^2, L00 L10,
 * L10^2 + L11^2) / s^2 as (A, B, C); opacity16, rgb16.
 */
void orc_record16(int N, const double* uv, const double* cov2d, const double* opacity, const double* rgb,
                  const unsigned char* valid, double* uv16, double* conic16, double* opacity16, double* rgb16)
{
    const double s2 = 0.5 / log(2.0); /* s^2 = log2(e) / 2 */
    const double s = sqrt(s2);
    for (int i = 0; i < N; ++i) {
        uv16[2 * i] = uv16[2 * i + 1] = 0;
        conic16[3 * i] = conic16[3 * i + 1] = conic16[3 * i + 2] = 0;
        opacity16[i] = 0;
        rgb16[3 * i] = rgb16[3 * i + 1] = rgb16[3 * i + 2] = 0;
        if (!valid[i]) continue;
        const double a = cov2d[3 * i], b = cov2d[3 * i + 1], c = cov2d[3 * i + 2];
        const double det = a * c - b * b;
        const double l00 = rec16(s * sqrt(c / det));
        const double l10 = rec16(-s * b / sqrt(c * det));
        const double l11 = rec16(s / sqrt(c));
        uv16[2 * i] = (float)uv[2 * i];
        uv16[2 * i + 1] = (float)uv[2 * i + 1];
        conic16[3 * i] = l00 * l00 / s2;
        conic16[3 * i + 1] = l00 * l10 / s2;
        conic16[3 * i + 2] = (l10 * l10 + l11 * l11) / s2;
        opacity16[i] = rec16(opacity[i]);
        for (int ch = 0; ch < 3; ++ch) rgb16[3 * i + ch] = rec16(rgb[3 * i + ch]);
    }
}

/* orc_round_binary16 over an array (out may alias in). */
void orc_round_binary16_array(int64_t n, const double* in, double* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_round_binary16(in[i]);
}
