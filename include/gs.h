/*
 * gs.h -- C ABI of the MI355X (gfx950) differentiable tile rasterizer for
 * 3D Gaussian Splatting.
 *
 * Sources cited by tag and section:
 *  [P3] lshu.cn/news/59090, "CUDA implementation of Gaussian Splatting
 *       backpropagation: from pixel gradients to 3D Gaussian parameter updates"
 *       (section 1 architecture and buffer reuse, section 2 gradient math,
 *       section 3 reverse per-pixel walk, section 4 2D -> 3D conversion,
 *       section 5 buffer reuse without dynamic allocation, section 6
 *       troubleshooting).
 *  [P4] notes.huajishe.fun, "3DGS training and optimisation" (C.2 Adam with
 *       per-parameter learning rates, D.1 densification statistic, D.4
 *       quaternion renormalisation, E.1 training loop, E.3 tile rasterization).
 *  [P1] qqiyuan.cn, "3D Gaussian splatting backward propagation: chain-rule
 *       gradients explained" (the compositing equation).
 *
 * Conventions shared by every call
 *  - Every array pointer is a DEVICE pointer (hipMalloc'd or a torch CUDA
 *    tensor's data_ptr), contiguous, in the row-major layout stated, aligned to
 *    16 bytes.  gs_camera / gs_settings / gs_adam_group arguments are HOST
 *    pointers, read during the call only.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Calls only enqueue work on that stream and return; none synchronises the
 *    host, none allocates device memory.  Scratch comes from caller-owned
 *    buffers ([P3] section 5: reuse buffers, no dynamic memory management).
 *  - The caller owns every buffer.  The library keeps no state between calls
 *    apart from its loaded code object; calls on different streams with
 *    disjoint buffers may run concurrently.
 *  - Return value: GS_OK (0) or a negative error code; on error nothing has
 *    been enqueued.  GS_EHIP means a kernel launch failed (the HIP error is
 *    left for hipGetLastError).  gs_error_string() names each code.
 *  - Tiles are 16 x 16 pixels.  Pixel (x, y) is sampled at (x + 0.5, y + 0.5).
 *    Images are planar [3, H, W] float32.
 */
#ifndef GS_MI355X_H
#define GS_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GS_TILE 16
#define GS_SPLAT_STRIDE 12  /* floats per projected-Gaussian record */
#define GS_GRAD2D_STRIDE 12 /* floats per 2D-gradient record */
#define GS_SPLAT16_STRIDE 6 /* 4-byte words per 16-bit projected-Gaussian record (24 bytes) */
#define GS_MAX_SH_DEGREE 3
#define GS_MAX_VIEWS 8      /* views one batched call renders */

enum {
    GS_OK = 0,
    GS_EINVAL = -1,     /* null pointer, negative size, unsupported degree, bad camera */
    GS_EALIGN = -2,     /* a pointer is not 16-byte aligned */
    GS_EWORKSPACE = -3, /* workspace_bytes smaller than gs_bin_workspace_size() */
    GS_EHIP = -4,       /* a kernel launch failed */
    GS_ECAPACITY = -5   /* a size exceeds what the kernels index (e.g. key_capacity > 2^30) */
};

/* Pinhole camera.  world -> camera: t = R mu + t.  u = fx t_x / t_z + cx. */
typedef struct gs_camera {
    double fx, fy, cx, cy;
    int32_t width, height;
    double R[9]; /* row-major */
    double t[3];
} gs_camera;

/* Rasterizer constants.  Defaults: near_z 0.2, alpha_min 1/255, alpha_max 0.99,
   T_min 1e-4, dilation 0.3 (pixels^2 added to the 2D covariance diagonal),
   bg = (0, 0, 0). */
typedef struct gs_settings {
    double near_z;
    double alpha_min;
    double alpha_max;
    double T_min;
    double dilation;
    double bg[3];
} gs_settings;

const char* gs_error_string(int code);
int gs_version(void);

/* Number of tiles along x and y for the camera's image. */
int gs_tile_grid(const gs_camera* cam, int32_t* tiles_x, int32_t* tiles_y);

/*
 * gs_preprocess -- per-Gaussian projection ([P3] sections 1 and 4 name the
 * forward intermediates the backward reuses; [P4] E.3: project, then cull
 * against tiles).  Computed in float64, stored in float32.
 *
 * In:  means [n,3], log_scales [n,3], quats [n,4] (w, x, y, z; any length,
 *      normalised inside), opacity_logits [n], sh [n, (deg+1)^2, 3]
 *      (index l*l + l + m, real SH with the Condon-Shortley phase).
 * Out (every Gaussian, culled ones zeroed):
 *   splats [n,12]: u, v        2D mean rounded to float32
 *                  u_res, v_res  (exact mean - rounded mean), float32
 *                  L00, L10, L11  lower Cholesky factor of the conic (inverse
 *                               2D covariance) times sqrt(log2(e)/2), so that
 *                               e = L^T d gives G = exp2(-|e|^2)
 *                  opacity     sigmoid(logit)
 *                  r, g, b     max(0, SH colour + 0.5)
 *                  0           (padding)
 *   depth [n]: camera-space z (sort key); rect [n,4] int16: tile rectangle
 *   [x0, x1) x [y0, y1) stored x0, y0, x1, y1 -- the bounding box of the exact
 *   alpha >= alpha_min ellipse; tiles_touched [n] int32: its area (0 = culled
 *   or off screen); clamp_mask [n] uint8: bit c set if colour channel c was
 *   clamped at 0.
 * Culling: t_z <= near_z, sigmoid(logit) < alpha_min, or det <= 0.
 */
int gs_preprocess(const gs_camera* cam, const gs_settings* set, int32_t n, int32_t sh_degree,
                  const float* means, const float* log_scales, const float* quats,
                  const float* opacity_logits, const float* sh,
                  float* splats, float* depth, int16_t* rect, int32_t* tiles_touched,
                  uint8_t* clamp_mask, void* stream);

/*
 * gs_preprocess_colorjac -- gs_preprocess that also keeps, for the 2D -> 3D
 * backward, the gradient of each colour channel with respect to the viewing
 * direction ([P3] section 4: the colour gradient reaches the mean through the
 * SH basis evaluated at the direction from the camera centre).
 * Out, besides gs_preprocess's: colorjac [n,9] float32, row-major by channel:
 *   colorjac[9 i + 3 c + j] = d(sum_k sh[i,k,c] Y_k(d)) / d d_j at the unit
 *   direction d of Gaussian i, the Y_k taken as polynomials of (d_x, d_y, d_z)
 *   (before the clamp at 0 and the +0.5; zero for culled Gaussians and at SH
 *   degree 0).  Caller-owned, 4-byte aligned; NULL is an error.
 * gs_preprocess_bwd_colorjac then needs no SH coefficients: 36 bytes per
 * Gaussian replace its (deg+1)^2 * 12 bytes of coefficients.
 */
int gs_preprocess_colorjac(const gs_camera* cam, const gs_settings* set, int32_t n, int32_t sh_degree,
                           const float* means, const float* log_scales, const float* quats,
                           const float* opacity_logits, const float* sh,
                           float* splats, float* depth, int16_t* rect, int32_t* tiles_touched,
                           uint8_t* clamp_mask, float* colorjac, void* stream);

/* Bytes of workspace gs_bin_sort needs for n Gaussians and key_capacity list
   entries. */
int gs_bin_workspace_size(int32_t n, const gs_camera* cam, int64_t key_capacity, size_t* bytes);

/*
 * gs_bin_sort -- tile binning and depth sort ([P4] E.3: cull against tiles,
 * sort by depth inside each tile; [P3] sections 1 and 5: the sorted list and
 * the tile ranges are reused by the backward).
 *
 * Produces, for every tile, the indices of the Gaussians whose rect covers it,
 * ordered by (float32 depth, Gaussian index): point_list [key_capacity] uint32
 * holds the lists tile after tile; tile_ranges [tiles, 2] uint32 holds each
 * tile's [begin, end) in point_list ([0, 0) when empty).
 * num_keys_dev [1] uint32 receives K = sum of tiles_touched (device memory; the
 * call does not read it back).  *overflow_dev [1] uint32 receives a status word:
 *   0      the lists and ranges are valid;
 *   bit 0  K > key_capacity: retry with a capacity of at least K;
 *   bit 1  a pass of the depth radix sort gave up waiting for the partitions
 *          before it (see gs_debug_sort_wait_limit; not expected in normal
 *          operation): the sort is void and a retry may succeed.
 * When the word is not 0, every range is written empty and point_list holds no
 * valid list.  The caller checks the word after its next synchronisation.
 * workspace: device scratch of at least gs_bin_workspace_size() bytes, 256-byte
 * aligned; its contents on entry do not matter.
 * Limits: GS_ECAPACITY when the image has more than 65536 tiles (the tile sort
 * takes two 8-bit digit passes; 65536 tiles is 4096 x 4096 pixels) or when
 * key_capacity or n exceeds 2^30 - 1.
 */
int gs_bin_sort(const gs_camera* cam, int32_t n, const float* depth, const int16_t* rect,
                const int32_t* tiles_touched, int64_t key_capacity,
                uint32_t* point_list, uint32_t* tile_ranges, uint32_t* num_keys_dev,
                uint32_t* overflow_dev, void* workspace, size_t workspace_bytes, void* stream);

/*
 * gs_debug_sort_wait_limit -- test hook for the sort's failure report.  Each
 * pass of the depth radix sort (an LSD "onesweep" pass: partitions add their
 * digit counts to a running prefix published by the partitions before them)
 * waits a bounded number of times for a predecessor's prefix; past the limit
 * the partition gives up and the call reports bit 1 in *overflow_dev.  Sets the limit for
 * later gs_bin_sort calls in this process (limit < 0: leave it) and returns
 * the previous one.  Default 4194304 waits; 0 makes every partition but the
 * first give up at once, so a sort deterministically reports failure while
 * every kernel still runs to completion.
 */
int64_t gs_debug_sort_wait_limit(int64_t limit);

/*
 * gs_bin_sort_noalloc -- gs_bin_sort for callers that cannot allocate device
 * memory or hand over a workspace: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Same arguments, results and status
 * word as gs_bin_sort, without the workspace: the call uses a scratch buffer of
 * gs_bin_scratch_bytes() (128 MiB) that the library holds on each GPU for the
 * life of the process, and allocates nothing.  GS_EWORKSPACE when
 * gs_bin_workspace_size(n, cam, key_capacity) exceeds it (about n = 1M
 * Gaussians with 8M list entries).  The first call on a device looks the
 * buffer's address up (hipGetSymbolAddress) and must run on the device the
 * stream belongs to; make it outside graph capture.  Every call on one GPU uses
 * the same buffer: calls that overlap in time on one GPU (other streams, other
 * threads) race and must be serialised by the caller.
 */
int gs_bin_sort_noalloc(const gs_camera* cam, int32_t n, const float* depth, const int16_t* rect,
                        const int32_t* tiles_touched, int64_t key_capacity, uint32_t* point_list,
                        uint32_t* tile_ranges, uint32_t* num_keys_dev, uint32_t* overflow_dev, void* stream);
int64_t gs_bin_scratch_bytes(void);

/* Diagnostic: the 64-bit sort keys (tile << 32 | float32 depth bits) of the
   sorted list, keys [key_capacity]; entries at and beyond K are left alone. */
int gs_bin_keys(const gs_camera* cam, const uint32_t* tile_ranges, const uint32_t* point_list,
                const float* depth, uint64_t* keys, void* stream);

/*
 * gs_render_fwd -- front-to-back compositing per pixel ([P1] compositing
 * equation; [P3] section 2: alpha = min(alpha_max, opacity G)).
 * A pair is skipped when alpha < alpha_min; a pixel stops before the entry
 * whose T (1 - alpha) would fall below T_min.
 * Out: image [3,H,W] = C + T_final bg; final_T [H,W]; n_contrib [H,W] int32 =
 * position in the tile's list of the last blended entry + 1 (0 if none);
 * contrib [key_capacity] uint8, one byte per point_list entry: bit q (q = 0..3,
 * the 8x8 quadrants of the tile in row-major order) is set if some pixel of
 * quadrant q blended the entry.  Only entries up to the last one any pixel of
 * the tile blends are written.  gs_render_bwd reads it back ([P3] sections 1
 * and 5: the backward reuses the forward's intermediates).
 * tile_order [2, tiles] int32, optional (NULL: tiles in image order): schedules,
 * each a permutation of the tile ids with the heaviest tiles first so that long
 * tiles start first.  Row 0 is the forward's own (work = list length), row 1
 * the backward's (work estimated from the flags): pass tile_order + tiles to
 * gs_render_bwd.
 * grad2d_clear [n,12] float32, optional: set to zero by the same kernel (its
 * memory traffic overlaps the blending), for a gs_render_bwd call with
 * accumulate = 1, which then needs no clearing pass of its own.
 */
int gs_render_fwd(const gs_camera* cam, const gs_settings* set, int32_t n,
                  const uint32_t* tile_ranges, const uint32_t* point_list, const float* splats,
                  float* image, float* final_T, int32_t* n_contrib, uint8_t* contrib,
                  int32_t* tile_order, float* grad2d_clear, void* stream);

/*
 * gs_render_fwd_loss -- gs_render_fwd with the image loss of gs_image_loss
 * fused into the blend ([P4] E.1: render, then the reconstruction loss): each
 * pixel's dL/dimage is written as soon as its colour is known.  loss_mode 1:
 * L1 (dL/dimage = sign(image - target), sign(0) = 0); 2: L2 (2 (image -
 * target)).  target, dL_dimage [3,H,W] float32.  loss_dev [1 + tiles] float64:
 * loss_dev[0] receives the loss (tile sums added in a fixed order:
 * deterministic), loss_dev[1 + t] the sum over tile t.  grad2d_clear [n,12]
 * float32, optional: set to zero by the same kernel, for a gs_render_bwd call
 * with accumulate = 1.  Other arguments and outputs as gs_render_fwd.
 */
int gs_render_fwd_loss(const gs_camera* cam, const gs_settings* set, int32_t n,
                       const uint32_t* tile_ranges, const uint32_t* point_list, const float* splats,
                       float* image, float* final_T, int32_t* n_contrib, uint8_t* contrib,
                       int32_t* tile_order, int32_t loss_mode, const float* target, float* dL_dimage,
                       double* loss_dev, float* grad2d_clear, void* stream);

/*
 * gs_render_bwd -- reverse per-pixel walk from the stored final
 * transmittance ([P3] section 3), gradients per [P3] section 2:
 *   dL/dc = T alpha dL/dpix;  dL/dalpha = T sum_ch dL/dpix_ch (c_ch - C_next,ch)
 * with C_next starting at the background; then through alpha = opacity G
 * (zero when clamped) and G = exp(power).
 * In: final_T, n_contrib and contrib from gs_render_fwd (only entries whose
 * contrib bit is set for a quadrant are walked by that quadrant's pixels),
 * tile_order [tiles]: row 1 of gs_render_fwd's tile_order, or NULL (tiles in
 * image order; any other content must be a permutation of the tile ids),
 * dL_dimage [3,H,W].  Out: grad2d [n,12]; with accumulate = 0 the call clears
 * it first, with accumulate = 1 the gradients are added to what it holds (the
 * caller cleared it, or sums several calls): dL/du, dL/dv, dL/dA, dL/dB, dL/dC (conic [[A,B],[B,C]],
 * power = -A dx^2/2 - B dx dy - C dy^2/2, d = pixel - mean), dL/dopacity,
 * dL/dr, dL/dg, dL/db, 0, 0, 0.  Accumulation order is not fixed, so the
 * float32 result varies in the last bits between runs.
 */
int gs_render_bwd(const gs_camera* cam, const gs_settings* set, int32_t n,
                  const uint32_t* tile_ranges, const uint32_t* point_list, const float* splats,
                  const float* final_T, const int32_t* n_contrib, const uint8_t* contrib,
                  const int32_t* tile_order, const float* dL_dimage, float* grad2d, int32_t accumulate,
                  void* stream);

/*
 * gs_preprocess_bwd -- 2D -> 3D gradients ([P3] section 4: through the view
 * transform and perspective Jacobian, dSigma = T^T dSigma2D T, the SH basis,
 * and Sigma = R S S^T R^T; [P4] D.4 quaternion).  Gaussians with
 * tiles_touched == 0 get zero gradients.  Outputs have the parameters' shapes
 * and are overwritten: dmeans [n,3], dlog_scales [n,3], dquats [n,4] (w.r.t.
 * the raw, unnormalised quaternion), dopacity_logits [n], dsh [n,(deg+1)^2,3].
 */
int gs_preprocess_bwd(const gs_camera* cam, const gs_settings* set, int32_t n, int32_t sh_degree,
                      const float* means, const float* log_scales, const float* quats,
                      const float* opacity_logits, const float* sh,
                      const int32_t* tiles_touched, const uint8_t* clamp_mask, const float* grad2d,
                      float* dmeans, float* dlog_scales, float* dquats, float* dopacity_logits,
                      float* dsh, void* stream);

/*
 * gs_preprocess_bwd_colorjac -- gs_preprocess_bwd with the colour's direction
 * gradient read from colorjac (gs_preprocess_colorjac of the same parameters
 * and camera) instead of being rebuilt from the SH coefficients, which it does
 * not read.  The view-direction term of dmeans is
 * sum_c drgb_c colorjac[i, c, :] projected onto the sphere, drgb_c = 0 for a
 * channel clamped at 0 (clamp_mask).  Same outputs, shapes and errors as
 * gs_preprocess_bwd; colorjac NULL is an error.
 */
int gs_preprocess_bwd_colorjac(const gs_camera* cam, const gs_settings* set, int32_t n, int32_t sh_degree,
                               const float* means, const float* log_scales, const float* quats,
                               const float* opacity_logits, const float* colorjac,
                               const int32_t* tiles_touched, const uint8_t* clamp_mask, const float* grad2d,
                               float* dmeans, float* dlog_scales, float* dquats, float* dopacity_logits,
                               float* dsh, void* stream);

/*
 * gs_image_loss -- image reconstruction loss ([P4] E.1).  mode 1: L1,
 * L = sum |pred - target|, dL/dpred = sign(pred - target) with sign(0) = 0;
 * mode 2: L2, L = sum (pred - target)^2, dL/dpred = 2 (pred - target).
 * pred, target, dL_dpred [count] float32.  loss_dev [1 + GS_LOSS_PARTIALS]
 * float64: loss_dev[0] receives L (summed in a fixed order, so the value is
 * deterministic); the other entries are scratch.
 */
#define GS_LOSS_PARTIALS 1024
int gs_image_loss(int32_t mode, int64_t count, const float* pred, const float* target,
                  float* dL_dpred, double* loss_dev, void* stream);

/*
 * gs_densify_accum -- densification statistic ([P4] D.1, E.1 step 2): for
 * each Gaussian with tiles_touched > 0, accum[i] += |(dL/du, dL/dv)| (this
 * view's 2D-mean gradient, pixel units) and count[i] += 1.  accum [n] float32,
 * count [n] int32 are read-modify-written.
 */
int gs_densify_accum(int32_t n, const int32_t* tiles_touched, const float* grad2d,
                     float* accum, int32_t* count, void* stream);

/* One Adam parameter group ([P4] C.2: per-parameter learning rates).  The
   group covers columns [col_begin, col_end) of a [rows, row_len] array; all
   four arrays share that layout.  normalize_rows != 0 renormalises each row
   to unit length after the update ([P4] D.4, quaternions) and requires the
   group to cover whole rows. */
typedef struct gs_adam_group {
    float* param;
    const float* grad;
    float* exp_avg;
    float* exp_avg_sq;
    int64_t rows;
    int32_t row_len;
    int32_t col_begin;
    int32_t col_end;
    int32_t normalize_rows;
    float lr;
} gs_adam_group;

#define GS_ADAM_MAX_GROUPS 16

/*
 * gs_adam_step -- one Adam step (Kingma and Ba): m = b1 m + (1 - b1) g,
 * v = b2 v + (1 - b2) g^2, p -= lr (m / (1 - b1^step)) / (sqrt(v / (1 - b2^step)) + eps),
 * for up to GS_ADAM_MAX_GROUPS groups in one launch.  step >= 1.
 */
int gs_adam_step(int32_t n_groups, const gs_adam_group* groups, float beta1, float beta2,
                 float eps, int32_t step, void* stream);

/* Adam state and hyper-parameters of the fused training-step tail.  Moment
   buffers have the shapes of the parameters they follow, in the order means,
   log_scales, quats, opacity_logits, sh; the quats moments are 16-byte
   aligned like quats.  lr: means, log_scales, quats, opacity_logits, SH band 0
   (the DC coefficients), SH bands >= 1. */
typedef struct gs_adam_state {
    float* exp_avg[5];
    float* exp_avg_sq[5];
    float lr[6];
    float beta1, beta2, eps;
    int32_t step;
} gs_adam_state;

/*
 * gs_preprocess_bwd_adam -- the training-step tail fused into one pass over
 * the Gaussians ([P4] E.1 steps 2-3: backpropagate, accumulate the position
 * gradient statistic, Adam update; C.2 per-parameter learning rates; D.4
 * renormalise the quaternion after the update).  Computes exactly the
 * gradients of gs_preprocess_bwd and, in the same kernel, applies one Adam
 * step (as gs_adam_step) to the parameters IN PLACE, and adds the
 * densification statistic (as gs_densify_accum) when densify_accum and
 * densify_count are both non-NULL.  The gradient outputs are optional: pass
 * all of dmeans, dlog_scales, dquats, dopacity_logits (and optionally dsh) to
 * also receive the gradients, or NULL to skip those writes.  Gaussians with
 * tiles_touched == 0 receive a zero gradient and still take the Adam step.
 */
int gs_preprocess_bwd_adam(const gs_camera* cam, const gs_settings* set, int32_t n, int32_t sh_degree,
                           float* means, float* log_scales, float* quats, float* opacity_logits, float* sh,
                           const int32_t* tiles_touched, const uint8_t* clamp_mask, const float* grad2d,
                           const gs_adam_state* adam, float* densify_accum, int32_t* densify_count,
                           float* dmeans, float* dlog_scales, float* dquats, float* dopacity_logits,
                           float* dsh, void* stream);

/*
 * Densification, pruning and opacity reset ([P4] D.1: Gaussians whose
 * accumulated position gradient is large are densified, a split replacing one
 * Gaussian by two smaller ones; D.2: split along the long axis when Sigma is
 * anisotropic (large eigenvalue ratio), clone to a slightly offset copy when
 * isotropic; D.3: remove Gaussians of low opacity; E.1 steps 4-6: densify
 * and prune every 100 iterations, scale every opacity by 0.3 every 3000).
 * The numbers the pages leave out are the fields below.
 */
typedef struct gs_densify_params {
    float grad_threshold; /* densify when count > 0 and accum / count >= this (mean |dL/d(u,v)|, pixels) */
    float prune_logit;    /* remove when the opacity logit is below this */
    float split_log_gap;  /* split (else clone) when max - min log-scale >= this; Sigma's eigenvalue ratio is exp(2 gap) */
    float split_shrink;   /* the children's log-scales are the parent's minus this (log of the shrink factor) */
    float split_offset;   /* children at mean +/- split_offset * s_max * e (e: the axis of the largest scale s_max) */
    float clone_offset;   /* the copy at mean + clone_offset * s_max * e */
} gs_densify_params;

/* A set of Gaussians: the five parameter groups ([n,3], [n,3], [n,4] 16-byte
   aligned, [n], [n, (deg+1)^2, 3] 16-byte aligned), optionally their Adam
   moments (all ten pointers, in the group order, the quats and sh moments
   16-byte aligned, or all NULL) and the densification statistic
   (densify_accum [n] float32, densify_count [n] int32, both or neither). */
typedef struct gs_gaussian_set {
    float* means;
    float* log_scales;
    float* quats;
    float* opacity_logits;
    float* sh;
    float* exp_avg[5];
    float* exp_avg_sq[5];
    float* densify_accum;
    int32_t* densify_count;
} gs_gaussian_set;

/* Bytes of workspace gs_densify needs for n Gaussians. */
int gs_densify_workspace_size(int32_t n, size_t* bytes);

/*
 * gs_densify -- densify and prune, out of place.  Gaussian i of `in` is
 * replaced, in index order, by consecutive rows of `out`:
 *   removed (opacity logit < prune_logit):             none;
 *   kept (not densified):                              itself;
 *   cloned (densified, max - min log-scale < gap):     itself, then a copy at
 *                                                      mean + clone_offset s_max e;
 *   split (densified, gap reached):                    mean + split_offset s_max e,
 *                                                      then mean - split_offset s_max e,
 *                                                      log-scales minus split_shrink.
 * Rotation, opacity and SH are copied.  e is the column of R(q / |q|) for the
 * largest log-scale (the first on ties).  The decisions compare the float32
 * inputs exactly (accum / count in double).  An original keeps its Adam
 * moments; a copy or a child gets zero moments.  Every output's statistic
 * (when out has one) is zero.  in needs the statistic.  Each side has all ten
 * moments or none; with capacity > 0 the two sides must agree (with capacity
 * 0 nothing is written and out's pointers are not used).
 * Outputs: *n_out_dev = number of output rows (at most 2 n); if it exceeds
 * capacity (rows the out arrays hold), *overflow_dev = 1 and nothing else is
 * written; else *overflow_dev = 0.  action [n] uint8 (optional) receives 0
 * removed, 1 kept, 2 cloned, 3 split.  `in` and `out` must not overlap.
 * workspace: device scratch of gs_densify_workspace_size() bytes, 256-byte
 * aligned, contents on entry irrelevant (may be NULL when n == 0).
 */
int gs_densify(const gs_densify_params* dp, int32_t n, int32_t sh_degree, const gs_gaussian_set* in,
               int64_t capacity, const gs_gaussian_set* out, uint32_t* n_out_dev, uint32_t* overflow_dev,
               uint8_t* action, void* workspace, size_t workspace_bytes, void* stream);

/*
 * gs_opacity_reset -- [P4] E.1 step 6: opacity <- factor * opacity for every
 * Gaussian (factor in (0, 1]; the pages use 0.3), written back in place as a
 * logit.  exp_avg / exp_avg_sq (optional, [n]): the opacity group's Adam
 * moments, set to zero, as for a parameter that starts afresh.
 */
int gs_opacity_reset(int32_t n, float factor, float* opacity_logits, float* exp_avg, float* exp_avg_sq,
                     void* stream);

/*
 * gs_count_pairs -- diagnostic pair counts of a forward pass (device int64
 * counters, overwritten): counts[0] = evaluated pairs (entries walked by the
 * forward up to and including the one that stops a pixel), counts[1] = sum of
 * n_contrib (entries walked by the backward, [P3] section 3: the reverse walk
 * starts at the last contributor), counts[2] = blended pairs.  evaluated_px
 * [H, W] int32 (optional, NULL to skip): each pixel's share of counts[0].
 */
int gs_count_pairs(const gs_camera* cam, const gs_settings* set, int32_t n, const uint32_t* tile_ranges,
                   const uint32_t* point_list, const float* splats, int64_t* counts, int32_t* evaluated_px,
                   void* stream);

/*
 * 16-bit splat records ([P3] section 5: some intermediate values stored as
 * 16-bit floats to save memory traffic; section 7: FP16 on the rendering path,
 * gradient sums in FP32).  The same calls as gs_preprocess / gs_render_fwd /
 * gs_render_bwd / gs_count_pairs with splats16 [n,6] in place of splats
 * [n,12]: a 24-byte record per Gaussian that a blend gathers per list entry,
 * half the 48 bytes of the float32 record.  Words 0-1: u, v (the 2D mean,
 * float32, no residual); words 2-5: binary16 pairs, low half first: (L00, L10),
 * (L11, opacity), (r, g), (b, 0), each the binary16 number nearest to the
 * float32 value gs_preprocess stores (ties to even).  Culled Gaussians have an
 * all-zero record.  splats16 must be 8-byte aligned (GS_EALIGN otherwise).
 * Range: binary16 holds magnitudes up to 65504 and, below 2^-14, only fixed
 * steps of 2^-24.  L00 and L11 stay in the normal range for any Gaussian from
 * the low-pass dilation's width up to about 10^4 pixels; L10, near zero for an
 * axis-aligned one, then has an absolute step of 2^-24.  A colour above 65504
 * (extreme SH coefficients) is stored as infinity.
 *
 * Precision contract: the blends compute in float32 from the record's values,
 * so their results are those of the float32 path for the Gaussians the record
 * represents: conic = L L^T 2 ln 2 from the rounded factor, opacity and colour
 * rounded.  Against the float32 record each alpha moves by a relative amount
 * of order 2^-11 (1 + condition number of the conic) ln(opacity / alpha_min),
 * which can flip skip and stop decisions of pairs at the thresholds.  The 2D
 * gradients are those at the rounded values; gs_preprocess_bwd and
 * gs_preprocess_bwd_colorjac take them as they take the float32 path's.
 * Binning is unchanged: rect, tiles_touched and depth are those of
 * gs_preprocess, bit for bit.
 *
 * gs_preprocess_h16: colorjac is optional here (NULL: not written); given, it
 * is gs_preprocess_colorjac's.
 */
int gs_preprocess_h16(const gs_camera* cam, const gs_settings* set, int32_t n, int32_t sh_degree,
                      const float* means, const float* log_scales, const float* quats,
                      const float* opacity_logits, const float* sh,
                      float* splats16, float* depth, int16_t* rect, int32_t* tiles_touched,
                      uint8_t* clamp_mask, float* colorjac, void* stream);
int gs_render_fwd_h16(const gs_camera* cam, const gs_settings* set, int32_t n,
                      const uint32_t* tile_ranges, const uint32_t* point_list, const float* splats16,
                      float* image, float* final_T, int32_t* n_contrib, uint8_t* contrib,
                      int32_t* tile_order, float* grad2d_clear, void* stream);
int gs_render_bwd_h16(const gs_camera* cam, const gs_settings* set, int32_t n,
                      const uint32_t* tile_ranges, const uint32_t* point_list, const float* splats16,
                      const float* final_T, const int32_t* n_contrib, const uint8_t* contrib,
                      const int32_t* tile_order, const float* dL_dimage, float* grad2d, int32_t accumulate,
                      void* stream);
int gs_count_pairs_h16(const gs_camera* cam, const gs_settings* set, int32_t n, const uint32_t* tile_ranges,
                       const uint32_t* point_list, const float* splats16, int64_t* counts, int32_t* evaluated_px,
                       void* stream);

/*
 * gs_count_nonfinite -- *out (device int64, overwritten) = the number of NaN
 * and infinite values among x[0, count) (float32, any alignment).  A debug
 * check for the inputs and outputs of the calls above ([P3] section 6: NaN
 * comes from invalid math; find the first tensor that holds one).  A NaN input
 * does not make any call fault: a Gaussian with a non-finite mean, scale or
 * rotation is culled by the preprocess, but a non-finite opacity or SH value
 * reaches the image.
 */
int gs_count_nonfinite(const float* x, int64_t count, int64_t* out, void* stream);

/*
 * Batched views ([P4] E.1 steps 1-3: an iteration renders a batch of views,
 * sums their losses, back-propagates and takes one optimizer step).  The
 * *_views calls take an array of `views` cameras (1 <= views <= GS_MAX_VIEWS),
 * all of one image size, and lay per-view outputs out view-major:
 *  - per-Gaussian arrays are [views, n, ...]: entry v n + i of splats, depth,
 *    rect, tiles_touched, clamp_mask, grad2d and of the point list's values
 *    is Gaussian i seen from view v (n = Gaussians, the same set in every
 *    view; rect is in view v's own tile coordinates);
 *  - tiles are numbered view after view: tile v T + t is tile t of view v
 *    (T = tiles of one view), and tile_ranges [views T, 2], tile_order
 *    [2, views T] and the loss partials loss_dev [1 + views T] cover them all;
 *    views T must stay <= 65536 for gs_bin_sort_views;
 *  - images are [views, 3, H, W], final_T and n_contrib [views, H, W].
 * Otherwise each call means what its single-view counterpart means, view by
 * view; with views == 1 it is that counterpart.  gs_preprocess_bwd_views
 * returns the gradients summed over the views (the batch's loss is the sum of
 * the views' losses); gs_preprocess_bwd_adam_views applies one Adam step with
 * those sums, and its densification statistic adds, for every view in which a
 * Gaussian touches a tile, that view's |dL/d(u,v)| and one count.
 * Workspace: gs_bin_workspace_size_views.
 */
int gs_preprocess_views(const gs_camera* cams, int32_t views, const gs_settings* set, int32_t n, int32_t sh_degree,
                        const float* means, const float* log_scales, const float* quats,
                        const float* opacity_logits, const float* sh, float* splats, float* depth, int16_t* rect,
                        int32_t* tiles_touched, uint8_t* clamp_mask, void* stream);
int gs_bin_workspace_size_views(int32_t n, const gs_camera* cams, int32_t views, int64_t key_capacity,
                                size_t* bytes);
int gs_bin_sort_views(const gs_camera* cams, int32_t views, int32_t n, const float* depth, const int16_t* rect,
                      const int32_t* tiles_touched, int64_t key_capacity, uint32_t* point_list,
                      uint32_t* tile_ranges, uint32_t* num_keys_dev, uint32_t* overflow_dev, void* workspace,
                      size_t workspace_bytes, void* stream);
int gs_render_fwd_views(const gs_camera* cams, int32_t views, const gs_settings* set, int32_t n,
                        const uint32_t* tile_ranges, const uint32_t* point_list, const float* splats, float* image,
                        float* final_T, int32_t* n_contrib, uint8_t* contrib, int32_t* tile_order,
                        float* grad2d_clear, void* stream);
int gs_render_fwd_loss_views(const gs_camera* cams, int32_t views, const gs_settings* set, int32_t n,
                             const uint32_t* tile_ranges, const uint32_t* point_list, const float* splats,
                             float* image, float* final_T, int32_t* n_contrib, uint8_t* contrib,
                             int32_t* tile_order, int32_t loss_mode, const float* target, float* dL_dimage,
                             double* loss_dev, float* grad2d_clear, void* stream);
int gs_render_bwd_views(const gs_camera* cams, int32_t views, const gs_settings* set, int32_t n,
                        const uint32_t* tile_ranges, const uint32_t* point_list, const float* splats,
                        const float* final_T, const int32_t* n_contrib, const uint8_t* contrib,
                        const int32_t* tile_order, const float* dL_dimage, float* grad2d, int32_t accumulate,
                        void* stream);
int gs_preprocess_bwd_views(const gs_camera* cams, int32_t views, const gs_settings* set, int32_t n,
                            int32_t sh_degree, const float* means, const float* log_scales, const float* quats,
                            const float* opacity_logits, const float* sh, const int32_t* tiles_touched,
                            const uint8_t* clamp_mask, const float* grad2d, float* dmeans, float* dlog_scales,
                            float* dquats, float* dopacity_logits, float* dsh, void* stream);
int gs_preprocess_bwd_adam_views(const gs_camera* cams, int32_t views, const gs_settings* set, int32_t n,
                                 int32_t sh_degree, float* means, float* log_scales, float* quats,
                                 float* opacity_logits, float* sh, const int32_t* tiles_touched,
                                 const uint8_t* clamp_mask, const float* grad2d, const gs_adam_state* adam,
                                 float* densify_accum, int32_t* densify_count, float* dmeans, float* dlog_scales,
                                 float* dquats, float* dopacity_logits, float* dsh, void* stream);
int gs_count_pairs_views(const gs_camera* cams, int32_t views, const gs_settings* set, int32_t n,
                         const uint32_t* tile_ranges, const uint32_t* point_list, const float* splats,
                         int64_t* counts, int32_t* evaluated_px /* [views, H, W] or NULL */, void* stream);

#ifdef __cplusplus
}
#endif
#endif
