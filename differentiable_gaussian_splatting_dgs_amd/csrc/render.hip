// Forward compositing and reverse-walk backward of the tile rasterizer.
//
// Method sources: chain-rule gradients page (qqiyuan.cn), compositing
// equation I = sum_i alpha_i c_i prod_{j<i} (1 - alpha_j); Gaussian Splatting
// backward CUDA page (lshu.cn), section 2 (alpha = min(0.99, opacity G), the
// recursion C_i = alpha_i c_i + (1 - alpha_i) C_{i+1} and the table of 2D
// gradients), section 3 (per-tile blocks, Gaussians staged in shared memory in
// batches, the reverse walk starting from the stored final transmittance and
// the last contributor, atomic accumulation), section 5 (merging the atomic
// updates of neighbouring pixels).
//
// Layout on CDNA4: one 256-lane workgroup per 16x16 tile, four wave64 each
// owning an 8x8 quadrant.  A batch of up to 256 list entries is staged in LDS
// (tile-relative mean, conic Cholesky factor, opacity, colour).  While staging,
// each entry's alpha >= alpha_min bounding box (slightly enlarged) is tested
// against the four quadrants; each wave then walks only the entries that can
// reach its quadrant, in list order.  Entries it drops have alpha < alpha_min
// at every pixel of the quadrant and would be skipped anyway, so the result is
// that of walking the whole list.
//
// Gaussian evaluation: with e = L^T d, L the scaled Cholesky factor of the
// conic, G = exp2(-|e|^2) = exp(-d^T conic d / 2).  The factor form keeps the
// float32 rounding error of the exponent proportional to sqrt(condition) of the
// 2D covariance instead of its condition number, and the tile-relative mean
// (float32 mean + float32 residual, less the tile origin) keeps the pixel
// offset d accurate at 4K.  Per list entry the staging precomputes the offsets
// of e at the tile origin and -log2(opacity), so a pair costs
//   e1 = L00 x + L10 y + c1,  e2 = L11 y + c2,  opacity G = exp2(-(e1^2 + e2^2 - log2 opacity))
// for the pixel centre (x, y): three FMAs for e and two for the exponent.
#include "gs_internal.h"

namespace gs {
namespace {

struct RenderArgs {
    BlendArgs b;
    uint32_t n;
    const uint32_t* ranges;
    const uint32_t* list;
    const float* splats;
    float* image;
    float* final_T;
    int32_t* n_contrib;
    uint8_t* contrib;   // [K] per list entry: bit q set if a pixel of quadrant q blends it
    const int32_t* sched;  // [tiles] tile of each block (null: image order, XCD-banded)
    int32_t* work;         // forward: [tiles] backward work estimate per tile (optional)
    const float* dL_dimage;
    float* grad2d;
    // forward with a fused image loss (mode 0: none, 1: L1, 2: L2)
    int32_t loss_mode;
    const float* target;  // [3,H,W]
    float* dL_out;        // [3,H,W] dL/dimage
    double* loss_part;    // [tiles] loss of each tile's pixels
    float4* clear;        // [clear4] float4s set to zero by the forward's blocks (optional)
    size_t clear4;
};

// The tile a block works on: sched[block] when a schedule is given, else image
// order banded over the XCDs; -1 for padding blocks or an out-of-range entry.
__device__ __forceinline__ int block_tile(const int32_t* sched, int ntiles, int idx) {
    if (sched) {
        if (idx >= ntiles) return -1;
        const int t = sched[idx];
        return (t >= 0 && t < ntiles) ? t : -1;
    }
    const int t = xcd_tile(idx, ntiles);
    return t < ntiles ? t : -1;
}
__device__ __forceinline__ int block_tile(const int32_t* sched, int ntiles) {
    return block_tile(sched, ntiles, (int)blockIdx.x);
}

// The alpha of one (pixel, Gaussian) pair.  Shared verbatim by the forward,
// the backward and the pair counter so all three take identical decisions.
// g0 = (L00, L10, L11, c1), g1 = (c2, -log2 opacity, r, g) as staged by
// stage_record; (fx, fy) is the pixel centre relative to the tile origin.
struct Pair {
    float e1, e2, sG, alpha;  // e = L^T d; sG = opacity G; alpha = min(alpha_max, sG)
};

__device__ __forceinline__ Pair eval_pair(float fx, float fy, float4 g0, float4 g1, float amax) {
#pragma clang fp contract(off)
    Pair p;
    p.e1 = __builtin_fmaf(g0.x, fx, __builtin_fmaf(g0.y, fy, g0.w));
    p.e2 = __builtin_fmaf(g0.z, fy, g1.x);
    const float q = __builtin_fmaf(p.e1, p.e1, __builtin_fmaf(p.e2, p.e2, g1.y));
    p.sG = __builtin_amdgcn_exp2f(-q);
    p.alpha = __builtin_amdgcn_fmed3f(p.sG, 0.f, amax);  // min(amax, sG) for sG >= 0, one instruction
    return p;
}

// The per-entry record the blends stage in LDS, from a splat record (three
// float4 rows: mean, mean residual; L00, L10, L11, opacity; r, g, b, 0) and the
// tile origin.  Every kernel that evaluates pairs builds it with this function,
// so they all round identically.
struct Staged {
    float4 g0, g1;
    float b;
    float ut, vt;  // the mean relative to the tile origin
};

__device__ __forceinline__ Staged stage_record(float4 r0, float4 r1, float4 r2, float x0, float y0) {
#pragma clang fp contract(off)
    Staged st;
    st.ut = (r0.x - x0) + r0.z;
    st.vt = (r0.y - y0) + r0.w;
    const float l00 = r1.x, l10 = r1.y, l11 = r1.z;
    // e1 = L00 (x - ut) + L10 (y - vt) = L00 x + L10 y + c1; e2 = L11 (y - vt) = L11 y + c2
    const float c1 = -__builtin_fmaf(l00, st.ut, l10 * st.vt);
    const float c2 = -(l11 * st.vt);
    st.g0 = make_float4(l00, l10, l11, c1);
    st.g1 = make_float4(c2, -__log2f(r1.w), r2.x, r2.y);  // opacity 0 gives +inf: G = 0
    st.b = r2.z;
    return st;
}

// The three float4 rows stage_record takes, from splat record g.  H16: a 16-bit
// record (u, v in float32; then L00, L10 | L11, opacity | r, g | b, 0 as binary16
// pairs, low half first), read as three 8-byte words and widened exactly; its
// mean residual is zero.
template <bool H16>
__device__ __forceinline__ void load_record(const float* splats, uint32_t g, float4& r0, float4& r1, float4& r2) {
    if constexpr (H16) {
        const uint2* sp = reinterpret_cast<const uint2*>(splats + (size_t)g * GS_SPLAT16_STRIDE);
        const uint2 w0 = sp[0], w1 = sp[1], w2 = sp[2];
        auto lo = [](uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu)); };
        auto hi = [](uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); };
        r0 = make_float4(__uint_as_float(w0.x), __uint_as_float(w0.y), 0.f, 0.f);
        r1 = make_float4(lo(w1.x), hi(w1.x), lo(w1.y), hi(w1.y));
        r2 = make_float4(lo(w2.x), hi(w2.x), lo(w2.y), 0.f);
    } else {
        const float4* sp = reinterpret_cast<const float4*>(splats + (size_t)g * GS_SPLAT_STRIDE);
        r0 = sp[0];
        r1 = sp[1];
        r2 = sp[2];
    }
}

// Transmittance after blending alpha: T (1 - alpha) as one fused operation.  The
// forward and the pair counter both use it, so they stop at the same entry.
__device__ __forceinline__ float trans_after(float T, float alpha) { return __builtin_fmaf(-alpha, T, T); }

// Stage list entry k of the tile into LDS slot `slot`; returns the quadrant mask.
struct Stage {
    float4* g0;
    float4* g1;
    float* g2;
};

// Minimum over the segment t in [t0, t1] of (a*c + b*t)^2 + (l*t)^2, the exponent
// |L^T d|^2 along an axis-parallel edge of a rectangle (c is the fixed coordinate).
__device__ __forceinline__ float edge_min(float a, float b, float l, float c, float t0, float t1, float slope) {
    const float t = fminf(fmaxf(c * slope, t0), t1);
    const float e1 = __builtin_fmaf(a, c, b * t);
    const float e2 = l * t;
    return __builtin_fmaf(e1, e1, e2 * e2);
}

template <bool H16>
__device__ __forceinline__ uint32_t stage_entry(const RenderArgs& a, uint32_t g, float x0, float y0,
                                                float log2_amin_inv, Stage st, int slot) {
    float4 r0, r1, r2;
    load_record<H16>(a.splats, g, r0, r1, r2);
    const Staged rec = stage_record(r0, r1, r2, x0, y0);
    const float ut = rec.ut, vt = rec.vt;
    st.g0[slot] = rec.g0;
    st.g1[slot] = rec.g1;
    st.g2[slot] = rec.b;
    // A quadrant can see the Gaussian only if min over its pixel centres of
    // q = |L^T d|^2 (d = p - mean) is <= k2 = log2(opacity / alpha_min).  The test
    // is exact for the rectangle of pixel centres; the threshold gets a relative
    // margin of 1/64 plus 1/16 so float32 rounding can only keep extra entries,
    // never drop one that a pixel would blend.
    const float l00 = r1.x, l10 = r1.y, l11 = r1.z;
    const float k2 = fmaxf(log2_amin_inv - rec.g1.y, 0.f);  // log2(opacity / alpha_min)
    const float kq = __builtin_fmaf(k2, 1.f + 1.f / 64.f, 1.f / 16.f);
    // minimiser slopes on vertical and horizontal edges (approximate reciprocals: the test has a margin)
    const float sv = -l00 * l10 * __builtin_amdgcn_rcpf(__builtin_fmaf(l10, l10, l11 * l11));
    const float sh = -l10 * __builtin_amdgcn_rcpf(l00);
    uint32_t m = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float rx0 = (float)((q & 1) * 8) + 0.5f - ut, rx1 = rx0 + 7.f;
        const float ry0 = (float)((q >> 1) * 8) + 0.5f - vt, ry1 = ry0 + 7.f;
        const bool inside = rx0 <= 0.f && rx1 >= 0.f && ry0 <= 0.f && ry1 >= 0.f;
        // vertical edges: dx fixed, dy free in [ry0, ry1]; horizontal: dy fixed, dx free
        float mn = fminf(edge_min(l00, l10, l11, rx0, ry0, ry1, sv), edge_min(l00, l10, l11, rx1, ry0, ry1, sv));
        const float th0 = fminf(fmaxf(ry0 * sh, rx0), rx1), th1 = fminf(fmaxf(ry1 * sh, rx0), rx1);
        const float a0 = __builtin_fmaf(l00, th0, l10 * ry0), b0 = l11 * ry0;
        const float a1 = __builtin_fmaf(l00, th1, l10 * ry1), b1 = l11 * ry1;
        mn = fminf(mn, fminf(__builtin_fmaf(a0, a0, b0 * b0), __builtin_fmaf(a1, a1, b1 * b1)));
        m |= (inside || mn <= kq) ? (1u << q) : 0u;
    }
    return m;
}

// Compact the slots whose mask has this wave's bit, in slot order.
__device__ __forceinline__ int compact(const uint8_t* s_mask, uint16_t* list, int wave, int lane) {
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const bool on = (s_mask[lane + 64 * i] >> wave) & 1u;
        const uint64_t b = __ballot(on);
        if (on) {
            const uint32_t pos = __builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32),
                                                           __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0u));
            list[cnt + pos] = (uint16_t)(lane + 64 * i);
        }
        cnt += __popcll(b);
    }
    __builtin_amdgcn_wave_barrier();
    return cnt;
}

template <bool H16>
__global__ __launch_bounds__(kBlock) void k_render_fwd(RenderArgs a) {
    __shared__ float4 s_g0[kBlock];
    __shared__ float4 s_g1[kBlock];
    __shared__ float s_g2[kBlock];
    __shared__ uint8_t s_mask[kBlock];
    __shared__ uint16_t s_list[4][kBlock];
    __shared__ uint32_t s_fb[kBlock];        // per slot: byte w set if a pixel of wave w blended it

    if (a.clear) {  // every block of the grid, before any may leave: the stores overlap the blending
        const size_t stride = (size_t)gridDim.x * blockDim.x;
        for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < a.clear4; i += stride)
            a.clear[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    const BlendArgs& b = a.b;
    const int ntv = b.tiles_x * b.tiles_y;
    const int tile = block_tile(a.sched, ntv * b.views);
    if (tile < 0) return;
    const int view = tile / ntv, vtile = tile - view * ntv;
    const int tx = vtile % b.tiles_x, ty = vtile / b.tiles_x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lx = (wave & 1) * 8 + (lane & 7), ly = (wave >> 1) * 8 + (lane >> 3);
    const int px = tx * kTile + lx, py = ty * kTile + ly;
    const bool inside = px < b.width && py < b.height;
    const float fx = (float)lx + 0.5f, fy = (float)ly + 0.5f;
    const float x0 = (float)(tx * kTile), y0 = (float)(ty * kTile);
    const float log2_amin_inv = -__log2f(b.alpha_min);
    const uint2 range = reinterpret_cast<const uint2*>(a.ranges)[tile];
    const Stage st{s_g0, s_g1, s_g2};

    float T = 1.f, C0 = 0.f, C1 = 0.f, C2 = 0.f;
    int last = 0;
    bool done = !inside;
    bool wave_done = __ballot(!done) == 0;
    uint32_t kprev = 0xffffffffu;  // list position whose blend flags this thread writes out
    uint32_t work = 0;             // backward work of the entries this thread flags
    uint8_t* const fb = reinterpret_cast<uint8_t*>(s_fb) + wave;  // this wave's flag byte of slot e: fb[4 e]
    // Backward cost model of one flagged entry: a fixed part (staging, the wave
    // reduction and the atomic update) plus a part per flagged quadrant.
    auto flag_out = [&](uint32_t kk) {
        const uint32_t f = s_fb[tid];
        const uint32_t mq = (f & 1u) | ((f >> 7) & 2u) | ((f >> 14) & 4u) | ((f >> 21) & 8u);
        a.contrib[kk] = (uint8_t)mq;
        work += mq ? 3u + 2u * (uint32_t)__popc(mq) : 0u;
    };
    for (uint32_t start = range.x; start < range.y; start += kBlock) {
        const uint32_t k = start + tid;
        uint32_t m = 0;
        if (k < range.y) {
            const uint32_t g = a.list[k];
            if (g < a.n) m = stage_entry<H16>(a, g, x0, y0, log2_amin_inv, st, tid);
        }
        // the previous batch's flags are final (the loop ends with a barrier)
        if (kprev != 0xffffffffu) flag_out(kprev);
        kprev = k < range.y ? k : 0xffffffffu;
        s_mask[tid] = (uint8_t)m;
        s_fb[tid] = 0u;
        __syncthreads();
        const int cnt = wave_done ? 0 : compact(s_mask, s_list[wave], wave, lane);
        const int base = (int)(start - range.x);
        int lslot = -1;  // the batch's last blended slot (walked in slot order): last = base + lslot + 1
        for (int j = 0; j < cnt; j += 2) {
            const bool has2 = j + 1 < cnt;
            const int ea = s_list[wave][j];
            const int eb = has2 ? s_list[wave][j + 1] : ea;
            const float4 ga0 = s_g0[ea], ga1 = s_g1[ea];
            const float4 gb0 = s_g0[eb], gb1 = s_g1[eb];
            const float cba = s_g2[ea], cbb = s_g2[eb];
            const Pair pa = eval_pair(fx, fy, ga0, ga1, b.alpha_max);
            const Pair pb = eval_pair(fx, fy, gb0, gb1, b.alpha_max);
            {
                const bool pass = !done && pa.alpha >= b.alpha_min;
                const float Tn = trans_after(T, pa.alpha);
                const bool stop = pass && Tn < b.T_min;  // ok = pass and not stop (stop implies pass)
                done = done || stop;
                const bool ok = pass != stop;
                const float Tb = ok ? Tn : T;
                const float w = T - Tb;  // the weight alpha T as the transmittance drop; 0 if not blended
                C0 = __builtin_fmaf(w, ga1.z, C0);
                C1 = __builtin_fmaf(w, ga1.w, C1);
                C2 = __builtin_fmaf(w, cba, C2);
                T = Tb;
                lslot = ok ? ea : lslot;
                if (ok) fb[4 * ea] = 1;  // lanes that blend all store the same byte
            }
            {
                const bool pass = has2 && !done && pb.alpha >= b.alpha_min;
                const float Tn = trans_after(T, pb.alpha);
                const bool stop = pass && Tn < b.T_min;  // ok = pass and not stop (stop implies pass)
                done = done || stop;
                const bool ok = pass != stop;
                const float Tb = ok ? Tn : T;
                const float w = T - Tb;  // the weight alpha T as the transmittance drop; 0 if not blended
                C0 = __builtin_fmaf(w, gb1.z, C0);
                C1 = __builtin_fmaf(w, gb1.w, C1);
                C2 = __builtin_fmaf(w, cbb, C2);
                T = Tb;
                lslot = ok ? eb : lslot;
                if (ok) fb[4 * eb] = 1;
            }
            if ((j & 2) && __ballot(!done) == 0) break;  // checked every other pair
        }
        if (lslot >= 0) last = base + lslot + 1;
        wave_done = __ballot(!done) == 0;
        if (__syncthreads_count(done ? 1 : 0) == kBlock) break;
    }
    if (kprev != 0xffffffffu) flag_out(kprev);
    if (a.work) {
        for (int o = 32; o > 0; o >>= 1) work += __shfl_xor(work, o, 64);
        __syncthreads();
        if (lane == 0) s_fb[wave] = work;
        __syncthreads();
        if (tid == 0) a.work[tile] = (int32_t)(s_fb[0] + s_fb[1] + s_fb[2] + s_fb[3]);
    }
    double lsum = 0.0;
    if (inside) {
        const size_t plane = (size_t)b.width * b.height;
        const size_t pix = (size_t)py * b.width + px + (size_t)view * plane;  // final_T, n_contrib: [views, H, W]
        const size_t pix3 = pix + (size_t)view * 2 * plane;                  // planar images: [views, 3, H, W]
        const float out[3] = {C0 + T * b.bg[0], C1 + T * b.bg[1], C2 + T * b.bg[2]};
#pragma unroll
        for (int ch = 0; ch < 3; ++ch) a.image[ch * plane + pix3] = out[ch];
        a.final_T[pix] = T;
        a.n_contrib[pix] = last;
        if (a.loss_mode) {
#pragma unroll
            for (int ch = 0; ch < 3; ++ch) {
                const float r = out[ch] - a.target[ch * plane + pix3];
                if (a.loss_mode == 1) {
                    lsum += (double)fabsf(r);
                    a.dL_out[ch * plane + pix3] = r > 0.f ? 1.f : (r < 0.f ? -1.f : 0.f);
                } else {
                    lsum += (double)r * (double)r;
                    a.dL_out[ch * plane + pix3] = 2.f * r;
                }
            }
        }
    }
    if (a.loss_mode) {  // the tile's loss, summed in a fixed order
        __shared__ double s_loss[4];
        for (int o = 32; o > 0; o >>= 1) lsum += __shfl_xor(lsum, o, 64);
        if (lane == 0) s_loss[wave] = lsum;
        __syncthreads();
        if (tid == 0) a.loss_part[tile] = (s_loss[0] + s_loss[1]) + (s_loss[2] + s_loss[3]);
    }
}

// ---- cross-lane reduction helpers (wave64) ----
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int kQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowRor8 = 0x128;

// a <- [a_lo, b_lo], b <- [a_hi, b_hi] (lo/hi = lanes 0-31 / 32-63)
__device__ __forceinline__ void xchg32(float& a, float& b) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
}
// a <- [a.r0, b.r0, a.r2, b.r2], b <- [a.r1, b.r1, a.r3, b.r3] (rows of 16 lanes)
__device__ __forceinline__ void xchg16(float& a, float& b) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
}

// Sums v[0..7] and v8 over the 64 lanes.  On return, every lane of 8-lane
// group j (lanes 8j..8j+7) holds the total of v[j], and every lane holds the
// total of v8 in v8.
__device__ __forceinline__ float reduce9(float v[8], float& v8, int lane) {
    float s[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        xchg32(v[k], v[k + 4]);
        s[k] = v[k] + v[k + 4];  // lo lanes: value k, hi lanes: value k+4
    }
    xchg16(s[0], s[2]);
    const float t0 = s[0] + s[2];  // rows: v0 v2 v4 v6
    xchg16(s[1], s[3]);
    const float t1 = s[1] + s[3];  // rows: v1 v3 v5 v7
    const bool hi8 = (lane & 8) != 0;
    const float keep = hi8 ? t1 : t0;
    const float send = hi8 ? t0 : t1;
    float u = keep + dpp<kRowRor8>(send);  // group j = lane >> 3 holds v_j over 8 lanes
    u += dpp<kQuadXor1>(u);
    u += dpp<kQuadXor2>(u);
    u += dpp<kRowHalfMirror>(u);
    // v8
    float x = v8, y = v8;
    xchg32(x, y);
    float w = x + y;
    float w2 = w;
    xchg16(w, w2);
    w = w + w2;
    w += dpp<kRowRor8>(w);
    w += dpp<kQuadXor1>(w);
    w += dpp<kQuadXor2>(w);
    w += dpp<kRowHalfMirror>(w);
    v8 = w;
    return u;
}

// Sums two entries' nine values over the 64 lanes at once (one transposing
// tree for 16 of them, a half tree for the two ninth values).  On return lane
// quad q (lanes 4q..4q+3) holds the total of value q & 7 of entry a (q < 8) or
// entry b (q >= 8) in the return value, and lanes 0..31 hold the total of a[8],
// lanes 32..63 that of b[8], in z.
__device__ __forceinline__ float reduce2x9(float a[9], float b[9], float& z, int lane) {
    float s[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        xchg32(a[k], b[k]);
        s[k] = a[k] + b[k];  // lanes 0-31: a_k, lanes 32-63: b_k
    }
    float t[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        xchg16(s[k], s[k + 4]);
        t[k] = s[k] + s[k + 4];  // rows: a_k, a_k+4, b_k, b_k+4
    }
    const bool hi8 = (lane & 8) != 0;
    const float u0 = (hi8 ? t[2] : t[0]) + dpp<kRowRor8>(hi8 ? t[0] : t[2]);  // half-rows: t0 | t2
    const float u1 = (hi8 ? t[3] : t[1]) + dpp<kRowRor8>(hi8 ? t[1] : t[3]);  // half-rows: t1 | t3
    const bool hi4 = (lane & 4) != 0;
    float w = (hi4 ? u1 : u0) + dpp<kRowHalfMirror>(hi4 ? u0 : u1);          // quads: u0 | u1
    w += dpp<kQuadXor1>(w);
    w += dpp<kQuadXor2>(w);
    // ninth values
    float p = a[8], r = b[8];
    xchg32(p, r);
    float y = p + r;  // lanes 0-31: a8, 32-63: b8
    float y2 = y;
    xchg16(y, y2);    // y: rows r0 r0 r2 r2, y2: rows r1 r1 r3 r3
    y += y2;
    y += dpp<kRowRor8>(y);
    y += dpp<kRowHalfMirror>(y);
    y += dpp<kQuadXor1>(y);
    y += dpp<kQuadXor2>(y);
    z = y;
    return w;
}

// ---- backward walk of one entry, specialised on its quadrant mask (QPW = 4) ----
// One staged entry as the walk reads it (s_g0, s_g1, s_g2 of the backward).
struct BwdEntry {
    float4 g0, g1, g2;
};

// Per-lane state of a wave that owns all four quadrants of its tile: pixel q of
// the lane has inverse transmittance U[q] = 1 / T, S[q] = dL/dpixel . C_next,
// dL/dpixel gp*[q], last contributor nc[q]; its centre is (fx[q & 1], fy[q >> 1]).
// Walking back over an entry, U <- (1 - alpha) U is one fused multiply-add,
// where T <- T / (1 - alpha) would take a subtraction and a reciprocal besides
// the product; T itself is then one reciprocal of U.
struct BwdLane4 {
    float U[4], S[4], gp0[4], gp1[4], gp2[4];
    int nc[4];
    float fx[2], fy[2];
};

// One flagged quadrant Q of entry E at list position pos.  e1r and pr are the
// row terms of eval_pair (L10 y + c1 and e2^2 - log2 opacity), dx and dy the
// pixel's offset from the mean, so alpha and the blend decision are those of
// eval_pair bit for bit.  FIRST: the first flagged quadrant of the entry, which
// writes the nine accumulators instead of adding to them.  CL: the entry's
// opacity can exceed alpha_max, so opacity G may be clamped; otherwise
// alpha = opacity G wherever the pair blends, and the clamp test drops out.
template <int Q, bool FIRST, bool CL>
__device__ __forceinline__ void bwd_quad(BwdLane4& L, const BwdEntry& E, int pos, float e1r, float pr, float dx,
                                         float dy, float amin, float amax, float v[9]) {
    const float e1 = __builtin_fmaf(E.g0.x, L.fx[Q & 1], e1r);
    const float sG = __builtin_amdgcn_exp2f(-__builtin_fmaf(e1, e1, pr));
    // 0 <= opacity G <= alpha_max without CL: eval_pair's clamp is the identity there
    const float alpha = CL ? __builtin_amdgcn_fmed3f(sG, 0.f, amax) : sG;
    const bool ok = pos < L.nc[Q] && alpha >= amin;
    const float ae = ok ? alpha : 0.f;
    L.U[Q] = __builtin_fmaf(-ae, L.U[Q], L.U[Q]);  // before the entry; unchanged where ae = 0
    const float T = __builtin_amdgcn_rcpf(L.U[Q]);
    const float w = ae * T;
    const float gc = __builtin_fmaf(L.gp2[Q], E.g2.x, __builtin_fmaf(L.gp1[Q], E.g1.w, L.gp0[Q] * E.g1.z));
    const float dS = gc - L.S[Q];
    const float dalpha = T * dS;
    L.S[Q] = __builtin_fmaf(ae, dS, L.S[Q]);
    float dpow;  // dL/dpower = dL/d(opacity G) opacity G
    if constexpr (CL) {
        const float dsG = (ok && !(sG > amax)) ? dalpha : 0.f;  // clamped: no dependence
        dpow = dsG * sG;
    } else {
        dpow = dalpha * ae;  // ae = opacity G where the pair blends, 0 elsewhere
    }
    const float t = dpow * dx, sy = dpow * dy;
    if constexpr (FIRST) {
        v[0] = t;
        v[1] = sy;
        v[2] = t * dx;
        v[3] = t * dy;
        v[4] = sy * dy;
        v[5] = dpow;
        v[6] = w * L.gp0[Q];
        v[7] = w * L.gp1[Q];
        v[8] = w * L.gp2[Q];
    } else {
        v[0] += t;
        v[1] += sy;
        v[2] = __builtin_fmaf(t, dx, v[2]);
        v[3] = __builtin_fmaf(t, dy, v[3]);
        v[4] = __builtin_fmaf(sy, dy, v[4]);
        v[5] += dpow;
        v[6] = __builtin_fmaf(w, L.gp0[Q], v[6]);
        v[7] = __builtin_fmaf(w, L.gp1[Q], v[7]);
        v[8] = __builtin_fmaf(w, L.gp2[Q], v[8]);
    }
}

// The quadrants of mask M (a compile-time constant): the row terms are computed
// once per row and the column terms once per column that a flagged quadrant uses.
template <int M, bool CL>
__device__ __forceinline__ void bwd_mask(BwdLane4& L, const BwdEntry& E, int pos, float amin, float amax,
                                         float v[9]) {
    float e1r[2] = {0.f, 0.f}, pr[2] = {0.f, 0.f}, dy[2] = {0.f, 0.f}, dx[2] = {0.f, 0.f};
#pragma unroll
    for (int r = 0; r < 2; ++r)
        if ((M >> (2 * r)) & 3) {
            e1r[r] = __builtin_fmaf(E.g0.y, L.fy[r], E.g0.w);
            const float e2 = __builtin_fmaf(E.g0.z, L.fy[r], E.g1.x);
            pr[r] = __builtin_fmaf(e2, e2, E.g1.y);
            dy[r] = L.fy[r] - E.g2.z;
        }
#pragma unroll
    for (int c = 0; c < 2; ++c)
        if ((M >> c) & 5) dx[c] = L.fx[c] - E.g2.y;
    if constexpr ((M & 1) != 0) bwd_quad<0, true, CL>(L, E, pos, e1r[0], pr[0], dx[0], dy[0], amin, amax, v);
    if constexpr ((M & 2) != 0) bwd_quad<1, (M & 1) == 0, CL>(L, E, pos, e1r[0], pr[0], dx[1], dy[0], amin, amax, v);
    if constexpr ((M & 4) != 0) bwd_quad<2, (M & 3) == 0, CL>(L, E, pos, e1r[1], pr[1], dx[0], dy[1], amin, amax, v);
    if constexpr ((M & 8) != 0) bwd_quad<3, (M & 7) == 0, CL>(L, E, pos, e1r[1], pr[1], dx[1], dy[1], amin, amax, v);
}

// Entry E with quadrant mask m (wave-uniform) into v; no quadrant (m = 0) leaves
// the additive identity -0 in every accumulator.
template <bool CL>
__device__ __forceinline__ void bwd_walk4(BwdLane4& L, const BwdEntry& E, uint32_t m, int pos, float amin,
                                          float amax, float v[9]) {
    switch (m) {
        case 1: bwd_mask<1, CL>(L, E, pos, amin, amax, v); break;
        case 2: bwd_mask<2, CL>(L, E, pos, amin, amax, v); break;
        case 3: bwd_mask<3, CL>(L, E, pos, amin, amax, v); break;
        case 4: bwd_mask<4, CL>(L, E, pos, amin, amax, v); break;
        case 5: bwd_mask<5, CL>(L, E, pos, amin, amax, v); break;
        case 6: bwd_mask<6, CL>(L, E, pos, amin, amax, v); break;
        case 7: bwd_mask<7, CL>(L, E, pos, amin, amax, v); break;
        case 8: bwd_mask<8, CL>(L, E, pos, amin, amax, v); break;
        case 9: bwd_mask<9, CL>(L, E, pos, amin, amax, v); break;
        case 10: bwd_mask<10, CL>(L, E, pos, amin, amax, v); break;
        case 11: bwd_mask<11, CL>(L, E, pos, amin, amax, v); break;
        case 12: bwd_mask<12, CL>(L, E, pos, amin, amax, v); break;
        case 13: bwd_mask<13, CL>(L, E, pos, amin, amax, v); break;
        case 14: bwd_mask<14, CL>(L, E, pos, amin, amax, v); break;
        case 15: bwd_mask<15, CL>(L, E, pos, amin, amax, v); break;
        default:
#pragma unroll
            for (int i = 0; i < 9; ++i) v[i] = -0.f;
            break;
    }
}

// The same result as reduce2x9 with the tree's row levels done through LDS:
// after the half-wave exchange each lane holds, for value k < 8, a sum of two
// partials of entry a (lanes 0-31) or b (lanes 32-63); it stores them to
// red[k][lane] (a wave-private block of 8 rows of kRedRow floats).  Lane l then
// sums 8 of the 32 partials of value l / 4 (row (l / 4) % 8, half l / 32): the
// 4-float groups l % 4 and l % 4 + 4, so that a quad's first reads cover 16
// contiguous floats and its second reads the next 16; the quad finishes the sum.
// Plain adds and two quad DPP steps replace the row-exchange, select and
// row-DPP instructions of the tree.  A row stride of 80 floats puts the 16-float
// spans of four neighbouring rows in different banks.
constexpr int kRedRow = 80;  // floats per row of the reduction's LDS block (64 partials + 16)
__device__ __forceinline__ float reduce2x9_lds(float a[9], float b[9], float& z, int lane, float* red) {
    float s[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        xchg32(a[k], b[k]);
        s[k] = a[k] + b[k];  // lanes 0-31: a_k, lanes 32-63: b_k
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) red[k * kRedRow + lane] = s[k];
    const float4* p = reinterpret_cast<const float4*>(red + ((lane >> 2) & 7) * kRedRow + (lane >> 5) * 32) + (lane & 3);
    const float4 x0 = p[0], x1 = p[4];
    float w = ((x0.x + x0.y) + (x0.z + x0.w)) + ((x1.x + x1.y) + (x1.z + x1.w));
    w += dpp<kQuadXor1>(w);
    w += dpp<kQuadXor2>(w);
    // ninth values
    float p9 = a[8], r9 = b[8];
    xchg32(p9, r9);
    float y = p9 + r9;  // lanes 0-31: a8, 32-63: b8
    float y2 = y;
    xchg16(y, y2);
    y += y2;
    y += dpp<kRowRor8>(y);
    y += dpp<kRowHalfMirror>(y);
    y += dpp<kQuadXor1>(y);
    y += dpp<kQuadXor2>(y);
    z = y;
    return w;
}

// Backward: one wave64 per tile (QPW = 4), each lane owning one pixel of each of
// the four 8x8 quadrants (pixel q of lane l sits at ((q & 1) 8 + l % 8,
// (q >> 1) 8 + l / 8)); or, for images with few tiles, two waves per tile
// (QPW = 2), wave h owning quadrants 2h and 2h + 1, so that the chip has twice
// the waves to hide latency with, at the price of a second reduction and atomic
// update for entries both halves blend.
// Entries are walked in reverse list order in batches of 64, only those the
// forward blended somewhere in the tile; for an entry, only its flagged
// quadrants run the per-pixel recursion, each adding its partials into the same
// nine per-lane accumulators, so the cross-lane reduction and the atomic update
// happen once per entry rather than once per quadrant.
//
// The accumulators hold moments: S_t = sum dpow dx, S_s = sum dpow dy,
// sum dpow dx^2, sum dpow dx dy, sum dpow dy^2 (dpow = dL/dpower, d = pixel -
// mean), sum dpow and the colour sums.  After the reduction they become
// gradients with the entry's conic (A, B, C): dL/dmean2D = (A S_t + B S_s,
// B S_t + C S_s) since dpower/dmean = conic d, dL/d(A, B, C) = (-1/2, -1, -1/2)
// times the second moments, and dL/dopacity = sum dpow / opacity (dpower is
// dL/d(opacity G) times opacity G).
constexpr int kBwdBatch = 64;
constexpr uint32_t kBwdClamp = 1u << 12;  // list flag: the entry's opacity can exceed alpha_max
// Below this many tiles the backward runs two waves per tile: with one wave per
// tile some of the 1024 SIMDs (256 CUs) would have none.  Above it the second
// reduction and atomic update per entry cost more than the extra waves give.
constexpr int kBwdSplitBelow = 1024;

template <int QPW, bool H16>
__global__ __launch_bounds__(64) void k_render_bwd(RenderArgs a) {
    static_assert(QPW == 4 || QPW == 2, "four or two quadrants per wave");
    constexpr int kSplit = 4 / QPW;
    __shared__ float4 s_g0[kBwdBatch];   // L00, L10, L11, c1 (stage_record)
    __shared__ float4 s_g1[kBwdBatch];   // c2, -log2 opacity, r, g
    __shared__ float4 s_g2[kBwdBatch];   // b, tile-relative mean (u, v), the Gaussian's index (bits)
    __shared__ float4 s_tab[kBwdBatch];  // for after the reduction: conic A, C, 1 / opacity, conic B
    __shared__ uint16_t s_list[kBwdBatch];  // slot | quadrant mask << 8 | kBwdClamp, in walk order
    __shared__ float4 s_red[8 * kRedRow / 4];  // the reduction's exchange block (reduce2x9_lds)

    const BlendArgs& b = a.b;
    const int ntv = b.tiles_x * b.tiles_y;
    const int tile = block_tile(a.sched, ntv * b.views, (int)blockIdx.x / kSplit);
    if (tile < 0) return;
    const int qbase = ((int)blockIdx.x % kSplit) * QPW;  // first quadrant of this wave
    const int view = tile / ntv, vtile = tile - view * ntv;
    const int tx = vtile % b.tiles_x, ty = vtile / b.tiles_x;
    const int lane = threadIdx.x;
    const float x0 = (float)(tx * kTile), y0 = (float)(ty * kTile);
    const uint2 range = reinterpret_cast<const uint2*>(a.ranges)[tile];
    constexpr float k2ln2 = 1.3862943611198906f;  // conic = 2 ln2 L L^T
    // an entry whose opacity is at most this has opacity G < alpha_max at every
    // pixel: G <= 1, and the float exponent and logarithm are within a few ulp
    const float op_noclamp = b.alpha_max * (1.f - 1.f / 65536.f);

    // Per pixel: U = 1 / T, S = dL/dpixel . C_next (the colour accumulated behind the
    // current entry, starting at the background), dL/dpixel and the centre.
    // dL/dalpha = T (dL/dpixel . c - S) and S <- S + alpha (dL/dpixel . c - S)
    // is C_next <- alpha c + (1 - alpha) C_next dotted with dL/dpixel.
    // Pixel q of the lane (q < QPW) is in quadrant qbase + q at (fx[q & 1], fy[q >> 1]).
    BwdLane4 L;
    L.fy[1] = 0.f;
    int ncmax = 0;
    const size_t plane = (size_t)b.width * b.height;
#pragma unroll
    for (int q = 0; q < QPW; ++q) {
        const int qg = qbase + q;
        const int lx = (qg & 1) * 8 + (lane & 7), ly = (qg >> 1) * 8 + (lane >> 3);
        const int px = tx * kTile + lx, py = ty * kTile + ly;
        L.fx[q & 1] = (float)lx + 0.5f;
        L.fy[q >> 1] = (float)ly + 0.5f;
        L.U[q] = 1.f; L.nc[q] = 0; L.gp0[q] = L.gp1[q] = L.gp2[q] = 0.f;
        if (px < b.width && py < b.height) {
            const size_t pix = (size_t)py * b.width + px + (size_t)view * plane;
            const size_t pix3 = pix + (size_t)view * 2 * plane;
            // final T >= T_min > 0 after a blended entry; a zero (T_min = 0) is kept
            // finite so that (1 - alpha) U stays a number and T stays 0
            L.U[q] = fminf(1.f / a.final_T[pix], 3.4028235e38f);
            L.nc[q] = a.n_contrib[pix];
            L.gp0[q] = a.dL_dimage[pix3];
            L.gp1[q] = a.dL_dimage[plane + pix3];
            L.gp2[q] = a.dL_dimage[2 * plane + pix3];
        }
        L.S[q] = __builtin_fmaf(L.gp2[q], b.bg[2], __builtin_fmaf(L.gp1[q], b.bg[1], L.gp0[q] * b.bg[0]));
        ncmax = max(ncmax, L.nc[q]);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) ncmax = max(ncmax, __shfl_xor(ncmax, o, 64));

    // Per-lane roles after a two-entry reduction: quad q (lanes 4q..4q+3) holds
    // value q & 7 of entry q >> 3; its first lane writes it, and lanes 1 and 33
    // write the two ninth values.  The value is turned into its gradient with
    // the entry's s_tab row: slot psel gives the factor for values 0 (conic A),
    // 1 (conic C) and 5 (1 / opacity); the others take the constant scl.
    const int vi = (lane >> 2) & 7;
    const bool entb = lane >= 32;
    const bool ninth = (lane & 31) == 1;
    const bool writer = (lane & 3) == 0 || ninth;
    const int widx = ninth ? 8 : vi;
    const float scl = vi == 2 ? -0.5f : vi == 3 ? -1.f : vi == 4 ? -0.5f : 1.f;
    const bool pvar = vi == 0 || vi == 1 || vi == 5;
    const int psel = vi == 0 ? 0 : vi == 1 ? 1 : vi == 5 ? 2 : 3;
    const int bmask = entb ? -1 : 0;

    // One entry's flagged quadrants, accumulated into v[0..8] (any QPW, any opacity).
    auto walk = [&](int e, uint32_t mm, int pos, float v[9]) {
        const float4 G0 = s_g0[e], G1 = s_g1[e], G2 = s_g2[e];
#pragma unroll
        for (int q = 0; q < QPW; ++q) {
            if (mm & (1u << q)) {
                const float fx = L.fx[q & 1], fy = L.fy[q >> 1];
                const Pair p = eval_pair(fx, fy, G0, G1, b.alpha_max);
                const bool ok = pos < L.nc[q] && p.alpha >= b.alpha_min;
                const float ae = ok ? p.alpha : 0.f;
                // transmittance before the entry; a pair that is not blended leaves U as it was
                L.U[q] = __builtin_fmaf(-ae, L.U[q], L.U[q]);
                const float T = __builtin_amdgcn_rcpf(L.U[q]);
                const float w = ae * T;
                const float gc = __builtin_fmaf(L.gp2[q], G2.x, __builtin_fmaf(L.gp1[q], G1.w, L.gp0[q] * G1.z));
                const float dS = gc - L.S[q];
                const float dalpha = T * dS;
                L.S[q] = __builtin_fmaf(ae, dS, L.S[q]);
                const float dsG = (ok && !(p.sG > b.alpha_max)) ? dalpha : 0.f;  // clamped: no dependence
                // dL/dpower = dsG opacity G (G = exp(power)); dL/dopacity = dsG G = dL/dpower / opacity
                const float dpow = dsG * p.sG;
                const float dx = fx - G2.y, dy = fy - G2.z;  // d = pixel - mean
                const float t = dpow * dx, sy = dpow * dy;
                v[0] += t;
                v[1] += sy;
                v[2] = __builtin_fmaf(t, dx, v[2]);
                v[3] = __builtin_fmaf(t, dy, v[3]);
                v[4] = __builtin_fmaf(sy, dy, v[4]);
                v[5] += dpow;
                v[6] = __builtin_fmaf(w, L.gp0[q], v[6]);
                v[7] = __builtin_fmaf(w, L.gp1[q], v[7]);
                v[8] = __builtin_fmaf(w, L.gp2[q], v[8]);
            }
        }
    };
    // The same for a wave that owns the whole tile, through the code specialised on
    // the entry's mask and on whether its opacity can be clamped.
    auto walk4 = [&](int e, uint32_t l, int pos, float v[9]) {
        const BwdEntry E{s_g0[e], s_g1[e], s_g2[e]};
        const uint32_t mm = (l >> 8) & 15u;
        if (l & kBwdClamp)
            bwd_walk4<true>(L, E, mm, pos, b.alpha_min, b.alpha_max, v);
        else
            bwd_walk4<false>(L, E, mm, pos, b.alpha_min, b.alpha_max, v);
    };

    const uint32_t end = range.x + (uint32_t)ncmax;
    for (int32_t hi = (int32_t)end; hi > (int32_t)range.x; hi -= kBwdBatch) {
        const int32_t k = hi - 1 - lane;  // slot `lane` holds list position k (descending)
        uint32_t m = 0;
        bool cl = false;
        if (k >= (int32_t)range.x) {
            const uint32_t g = a.list[k];
            if (g < a.n) {
                m = ((uint32_t)a.contrib[k] >> qbase) & ((1u << QPW) - 1u);  // this wave's quadrants
                if (m) {
                    float4 r0, r1, r2;
                    load_record<H16>(a.splats, g, r0, r1, r2);
                    const Staged rec = stage_record(r0, r1, r2, x0, y0);
                    s_g0[lane] = rec.g0;
                    s_g1[lane] = rec.g1;
                    s_g2[lane] = make_float4(rec.b, rec.ut, rec.vt, __uint_as_float(g));
                    const float l00 = r1.x, l10 = r1.y, l11 = r1.z;
                    s_tab[lane] = make_float4(k2ln2 * (l00 * l00), k2ln2 * __builtin_fmaf(l10, l10, l11 * l11),
                                                  __builtin_amdgcn_rcpf(r1.w), k2ln2 * (l00 * l10));
                    cl = !(r1.w <= op_noclamp);
                }
            }
        }
        const uint64_t bal = __ballot(m != 0);
        if (m) {
            const uint32_t at = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
            s_list[at] = (uint16_t)(lane | (m << 8) | (cl ? kBwdClamp : 0u));
        }
        const int cnt = __popcll(bal);
        __syncthreads();
        const int top = hi - 1 - (int)range.x;  // list position of slot 0
        // entries in pairs: the walk order is kept (a before b), the reduction and
        // the atomic update are shared
        for (int j = 0; j < cnt; j += 2) {
            const bool two = j + 1 < cnt;
            const uint32_t la = __builtin_amdgcn_readfirstlane((uint32_t)s_list[j]);
            const uint32_t lb = two ? __builtin_amdgcn_readfirstlane((uint32_t)s_list[j + 1]) : 0u;
            const int ea = (int)(la & 63u), eb = (int)(lb & 63u);
            float va[9], vb[9];
            if constexpr (QPW == 4) {
                walk4(ea, la, top - ea, va);
                walk4(eb, lb, top - eb, vb);  // no quadrant when there is no second entry
            } else {
                // -0 is the additive identity (x + -0 == x for every x)
#pragma unroll
                for (int i = 0; i < 9; ++i) { va[i] = -0.f; vb[i] = -0.f; }
                walk(ea, la >> 8, top - ea, va);
                walk(eb, lb >> 8, top - eb, vb);
            }
            float z;
            const float wv = reduce2x9_lds(va, vb, z, lane, reinterpret_cast<float*>(s_red));
            // quads 0 / 8: A S_t + B S_s; quads 1 / 9: C S_s + B S_t; 2-4: scale * moment;
            // 5: sum dpow / opacity (dL/dopacity = dsG G); 6, 7 and the ninth: as summed
            // the entry's s_tab row: ea's in lanes 0-31, eb's in lanes 32-63 (bmask selects
            // the difference of the two rows' offsets; the offsets are scalar)
            const int row = 4 * ea + (bmask & (4 * (eb - ea)));
            const float* tab = reinterpret_cast<const float*>(s_tab) + row;
            const float pv = tab[psel], bv = tab[3];
            const uint32_t gid = __float_as_uint(reinterpret_cast<const float*>(s_g2)[row + 3]);
            const float x = dpp<kRowHalfMirror>(wv);  // the other first moment of the same entry
            const float P = pvar ? pv : scl;
            const float Bx = vi < 2 ? bv * x : 0.f;
            const float out = ninth ? z : __builtin_fmaf(P, wv, Bx);
            if (writer && (two || !entb))
                unsafeAtomicAdd(a.grad2d + (size_t)gid * GS_GRAD2D_STRIDE + widx, out);
        }
        __syncthreads();
    }
}

// Tile schedules: a one-block bucket sort of per-tile work estimates into tile
// ids, heaviest first, so that the longest tiles start first and a kernel does
// not end on a few late, long tiles.  The work of tile t is the length of its
// list (ranges given) or work[t]; order may alias work.  Buckets are
// quarter-octaves of the work; order inside a bucket is arbitrary.
constexpr int kOrderThreads = 1024;
constexpr int kOrderBuckets = 128;
constexpr int kOrderMaxTiles = 65536;
constexpr int kOrderRunsFrom = 16384;  // tiles from which the forward's schedule counts per run (k_tile_order<true>)

__device__ __forceinline__ uint32_t work_bucket(uint32_t w) {
    if (w == 0) return 0;
    const uint32_t oct = 31u - __clz(w);  // floor(log2 w)
    const uint32_t sub = oct >= 2 ? (w >> (oct - 2)) & 3u : (w << (2 - oct)) & 3u;
    return min(1u + 4u * oct + sub, (uint32_t)kOrderBuckets - 1u);
}

// Sum of part[0..n) in a fixed order by one block (1024 threads) into *out.
__device__ void block_sum_f64(const double* part, int n, double* out) {
    __shared__ double s_w[kOrderThreads / 64];
    double acc = 0.0;
    for (int i = threadIdx.x; i < n; i += blockDim.x) acc += part[i];
    for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
    if ((threadIdx.x & 63) == 0) s_w[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        double t = 0.0;
        for (int w = 0; w < (int)(blockDim.x >> 6); ++w) t += s_w[w];
        *out = t;
    }
}

// One block: the total of per-tile loss partials (when the forward has no schedule to sort).
__global__ __launch_bounds__(kOrderThreads) void k_sum_tiles(const double* part, int n, double* out) {
    block_sum_f64(part, n, out);
}

// Runs of equal bucket over the valid lanes of a wave (valid lanes are a prefix).
// Returns the first lane of this lane's run; the run's length goes to len (set
// on every valid lane).
__device__ __forceinline__ int bucket_run(uint32_t bk, bool ok, uint32_t& len) {
    const int lane = threadIdx.x & 63;
    const uint32_t prev = (uint32_t)__shfl_up((int)bk, 1, 64);
    const uint64_t heads = __ballot(ok && (lane == 0 || prev != bk));
    const uint32_t nok = (uint32_t)__popcll(__ballot(ok));
    const uint64_t upto = lane == 63 ? ~0ull : ((2ull << lane) - 1ull);  // lanes 0..lane
    const uint64_t hb = heads & upto;
    const int head = hb ? 63 - __builtin_clzll(hb) : 0;
    const uint64_t above = head == 63 ? 0ull : heads >> (head + 1);
    len = (above ? (uint32_t)head + 1u + (uint32_t)__builtin_ctzll(above) : nok) - (uint32_t)head;
    return head;
}

// RUNS: bucket counts and slots are taken per run of lanes with one bucket (one
// LDS atomic per run) instead of per lane.  Neighbouring tiles' list lengths
// mostly share a bucket, so per-lane atomics collide on one address; finding the
// runs costs about 1.4 us of VALU at 8160 tiles, and it pays from a few tens of
// thousands of tiles (the 4K forward schedule: 48 -> 28 us).
template <bool RUNS>
__global__ __launch_bounds__(kOrderThreads) void k_tile_order(const uint32_t* ranges, const int32_t* work,
                                                              int32_t* order, int ntiles, const double* loss_part,
                                                              double* loss_out) {
    __shared__ uint8_t s_b[kOrderMaxTiles];
    __shared__ uint32_t s_cnt[kOrderBuckets];
    __shared__ uint32_t s_w1;
    const int tid = threadIdx.x, lane = tid & 63;
    if (loss_part) block_sum_f64(loss_part, ntiles, loss_out);  // the one-block pass also totals the loss
    if (tid < kOrderBuckets) s_cnt[tid] = 0;
    __syncthreads();
    for (int t0 = 0; t0 < ntiles; t0 += kOrderThreads) {  // the same trip count for every lane
        const int t = t0 + tid;
        const bool ok = t < ntiles;  // valid lanes are a prefix of the wave
        uint32_t bk = kOrderBuckets;
        if (ok) {
            const uint32_t w = ranges ? ranges[2 * t + 1] - ranges[2 * t] : (uint32_t)max(work[t], 0);
            bk = work_bucket(w);
            s_b[t] = (uint8_t)bk;
        }
        if constexpr (RUNS) {
            uint32_t len;
            const int head = bucket_run(bk, ok, len);
            if (ok && head == lane) atomicAdd(&s_cnt[bk], len);
        } else {
            if (ok) atomicAdd(&s_cnt[bk], 1u);
        }
    }
    __syncthreads();
    // exclusive offsets, heaviest bucket first: a scan over the reversed buckets by two waves
    uint32_t x = 0, c = 0;
    if (tid < kOrderBuckets) {
        c = s_cnt[kOrderBuckets - 1 - tid];
        x = c;
        for (int o = 1; o < 64; o <<= 1) {
            const uint32_t y = __shfl_up(x, o, 64);
            if (lane >= o) x += y;
        }
        if (tid == 63) s_w1 = x;
    }
    __syncthreads();
    if (tid < kOrderBuckets) s_cnt[kOrderBuckets - 1 - tid] = x - c + (tid >= 64 ? s_w1 : 0u);
    __syncthreads();
    if constexpr (RUNS) {
        // the same runs: the first lane of a run claims the run's slots, the others follow it
        for (int t0 = 0; t0 < ntiles; t0 += kOrderThreads) {
            const int t = t0 + tid;
            const bool ok = t < ntiles;
            const uint32_t bk = ok ? (uint32_t)s_b[t] : (uint32_t)kOrderBuckets;
            uint32_t len;
            const int head = bucket_run(bk, ok, len);
            uint32_t at = 0;
            if (ok && head == lane) at = atomicAdd(&s_cnt[bk], len);
            at = (uint32_t)__shfl((int)at, head, 64) + (uint32_t)(lane - head);
            if (ok) order[at] = t;
        }
    } else {
        for (int t = tid; t < ntiles; t += kOrderThreads) order[atomicAdd(&s_cnt[s_b[t]], 1u)] = t;
    }
}

// p[i] = i mod period for i < 2 period.
__global__ void k_iota(int32_t* p, int period) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < 2 * period) p[i] = i < period ? i : i - period;
}

__global__ void k_zero_f32(float* p, size_t count) {
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (; i < count; i += stride) p[i] = 0.f;
}

// Pair counts: one thread per pixel, walking the whole tile list.  ev_px
// (optional, [views, H, W]) receives each pixel's evaluated entries.
template <bool H16>
__global__ __launch_bounds__(256) void k_count_pairs(RenderArgs a, unsigned long long* counts, int32_t* ev_px) {
    __shared__ unsigned long long s_c[3];
    const BlendArgs& b = a.b;
    if (threadIdx.x < 3) s_c[threadIdx.x] = 0;
    __syncthreads();
    const int px = blockIdx.x * 16 + (threadIdx.x & 15);
    const int py = blockIdx.y * 16 + (threadIdx.x >> 4);
    unsigned long long ev = 0, nc = 0, nb = 0;
    if (px < b.width && py < b.height) {
        const int tile = (blockIdx.z * b.tiles_y + blockIdx.y) * b.tiles_x + blockIdx.x;
        const uint2 range = reinterpret_cast<const uint2*>(a.ranges)[tile];
        const float fx = (float)(px % kTile) + 0.5f, fy = (float)(py % kTile) + 0.5f;
        const float x0 = (float)(blockIdx.x * kTile), y0 = (float)(blockIdx.y * kTile);
        float T = 1.f;
        for (uint32_t k = range.x; k < range.y; ++k) {
            const uint32_t g = a.list[k];
            if (g >= a.n) continue;
            float4 r0, r1, r2;
            load_record<H16>(a.splats, g, r0, r1, r2);
            const Staged rec = stage_record(r0, r1, r2, x0, y0);
            const Pair p = eval_pair(fx, fy, rec.g0, rec.g1, b.alpha_max);
            ++ev;
            if (p.alpha < b.alpha_min) continue;
            const float Tn = trans_after(T, p.alpha);
            if (Tn < b.T_min) break;
            T = Tn;
            ++nb;
            nc = k - range.x + 1;
        }
        if (ev_px) ev_px[((size_t)blockIdx.z * b.height + py) * b.width + px] = (int32_t)ev;
    }
    atomicAdd(&s_c[0], ev);
    atomicAdd(&s_c[1], nc);
    atomicAdd(&s_c[2], nb);
    __syncthreads();
    if (threadIdx.x < 3) atomicAdd(&counts[threadIdx.x], s_c[threadIdx.x]);
}

__global__ void k_zero_i64(unsigned long long* p, int n) {
    if ((int)threadIdx.x < n) p[threadIdx.x] = 0ull;
}

inline int render_common_checks(const gs_camera* cams, int32_t views, const gs_settings* set,
                                const uint32_t* ranges, const float* splats, bool h16 = false) {
    if (!views_ok(cams, views) || !set || !ranges) return GS_EINVAL;
    if (!(h16 ? aligned8(splats) : aligned16(splats)) || !aligned16(ranges)) return GS_EALIGN;
    return GS_OK;
}

inline int render_grid(const gs_camera* cam, int32_t views) {
    const int nt = views * tiles_x(cam) * tiles_y(cam);
    return 8 * ((nt + 7) / 8);
}

inline BlendArgs blend_views(const gs_camera* cam, int32_t views, const gs_settings* set) {
    BlendArgs b = blend_args(cam, set);
    b.views = views;
    return b;
}

}  // namespace
}  // namespace gs

using namespace gs;

namespace gs {
namespace {

// Forward blend, its tile schedules and, when a.loss_mode != 0, the fused loss.
int render_fwd_impl(const gs_camera* cam, RenderArgs& a, int32_t* tile_order, double* loss_dev, hipStream_t s,
                    bool h16) {
    const auto fwd = h16 ? k_render_fwd<true> : k_render_fwd<false>;
    const int views = a.b.views;
    const int ntiles = views * tiles_x(cam) * tiles_y(cam);
    if (tile_order && ntiles <= kOrderMaxTiles) {
        // row 0: the forward's own schedule (list lengths); row 1: the backward's (flag counts)
        int32_t* fwd_order = tile_order;
        int32_t* bwd_order = tile_order + ntiles;
        if (ntiles >= kOrderRunsFrom)
            hipLaunchKernelGGL(k_tile_order<true>, dim3(1), dim3(kOrderThreads), 0, s, a.ranges, nullptr, fwd_order,
                               ntiles, nullptr, nullptr);
        else
            hipLaunchKernelGGL(k_tile_order<false>, dim3(1), dim3(kOrderThreads), 0, s, a.ranges, nullptr, fwd_order,
                               ntiles, nullptr, nullptr);
        a.sched = fwd_order;
        a.work = bwd_order;
        hipLaunchKernelGGL(fwd, dim3(render_grid(cam, views)), dim3(kBlock), 0, s, a);
        hipLaunchKernelGGL(k_tile_order<false>, dim3(1), dim3(kOrderThreads), 0, s, nullptr, bwd_order, bwd_order, ntiles,
                           a.loss_part, loss_dev);
    } else {
        hipLaunchKernelGGL(fwd, dim3(render_grid(cam, views)), dim3(kBlock), 0, s, a);
        if (tile_order)  // too many tiles for the one-block sort: image order
            hipLaunchKernelGGL(k_iota, dim3((2 * ntiles + 255) / 256), dim3(256), 0, s, tile_order, ntiles);
        if (a.loss_mode)
            hipLaunchKernelGGL(k_sum_tiles, dim3(1), dim3(kOrderThreads), 0, s, a.loss_part, ntiles, loss_dev);
    }
    return launch_status();
}

// n: Gaussians per view; the splat records are [views, n, 12] and list entries index them.
int fwd_args(const gs_camera* cam, int32_t views, const gs_settings* set, int32_t n, const uint32_t* tile_ranges,
             const uint32_t* point_list, const float* splats, float* image, float* final_T, int32_t* n_contrib,
             uint8_t* contrib, RenderArgs& a, bool h16) {
    int rc = render_common_checks(cam, views, set, tile_ranges, splats, h16);
    if (rc) return rc;
    if (n < 0 || !image || !final_T || !n_contrib) return GS_EINVAL;
    if ((int64_t)views * n > (int64_t)INT32_MAX) return GS_ECAPACITY;
    if (n > 0 && (!point_list || !splats || !contrib)) return GS_EINVAL;
    a = RenderArgs{};
    a.b = blend_views(cam, views, set);
    a.n = (uint32_t)(views * n);
    a.ranges = tile_ranges; a.list = point_list; a.splats = splats;
    a.image = image; a.final_T = final_T; a.n_contrib = n_contrib; a.contrib = contrib;
    return GS_OK;
}

}  // namespace
}  // namespace gs

namespace gs {
namespace {

int render_fwd_loss_impl(const gs_camera* cams, int32_t views, const gs_settings* set, int32_t n,
                         const uint32_t* tile_ranges, const uint32_t* point_list, const float* splats, float* image,
                         float* final_T, int32_t* n_contrib, uint8_t* contrib, int32_t* tile_order,
                         int32_t loss_mode, const float* target, float* dL_dimage, double* loss_dev,
                         float* grad2d_clear, void* stream, bool h16 = false) {
    RenderArgs a;
    const int rc = fwd_args(cams, views, set, n, tile_ranges, point_list, splats, image, final_T, n_contrib, contrib,
                            a, h16);
    if (rc) return rc;
    if (grad2d_clear && !aligned16(grad2d_clear)) return GS_EALIGN;
    if (grad2d_clear && n > 0) {
        a.clear = reinterpret_cast<float4*>(grad2d_clear);
        a.clear4 = (size_t)a.n * GS_GRAD2D_STRIDE / 4;
    }
    if (loss_mode == 0) return render_fwd_impl(cams, a, tile_order, nullptr, as_stream(stream), h16);
    if (loss_mode != 1 && loss_mode != 2) return GS_EINVAL;
    if (!target || !dL_dimage || !loss_dev) return GS_EINVAL;
    a.loss_mode = loss_mode;
    a.target = target;
    a.dL_out = dL_dimage;
    a.loss_part = loss_dev + 1;
    return render_fwd_impl(cams, a, tile_order, loss_dev, as_stream(stream), h16);
}

int render_bwd_impl(const gs_camera* cams, int32_t views, const gs_settings* set, int32_t n,
                    const uint32_t* tile_ranges, const uint32_t* point_list, const float* splats,
                    const float* final_T, const int32_t* n_contrib, const uint8_t* contrib, const int32_t* tile_order,
                    const float* dL_dimage, float* grad2d, int32_t accumulate, void* stream, bool h16 = false) {
    int rc = render_common_checks(cams, views, set, tile_ranges, splats, h16);
    if (rc) return rc;
    if (n < 0 || !final_T || !n_contrib || !dL_dimage) return GS_EINVAL;
    if ((int64_t)views * n > (int64_t)INT32_MAX) return GS_ECAPACITY;
    if (n > 0 && (!point_list || !splats || !grad2d || !contrib)) return GS_EINVAL;
    if (n > 0 && !aligned16(grad2d)) return GS_EALIGN;
    hipStream_t s = as_stream(stream);
    if (accumulate != 0 && accumulate != 1) return GS_EINVAL;
    const int32_t ntot = views * n;
    if (n > 0 && !accumulate) {
        const size_t cnt = (size_t)ntot * GS_GRAD2D_STRIDE;
        hipLaunchKernelGGL(k_zero_f32, dim3((unsigned)std::min<size_t>((cnt + 255) / 256, 4096)), dim3(256), 0, s,
                           grad2d, cnt);
    }
    RenderArgs a{};
    a.b = blend_views(cams, views, set);
    a.n = (uint32_t)ntot;
    a.ranges = tile_ranges; a.list = point_list; a.splats = splats;
    a.final_T = const_cast<float*>(final_T); a.n_contrib = const_cast<int32_t*>(n_contrib);
    a.contrib = const_cast<uint8_t*>(contrib);
    a.dL_dimage = dL_dimage; a.grad2d = grad2d;
    a.sched = tile_order;
    const auto bwd2 = h16 ? k_render_bwd<2, true> : k_render_bwd<2, false>;
    const auto bwd4 = h16 ? k_render_bwd<4, true> : k_render_bwd<4, false>;
    if (views * tiles_x(cams) * tiles_y(cams) < kBwdSplitBelow)
        hipLaunchKernelGGL(bwd2, dim3(2 * render_grid(cams, views)), dim3(64), 0, s, a);
    else
        hipLaunchKernelGGL(bwd4, dim3(render_grid(cams, views)), dim3(64), 0, s, a);
    return launch_status();
}

int count_pairs_impl(const gs_camera* cams, int32_t views, const gs_settings* set, int32_t n,
                     const uint32_t* tile_ranges, const uint32_t* point_list, const float* splats, int64_t* counts,
                     int32_t* evaluated_px, void* stream, bool h16 = false) {
    int rc = render_common_checks(cams, views, set, tile_ranges, splats, h16);
    if (rc) return rc;
    if (!counts || n < 0) return GS_EINVAL;
    if ((int64_t)views * n > (int64_t)INT32_MAX) return GS_ECAPACITY;
    hipStream_t s = as_stream(stream);
    RenderArgs a{};
    a.b = blend_views(cams, views, set);
    a.n = (uint32_t)(views * n);
    a.ranges = tile_ranges; a.list = point_list; a.splats = splats;
    auto* c = reinterpret_cast<unsigned long long*>(counts);
    hipLaunchKernelGGL(k_zero_i64, dim3(1), dim3(64), 0, s, c, 3);
    const auto count = h16 ? k_count_pairs<true> : k_count_pairs<false>;
    hipLaunchKernelGGL(count, dim3(tiles_x(cams), tiles_y(cams), views), dim3(256), 0, s, a, c, evaluated_px);
    return launch_status();
}

}  // namespace
}  // namespace gs

extern "C" int gs_render_fwd(const gs_camera* cam, const gs_settings* set, int32_t n, const uint32_t* tile_ranges,
                             const uint32_t* point_list, const float* splats, float* image, float* final_T,
                             int32_t* n_contrib, uint8_t* contrib, int32_t* tile_order, float* grad2d_clear,
                             void* stream) {
    return render_fwd_loss_impl(cam, 1, set, n, tile_ranges, point_list, splats, image, final_T, n_contrib, contrib,
                                tile_order, 0, nullptr, nullptr, nullptr, grad2d_clear, stream);
}

extern "C" int gs_render_fwd_views(const gs_camera* cams, int32_t views, const gs_settings* set, int32_t n,
                                   const uint32_t* tile_ranges, const uint32_t* point_list, const float* splats,
                                   float* image, float* final_T, int32_t* n_contrib, uint8_t* contrib,
                                   int32_t* tile_order, float* grad2d_clear, void* stream) {
    return render_fwd_loss_impl(cams, views, set, n, tile_ranges, point_list, splats, image, final_T, n_contrib,
                                contrib, tile_order, 0, nullptr, nullptr, nullptr, grad2d_clear, stream);
}

extern "C" int gs_render_fwd_loss(const gs_camera* cam, const gs_settings* set, int32_t n,
                                  const uint32_t* tile_ranges, const uint32_t* point_list, const float* splats,
                                  float* image, float* final_T, int32_t* n_contrib, uint8_t* contrib,
                                  int32_t* tile_order, int32_t loss_mode, const float* target, float* dL_dimage,
                                  double* loss_dev, float* grad2d_clear, void* stream) {
    if (loss_mode == 0) return GS_EINVAL;
    return render_fwd_loss_impl(cam, 1, set, n, tile_ranges, point_list, splats, image, final_T, n_contrib, contrib,
                                tile_order, loss_mode, target, dL_dimage, loss_dev, grad2d_clear, stream);
}

extern "C" int gs_render_fwd_loss_views(const gs_camera* cams, int32_t views, const gs_settings* set, int32_t n,
                                        const uint32_t* tile_ranges, const uint32_t* point_list, const float* splats,
                                        float* image, float* final_T, int32_t* n_contrib, uint8_t* contrib,
                                        int32_t* tile_order, int32_t loss_mode, const float* target,
                                        float* dL_dimage, double* loss_dev, float* grad2d_clear, void* stream) {
    if (loss_mode == 0) return GS_EINVAL;
    return render_fwd_loss_impl(cams, views, set, n, tile_ranges, point_list, splats, image, final_T, n_contrib,
                                contrib, tile_order, loss_mode, target, dL_dimage, loss_dev, grad2d_clear, stream);
}

extern "C" int gs_render_bwd(const gs_camera* cam, const gs_settings* set, int32_t n, const uint32_t* tile_ranges,
                             const uint32_t* point_list, const float* splats, const float* final_T,
                             const int32_t* n_contrib, const uint8_t* contrib, const int32_t* tile_order,
                             const float* dL_dimage, float* grad2d, int32_t accumulate, void* stream) {
    return render_bwd_impl(cam, 1, set, n, tile_ranges, point_list, splats, final_T, n_contrib, contrib, tile_order,
                           dL_dimage, grad2d, accumulate, stream);
}

extern "C" int gs_render_bwd_views(const gs_camera* cams, int32_t views, const gs_settings* set, int32_t n,
                                   const uint32_t* tile_ranges, const uint32_t* point_list, const float* splats,
                                   const float* final_T, const int32_t* n_contrib, const uint8_t* contrib,
                                   const int32_t* tile_order, const float* dL_dimage, float* grad2d,
                                   int32_t accumulate, void* stream) {
    return render_bwd_impl(cams, views, set, n, tile_ranges, point_list, splats, final_T, n_contrib, contrib,
                           tile_order, dL_dimage, grad2d, accumulate, stream);
}

extern "C" int gs_count_pairs(const gs_camera* cam, const gs_settings* set, int32_t n, const uint32_t* tile_ranges,
                              const uint32_t* point_list, const float* splats, int64_t* counts,
                              int32_t* evaluated_px, void* stream) {
    return count_pairs_impl(cam, 1, set, n, tile_ranges, point_list, splats, counts, evaluated_px, stream);
}

extern "C" int gs_count_pairs_views(const gs_camera* cams, int32_t views, const gs_settings* set, int32_t n,
                                    const uint32_t* tile_ranges, const uint32_t* point_list, const float* splats,
                                    int64_t* counts, int32_t* evaluated_px, void* stream) {
    return count_pairs_impl(cams, views, set, n, tile_ranges, point_list, splats, counts, evaluated_px, stream);
}

// 16-bit splat records (gs_preprocess_h16): the single-view forward, backward and pair count.
extern "C" int gs_render_fwd_h16(const gs_camera* cam, const gs_settings* set, int32_t n,
                                 const uint32_t* tile_ranges, const uint32_t* point_list, const float* splats16,
                                 float* image, float* final_T, int32_t* n_contrib, uint8_t* contrib,
                                 int32_t* tile_order, float* grad2d_clear, void* stream) {
    return render_fwd_loss_impl(cam, 1, set, n, tile_ranges, point_list, splats16, image, final_T, n_contrib,
                                contrib, tile_order, 0, nullptr, nullptr, nullptr, grad2d_clear, stream, true);
}

extern "C" int gs_render_bwd_h16(const gs_camera* cam, const gs_settings* set, int32_t n,
                                 const uint32_t* tile_ranges, const uint32_t* point_list, const float* splats16,
                                 const float* final_T, const int32_t* n_contrib, const uint8_t* contrib,
                                 const int32_t* tile_order, const float* dL_dimage, float* grad2d, int32_t accumulate,
                                 void* stream) {
    return render_bwd_impl(cam, 1, set, n, tile_ranges, point_list, splats16, final_T, n_contrib, contrib,
                           tile_order, dL_dimage, grad2d, accumulate, stream, true);
}

extern "C" int gs_count_pairs_h16(const gs_camera* cam, const gs_settings* set, int32_t n,
                                  const uint32_t* tile_ranges, const uint32_t* point_list, const float* splats16,
                                  int64_t* counts, int32_t* evaluated_px, void* stream) {
    return count_pairs_impl(cam, 1, set, n, tile_ranges, point_list, splats16, counts, evaluated_px, stream, true);
}
