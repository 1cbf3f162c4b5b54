// Tile binning and per-tile depth order.
//
// Method sources: 3DGS training notes (huajishe), section E.3 (cull against
// tiles with an AABB, sort by depth inside each tile, tiles independent);
// Gaussian Splatting backward CUDA page (lshu.cn), sections 1 and 5 (the
// sorted list and the tile ranges are reused by the backward).
//
// The required order is (tile, float32 depth, Gaussian index).  Instead of
// one radix sort over 64-bit (tile | depth) keys for every (tile, Gaussian)
// pair, the work is split so the wide key is sorted over N items and only
// the narrow tile id over K items:
//   1. depth keys: key = float32 depth bits (visible) or 0xffffffff, val = index;
//      digit histograms for the 4 depth passes.
//   2. LSD onesweep radix sort of (depth key, index) over N, 4 x 8-bit passes.
//      Stable, so equal depths stay in index order.
//   3. emit: an exclusive scan of tiles_touched in depth order gives every
//      Gaussian its first output slot; then fixed-size blocks of output slots
//      each write (tile id, Gaussian) for their slots (balanced however many
//      tiles a Gaussian covers) and count the tile digits, in total and per
//      block.
//   4. LSD radix sort of (tile id, Gaussian) over K, 1-2 x 8-bit passes, by
//      reduce-then-scan: per-block digit counts (from step 3 for the first
//      digit, a counting pass for the second), a scan of them into output
//      positions, and a scatter pass that ranks and writes each partition on
//      its own.  Stable, so each tile keeps the depth order of step 2.
//   5. tile ranges from the sorted tile ids.
// The onesweep pass (one kernel per digit: stable wave-level ranking by
// ballot matching, then decoupled look-back across partitions for the digit
// offsets) follows Adinets and Merrill, "Onesweep" (2022), with partitions
// claimed from an atomic ticket so look-back only waits on running blocks.
// Over N it fits in one wave of blocks; over K (several waves of blocks) the
// look-back's serial chain costs more than the tile sort's counting and
// scanning, and without waits between partitions the scatter can hand each
// XCD a contiguous range of partitions.
#include <algorithm>
#include <atomic>
#include <mutex>

#include "gs_internal.h"

namespace gs {
namespace {

// Sort passes: THREADS x IPT items per partition.  More waves with fewer items
// each shorten every wave's serial ranking and write-out chains, which set the
// time of a pass when there is about one block per CU.
constexpr int kDepthThreads = 512;
constexpr int kDepthIPT = 8;                        // depth sort over N: 4096 items per partition
constexpr int kTileThreads = 512;
constexpr int kTileIPT = 8;                         // tile sort over K: 4096 items per partition
constexpr int kDepthPart = kDepthThreads * kDepthIPT;
constexpr int kTilePart = kTileThreads * kTileIPT;
constexpr int kKeyIPT = 8;                          // depth-key pass: Gaussians per thread
constexpr int kRangeIPT = 8;                        // tile-range pass: keys per thread
constexpr int kStripes = 32;                        // histogram copies that blocks add into
constexpr int kHistBins = 6 * 256;                  // 4 depth digits + 2 tile digits
constexpr int kLookWindow = 8;                      // predecessors read at once per digit
constexpr uint32_t kLookGroup = 16;                 // partitions per look-back group
constexpr int kRadix = 256;
constexpr uint32_t kXcds = 8;                       // accelerator complex dies: blocks are dealt to them round-robin
constexpr uint32_t kFlagAgg = 1u << 30;
constexpr uint32_t kFlagInc = 2u << 30;
constexpr uint32_t kValMask = (1u << 30) - 1u;
constexpr uint32_t kWaitLimit = 1u << 22;        // default look-back waits before a pass gives up

constexpr int kEmitThreads = 256;
constexpr int kEmitIPT = 4;
constexpr int kEmitPart = kEmitThreads * kEmitIPT;  // 1024 Gaussians per scan partition
constexpr int kSlotsPT = 8;
constexpr int kSlots = kEmitThreads * kSlotsPT;     // 2048 output slots per expand block
static_assert(kTilePart % kSlots == 0, "expand blocks tile the tile sort's partitions");

__device__ inline uint32_t ld_acquire(const uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void st_release(uint32_t* p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline uint64_t lanemask_lt() {
    const uint32_t lane = threadIdx.x & 63;
    return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// Bit b of d sign-extended: 0 or ~0.  Written as one VALU instruction the
// compiler cannot see through, so the ballot on it below compares it with 0
// instead of shifting d again.
template <int B>
__device__ inline uint32_t bit_mask(uint32_t d) {
    uint32_t s;
    asm volatile("v_bfe_i32 %0, %1, %2, 1" : "=v"(s) : "v"(d), "n"(B));
    return s;
}

// Lanes whose 8-bit digit equals this lane's (among lanes with valid set),
// when the digits of all items can differ only in the bits of vm (uniform).
// A lane matches when, for every bit of vm, its bit equals ours: the XOR of
// that bit's ballot with our bit replicated is 0 in its position.
__device__ inline uint64_t match_digits(uint32_t d, bool valid, uint32_t vm) {
    uint32_t xlo = 0, xhi = 0;
#define GS_MATCH_BIT(B)                                   \
    if (vm & (1u << B)) {                                 \
        const uint32_t sb = bit_mask<B>(d);               \
        const uint64_t bb = __ballot(sb != 0u);           \
        xlo |= (uint32_t)bb ^ sb;                         \
        xhi |= (uint32_t)(bb >> 32) ^ sb;                 \
    }
    GS_MATCH_BIT(0) GS_MATCH_BIT(1) GS_MATCH_BIT(2) GS_MATCH_BIT(3)
    GS_MATCH_BIT(4) GS_MATCH_BIT(5) GS_MATCH_BIT(6) GS_MATCH_BIT(7)
#undef GS_MATCH_BIT
    return __ballot(valid) & ~(((uint64_t)xhi << 32) | xlo);
}

// Sum over the kStripes histogram copies of bin b.
__device__ inline uint32_t stripe_sum(const uint32_t* stripes, int b) {
    uint32_t acc = 0;
#pragma unroll
    for (int p = 0; p < kStripes; ++p) acc += stripes[(size_t)p * kHistBins + b];
    return acc;
}

// Partitions are claimed in groups so that no single counter sees more than
// 1/kTicketGroups of the blocks' atomics (same-address atomics from many
// blocks serialise): block b takes the next ticket t of group b % kTicketGroups
// and works on partition t * kTicketGroups + b % kTicketGroups.  Claims stay in
// dispatch order within each group, which keeps the look-back deadlock-free.
constexpr int kTicketGroups = 64;
constexpr int kTicketStride = 16;  // one 64-byte line per counter

// Workspace layout (all offsets 256-byte aligned).
struct Layout {
    size_t tickets;     // uint32 [4 depth passes][kTicketGroups][kTicketStride] partition tickets
    size_t err;         // uint32 [1] look-back spin-limit flag
    size_t dstatus;     // uint32 [4][dparts][256]
    size_t dgstatus;    // uint32 [4][dgroups][256]
    size_t etotal;      // uint32 [eparts] entries per emit partition, then their exclusive offsets
    size_t vmw;         // uint32 [2 passes][2] OR of the tile digits present, OR of their complements
    size_t zero_end;    // everything above is zeroed per call
    size_t stripes;     // uint32 [kStripes][kHistBins] striped digit counts (zeroed)
    size_t dkeys0, dvals0, dkeys1, dvals1;  // uint32 [n] each
    size_t tcnt0, tpre0;                    // uint32 [xblocks][256] tile digit-0 counts per expand block, [256][xblocks] prefixes
    size_t tcnt1, tpre1;                    // uint32 [tparts][256] tile digit-1 counts per partition, [256][tparts] prefixes
    size_t goff;                            // uint32 [n] first output slot, depth order
    size_t bstart;                          // uint32 [xblocks + 1] first Gaussian (depth order) of each expand block
    size_t tkeys0, tkeys1, tvals0;          // uint16 [cap] tile ids (two), uint32 [cap] values
    size_t total;
    uint32_t dparts, eparts, tparts, xblocks;
};

inline size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }

inline Layout make_layout(int32_t n, int64_t cap) {
    Layout L;
    L.dparts = (uint32_t)((n + kDepthPart - 1) / kDepthPart);
    L.eparts = (uint32_t)((n + kEmitPart - 1) / kEmitPart);
    L.tparts = (uint32_t)((cap + kTilePart - 1) / kTilePart);
    L.xblocks = (uint32_t)((cap + kSlots - 1) / kSlots);
    size_t o = 0;
    L.tickets = o; o = up256(o + (size_t)4 * kTicketGroups * kTicketStride * 4);
    L.err = o; o = up256(o + 4);
    L.dstatus = o; o = up256(o + (size_t)4 * L.dparts * kRadix * 4);
    L.dgstatus = o; o = up256(o + (size_t)4 * ((L.dparts + kLookGroup - 1) / kLookGroup) * kRadix * 4);
    L.etotal = o; o = up256(o + (size_t)L.eparts * 4);
    L.vmw = o; o = up256(o + 4 * 4);
    L.stripes = o; o = up256(o + (size_t)kStripes * kHistBins * 4);
    L.zero_end = o;
    L.dkeys0 = o; o = up256(o + (size_t)n * 4);
    L.dvals0 = o; o = up256(o + (size_t)n * 4);
    L.dkeys1 = o; o = up256(o + (size_t)n * 4);
    L.dvals1 = o; o = up256(o + (size_t)n * 4);
    L.tcnt0 = o; o = up256(o + (size_t)kRadix * L.xblocks * 4);
    L.tpre0 = o; o = up256(o + (size_t)kRadix * L.xblocks * 4);
    L.tcnt1 = o; o = up256(o + (size_t)kRadix * L.tparts * 4);
    L.tpre1 = o; o = up256(o + (size_t)kRadix * L.tparts * 4);
    L.goff = o; o = up256(o + (size_t)n * 4);
    L.bstart = o; o = up256(o + ((size_t)L.xblocks + 1) * 4);
    L.tkeys0 = o; o = up256(o + (size_t)cap * 2);
    L.tkeys1 = o; o = up256(o + (size_t)cap * 2);
    L.tvals0 = o; o = up256(o + (size_t)cap * 4);
    L.total = o;
    return L;
}

// Clears up to four buffers in one launch.
struct ClearArgs {
    uint32_t* p[4];
    size_t count[4];
};

__global__ void k_clear(ClearArgs c) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
#pragma unroll
    for (int b = 0; b < 4; ++b)
        for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < c.count[b]; i += stride) c.p[b][i] = 0u;
}

// 1. depth keys + counts of the 4 depth digits.  Each thread loads its
// kKeyIPT Gaussians before using any (one memory latency per thread, not one
// per item).  Blocks add their counts into one of kStripes histogram copies, so
// no address sees more than a few dozen global atomics; the sort passes sum the
// copies.
__global__ __launch_bounds__(256) void k_depth_keys(int32_t n, const float* depth, const int32_t* tt,
                                                    uint32_t* keys, uint32_t* vals, uint32_t* stripes) {
    __shared__ uint32_t sh[4 * kRadix];
    for (int i = threadIdx.x; i < 4 * kRadix; i += blockDim.x) sh[i] = 0;
    const int64_t base = (int64_t)blockIdx.x * 256 * kKeyIPT + threadIdx.x;
    float dep[kKeyIPT];
    int32_t cnt[kKeyIPT];
#pragma unroll
    for (int u = 0; u < kKeyIPT; ++u) {
        const int64_t i = base + u * 256;
        dep[u] = i < n ? depth[i] : 0.f;
        cnt[u] = i < n ? tt[i] : 0;
    }
    uint32_t k[kKeyIPT];
#pragma unroll
    for (int u = 0; u < kKeyIPT; ++u) {
        const int64_t i = base + u * 256;
        k[u] = cnt[u] > 0 ? __float_as_uint(dep[u]) : 0xffffffffu;
        if (i < n) {
            keys[i] = k[u];
            vals[i] = (uint32_t)i;
        }
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kKeyIPT; ++u) {
        if (base + u * 256 < n) {
#pragma unroll
            for (int d = 0; d < 4; ++d) atomicAdd(&sh[d * kRadix + ((k[u] >> (8 * d)) & 255u)], 1u);
        }
    }
    __syncthreads();
    uint32_t* out = stripes + (size_t)(blockIdx.x % kStripes) * kHistBins;
    for (int b = threadIdx.x; b < 4 * kRadix; b += blockDim.x)
        if (sh[b]) atomicAdd(&out[b], sh[b]);
}

struct PassArgs {
    const void* keys_in;   // KeyT [count]: uint32 depth keys or uint16 tile ids
    const uint32_t* vals_in;
    void* keys_out;        // KeyT, may be null: keys not needed after this pass
    uint32_t* vals_out;
    const uint32_t* count_dev;  // items = min(*count_dev, cap) when non-null, else count_host
    uint32_t count_host;
    uint32_t cap;
    const uint32_t* stripes;  // striped digit counts; this pass's bins start at hist_bin
    int hist_bin;
    uint32_t* status;      // [parts][256], zeroed
    uint32_t* gstatus;     // [groups of kLookGroup parts][256], zeroed
    uint32_t* ticket;      // [kTicketGroups][kTicketStride], zeroed
    uint32_t* err;         // bit p set when a partition of pass p gave up waiting for its predecessors
    uint32_t err_bit;      // this pass's bit
    uint32_t err_before;   // bits of the earlier passes: if any is set the pass does nothing
    const uint32_t* skip;  // optional: the pass does nothing when *skip != 0 (list overflow)
    uint32_t wait_limit;   // waits per look-back before giving up
    int shift;
    // passes with precomputed prefixes (k_pass_scatter)
    const uint32_t* prefix;   // [256][stride]: items of digit d before column c (k_digit_scan)
    uint32_t stride;
    uint32_t cols_per_part;   // columns per partition: partition p starts at column p cols_per_part
    const uint32_t* vmw;      // [2]: OR of the digits present, OR of their complements (k_digit_scan)
};

// Inclusive sum over the 64 lanes of a wave.
__device__ inline uint32_t wave_incl_sum(uint32_t v) {
    const int lane = threadIdx.x & 63;
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(v, o, 64);
        if (lane >= o) v += y;
    }
    return v;
}

// 2/4. one onesweep pass over 8 bits of a 32-bit key, THREADS threads with IPT
// items each.  Threads 0..255 (waves 0-3) also own one digit each for the
// histogram scan and the look-back.
template <int THREADS, int IPT, typename KeyT>
__global__ __launch_bounds__(THREADS) void k_onesweep(PassArgs p) {
    constexpr int kWaves = THREADS / 64;
    constexpr int kSortPart = THREADS * IPT;
    static_assert(THREADS >= kRadix && THREADS % 64 == 0, "one thread per digit");
    __shared__ uint32_t s_off[kRadix];          // global exclusive digit offsets
    __shared__ uint32_t s_wave[kWaves][kRadix]; // per-wave digit counts -> prefixes
    __shared__ uint32_t s_base[kRadix];         // global offset of this partition's first item of digit d
    __shared__ uint32_t s_blk[kRadix];          // block-local exclusive digit offsets
    __shared__ KeyT s_keys[kSortPart];          // partition in digit order
    __shared__ uint32_t s_vals[kSortPart];
    __shared__ uint32_t s_wsum[2][4];
    __shared__ uint32_t s_dig[2][4];            // OR and AND of the digits present, per digit wave
    __shared__ uint32_t s_part;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const bool digit_thread = tid < kRadix;
    // An earlier pass failed, or the list overflowed: the sort is void.  Both words
    // were written by earlier kernels, so every block of the grid reads the same.
    if ((*p.err & p.err_before) != 0u || (p.skip && *p.skip != 0u)) return;

    if (tid == 0) {
        const uint32_t grp = blockIdx.x % kTicketGroups;
        s_part = atomicAdd(p.ticket + grp * kTicketStride, 1u) * kTicketGroups + grp;
    }
    for (int i = tid; i < kWaves * kRadix; i += THREADS) (&s_wave[0][0])[i] = 0;
    // exclusive scan of the digit histogram (256 entries, one per digit thread)
    uint32_t h = 0, hx = 0;
    if (digit_thread) {
        h = stripe_sum(p.stripes, p.hist_bin + tid);
        hx = wave_incl_sum(h);
        if (lane == 63) s_wsum[0][wave] = hx;
        // the digits present in this pass (tid is the digit)
        uint32_t dor = h ? (uint32_t)tid : 0u, dand = h ? (uint32_t)tid : 255u;
        for (int o = 32; o >= 1; o >>= 1) {
            dor |= __shfl_xor(dor, o, 64);
            dand &= __shfl_xor(dand, o, 64);
        }
        if (lane == 0) { s_dig[0][wave] = dor; s_dig[1][wave] = dand; }
    }
    __syncthreads();
    // bits in which the pass's digits differ: only these need matching
    uint32_t vm;
    {
        uint32_t dor = 0, dand = 255u;
#pragma unroll
        for (int w = 0; w < kRadix / 64; ++w) { dor |= s_dig[0][w]; dand &= s_dig[1][w]; }
        vm = (dor ^ dand) & 255u;
    }
    if (digit_thread) {
        uint32_t add = 0;
        for (int w = 0; w < wave; ++w) add += s_wsum[0][w];
        s_off[tid] = hx - h + add;
    }
    const uint32_t part = s_part;
    uint32_t count = p.count_dev ? *p.count_dev : p.count_host;
    if (count > p.cap) count = p.cap;
    const uint32_t nparts = (count + kSortPart - 1) / kSortPart;
    if (part >= nparts) return;  // uniform over the block

    // load: wave w owns [part*P + w*64*IPT, +64*IPT), item i of lane l at + i*64 + l
    const uint32_t base = part * kSortPart + wave * 64 * IPT;
    uint32_t key[IPT], val[IPT], rank[IPT];
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
        const uint32_t idx = base + i * 64 + lane;
        key[i] = idx < count ? (uint32_t) static_cast<const KeyT*>(p.keys_in)[idx] : 0u;
        val[i] = idx < count ? p.vals_in[idx] : 0u;
    }
    const uint64_t lt = lanemask_lt();
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
        const bool valid = (base + i * 64 + lane) < count;
        const uint32_t d = (key[i] >> p.shift) & 255u;
        const uint64_t m = match_digits(d, valid, vm);
        const uint32_t below = (uint32_t)__popcll(m & lt);
        const uint32_t prev = valid ? s_wave[wave][d] : 0u;
        rank[i] = prev + below;
        __builtin_amdgcn_wave_barrier();
        if (valid && below == 0) s_wave[wave][d] = prev + (uint32_t)__popcll(m);
        __builtin_amdgcn_wave_barrier();
    }
    __syncthreads();
    // per digit: prefix over waves, then a block-local exclusive scan of the digit totals
    uint32_t total = 0, tx = 0;
    if (digit_thread) {
        uint32_t run = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const uint32_t c = s_wave[w][tid];
            s_wave[w][tid] = run;
            run += c;
        }
        total = run;
        tx = wave_incl_sum(total);
        if (lane == 63) s_wsum[1][wave] = tx;
    }
    __syncthreads();
    if (digit_thread) {
        const int d = tid;
        uint32_t add = 0;
        for (int w = 0; w < wave; ++w) add += s_wsum[1][w];
        const uint32_t blk = tx - total + add;
        s_blk[d] = blk;

        // Two-level look-back.  Every partition publishes its own digit count.  The
        // last partition of each group of kLookGroup adds up its group, publishes the
        // group's count and looks back over the earlier groups for the group's
        // inclusive prefix.  Every other partition needs only the counts of its
        // group's earlier partitions and the previous group's inclusive prefix.  All
        // waits are on lower partitions, claimed earlier, and bounded.
        const uint32_t grp = part / kLookGroup, first = grp * kLookGroup;
        const uint32_t last = min(first + kLookGroup, nparts) - 1u;
        st_release(p.status + (size_t)part * kRadix + d, kFlagAgg | total);
        uint32_t spins = 0;
        bool failed = false;
        auto give_up = [&]() {  // the pass's result is void and flagged
            atomicOr(p.err, p.err_bit);
            failed = true;
        };
        if (part > 0 && p.wait_limit == 0) give_up();  // a limit of 0: every partition but the first gives up at once
        // counts of the group's partitions before this one, kLookWindow loads in flight
        uint32_t within = 0;
        for (uint32_t q = first; q < part && !failed;) {
            uint32_t sv[kLookWindow];
#pragma unroll
            for (int w = 0; w < kLookWindow; ++w)
                sv[w] = q + w < part ? ld_acquire(p.status + (size_t)(q + w) * kRadix + d) : kFlagAgg;
            bool stall = false;
#pragma unroll
            for (int w = 0; w < kLookWindow; ++w) {
                if (stall || q + w >= part) continue;
                if ((sv[w] & ~kValMask) == 0u) { stall = true; continue; }
                within += sv[w] & kValMask;
            }
            uint32_t adv = 0;
#pragma unroll
            for (int w = 0; w < kLookWindow; ++w)
                if (adv == (uint32_t)w && q + w < part && (sv[w] & ~kValMask) != 0u) ++adv;
            q += adv;
            if (stall) {
                if (++spins >= p.wait_limit) give_up();
                __builtin_amdgcn_s_sleep(1);
            }
        }
        uint32_t gprefix = 0;
        uint32_t* gst = p.gstatus + (size_t)grp * kRadix + d;
        if (part == last) {
            const uint32_t gtotal = within + total;
            if (grp == 0) {
                st_release(gst, kFlagInc | gtotal);
            } else {
                st_release(gst, kFlagAgg | gtotal);
                // look back over the groups with kLookWindow loads in flight; groups
                // below 0 read as an inclusive prefix of 0
                int j = (int)grp - 1;
                while (!failed) {
                    uint32_t sv[kLookWindow];
#pragma unroll
                    for (int w = 0; w < kLookWindow; ++w)
                        sv[w] = j - w >= 0 ? ld_acquire(p.gstatus + (size_t)(j - w) * kRadix + d) : kFlagInc;
                    int used = 0;
                    bool found = false, stall = false;
#pragma unroll
                    for (int w = 0; w < kLookWindow; ++w) {
                        if (found || stall) continue;
                        if ((sv[w] & ~kValMask) == 0u) { stall = true; continue; }
                        gprefix += sv[w] & kValMask;
                        ++used;
                        if (sv[w] & kFlagInc) found = true;
                    }
                    if (found) break;
                    j -= used;
                    if (stall) {
                        if (++spins >= p.wait_limit) give_up();
                        __builtin_amdgcn_s_sleep(1);
                    }
                }
                st_release(gst, kFlagInc | ((gprefix + gtotal) & kValMask));
            }
        } else if (grp > 0) {
            // the previous group's inclusive prefix
            const uint32_t* pg = p.gstatus + (size_t)(grp - 1) * kRadix + d;
            while (!failed) {
                const uint32_t v = ld_acquire(pg);
                if (v & kFlagInc) { gprefix = v & kValMask; break; }
                if (++spins >= p.wait_limit) give_up();
                __builtin_amdgcn_s_sleep(1);
            }
        }
        const uint32_t prefix = gprefix + within;
        // global position of local slot q (digit d) = s_base[d] + q
        s_base[d] = s_off[d] + prefix - blk;
    }
    __syncthreads();
    // stage the partition in digit order in LDS ...
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
        if (base + i * 64 + lane < count) {
            const uint32_t d = (key[i] >> p.shift) & 255u;
            const uint32_t q = s_blk[d] + s_wave[wave][d] + rank[i];
            if (q < (uint32_t)kSortPart) {  // always true for a consistent ranking
                s_keys[q] = (KeyT)key[i];
                s_vals[q] = val[i];
            }
        }
    }
    __syncthreads();
    // ... and write it out: consecutive slots of one digit go to consecutive addresses
    const uint32_t nloc = min((uint32_t)kSortPart, count - part * kSortPart);
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
        const uint32_t q = (uint32_t)(i * THREADS + tid);
        if (q < nloc) {
            const uint32_t k = (uint32_t)s_keys[q];
            const uint32_t pos = s_base[(k >> p.shift) & 255u] + q;
            if (pos < count) {  // always true for a consistent histogram; guards the buffers
                if (p.keys_out) static_cast<KeyT*>(p.keys_out)[pos] = (KeyT)k;
                p.vals_out[pos] = s_vals[q];
            }
        }
    }
}

struct EmitArgs {
    int32_t n;               // Gaussians over all views
    int32_t tiles_x;
    int32_t n_view;          // Gaussians per view (batched views: entry v n_view + i is Gaussian i in view v)
    int32_t tiles_y;         // tile rows per view
    int32_t views;
    uint32_t cap;
    uint32_t eparts;
    uint32_t xblocks;
    const uint32_t* order;   // Gaussians in depth order (visible ones first)
    const int16_t* rect;
    const int32_t* tt;
    uint32_t* part;          // [eparts] entries per scan partition -> exclusive offsets
    uint32_t* goff;          // [n] tile count, then first output slot, of the j-th Gaussian in depth order
    uint32_t* bstart;        // [xblocks + 1] depth-order index of each expand block's first Gaussian
    uint16_t* tkeys;         // [cap] tile id (at most 65536 tiles)
    uint32_t* tvals;         // [cap] Gaussian
    uint32_t* stripes;       // [kStripes][kHistBins] striped digit counts
    uint32_t* tcnt0;         // [xblocks][256] tile digit-0 counts of each expand block
    uint32_t* num_keys;
    uint32_t* overflow;
    const uint32_t* err;     // look-back failures of the depth passes
};

__device__ inline void unpack_rect(uint2 r, int& x0, int& y0, int& x1, int& y1) {
    x0 = (int)(int16_t)(r.x & 0xffffu); y0 = (int)(int16_t)(r.x >> 16);
    x1 = (int)(int16_t)(r.y & 0xffffu); y1 = (int)(int16_t)(r.y >> 16);
}

// Block-wide exclusive sum over 256 threads; returns this thread's prefix and the total.
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
    for (int w = 0; w < 4; ++w) {
        if (w < wave) add += s_wsum[w];
        total += s_wsum[w];
    }
    return x - v + add;
}

// Tile sort passes by reduce-then-scan: the digit counts of every block of
// the pass's input are known before the pass (the emission counts digit 0 per
// expand block, k_digit_count digit 1 per partition), k_digit_scan turns them
// into per-digit prefixes, and k_pass_scatter ranks and writes each partition
// with no wait on other partitions.  Same partitions, ranking and output as
// k_onesweep.

// Digit counts of every partition of the pass's input: cnt[part][d].  Every
// entry is written (zeros past the items).
template <int THREADS, int IPT>
__global__ __launch_bounds__(THREADS) void k_digit_count(const uint16_t* keys, const uint32_t* count_dev, uint32_t cap,
                                                         int shift, uint32_t* cnt, const uint32_t* skip) {
    static_assert(IPT == 8, "one 16-byte load of eight 16-bit keys per thread");
    __shared__ uint32_t h[kRadix];
    const int tid = threadIdx.x;
    for (int i = tid; i < kRadix; i += THREADS) h[i] = 0;
    __syncthreads();
    if (*skip == 0u) {
        const uint32_t count = min(*count_dev, cap);
        const uint32_t k0 = blockIdx.x * (uint32_t)(THREADS * IPT) + (uint32_t)tid * IPT;
        uint32_t k[IPT];
        if (k0 + IPT <= count) {  // keys are 256-byte aligned and k0 a multiple of 8
            const uint4 v = *reinterpret_cast<const uint4*>(keys + k0);
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int u = 0; u < 4; ++u) { k[2 * u] = w[u] & 0xffffu; k[2 * u + 1] = w[u] >> 16; }
        } else {
#pragma unroll
            for (int u = 0; u < IPT; ++u) k[u] = k0 + u < count ? (uint32_t)keys[k0 + u] : 0xffffffffu;
        }
#pragma unroll
        for (int u = 0; u < IPT; ++u)
            if (k[u] != 0xffffffffu) atomicAdd(&h[(k[u] >> shift) & 255u], 1u);
    }
    __syncthreads();
    for (int d = tid; d < kRadix; d += THREADS) cnt[(size_t)blockIdx.x * kRadix + d] = h[d];
}

// One block per digit d: pre[d][c] = the output position of the first item
// of digit d in block c of the pass's input: the items of smaller digits in
// the whole pass (from the pass histogram) plus the items of digit d in the
// blocks before c (from the counts cnt[c][d]; column reads, row writes, so
// both sides write whole cache lines).  Every load of a chunk of columns is
// issued before the scan.  Also records which digits occur, for the
// ranking's bit mask.
constexpr int kScanCols = 16;  // columns per thread per chunk
__global__ __launch_bounds__(kRadix) void k_digit_scan(const uint32_t* stripes, int hist_bin, const uint32_t* cnt,
                                                       uint32_t* pre, uint32_t cols, uint32_t* vmw,
                                                       const uint32_t* skip) {
    __shared__ uint32_t s_wsum[4];
    __shared__ uint32_t s_base;
    if (*skip != 0u) return;
    const int tid = threadIdx.x;
    const uint32_t d = blockIdx.x;
    uint32_t* row = pre + (size_t)d * cols;
    uint32_t run = 0;
    for (uint32_t c0 = 0; c0 < cols; c0 += kScanCols * kRadix) {
        const uint32_t j0 = c0 + kScanCols * tid;
        uint32_t c[kScanCols];
#pragma unroll
        for (int k = 0; k < kScanCols; ++k) c[k] = j0 + k < cols ? cnt[(size_t)(j0 + k) * kRadix + d] : 0u;
        if (c0 == 0) {
            // digit base: thread t sums the histogram of digit t, the block scans them
            uint32_t tot;
            const uint32_t h = stripe_sum(stripes, hist_bin + tid);
            const uint32_t ex = block_excl_sum(h, s_wsum, tot);
            if ((uint32_t)tid == d) {
                s_base = ex;
                if (h) {
                    atomicOr(&vmw[0], d);
                    atomicOr(&vmw[1], ~d & 255u);
                }
            }
            __syncthreads();
            run = s_base;
        }
        uint32_t sum = 0;
#pragma unroll
        for (int k = 0; k < kScanCols; ++k) sum += c[k];
        uint32_t ctot;
        uint32_t off = run + block_excl_sum(sum, s_wsum, ctot);
#pragma unroll
        for (int k = 0; k < kScanCols; ++k) {
            if (j0 + k < cols) row[j0 + k] = off;
            off += c[k];
        }
        run += ctot;
    }
}

template <int THREADS, int IPT, typename KeyT>
__global__ __launch_bounds__(THREADS) void k_pass_scatter(PassArgs p) {
    constexpr int kWaves = THREADS / 64;
    constexpr int kSortPart = THREADS * IPT;
    static_assert(THREADS >= kRadix && THREADS % 64 == 0, "one thread per digit");
    __shared__ uint32_t s_wave[kWaves][kRadix];  // per-wave digit counts -> prefixes
    __shared__ uint32_t s_base[kRadix];          // output position of local slot q of digit d: s_base[d] + q
    __shared__ uint32_t s_blk[kRadix];           // block-local exclusive digit offsets
    __shared__ KeyT s_keys[kSortPart];           // partition in digit order
    __shared__ uint32_t s_vals[kSortPart];
    __shared__ uint32_t s_wsum[kRadix / 64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (p.skip && *p.skip != 0u) return;  // the list overflowed or the depth sort failed
    uint32_t count = p.count_dev ? *p.count_dev : p.count_host;
    if (count > p.cap) count = p.cap;
    // Blocks go to the 8 XCDs round-robin; give each XCD a contiguous range of
    // partitions, so that the output runs of one digit from neighbouring
    // partitions meet in one L2 and leave it as whole lines.
    const uint32_t per_xcd = gridDim.x / kXcds;  // the grid is a multiple of kXcds
    const uint32_t part = (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
    if (part * (uint32_t)kSortPart >= count) return;  // uniform over the block
    const uint32_t vm = (p.vmw[0] ^ (~p.vmw[1] & 255u)) & 255u;  // bits in which the digits differ
    for (int i = tid; i < kWaves * kRadix; i += THREADS) (&s_wave[0][0])[i] = 0;
    const uint32_t base = part * kSortPart + wave * 64 * IPT;
    uint32_t key[IPT], val[IPT], rank[IPT];
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
        const uint32_t idx = base + i * 64 + lane;
        key[i] = idx < count ? (uint32_t) static_cast<const KeyT*>(p.keys_in)[idx] : 0u;
        val[i] = idx < count ? p.vals_in[idx] : 0u;
    }
    // digit thread d: output position of this partition's first item of digit d
    const uint32_t first = tid < kRadix ? p.prefix[(size_t)tid * p.stride + (size_t)part * p.cols_per_part] : 0u;
    __syncthreads();
    const uint64_t lt = lanemask_lt();
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
        const bool valid = (base + i * 64 + lane) < count;
        const uint32_t d = (key[i] >> p.shift) & 255u;
        const uint64_t m = match_digits(d, valid, vm);
        const uint32_t below = (uint32_t)__popcll(m & lt);
        const uint32_t prev = valid ? s_wave[wave][d] : 0u;
        rank[i] = prev + below;
        __builtin_amdgcn_wave_barrier();
        if (valid && below == 0) s_wave[wave][d] = prev + (uint32_t)__popcll(m);
        __builtin_amdgcn_wave_barrier();
    }
    __syncthreads();
    uint32_t total = 0, tx = 0;
    if (tid < kRadix) {
        const int d = tid;
        uint32_t run = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const uint32_t c = s_wave[w][d];
            s_wave[w][d] = run;
            run += c;
        }
        total = run;
        tx = wave_incl_sum(total);
        if (lane == 63) s_wsum[wave] = tx;
    }
    __syncthreads();
    if (tid < kRadix) {
        const int d = tid;
        uint32_t add = 0;
        for (int w = 0; w < wave; ++w) add += s_wsum[w];
        const uint32_t blk = tx - total + add;
        s_blk[d] = blk;
        s_base[d] = first - blk;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
        if (base + i * 64 + lane < count) {
            const uint32_t d = (key[i] >> p.shift) & 255u;
            const uint32_t q = s_blk[d] + s_wave[wave][d] + rank[i];
            if (q < (uint32_t)kSortPart) {  // always true for a consistent ranking
                s_keys[q] = (KeyT)key[i];
                s_vals[q] = val[i];
            }
        }
    }
    __syncthreads();
    const uint32_t nloc = min((uint32_t)kSortPart, count - part * kSortPart);
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
        const uint32_t q = (uint32_t)(i * THREADS + tid);
        if (q < nloc) {
            const uint32_t kq = (uint32_t)s_keys[q];
            const uint32_t pos = s_base[(kq >> p.shift) & 255u] + q;
            if (pos < count) {  // always true for consistent counts; guards the buffers
                if (p.keys_out) static_cast<KeyT*>(p.keys_out)[pos] = (KeyT)kq;
                p.vals_out[pos] = s_vals[q];
            }
        }
    }
}

__device__ inline uint32_t tiles_of(const EmitArgs& a, int64_t j) {
    if (j >= a.n) return 0u;
    const uint32_t g = a.order[j];
    return g < (uint32_t)a.n ? (uint32_t)max(a.tt[g], 0) : 0u;
}

// 3a. entries per scan partition of 1024 depth-ordered Gaussians.  The tile
// count of the j-th Gaussian in depth order is gathered here once and left in
// goff[j], where the offsets pass reads it with coalesced loads.
__global__ __launch_bounds__(kEmitThreads) void k_emit_count(EmitArgs a) {
    __shared__ uint32_t s_wsum[4];
    const int tid = threadIdx.x;
    uint32_t c = 0;
#pragma unroll
    for (int k = 0; k < kEmitIPT; ++k) {
        const int64_t j = (int64_t)blockIdx.x * kEmitPart + k * kEmitThreads + tid;
        const uint32_t t = tiles_of(a, j);
        if (j < a.n) a.goff[j] = t;
        c += t;
    }
    uint32_t total;
    block_excl_sum(c, s_wsum, total);
    if (tid == 0) a.part[blockIdx.x] = total;
}

// 3b. first output slot of every Gaussian (depth order), and for every expand
// block (kSlots consecutive slots) the Gaussian whose range holds its first slot.
// The partition's offset is the sum of the earlier partitions' totals (at most
// a few thousand L2-resident words per block, no separate scan pass); the last
// partition also writes K and the overflow flag.
__global__ __launch_bounds__(kEmitThreads) void k_emit_offsets(EmitArgs a) {
    __shared__ uint32_t s_wsum[4];
    const int tid = threadIdx.x;
    uint32_t before = 0;
    for (uint32_t i = tid; i < blockIdx.x; i += kEmitThreads) before += a.part[i];
    uint32_t pbase;
    block_excl_sum(before, s_wsum, pbase);
    const int64_t j0 = (int64_t)blockIdx.x * kEmitPart + (int64_t)tid * kEmitIPT;
    // the depth-ordered tile counts k_emit_count left in goff (overwritten below by the offsets)
    uint32_t c[kEmitIPT], sum = 0;
    static_assert(kEmitIPT == 4, "one 16-byte load per thread");
    if (j0 + kEmitIPT <= a.n) {  // goff is 256-byte aligned and j0 a multiple of 4
        const uint4 v = *reinterpret_cast<const uint4*>(a.goff + j0);
        c[0] = v.x; c[1] = v.y; c[2] = v.z; c[3] = v.w;
    } else {
#pragma unroll
        for (int k = 0; k < kEmitIPT; ++k) c[k] = j0 + k < a.n ? a.goff[j0 + k] : 0u;
    }
#pragma unroll
    for (int k = 0; k < kEmitIPT; ++k) sum += c[k];
    uint32_t total;
    uint32_t off = pbase + block_excl_sum(sum, s_wsum, total);
    if (blockIdx.x == gridDim.x - 1 && tid == 0) {
        const uint32_t K = pbase + total;
        *a.num_keys = K;
        // bit 0: more entries than capacity; bit 1: the depth sort failed (its order is void)
        *a.overflow = (K > a.cap ? 1u : 0u) | (*a.err != 0u ? 2u : 0u);
    }
#pragma unroll
    for (int k = 0; k < kEmitIPT; ++k) {
        const int64_t j = j0 + k;
        if (j < a.n) a.goff[j] = off;
        if (c[k]) {
            // expand blocks whose first slot lies in [off, off + c)
            for (uint32_t b = (off + kSlots - 1) / kSlots; (uint64_t)b * kSlots < (uint64_t)off + c[k] &&
                                                             b < a.xblocks; ++b)
                a.bstart[b] = (uint32_t)j;
        }
        off += c[k];
    }
}

// 3c. expansion over output slots: block b writes slots [b kSlots, (b+1) kSlots).
// Its Gaussians are a run of the depth order starting at bstart[b]; each slot's
// owner is the last Gaussian whose first slot is at or before it (a max-scan over
// the heads), and the slot's rank inside the owner's rect gives the tile
// (row-major).  Also counts the two tile-id digits for the sort.
__global__ __launch_bounds__(kEmitThreads) void k_emit_expand(EmitArgs a) {
    __shared__ uint32_t s_gid[kSlots];
    __shared__ uint32_t s_goff[kSlots];
    __shared__ uint2 s_rect[kSlots];
    __shared__ uint16_t s_owner[kSlots];  // owner q < kSlots; 16 bits keep the block under 40 KB of LDS (4 per CU)
    __shared__ uint32_t s_hist[2 * kRadix];
    __shared__ uint32_t s_wsum[4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint32_t K = min(*a.num_keys, a.cap);
    const uint32_t base = blockIdx.x * (uint32_t)kSlots;
    const bool active = !*a.overflow && base < K;
    for (int i = tid; i < 2 * kRadix; i += kEmitThreads) s_hist[i] = 0;
    if (!active)  // the tile sort reads every block's counts
        for (int i = tid; i < kRadix; i += kEmitThreads) a.tcnt0[(size_t)blockIdx.x * kRadix + i] = 0u;
    if (active) {
        const uint32_t nout = min((uint32_t)kSlots, K - base);
        const uint32_t jb = a.bstart[blockIdx.x];
        for (int s = tid; s < kSlots; s += kEmitThreads) s_owner[s] = 0;
        __syncthreads();
        // the block's Gaussians: jb + q (q < nout) whose first slot is < base + nout
        for (uint32_t q0 = 0; q0 < nout; q0 += kEmitThreads) {
            const uint32_t q = q0 + tid;
            const int64_t j = (int64_t)jb + q;
            const uint32_t go = (q < nout && j < a.n) ? a.goff[j] : 0xffffffffu;
            const bool in = go < base + nout;
            if (in) {
                const uint32_t g = a.order[j];
                s_goff[q] = go;
                s_gid[q] = g;
                uint2 r = reinterpret_cast<const uint2*>(a.rect)[g];
                if (a.views > 1) {
                    // view v's tiles follow the earlier views' (v tiles_y rows down): shift the rect's rows
                    const uint32_t dy = (g / (uint32_t)a.n_view) * (uint32_t)a.tiles_y;
                    r.x += dy << 16;
                    r.y += dy << 16;
                }
                s_rect[q] = r;
                // head: the slot where this Gaussian's run starts (0 for the first)
                const uint32_t h = q == 0 ? 0u : go - base;
                if (h < (uint32_t)kSlots) s_owner[h] = q;
            }
            if (!__syncthreads_or(in)) break;  // first slots increase with q
        }
        __syncthreads();
        // inclusive max-scan of s_owner: kSlotsPT consecutive slots per thread
        uint32_t v[kSlotsPT], run = 0;
#pragma unroll
        for (int k = 0; k < kSlotsPT; ++k) { run = max(run, s_owner[tid * kSlotsPT + k]); v[k] = run; }
        uint32_t x = run;
        for (int o = 1; o < 64; o <<= 1) {
            const uint32_t y = __shfl_up(x, o, 64);
            if (lane >= o) x = max(x, y);
        }
        if (lane == 63) s_wsum[wave] = x;
        __syncthreads();
        uint32_t pre = __shfl_up(x, 1, 64);
        if (lane == 0) pre = 0;
        for (int w = 0; w < wave; ++w) pre = max(pre, s_wsum[w]);
#pragma unroll
        for (int k = 0; k < kSlotsPT; ++k) s_owner[tid * kSlotsPT + k] = max(pre, v[k]);
        __syncthreads();
        for (uint32_t s = tid; s < (uint32_t)kSlots; s += kEmitThreads) {
            const bool ok = s < nout;
            uint32_t tile = 0;
            if (ok) {
                const uint32_t q = s_owner[s];
                int x0, y0, x1, y1;
                unpack_rect(s_rect[q], x0, y0, x1, y1);
                const uint32_t w = (uint32_t)(x1 - x0);
                const uint32_t r = base + s - s_goff[q];
                const uint32_t ry = r / w;
                tile = (uint32_t)(y0 + (int)ry) * (uint32_t)a.tiles_x + (uint32_t)x0 + (r - ry * w);
                a.tkeys[base + s] = (uint16_t)tile;
                a.tvals[base + s] = s_gid[q];
            }
            if (ok) {
                atomicAdd(&s_hist[tile & 255u], 1u);
                atomicAdd(&s_hist[kRadix + ((tile >> 8) & 255u)], 1u);
            }
        }
        __syncthreads();
        uint32_t* out = a.stripes + (size_t)(blockIdx.x % kStripes) * kHistBins + 4 * kRadix;
        for (int i = tid; i < 2 * kRadix; i += kEmitThreads) {
            if (s_hist[i]) atomicAdd(&out[i], s_hist[i]);
            if (i < kRadix) a.tcnt0[(size_t)blockIdx.x * kRadix + i] = s_hist[i];
        }
    }
}

// 5. tile ranges from sorted tile ids (ranges zeroed beforehand).  Each thread
// reads kRangeIPT consecutive keys with one vector load, plus one neighbour on
// each side.
__global__ __launch_bounds__(256) void k_ranges(const uint16_t* tkeys, const uint32_t* num_keys, uint32_t cap,
                                                uint32_t* overflow, const uint32_t* err, uint32_t* ranges,
                                                uint32_t ntiles) {
    // a failed tile pass voids the lists: report it with the overflow word and leave the ranges empty
    const bool failed = *err != 0u;
    if (failed && blockIdx.x == 0 && threadIdx.x == 0) atomicOr(overflow, 2u);
    if (failed || *overflow) return;
    const uint32_t K = min(*num_keys, cap);
    const uint32_t k0 = (blockIdx.x * blockDim.x + threadIdx.x) * (uint32_t)kRangeIPT;
    if (k0 >= K) return;
    constexpr uint32_t kNone = 0xffffffffu;  // never a tile id
    static_assert(kRangeIPT == 8, "one 16-byte load of eight 16-bit keys per thread");
    uint32_t t[kRangeIPT];
    if (k0 + kRangeIPT <= K) {  // tkeys is 256-byte aligned and k0 a multiple of 8
        const uint4 a = *reinterpret_cast<const uint4*>(tkeys + k0);
        const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            t[2 * u] = w[u] & 0xffffu;
            t[2 * u + 1] = w[u] >> 16;
        }
    } else {
#pragma unroll
        for (int u = 0; u < kRangeIPT; ++u) t[u] = k0 + u < K ? (uint32_t)tkeys[k0 + u] : kNone;
    }
    const uint32_t prev = k0 > 0 ? (uint32_t)tkeys[k0 - 1] : kNone;
    const uint32_t next = k0 + kRangeIPT < K ? (uint32_t)tkeys[k0 + kRangeIPT] : kNone;
#pragma unroll
    for (int u = 0; u < kRangeIPT; ++u) {
        const uint32_t k = k0 + u, cur = t[u];
        if (k >= K || cur >= ntiles) continue;
        const uint32_t left = u == 0 ? prev : t[u - 1];
        const uint32_t right = u == kRangeIPT - 1 ? next : t[u + 1];
        if (left != cur) ranges[2 * cur] = k;
        if (right != cur) ranges[2 * cur + 1] = k + 1;
    }
}

__global__ void k_keys(const uint32_t* ranges, const uint32_t* list, const float* depth, uint64_t* keys,
                       int ntiles) {
    const int t = blockIdx.x;
    if (t >= ntiles) return;
    const uint32_t b = ranges[2 * t], e = ranges[2 * t + 1];
    for (uint32_t k = b + threadIdx.x; k < e; k += blockDim.x)
        keys[k] = ((uint64_t)t << 32) | (uint64_t)__float_as_uint(depth[list[k]]);  // list entries < n by construction
}

}  // namespace
}  // namespace gs

using namespace gs;

namespace {
std::atomic<uint32_t> g_wait_limit{kWaitLimit};  // look-back waits before a sort pass gives up
}

extern "C" int64_t gs_debug_sort_wait_limit(int64_t limit) {
    const uint32_t prev = g_wait_limit.load();
    if (limit >= 0) g_wait_limit.store(limit > (int64_t)UINT32_MAX ? UINT32_MAX : (uint32_t)limit);
    return (int64_t)prev;
}

extern "C" int gs_bin_workspace_size_views(int32_t n, const gs_camera* cams, int32_t views, int64_t key_capacity,
                                           size_t* bytes) {
    if (n < 0 || !views_ok(cams, views) || key_capacity < 0 || !bytes) return GS_EINVAL;
    if (key_capacity > (int64_t)kValMask || (int64_t)views * n > (int64_t)kValMask) return GS_ECAPACITY;
    *bytes = make_layout(views * n, key_capacity).total;
    return GS_OK;
}

extern "C" int gs_bin_workspace_size(int32_t n, const gs_camera* cam, int64_t key_capacity, size_t* bytes) {
    return gs_bin_workspace_size_views(n, cam, 1, key_capacity, bytes);
}

extern "C" int gs_bin_sort(const gs_camera* cam, int32_t n, const float* depth, const int16_t* rect,
                           const int32_t* tiles_touched, int64_t key_capacity, uint32_t* point_list,
                           uint32_t* tile_ranges, uint32_t* num_keys_dev, uint32_t* overflow_dev,
                           void* workspace, size_t workspace_bytes, void* stream) {
    return gs_bin_sort_views(cam, 1, n, depth, rect, tiles_touched, key_capacity, point_list, tile_ranges,
                             num_keys_dev, overflow_dev, workspace, workspace_bytes, stream);
}

extern "C" int gs_bin_sort_views(const gs_camera* cams, int32_t views, int32_t n_view, const float* depth,
                                 const int16_t* rect, const int32_t* tiles_touched, int64_t key_capacity,
                                 uint32_t* point_list, uint32_t* tile_ranges, uint32_t* num_keys_dev,
                                 uint32_t* overflow_dev, void* workspace, size_t workspace_bytes, void* stream) {
    if (n_view < 0 || !views_ok(cams, views) || key_capacity < 0) return GS_EINVAL;
    if (key_capacity > (int64_t)kValMask || (int64_t)views * n_view > (int64_t)kValMask) return GS_ECAPACITY;
    const gs_camera* cam = cams;
    const int32_t n = views * n_view;  // all views' Gaussians, view-major
    if (!tile_ranges || !num_keys_dev || !overflow_dev || !workspace) return GS_EINVAL;
    if (n > 0 && (!depth || !rect || !tiles_touched)) return GS_EINVAL;
    if (key_capacity > 0 && !point_list) return GS_EINVAL;
    if (!aligned16(rect) || (reinterpret_cast<uintptr_t>(workspace) & 255u)) return GS_EALIGN;
    const Layout L = make_layout(n, key_capacity);
    if (workspace_bytes < L.total) return GS_EWORKSPACE;
    const int ntiles = views * tiles_x(cam) * tiles_y(cam);
    const int tile_passes = ntiles <= 256 ? 1 : (ntiles <= 65536 ? 2 : 3);
    if (tile_passes > 2) return GS_ECAPACITY;
    hipStream_t s = as_stream(stream);
    char* ws = static_cast<char*>(workspace);
    auto U = [&](size_t off) { return reinterpret_cast<uint32_t*>(ws + off); };
    auto H = [&](size_t off) { return reinterpret_cast<uint16_t*>(ws + off); };

    // zero counters, histograms, look-back status, ranges, K and the overflow flag
    {
        ClearArgs c;
        c.p[0] = U(0); c.count[0] = L.zero_end / 4;
        c.p[1] = tile_ranges; c.count[1] = (size_t)2 * ntiles;
        c.p[2] = num_keys_dev; c.count[2] = 1;
        c.p[3] = overflow_dev; c.count[3] = 1;
        hipLaunchKernelGGL(k_clear, dim3(512), dim3(256), 0, s, c);
    }
    if (n == 0) return launch_status();

    uint32_t* tickets = U(L.tickets);
    auto ticket = [&](int pass) { return tickets + (size_t)pass * kTicketGroups * kTicketStride; };
    uint32_t* err = U(L.err);  // bit p: depth sort pass p gave up
    const uint32_t wait_limit = g_wait_limit.load();
    const int key_blocks = (int)((n + 256 * kKeyIPT - 1) / (256 * kKeyIPT));
    hipLaunchKernelGGL(k_depth_keys, dim3(key_blocks), dim3(256), 0, s, n, depth, tiles_touched, U(L.dkeys0),
                       U(L.dvals0), U(L.stripes));
    // depth sort: 4 passes, 0 -> 1 -> 0 -> 1 -> 0
    uint32_t* dk[2] = {U(L.dkeys0), U(L.dkeys1)};
    uint32_t* dv[2] = {U(L.dvals0), U(L.dvals1)};
    for (int pass = 0; pass < 4; ++pass) {
        PassArgs p;
        p.keys_in = dk[pass & 1]; p.vals_in = dv[pass & 1];
        p.keys_out = pass < 3 ? dk[(pass + 1) & 1] : nullptr;
        p.vals_out = dv[(pass + 1) & 1];
        p.count_dev = nullptr; p.count_host = (uint32_t)n; p.cap = (uint32_t)n;
        p.stripes = U(L.stripes); p.hist_bin = pass * kRadix;
        p.status = U(L.dstatus) + (size_t)pass * L.dparts * kRadix;
        p.gstatus = U(L.dgstatus) + (size_t)pass * ((L.dparts + kLookGroup - 1) / kLookGroup) * kRadix;
        p.ticket = ticket(pass);
        p.err = err; p.err_bit = 1u << pass; p.err_before = (1u << pass) - 1u; p.skip = nullptr;
        p.wait_limit = wait_limit;
        p.shift = 8 * pass;
        hipLaunchKernelGGL((k_onesweep<kDepthThreads, kDepthIPT, uint32_t>), dim3(L.dparts), dim3(kDepthThreads), 0, s, p);
    }
    // emit (tile, Gaussian) pairs in depth order, then the stable tile sort.
    // Buffers are routed so the final values land in point_list:
    //   1 pass : emit -> (tkeys0, tvals0) -> (tkeys1, point_list)
    //   2 passes: emit -> (tkeys0, point_list) -> (tkeys1, tvals0) -> (tkeys0, point_list)
    EmitArgs e;
    e.n = n; e.tiles_x = tiles_x(cam); e.n_view = n_view; e.tiles_y = tiles_y(cam); e.views = views;
    e.cap = (uint32_t)key_capacity; e.eparts = L.eparts;
    e.xblocks = L.xblocks;
    e.order = dv[0]; e.rect = rect; e.tt = tiles_touched;
    e.part = U(L.etotal); e.goff = U(L.goff); e.bstart = U(L.bstart);
    e.tkeys = H(L.tkeys0); e.tvals = tile_passes == 1 ? U(L.tvals0) : point_list;
    e.stripes = U(L.stripes); e.tcnt0 = U(L.tcnt0);
    e.num_keys = num_keys_dev; e.overflow = overflow_dev; e.err = err;
    hipLaunchKernelGGL(k_emit_count, dim3(L.eparts), dim3(kEmitThreads), 0, s, e);
    hipLaunchKernelGGL(k_emit_offsets, dim3(L.eparts), dim3(kEmitThreads), 0, s, e);
    if (key_capacity == 0) return launch_status();
    hipLaunchKernelGGL(k_emit_expand, dim3(L.xblocks), dim3(kEmitThreads), 0, s, e);
    // the tile passes: offsets from the partition counts, then a scatter per digit;
    // everything skips when the emission found an overflow or a failed depth sort
    uint32_t* vmw = U(L.vmw);
    hipLaunchKernelGGL(k_digit_scan, dim3(kRadix), dim3(kRadix), 0, s, (const uint32_t*)U(L.stripes), 4 * kRadix,
                       (const uint32_t*)U(L.tcnt0), U(L.tpre0), L.xblocks, vmw, (const uint32_t*)overflow_dev);
    PassArgs p = {};
    p.count_dev = num_keys_dev; p.count_host = 0; p.cap = (uint32_t)key_capacity;
    p.skip = overflow_dev;
    p.keys_in = H(L.tkeys0); p.vals_in = e.tvals;
    p.keys_out = H(L.tkeys1); p.vals_out = tile_passes == 1 ? point_list : U(L.tvals0);
    p.shift = 0; p.prefix = U(L.tpre0); p.stride = L.xblocks; p.cols_per_part = kTilePart / kSlots; p.vmw = vmw;
    const uint32_t sgrid = (L.tparts + kXcds - 1) / kXcds * kXcds;
    hipLaunchKernelGGL((k_pass_scatter<kTileThreads, kTileIPT, uint16_t>), dim3(sgrid), dim3(kTileThreads), 0, s, p);
    const uint16_t* tk_final = H(L.tkeys1);
    if (tile_passes == 2) {
        hipLaunchKernelGGL((k_digit_count<kTileThreads, kTileIPT>), dim3(L.tparts), dim3(kTileThreads), 0, s,
                           (const uint16_t*)H(L.tkeys1), (const uint32_t*)num_keys_dev, (uint32_t)key_capacity, 8,
                           U(L.tcnt1), (const uint32_t*)overflow_dev);
        hipLaunchKernelGGL(k_digit_scan, dim3(kRadix), dim3(kRadix), 0, s, (const uint32_t*)U(L.stripes), 5 * kRadix,
                           (const uint32_t*)U(L.tcnt1), U(L.tpre1), L.tparts, vmw + 2, (const uint32_t*)overflow_dev);
        PassArgs p2 = p;
        p2.keys_in = H(L.tkeys1); p2.vals_in = U(L.tvals0);
        p2.keys_out = H(L.tkeys0); p2.vals_out = point_list;
        p2.shift = 8; p2.prefix = U(L.tpre1); p2.stride = L.tparts; p2.cols_per_part = 1; p2.vmw = vmw + 2;
        hipLaunchKernelGGL((k_pass_scatter<kTileThreads, kTileIPT, uint16_t>), dim3(sgrid), dim3(kTileThreads), 0, s, p2);
        tk_final = H(L.tkeys0);
    }
    const uint32_t rblocks = (uint32_t)((key_capacity + 256 * kRangeIPT - 1) / (256 * kRangeIPT));
    hipLaunchKernelGGL(k_ranges, dim3(rblocks), dim3(256), 0, s, tk_final, num_keys_dev, (uint32_t)key_capacity,
                       overflow_dev, err, tile_ranges, (uint32_t)ntiles);
    return launch_status();
}

// ---- the allocation-free variant: gs_bin_sort with the library's own scratch ----

namespace gs {
namespace {
constexpr size_t kScratchBytes = (size_t)128 << 20;  // the binning workspace the variant can use
constexpr int kMaxDevices = 64;
}  // namespace
}  // namespace gs

// Device scratch of the allocation-free binning call: one copy per GPU, held
// until the process ends.  Host code never uses this name as an address (in
// host code it is a stand-in, not device memory); it uses the per-device
// address hipGetSymbolAddress returns.
static __device__ __align__(256) unsigned char scratch[gs::kScratchBytes];

namespace {
std::mutex g_scratch_mutex;
void* g_scratch_ptr[gs::kMaxDevices] = {};
}  // namespace

// The current device's copy of `scratch`, looked up once per device.
static int scratch_address(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return GS_EHIP;
    if (dev < 0 || dev >= gs::kMaxDevices) return GS_EINVAL;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return GS_EHIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return GS_OK;
}

extern "C" int64_t gs_bin_scratch_bytes(void) { return (int64_t)gs::kScratchBytes; }

extern "C" int gs_bin_sort_noalloc(const gs_camera* cam, int32_t n, const float* depth, const int16_t* rect,
                                   const int32_t* tiles_touched, int64_t key_capacity, uint32_t* point_list,
                                   uint32_t* tile_ranges, uint32_t* num_keys_dev, uint32_t* overflow_dev,
                                   void* stream) {
    size_t need = 0;
    int rc = gs_bin_workspace_size(n, cam, key_capacity, &need);
    if (rc) return rc;
    if (need > gs::kScratchBytes) return GS_EWORKSPACE;
    void* ws = nullptr;
    rc = scratch_address(&ws);
    if (rc) return rc;
    return gs_bin_sort(cam, n, depth, rect, tiles_touched, key_capacity, point_list, tile_ranges, num_keys_dev,
                       overflow_dev, ws, gs::kScratchBytes, stream);
}

extern "C" int gs_bin_keys(const gs_camera* cam, const uint32_t* tile_ranges, const uint32_t* point_list,
                           const float* depth, uint64_t* keys, void* stream) {
    if (!camera_ok(cam) || !tile_ranges || !point_list || !depth || !keys) return GS_EINVAL;
    const int ntiles = tiles_x(cam) * tiles_y(cam);
    hipLaunchKernelGGL(k_keys, dim3(ntiles), dim3(256), 0, as_stream(stream), tile_ranges, point_list, depth,
                       keys, ntiles);
    return launch_status();
}
