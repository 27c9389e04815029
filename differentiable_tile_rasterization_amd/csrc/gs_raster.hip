// gs_raster.hip -- gs_rasterize_fwd and gs_rasterize_bwd for gfx950.
//
// Both kernels run one 256-thread workgroup (4 wave64) per 16x16 tile; a
// 16x16 tile of 256 pixels per workgroup is the decomposition on page
// "Phase 5 step 30b — kernel-by-kernel timing" (section 結論と次着手). Each wave
// owns one 8x8 quadrant of the tile (lane l -> pixel (l & 7, l >> 3) of the
// quadrant), so a wave's pixels are as close together as possible: small
// splats then touch few waves.
//
// Data path, per call:
//   prep_kernel   one thread per splat packs a 48-byte record: mean, the
//                 scaled Cholesky factor of the conic and log2(opacity) (the
//                 alpha coefficients), colour, the culling threshold and the
//                 radius. Tile lists reference splats in depth order, i.e. at
//                 random ids; a record costs one 48-byte read per list entry
//                 where the caller's four separate arrays cost about five
//                 cache lines.
//   staging       per batch of list entries (255 and a dummy; 191 or 127
//                 and a dummy in some reverse walks), thread t loads
//                 entry t's record, writes the alpha coefficients and colour
//                 to LDS and tests the splat's alpha >= 1/255 ellipse against
//                 each 8x4 half-quadrant; ballots build one compacted list per
//                 half.
//   walk          each wave walks its two halves' lists in lockstep, each
//                 half reading its entry's coefficients with broadcast LDS
//                 loads.
// Optional outputs are template parameters, so a variant without the
// accumulated weight spends no instruction, register or global store on it,
// and its stored-partials records are a float shorter (the lesson of section
// 机制拆解 of the Spirula Studio page, where optional feature arrays sized
// regardless of the switch cut occupancy). The LDS-add walk keeps the same
// 80-byte slot in both instances: its records must stay 16-byte aligned, the
// next smaller aligned stride (64 bytes) cannot hold the nine sums beside the
// coefficients, and at 72 bytes (unaligned, seven workgroups per CU instead of
// six) the walk ran slower (0.500 against 0.464 ms on the 2M-splat scene).
#include <cstddef>
#include <mutex>
#include <type_traits>

#include "gs_common.hpp"

namespace gs {
namespace {

// Packed per-splat record (48 bytes). The culling test runs on the scaled
// form q' = (l11 dx + l21 dy)^2 + (l22 dy)^2 = q log2(e) / 2, whose
// coefficients come from the factor itself, so the record needs no conic.
struct SplatRec {
    float4 a;  // mean x, mean y, l11, l21 (scaled factor)
    float4 b;  // l22, log2(opacity), red, green
    float4 c;  // blue, culling threshold on q', radius (int bits), first pair slot (int bits; backward)
};

constexpr float kQScale = 0.72134752044448170f;  // log2(e) / 2: q' = kQScale q

// The record of splat i, from the caller's arrays (radii and first_slot may
// be NULL: the forward needs neither).
__device__ __forceinline__ SplatRec make_rec(int i, const float2* __restrict__ means,
                                             const float* __restrict__ conics, const float* __restrict__ colors,
                                             const float* __restrict__ opac, const int* __restrict__ radii,
                                             const int* __restrict__ first_slot = nullptr)
{
    const float2 m = means[i];
    const float a = conics[3 * i + 0], b = conics[3 * i + 1], c = conics[3 * i + 2];
    const float o = opac[i];
    const AlphaCoef k = make_alpha_coef(m.x, m.y, a, b, c, o);
    SplatRec r;
    r.a = make_float4(k.mx, k.my, k.l11, k.l21);
    r.b = make_float4(k.l22, k.lo, colors[3 * i + 0], colors[3 * i + 1]);
    r.c = make_float4(colors[3 * i + 2], kQScale * cull_tau(o), __int_as_float(radii ? radii[i] : 0),
                      __int_as_float(first_slot ? first_slot[i] : 0));
    return r;
}

// Stores the records of a 256-thread block (thread t: record i0 + t, those
// below n) through LDS, as consecutive 16-byte stores by consecutive threads
// rather than three 16-byte stores per thread at a 48-byte stride. Every
// thread of the block must call it.
__device__ __forceinline__ void store_recs_block(SplatRec* __restrict__ recs, const SplatRec& r, int i0, int n)
{
    __shared__ float4 buf[3 * 256];
    const int t = threadIdx.x;
    buf[3 * t + 0] = r.a;
    buf[3 * t + 1] = r.b;
    buf[3 * t + 2] = r.c;
    __syncthreads();
    const int cnt = 3 * min(256, n - i0);
    float4* const out = reinterpret_cast<float4*>(recs + i0);
    for (int k = t; k < cnt; k += 256) out[k] = buf[k];
}

// depths may be NULL; when given (the forward's depth outputs) the depth takes
// the record's last word, which only the backward uses otherwise.
__global__ __launch_bounds__(256) void prep_kernel(int n, const float2* __restrict__ means,
                                                   const float* __restrict__ conics, const float* __restrict__ colors,
                                                   const float* __restrict__ opac, const int* __restrict__ radii,
                                                   const float* __restrict__ depths, SplatRec* __restrict__ recs)
{
    const int i0 = blockIdx.x * 256, i = i0 + threadIdx.x;
    SplatRec r{};
    if (i < n) {
        r = make_rec(i, means, conics, colors, opac, radii);
        if (depths) r.c.w = depths[i];
    }
    store_recs_block(recs, r, i0, n);
}

// Pixel of thread threadIdx.x in the walks: wave w owns the 8x8 quadrant
// (w & 1, w >> 1) of the tile, lane l its pixel (l & 7, l >> 3).
__device__ __forceinline__ void quadrant_pixel(int tile, int GX, int& x, int& y)
{
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    x = (tile % GX) * kTile + (w & 1) * 8 + (l & 7);
    y = (tile / GX) * kTile + (w >> 1) * 8 + (l >> 3);
}

// ---------------------------------------------------------------------------
// Backward
//
// Per (splat, pixel) pair the kernel forms the pixel's share of
//   sum w g_r, sum w g_g, sum w g_b          (w = alpha T: colour gradient)
//   sum s, sum s dx, sum s dy, sum s dx^2, sum s dx dy, sum s dy^2
//                                          (s = dL/dsigma = alpha dL/dalpha)
//   [sum w]                                (accumulated weight, optional)
// The nine gradient fields are linear in these sums (dmean = Q (sum s d),
// dconic = -(1/2 sum s dx^2, sum s dx dy, 1/2 sum s dy^2), dopacity =
// sum s / opacity), so the per-splat constants are applied once per splat, in
// the gather, instead of once per pixel.
//
// Half-wave walk. A wave's 64 lanes are its quadrant's two 8x4 halves (lanes
// 0-31 and 32-63), and each half has its own culled list. The wave steps both
// lists in lockstep, each half on its own splat, so a small splat that reaches
// only one half no longer costs the whole wave a step: on the 2M-splat scene
// this cuts wave steps from 4.67M to about 3.3M. Once the shorter list is
// exhausted its half takes a dummy entry of opacity 0. The per-step reduction
// stays inside each half: v_permlane16_swap + adds fold rows (0, 1) and
// (2, 3) pairwise, leaving registers whose four rows hold (field, half) pairs,
// and bank-masked DPP adds merge them while finishing each row; a few leader
// lanes then add the totals into the workgroup's LDS partial of their half's
// entry.
//
// Finer lists (one per 4x4 block, four per wave) take about 18% fewer steps
// but were slower here: the workgroup meets at a barrier after every batch,
// and the slowest of sixteen lists keeps the other waves waiting longer than
// the slowest of eight.
//
// No global atomics: every (splat, tile) pair owns a fixed record slot, the
// pair's index in the binning's enumeration (the splat's first slot plus the
// tile's row-major index inside the splat's tile rectangle, recomputed from
// mean and radius with the binning's float32 rule). After each batch one
// thread per entry stores the entry's sums there with plain vector stores and
// marks the slot; gather_kernel then sums each splat's slots in a fixed order.
// Scattered float atomics cost about 1 ms for the 2.1e7 field updates of the
// 2M-splat scene on this part; the stores cost about 0.04 ms.
// ---------------------------------------------------------------------------
constexpr int kRaw = 10;   // w g_r, w g_g, w g_b, s, s dx, s dy, s dx^2, s dx dy, s dy^2, w
// float4 per (splat, tile) pair slot in the workspace: ten sums (eleven with
// the depth gradient) in three. A 64-byte stride (every slot in one line
// instead of 1.5 lines on average) measured no faster in the walk or the
// gather.
constexpr int kSlotF4 = 3;
constexpr int kHalves = 8; // 4 waves x 2 halves

// Staging test of the half-wave walk: bit `lane` of hits[hq] (a wave ballot,
// so that the lists are built from wave masks with no per-lane flags to pack
// and unpack) says whether the lane's splat can reach half h of quadrant q (hq = 2 q + h; the 8x4 pixels of rows 4 h ..
// 4 h + 3 of the quadrant), i.e. column q & 1 of 8-pixel columns and row
// 2 (q >> 1) + h of 4-pixel rows. Over a rectangle of pixel centres, the
// minimum of the convex form q' is 0 if the mean lies inside; otherwise it
// lies on the vertical edge facing the mean or on the horizontal edge facing
// it, and along a line the minimiser has a closed form, clamped to the edge.
// Clamping the mean's own coordinate into the column (row) range picks the
// facing edge, or the line through the mean when the mean lies within that
// range, where the candidate is 0 or a value at a point of the rectangle (an
// upper bound on the minimum). So min(vertical candidate, horizontal
// candidate) is the exact minimum, with no branch. Both candidates are
// evaluated as the sum of squares (l11 u + l21 v)^2 + (l22 v)^2, which loses
// nothing to cancellation for elongated splats. Halves whose walk ends at or
// before entry k (`hend`, wave-uniform) drop the entry.
__device__ __forceinline__ void half_hits(const SplatRec& r, float ox, float oy, int k, const int (&hend)[kHalves],
                                          unsigned long long (&hits)[kHalves])
{
    const float l11 = r.a.z, l21 = r.a.w, l22 = r.b.x, tau = r.c.y;
    // the minimiser along x = u is y = kv u; along y = v it is x = kh v
    const float kv = -l11 * l21 * __builtin_amdgcn_rcpf(__builtin_fmaf(l21, l21, l22 * l22));
    const float kh = -l21 * __builtin_amdgcn_rcpf(l11);
    const float bu = ox - r.a.x, bv = oy - r.a.y;
    float u0[2], u1[2], pu[2], yu[2], v0[4], v1[4], pv[4], sv[4], xv[4];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        u0[c] = bu + (float)(8 * c);
        u1[c] = u0[c] + 7.0f;
        const float u = __builtin_amdgcn_fmed3f(0.0f, u0[c], u1[c]);
        pu[c] = l11 * u;
        yu[c] = kv * u;
    }
#pragma unroll
    for (int rw = 0; rw < 4; ++rw) {
        v0[rw] = bv + (float)(4 * rw);
        v1[rw] = v0[rw] + 3.0f;
        const float v = __builtin_amdgcn_fmed3f(0.0f, v0[rw], v1[rw]);
        pv[rw] = l21 * v;
        const float t = l22 * v;
        sv[rw] = t * t;
        xv[rw] = kh * v;
    }
#pragma unroll
    for (int hq = 0; hq < kHalves; ++hq) {
        const int q = hq >> 1, c = q & 1, rw = 2 * (q >> 1) + (hq & 1);
        const float ys = __builtin_amdgcn_fmed3f(yu[c], v0[rw], v1[rw]);
        const float a1 = __builtin_fmaf(l21, ys, pu[c]);
        const float b1 = l22 * ys;
        const float qv = __builtin_fmaf(a1, a1, b1 * b1);
        const float xs = __builtin_amdgcn_fmed3f(xv[rw], u0[c], u1[c]);
        const float a2 = __builtin_fmaf(l11, xs, pv[rw]);
        const float qh = __builtin_fmaf(a2, a2, sv[rw]);
        hits[hq] = __ballot((fminf(qv, qh) <= tau) & (k < hend[hq]));
    }
}

// LDS slot of one staged entry: its alpha coefficients and colour, and its
// position in each half's list. One base address serves every record read of
// a walk step (the lists hold slot byte offsets).
struct StoreSlot {
    float4 a;                      // mean x, mean y, l11, l21 (scaled factor)
    float4 b;                      // l22, log2(opacity), red, green
    float c;                       // blue
    unsigned char pos[kHalves];    // list position in each half, 0xff: not in that list
    int slot;                      // the entry's (splat, tile) pair slot, -1: nothing to flush; in the
                                   // deferred walk with depth terms, the splat's depth (float bits), the
                                   // pair slot then staying in the staging thread's register
};

// Per-pixel inputs of the backward's depth terms (distortion, median depth).
struct DepthIn {
    const float* depths;      // [n]
    const float4* totals;     // [H][W]: A, B, C about the median depth, D (distortion)
    const int* median_pos;    // [H][W]: median list position + 1, 0: none
    const float* g_dist;      // [H][W]: dL/dD
    const float* g_med;       // [H][W]: dL/dmedian
};
static_assert(sizeof(StoreSlot) == 48 && offsetof(StoreSlot, pos) == 36, "StoreSlot layout");

constexpr int kBatch = kBlock - 1;                                    // entries staged per batch, at most
constexpr int kDummy = kBlock - 1;                                    // slot of the dummy entry
constexpr int kListLen = kBlock + 4;  // list row: up to 255 entries, then dummies read ahead of use

// Partial sums: one record of kRaw (or kRaw - 1 without the weight) floats per
// (half, list position) walked in a batch, written once with plain stores.
// Half q's records start at the sum of the lengths of the lists before it. A
// batch keeps as many of its candidate entries (from the top: the walk runs
// backwards) as fit: on the 2M-splat scene a 255-entry batch holds a median
// of about 340 half-list entries.
template <bool AW> struct BwdParts {
    static constexpr int kF = AW ? kRaw : kRaw - 1;  // floats per record
    static constexpr int kCap = AW ? 453 : 503;      // records per batch (at most 26 KB of LDS in all: six workgroups per CU)
};

// The deferred walk: per (half list, position) records like the stored-partials
// walk, of the same batch size, at four workgroups per CU (its per-wave pads
// take 16 KB): 40 KB of LDS in all.
// NB: entries staged per batch (NB + 1 slots, the last the dummy); KC: lockstep
// steps between two deferred reductions; WG: workgroups per CU the LDS is
// sized for. The partial records take what the slots, lists and per-wave
// pads leave of 160 KB / WG.
// DEP: the depth terms (bit 0 distortion, bit 1 median), one more record
// field (the depth gradient) and a per-wave pad of one float per lane and step.
template <bool AW, int NB, int KC, int WG, int DEP = 0> struct DeferShape {
    static constexpr int kF = (AW ? kRaw : kRaw - 1) + (DEP ? 1 : 0);
    static constexpr int kZ = AW ? kRaw : kRaw - 1;  // the depth gradient's field (DEP)
    static constexpr int kSlots = NB + 1;
    static constexpr int kListLen = NB + 5;  // up to NB entries, then dummies read ahead of use
    static constexpr unsigned short kDummyOff = (unsigned short)(NB * sizeof(StoreSlot));
    static constexpr int kFixed = kSlots * (int)sizeof(StoreSlot) + kHalves * kListLen * 2 + 4 * KC * 64 * 8 +
                                  (DEP ? 4 * KC * 64 * 4 : 4) + 2 * 4 * (kHalves + 1) * 4 + 2 * kHalves * 4 + 4 * 4 + 4;
    static constexpr int kCap = ((160 * 1024) / WG - kFixed - 256) / (kF * 4);
    static_assert(kCap >= 2 * kHalves * KC, "the partial records must hold at least one chunk");
};

// The stored-partials walk stages at most 127 entries per batch (waves 0 and
// 1; slot 127 is the dummy): the records, not the slots, bound its batches
// (a 255-entry batch holds a median of ~590 half-list entries on the
// high-overlap scene), and the LDS the smaller slots free holds more records.
constexpr int kSBatch = 127;
constexpr int kSSlots = kSBatch + 1;
constexpr int kSListLen = kSBatch + 5;  // list row: up to 127 entries, then dummies read ahead of use
constexpr unsigned short kSDummyOff = (unsigned short)(kSBatch * sizeof(StoreSlot));

// Per-half lists of the staged slots whose hit bit is set, as slot byte
// offsets in descending slot order (the walk's order); each listed entry's
// position is also written into its own slot's pos bytes. The same exchange of
// per-wave counts also ORs `flag` over the workgroup, which is returned, and
// gives every half's list length (len, wave-uniform). Ends with a barrier.
// The exchange is split in two: publish_counts (each wave's per-half counts
// and flag, before a workgroup barrier) and place_lists (after it);
// build_store_lists does both.
__device__ __forceinline__ void publish_counts(const unsigned long long (&hits)[kHalves], bool flag,
                                               int (*cnt)[kHalves + 1])
{
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int mine = __ballot(flag) != 0 ? 1 : 0;  // lane kHalves: the wave's flag
#pragma unroll
    for (int q = 0; q < kHalves; ++q) {
        const int c = __popcll(hits[q]);
        mine = lane == q ? c : mine;
    }
    if (lane <= kHalves) cnt[wv][lane] = mine;
}

template <int NSlots = kSSlots, int ListLen = kSListLen>
__device__ __forceinline__ bool place_lists(const unsigned long long (&hits)[kHalves], StoreSlot* S,
                                           unsigned short (*list)[ListLen], int (*cnt)[kHalves + 1],
                                           int (&len)[kHalves])
{
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const bool any_flag = (cnt[0][kHalves] | cnt[1][kHalves] | cnt[2][kHalves] | cnt[3][kHalves]) != 0;
    // lane q: list position of this wave's lowest hit of half q, counted from
    // the front (slots of higher waves come first)
    int top = 0, tot = 0;
    if (lane < kHalves) {
        int below = 0;
        for (int w2 = 0; w2 < 4; ++w2) {
            const int c = cnt[w2][lane];
            tot += c;
            below += w2 < wv ? c : 0;
        }
        top = tot - 1 - below;
    }
    if (threadIdx.x < NSlots) *reinterpret_cast<uint2*>(S[threadIdx.x].pos) = make_uint2(0xffffffffu, 0xffffffffu);
#pragma unroll
    for (int q = 0; q < kHalves; ++q) {
        len[q] = __builtin_amdgcn_readlane(tot, q);
        const unsigned long long bal = hits[q];
        if (__builtin_amdgcn_inverse_ballot_w64(bal)) {
            const int rank = (int)__builtin_amdgcn_mbcnt_hi((unsigned)(bal >> 32),
                                                            __builtin_amdgcn_mbcnt_lo((unsigned)bal, 0u));
            const int at = __builtin_amdgcn_readlane(top, q) - rank;
            list[q][at] = (unsigned short)(threadIdx.x * sizeof(StoreSlot));
            S[threadIdx.x].pos[q] = (unsigned char)at;  // after the 0xff fill: the same thread, in order
        }
    }
    __syncthreads();
    return any_flag;
}

template <int NSlots = kSSlots, int ListLen = kSListLen>
__device__ __forceinline__ bool build_store_lists(const unsigned long long (&hits)[kHalves], bool flag, StoreSlot* S,
                                                 unsigned short (*list)[ListLen], int (*cnt)[kHalves + 1],
                                                 int (&len)[kHalves])
{
    publish_counts(hits, flag, cnt);
    __syncthreads();
    return place_lists<NSlots, ListLen>(hits, S, list, cnt, len);
}

// Six waves per SIMD: the LDS allows six workgroups per CU, and the walk's
// registers fit 80 VGPRs.
template <bool AW>
__global__ __launch_bounds__(kBlock, 6) void bwd_store_kernel(
    int W, int H, int GX, int GY, int tiles, int n, const int2* __restrict__ ranges, const int* __restrict__ ids,
    const SplatRec* __restrict__ recs, const int* __restrict__ splat_offsets, long long n_isect, long long n_slots,
    const float* __restrict__ bg, const float* __restrict__ final_T, const int* __restrict__ n_contrib,
    const float* __restrict__ dimg, const int* __restrict__ order, float4* __restrict__ rec_out,
    unsigned char* __restrict__ slot_used)
{
    using PP = BwdParts<AW>;
    constexpr int kF = PP::kF, kCap = PP::kCap;
    __shared__ StoreSlot S[kSSlots];
    __shared__ float parts[kCap * kF];
    __shared__ unsigned short list[kHalves][kSListLen];  // per half: slots that may touch it, then dummies
    __shared__ int list_cnt[4][kHalves + 1];           // [staging wave][half], then the wave's clamp flag
    __shared__ int half_end[kHalves];
    __shared__ int half_base[kHalves];                 // first partial record of each half, for the flush
    __shared__ int wave_hits[4];                       // half-list entries of each wave's candidates
    __shared__ int cut;                                // lowest kept candidate of the batch

    const int tile = order ? order[blockIdx.x] : xcd_tile(blockIdx.x, tiles);
    if (tile < 0 || tile >= tiles) return;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int half = lane >> 5, hq = 2 * wv + half;
    int x, y;
    quadrant_pixel(tile, GX, x, y);
    const bool inside = x < W && y < H;
    const float px = (float)x + 0.5f, py = (float)y + 0.5f;
    const float ox = (float)((tile % GX) * kTile) + 0.5f, oy = (float)((tile / GX) * kTile) + 0.5f;
    const int2 rg = clamp_range(ranges[tile], n_isect);  // a range past the pair list reads nothing wild

    float T = 1.0f, g0 = 0.0f, g1 = 0.0f, g2 = 0.0f;
    int nc = 0;
    if (inside) {
        const int p = y * W + x;  // < 2^30: the HWC offset 3 p fits 32 unsigned bits
        T = final_T[p];
        // never walk past the tile's list, whatever n_contrib holds
        nc = min(max(n_contrib[p], 0), rg.y - rg.x);
        g0 = dimg[3u * (unsigned)p + 0];
        g1 = dimg[3u * (unsigned)p + 1];
        g2 = dimg[3u * (unsigned)p + 2];
    }
    // Colour "behind" the current splat (normalised by the transmittance after
    // it; the background at the start), carried only as its dot product with
    // the pixel's colour gradient
    float Bg = 0.0f;
    if (bg) Bg = __builtin_fmaf(bg[0], g0, __builtin_fmaf(bg[1], g1, bg[2] * g2));

    int hmax = nc;  // largest n_contrib of this half (32 lanes)
    for (int off = 16; off > 0; off >>= 1) hmax = max(hmax, __shfl_xor(hmax, off, 64));
    if ((lane & 31) == 0) half_end[hq] = hmax;
    if (threadIdx.x == 0) {  // the dummy entry: opacity 0, reaches no pixel
        S[kSBatch].a = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        S[kSBatch].b = make_float4(0.0f, -__builtin_inff(), 0.0f, 0.0f);
        S[kSBatch].c = 0.0f;
    }
    __syncthreads();
    int hend[kHalves];  // walk end of every half, wave-uniform
    int tmax = 0;
#pragma unroll
    for (int q = 0; q < kHalves; ++q) {
        hend[q] = __builtin_amdgcn_readfirstlane(half_end[q]);
        tmax = max(tmax, hend[q]);
    }
    if (tmax == 0) return;

    // Leaders of the merged reduction, which store the totals: one lane per
    // 4-lane bank of W (bank b of row r holds field 2 k + (r & 1),
    // k = 0, 2, 1, 3 for b = 0..3) and, for the fields 8, 9, one lane per
    // half (lane 16; its row holds the half's field 8 once the two rows are
    // added) or, with the weight, one per row.
    const int odd = (lane >> 4) & 1;
    const bool bank_lead = (lane & 3) == 0, row_lead = (lane & 15) == 0;
    const int w_field = 2 * ((0x3120 >> (4 * ((lane >> 2) & 3))) & 3) + odd;  // a bank leader's field
    const int z_field = AW ? 8 + odd : 8;                                     // a row leader's field
    // wave masks of the leaders, so that a step can switch off those of a half
    // whose list is exhausted on scalar registers
    const unsigned long long bank_mask = __ballot(bank_lead);
    const unsigned long long row_mask = __ballot(AW ? row_lead : (lane & 31) == 16);

    // No barrier at the top of a batch: thread t flushes slot t and then stages
    // slot t itself, and the barrier after the walk already separates the
    // walk's reads of the slots and lists from their rewriting; the partial
    // records are cleared only after the next barrier.
    int hi = tmax;  // the batches cover [0, tmax) from the top down
    while (hi > 0) {
        const int lo = max(0, hi - kSBatch);  // candidates [lo, hi): entry lo + t in slot t
        const int k = lo + (int)threadIdx.x;
        const bool cand = (int)threadIdx.x < kSBatch && k < hi;
        int id = -1, radius = 0;
        SplatRec r;
        r.a = r.b = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        r.c = make_float4(0.0f, -1.0f, 0.0f, 0.0f);  // no entry: reaches nothing
        if (cand) id = ids[rg.x + k];
        if ((unsigned)id >= (unsigned)n) id = -1;  // an id outside [0, n) is no entry
        if (id >= 0) {
            r = recs[id];
            radius = __float_as_int(r.c.z);
            S[threadIdx.x].a = r.a;
            S[threadIdx.x].b = r.b;
            S[threadIdx.x].c = r.c.x;
        }
        unsigned long long hits[kHalves] = {0, 0, 0, 0, 0, 0, 0, 0};
        if (threadIdx.x < kSSlots) half_hits(r, ox, oy, k, hend, hits);  // waves 0, 1: the candidates' waves
        // Keep the top candidates whose half-list entries fit the partial
        // records: suffix sums of the hit counts over the slots, from the top.
        int hc = 0;
#pragma unroll
        for (int q = 0; q < kHalves; ++q) hc += __builtin_amdgcn_inverse_ballot_w64(hits[q]) ? 1 : 0;
        int suf = hc;  // inclusive suffix sum inside the wave (higher lanes)
        for (int off = 1; off < kWave; off <<= 1) {
            const int u = __shfl_down(suf, off, kWave);
            if (lane + off < kWave) suf += u;
        }
        if (lane == 0) wave_hits[wv] = suf;
        if (threadIdx.x == 0) cut = kSBatch;
        __syncthreads();
        for (int w2 = wv + 1; w2 < 4; ++w2) suf += wave_hits[w2];
        const bool keep = cand && suf <= kCap;  // monotone: every slot above a kept one is kept
        const unsigned long long kb = __ballot(keep);
        if (kb != 0 && lane == 0) atomicMin(&cut, (int)threadIdx.x + __builtin_ctzll(kb));
#pragma unroll
        for (int q = 0; q < kHalves; ++q) hits[q] &= kb;
        // The entry's pair slot: the splat's first slot (from its record) plus
        // the tile's row-major index inside the splat's tile rectangle
        // (recomputed from mean and radius with the binning's float32 rule).
        // The tile lies in the rectangle whenever the inputs come from one
        // binning; anything else gets no slot and is never written wild.
        {
            int slot = -1;
            if (keep && id >= 0) {
                int tx0, tx1, ty0, ty1;
                tile_rect(r.a.x, r.a.y, radius, GX, GY, tx0, tx1, ty0, ty1);
                const int tx = tile % GX, ty = tile / GX;
                const long long sl =
                    (long long)__float_as_int(r.c.w) + (long long)(ty - ty0) * (tx1 - tx0) + (tx - tx0);
                if (tx >= tx0 && tx < tx1 && ty >= ty0 && ty < ty1 && sl >= 0 && sl < n_slots) slot = (int)sl;
            }
            if (threadIdx.x < kSSlots) S[threadIdx.x].slot = slot;  // thread t's own slot; the walk does not read it
        }
        // Can any entry of the batch reach the 0.99 clamp? alpha_raw's
        // exponent never exceeds log2 o, so alpha_raw never exceeds
        // exp2(log2 o) (the same monotone v_exp_f32): an entry with exp2(log2 o) clearly below
        // 0.99 never clamps. Most batches have none, and their walk skips the
        // clamp's three instructions per step.
        const bool may_clamp = keep && id >= 0 && !(__builtin_amdgcn_exp2f(r.b.y) < kAlphaMax * (1.0f - 0x1p-20f));
        int len[kHalves];
        const bool clamp_batch = build_store_lists(hits, may_clamp, S, list, list_cnt, len);
        int base[kHalves];  // first partial record of each half
        base[0] = 0;
#pragma unroll
        for (int q = 1; q < kHalves; ++q) base[q] = base[q - 1] + len[q - 1];
        const int next_hi = lo + cut;
        // the wave's two list lengths and first records (wave-uniform selects
        // over the unrolled halves: no indexing of the register arrays by the
        // wave number), then this lane's half
        const int wvu = __builtin_amdgcn_readfirstlane(wv);
        int len_a = 0, len_b = 0, base_a = 0, base_b = 0;
#pragma unroll
        for (int q = 0; q < kHalves; q += 2) {
            len_a = q == 2 * wvu ? len[q] : len_a;
            len_b = q == 2 * wvu ? len[q + 1] : len_b;
            base_a = q == 2 * wvu ? base[q] : base_a;
            base_b = q == 2 * wvu ? base[q + 1] : base_b;
        }
        const int my_len = half ? len_b : len_a, len_other = half ? len_a : len_b;
        const int my_base = half ? base_b : base_a;
        // the bases wait in LDS for the flush (past the barrier after the walk)
        // rather than in registers through the walk
        if (threadIdx.x == 0) {
#pragma unroll
            for (int q = 0; q < kHalves; ++q) half_base[q] = base[q];
        }
        // the same for both halves: wave-uniform, so the loop runs on scalar control
        const int steps = __builtin_amdgcn_readfirstlane(max(my_len, len_other));
        // the shorter half takes the dummy entry once its list is exhausted
        // (and both read up to four entries past the end, ahead of use)
        for (int p = my_len + (lane & 31); p < steps + 4; p += 32) list[hq][p] = kSDummyOff;
        // batch slots below this pixel's walk end, as a byte offset bound
        const int ncb_off = (nc - lo) * (int)sizeof(StoreSlot);
        const unsigned short* L = list[hq];
        const char* Sb = reinterpret_cast<const char*>(S);
        // a leader's partial record fields for step 0 of its half; step j adds j records
        // (lanes 0 and 16 of a half lead both a bank and a row: two fields)
        float* const rec0 = parts + my_base * kF;

        // A step's alpha does not depend on the previous step, so the next
        // entry's record is read one step ahead and its list entry two steps
        // ahead: their LDS reads leave the chain of dependent instructions.
        // Two register sets take turns (the loop is unrolled by two), so the
        // read-ahead costs no register copies.
        auto rec_at = [&](int o) -> const StoreSlot& { return *reinterpret_cast<const StoreSlot*>(Sb + o); };
        auto list_at = [&](int i) -> int { return L[i]; };
        auto step = [&](const float4& A, const float4& Bq, float Cb, int cur, int j, auto clamp_tag) {
            constexpr bool kClamp = decltype(clamp_tag)::value;
            const AlphaCoef kf{A.x, A.y, A.z, A.w, Bq.x, Bq.y};
            float dx, dy;
            const float ar = alpha_raw(kf, px, py, dx, dy);
            const float al = kClamp ? fminf(kAlphaMax, ar) : ar;
            // contributing lanes (position below n_contrib, alpha >= 1/255) as
            // a wave mask built from the two compares, which keeps the
            // per-half tests below on scalar registers
            const unsigned long long bal = __builtin_amdgcn_fcmpf(al, kAlphaMin, 3 /* ordered >= */) &
                                           __builtin_amdgcn_sicmp(cur, ncb_off, 40 /* signed < */);
            const bool contrib = __builtin_amdgcn_inverse_ballot_w64(bal);
            // colour . gradient ahead of the test, so that the colour loads
            // issue with the rest of the record
            float cg = __builtin_fmaf(Bq.z, g0, __builtin_fmaf(Bq.w, g1, Cb * g2));
            asm volatile("" : "+v"(cg));  // not sunk into the branch below
            // Every listed (half, position) record is written, zeros included:
            // the records need no clearing. The dummy positions past a
            // half's list write nothing.
            const unsigned long long valid = (j < len_a ? 0x00000000ffffffffull : 0ull) |
                                             (j < len_b ? 0xffffffff00000000ull : 0ull);
            float* const rec = rec0 + j * kF;
            if (bal == 0) {
                if (__builtin_amdgcn_inverse_ballot_w64(bank_mask & valid)) rec[w_field] = 0.0f;
                if (__builtin_amdgcn_inverse_ballot_w64(row_mask & valid)) rec[z_field] = 0.0f;
                return;
            }

            const float ae = contrib ? al : 0.0f;   // non-contributing lanes: no-op update
            const float Ti = T * __builtin_amdgcn_rcpf(1.0f - ae);
            // dL/dalpha = T_i (c - colour behind) . g needs the colour behind
            // only through its dot product with the pixel's colour gradient,
            // which follows the same recurrence as the colour itself; then
            // s = dL/dsigma = alpha dL/dalpha = w (c - behind) . g
            const float eg = cg - Bg;
            Bg = __builtin_fmaf(ae, eg, Bg);
            T = Ti;
            const float w = ae * Ti;
            const float s = (!kClamp || ar < kAlphaMax) ? w * eg : 0.0f;  // clamped alpha: no sigma path
            // all values first, then the folds (no value is read after its
            // register has been swapped)
            const float sdx = s * dx, sdy = s * dy;
            const float f0 = w * g0, f1 = w * g1, f2 = w * g2;
            const float f6 = sdx * dx, f7 = sdx * dy;
            float f8 = sdy * dy;
            // a plain product: left alone, the compiler fuses it into the first
            // DPP add as mov + DPP mov + fma, and copies sdy around the swaps
            asm volatile("" : "+v"(f8));
            // Fold rows (0, 1) and (2, 3): register R_k row r then holds field
            // 2k + (r & 1) of half r >> 1, summed over its two rows.
            const float r0 = fold16(f0, f1);
            const float r1 = fold16(f2, s);
            const float r2 = fold16(sdx, sdy);
            const float r3 = fold16(f6, f7);
            // Inside each row: merge pairs of registers while halving the
            // lanes each partial covers (8 -> 4 -> 1 lanes): W's 4-lane bank b
            // ends with the total of R_{0,2,1,3}[b].
            const float wq = merge_half_mirror(merge_ror8(r0, r1), merge_ror8(r2, r3));
            float wt = dpp_add_quad_xor1(dpp_add_quad_xor2(wq));
            // field 8 (and the weight): folded with the weight when it is
            // wanted (rows 0 and 2 then hold field 8, rows 1 and 3 the
            // weight), else summed per row and the two rows of each half
            // added in registers
            float zt = AW ? fold16(f8, w) : f8;
            zt = dpp_add_quad_xor1(dpp_add_quad_xor2(dpp_add_half_mirror(dpp_add_ror8(zt))));
            if (!AW) zt = dpp_add_prev_row_odd(zt);
            // keep the last fused DPP adds here rather than under the leader masks
            asm volatile("" : "+v"(wt), "+v"(zt));
            // The (half, position) record is this step's alone: plain stores
            // (a half with no contributing lane stores its exact zeros).
            if (__builtin_amdgcn_inverse_ballot_w64(bank_mask & valid)) rec[w_field] = wt;
            if (__builtin_amdgcn_inverse_ballot_w64(row_mask & valid)) rec[z_field] = zt;
        };
        auto walk = [&](auto clamp_tag) {
            int o0 = list_at(0), o1 = list_at(1), on0 = list_at(2);
            float4 A0 = rec_at(o0).a, B0 = rec_at(o0).b;
            float C0 = rec_at(o0).c;
            for (int it = 0; it < steps; it += 2) {
                // set 1 <- position it + 1; list position it + 3
                const float4 A1 = rec_at(o1).a, B1 = rec_at(o1).b;
                const float C1 = rec_at(o1).c;
                const int on1 = list_at(it + 3);
                step(A0, B0, C0, o0, it, clamp_tag);
                if (it + 1 >= steps) break;
                // set 0 <- position it + 2; list position it + 4
                o0 = on0;
                A0 = rec_at(o0).a;
                B0 = rec_at(o0).b;
                C0 = rec_at(o0).c;
                on0 = list_at(it + 4);
                step(A1, B1, C1, o1, it + 1, clamp_tag);
                o1 = on1;
            }
        };
        if (clamp_batch)
            walk(std::true_type{});
        else
            walk(std::false_type{});
        __syncthreads();

        // Flush: thread t owns the entry it staged; its sums are those of the
        // records of the halves that listed it.
        const int slot = threadIdx.x < kSSlots ? S[threadIdx.x].slot : -1;
        if (slot >= 0) {
            const uint2 pw = *reinterpret_cast<const uint2*>(S[threadIdx.x].pos);
            float u[kRaw] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int q = 0; q < kHalves; ++q) {
                const unsigned at = ((q < 4 ? pw.x : pw.y) >> (8 * (q & 3))) & 0xffu;
                if (at != 0xffu) {
                    // 24-bit multiply (full rate; the record index is below 2^24)
                    const float* pr = parts + __mul24(half_base[q] + (int)at, kF);
#pragma unroll
                    for (int f = 0; f < kF; ++f) u[f] += pr[f];
                }
            }
            const bool any = (u[0] != 0.0f) | (u[1] != 0.0f) | (u[2] != 0.0f) | (u[3] != 0.0f) |
                             (u[4] != 0.0f) | (u[5] != 0.0f) | (u[6] != 0.0f) | (u[7] != 0.0f) |
                             (u[8] != 0.0f) | (AW && u[9] != 0.0f);
            if (any) {
                rec_out[kSlotF4 * (long long)slot + 0] = make_float4(u[0], u[1], u[2], u[3]);
                rec_out[kSlotF4 * (long long)slot + 1] = make_float4(u[4], u[5], u[6], u[7]);
                // the third part's last 8 bytes are padding, never read
                *reinterpret_cast<float2*>(rec_out + kSlotF4 * (long long)slot + 2) = make_float2(u[8], AW ? u[9] : 0.0f);
                slot_used[slot] = 1;
            }
        }
        hi = next_hi;
    }
}

// ---------------------------------------------------------------------------
// The deferred walk (the default). The same batches, half lists, (half list,
// position) records and flush as the stored-partials walk, with the per-step
// reduction taken out of the lockstep loop:
//   phase 1, every step: alpha, the contributing lanes, T and the colour
//     behind, and each lane's w = alpha T and s = dL/dsigma (zeros where it
//     does not contribute), written to the wave's pad (one float2 per lane);
//   phase 2, every KC steps: the 2 KC records of those steps (KC steps x two
//     halves) are split over the 64 lanes, 32 / KC lanes per record, each
//     lane summing KC pixels of one row of its record's half in registers
//     (sum w g_r, w g_g, w g_b, s, s k, s k^2 over its column offsets k;
//     dx = dx0 + k and dy is constant along the row), turning them into the
//     record's ten sums about the entry's mean, and the record's lanes add
//     theirs with fused DPP adds; the first lane stores the record.
// A step then costs 19 VALU instructions instead of about 50 (the
// cross-lane tree of the other walks: ~21 per step, and the LDS float adds
// of the first walk, ~25 LDS cycles each), and phase 2 about 14 per step
// (about 130 VALU per four-step chunk in all).
// The pads (KC x 64 float2 per wave) are written and read by the same wave,
// whose LDS accesses are served in order: no barrier is needed around them.
// ---------------------------------------------------------------------------
template <bool AW, int NB, int KC, int WG, int DEP>
__global__ __launch_bounds__(kBlock, WG) void bwd_defer_kernel(
    int W, int H, int GX, int GY, int tiles, int n, const int2* __restrict__ ranges, const int* __restrict__ ids,
    const SplatRec* __restrict__ recs, const int* __restrict__ splat_offsets, long long n_isect, long long n_slots,
    const float* __restrict__ bg, const float* __restrict__ final_T, const int* __restrict__ n_contrib,
    const float* __restrict__ dimg, const int* __restrict__ order, float4* __restrict__ rec_out,
    unsigned char* __restrict__ slot_used, DepthIn dz)
{
    using PP = DeferShape<AW, NB, KC, WG, DEP>;
    constexpr int kF = PP::kF, kCap = PP::kCap, kDSlots = PP::kSlots, kDListLen = PP::kListLen;
    constexpr int kZ = PP::kZ;
    constexpr unsigned short kDDummyOff = PP::kDummyOff;
    // list entries read ahead of the step that uses them (four record buffers
    // where the registers allow, two with the depth terms)
    constexpr int kAhead = DEP ? 2 : 4;
    constexpr int kLPR = 32 / KC;   // phase 2: lanes per (half, position) record
    constexpr int kPPL = KC;        // phase 2: pixels per lane (a row or part of one)
    __shared__ StoreSlot S[kDSlots];
    __shared__ float parts[kCap * kF];
    __shared__ unsigned short list[kHalves][kDListLen];  // per half: slots that may touch it, then dummies
    __shared__ int list_cnt[4][kHalves + 1];           // [staging wave][half], then the wave's clamp flag
    __shared__ int pre_cnt[4][kHalves + 1];            // the same before any cut
    __shared__ int half_end[kHalves];
    __shared__ int half_base[kHalves];                 // first partial record of each half, for the flush
    __shared__ int wave_hits[4];                       // half-list entries of each wave's candidates
    __shared__ int cut;                                // lowest kept candidate of the batch
    // per wave: each lane's (w, s) at each step of the current chunk
    __shared__ __align__(16) float2 pad[4][KC][kWave];
    // DEP: each lane's depth gradient at each step of the chunk
    __shared__ __align__(16) float padz[DEP ? 4 : 1][DEP ? KC : 1][DEP ? kWave : 1];

    const int tile = order ? order[blockIdx.x] : xcd_tile(blockIdx.x, tiles);
    if (tile < 0 || tile >= tiles) return;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int half = lane >> 5, hq = 2 * wv + half;
    int x, y;
    quadrant_pixel(tile, GX, x, y);
    const bool inside = x < W && y < H;
    const float px = (float)x + 0.5f, py = (float)y + 0.5f;
    const float ox = (float)((tile % GX) * kTile) + 0.5f, oy = (float)((tile / GX) * kTile) + 0.5f;
    const int2 rg = clamp_range(ranges[tile], n_isect);  // a range past the pair list reads nothing wild

    // the reciprocal of the transmittance after the current entry (1 / final_T
    // at the start): the walk multiplies it by (1 - alpha) and takes T before
    // the entry as its reciprocal, so rounding does not accumulate through
    // the reciprocals
    float IT = 1.0f, g0 = 0.0f, g1 = 0.0f, g2 = 0.0f;
    int nc = 0;
    // DEP: the median depth zm and list position mp; the distortion totals
    // about zm (A, -2B, C) and its upstream gD, with 2 gD A and -2 gD B; the
    // median's upstream gM; E, the distortion behind the current entry
    // (normalised by the transmittance after it, like the colour behind)
    float zm = 0.0f, dA = 0.0f, nB2 = 0.0f, dC = 0.0f, gD = 0.0f, A2g = 0.0f, mB2g = 0.0f, gM = 0.0f, E = 0.0f;
    int mp = 0;
    if (inside) {
        const int p = y * W + x;  // < 2^30: the HWC offset 3 p fits 32 unsigned bits
        IT = 1.0f / final_T[p];
        // never walk past the tile's list, whatever n_contrib holds
        nc = min(max(n_contrib[p], 0), rg.y - rg.x);
        g0 = dimg[3u * (unsigned)p + 0];
        g1 = dimg[3u * (unsigned)p + 1];
        g2 = dimg[3u * (unsigned)p + 2];
        if (DEP) {
            mp = min(max(dz.median_pos[p], 0), nc);  // the median is a composited entry
            if (mp > 0) {
                const int mid = ids[rg.x + mp - 1];
                zm = (unsigned)mid < (unsigned)n ? dz.depths[mid] : 0.0f;
            }
            if (DEP & 1) {
                const float4 t = dz.totals[p];
                gD = dz.g_dist[p];
                dA = t.x;
                nB2 = -2.0f * t.y;
                dC = t.z;
                A2g = 2.0f * gD * t.x;
                mB2g = -2.0f * gD * t.y;
            }
            if (DEP & 2) gM = dz.g_med[p];
        }
    }
    // Colour "behind" the current splat (normalised by the transmittance after
    // it; the background at the start), carried only as its dot product with
    // the pixel's colour gradient
    float Bg = 0.0f;
    if (bg) Bg = __builtin_fmaf(bg[0], g0, __builtin_fmaf(bg[1], g1, bg[2] * g2));

    int hmax = nc;  // largest n_contrib of this half (32 lanes)
    for (int off = 16; off > 0; off >>= 1) hmax = max(hmax, __shfl_xor(hmax, off, 64));
    if ((lane & 31) == 0) half_end[hq] = hmax;
    if (threadIdx.x == 0) {  // the dummy entry: opacity 0, reaches no pixel
        S[NB].a = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        S[NB].b = make_float4(0.0f, -__builtin_inff(), 0.0f, 0.0f);
        S[NB].c = 0.0f;
    }
    __syncthreads();
    int hend[kHalves];  // walk end of every half, wave-uniform
    int tmax = 0;
#pragma unroll
    for (int q = 0; q < kHalves; ++q) {
        hend[q] = __builtin_amdgcn_readfirstlane(half_end[q]);
        tmax = max(tmax, hend[q]);
    }
    if (tmax == 0) return;

    // Phase-2 role of this lane (fixed for the whole walk): for the record of
    // step lane / (2 kLPR) of each chunk, it sums kPPL consecutive pixels of
    // half h of its wave's quadrant (8 x 4 pixels, row-major: pixel u * 8 + kx
    // is lane 32 h + 8 u + kx), all in one row u, from column kx0. Their colour
    // gradients come over once through the pad.
    const int ph = (lane / kLPR) & 1, pv = lane % kLPR;
    const int pu = (pv * kPPL) >> 3, pkx0 = (pv * kPPL) & 7;
    float gr[kPPL], gg[kPPL], gb[kPPL];
    {
        float* gt = reinterpret_cast<float*>(&pad[wv][0][0]);
        gt[3 * lane + 0] = g0;
        gt[3 * lane + 1] = g1;
        gt[3 * lane + 2] = g2;
        // the LDS serves one wave's accesses in order, so the reads below see
        // the other lanes' writes; the compiler must not move them across
        asm volatile("" ::: "memory");
#pragma unroll
        for (int kx = 0; kx < kPPL; ++kx) {
            const int src = 32 * ph + 8 * pu + pkx0 + kx;
            gr[kx] = gt[3 * src + 0];
            gg[kx] = gt[3 * src + 1];
            gb[kx] = gt[3 * src + 2];
        }
        asm volatile("" ::: "memory");
    }
    // centre of this lane's first pixel (pkx0, 4 h + u) of the quadrant
    const float row_x0 = ox + (float)((wv & 1) * 8 + pkx0);
    const float row_y = oy + (float)((wv >> 1) * 8 + 4 * ph + pu);

    // No barrier at the top of a batch: thread t flushes slot t and then stages
    // slot t itself, and the barrier after the walk already separates the
    // walk's reads of the slots and lists from their rewriting; the partial
    // records are cleared only after the next barrier.
    int hi = tmax;  // the batches cover [0, tmax) from the top down
    while (hi > 0) {
        __builtin_amdgcn_s_setprio(2);  // staging and flush: their loads and stores issue first
        int my_slot = -1;  // this thread's staged entry's pair slot
        const int lo = max(0, hi - NB);  // candidates [lo, hi): entry lo + t in slot t
        const int k = lo + (int)threadIdx.x;
        const bool cand = (int)threadIdx.x < NB && k < hi;
        int id = -1, radius = 0;
        SplatRec r;
        r.a = r.b = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        r.c = make_float4(0.0f, -1.0f, 0.0f, 0.0f);  // no entry: reaches nothing
        if (cand) id = ids[rg.x + k];
        if ((unsigned)id >= (unsigned)n) id = -1;  // an id outside [0, n) is no entry
        float zent = 0.0f;  // DEP: the entry's depth (0 for no entry and the dummy)
        if (id >= 0) {
            r = recs[id];
            if (DEP) zent = dz.depths[id];
            radius = __float_as_int(r.c.z);
            S[threadIdx.x].a = r.a;
            S[threadIdx.x].b = r.b;
            S[threadIdx.x].c = r.c.x;
        }
        unsigned long long hits[kHalves] = {0, 0, 0, 0, 0, 0, 0, 0};
        if (threadIdx.x < kDSlots) half_hits(r, ox, oy, k, hend, hits);  // the candidates' waves
        // Keep the top candidates whose half-list entries fit the partial
        // records. Usually all of them do (the wave totals, from ballots, say
        // so); otherwise suffix sums of the hit counts over the slots, from
        // the top, pick the candidates that fit. The per-half counts and the
        // clamp flag as they stand when all fit go out with the wave totals,
        // so that the usual batch builds its lists after this one barrier.
        // Can an entry reach the 0.99 clamp? alpha_raw's exponent never
        // exceeds log2 o, so alpha_raw never exceeds exp2(log2 o) (the same
        // monotone v_exp_f32): an entry with exp2(log2 o) clearly below 0.99
        // never clamps. Most batches have none, and their walk skips the
        // clamp's three instructions per step.
        const bool clamps = id >= 0 && !(__builtin_amdgcn_exp2f(r.b.y) < kAlphaMax * (1.0f - 0x1p-20f));
        {
            int wtot = 0;  // this wave's half-list entries (wave-uniform)
#pragma unroll
            for (int q = 0; q < kHalves; ++q) wtot += __popcll(hits[q]);
            if (lane == 0) wave_hits[wv] = wtot;
            if (threadIdx.x == 0) cut = NB;
            publish_counts(hits, cand && clamps, pre_cnt);
        }
        __syncthreads();
        const int total = wave_hits[0] + wave_hits[1] + wave_hits[2] + wave_hits[3];
        bool keep = cand;
        if (total > kCap) {  // workgroup-uniform
            int hc = 0;
#pragma unroll
            for (int q = 0; q < kHalves; ++q) hc += __builtin_amdgcn_inverse_ballot_w64(hits[q]) ? 1 : 0;
            int suf = hc;  // inclusive suffix sum inside the wave (higher lanes)
            for (int off = 1; off < kWave; off <<= 1) {
                const int u = __shfl_down(suf, off, kWave);
                if (lane + off < kWave) suf += u;
            }
            for (int w2 = wv + 1; w2 < 4; ++w2) suf += wave_hits[w2];
            keep = cand && suf <= kCap;  // monotone: every slot above a kept one is kept
            const unsigned long long kb = __ballot(keep);
            if (kb != 0 && lane == 0) atomicMin(&cut, (int)threadIdx.x + __builtin_ctzll(kb));  // lowest kept
#pragma unroll
            for (int q = 0; q < kHalves; ++q) hits[q] &= kb;
        }
        // The entry's pair slot: the splat's first slot (from its record) plus
        // the tile's row-major index inside the splat's tile rectangle
        // (recomputed from mean and radius with the binning's float32 rule).
        // The tile lies in the rectangle whenever the inputs come from one
        // binning; anything else gets no slot and is never written wild.
        {
            int slot = -1;
            if (keep && id >= 0) {
                int tx0, tx1, ty0, ty1;
                tile_rect(r.a.x, r.a.y, radius, GX, GY, tx0, tx1, ty0, ty1);
                const int tx = tile % GX, ty = tile / GX;
                const long long sl =
                    (long long)__float_as_int(r.c.w) + (long long)(ty - ty0) * (tx1 - tx0) + (tx - tx0);
                if (tx >= tx0 && tx < tx1 && ty >= ty0 && ty < ty1 && sl >= 0 && sl < n_slots) slot = (int)sl;
            }
            // thread t's own slot; the walk does not read it (with depth terms
            // the slot word carries the depth, which the walk reads)
            if (threadIdx.x < kDSlots) S[threadIdx.x].slot = DEP ? __float_as_int(zent) : slot;
            my_slot = slot;
        }
        int len[kHalves];
        const bool clamp_batch = total > kCap  // workgroup-uniform: a cut batch exchanges its counts again
                                     ? build_store_lists<kDSlots, kDListLen>(hits, keep && clamps, S, list, list_cnt,
                                                                             len)
                                     : place_lists<kDSlots, kDListLen>(hits, S, list, pre_cnt, len);
        int base[kHalves];  // first partial record of each half
        base[0] = 0;
#pragma unroll
        for (int q = 1; q < kHalves; ++q) base[q] = base[q - 1] + len[q - 1];
        // the candidates below the lowest kept one go to the next batch (all
        // were kept when the records fit)
        const int next_hi = total > kCap ? lo + cut : lo;
        // DEP: the slot offset of this pixel's median entry when this batch
        // walks it (the kept candidates [next_hi, hi)), else -1
        const int med_off = (DEP & 2) && mp - 1 >= next_hi && mp - 1 < hi
                                ? (mp - 1 - lo) * (int)sizeof(StoreSlot) : -1;
        // the wave's two list lengths and first records (wave-uniform selects
        // over the unrolled halves: no indexing of the register arrays by the
        // wave number), then this lane's half
        const int wvu = __builtin_amdgcn_readfirstlane(wv);
        int len_a = 0, len_b = 0, base_a = 0, base_b = 0;
#pragma unroll
        for (int q = 0; q < kHalves; q += 2) {
            len_a = q == 2 * wvu ? len[q] : len_a;
            len_b = q == 2 * wvu ? len[q + 1] : len_b;
            base_a = q == 2 * wvu ? base[q] : base_a;
            base_b = q == 2 * wvu ? base[q + 1] : base_b;
        }
        const int my_len = half ? len_b : len_a, len_other = half ? len_a : len_b;
        // the bases wait in LDS for the flush (past the barrier after the walk)
        // rather than in registers through the walk
        if (threadIdx.x == 0) {
#pragma unroll
            for (int q = 0; q < kHalves; ++q) half_base[q] = base[q];
        }
        // the same for both halves: wave-uniform, so the loop runs on scalar control
        const int steps = __builtin_amdgcn_readfirstlane(max(my_len, len_other));
        // the shorter half takes the dummy entry once its list is exhausted;
        // both run a whole number of chunks (steps rounded up to KC) and read
        // two entries past that, ahead of use
        const int steps_kc = (steps + KC - 1) & ~(KC - 1);
        for (int p = my_len + (lane & 31); p < steps_kc + kAhead; p += 32) list[hq][p] = kDDummyOff;
        // batch slots below this pixel's walk end, as a byte offset bound
        const int ncb_off = (nc - lo) * (int)sizeof(StoreSlot);
        const unsigned short* L = list[hq];
        const char* Sb = reinterpret_cast<const char*>(S);
        // phase 2: this lane's record (half ph of the wave) and its first record
        const int ph_len = ph ? len_b : len_a, ph_base = ph ? base_b : base_a;
        const unsigned short* Lp = list[2 * wvu + ph];
        float2* const my_pad = &pad[wv][0][lane];
        float* const my_padz = &padz[DEP ? wv : 0][0][DEP ? lane : 0];

        auto rec_at = [&](int o) -> const StoreSlot& { return *reinterpret_cast<const StoreSlot*>(Sb + o); };
        auto z_at = [&](int o) -> float { return DEP ? __int_as_float(rec_at(o).slot) : 0.0f; };
        auto list_at = [&](int i) -> int {
            int o = L[i];
            asm("" : "+v"(o));
            return o;
        };
        // Phase 1, one lockstep step: alpha, the contributing lanes, T and the
        // colour behind recovered; the lane's w = alpha T and s = dL/dsigma go
        // to the pad (zeros where it does not contribute).
        auto step = [&](const float4& A, const float4& Bq, float Cb, float Zc, int cur, int j, auto clamp_tag) {
            constexpr bool kClamp = decltype(clamp_tag)::value;
            const AlphaCoef kf{A.x, A.y, A.z, A.w, Bq.x, Bq.y};
            float dx, dy;
            const float ar = alpha_raw(kf, px, py, dx, dy);
            const float al = kClamp ? fminf(kAlphaMax, ar) : ar;
            const unsigned long long bal = __builtin_amdgcn_fcmpf(al, kAlphaMin, 3 /* ordered >= */) &
                                           __builtin_amdgcn_sicmp(cur, ncb_off, 40 /* signed < */);
            const bool contrib = __builtin_amdgcn_inverse_ballot_w64(bal);
            // (colour - colour behind) . dL/dC
            const float eg = __builtin_fmaf(Bq.z, g0, __builtin_fmaf(Bq.w, g1, __builtin_fmaf(Cb, g2, -Bg)));
            // no branch on "no lane contributes" (a few percent of the steps):
            // those lanes' updates are exact no-ops (alpha 0: 1 / T, the colour
            // behind and w, s unchanged or zero)
            const float ae = contrib ? al : 0.0f;   // non-contributing lanes: no-op update
            IT = __builtin_fmaf(-ae, IT, IT);       // 1 / T before the entry
            const float Ti = __builtin_amdgcn_rcpf(IT);
            Bg = __builtin_fmaf(ae, eg, Bg);
            const float w = ae * Ti;
            float egt = eg;  // dL/dalpha / T
            if (DEP) {
                const float u = Zc - zm;
                float vz = 0.0f;
                if (DEP & 1) {
                    // dD/dw = u^2 A - 2 u B + C, less the distortion behind
                    const float ed = __builtin_fmaf(u, __builtin_fmaf(u, dA, nB2), dC) - E;
                    E = __builtin_fmaf(ae, ed, E);
                    egt = __builtin_fmaf(gD, ed, eg);
                    vz = w * __builtin_fmaf(u, A2g, mB2g);  // gD dD/dz = 2 gD w (u A - B)
                }
                if (DEP & 2) vz += cur == med_off ? gM : 0.0f;
                my_padz[j * kWave] = vz;
            }
            const float s = (!kClamp || ar < kAlphaMax) ? w * egt : 0.0f;  // clamped alpha: no sigma path
            my_pad[j * kWave] = make_float2(w, s);
        };
        // Phase 2, after each chunk of steps: lane (j, h, u) sums row u of
        // half h at step c + j in registers: the moments of s over the row's
        // column offsets kx = 0..7 (dx = dx0 + kx, dy constant along the row)
        // and w g; four lanes (the rows of the half) then add their totals,
        // and the first stores the (half, position) record.
        const int jr = lane / (2 * kLPR);   // phase 2: this lane's record is step c + jr of half ph
        // the mean of that record's entry (both halves' lists hold entries or
        // dummies up to the padded step count, which c + jr stays below)
        auto rec_mean = [&](int c) -> float2 {
            const int off = (int)Lp[c + jr];
            return *reinterpret_cast<const float2*>(Sb + off);
        };
        auto phase2 = [&](int c, float2 mu) {
            const int p = c + jr;
            const bool valid = p < ph_len;
            const float4* pp = reinterpret_cast<const float4*>(&pad[wv][jr][32 * ph + 8 * pu + pkx0]);
            float w_[kPPL], s_[kPPL];
#pragma unroll
            for (int i = 0; i < kPPL / 2; ++i) {
                const float4 q = pp[i];
                w_[2 * i] = q.x;
                s_[2 * i] = q.y;
                w_[2 * i + 1] = q.z;
                s_[2 * i + 1] = q.w;
            }
            // moments of s over the lane's column offsets k (dx = dx0 + k)
            float S0 = s_[0] + s_[1], Sx = s_[1], Sxx = s_[1];
            float Wr = w_[0] * gr[0], Wg = w_[0] * gg[0], Wb = w_[0] * gb[0], Wt = w_[0];
#pragma unroll
            for (int kx = 1; kx < kPPL; ++kx) {
                if (kx >= 2) {
                    S0 += s_[kx];
                    Sx = __builtin_fmaf((float)kx, s_[kx], Sx);
                    Sxx = __builtin_fmaf((float)(kx * kx), s_[kx], Sxx);
                }
                Wr = __builtin_fmaf(w_[kx], gr[kx], Wr);
                Wg = __builtin_fmaf(w_[kx], gg[kx], Wg);
                Wb = __builtin_fmaf(w_[kx], gb[kx], Wb);
                if (AW) Wt += w_[kx];
            }
            float Vz = 0.0f;  // DEP: the depth gradients of the lane's pixels
            if (DEP) {
                static_assert(DEP == 0 || kPPL % 4 == 0, "depth pad read as float4");
                const float4* pz = reinterpret_cast<const float4*>(&padz[wv][jr][32 * ph + 8 * pu + pkx0]);
#pragma unroll
                for (int i = 0; i < kPPL / 4; ++i) {
                    const float4 q = pz[i];
                    Vz += (q.x + q.y) + (q.z + q.w);
                }
            }
            const float dx0 = row_x0 - mu.x, dyr = row_y - mu.y;
            // The two lanes of each pixel row (lanes 2u, 2u + 1 of the record)
            // add their sums first; the row's dy then turns the row totals of
            // s and s dx into those of s dy, s dx dy and s dy^2, with no cross-
            // lane adds of their own.
            static_assert(kPPL == 4, "two lanes per pixel row");
            float f[kRaw + 1];
            f[0] = dpp_add_quad_xor1(Wr);
            f[1] = dpp_add_quad_xor1(Wg);
            f[2] = dpp_add_quad_xor1(Wb);
            f[3] = dpp_add_quad_xor1(S0);                                                      // sum s
            f[4] = dpp_add_quad_xor1(__builtin_fmaf(dx0, S0, Sx));                             // sum s dx
            f[6] = dpp_add_quad_xor1(__builtin_fmaf(dx0, __builtin_fmaf(dx0, S0, Sx + Sx), Sxx));  // sum s dx^2
            f[5] = dyr * f[3];                                                                   // sum s dy
            f[7] = dyr * f[4];                                                                   // sum s dx dy
            f[8] = dyr * f[5];                                                                   // sum s dy^2
            // plain products: folded into the next DPP add they would cost a
            // DPP move, a zeroing move and a fused multiply-add each
            asm volatile("" : "+v"(f[5]), "+v"(f[7]), "+v"(f[8]));
            f[9] = dpp_add_quad_xor1(AW ? Wt : Vz);
            f[10] = dpp_add_quad_xor1(Vz);  // field kZ: 9 or 10
            // then the rows: the two pairs of each quad, and (eight lanes) the
            // two quads of each 8-lane half-row
#pragma unroll
            for (int q = 0; q < kF; ++q) {
                f[q] = dpp_add_quad_xor2(f[q]);
                if (kLPR == 8) f[q] = dpp_add_half_mirror(f[q]);
                asm volatile("" : "+v"(f[q]));  // fused DPP adds, outside the store's lane mask
            }
            if (pv == 0 && valid) {
                float* rec = parts + (ph_base + p) * kF;
#pragma unroll
                for (int q = 0; q < kF; ++q) rec[q] = f[q];
            }
        };
        // Every chunk runs all KC steps (the lists hold dummies up to a whole
        // number of chunks) over kAhead record buffers, each refilled kAhead - 1
        // entries ahead of its use: the loads land where a later step reads
        // them, with no register copies.
        static_assert(KC % 2 == 0, "steps run in pairs");
        auto walk = [&](auto clamp_tag) {
            if constexpr (kAhead == 4) {
                // four record buffers: each entry's coefficients are requested
                // three steps before its use
                static_assert(KC == 4, "one rotation of the four buffers per chunk");
                int o0 = list_at(0), o1 = list_at(1), o2 = list_at(2), o3 = list_at(3);
                float4 A0 = rec_at(o0).a, B0 = rec_at(o0).b;
                float C0 = rec_at(o0).c;
                float4 A1 = rec_at(o1).a, B1 = rec_at(o1).b;
                float C1 = rec_at(o1).c;
                float4 A2 = rec_at(o2).a, B2 = rec_at(o2).b;
                float C2 = rec_at(o2).c;
                for (int c = 0; c < steps_kc; c += KC) {
                    const float2 mu = rec_mean(c);  // phase 2's, requested before the steps
                    const float4 A3 = rec_at(o3).a, B3 = rec_at(o3).b;
                    const float C3 = rec_at(o3).c;
                    const int n0 = list_at(c + 4);
                    step(A0, B0, C0, 0.0f, o0, 0, clamp_tag);
                    A0 = rec_at(n0).a;
                    B0 = rec_at(n0).b;
                    C0 = rec_at(n0).c;
                    const int n1 = list_at(c + 5);
                    step(A1, B1, C1, 0.0f, o1, 1, clamp_tag);
                    A1 = rec_at(n1).a;
                    B1 = rec_at(n1).b;
                    C1 = rec_at(n1).c;
                    const int n2 = list_at(c + 6);
                    step(A2, B2, C2, 0.0f, o2, 2, clamp_tag);
                    A2 = rec_at(n2).a;
                    B2 = rec_at(n2).b;
                    C2 = rec_at(n2).c;
                    const int n3 = list_at(c + 7);
                    step(A3, B3, C3, 0.0f, o3, 3, clamp_tag);
                    o0 = n0;
                    o1 = n1;
                    o2 = n2;
                    o3 = n3;
                    asm volatile("" ::: "memory");
                    phase2(c, mu);
                    asm volatile("" ::: "memory");
                }
                return;
            }
            int o0 = list_at(0), o1 = list_at(1);
            float4 A0 = rec_at(o0).a, B0 = rec_at(o0).b;
            float C0 = rec_at(o0).c, Z0 = z_at(o0);
            for (int c = 0; c < steps_kc; c += KC) {
#pragma unroll
                for (int j = 0; j < KC; j += 2) {
                    const int it = c + j;
                    const float4 A1 = rec_at(o1).a, B1 = rec_at(o1).b;
                    const float C1 = rec_at(o1).c, Z1 = z_at(o1);
                    const int n0 = list_at(it + 2);
                    step(A0, B0, C0, Z0, o0, j, clamp_tag);
                    A0 = rec_at(n0).a;
                    B0 = rec_at(n0).b;
                    C0 = rec_at(n0).c;
                    Z0 = z_at(n0);
                    const int n1 = list_at(it + 3);
                    step(A1, B1, C1, Z1, o1, j + 1, clamp_tag);
                    o0 = n0;
                    o1 = n1;
                }
                // the pad's rows go from the lanes that wrote them to the lanes
                // that sum them: LDS accesses of one wave are served in order, so
                // keeping the compiler from reordering them is enough
                asm volatile("" ::: "memory");
                phase2(c, rec_mean(c));
                asm volatile("" ::: "memory");
            }
        };
        __builtin_amdgcn_s_setprio(0);
        if (clamp_batch)
            walk(std::true_type{});
        else
            walk(std::false_type{});
        __builtin_amdgcn_s_setprio(2);
        __syncthreads();

        // Flush: thread t owns the entry it staged; its sums are those of the
        // records of the halves that listed it.
        const int slot = threadIdx.x < kDSlots ? (DEP ? my_slot : S[threadIdx.x].slot) : -1;
        if (slot >= 0) {
            const uint2 pw = *reinterpret_cast<const uint2*>(S[threadIdx.x].pos);
            float u[kRaw + 1] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int q = 0; q < kHalves; ++q) {
                const unsigned at = ((q < 4 ? pw.x : pw.y) >> (8 * (q & 3))) & 0xffu;
                if (at != 0xffu) {
                    // 24-bit multiply (full rate; the record index is below 2^24)
                    const float* pr = parts + __mul24(half_base[q] + (int)at, kF);
#pragma unroll
                    for (int f = 0; f < kF; ++f) u[f] += pr[f];
                }
            }
            // some sum != 0 (as a float compare: -0 counts as zero, NaN not):
            // the OR of the bit patterns without their sign bits
            unsigned bits = 0;
#pragma unroll
            for (int f = 0; f < kF; ++f) bits |= __float_as_uint(u[f]);
            if ((bits << 1) != 0u) {
                rec_out[kSlotF4 * (long long)slot + 0] = make_float4(u[0], u[1], u[2], u[3]);
                rec_out[kSlotF4 * (long long)slot + 1] = make_float4(u[4], u[5], u[6], u[7]);
                const float uw = AW ? u[9] : 0.0f;
                if (DEP)  // the depth gradient in the third part's third word
                    rec_out[kSlotF4 * (long long)slot + 2] = make_float4(u[8], uw, u[kZ], 0.0f);
                else      // the third part's last 8 bytes are padding, never read
                    *reinterpret_cast<float2*>(rec_out + kSlotF4 * (long long)slot + 2) = make_float2(u[8], uw);
                slot_used[slot] = 1;
            }
        }
        hi = next_hi;
    }
}

// LDS slot of one staged entry: its alpha coefficients and colour, and the
// partial sums the walk adds into it. One base address serves every access of
// a walk step (the lists hold slot byte offsets), so a step spends no VALU
// instruction on addressing beyond the leaders' field offset.
// The 80-byte stride is an odd multiple of 16 bytes, so the per-entry 16-byte
// accesses of staging, zeroing and flushing hit distinct banks. The weight's
// word (part[9]) is in the slot of both instances: without it the slot would
// still be 80 bytes (see the note on optional outputs at the top).
struct AddSlot {
    float4 a;           // mean x, mean y, l11, l21 (scaled factor)
    float4 b;           // l22, log2(opacity), red, green
    float part[kRaw];   // w g_r, w g_g, w g_b, s, s dx, s dy, s dx^2, s dx dy, s dy^2, [w]
    float c;            // blue
    float pad;
};
static_assert(sizeof(AddSlot) == 80 && offsetof(AddSlot, part) == 32, "AddSlot layout");

__device__ __forceinline__ float4* add_part4(AddSlot& e, int i) { return reinterpret_cast<float4*>(e.part) + i; }
constexpr unsigned short kAddDummyOff = (unsigned short)(kDummy * sizeof(AddSlot));

// Per-half lists of the staged slots whose hit bit is set, as slot byte
// offsets in descending slot order (the walk's order). The same exchange of
// per-wave counts also ORs `flag` over the workgroup, which is returned.
// Ends with a workgroup barrier.
__device__ __forceinline__ bool build_add_lists(const unsigned long long (&hits)[kHalves], bool flag,
                                                 unsigned short (*list)[kListLen], int (*cnt)[kHalves + 1])
{
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int mine = __ballot(flag) != 0 ? 1 : 0;  // lane kHalves: the wave's flag
#pragma unroll
    for (int q = 0; q < kHalves; ++q) {
        const int c = __popcll(hits[q]);
        mine = lane == q ? c : mine;
    }
    if (lane <= kHalves) cnt[wv][lane] = mine;
    __syncthreads();
    const bool any_flag = (cnt[0][kHalves] | cnt[1][kHalves] | cnt[2][kHalves] | cnt[3][kHalves]) != 0;
    // lane q: list position of this wave's lowest hit of half q, counted from
    // the front (slots of higher waves come first)
    int top = 0;
    if (lane < kHalves) {
        int tot = 0, below = 0;
        for (int w2 = 0; w2 < 4; ++w2) {
            const int c = cnt[w2][lane];
            tot += c;
            below += w2 < wv ? c : 0;
        }
        top = tot - 1 - below;
    }
#pragma unroll
    for (int q = 0; q < kHalves; ++q) {
        const unsigned long long bal = hits[q];
        if (__builtin_amdgcn_inverse_ballot_w64(bal)) {
            const int rank = (int)__builtin_amdgcn_mbcnt_hi((unsigned)(bal >> 32),
                                                            __builtin_amdgcn_mbcnt_lo((unsigned)bal, 0u));
            list[q][__builtin_amdgcn_readlane(top, q) - rank] =
                (unsigned short)(threadIdx.x * sizeof(AddSlot));
        }
    }
    __syncthreads();
    return any_flag;
}

template <bool AW>
__global__ __launch_bounds__(kBlock) void bwd_kernel(
    int W, int H, int GX, int GY, int tiles, int n, const int2* __restrict__ ranges, const int* __restrict__ ids,
    const SplatRec* __restrict__ recs, const int* __restrict__ splat_offsets, long long n_isect, long long n_slots,
    const float* __restrict__ bg, const float* __restrict__ final_T, const int* __restrict__ n_contrib,
    const float* __restrict__ dimg, const int* __restrict__ order, float4* __restrict__ rec_out,
    unsigned char* __restrict__ slot_used)
{
    __shared__ AddSlot S[kBlock];
    __shared__ int half_end[kHalves];
    __shared__ unsigned short list[kHalves][kListLen];  // per half: slots that may touch it, then dummies
    __shared__ int list_cnt[4][kHalves + 1];           // [staging wave][half], then the wave's clamp flag

    const int tile = order ? order[blockIdx.x] : xcd_tile(blockIdx.x, tiles);
    if (tile < 0 || tile >= tiles) return;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int half = lane >> 5, hq = 2 * wv + half;
    int x, y;
    quadrant_pixel(tile, GX, x, y);
    const bool inside = x < W && y < H;
    const float px = (float)x + 0.5f, py = (float)y + 0.5f;
    const float ox = (float)((tile % GX) * kTile) + 0.5f, oy = (float)((tile / GX) * kTile) + 0.5f;
    const int2 rg = clamp_range(ranges[tile], n_isect);  // a range past the pair list reads nothing wild

    float T = 1.0f, g0 = 0.0f, g1 = 0.0f, g2 = 0.0f;
    int nc = 0;
    if (inside) {
        const int p = y * W + x;  // < 2^30: the HWC offset 3 p fits 32 unsigned bits
        T = final_T[p];
        // never walk past the tile's list, whatever n_contrib holds
        nc = min(max(n_contrib[p], 0), rg.y - rg.x);
        g0 = dimg[3u * (unsigned)p + 0];
        g1 = dimg[3u * (unsigned)p + 1];
        g2 = dimg[3u * (unsigned)p + 2];
    }
    // Colour "behind" the current splat (normalised by the transmittance after
    // it; the background at the start), carried only as its dot product with
    // the pixel's colour gradient
    float Bg = 0.0f;
    if (bg) Bg = __builtin_fmaf(bg[0], g0, __builtin_fmaf(bg[1], g1, bg[2] * g2));

    int hmax = nc;  // largest n_contrib of this half (32 lanes)
    for (int off = 16; off > 0; off >>= 1) hmax = max(hmax, __shfl_xor(hmax, off, 64));
    if ((lane & 31) == 0) half_end[hq] = hmax;
    if (threadIdx.x == 0) {  // the dummy entry: opacity 0, reaches no pixel, sums stay 0
        S[kDummy].a = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        S[kDummy].b = make_float4(0.0f, -__builtin_inff(), 0.0f, 0.0f);
        S[kDummy].c = 0.0f;
    }
    __syncthreads();
    int hend[kHalves];  // walk end of every half, wave-uniform
    int tmax = 0;
#pragma unroll
    for (int q = 0; q < kHalves; ++q) {
        hend[q] = __builtin_amdgcn_readfirstlane(half_end[q]);
        tmax = max(tmax, hend[q]);
    }
    if (tmax == 0) return;

    // leaders of the merged reduction: one lane per 4-lane bank of W (bank b
    // of row r holds field 2 k + (r & 1), k = 0, 2, 1, 3 for b = 0..3) and
    // one lane per row for the fields 8, 9
    const int odd = (lane >> 4) & 1;
    const bool bank_lead = (lane & 3) == 0, row_lead = (lane & 15) == 0;
    const int w_field = 2 * ((0x3120 >> (4 * ((lane >> 2) & 3))) & 3) + odd;
    const int lead_off = (int)offsetof(AddSlot, part) + 4 * w_field;  // byte offset of the bank leader's field
    // the same as wave masks, so that a step can switch off the leaders of a
    // half with no contributing lane (an exhausted list's dummy entry, or an
    // entry that reaches none of the half's walked pixels) on scalar
    // registers: each LDS add lane costs the LDS several cycles
    const unsigned long long bank_mask = __ballot(bank_lead);
    const unsigned long long row_mask = __ballot(AW ? row_lead : (lane & 31) == 16);

    // No barrier at the top of a batch: thread t flushes slot t and then stages
    // slot t itself, and the barrier after the walk already separates the
    // walk's reads of the slots and lists from their rewriting.
    for (int bs = ((tmax - 1) / kBatch) * kBatch; bs >= 0; bs -= kBatch) {
        const int k = bs + (int)threadIdx.x;
        int id = -1, radius = 0;
        SplatRec r;
        r.a = r.b = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        r.c = make_float4(0.0f, -1.0f, 0.0f, 0.0f);  // no entry: reaches nothing
        if (threadIdx.x < kBatch && k < tmax) id = ids[rg.x + k];
        if ((unsigned)id >= (unsigned)n) id = -1;  // an id outside [0, n) is no entry
        if (id >= 0) {
            r = recs[id];
            radius = __float_as_int(r.c.z);
            S[threadIdx.x].a = r.a;
            S[threadIdx.x].b = r.b;
            S[threadIdx.x].c = r.c.x;
        }
        *add_part4(S[threadIdx.x], 0) = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        *add_part4(S[threadIdx.x], 1) = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        *reinterpret_cast<float2*>(S[threadIdx.x].part + 8) = make_float2(0.0f, 0.0f);
        unsigned long long hits[kHalves];
        half_hits(r, ox, oy, k, hend, hits);
        // Can any entry of the batch reach the 0.99 clamp? alpha_raw's
        // exponent never exceeds log2 o, so alpha_raw never exceeds
        // exp2(log2 o) (the same monotone v_exp_f32): an entry with exp2(log2 o) clearly below
        // 0.99 never clamps. Most batches have none, and their walk skips the
        // clamp's three instructions per step.
        const bool may_clamp = id >= 0 && !(__builtin_amdgcn_exp2f(r.b.y) < kAlphaMax * (1.0f - 0x1p-20f));
        const bool clamp_batch = build_add_lists(hits, may_clamp, list, list_cnt);
        // this half's list length, and the wave's step count (longer half)
        const int my_len = list_cnt[0][hq] + list_cnt[1][hq] + list_cnt[2][hq] + list_cnt[3][hq];
        const int other = hq ^ 1;
        const int len_other = list_cnt[0][other] + list_cnt[1][other] + list_cnt[2][other] + list_cnt[3][other];
        // the same for both halves: wave-uniform, so the loop runs on scalar control
        const int steps = __builtin_amdgcn_readfirstlane(max(my_len, len_other));
        // the shorter half takes the dummy entry once its list is exhausted
        // (and both read up to four entries past the end, ahead of use)
        for (int p = my_len + (lane & 31); p < steps + 4; p += 32) list[hq][p] = kAddDummyOff;
        // batch slots below this pixel's walk end, as a byte offset bound
        const int ncb_off = (nc - bs) * (int)sizeof(AddSlot);
        const unsigned short* L = list[hq];
        const char* Sb = reinterpret_cast<const char*>(S);

        // A step's alpha does not depend on the previous step, so the next
        // entry's record is read one step ahead and its list entry two steps
        // ahead: their LDS reads leave the chain of dependent instructions.
        // Two register sets take turns (the loop is unrolled by two), so the
        // read-ahead costs no register copies.
        auto rec_at = [&](int o) -> const AddSlot& { return *reinterpret_cast<const AddSlot*>(Sb + o); };
        // list entries as 32-bit values: the 16-bit load zero-extends, and
        // holding the widened value keeps the compiler from masking it again
        // at every use
        auto list_at = [&](int i) -> int {
            int o = L[i];
            asm("" : "+v"(o));
            return o;
        };
        auto step = [&](const float4& A, const float4& Bq, float Cb, int cur, auto clamp_tag) {
            constexpr bool kClamp = decltype(clamp_tag)::value;
            const AlphaCoef kf{A.x, A.y, A.z, A.w, Bq.x, Bq.y};
            float dx, dy;
            const float ar = alpha_raw(kf, px, py, dx, dy);
            const float al = kClamp ? fminf(kAlphaMax, ar) : ar;
            // contributing lanes (position below n_contrib, alpha >= 1/255) as
            // a wave mask built from the two compares, which keeps the
            // per-half tests below on scalar registers
            const unsigned long long bal = __builtin_amdgcn_fcmpf(al, kAlphaMin, 3 /* ordered >= */) &
                                           __builtin_amdgcn_sicmp(cur, ncb_off, 40 /* signed < */);
            const bool contrib = __builtin_amdgcn_inverse_ballot_w64(bal);
            // colour . gradient ahead of the test, so that the colour loads
            // issue with the rest of the record
            float cg = __builtin_fmaf(Bq.z, g0, __builtin_fmaf(Bq.w, g1, Cb * g2));
            asm volatile("" : "+v"(cg));  // not sunk into the branch below
            if (bal == 0) return;
            unsigned bal_hi = (unsigned)(bal >> 32);
            asm("" : "+s"(bal_hi));  // a 32-bit test (a 64-bit unsigned compare has no scalar form)
            const unsigned long long live = ((unsigned)bal != 0u ? 0x00000000ffffffffull : 0ull) |
                                            (bal_hi != 0u ? 0xffffffff00000000ull : 0ull);

            const float ae = contrib ? al : 0.0f;   // non-contributing lanes: no-op update
            const float Ti = T * __builtin_amdgcn_rcpf(1.0f - ae);
            // dL/dalpha = T_i (c - colour behind) . g needs the colour behind
            // only through its dot product with the pixel's colour gradient,
            // which follows the same recurrence as the colour itself; then
            // s = dL/dsigma = alpha dL/dalpha = w (c - behind) . g
            const float eg = cg - Bg;
            Bg = __builtin_fmaf(ae, eg, Bg);
            T = Ti;
            const float w = ae * Ti;
            const float s = (!kClamp || ar < kAlphaMax) ? w * eg : 0.0f;  // clamped alpha: no sigma path
            // all values first, then the folds (no value is read after its
            // register has been swapped)
            const float sdx = s * dx, sdy = s * dy;
            const float f0 = w * g0, f1 = w * g1, f2 = w * g2;
            const float f6 = sdx * dx, f7 = sdx * dy;
            float f8 = sdy * dy;
            // a plain product: left alone, the compiler fuses it into the first
            // DPP add as mov + DPP mov + fma, and copies sdy around the swaps
            asm volatile("" : "+v"(f8));
            // Fold rows (0, 1) and (2, 3): register R_k row r then holds field
            // 2k + (r & 1) of half r >> 1, summed over its two rows.
            const float r0 = fold16(f0, f1);
            const float r1 = fold16(f2, s);
            const float r2 = fold16(sdx, sdy);
            const float r3 = fold16(f6, f7);
            // Inside each row: merge pairs of registers while halving the
            // lanes each partial covers (8 -> 4 -> 1 lanes): W's 4-lane bank b
            // ends with the total of R_{0,2,1,3}[b]. (Leaving the last two
            // levels to the LDS, with four lanes adding into one address, is
            // far slower: same-address LDS float adds serialize.)
            const float wq = merge_half_mirror(merge_ror8(r0, r1), merge_ror8(r2, r3));
            float wt = dpp_add_quad_xor1(dpp_add_quad_xor2(wq));
            // field 8 (and the weight): folded with the weight when it is
            // wanted (rows 0 and 2 then hold field 8, rows 1 and 3 the
            // weight), else summed per row and the two rows of each half
            // added in registers (so that no two lanes add into one address:
            // same-address LDS adds serialize)
            float zt = AW ? fold16(f8, w) : f8;
            zt = dpp_add_quad_xor1(dpp_add_quad_xor2(dpp_add_half_mirror(dpp_add_ror8(zt))));
            if (!AW) zt = dpp_add_prev_row_odd(zt);
            // keep the last fused DPP adds here rather than under the leader masks
            asm volatile("" : "+v"(wt), "+v"(zt));
            char* P = const_cast<char*>(Sb) + cur;
            if (__builtin_amdgcn_inverse_ballot_w64(bank_mask & live))
                atomicAdd(reinterpret_cast<float*>(P + lead_off), wt);
            if (__builtin_amdgcn_inverse_ballot_w64(row_mask & live))
                atomicAdd(reinterpret_cast<float*>(P + offsetof(AddSlot, part)) + (AW ? 8 + odd : 8), zt);
        };
        auto walk = [&](auto clamp_tag) {
            int o0 = list_at(0), o1 = list_at(1), on0 = list_at(2);
            float4 A0 = rec_at(o0).a, B0 = rec_at(o0).b;
            float C0 = rec_at(o0).c;
            for (int it = 0; it < steps; it += 2) {
                // set 1 <- position it + 1; list position it + 3
                const float4 A1 = rec_at(o1).a, B1 = rec_at(o1).b;
                const float C1 = rec_at(o1).c;
                const int on1 = list_at(it + 3);
                step(A0, B0, C0, o0, clamp_tag);
                if (it + 1 >= steps) break;
                // set 0 <- position it + 2; list position it + 4
                o0 = on0;
                A0 = rec_at(o0).a;
                B0 = rec_at(o0).b;
                C0 = rec_at(o0).c;
                on0 = list_at(it + 4);
                step(A1, B1, C1, o1, clamp_tag);
                o1 = on1;
            }
        };
        if (clamp_batch)
            walk(std::true_type{});
        else
            walk(std::false_type{});
        __syncthreads();

        // Flush: thread t owns the entry it staged.
        if (id >= 0) {
            const float4 P0 = *add_part4(S[threadIdx.x], 0), P1 = *add_part4(S[threadIdx.x], 1);
            const float2 P2 = *reinterpret_cast<const float2*>(S[threadIdx.x].part + 8);
            const float Swr = P0.x, Swg = P0.y, Swb = P0.z, Ss = P0.w, Sdx = P1.x, Sdy = P1.y;
            const float Sdxx = P1.z, Sdxy = P1.w, Sdyy = P2.x;
            const float Sw = AW ? P2.y : 0.0f;
            const bool any = (Swr != 0.0f) | (Swg != 0.0f) | (Swb != 0.0f) | (Ss != 0.0f) |
                             (Sdx != 0.0f) | (Sdy != 0.0f) | (Sdxx != 0.0f) | (Sdxy != 0.0f) |
                             (Sdyy != 0.0f) | (Sw != 0.0f);
            if (any) {
                int tx0, tx1, ty0, ty1;
                tile_rect(r.a.x, r.a.y, radius, GX, GY, tx0, tx1, ty0, ty1);
                const int tx = tile % GX, ty = tile / GX;
                // the splat's first slot travels in its record
                const long long slot =
                    (long long)__float_as_int(r.c.w) + (long long)(ty - ty0) * (tx1 - tx0) + (tx - tx0);
                // the tile lies in the splat's rectangle whenever the inputs come
                // from one binning; anything else is dropped, never written wild
                if (tx >= tx0 && tx < tx1 && ty >= ty0 && ty < ty1 && slot >= 0 && slot < n_slots) {
                    rec_out[kSlotF4 * slot + 0] = make_float4(Swr, Swg, Swb, Ss);
                    rec_out[kSlotF4 * slot + 1] = make_float4(Sdx, Sdy, Sdxx, Sdxy);
                    // the third part's last 8 bytes are padding, never read
                    *reinterpret_cast<float2*>(rec_out + kSlotF4 * slot + 2) = make_float2(Sdyy, Sw);
                    slot_used[slot] = 1;
                }
            }
        }
    }
}

// Zero fill (the max-weight output, raised by atomic max from 0).
__global__ __launch_bounds__(256) void zero_u32_kernel(unsigned* __restrict__ p, int n)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

// ---------------------------------------------------------------------------
// Forward
//
// The same half-wave walk as the backward, front to back: per batch of 255
// list entries, thread t stages entry t's record in a 48-byte LDS slot and
// tests it against the 8x4 halves whose pixels have not all stopped; ballots
// build one list per half (slot byte offsets, ascending: the walk's order),
// the shorter list of a wave padded with a dummy entry of opacity 0. A wave
// walks both of its lists in lockstep, the next record read one step ahead,
// and leaves the batch once its 64 pixels have stopped; the workgroup stops
// when all 256 have.
//
// Optional per-splat max weight (MW): the largest alpha T a splat receives
// over the pixels that composite it. After each pair of steps, each half's
// largest weight of either step (DPP max over its 32 lanes, the two steps'
// chains interleaved) is stored by one lane per half into a record of its own
// per (half, list position), cleared at every batch; after the batch, thread
// t takes the max over the records of the halves that listed its entry (the
// positions kept in its slot) and raises the splat's global maximum with one
// integer atomic max. Weights are >= 0, so the order of their float32 bit
// patterns is the order of their values, and a max is the same in any order:
// the result does not depend on scheduling.
//
// Optional depth outputs (DEP: 0 none, 1 the median, 2 the median and the
// distortion totals). The median entry of a pixel is the last composited
// entry whose transmittance before it is > 1/2; since T only falls, a lane
// keeps the latest such entry and its depth. The totals A = sum w, B = sum w u,
// C = sum w u^2 (u = z - reference) are summed about the depth of the current
// median candidate: each new candidate moves them to its own depth (B' = B -
// d A, C' = C - d (B + B'), d = new - old reference), which happens only while
// T > 1/2, i.e. over a pixel's first few composited entries, while the sums
// are still small; every later entry is summed about the final median, so
// the rounding error stays relative to the moments about the median rather
// than about a distant depth. The distortion is D = A C - B^2: half the double
// sum of w_i w_j (z_i - z_j)^2 over all pairs, i.e. the sum over pairs i < j.
// ---------------------------------------------------------------------------
struct FwdSlot {
    float4 a;       // mean x, mean y, l11, l21 (scaled factor)
    float4 b;       // l22, log2(opacity), red, green
    float c;        // blue
    float z;        // depth (depth outputs only)
    unsigned char pos[kHalves];  // list position in each half, 0xff: not listed (MW only)
};
static_assert(sizeof(FwdSlot) == 48 && offsetof(FwdSlot, pos) == 40, "FwdSlot layout");

template <bool MW, int DEP>
__global__ __launch_bounds__(kBlock) void fwd_kernel(int n, int W, int H, int GX, int tiles,
                                                     const int2* __restrict__ ranges, long long n_pairs,
                                                     const int* __restrict__ ids,
                                                     const SplatRec* __restrict__ recs,
                                                     const float* __restrict__ bg, float* __restrict__ image,
                                                     float* __restrict__ final_T, int* __restrict__ n_contrib,
                                                     unsigned* __restrict__ max_weight, float4* __restrict__ dist_totals,
                                                     float* __restrict__ median_depth, int* __restrict__ median_pos)
{
    __shared__ FwdSlot S[kBlock];
    __shared__ unsigned short list[kHalves][kListLen];  // per half: slots that may touch it, then dummies
    __shared__ int list_cnt[4][kHalves + 1];
    __shared__ int half_live[kHalves];
    // MW: largest weight per (half, list position), float bits; 0: none
    __shared__ __align__(16) unsigned mw_rec[MW ? kHalves : 1][MW ? kBlock : 4];
    const int tile = xcd_tile(blockIdx.x, tiles);
    if (tile >= tiles) return;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int half = lane >> 5, hq = 2 * wv + half;
    int x, y;
    quadrant_pixel(tile, GX, x, y);
    const bool inside = x < W && y < H;
    const float px = (float)x + 0.5f, py = (float)y + 0.5f;
    const float ox = (float)((tile % GX) * kTile) + 0.5f, oy = (float)((tile / GX) * kTile) + 0.5f;
    const int2 rg = clamp_range(ranges[tile], n_pairs);  // a range past the pair list reads nothing wild
    if (threadIdx.x == 0) {  // the dummy entry: opacity 0, reaches no pixel
        S[kDummy].a = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        S[kDummy].b = make_float4(0.0f, -__builtin_inff(), 0.0f, 0.0f);
        S[kDummy].c = 0.0f;
        S[kDummy].z = 0.0f;  // every lane reads it (weight 0 times a finite depth)
    }
    constexpr unsigned short kDummyFwd = (unsigned short)(kDummy * sizeof(FwdSlot));
    const char* Sb = reinterpret_cast<const char*>(S);
    auto rec_at = [&](int o) -> const FwdSlot& { return *reinterpret_cast<const FwdSlot*>(Sb + o); };

    float T = 1.0f, C0 = 0.0f, C1 = 0.0f, C2 = 0.0f;
    int last_n = 0;  // list position of the last composited entry, plus one
    // DEP: the median entry's list position plus one, and depth; the totals
    float zmed = 0.0f, zmed_ref = 0.0f, Aw = 0.0f, Bw = 0.0f, Cw = 0.0f;
    int med_n = 0;
    // the wave's stopped pixels (and those outside the image), as a lane mask:
    // the walk's tests then build their masks with compare instructions alone
    unsigned long long done_m = __ballot(!inside);
    for (int bs = rg.x; bs < rg.y; bs += kBatch) {
        __builtin_amdgcn_s_setprio(2);  // staging: its loads issue first
        // halves with a pixel still compositing; the tile stops when none is left
        const bool half_alive = ~done_m & (half ? 0xffffffff00000000ull : 0xffffffffull);
        if ((lane & 31) == 0) half_live[hq] = half_alive ? 1 : 0;
        if (__syncthreads_count(__builtin_amdgcn_inverse_ballot_w64(done_m)) == kBlock)
            break;  // every pixel of the tile has stopped
        int hend[kHalves];  // halves with no live pixel take no entries
#pragma unroll
        for (int q = 0; q < kHalves; ++q) hend[q] = half_live[q] ? 0x7fffffff : 0;
        const int idx = bs + (int)threadIdx.x;
        SplatRec r;
        r.a = r.b = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        r.c = make_float4(0.0f, -1.0f, 0.0f, 0.0f);  // no entry: reaches nothing
        int id = -1;
        if (threadIdx.x < kBatch && idx < rg.y) id = ids[idx];
        if ((unsigned)id >= (unsigned)n) id = -1;  // an id outside [0, n) is no entry
        if (id >= 0) {
            r = recs[id];
            S[threadIdx.x].a = r.a;
            S[threadIdx.x].b = r.b;
            S[threadIdx.x].c = r.c.x;
            if (DEP) S[threadIdx.x].z = r.c.w;
        }
        if (MW) {  // this batch's records start cleared
            uint4* z = reinterpret_cast<uint4*>(&mw_rec[0][0]) + 2 * threadIdx.x;
            z[0] = z[1] = make_uint4(0u, 0u, 0u, 0u);
        }
        unsigned long long hits[kHalves];
        half_hits(r, ox, oy, 0, hend, hits);
        // ascending slot order: list position = (hits in lower waves and lanes)
        int mine = 0;
#pragma unroll
        for (int q = 0; q < kHalves; ++q) {
            const int c = __popcll(hits[q]);
            mine = lane == q ? c : mine;
        }
        if (lane < kHalves) list_cnt[wv][lane] = mine;
        __syncthreads();
        int below = 0;
        if (lane < kHalves)
            for (int w2 = 0; w2 < wv; ++w2) below += list_cnt[w2][lane];
        unsigned pos_lo = ~0u, pos_hi = ~0u;  // MW: the entry's list positions, a byte per half
#pragma unroll
        for (int q = 0; q < kHalves; ++q) {
            const unsigned long long bal = hits[q];
            if (__builtin_amdgcn_inverse_ballot_w64(bal)) {
                const int rank = (int)__builtin_amdgcn_mbcnt_hi((unsigned)(bal >> 32),
                                                                __builtin_amdgcn_mbcnt_lo((unsigned)bal, 0u));
                const int at = __builtin_amdgcn_readlane(below, q) + rank;
                list[q][at] = (unsigned short)(threadIdx.x * sizeof(FwdSlot));
                if (MW) {
                    if (q < 4) pos_lo = (pos_lo & ~(0xffu << (8 * q))) | ((unsigned)at << (8 * q));
                    else pos_hi = (pos_hi & ~(0xffu << (8 * (q - 4)))) | ((unsigned)at << (8 * (q - 4)));
                }
            }
        }
        if (MW) *reinterpret_cast<uint2*>(S[threadIdx.x].pos) = make_uint2(pos_lo, pos_hi);
        __syncthreads();
        const int my_len = list_cnt[0][hq] + list_cnt[1][hq] + list_cnt[2][hq] + list_cnt[3][hq];
        const int other = hq ^ 1;
        const int len_other = list_cnt[0][other] + list_cnt[1][other] + list_cnt[2][other] + list_cnt[3][other];
        // the same for both halves: wave-uniform, so the loop runs on scalar control
        const int steps = __builtin_amdgcn_readfirstlane(max(my_len, len_other));
        // dummies past the end: up to a whole number of four-step groups and
        // the four entries read ahead of them (two entries read ahead with
        // the depth outputs)
        const int pad_end = DEP == 0 ? ((steps + 3) & ~3) + 4 : steps + 3;
        for (int p = my_len + (lane & 31); p < pad_end; p += 32) list[hq][p] = kDummyFwd;
        const unsigned short* L = list[hq];

        int bl_cur = -1;  // slot offset of this batch's last composited entry (-1: none)
        int med_cur = -1; // DEP: slot offset of this batch's last median candidate (-1: none)
        // One entry against the lane's pixel. Lanes whose alpha reaches 1/255
        // are walked; of those, the ones whose T stays >= 1e-4 composite and
        // the others stop here.
        unsigned long long any_c = 0;  // MW: lanes that composited in the current pair of steps
        auto step = [&](const float4& A, const float4& B, float2 Cz, int cur) -> float {
            const AlphaCoef k{A.x, A.y, A.z, A.w, B.x, B.y};
            float dx, dy;
            const float al = fminf(kAlphaMax, alpha_raw(k, px, py, dx, dy));
            const float test = __builtin_fmaf(-al, T, T);  // T (1 - alpha), rounded once
            const unsigned long long a_m = __builtin_amdgcn_fcmpf(al, kAlphaMin, 3 /* ordered >= */) & ~done_m;
            const unsigned long long c_m = a_m & __builtin_amdgcn_fcmpf(test, kTMin, 3 /* ordered >= */);
            done_m |= a_m & ~c_m;
            if (c_m == 0) return 0.0f;
            const bool comp = __builtin_amdgcn_inverse_ballot_w64(c_m);
            const float wgt = comp ? al * T : 0.0f;  // other lanes add exact zeros
            C0 = __builtin_fmaf(B.z, wgt, C0);
            C1 = __builtin_fmaf(B.w, wgt, C1);
            C2 = __builtin_fmaf(Cz.x, wgt, C2);
            if (DEP) {  // a median candidate: composited with T before it > 1/2
                const bool mh = comp && T > 0.5f;
                med_cur = mh ? cur : med_cur;
                zmed = mh ? Cz.y : zmed;
                // DEP 2: a new candidate moves the sums' reference to its depth
                // (only while T > 1/2: a few steps per pixel)
                if (DEP == 2 && __builtin_amdgcn_ballot_w64(mh) != 0) {
                    const float d = mh ? Cz.y - zmed_ref : 0.0f;
                    const float Bn = __builtin_fmaf(-d, Aw, Bw);
                    Cw = __builtin_fmaf(-d, Bw + Bn, Cw);
                    Bw = Bn;
                    zmed_ref = mh ? Cz.y : zmed_ref;
                }
            }
            if (DEP == 2) {  // the totals about the current median candidate's depth
                const float u = Cz.y - zmed_ref, wu = wgt * u;
                Aw += wgt;
                Bw += wu;
                Cw = __builtin_fmaf(wu, u, Cw);
            }
            T = comp ? test : T;
            bl_cur = comp ? cur : bl_cur;
            if (MW) any_c |= c_m;
            return wgt;
        };
        // MW: the pair's largest weights per half go to positions it, it + 1:
        // row 0 (2) of the wave holds half 0's (1's) for the first step, row 1
        // (3) for the second, and the first lane of each row stores its own
        auto store_max = [&](float w0, float w1, int it) {
            if (any_c == 0) return;  // the records stay 0
            any_c = 0;
            const unsigned m = half_umax_pair(__float_as_uint(w0), __float_as_uint(w1));
            if (__builtin_amdgcn_inverse_ballot_w64(0x0001000100010001ull))
                mw_rec[hq][it + ((lane >> 4) & 1)] = m;
        };
        // blue, and the depth where it is used
        auto cz_at = [&](int o) -> float2 { return make_float2(rec_at(o).c, DEP ? rec_at(o).z : 0.0f); };
        __builtin_amdgcn_s_setprio(0);
        if constexpr (DEP == 0) {
        // Four record buffers, each refilled three entries ahead of its use;
        // the steps past the end of a half's list take dummies (weight 0).
        static_assert(kListLen >= ((kBatch + 3) & ~3) + 4, "list rows hold the four-step read-ahead");
        int o0 = L[0], o1 = L[1], o2 = L[2], o3 = L[3];
        float4 A0 = rec_at(o0).a, B0 = rec_at(o0).b;
        float2 K0 = cz_at(o0);
        float4 A1 = rec_at(o1).a, B1 = rec_at(o1).b;
        float2 K1 = cz_at(o1);
        float4 A2 = rec_at(o2).a, B2 = rec_at(o2).b;
        float2 K2 = cz_at(o2);
        for (int it = 0; it < steps; it += 4) {
            if (done_m == ~0ull) break;  // the wave's 64 pixels have stopped
            const float4 A3 = rec_at(o3).a, B3 = rec_at(o3).b;
            const float2 K3 = cz_at(o3);
            const int n0 = L[it + 4];
            const float w0 = step(A0, B0, K0, o0);
            A0 = rec_at(n0).a;
            B0 = rec_at(n0).b;
            K0 = cz_at(n0);
            const int n1 = L[it + 5];
            const float w1 = step(A1, B1, K1, o1);
            if (MW) store_max(w0, w1, it);
            A1 = rec_at(n1).a;
            B1 = rec_at(n1).b;
            K1 = cz_at(n1);
            const int n2 = L[it + 6];
            const float w2 = step(A2, B2, K2, o2);
            A2 = rec_at(n2).a;
            B2 = rec_at(n2).b;
            K2 = cz_at(n2);
            const int n3 = L[it + 7];
            const float w3 = step(A3, B3, K3, o3);
            if (MW) store_max(w2, w3, it + 2);
            o0 = n0;
            o1 = n1;
            o2 = n2;
            o3 = n3;
        }
        } else {
        // With the depth outputs (whose sums take the registers): two record
        // buffers, each refilled one entry ahead of its use.
        int o0 = L[0], o1 = L[1];
        float4 A0 = rec_at(o0).a, B0 = rec_at(o0).b;
        float2 K0 = cz_at(o0);
        float w_tail = 0.0f;  // MW: the weights of an odd count's last step, stored after the loop
        for (int it = 0; it < steps; it += 2) {
            if (done_m == ~0ull) break;  // the wave's 64 pixels have stopped
            const float4 A1 = rec_at(o1).a, B1 = rec_at(o1).b;
            const float2 K1 = cz_at(o1);
            const int n0 = L[it + 2];
            const float w0 = step(A0, B0, K0, o0);
            if (it + 1 >= steps) {
                w_tail = w0;
                break;
            }
            A0 = rec_at(n0).a;
            B0 = rec_at(n0).b;
            K0 = cz_at(n0);
            const int n1 = L[it + 3];
            const float w1 = step(A1, B1, K1, o1);
            if (MW) store_max(w0, w1, it);
            o0 = n0;
            o1 = n1;
        }
        if (MW && (steps & 1)) store_max(w_tail, 0.0f, steps - 1);  // any_c is 0 if it was not walked
        }
        if (bl_cur >= 0) last_n = bs - rg.x + bl_cur / (int)sizeof(FwdSlot) + 1;
        if (DEP && med_cur >= 0) med_n = bs - rg.x + med_cur / (int)sizeof(FwdSlot) + 1;
        __syncthreads();  // the walk's reads of the slots and lists precede their rewriting
        if (MW && id >= 0 && id < n) {  // thread t owns slot t until it restages it
            const uint2 pp = *reinterpret_cast<const uint2*>(S[threadIdx.x].pos);
            unsigned v = 0u;
#pragma unroll
            for (int q = 0; q < kHalves; ++q) {
                const unsigned p = ((q < 4 ? pp.x : pp.y) >> (8 * (q & 3))) & 0xffu;
                if (p != 0xffu) v = max(v, mw_rec[q][p]);
            }
            if (v != 0u) atomicMax(max_weight + id, v);
        }
    }
    if (inside) {
        const int p = y * W + x;  // < 2^30: the HWC offset 3 p fits 32 unsigned bits
        float b0 = 0.0f, b1 = 0.0f, b2 = 0.0f;
        if (bg) { b0 = bg[0]; b1 = bg[1]; b2 = bg[2]; }
        image[3u * (unsigned)p + 0] = __builtin_fmaf(T, b0, C0);
        image[3u * (unsigned)p + 1] = __builtin_fmaf(T, b1, C1);
        image[3u * (unsigned)p + 2] = __builtin_fmaf(T, b2, C2);
        final_T[p] = T;
        n_contrib[p] = last_n;
        if (DEP) {
            // the first composited entry is always a median candidate (T = 1
            // before it), so med_n == 0 exactly when nothing composited
            const float zm = med_n > 0 ? zmed : 0.0f;
            if (median_depth) median_depth[p] = zm;
            if (median_pos) median_pos[p] = med_n;
            if (DEP == 2)  // already about the median (zmed_ref == zm); 0 when nothing composited
                dist_totals[p] = make_float4(Aw, Bw, Cw, fmaxf(__builtin_fmaf(Aw, Cw, -Bw * Bw), 0.0f));
        }
    }
}

// ---------------------------------------------------------------------------
// Launch order of the backward's tiles inside each XCD's band.
//
// The backward runs about 2.6 rounds of resident workgroups per CU, and tile
// costs vary (on the 2M-splat scene the costliest tile takes 1.5x the mean):
// in plain tile order the last workgroups start late and leave CUs idle at
// the end. The cost of a tile is its largest n_contrib (the walk length;
// correlation 0.9 with the walk's cost). Workgroup w still runs a tile of band
// w % 8 (the band of tile rows that XCD w % 8 works on), as in the plain
// mapping.
// ---------------------------------------------------------------------------

// Setup of a backward call, one launch. Blocks [0, cost_blocks) give one
// wave per tile its largest n_contrib, clamped to its list length (the walk
// length); the next rec_blocks pack one splat record per thread (as
// prep_kernel, and with each splat's first pair slot, so that the walk's
// flush needs no scattered read of splat_offsets); the rest clear the slot
// flags with 16-byte stores.
__global__ __launch_bounds__(256) void bwd_setup_kernel(int W, int H, int GX, int tiles, int cost_blocks,
                                                        const int2* __restrict__ ranges,
                                                        const int* __restrict__ n_contrib, int* __restrict__ cost,
                                                        int n, int rec_blocks, const float2* __restrict__ means,
                                                        const float* __restrict__ conics,
                                                        const float* __restrict__ colors,
                                                        const float* __restrict__ opac, const int* __restrict__ radii,
                                                        const int* __restrict__ splat_offsets,
                                                        SplatRec* __restrict__ recs, uint4* __restrict__ flags16,
                                                        long long n16)
{
    const int b = blockIdx.x;
    if (b < cost_blocks) {
        const int tile = b * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
        if (tile >= tiles) return;
        const int2 rg = ranges[tile];
        const int y = (tile / GX) * kTile + (lane >> 2), x0 = (tile % GX) * kTile + 4 * (lane & 3);
        int v = 0;
        if (y < H) {
#pragma unroll
            for (int c = 0; c < 4; ++c)
                if (x0 + c < W) v = max(v, n_contrib[y * W + x0 + c]);
        }
        v = max(min(v, rg.y - rg.x), 0);  // an inverted range costs nothing
        v = wave_max_i32(v);
        if (lane == 0) cost[tile] = v;
        return;
    }
    if (b < cost_blocks + rec_blocks) {  // block-uniform
        const int i0 = (b - cost_blocks) * 256, i = i0 + threadIdx.x;
        SplatRec r{};
        if (i < n) r = make_rec(i, means, conics, colors, opac, radii, splat_offsets);
        store_recs_block(recs, r, i0, n);
        return;
    }
    const long long i = (long long)(b - cost_blocks - rec_blocks) * 256 + threadIdx.x;
    if (i < n16) flags16[i] = make_uint4(0, 0, 0, 0);
}

// One workgroup per band. The band's cheapest tiles (a quarter of them, by a
// 256-bucket cost histogram) go last, costliest first (the longest-processing-
// time rule for the end of the launch, where late long tiles would leave CUs
// idle); the others go first in tile-id order, so that workgroups running at
// the same time on the band's XCD work on neighbouring tiles, whose lists
// share splats: their records are then re-read from that XCD's L2 rather than
// from HBM. order[r * 8 + band] = the band's r-th tile (-1 for padding).
// No result depends on the launch order, only the time and traffic do.
__global__ __launch_bounds__(1024) void band_order_kernel(int tiles, const int* __restrict__ cost,
                                                          int* __restrict__ order)
{
    __shared__ int hist[256];
    __shared__ int cmax;
    __shared__ int cut_key;               // keys above it (the cheapest tiles) form the tail
    __shared__ int wsum[1024 / 64];       // head tiles per wave's chunk range, then its prefix
    const int per = (tiles + kXcds - 1) / kXcds;
    const int band = blockIdx.x, t0 = band * per;
    const int n = max(0, min(per, tiles - t0));
    if (threadIdx.x < 256) hist[threadIdx.x] = 0;
    if (threadIdx.x == 0) cmax = 0;
    __syncthreads();
    int m = 0;
    for (int i = threadIdx.x; i < n; i += blockDim.x) m = max(m, cost[t0 + i]);
    m = wave_max_i32(m);
    if ((threadIdx.x & 63) == 0) atomicMax(&cmax, m);
    __syncthreads();
    const int top = max(cmax, 1);
    auto key = [&](int c) { return 255 - (int)(((long long)max(c, 0) * 255) / top); };  // 0 = costliest, in [0, 255]
    for (int i = threadIdx.x; i < n; i += blockDim.x) atomicAdd(&hist[key(cost[t0 + i])], 1);
    __syncthreads();
    if (threadIdx.x < 64) {  // exclusive scan of the 256 buckets by one wave, 4 per lane
        const int l = threadIdx.x;
        const int h0 = hist[4 * l], h1 = hist[4 * l + 1], h2 = hist[4 * l + 2], h3 = hist[4 * l + 3];
        int incl = h0 + h1 + h2 + h3;
        for (int d = 1; d < 64; d <<= 1) {
            const int u = __shfl_up(incl, d, 64);
            if (l >= d) incl += u;
        }
        const int ex = incl - (h0 + h1 + h2 + h3);
        hist[4 * l] = ex;
        hist[4 * l + 1] = ex + h0;
        hist[4 * l + 2] = ex + h0 + h1;
        hist[4 * l + 3] = ex + h0 + h1 + h2;
        // the tail: the buckets whose tiles all start at or after 3/4 of the
        // band (bucket k starts at hist[k]); the smallest such key
        int first = 256;
        for (int j = 3; j >= 0; --j)
            if (hist[4 * l + j] * 4 >= 3 * n) first = 4 * l + j;
        first = -wave_max_i32(-first);
        if (l == 0) cut_key = first;
    }
    __syncthreads();
    const int ck = cut_key;
    // head: tiles with key < ck, in tile-id order. Each thread takes a
    // contiguous range of the band's tiles; a block scan of the per-thread
    // counts gives each head tile its position.
    const int chunk = (n + (int)blockDim.x - 1) / (int)blockDim.x;
    const int i0 = (int)threadIdx.x * chunk, i1 = min(n, i0 + chunk);
    int cnt = 0;
    for (int i = i0; i < i1; ++i) cnt += key(cost[t0 + i]) < ck ? 1 : 0;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    int incl = cnt;  // inclusive scan inside the wave
    for (int d = 1; d < 64; d <<= 1) {
        const int u = __shfl_up(incl, d, 64);
        if (lane >= d) incl += u;
    }
    if (lane == 63) wsum[wv] = incl;
    __syncthreads();
    if (threadIdx.x == 0) {
        int acc = 0;
        for (int w = 0; w < (int)blockDim.x / 64; ++w) {
            const int c = wsum[w];
            wsum[w] = acc;
            acc += c;
        }
    }
    __syncthreads();
    int pos = wsum[wv] + incl - cnt;
    for (int i = i0; i < i1; ++i)
        if (key(cost[t0 + i]) < ck) order[(pos++) * kXcds + band] = t0 + i;
    // tail: after the head, by bucket (costliest first); the head's tiles are
    // exactly those of the buckets before ck, so the bucket offsets carry over
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
        const int k = key(cost[t0 + i]);
        if (k >= ck) {
            const int r = atomicAdd(&hist[k], 1);
            order[r * kXcds + band] = t0 + i;
        }
    }
    for (int r = n + threadIdx.x; r < per; r += blockDim.x) order[r * kXcds + band] = -1;
}

// Output stage of both gathers: u = (w g_r, w g_g, w g_b, s, s dx, s dy,
// s dx^2, s dx dy, s dy^2, [w]) summed over the splat's pairs; applies the
// splat's conic and opacity and writes every output.
// The splat's conic and opacity, requested when the gather starts (they do
// not depend on the pairs), so that their latency overlaps the pair scan.
struct SplatConsts {
    float a, b, c, o;
};
__device__ __forceinline__ SplatConsts load_consts(int i, int n, const float* __restrict__ conics,
                                                   const float* __restrict__ opac)
{
    if (i >= n) return SplatConsts{0.0f, 0.0f, 0.0f, 1.0f};
    return SplatConsts{conics[3 * i + 0], conics[3 * i + 1], conics[3 * i + 2], opac[i]};
}

// Per splat: u[0..8] the nine sums, u[9] the weight (AW), u[10] the depth
// gradient (DZ).
template <bool AW, bool DZ>
__device__ __forceinline__ void gather_write(int i, const float (&u)[11], const SplatConsts& k,
                                             float2* __restrict__ d_means, float* __restrict__ d_conics,
                                             float* __restrict__ d_colors, float* __restrict__ d_opac,
                                             float* __restrict__ accum_w, float* __restrict__ d_depths)
{
    d_means[i] = make_float2(__builtin_fmaf(k.a, u[4], k.b * u[5]), __builtin_fmaf(k.b, u[4], k.c * u[5]));
    d_conics[3 * i + 0] = -0.5f * u[6];
    d_conics[3 * i + 1] = -u[7];
    d_conics[3 * i + 2] = -0.5f * u[8];
    d_colors[3 * i + 0] = u[0];
    d_colors[3 * i + 1] = u[1];
    d_colors[3 * i + 2] = u[2];
    d_opac[i] = u[3] != 0.0f ? u[3] / k.o : 0.0f;
    if (AW) accum_w[i] = u[9];
    if (DZ) d_depths[i] = u[10];
}

// Gathers: one wave per 64 consecutive splats. Their pairs are contiguous,
// [offsets[i0], offsets[i0 + 64]), and most pair slots are unused (78% on the
// 2M-splat scene, 98% on the 1M-splat high-overlap scene, where early stop
// leaves most of each tile list unwalked), so the wave scans the flag bytes
// together, 16 per lane (1 KB per step, coalesced, the next kilobyte requested
// before the current one is used), and compacts the used pair positions into
// an LDS list in pair order. Lane l finds the part of the list that belongs
// to splat i0 + l (a binary search for its first pair; the next lane's start
// ends it) and sums it in registers, in slot order. For a few pairs per splat
// (gather_kernel) each lane loads its own records, two at a time. For many
// (large splats: a kilobyte of flags then holds only a dozen splats' pairs,
// and few lanes would load), gather_staged_kernel loads the listed records one
// per lane, every lane busy, stages them in LDS, and each lane then adds its
// splat's part from there. Finally lane l applies its splat's conic and
// opacity and writes every output (zeros for a splat no pixel took).
constexpr int kGatherWin = 16 * kWave;  // flag bytes scanned per step
constexpr int kGatherRegMaxPairs = 32;  // mean pairs per splat up to which gather_kernel runs
constexpr int kWalkManyPairs = 16;  // mean pairs per splat above which the deferred walk takes smaller batches
// Shapes of the deferred walk (entries per batch, steps per chunk, workgroups
// per CU), measured on the 2M-splat and the high-overlap scenes with the
// culled tile lists: 191-entry batches where splats cover few tiles; 127
// where they cover many (more half-list records per entry: a smaller batch
// leaves room for more records, and fewer batches are cut). Four-step chunks
// keep the per-wave pads at 2 KB, so four workgroups per CU fit; three per CU
// (more records) ran 40% slower, five (fewer) no faster.
constexpr int kDeferChunk = 4, kDeferWG = 4;
constexpr int kDeferBatchFew = 191, kDeferBatchMany = 127;

template <bool AW, bool DZ>
__global__ __launch_bounds__(kWave) void gather_kernel(int n, const int* __restrict__ splat_offsets, long long n_slots,
                                                       const float4* __restrict__ rec,
                                                       const uint4* __restrict__ flags16,
                                                       const float* __restrict__ conics, const float* __restrict__ opac,
                                                       float2* __restrict__ d_means, float* __restrict__ d_conics,
                                                       float* __restrict__ d_colors, float* __restrict__ d_opac,
                                                       float* __restrict__ accum_w, float* __restrict__ d_depths)
{
    __shared__ int used_list[kGatherWin];  // used pairs of the current window, relative to its start
    const int lane = threadIdx.x;
    const int i0 = blockIdx.x * kWave;
    const int i = i0 + lane;
    const long long my_off = min(max((long long)splat_offsets[min(i, n)], 0ll), n_slots);
    const SplatConsts sc = load_consts(i, n, conics, opac);
    const long long p0 = __shfl(my_off, 0, kWave);
    const long long p1 = min(max((long long)splat_offsets[min(i0 + kWave, n)], 0ll), n_slots);
    float u[11] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
    auto add_rec = [&](long long P) {
        const float4 a = rec[kSlotF4 * P + 0], b = rec[kSlotF4 * P + 1];
        float4 c;
        if (DZ) {
            c = rec[kSlotF4 * P + 2];
        } else {  // the last 8 bytes are padding
            const float2 c2 = *reinterpret_cast<const float2*>(rec + kSlotF4 * P + 2);
            c = make_float4(c2.x, c2.y, 0.0f, 0.0f);
        }
        u[0] += a.x; u[1] += a.y; u[2] += a.z; u[3] += a.w;
        u[4] += b.x; u[5] += b.y; u[6] += b.z; u[7] += b.w;
        u[8] += c.x;
        if (AW) u[9] += c.y;
        if (DZ) u[10] += c.z;
    };
    const long long w0 = p0 & ~15ll;  // windows start on 16-byte flag boundaries
    auto window = [&](long long wb) -> uint4 {
        const long long q = wb + 16 * lane;
        return q < p1 ? flags16[q >> 4] : make_uint4(0, 0, 0, 0);
    };
    uint4 fl_next = w0 < p1 ? window(w0) : make_uint4(0, 0, 0, 0);
    for (long long wb = w0; wb < p1; wb += kGatherWin) {
        const uint4 fl = fl_next;
        if (wb + kGatherWin < p1) fl_next = window(wb + kGatherWin);
        // this lane's 16 flag bytes -> used pair positions, kept in [p0, p1)
        const long long q = wb + 16 * lane;
        const unsigned wd[4] = {fl.x, fl.y, fl.z, fl.w};
        unsigned mask = 0;
#pragma unroll
        for (int b = 0; b < 16; ++b) {
            const long long pb = q + b;
            if (((wd[b >> 2] >> (8 * (b & 3))) & 0xffu) && pb >= p0 && pb < p1) mask |= 1u << b;
        }
        // compaction: exclusive prefix of the per-lane counts over the wave
        const int cnt = __popc(mask);
        int incl = cnt;
        for (int d = 1; d < kWave; d <<= 1) {
            const int v = __shfl_up(incl, d, kWave);
            if (lane >= d) incl += v;
        }
        const int total = __shfl(incl, kWave - 1, kWave);
        if (total == 0) continue;  // wave-uniform
        int pos = incl - cnt;
        while (mask) {
            const int b = __builtin_ctz(mask);
            mask &= mask - 1;
            used_list[pos++] = 16 * lane + b;
        }
        __syncthreads();
        // this splat's part of the list: from the first listed pair at or
        // after its first slot to the next splat's start
        const long long rel = my_off - wb;
        int beg = 0;
        if (i >= n || rel >= (long long)kGatherWin) {
            beg = total;
        } else if (rel > 0) {
            int lo = 0, hi = total;  // first r with used_list[r] >= rel
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (used_list[mid] < (int)rel) lo = mid + 1; else hi = mid;
            }
            beg = lo;
        }
        int end = __shfl_down(beg, 1, kWave);
        if (lane == kWave - 1) end = total;
        end = max(end, beg);
        int r = beg;
        for (; r + 1 < end; r += 2) {
            add_rec(wb + used_list[r]);
            add_rec(wb + used_list[r + 1]);
        }
        if (r < end) add_rec(wb + used_list[r]);
        __syncthreads();  // used_list is rewritten by the next window
    }
    if (i >= n) return;
    gather_write<AW, DZ>(i, u, sc, d_means, d_conics, d_colors, d_opac, accum_w, d_depths);
}

template <bool AW, bool DZ>
__global__ __launch_bounds__(kWave) void gather_staged_kernel(int n, const int* __restrict__ splat_offsets,
                                                              long long n_slots, const float4* __restrict__ rec,
                                                              const uint4* __restrict__ flags16,
                                                              const float* __restrict__ conics,
                                                              const float* __restrict__ opac,
                                                              float2* __restrict__ d_means,
                                                              float* __restrict__ d_conics,
                                                              float* __restrict__ d_colors,
                                                              float* __restrict__ d_opac, float* __restrict__ accum_w,
                                                              float* __restrict__ d_depths)
{
    __shared__ int used_list[kGatherWin];  // used pairs of the current window, relative to its start
    __shared__ float4 stage[kWave][3];     // records of up to 64 listed pairs
    const int lane = threadIdx.x;
    const int i0 = blockIdx.x * kWave;
    const int i = i0 + lane;
    const long long my_off = min(max((long long)splat_offsets[min(i, n)], 0ll), n_slots);
    const SplatConsts sc = load_consts(i, n, conics, opac);
    const long long p0 = __shfl(my_off, 0, kWave);
    const long long p1 = min(max((long long)splat_offsets[min(i0 + kWave, n)], 0ll), n_slots);
    float u[11] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
    const long long w0 = p0 & ~15ll;  // windows start on 16-byte flag boundaries
    auto window = [&](long long wb) -> uint4 {
        const long long q = wb + 16 * lane;
        return q < p1 ? flags16[q >> 4] : make_uint4(0, 0, 0, 0);
    };
    uint4 fl_next = w0 < p1 ? window(w0) : make_uint4(0, 0, 0, 0);
    for (long long wb = w0; wb < p1; wb += kGatherWin) {
        const uint4 fl = fl_next;
        if (wb + kGatherWin < p1) fl_next = window(wb + kGatherWin);
        // this lane's 16 flag bytes -> used pair positions, kept in [p0, p1)
        const long long q = wb + 16 * lane;
        const unsigned wd[4] = {fl.x, fl.y, fl.z, fl.w};
        unsigned mask = 0;
#pragma unroll
        for (int b = 0; b < 16; ++b) {
            const long long pb = q + b;
            if (((wd[b >> 2] >> (8 * (b & 3))) & 0xffu) && pb >= p0 && pb < p1) mask |= 1u << b;
        }
        // compaction: exclusive prefix of the per-lane counts over the wave
        const int cnt = __popc(mask);
        int incl = cnt;
        for (int d = 1; d < kWave; d <<= 1) {
            const int v = __shfl_up(incl, d, kWave);
            if (lane >= d) incl += v;
        }
        const int total = __shfl(incl, kWave - 1, kWave);
        if (total == 0) continue;  // wave-uniform
        int pos = incl - cnt;
        while (mask) {
            const int b = __builtin_ctz(mask);
            mask &= mask - 1;
            used_list[pos++] = 16 * lane + b;
        }
        __syncthreads();
        // this splat's part of the list: from the first listed pair at or
        // after its first slot to the next splat's start
        const long long rel = my_off - wb;
        int beg = 0;
        if (i >= n || rel >= (long long)kGatherWin) {
            beg = total;
        } else if (rel > 0) {
            int lo = 0, hi = total;  // first r with used_list[r] >= rel
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (used_list[mid] < (int)rel) lo = mid + 1; else hi = mid;
            }
            beg = lo;
        }
        int end = __shfl_down(beg, 1, kWave);
        if (lane == kWave - 1) end = total;
        end = max(end, beg);
        // the listed records, 64 at a time: loaded one per lane (every lane
        // busy), staged in LDS, and summed by their splats' lanes in order
        for (int r0 = 0; r0 < total; r0 += kWave) {
            const int r = r0 + lane;
            if (r < total) {
                const long long P = wb + used_list[r];
                stage[lane][0] = rec[kSlotF4 * P + 0];
                stage[lane][1] = rec[kSlotF4 * P + 1];
                if (DZ) {
                    stage[lane][2] = rec[kSlotF4 * P + 2];
                } else {  // the last 8 bytes are padding
                    const float2 c2 = *reinterpret_cast<const float2*>(rec + kSlotF4 * P + 2);
                    stage[lane][2] = make_float4(c2.x, c2.y, 0.0f, 0.0f);
                }
            }
            __syncthreads();
            const int k1 = min(end, r0 + kWave);
            for (int k = max(beg, r0); k < k1; ++k) {
                const float4 a = stage[k - r0][0], b = stage[k - r0][1], c = stage[k - r0][2];
                u[0] += a.x; u[1] += a.y; u[2] += a.z; u[3] += a.w;
                u[4] += b.x; u[5] += b.y; u[6] += b.z; u[7] += b.w;
                u[8] += c.x;
                if (AW) u[9] += c.y;
                if (DZ) u[10] += c.z;
            }
            __syncthreads();  // stage is rewritten by the next round
        }
        __syncthreads();  // used_list is rewritten by the next window
    }
    if (i >= n) return;
    gather_write<AW, DZ>(i, u, sc, d_means, d_conics, d_colors, d_opac, accum_w, d_depths);
}

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

// Workspace layouts. Forward: splat records. Backward: splat records, then the
// per-(splat, tile) slots (3 float4 each) and their used-flags, then the tile
// costs and the launch order.
struct Layout {
    size_t recs, slots, used, cost, order, bytes;
};

Layout layout(long long n_recs, long long n_slots, long long tiles)
{
    Layout L{};
    L.recs = 0;
    L.slots = n_recs > 0 ? align256(sizeof(SplatRec) * (size_t)n_recs) : 0;
    L.used = L.slots + (n_slots > 0 ? align256(sizeof(float4) * kSlotF4 * (size_t)n_slots) : 0);
    L.cost = L.used + (n_slots > 0 ? align256((size_t)n_slots + 16) : 0);
    L.order = L.cost + (tiles > 0 ? align256(sizeof(int) * (size_t)tiles) : 0);
    L.bytes = L.order + (tiles > 0 ? align256(sizeof(int) * (size_t)xcd_grid((int)tiles)) : 0);
    return L;
}

}  // namespace
}  // namespace gs

using namespace gs;

extern "C" size_t gs_rasterize_fwd_workspace_size(int32_t n)
{
    if (n < 0 || n > kMaxSplats) return 0;
    return layout(n > 0 ? n : 1, 0, 0).bytes;
}

namespace {
gs_status fwd_impl(const char* name, int32_t n, const float* means2d, const float* conics, const float* colors,
                   const float* opacities, const float* depths, const float* background, int32_t width,
                   int32_t height, const int32_t* tile_ranges, const int32_t* sorted_ids, int64_t n_isect,
                   float* image, float* final_T, int32_t* n_contrib, float* max_weight, float* dist_totals,
                   float* median_depth, int32_t* median_pos, void* workspace, size_t workspace_bytes,
                   hipStream_t st)
{
    GS_CHECK_ARG(n >= 0 && n <= kMaxSplats, "%s: n = %d outside 0..%d", name, n, kMaxSplats);
    GS_CHECK_ARG(n_isect >= 0 && n_isect <= 0x7fffffffll, "%s: n_isect = %lld out of range", name,
                 (long long)n_isect);
    GS_CHECK_ARG(width > 0 && height > 0 && width <= kMaxDim && height <= kMaxDim,
                 "%s: image size %d x %d outside 1..%d", name, width, height, kMaxDim);
    GS_CHECK_ARG(n == 0 || (means2d && conics && colors && opacities), "%s: NULL splat array", name);
    GS_CHECK_ARG(tile_ranges && image && final_T && n_contrib, "%s: NULL image-side array", name);
    GS_CHECK_ARG(n_isect == 0 || sorted_ids, "%s: sorted_ids is NULL", name);
    const int dep = dist_totals ? 2 : (median_depth || median_pos) ? 1 : 0;
    GS_CHECK_ARG(dep == 0 || n == 0 || depths, "%s: depth outputs requested with depths NULL", name);
    const Layout L = layout(n > 0 ? n : 1, 0, 0);
    GS_CHECK_ARG(n == 0 || (workspace && workspace_bytes >= L.bytes), "%s: workspace %zu bytes, need %zu", name,
                 workspace_bytes, L.bytes);
    GS_CHECK_ARG(n == 0 || ((uintptr_t)workspace & 255) == 0, "%s: workspace not 256-byte aligned", name);
    SplatRec* recs = n ? (SplatRec*)((char*)workspace + L.recs) : nullptr;
    if (n > 0) {
        prep_kernel<<<(n + 255) / 256, 256, 0, st>>>(n, (const float2*)means2d, conics, colors, opacities, nullptr,
                                                     dep ? depths : nullptr, recs);
        GS_HIP(hipGetLastError());
    }
    const int GX = grid_x(width), tiles = GX * grid_y(height);
    if (max_weight && n > 0) {
        zero_u32_kernel<<<(n + 255) / 256, 256, 0, st>>>((unsigned*)max_weight, n);
        GS_HIP(hipGetLastError());
    }
    auto launch = [&](auto kernel) {
        kernel<<<xcd_grid(tiles), kBlock, 0, st>>>(n, width, height, GX, tiles, (const int2*)tile_ranges, n_isect,
                                                   sorted_ids, recs, background, image, final_T, n_contrib,
                                                   (unsigned*)max_weight, (float4*)dist_totals, median_depth,
                                                   median_pos);
    };
    // every combination of the optional outputs is its own instance
    if (max_weight) {
        if (dep == 2) launch(fwd_kernel<true, 2>);
        else if (dep == 1) launch(fwd_kernel<true, 1>);
        else launch(fwd_kernel<true, 0>);
    } else {
        if (dep == 2) launch(fwd_kernel<false, 2>);
        else if (dep == 1) launch(fwd_kernel<false, 1>);
        else launch(fwd_kernel<false, 0>);
    }
    GS_HIP(hipGetLastError());
    return GS_OK;
}
}  // namespace

extern "C" gs_status gs_rasterize_fwd(int32_t n, const float* means2d, const float* conics, const float* colors,
                                      const float* opacities, const float* background, int32_t width,
                                      int32_t height, const int32_t* tile_ranges, const int32_t* sorted_ids,
                                      int64_t n_isect, float* image, float* final_T, int32_t* n_contrib,
                                      float* max_weight, void* workspace, size_t workspace_bytes,
                                      gs_stream_t stream)
{
    return fwd_impl("gs_rasterize_fwd", n, means2d, conics, colors, opacities, nullptr, background, width, height,
                    tile_ranges, sorted_ids, n_isect, image, final_T, n_contrib, max_weight, nullptr, nullptr,
                    nullptr, workspace, workspace_bytes, (hipStream_t)stream);
}

extern "C" gs_status gs_rasterize_fwd_depth(int32_t n, const float* means2d, const float* conics,
                                            const float* colors, const float* opacities, const float* depths,
                                            const float* background, int32_t width, int32_t height,
                                            const int32_t* tile_ranges, const int32_t* sorted_ids, int64_t n_isect,
                                            float* image, float* final_T, int32_t* n_contrib, float* max_weight,
                                            float* dist_totals, float* median_depth, int32_t* median_pos,
                                            void* workspace, size_t workspace_bytes, gs_stream_t stream)
{
    return fwd_impl("gs_rasterize_fwd_depth", n, means2d, conics, colors, opacities, depths, background, width,
                    height, tile_ranges, sorted_ids, n_isect, image, final_T, n_contrib, max_weight, dist_totals,
                    median_depth, median_pos, workspace, workspace_bytes, (hipStream_t)stream);
}

extern "C" size_t gs_rasterize_bwd_workspace_size(int32_t n, int64_t n_slots, int32_t width, int32_t height)
{
    if (n < 0 || n > kMaxSplats || n_slots < 0 || width <= 0 || height <= 0 || width > kMaxDim || height > kMaxDim) return 0;
    return layout(n > 0 ? n : 1, n_slots, (long long)grid_x(width) * grid_y(height)).bytes;
}

namespace {
// dep: the depth terms taken (bit 0 distortion, bit 1 median; dz holds their
// inputs, dL_ddepths their output), 0 for none.
gs_status bwd_impl(int32_t n, const float* means2d, const float* conics, const float* colors,
                   const float* opacities, const int32_t* radii, const float* background, int32_t width,
                   int32_t height, const int32_t* tile_ranges, const int32_t* sorted_ids,
                   const int32_t* splat_offsets, int64_t n_isect, int64_t n_slots, const float* final_T,
                   const int32_t* n_contrib, const float* dL_dimage, float* dL_dmeans2d, float* dL_dconics, float* dL_dcolors,
                   float* dL_dopacities, float* accum_weight, uint32_t flags, void* workspace,
                   size_t workspace_bytes, gs_stream_t stream_, const gs_event_t* events, int dep = 0,
                   DepthIn dz = DepthIn{}, float* dL_ddepths = nullptr)
{
    hipStream_t st = (hipStream_t)stream_;
    // stage-boundary events of gs_rasterize_bwd_timed (none for gs_rasterize_bwd)
    auto mark = [&](int k) -> hipError_t {
        return (events && events[k]) ? hipEventRecord((hipEvent_t)events[k], st) : hipSuccess;
    };
    GS_CHECK_ARG(n >= 0 && n <= kMaxSplats, "gs_rasterize_bwd: n = %d outside 0..%d", n, kMaxSplats);
    GS_CHECK_ARG(n_isect >= 0 && n_isect <= 0x7fffffffll, "gs_rasterize_bwd: n_isect = %lld out of range",
                 (long long)n_isect);
    GS_CHECK_ARG(n_slots >= n_isect && n_slots <= 0x7fffffffll,
                 "gs_rasterize_bwd: n_slots = %lld outside n_isect .. 2^31 - 1 (n_isect = %lld)", (long long)n_slots,
                 (long long)n_isect);
    GS_CHECK_ARG(width > 0 && height > 0 && width <= kMaxDim && height <= kMaxDim,
                 "gs_rasterize_bwd: image size %d x %d outside 1..%d", width, height, kMaxDim);
    constexpr uint32_t kWalkFlags = GS_FLAG_WALK_ADD | GS_FLAG_WALK_STORE | GS_FLAG_WALK_DEFER;
    GS_CHECK_ARG((flags & ~(uint32_t)(GS_FLAG_ACCUM_WEIGHT | kWalkFlags)) == 0,
                 "gs_rasterize_bwd: unknown flags 0x%x", flags);
    GS_CHECK_ARG(__builtin_popcount(flags & kWalkFlags) <= 1,
                 "gs_rasterize_bwd: more than one walk flag set (GS_FLAG_WALK_ADD, _STORE, _DEFER)");
    const bool aw = (flags & GS_FLAG_ACCUM_WEIGHT) != 0;
    // the stored-partials walk pays off where splats cover many tiles (more
    // contributing lanes per step, more LDS adds per entry)
    // the deferred walk unless another is forced; its batch size by the mean
    // tiles per splat
    const bool store_walk = (flags & GS_FLAG_WALK_STORE) != 0;
    const bool add_walk = (flags & GS_FLAG_WALK_ADD) != 0;
    const bool many_tiles = n_isect > (long long)kWalkManyPairs * n;
    GS_CHECK_ARG(n == 0 || (means2d && conics && colors && opacities && radii && splat_offsets),
                 "gs_rasterize_bwd: NULL splat array");
    GS_CHECK_ARG(n == 0 || (dL_dmeans2d && dL_dconics && dL_dcolors && dL_dopacities),
                 "gs_rasterize_bwd: NULL gradient output");
    GS_CHECK_ARG(!aw || n == 0 || accum_weight, "gs_rasterize_bwd: GS_FLAG_ACCUM_WEIGHT with accum_weight NULL");
    GS_CHECK_ARG(tile_ranges && final_T && n_contrib && dL_dimage, "gs_rasterize_bwd: NULL image-side array");
    GS_CHECK_ARG(n_isect == 0 || sorted_ids, "gs_rasterize_bwd: sorted_ids is NULL");
    if (dep) {
        GS_CHECK_ARG(n == 0 || (dz.depths && dL_ddepths), "gs_rasterize_bwd_depth: depths or dL_ddepths NULL");
        GS_CHECK_ARG(dz.median_pos, "gs_rasterize_bwd_depth: median_pos is NULL");
        GS_CHECK_ARG(!(dep & 1) || dz.totals, "gs_rasterize_bwd_depth: dL_ddist given with dist_totals NULL");
        if (store_walk || add_walk) {
            set_error("gs_rasterize_bwd_depth: the depth terms run on the deferred walk only "
                      "(GS_FLAG_WALK_ADD / GS_FLAG_WALK_STORE set)");
            return GS_ERR_UNSUPPORTED;
        }
    }
    const int GX = grid_x(width), GY = grid_y(height), tiles = GX * GY;
    const Layout L = layout(n, n_slots, tiles);
    GS_CHECK_ARG(n == 0 || (workspace && workspace_bytes >= L.bytes),
                 "gs_rasterize_bwd: workspace %zu bytes, need %zu", workspace_bytes, L.bytes);
    GS_CHECK_ARG(n == 0 || ((uintptr_t)workspace & 255) == 0, "gs_rasterize_bwd: workspace not 256-byte aligned");
    GS_HIP(mark(0));
    if (n == 0) {
        GS_HIP(mark(1));
        GS_HIP(mark(2));
        GS_HIP(mark(3));
        return GS_OK;
    }
    SplatRec* recs = (SplatRec*)((char*)workspace + L.recs);
    // without pairs no slot is written (nor its flag cleared): the gather then
    // sees no slots at all
    const long long n_slots_live = n_isect > 0 ? n_slots : 0;
    float4* slots = n_slots_live ? (float4*)((char*)workspace + L.slots) : nullptr;
    unsigned char* used = n_slots_live ? (unsigned char*)workspace + L.used : nullptr;
    int* cost = (int*)((char*)workspace + L.cost);
    int* order = (int*)((char*)workspace + L.order);
    if (n_isect > 0) {
        // flags cleared in whole 16-byte units (the region is padded)
        const long long n16 = (n_slots + 15) >> 4;
        const int cost_blocks = (tiles + 3) / 4, rec_blocks = (n + 255) / 256;
        const long long blocks = (long long)cost_blocks + rec_blocks + (n16 + 255) / 256;
        bwd_setup_kernel<<<(unsigned)blocks, 256, 0, st>>>(
            width, height, GX, tiles, cost_blocks, (const int2*)tile_ranges, n_contrib, cost, n, rec_blocks,
            (const float2*)means2d, conics, colors, opacities, radii, splat_offsets, recs, (uint4*)used, n16);
        GS_HIP(hipGetLastError());
        band_order_kernel<<<kXcds, 1024, 0, st>>>(tiles, cost, order);
        GS_HIP(hipGetLastError());
        GS_HIP(mark(1));
        const int* ord = order;
        auto launch = [&](auto kernel, auto... extra) {
            kernel<<<xcd_grid(tiles), kBlock, 0, st>>>(width, height, GX, GY, tiles, n, (const int2*)tile_ranges,
                                                       sorted_ids, recs, splat_offsets, n_isect, n_slots,
                                                       background,
                                                       final_T, n_contrib, dL_dimage, ord, slots, used, extra...);
        };
        // the deferred walk: one instance per (weight, batch size, depth terms)
        auto defer = [&](auto nb_tag) {
            constexpr int NB = decltype(nb_tag)::value;
            using std::integral_constant;
            auto go = [&](auto dep_tag) {
                constexpr int D = decltype(dep_tag)::value;
                aw ? launch(bwd_defer_kernel<true, NB, kDeferChunk, kDeferWG, D>, dz)
                   : launch(bwd_defer_kernel<false, NB, kDeferChunk, kDeferWG, D>, dz);
            };
            if (dep == 3) go(integral_constant<int, 3>{});
            else if (dep == 2) go(integral_constant<int, 2>{});
            else if (dep == 1) go(integral_constant<int, 1>{});
            else go(integral_constant<int, 0>{});
        };
        if (store_walk)
            aw ? launch(bwd_store_kernel<true>) : launch(bwd_store_kernel<false>);
        else if (add_walk)
            aw ? launch(bwd_kernel<true>) : launch(bwd_kernel<false>);
        else if (many_tiles)
            defer(std::integral_constant<int, kDeferBatchMany>{});
        else
            defer(std::integral_constant<int, kDeferBatchFew>{});
        GS_HIP(hipGetLastError());
        GS_HIP(mark(2));
    } else {
        GS_HIP(mark(1));
        GS_HIP(mark(2));
    }
    const uint4* flags16 = reinterpret_cast<const uint4*>(used);  // padded to whole 16-byte units
    const unsigned gb = (unsigned)((n + kWave - 1) / kWave);
#define GS_GATHER(K, AWV, ACC, DZV, DD)                                                                            \
    K<AWV, DZV><<<gb, kWave, 0, st>>>(n, splat_offsets, n_slots_live, slots, flags16, conics, opacities,              \
                                      (float2*)dL_dmeans2d, dL_dconics, dL_dcolors, dL_dopacities, ACC, DD)
    const bool dzo = dep != 0;
    if (n_slots_live <= (long long)kGatherRegMaxPairs * n) {
        if (aw) dzo ? GS_GATHER(gather_kernel, true, accum_weight, true, dL_ddepths)
                    : GS_GATHER(gather_kernel, true, accum_weight, false, nullptr);
        else dzo ? GS_GATHER(gather_kernel, false, nullptr, true, dL_ddepths)
                 : GS_GATHER(gather_kernel, false, nullptr, false, nullptr);
    } else {
        if (aw) dzo ? GS_GATHER(gather_staged_kernel, true, accum_weight, true, dL_ddepths)
                    : GS_GATHER(gather_staged_kernel, true, accum_weight, false, nullptr);
        else dzo ? GS_GATHER(gather_staged_kernel, false, nullptr, true, dL_ddepths)
                 : GS_GATHER(gather_staged_kernel, false, nullptr, false, nullptr);
    }
#undef GS_GATHER
    GS_HIP(hipGetLastError());
    GS_HIP(mark(3));
    return GS_OK;
}
}  // namespace

extern "C" gs_status gs_rasterize_bwd(int32_t n, const float* means2d, const float* conics, const float* colors,
                                      const float* opacities, const int32_t* radii, const float* background,
                                      int32_t width, int32_t height, const int32_t* tile_ranges,
                                      const int32_t* sorted_ids, const int32_t* splat_offsets, int64_t n_isect, int64_t n_slots,
                                      const float* final_T, const int32_t* n_contrib, const float* dL_dimage,
                                      float* dL_dmeans2d, float* dL_dconics, float* dL_dcolors,
                                      float* dL_dopacities, float* accum_weight, uint32_t flags, void* workspace,
                                      size_t workspace_bytes, gs_stream_t stream)
{
    return bwd_impl(n, means2d, conics, colors, opacities, radii, background, width, height, tile_ranges,
                    sorted_ids, splat_offsets, n_isect, n_slots, final_T, n_contrib, dL_dimage, dL_dmeans2d, dL_dconics,
                    dL_dcolors, dL_dopacities, accum_weight, flags, workspace, workspace_bytes, stream, nullptr);
}

extern "C" gs_status gs_rasterize_bwd_depth(int32_t n, const float* means2d, const float* conics,
                                            const float* colors, const float* opacities, const float* depths,
                                            const int32_t* radii, const float* background, int32_t width,
                                            int32_t height, const int32_t* tile_ranges, const int32_t* sorted_ids,
                                            const int32_t* splat_offsets, int64_t n_isect, int64_t n_slots, const float* final_T,
                                            const int32_t* n_contrib, const float* dist_totals,
                                            const int32_t* median_pos, const float* dL_dimage,
                                            const float* dL_ddist, const float* dL_dmedian, float* dL_dmeans2d,
                                            float* dL_dconics, float* dL_dcolors, float* dL_dopacities,
                                            float* dL_ddepths, float* accum_weight, uint32_t flags,
                                            void* workspace, size_t workspace_bytes, gs_stream_t stream)
{
    const int dep = (dL_ddist ? 1 : 0) | (dL_dmedian ? 2 : 0);
    if (dep == 0) {  // no depth term: the plain backward, and zero depth gradients if asked for
        const gs_status r = bwd_impl(n, means2d, conics, colors, opacities, radii, background, width, height,
                                     tile_ranges, sorted_ids, splat_offsets, n_isect, n_slots, final_T, n_contrib,
                                     dL_dimage, dL_dmeans2d, dL_dconics, dL_dcolors, dL_dopacities, accum_weight,
                                     flags, workspace, workspace_bytes, stream, nullptr);
        if (r != GS_OK || !dL_ddepths || n <= 0) return r;
        zero_u32_kernel<<<(n + 255) / 256, 256, 0, (hipStream_t)stream>>>((unsigned*)dL_ddepths, n);
        GS_HIP(hipGetLastError());
        return GS_OK;
    }
    const DepthIn dz{depths, (const float4*)dist_totals, median_pos, dL_ddist, dL_dmedian};
    return bwd_impl(n, means2d, conics, colors, opacities, radii, background, width, height, tile_ranges,
                    sorted_ids, splat_offsets, n_isect, n_slots, final_T, n_contrib, dL_dimage, dL_dmeans2d, dL_dconics,
                    dL_dcolors, dL_dopacities, accum_weight, flags, workspace, workspace_bytes, stream, nullptr,
                    dep, dz, dL_ddepths);
}

extern "C" gs_status gs_rasterize_bwd_timed(int32_t n, const float* means2d, const float* conics,
                                            const float* colors, const float* opacities, const int32_t* radii,
                                            const float* background, int32_t width, int32_t height,
                                            const int32_t* tile_ranges, const int32_t* sorted_ids,
                                            const int32_t* splat_offsets, int64_t n_isect, int64_t n_slots, const float* final_T,
                                            const int32_t* n_contrib, const float* dL_dimage, float* dL_dmeans2d,
                                            float* dL_dconics, float* dL_dcolors, float* dL_dopacities,
                                            float* accum_weight, uint32_t flags, void* workspace,
                                            size_t workspace_bytes, gs_stream_t stream, const gs_event_t events[4])
{
    GS_CHECK_ARG(events, "gs_rasterize_bwd_timed: events is NULL");
    return bwd_impl(n, means2d, conics, colors, opacities, radii, background, width, height, tile_ranges,
                    sorted_ids, splat_offsets, n_isect, n_slots, final_T, n_contrib, dL_dimage, dL_dmeans2d, dL_dconics,
                    dL_dcolors, dL_dopacities, accum_weight, flags, workspace, workspace_bytes, stream, events);
}

// ---------------------------------------------------------------------------
// gs_rasterize_bwd_noalloc: the backward with its workspace in a fixed device
// array, for callers that cannot allocate (graph capture, tight serving
// loops). The array is a file-scope device variable: every GPU the library
// runs on holds its own copy, at its own address, until the process ends. Host
// code never passes the array's name to a kernel (on the host it only stands
// for the symbol): the device address comes from hipGetSymbolAddress, taken
// once per device with that device current, and is kept per device.
// ---------------------------------------------------------------------------
namespace gs {
namespace {
constexpr size_t kScratchBytes = size_t(64) << 20;   // 64 MiB per device
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace
}  // namespace gs

static __device__ __align__(256) unsigned char scratch[gs::kScratchBytes];

namespace {
// The current device's address of the scratch array (looked up on the first
// call on that device).
gs_status scratch_address(void** out)
{
    int dev = -1;
    GS_HIP(hipGetDevice(&dev));
    GS_CHECK_ARG(dev >= 0 && dev < kMaxDevices, "gs_rasterize_bwd_noalloc: device %d beyond %d devices", dev,
                 kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        GS_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
        GS_CHECK_ARG(p != nullptr && ((uintptr_t)p & 255) == 0, "gs_rasterize_bwd_noalloc: scratch address %p",
                     p);
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return GS_OK;
}
}  // namespace

extern "C" size_t gs_rasterize_bwd_noalloc_capacity(void) { return kScratchBytes; }

extern "C" gs_status gs_rasterize_bwd_noalloc(int32_t n, const float* means2d, const float* conics,
                                              const float* colors, const float* opacities, const int32_t* radii,
                                              const float* background, int32_t width, int32_t height,
                                              const int32_t* tile_ranges, const int32_t* sorted_ids,
                                              const int32_t* splat_offsets, int64_t n_isect, int64_t n_slots, const float* final_T,
                                              const int32_t* n_contrib, const float* dL_dimage,
                                              float* dL_dmeans2d, float* dL_dconics, float* dL_dcolors,
                                              float* dL_dopacities, float* accum_weight, uint32_t flags,
                                              gs_stream_t stream)
{
    // sizes first, on the host: a call that would not fit touches no device
    const size_t need = gs_rasterize_bwd_workspace_size(n, n_slots, width, height);
    GS_CHECK_ARG(need > 0, "gs_rasterize_bwd_noalloc: n = %d, n_slots = %lld or image %d x %d out of range", n,
                 (long long)n_slots, width, height);
    if (need > kScratchBytes) {
        set_error("gs_rasterize_bwd_noalloc: %d splats, %lld pair slots and %d x %d pixels need %zu bytes of scratch; "
                  "the fixed scratch holds %zu (use gs_rasterize_bwd with a workspace)",
                  n, (long long)n_slots, width, height, need, kScratchBytes);
        return GS_ERR_CAPACITY;
    }
    void* ws = nullptr;
    const gs_status st = scratch_address(&ws);
    if (st != GS_OK) return st;
    return bwd_impl(n, means2d, conics, colors, opacities, radii, background, width, height, tile_ranges,
                    sorted_ids, splat_offsets, n_isect, n_slots, final_T, n_contrib, dL_dimage, dL_dmeans2d, dL_dconics,
                    dL_dcolors, dL_dopacities, accum_weight, flags, ws, kScratchBytes, stream, nullptr);
}
