// gs_bin.hip -- gs_bin_tiles: tile binning, stable radix sorts, tile ranges.
//
// Stages (the binning / sort / range kernels of the 3dgs-rs pipeline listed in
// the timing table of "Phase 5 step 30b — kernel-by-kernel timing", section
// 計測結果: emit_pairs, radix_hist, radix_scatter, extract_offsets):
//   1. count   one thread per splat: float32 tile rectangle and its number
//              of tiles; the number of them the splat's culling ellipse
//              (alpha >= 1/255) keeps, row by row
//   2. scan    exclusive prefix sum of the rectangle counts in splat order
//              (device-wide, 32-bit items and offsets, sums and the total in
//              64 bits): each splat's first pair slot, splat_offsets; and the
//              total of the kept counts
//   3. host    read both totals back (the call's only synchronisation; the
//              depth sort is already queued behind the copy)
//   4. depth   stable LSD radix sort of the splats by the bit pattern of their
//              depth (32 bits, 8-bit digits), splat ids starting in id order;
//              the last pass also gathers the kept counts into depth order
//   5. emit    the kept counts in depth order scanned; the
//              splat of depth rank k reads its rectangle and ellipse factors
//              (stored by the count pass) and writes its kept tiles,
//              row-major, at that offset, as (tile id, splat id), tile ids
//              16-bit up to 65536 tiles
//   6. tiles   stable LSD radix sort of the pairs by tile id over only the
//              ceil(log2(tiles)) bits it can have, split as evenly as possible
//              over as few passes as 8-bit digits allow, narrower digits first
//              (6 + 6 bits at 4056 tiles, 6 + 7 at 8160).
//              Stability keeps each tile's pairs in depth order, equal depths
//              by ascending splat id.
//   7. ranges  [start, end) per tile from the boundaries of the sorted keys
// Sorting the splats by depth first moves the 32 depth bits off the pairs:
// the passes over all pairs fall from six (tile and depth bits together) to
// two, over 6-byte instead of 12-byte elements.
#include "gs_common.hpp"

namespace gs {
namespace {

constexpr int kScanThreads = 256;
constexpr int kScanItems = 4;                         // per thread: one 16-byte load
constexpr int kScanTile = kScanThreads * kScanItems;  // 1024 items per workgroup

// Radix sort tiling: a workgroup of W waves sorts W * 1024 keys, 16 per
// thread. The pair passes use 8 waves (8192 keys: longer runs per digit in
// each workgroup's output, so fewer partly written cache lines); the splats'
// depth sort 4 (4096 keys: its 1-2M keys then still make enough workgroups to
// fill the chip).
constexpr int kSortRounds = 16;                       // rounds of W * 64 keys per workgroup
constexpr int kRadixBits = 8;                         // widest digit
constexpr int kRadix = 1 << kRadixBits;
constexpr int kDepthWaves = 4, kPairWaves = 8;
constexpr int kSortTileMin = kDepthWaves * kWave * kSortRounds;  // the smaller tile: workspace sizing
template <int W> struct SortTiling {
    static constexpr int kThreads = W * kWave;
    static constexpr int kTile = kThreads * kSortRounds;
    static_assert(kThreads >= kRadix, "at most one digit per thread");
};

__device__ __forceinline__ bool splat_rect(float mx, float my, int r, float depth, int GX, int GY,
                                           int& tx0, int& tx1, int& ty0, int& ty1)
{
    tile_rect(mx, my, r, GX, GY, tx0, tx1, ty0, ty1);
    const bool live = r > 0 && depth > 0.0f && __builtin_isfinite(mx) && __builtin_isfinite(my);
    return live && tx1 > tx0 && ty1 > ty0;
}

// ---------------------------------------------------------------------------
// The culling ellipse. A splat reaches alpha >= 1/255 only where its quadratic
// form Q = a dx^2 + 2 b dx dy + c dy^2 is at most 2 ln(255 o); a tile of the
// rectangle is kept only if the ellipse {Q <= T} meets the tile's pixel-centre
// rectangle, T an upper bound on 2 ln(255 o). Everything here is float32 with
// each operation rounded once, in the order written (no fused multiply-adds;
// division and square root correctly rounded), so the decisions are those of
// any IEEE float32 evaluation of the same expressions:
//   255 o = m2 2^e2, m2 in [1, 2):  ln(255 o) <= e2 ln 2 + (m2 - 1) / sqrt(m2)
//   (ln x <= (x - 1) / sqrt(x) for x >= 1; ln 2 taken as float32 ln 2, which
//   rounds up), T = 2 lnb (1 + 2^-10) + 2^-10 (a margin for the rounding of Q
//   in the compositing);
//   Q = (l11 u + l21 v)^2 + (l22 v)^2 with the conic's Cholesky factors
//   l11 = sqrt(a), l21 = b / l11, l22 = sqrt(max(c - l21^2, 0)), u = x - mean_x,
//   v = y - mean_y;
//   per tile row, over its band of pixel centres v in [v0, v0 + 15]: the
//   ellipse's left end u = (-l21 v - sqrt(T - (l22 v)^2)) / l11 is convex in v,
//   least at the leftmost point's v = vL = sqrt(T) l21 / (l22 sqrt(l21^2 +
//   l22^2)), so it is taken at vL clamped to the band (and to |v| <= vmax =
//   sqrt(T) / l22); the right end likewise at -vL. Column c (pixel centres
//   16 c + 0.5 .. 16 c + 15.5) is kept iff 16 c + 15.5 >= x_left and
//   16 c + 0.5 <= x_right.
// A splat whose float32 product 255 o is below 1 is kept nowhere (alpha <= o <
// 1/255); one whose factors are not finite and positive keeps its whole
// rectangle.
// ---------------------------------------------------------------------------
enum : int { kCullNone = 0, kCullRect = 1, kCullRows = 2 };

struct CullEllipse {
    float mx, my, l11, l21, l22, T, vmax, vL;
    int mode;
};

// What the emission needs of a splat, written by the count pass in splat
// order and read once per splat in depth order (32 bytes, one aligned load
// pair): the mean, the factors (l11 = 0 marks a splat that keeps its whole
// rectangle) and T, and the rectangle. vmax and vL are recomputed from these
// by the same operations.
struct alignas(16) CullRec {
    float mx, my, l11, l21, l22, T;
    ushort4 rect;  // tx0, ty0, tx1, ty1
};

__device__ __forceinline__ bool finite_f(float x) { return __builtin_isfinite(x); }

// vmax and vL from l21, l22 and T.
__device__ __forceinline__ void ellipse_extents(CullEllipse& E)
{
#pragma clang fp contract(off)
    const float sT = __builtin_sqrtf(E.T);
    E.vmax = sT / E.l22;
    const float nrm = __builtin_sqrtf(E.l21 * E.l21 + E.l22 * E.l22);
    E.vL = (sT * E.l21) / (E.l22 * nrm);
}

__device__ __forceinline__ CullEllipse ellipse_of(const CullRec& r)
{
    CullEllipse E{};
    E.mx = r.mx;
    E.my = r.my;
    E.l11 = r.l11;
    E.l21 = r.l21;
    E.l22 = r.l22;
    E.T = r.T;
    E.mode = r.l11 > 0.0f ? kCullRows : kCullRect;
    if (E.mode == kCullRows) ellipse_extents(E);
    return E;
}

__device__ __forceinline__ CullEllipse cull_ellipse(float2 m, float a, float b, float c, float o)
{
#pragma clang fp contract(off)
    CullEllipse E{};
    E.mx = m.x;
    E.my = m.y;
    const float y = 255.0f * o;
    if (!(y >= 1.0f)) {  // also NaN
        E.mode = kCullNone;
        return E;
    }
    // y = m2 2^e2 from its bit pattern (y >= 1 is normal; an infinite y gives
    // an unusable ellipse below)
    const unsigned yb = __float_as_uint(y);
    const float e2 = (float)((int)(yb >> 23) - 127);
    const float m2 = __uint_as_float((yb & 0x7fffffu) | 0x3f800000u);
    const float ln2_up = 0x1.62e430p-1f;  // float32 nearest ln 2, above it
    const float lnb = e2 * ln2_up + (m2 - 1.0f) / __builtin_sqrtf(m2);
    float T = 2.0f * lnb;
    T = (T + T * 0x1p-10f) + 0x1p-10f;
    E.T = T;
    E.l11 = __builtin_sqrtf(a);
    E.l21 = b / E.l11;
    E.l22 = __builtin_sqrtf(fmaxf(c - E.l21 * E.l21, 0.0f));
    ellipse_extents(E);
    const bool usable = finite_f(y) && finite_f(T) && finite_f(E.l11) && finite_f(E.l21) && finite_f(E.l22) &&
                        finite_f(E.vmax) && finite_f(E.vL) && E.l11 > 0.0f && E.l22 > 0.0f && finite_f(m.x) &&
                        finite_f(m.y);
    E.mode = usable ? kCullRows : kCullRect;
    return E;
}

// The kept columns [x, y] of tile row ty within [tx0, tx1) (x > y: none).
__device__ __forceinline__ int2 cull_row(const CullEllipse E, int ty, int tx0, int tx1)
{
#pragma clang fp contract(off)
    if (E.mode != kCullRows) return E.mode == kCullRect ? make_int2(tx0, tx1 - 1) : make_int2(tx1, tx1 - 1);
    const float v0 = ((float)ty * 16.0f + 0.5f) - E.my;
    const float v1 = v0 + 15.0f;
    const float lo = fmaxf(v0, -E.vmax), hi = fminf(v1, E.vmax);
    if (!(lo <= hi)) return make_int2(tx1, tx1 - 1);
    const float vl = fminf(fmaxf(E.vL, lo), hi);
    const float vr = fminf(fmaxf(-E.vL, lo), hi);
    const float tl = E.l22 * vl;
    const float sl = __builtin_sqrtf(fmaxf(E.T - tl * tl, 0.0f));
    const float xl = E.mx + (-(E.l21 * vl) - sl) / E.l11;
    const float tr = E.l22 * vr;
    const float sr = __builtin_sqrtf(fmaxf(E.T - tr * tr, 0.0f));
    const float xr = E.mx + (-(E.l21 * vr) + sr) / E.l11;
    const float f0 = (float)tx0, f1 = (float)tx1;
    // smallest c with 16 c + 15.5 >= xl, largest with 16 c + 0.5 <= xr: an
    // estimate clamped near the rectangle, then corrected by one either way
    float cl = fminf(fmaxf(ceilf((xl - 15.5f) * 0.0625f), f0 - 1.0f), f1 + 1.0f);
    if ((cl - 1.0f) * 16.0f + 15.5f >= xl) cl = cl - 1.0f;
    if (cl * 16.0f + 15.5f < xl) cl = cl + 1.0f;
    float ch = fminf(fmaxf(floorf((xr - 0.5f) * 0.0625f), f0 - 2.0f), f1);
    if ((ch + 1.0f) * 16.0f + 0.5f <= xr) ch = ch + 1.0f;
    if (ch * 16.0f + 0.5f > xr) ch = ch - 1.0f;
    return make_int2(max((int)cl, tx0), min((int)ch, tx1 - 1));
}

// One splat's counts and emission record (count_kernel below); returns its
// kept count.
__device__ __forceinline__ unsigned count_splat(int i, const float2* __restrict__ means,
                                                const float* __restrict__ conics,
                                                const float* __restrict__ opacities, const int* __restrict__ radii,
                                                const float* __restrict__ depths, int GX, int GY,
                                                unsigned* __restrict__ counts, unsigned* __restrict__ kept,
                                                CullRec& r)
{
    const float2 m = means[i];
    int tx0, tx1, ty0, ty1;
    const bool live = splat_rect(m.x, m.y, radii[i], depths[i], GX, GY, tx0, tx1, ty0, ty1);
    unsigned k = 0;
    r = CullRec{};
    if (live) {
        const CullEllipse E = cull_ellipse(m, conics[3 * i], conics[3 * i + 1], conics[3 * i + 2], opacities[i]);
        for (int ty = ty0; ty < ty1; ++ty) {
            const int2 cr = cull_row(E, ty, tx0, tx1);
            k += cr.y >= cr.x ? (unsigned)(cr.y - cr.x + 1) : 0u;
        }
        r.mx = E.mx;
        r.my = E.my;
        r.l11 = E.mode == kCullRows ? E.l11 : 0.0f;
        r.l21 = E.l21;
        r.l22 = E.l22;
        r.T = E.T;
        r.rect = make_ushort4((unsigned short)tx0, (unsigned short)ty0, (unsigned short)tx1, (unsigned short)ty1);
    }
    counts[i] = live ? (unsigned)((tx1 - tx0) * (ty1 - ty0)) : 0u;  // at most 2048 x 2048
    kept[i] = k;
    return k;
}

// counts[i] = number of tiles of splat i's rectangle, kept[i] = the number of
// them its culling ellipse keeps; recs[i] = what the emission needs (the
// rectangle (tx0, ty0, tx1, ty1), empty for a culled splat: a grid has at
// most 2048 tiles per side, so 16 bits per bound suffice).
__global__ __launch_bounds__(256) void count_kernel(int n, const float2* __restrict__ means,
                                                    const float* __restrict__ conics,
                                                    const float* __restrict__ opacities,
                                                    const int* __restrict__ radii,
                                                    const float* __restrict__ depths, int GX, int GY,
                                                    unsigned* __restrict__ counts, unsigned* __restrict__ kept,
                                                    CullRec* __restrict__ recs)
{
    // the block's records go out through LDS as consecutive 16-byte stores by
    // consecutive threads (not two per thread at a 32-byte stride)
    __shared__ float4 buf[2 * 256];
    const int i0 = blockIdx.x * 256, i = i0 + threadIdx.x;
    CullRec r{};
    if (i < n) count_splat(i, means, conics, opacities, radii, depths, GX, GY, counts, kept, r);
    static_assert(sizeof(CullRec) == 2 * sizeof(float4), "two float4 per record");
    const float4* rv = reinterpret_cast<const float4*>(&r);
    buf[2 * threadIdx.x + 0] = rv[0];
    buf[2 * threadIdx.x + 1] = rv[1];
    __syncthreads();
    const int cnt = 2 * min(256, n - i0);
    float4* const out = reinterpret_cast<float4*>(recs + i0);
    for (int k = threadIdx.x; k < cnt; k += 256) out[k] = buf[k];
}

// ---------------------------------------------------------------------------
// Device-wide exclusive scan of 32-bit items (2 kernels): per-workgroup totals,
// then a per-workgroup scan seeded with the sum of the earlier totals. Thread
// t of workgroup b holds items 1024 b + 4 t .. + 3 (one 16-byte load and
// store: consecutive threads, consecutive addresses). Sums are carried in
// 64 bits; the outputs are their low 32 bits (exact whenever the total fits,
// which the callers check before using them).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint4 load_items4(const unsigned* __restrict__ in, long long idx, long long n)
{
    if (idx + 4 <= n) return *reinterpret_cast<const uint4*>(in + idx);  // arrays are 256-byte aligned
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (idx < n) v.x = in[idx];
    if (idx + 1 < n) v.y = in[idx + 1];
    if (idx + 2 < n) v.z = in[idx + 2];
    return v;
}

__global__ __launch_bounds__(kScanThreads) void scan_reduce_kernel(const unsigned* __restrict__ in, long long n,
                                                                   unsigned long long* __restrict__ part)
{
    __shared__ unsigned long long red[kScanThreads / kWave];
    const uint4 v = load_items4(in, (long long)blockIdx.x * kScanTile + kScanItems * threadIdx.x, n);
    unsigned long long s = (unsigned long long)v.x + v.y + v.z + v.w;
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
    __syncthreads();
    if (threadIdx.x == 0) part[blockIdx.x] = red[0] + red[1] + red[2] + red[3];
}

// Workgroup-wide inclusive scan of one value per thread (256 threads).
__device__ __forceinline__ unsigned long long block_incl_scan(unsigned long long v, unsigned long long* wsum)
{
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    for (int off = 1; off < 64; off <<= 1) {
        const unsigned long long t = __shfl_up(v, off, 64);
        if (lane >= off) v += t;
    }
    if (lane == 63) wsum[w] = v;
    __syncthreads();
    unsigned long long pre = 0;
    for (int k = 0; k < w; ++k) pre += wsum[k];
    return v + pre;
}

// Second kernel of the scan: workgroup b first sums the per-workgroup totals
// part[0..b) itself (a few thousand at most, so this costs less than a
// separate scan of them would cost in launch latency), then scans its tile;
// the last workgroup also writes the grand total to *total (if not null).
// in == out is allowed (each workgroup reads its items before writing them).
__global__ __launch_bounds__(kScanThreads) void scan_down_kernel(const unsigned* in, unsigned* out, long long n,
                                                                 const unsigned long long* __restrict__ part,
                                                                 int m, unsigned long long* __restrict__ total)
{
    __shared__ unsigned long long wsum[kScanThreads / kWave];
    __shared__ unsigned long long red[kScanThreads / kWave];
    const long long idx = (long long)blockIdx.x * kScanTile + kScanItems * threadIdx.x;
    const uint4 v = load_items4(in, idx, n);
    unsigned long long pre = 0;
    for (int k = threadIdx.x; k < (int)blockIdx.x; k += kScanThreads) pre += part[k];
    for (int off = 32; off > 0; off >>= 1) pre += __shfl_xor(pre, off, 64);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = pre;
    __syncthreads();
    pre = red[0] + red[1] + red[2] + red[3];
    if (total && threadIdx.x == 0 && (int)blockIdx.x == m - 1) *total = pre + part[blockIdx.x];
    const unsigned long long s = (unsigned long long)v.x + v.y + v.z + v.w;
    const unsigned long long incl = block_incl_scan(s, wsum);
    uint4 o;
    o.x = (unsigned)(pre + incl - s);
    o.y = o.x + v.x;
    o.z = o.y + v.y;
    o.w = o.z + v.z;
    if (idx + 4 <= n) {
        *reinterpret_cast<uint4*>(out + idx) = o;
    } else {
        if (idx < n) out[idx] = o.x;
        if (idx + 1 < n) out[idx + 1] = o.y;
        if (idx + 2 < n) out[idx + 2] = o.z;
    }
}

hipError_t exclusive_scan(const unsigned* in, unsigned* out, long long n, unsigned long long* part,
                          unsigned long long* total, hipStream_t st)
{
    const int m = (int)((n + kScanTile - 1) / kScanTile);
    if (m == 0) return hipMemsetAsync(total, 0, sizeof(unsigned long long), st);
    scan_reduce_kernel<<<m, kScanThreads, 0, st>>>(in, n, part);
    scan_down_kernel<<<m, kScanThreads, 0, st>>>(in, out, n, part, m, total);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Depth order and emission.
// ---------------------------------------------------------------------------

// Emission: one thread per depth rank k. The splat of rank k writes its kept
// tiles, row by row and left to right, from emit_off[k], as (tile id, splat
// id): the rows' columns by the same operations on the same values as in the
// count pass, whose kept count also bounds the writes.
template <typename K>
__global__ __launch_bounds__(256) void emit_kernel(int n, const int* __restrict__ by_depth,
                                                   const unsigned* __restrict__ cnt_sorted,
                                                   const unsigned* __restrict__ emit_off,
                                                   const CullRec* __restrict__ recs, int GX,
                                                   K* __restrict__ keys, int* __restrict__ vals)
{
    const int k = blockIdx.x * blockDim.x + threadIdx.x;
    if (k >= n) return;
    const unsigned cnt = cnt_sorted[k];
    if (cnt == 0) return;
    const int i = by_depth[k];
    const CullRec r = recs[i];
    const ushort4 b = r.rect;
    unsigned p = emit_off[k];  // the pair count is below 2^31 here (checked before emission)
    const unsigned pend = p + cnt;
    const CullEllipse E = ellipse_of(r);
    for (int ty = b.y; ty < (int)b.w && p < pend; ++ty) {
        const int2 cr = cull_row(E, ty, b.x, b.z);
        for (int c = cr.x; c <= cr.y && p < pend; ++c, ++p) {
            keys[p] = (K)(ty * GX + c);
            vals[p] = i;
        }
    }
}

// ---------------------------------------------------------------------------
// Stable LSD radix sort pass over digit [shift, shift + BITS), BITS <= 8.
// hist: per workgroup digit counts, stored digit-major (digit * nwg + wg) so
// that one exclusive scan yields every workgroup's output offset per digit.
// ---------------------------------------------------------------------------
template <typename K, int BITS, int W>
__global__ __launch_bounds__(SortTiling<W>::kThreads) void radix_hist_kernel(const K* __restrict__ keys, long long n,
                                                                             int shift, int nwg,
                                                                             unsigned* __restrict__ hist)
{
    constexpr int R = 1 << BITS;
    constexpr int kSortWaves = W, kSortThreads = SortTiling<W>::kThreads, kSortTile = SortTiling<W>::kTile;
    __shared__ unsigned h[kSortWaves][R];  // one copy per wave: fewer lanes per address
    for (int k = threadIdx.x; k < kSortWaves * R; k += kSortThreads) (&h[0][0])[k] = 0;
    __syncthreads();
    const int w = threadIdx.x >> 6;
    const long long base = (long long)blockIdx.x * kSortTile;
    // every key of the thread requested before the first count (one wait)
    K key[kSortRounds];
    const bool full = base + kSortTile <= n;
#pragma unroll
    for (int r = 0; r < kSortRounds; ++r) {
        const long long idx = base + (long long)r * kSortThreads + threadIdx.x;
        key[r] = full || idx < n ? keys[idx] : K(0);
    }
#pragma unroll
    for (int r = 0; r < kSortRounds; ++r) {
        const long long idx = base + (long long)r * kSortThreads + threadIdx.x;
        if (full || idx < n) atomicAdd(&h[w][(unsigned)(key[r] >> shift) & (R - 1)], 1u);
    }
    __syncthreads();
    const int d = threadIdx.x;
    if (d < R) {
        unsigned c = 0;
#pragma unroll
        for (int k = 0; k < kSortWaves; ++k) c += h[k][d];
        hist[(long long)d * nwg + blockIdx.x] = c;
    }
}

// Scatter of one pass. The workgroup's keys are first ranked stably by digit
// and placed in LDS in digit order; the tile is then written out from LDS, so
// that consecutive threads store consecutive addresses inside each digit's
// run instead of one key at a time into up to 256 different runs.
// Ranking: wave w holds the tile's keys 1024 w .. 1024 w + 1023, 64 per round
// (round r: keys 1024 w + 64 r + lane). Within a round, BITS ballots give each
// lane its rank among the wave's lanes with the same digit; a per-wave running
// count per digit (read by those lanes, then advanced by the first of them:
// LDS operations of one wave take effect in order) carries the rank across
// the wave's rounds, with no workgroup barrier. After the rounds, each digit's
// block-local start and each wave's offset inside it come from one scan; as
// the waves hold consecutive parts of the tile, wave order then round order
// is the tile's order: the placement is stable.
template <typename K, int BITS, int W>
__global__ __launch_bounds__(SortTiling<W>::kThreads) void radix_scatter_kernel(const K* __restrict__ keys_in,
                                                                                const int* __restrict__ vals_in,
                                                                                long long n, int shift, int nwg,
                                                                                const unsigned* __restrict__ offs,
                                                                                K* __restrict__ keys_out,
                                                                                int* __restrict__ vals_out,
                                                                                const unsigned* __restrict__ gat_in,
                                                                                unsigned* __restrict__ gat_out)
{
    constexpr int R = 1 << BITS;
    constexpr int kSortWaves = W, kSortThreads = SortTiling<W>::kThreads, kSortTile = SortTiling<W>::kTile;
    __shared__ unsigned wave_run[kSortWaves][R];  // per wave: keys of digit d ranked so far, then its offset
    __shared__ unsigned local_start[R];           // block-local start of digit d
    __shared__ unsigned global_off[R];
    __shared__ unsigned scan_part[kSortWaves];
    __shared__ K lkey[kSortTile];
    __shared__ int lval[kSortTile];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const long long base = (long long)blockIdx.x * kSortTile;
    const int cnt = (int)(n - base < (long long)kSortTile ? n - base : (long long)kSortTile);
    const int td = threadIdx.x;  // thread td < R looks after digit td
    const bool has_digit = td < R;
    K key[kSortRounds];
    int val[kSortRounds];
    unsigned rk[kSortRounds];  // rank among the wave's keys of the same digit
    for (int k = lane; k < R; k += kWave) wave_run[w][k] = 0u;  // each wave clears its own row
    const unsigned goff = has_digit ? offs[(long long)td * nwg + blockIdx.x] : 0u;  // stored after the ranking
    const int wbase = w * (kSortTile / kSortWaves);  // this wave's part of the tile
    // all loads issued before the first use (the branches are uniform)
    const bool full = cnt == kSortTile;
#pragma unroll
    for (int r = 0; r < kSortRounds; ++r) {
        const int li = wbase + r * kWave + lane;
        key[r] = full || li < cnt ? keys_in[base + li] : K(0);
    }
    if (vals_in) {
#pragma unroll
        for (int r = 0; r < kSortRounds; ++r) {
            const int li = wbase + r * kWave + lane;
            val[r] = full || li < cnt ? vals_in[base + li] : 0;
        }
    } else {  // no values: the index
#pragma unroll
        for (int r = 0; r < kSortRounds; ++r) val[r] = (int)(base + wbase + r * kWave + lane);
    }
    const unsigned long long lt_mask = (1ull << lane) - 1ull;
#pragma unroll
    for (int r = 0; r < kSortRounds; ++r) {
        const bool valid = wbase + r * kWave + lane < cnt;
        const unsigned d = valid ? (unsigned)(key[r] >> shift) & (R - 1) : 0u;
        unsigned long long peers = __ballot(valid);
#pragma unroll
        for (int b = 0; b < BITS; ++b) {
            const bool bit = (d >> b) & 1u;
            const unsigned long long bal = __ballot(bit);
            peers &= bit ? bal : ~bal;
        }
        const unsigned rank = (unsigned)__popcll(peers & lt_mask);
        const unsigned before = valid ? wave_run[w][d] : 0u;
        rk[r] = before + rank;
        if (valid && rank == 0) wave_run[w][d] = before + (unsigned)__popcll(peers);
    }
    if (has_digit) global_off[td] = goff;
    __syncthreads();
    // digit td: its count over the tile, the exclusive scan of the counts over
    // the digits, and each wave's offset inside the digit's run
    unsigned c[kSortWaves];
    unsigned tot = 0;
#pragma unroll
    for (int k = 0; k < kSortWaves; ++k) {
        c[k] = has_digit ? wave_run[k][td] : 0u;
        tot += c[k];
    }
    unsigned incl = tot;
    for (int dl = 1; dl < kWave; dl <<= 1) {
        const unsigned u = __shfl_up(incl, dl, kWave);
        if (lane >= dl) incl += u;
    }
    if (lane == kWave - 1) scan_part[w] = incl;
    __syncthreads();
    unsigned before_w = 0;
    for (int k = 0; k < w; ++k) before_w += scan_part[k];
    const unsigned start = before_w + incl - tot;
    if (has_digit) {
        local_start[td] = start;
        unsigned run = start;
#pragma unroll
        for (int k = 0; k < kSortWaves; ++k) {
            wave_run[k][td] = run;
            run += c[k];
        }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kSortRounds; ++r) {
        if (wbase + r * kWave + lane < cnt) {
            const unsigned d = (unsigned)(key[r] >> shift) & (R - 1);
            const unsigned lp = wave_run[w][d] + rk[r];
            lkey[lp] = key[r];
            lval[lp] = val[r];
        }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kSortRounds; ++r) {
        const int lp = r * kSortThreads + threadIdx.x;
        if (lp < cnt) {
            const K k = lkey[lp];
            const unsigned d = (unsigned)(k >> shift) & (R - 1);
            const unsigned pos = global_off[d] + ((unsigned)lp - local_start[d]);
            keys_out[pos] = k;
            const int v = lval[lp];
            vals_out[pos] = v;
            if (gat_out) gat_out[pos] = gat_in[v];  // a word of the value's, into the output order
        }
    }
}

// Tile ranges from the boundaries of the sorted tile keys. Thread i takes keys
// 4 i .. 4 i + 3 (one vector load) and their two neighbours.
template <typename K>
struct alignas(4 * sizeof(K)) Keys4 {
    K v[4];
};

template <typename K>
__global__ __launch_bounds__(256) void ranges_kernel(const K* __restrict__ keys, long long n, int tiles,
                                                     int2* __restrict__ ranges)
{
    const long long i0 = 4 * ((long long)blockIdx.x * blockDim.x + threadIdx.x);
    if (i0 >= n) return;
    int k[4];
    if (i0 + 4 <= n) {
        const Keys4<K> v = *reinterpret_cast<const Keys4<K>*>(keys + i0);  // keys are 256-byte aligned
#pragma unroll
        for (int j = 0; j < 4; ++j) k[j] = (int)v.v[j];
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) k[j] = i0 + j < n ? (int)keys[i0 + j] : -1;
    }
    int prev = i0 > 0 ? (int)keys[i0 - 1] : -1;
    const int next = i0 + 4 < n ? (int)keys[i0 + 4] : -1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const long long i = i0 + j;
        if (i >= n) break;
        const int t = k[j];
        const bool in = (unsigned)t < (unsigned)tiles;  // every emitted key is; bounds the writes regardless
        if (t != prev && in) ranges[t].x = (int)i;
        const int nx = j < 3 && i + 1 < n ? k[j + 1] : (j < 3 ? -1 : next);
        if (nx != t && in) ranges[t].y = (int)(i + 1);
        prev = t;
    }
}

// After the count check: splat_offsets[i] = first slot of splat i's (splat,
// tile) pairs, [n] = the pair count (0 without splats); tile_ranges cleared
// (the ranges pass fills the non-empty tiles).
__global__ __launch_bounds__(256) void outputs_kernel(int n, int tiles, const unsigned* __restrict__ offsets,
                                                      const unsigned long long* __restrict__ pairs,
                                                      int* __restrict__ splat_offsets, int* __restrict__ tile_ranges)
{
    const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) splat_offsets[i] = (int)offsets[i];
    if (i == n) splat_offsets[n] = pairs ? (int)*pairs : 0;
    if (i < 2ll * tiles) tile_ranges[i] = 0;
}

inline size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

struct BinLayout {
    size_t counts, kept, recs, offsets, part, total, pairs, dkeys_a, dkeys_b, dvals_a, dvals_b, cnt_sorted,
        emit_off, keys_a, keys_b, vals_tmp, hist, bytes;
};

BinLayout bin_layout(long long n, long long cap)
{
    BinLayout L{};
    size_t o = 0;
    const long long nmax = n > cap ? n : cap;
    const long long nwg_sort = (nmax + kSortTileMin - 1) / kSortTileMin;  // the most workgroups a sort uses
    const long long scan_items = n > (long long)kRadix * nwg_sort ? n : (long long)kRadix * nwg_sort;
    const long long nparts = (scan_items + kScanTile - 1) / kScanTile + 1;
    const size_t n1 = (size_t)(n > 0 ? n : 1), c1 = (size_t)(cap > 0 ? cap : 1);
    L.counts = o;     o += align256(sizeof(unsigned) * n1);
    L.kept = o;       o += align256(sizeof(unsigned) * n1);
    L.recs = o;       o += align256(sizeof(CullRec) * n1);
    L.offsets = o;    o += align256(sizeof(unsigned) * n1);
    L.part = o;       o += align256(sizeof(unsigned long long) * (size_t)nparts);
    L.total = o;      o += align256(sizeof(unsigned long long));
    L.pairs = o;      o += align256(2 * sizeof(unsigned long long));  // rectangle and kept pair counts, apart from the scans' totals
    L.dkeys_a = o;    o += align256(sizeof(unsigned) * n1);
    L.dkeys_b = o;    o += align256(sizeof(unsigned) * n1);
    L.dvals_a = o;    o += align256(sizeof(int) * n1);
    L.dvals_b = o;    o += align256(sizeof(int) * n1);
    L.cnt_sorted = o; o += align256(sizeof(unsigned) * n1);
    L.emit_off = o;   o += align256(sizeof(unsigned) * n1);
    L.keys_a = o;     o += align256(sizeof(unsigned) * c1);
    L.keys_b = o;     o += align256(sizeof(unsigned) * c1);
    L.vals_tmp = o;   o += align256(sizeof(int) * c1);
    L.hist = o;       o += align256(sizeof(unsigned) * (size_t)kRadix * (size_t)(nwg_sort > 0 ? nwg_sort : 1));
    L.bytes = o;
    return L;
}

// One stable LSD pass over the BITS-bit digit at `shift` of keys_in -> keys_out.
template <typename K, int BITS, int W>
hipError_t radix_pass_b(const K* kin, const int* vin, K* kout, int* vout, long long cnt, int shift, unsigned* hist,
                        unsigned long long* part, unsigned long long* total, hipStream_t st,
                        const unsigned* gat_in = nullptr, unsigned* gat_out = nullptr)
{
    constexpr int kSortThreads = SortTiling<W>::kThreads, kSortTile = SortTiling<W>::kTile;
    const int nwg = (int)((cnt + kSortTile - 1) / kSortTile);
    radix_hist_kernel<K, BITS, W><<<nwg, kSortThreads, 0, st>>>(kin, cnt, shift, nwg, hist);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = exclusive_scan(hist, hist, (long long)(1 << BITS) * nwg, part, total, st);
    if (e != hipSuccess) return e;
    radix_scatter_kernel<K, BITS, W><<<nwg, kSortThreads, 0, st>>>(kin, vin, cnt, shift, nwg, hist, kout, vout,
                                                                   gat_in, gat_out);
    return hipGetLastError();
}

template <typename K>
hipError_t radix_pass(const K* kin, const int* vin, K* kout, int* vout, long long cnt, int shift, int bits,
                      unsigned* hist, unsigned long long* part, unsigned long long* total, hipStream_t st)
{
    constexpr int W = kPairWaves;  // the pair passes
    switch (bits) {
    case 4: return radix_pass_b<K, 4, W>(kin, vin, kout, vout, cnt, shift, hist, part, total, st);
    case 5: return radix_pass_b<K, 5, W>(kin, vin, kout, vout, cnt, shift, hist, part, total, st);
    case 6: return radix_pass_b<K, 6, W>(kin, vin, kout, vout, cnt, shift, hist, part, total, st);
    case 7: return radix_pass_b<K, 7, W>(kin, vin, kout, vout, cnt, shift, hist, part, total, st);
    default: return radix_pass_b<K, 8, W>(kin, vin, kout, vout, cnt, shift, hist, part, total, st);
    }
}

// Emission, the tile passes (ping-ponged so that the last one writes its
// values into sorted_ids) and the ranges, with keys of type K.
template <typename K>
hipError_t tile_sort(int n, long long I, const int* by_depth, const unsigned* cnt_sorted, const unsigned* emit_off,
                     const CullRec* recs, int GX, int tiles, int np, int tb, K* keys_a, K* keys_b, int* vals_t,
                     int* sorted_ids, unsigned* hist, unsigned long long* part, unsigned long long* total,
                     int2* tile_ranges, hipStream_t st)
{
    K* kin = keys_a;
    K* kout = keys_b;
    int* vin = (np % 2 == 0) ? sorted_ids : vals_t;
    int* vout = (np % 2 == 0) ? vals_t : sorted_ids;
    emit_kernel<K><<<(n + 255) / 256, 256, 0, st>>>(n, by_depth, cnt_sorted, emit_off, recs, GX, kin, vin);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    int shift = 0;
    for (int p = 0; p < np; ++p) {
        // tb bits over np passes, the narrower digits first (the first pass,
        // reading the pairs in emission order, writes the most scattered runs)
        const int bits = max(4, tb / np + (p >= np - tb % np ? 1 : 0));
        e = radix_pass<K>(kin, vin, kout, vout, I, shift, bits, hist, part, total, st);
        shift += bits;
        if (e != hipSuccess) return e;
        K* tk = kin; kin = kout; kout = tk;
        int* tv = vin; vin = vout; vout = tv;
    }
    ranges_kernel<K><<<(unsigned)((I + 1023) / 1024), 256, 0, st>>>(kin, I, tiles, tile_ranges);
    return hipGetLastError();
}

int bits_for(long long v)  // smallest b with (1 << b) > v - 1, i.e. enough bits for values 0..v-1
{
    int b = 0;
    while ((1ll << b) < v) ++b;
    return b;
}

}  // namespace
}  // namespace gs

using namespace gs;

extern "C" size_t gs_bin_tiles_workspace_size(int32_t n, int64_t capacity, int32_t width, int32_t height)
{
    (void)width;
    (void)height;
    if (n < 0 || n > kMaxSplats || capacity < 0) return 0;
    return bin_layout(n, capacity).bytes;
}

namespace gs {
namespace {

// One small pinned host buffer per calling thread, for the pair count's
// readback (allocated on the thread's first call, kept until the process ends;
// pinned, so that the copy is asynchronous). nullptr if it cannot be had.
unsigned long long* pinned_count()
{
    thread_local unsigned long long* p = nullptr;
    if (!p) {
        void* q = nullptr;
        if (hipHostMalloc(&q, 64, hipHostMallocPortable) != hipSuccess) {
            (void)hipGetLastError();
            return nullptr;
        }
        p = static_cast<unsigned long long*>(q);
    }
    return p;
}

struct CountEvent {  // destroyed on every return path
    hipEvent_t e = nullptr;
    ~CountEvent()
    {
        if (e) (void)hipEventDestroy(e);
    }
};

}  // namespace
}  // namespace gs

using namespace gs;

extern "C" gs_status gs_bin_tiles(int32_t n, const float* means2d, const float* conics, const float* opacities,
                                  const int32_t* radii, const float* depths, int32_t width, int32_t height,
                                  int64_t capacity, int32_t* sorted_ids, int32_t* tile_ranges,
                                  int32_t* splat_offsets, int64_t* n_isect, int64_t* n_slots, void* workspace,
                                  size_t workspace_bytes, gs_stream_t stream_)
{
    hipStream_t st = (hipStream_t)stream_;
    GS_CHECK_ARG(n >= 0 && n <= kMaxSplats, "gs_bin_tiles: n = %d outside 0..%d", n, kMaxSplats);
    GS_CHECK_ARG(width > 0 && height > 0 && width <= kMaxDim && height <= kMaxDim,
                 "gs_bin_tiles: image size %d x %d outside 1..%d", width, height, kMaxDim);
    GS_CHECK_ARG(capacity >= 0, "gs_bin_tiles: capacity %lld < 0", (long long)capacity);
    GS_CHECK_ARG(n_isect != nullptr, "gs_bin_tiles: n_isect is NULL");
    GS_CHECK_ARG(tile_ranges != nullptr, "gs_bin_tiles: tile_ranges is NULL");
    GS_CHECK_ARG(splat_offsets != nullptr, "gs_bin_tiles: splat_offsets is NULL");
    GS_CHECK_ARG(n == 0 || (means2d && conics && opacities && radii && depths), "gs_bin_tiles: NULL splat array");
    GS_CHECK_ARG(capacity == 0 || sorted_ids != nullptr, "gs_bin_tiles: sorted_ids is NULL");
    const BinLayout L = bin_layout(n, capacity);
    GS_CHECK_ARG(workspace != nullptr && workspace_bytes >= L.bytes,
                 "gs_bin_tiles: workspace %zu bytes, need %zu", workspace_bytes, L.bytes);
    GS_CHECK_ARG(((uintptr_t)workspace & 255) == 0, "gs_bin_tiles: workspace not 256-byte aligned");

    const int GX = grid_x(width), GY = grid_y(height);
    const int tiles = GX * GY;
    char* ws = (char*)workspace;
    auto* counts = (unsigned*)(ws + L.counts);
    auto* kept = (unsigned*)(ws + L.kept);
    auto* offsets = (unsigned*)(ws + L.offsets);
    auto* part = (unsigned long long*)(ws + L.part);
    auto* total = (unsigned long long*)(ws + L.total);
    auto* recs = (CullRec*)(ws + L.recs);

    auto* pairs = (unsigned long long*)(ws + L.pairs);  // [0] rectangle pairs, [1] kept pairs
    auto* dka = (unsigned*)(ws + L.dkeys_a);
    auto* dkb = (unsigned*)(ws + L.dkeys_b);
    auto* dva = (int*)(ws + L.dvals_a);
    auto* dvb = (int*)(ws + L.dvals_b);
    auto* hist = (unsigned*)(ws + L.hist);
    auto* cnt_sorted = (unsigned*)(ws + L.cnt_sorted);
    auto* emit_off = (unsigned*)(ws + L.emit_off);
    const int* by_depth = dva;

    // Both pair counts are read back with one asynchronous copy into pinned
    // host memory, and everything that does not need them (the splats' depth
    // sort and their kept counts in depth order; workspace only) is enqueued before the host waits for that copy: the GPU stays
    // busy while the host waits and then enqueues the pair stages behind the
    // depth sort.
    unsigned long long h_tot[2] = {0, 0};
    if (n > 0) {
        count_kernel<<<(n + 255) / 256, 256, 0, st>>>(n, (const float2*)means2d, conics, opacities, radii, depths,
                                                      GX, GY, counts, kept, recs);
        GS_HIP(hipGetLastError());
        GS_HIP(exclusive_scan(counts, offsets, n, part, pairs, st));
        // the kept total (one atomic per wave into a single word serialised at
        // the L2 and doubled the binning's time); the scan's output goes to
        // emit_off, rewritten below
        GS_HIP(exclusive_scan(kept, emit_off, n, part, pairs + 1, st));
        unsigned long long* pin = pinned_count();
        CountEvent ev;
        if (pin) {
            GS_HIP(hipMemcpyAsync(pin, pairs, 2 * sizeof(*pin), hipMemcpyDeviceToHost, st));
            GS_HIP(hipEventCreateWithFlags(&ev.e, hipEventDisableTiming));
            GS_HIP(hipEventRecord(ev.e, st));
        } else {  // no pinned buffer: a plain synchronous read
            GS_HIP(hipMemcpyAsync(h_tot, pairs, sizeof(h_tot), hipMemcpyDeviceToHost, st));
            GS_HIP(hipStreamSynchronize(st));
        }
        // Splats in depth order: stable sort of (depth bits, id). The first
        // pass reads the depths' bit patterns in place, with the index as id.
        const unsigned* dk_in = reinterpret_cast<const unsigned*>(depths);
        const int* dv_in = nullptr;
        unsigned* dk_out = dkb;
        int* dv_out = dvb;
        for (int shift = 0; shift < 32; shift += kRadixBits) {
            // the last pass also gathers the kept counts into depth order
            const bool last = shift + kRadixBits >= 32;
            GS_HIP((radix_pass_b<unsigned, kRadixBits, kDepthWaves>(dk_in, dv_in, dk_out, dv_out, n, shift, hist, part,
                                                                     total, st, last ? kept : nullptr,
                                                                     last ? cnt_sorted : nullptr)));
            dk_in = dk_out;
            dv_in = dv_out;
            dk_out = dk_out == dkb ? dka : dkb;
            dv_out = dv_out == dvb ? dva : dvb;
        }
        by_depth = dv_in;
        // Emission offsets in depth order.
        GS_HIP(exclusive_scan(cnt_sorted, emit_off, n, part, total, st));
        if (pin) {
            GS_HIP(hipEventSynchronize(ev.e));
            h_tot[0] = pin[0];
            h_tot[1] = pin[1];
        }
    }
    *n_isect = (int64_t)h_tot[1];
    if (n_slots) *n_slots = (int64_t)h_tot[0];
    if (h_tot[0] > 0x7fffffffull) {  // the kept pairs are among them
        set_error("gs_bin_tiles: %llu rectangle pairs exceed the int32 index range", h_tot[0]);
        return GS_ERR_UNSUPPORTED;
    }
    if ((long long)h_tot[1] > capacity) {
        set_error("gs_bin_tiles: capacity %lld < %llu intersections", (long long)capacity, h_tot[1]);
        return GS_ERR_CAPACITY;
    }
    const long long I = (long long)h_tot[1];
    {
        const long long cover = (long long)n + 1 > 2ll * tiles ? (long long)n + 1 : 2ll * tiles;
        outputs_kernel<<<(unsigned)((cover + 255) / 256), 256, 0, st>>>(n, tiles, offsets, n > 0 ? pairs : nullptr,
                                                                        splat_offsets, tile_ranges);
        GS_HIP(hipGetLastError());
    }
    if (I == 0) return GS_OK;

    // Tile passes, ping-ponged so that the last one writes its values into
    // sorted_ids: as few passes as 8-bit digits allow, the tile id's bits
    // split as evenly as possible over them, the narrower digits first
    // (narrower digits make longer runs per digit in each workgroup's output,
    // i.e. fuller cache lines), at least 4 bits each.
    const int tb = bits_for(tiles);
    const int np = (tb + kRadixBits - 1) / kRadixBits;

    int* vals_t = (int*)(ws + L.vals_tmp);
    // 16-bit tile keys up to 65536 tiles (a quarter less traffic per pass)
    if (tiles <= 65536)
        GS_HIP(tile_sort<unsigned short>(n, I, by_depth, cnt_sorted, emit_off, recs, GX, tiles, np, tb,
                                         (unsigned short*)(ws + L.keys_a), (unsigned short*)(ws + L.keys_b), vals_t,
                                         sorted_ids, hist, part, total, (int2*)tile_ranges, st));
    else
        GS_HIP(tile_sort<unsigned>(n, I, by_depth, cnt_sorted, emit_off, recs, GX, tiles, np, tb,
                                   (unsigned*)(ws + L.keys_a), (unsigned*)(ws + L.keys_b), vals_t, sorted_ids, hist,
                                   part, total, (int2*)tile_ranges, st));
    return GS_OK;
}
