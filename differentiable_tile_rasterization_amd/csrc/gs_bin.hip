// gs_bin.hip -- gs_bin_tiles: tile binning, stable radix sort, tile ranges.
//
// Stages (the binning / sort / range kernels of the 3dgs-rs pipeline listed in
// the timing table of "Phase 5 step 30b — kernel-by-kernel timing", section
// 計測結果: emit_pairs, radix_hist, radix_scatter, extract_offsets):
//   1. count   one thread per splat: float32 tile rectangle, number of tiles
//   2. scan    exclusive prefix sum of the counts (device-wide, 64-bit)
//   3. host    read the total back (the call's only synchronisation)
//   4. emit    one thread per splat writes (tile << 32 | depth bits, id) for its
//              tiles, row-major, at its scan offset: the pair order is
//              deterministic (no atomic counter)
//   5. sort    stable LSD radix sort, 8-bit digits, over only the key bits that
//              can be non-zero: 31 depth bits (depth > 0, so the sign bit is 0)
//              and ceil(log2(tiles)) tile bits. Stability plus emission in
//              splat order makes equal depths come out by ascending splat id.
//   6. ranges  [start, end) per tile from the boundaries of the sorted keys
#include "gs_common.hpp"

namespace gs {
namespace {

constexpr int kScanThreads = 256;
constexpr int kScanItems = 16;                        // per thread
constexpr int kScanTile = kScanThreads * kScanItems;  // 4096 items per workgroup

constexpr int kSortThreads = 256;
constexpr int kSortRounds = 16;                       // rounds of 256 keys per workgroup
constexpr int kSortTile = kSortThreads * kSortRounds; // 4096 keys per workgroup
constexpr int kRadixBits = 8;
constexpr int kRadix = 1 << kRadixBits;

__device__ __forceinline__ bool splat_rect(float mx, float my, int r, float depth, int GX, int GY,
                                           int& tx0, int& tx1, int& ty0, int& ty1)
{
    tile_rect(mx, my, r, GX, GY, tx0, tx1, ty0, ty1);
    const bool live = r > 0 && depth > 0.0f && __builtin_isfinite(mx) && __builtin_isfinite(my);
    return live && tx1 > tx0 && ty1 > ty0;
}

__global__ __launch_bounds__(256) void count_kernel(int n, const float2* __restrict__ means,
                                                    const int* __restrict__ radii,
                                                    const float* __restrict__ depths, int GX, int GY,
                                                    unsigned long long* __restrict__ counts)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const float2 m = means[i];
    int tx0, tx1, ty0, ty1;
    const bool live = splat_rect(m.x, m.y, radii[i], depths[i], GX, GY, tx0, tx1, ty0, ty1);
    counts[i] = live ? (unsigned long long)(tx1 - tx0) * (unsigned long long)(ty1 - ty0) : 0ull;
}

// ---------------------------------------------------------------------------
// Device-wide exclusive scan (3 kernels): per-workgroup totals, a one-workgroup
// scan of those totals, then a per-workgroup scan seeded with its offset.
// T is the element type (uint32 or uint64); sums are carried in uint64.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kScanThreads) void scan_reduce_kernel(const T* __restrict__ in, long long n,
                                                                   unsigned long long* __restrict__ part)
{
    __shared__ unsigned long long red[kScanThreads / kWave];
    const long long base = (long long)blockIdx.x * kScanTile;
    unsigned long long s = 0;
#pragma unroll
    for (int k = 0; k < kScanItems; ++k) {
        const long long idx = base + (long long)k * kScanThreads + threadIdx.x;
        if (idx < n) s += (unsigned long long)in[idx];
    }
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
    __syncthreads();
    if (threadIdx.x == 0) part[blockIdx.x] = red[0] + red[1] + red[2] + red[3];
}

// One workgroup: exclusive scan of part[0..m) in place; grand total to *total.
__global__ __launch_bounds__(kScanThreads) void scan_parts_kernel(unsigned long long* __restrict__ part, int m,
                                                                  unsigned long long* __restrict__ total)
{
    __shared__ unsigned long long buf[kScanThreads];
    __shared__ unsigned long long carry;
    if (threadIdx.x == 0) carry = 0;
    __syncthreads();
    for (int base = 0; base < m; base += kScanThreads) {
        const int i = base + threadIdx.x;
        const unsigned long long v = i < m ? part[i] : 0ull;
        buf[threadIdx.x] = v;
        __syncthreads();
        for (int off = 1; off < kScanThreads; off <<= 1) {
            const unsigned long long t = threadIdx.x >= off ? buf[threadIdx.x - off] : 0ull;
            __syncthreads();
            buf[threadIdx.x] += t;
            __syncthreads();
        }
        const unsigned long long incl = buf[threadIdx.x];
        const unsigned long long c = carry;
        if (i < m) part[i] = c + incl - v;
        __syncthreads();
        if (threadIdx.x == kScanThreads - 1) carry = c + incl;
        __syncthreads();
    }
    if (threadIdx.x == 0 && total) *total = carry;
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

template <typename TI, typename TO>
__global__ __launch_bounds__(kScanThreads) void scan_down_kernel(const TI* __restrict__ in, TO* __restrict__ out,
                                                                 long long n,
                                                                 const unsigned long long* __restrict__ part)
{
    __shared__ unsigned long long wsum[kScanThreads / kWave];
    // Blocked arrangement: thread t owns items [t*16, t*16+16) of the tile.
    const long long base = (long long)blockIdx.x * kScanTile + (long long)threadIdx.x * kScanItems;
    unsigned long long v[kScanItems];
    unsigned long long s = 0;
#pragma unroll
    for (int k = 0; k < kScanItems; ++k) {
        const long long idx = base + k;
        v[k] = idx < n ? (unsigned long long)in[idx] : 0ull;
        s += v[k];
    }
    const unsigned long long incl = block_incl_scan(s, wsum);
    unsigned long long run = part[blockIdx.x] + incl - s;
#pragma unroll
    for (int k = 0; k < kScanItems; ++k) {
        const long long idx = base + k;
        if (idx < n) out[idx] = (TO)run;
        run += v[k];
    }
}

template <typename TI, typename TO>
hipError_t exclusive_scan(const TI* in, TO* out, long long n, unsigned long long* part,
                          unsigned long long* total, hipStream_t st)
{
    const int m = (int)((n + kScanTile - 1) / kScanTile);
    if (m == 0) return hipMemsetAsync(total, 0, sizeof(unsigned long long), st);
    scan_reduce_kernel<TI><<<m, kScanThreads, 0, st>>>(in, n, part);
    scan_parts_kernel<<<1, kScanThreads, 0, st>>>(part, m, total);
    scan_down_kernel<TI, TO><<<m, kScanThreads, 0, st>>>(in, out, n, part);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Emit: splat i writes its tiles, row-major, at offsets[i].
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void emit_kernel(int n, const float2* __restrict__ means,
                                                   const int* __restrict__ radii,
                                                   const float* __restrict__ depths, int GX, int GY,
                                                   const unsigned long long* __restrict__ offsets,
                                                   unsigned long long* __restrict__ keys,
                                                   int* __restrict__ vals)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const float2 m = means[i];
    const float d = depths[i];
    int tx0, tx1, ty0, ty1;
    if (!splat_rect(m.x, m.y, radii[i], d, GX, GY, tx0, tx1, ty0, ty1)) return;
    const unsigned long long dbits = (unsigned long long)__float_as_uint(d);
    unsigned long long o = offsets[i];
    for (int ty = ty0; ty < ty1; ++ty)
        for (int tx = tx0; tx < tx1; ++tx) {
            keys[o] = ((unsigned long long)(ty * GX + tx) << 32) | dbits;
            vals[o] = i;
            ++o;
        }
}

// ---------------------------------------------------------------------------
// Stable LSD radix sort pass over digit [shift, shift + 8).
// hist: per workgroup digit counts, stored digit-major (digit * nwg + wg) so
// that one exclusive scan yields every workgroup's output offset per digit.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kSortThreads) void radix_hist_kernel(const unsigned long long* __restrict__ keys,
                                                                  long long n, int shift, int nwg,
                                                                  unsigned* __restrict__ hist)
{
    __shared__ unsigned h[4][kRadix];
    for (int k = threadIdx.x; k < 4 * kRadix; k += kSortThreads) (&h[0][0])[k] = 0;
    __syncthreads();
    const int w = threadIdx.x >> 6;
    const long long base = (long long)blockIdx.x * kSortTile;
    for (int r = 0; r < kSortRounds; ++r) {
        const long long idx = base + (long long)r * kSortThreads + threadIdx.x;
        if (idx < n) {
            const unsigned d = (unsigned)(keys[idx] >> shift) & (kRadix - 1);
            atomicAdd(&h[w][d], 1u);
        }
    }
    __syncthreads();
    const int d = threadIdx.x;  // kSortThreads == kRadix
    hist[(long long)d * nwg + blockIdx.x] = h[0][d] + h[1][d] + h[2][d] + h[3][d];
}

__global__ __launch_bounds__(kSortThreads) void radix_scatter_kernel(
    const unsigned long long* __restrict__ keys_in, const int* __restrict__ vals_in, long long n, int shift,
    int nwg, const unsigned* __restrict__ offs, unsigned long long* __restrict__ keys_out,
    int* __restrict__ vals_out)
{
    __shared__ unsigned wave_cnt[4][kRadix];  // keys of digit d in wave w, this round
    __shared__ unsigned wave_off[4][kRadix];  // where wave w's keys of digit d start
    __shared__ unsigned running[kRadix];      // keys of digit d placed by earlier rounds
    __shared__ unsigned global_off[kRadix];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    {
        const int d = threadIdx.x;
        running[d] = 0;
        global_off[d] = offs[(long long)d * nwg + blockIdx.x];
        for (int k = 0; k < 4; ++k) wave_cnt[k][d] = 0;
    }
    __syncthreads();
    const unsigned long long lt_mask = (1ull << lane) - 1ull;
    const long long base = (long long)blockIdx.x * kSortTile;
    for (int r = 0; r < kSortRounds; ++r) {
        const long long idx = base + (long long)r * kSortThreads + threadIdx.x;
        const bool valid = idx < n;
        unsigned long long key = 0;
        int val = 0;
        unsigned d = 0;
        if (valid) {
            key = keys_in[idx];
            val = vals_in[idx];
            d = (unsigned)(key >> shift) & (kRadix - 1);
        }
        // lanes of this wave holding the same digit (8 ballots)
        unsigned long long peers = __ballot(valid);
#pragma unroll
        for (int b = 0; b < kRadixBits; ++b) {
            const bool bit = (d >> b) & 1u;
            const unsigned long long bal = __ballot(bit);
            peers &= bit ? bal : ~bal;
        }
        const unsigned rank = (unsigned)__popcll(peers & lt_mask);
        if (valid && rank == 0) wave_cnt[w][d] = (unsigned)__popcll(peers);
        __syncthreads();
        {
            const int dd = threadIdx.x;
            unsigned run = running[dd];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                wave_off[k][dd] = run;
                run += wave_cnt[k][dd];
                wave_cnt[k][dd] = 0;
            }
            running[dd] = run;
        }
        __syncthreads();
        if (valid) {
            const unsigned pos = global_off[d] + wave_off[w][d] + rank;
            keys_out[pos] = key;
            vals_out[pos] = val;
        }
    }
}

__global__ __launch_bounds__(256) void ranges_kernel(const unsigned long long* __restrict__ keys, long long n,
                                                     int2* __restrict__ ranges)
{
    const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const int t = (int)(keys[i] >> 32);
    if (i == 0 || (int)(keys[i - 1] >> 32) != t) ranges[t].x = (int)i;
    if (i == n - 1 || (int)(keys[i + 1] >> 32) != t) ranges[t].y = (int)(i + 1);
}

// splat_offsets[i] = first slot of splat i's (splat, tile) pairs, [n] = total.
__global__ __launch_bounds__(256) void offsets_kernel(int n, const unsigned long long* __restrict__ offsets,
                                                      const unsigned long long* __restrict__ total,
                                                      int* __restrict__ splat_offsets)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) splat_offsets[i] = (int)offsets[i];
    if (i == n) splat_offsets[n] = (int)*total;
}

inline size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

struct BinLayout {
    size_t counts, offsets, part, total, keys_a, keys_b, vals_tmp, hist, bytes;
};

BinLayout bin_layout(long long n, long long cap)
{
    BinLayout L{};
    size_t o = 0;
    const long long nwg_sort = (cap + kSortTile - 1) / kSortTile;
    const long long scan_items = n > (long long)kRadix * nwg_sort ? n : (long long)kRadix * nwg_sort;
    const long long nparts = (scan_items + kScanTile - 1) / kScanTile + 1;
    L.counts = o;   o += align256(sizeof(unsigned long long) * (size_t)(n > 0 ? n : 1));
    L.offsets = o;  o += align256(sizeof(unsigned long long) * (size_t)(n > 0 ? n : 1));
    L.part = o;     o += align256(sizeof(unsigned long long) * (size_t)nparts);
    L.total = o;    o += align256(sizeof(unsigned long long));
    L.keys_a = o;   o += align256(sizeof(unsigned long long) * (size_t)(cap > 0 ? cap : 1));
    L.keys_b = o;   o += align256(sizeof(unsigned long long) * (size_t)(cap > 0 ? cap : 1));
    L.vals_tmp = o; o += align256(sizeof(int) * (size_t)(cap > 0 ? cap : 1));
    L.hist = o;     o += align256(sizeof(unsigned) * (size_t)kRadix * (size_t)(nwg_sort > 0 ? nwg_sort : 1));
    L.bytes = o;
    return L;
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
    if (n < 0 || capacity < 0) return 0;
    return bin_layout(n, capacity).bytes;
}

extern "C" gs_status gs_bin_tiles(int32_t n, const float* means2d, const int32_t* radii, const float* depths,
                                  int32_t width, int32_t height, int64_t capacity, int32_t* sorted_ids,
                                  int32_t* tile_ranges, int32_t* splat_offsets, int64_t* n_isect,
                                  void* workspace, size_t workspace_bytes, gs_stream_t stream_)
{
    hipStream_t st = (hipStream_t)stream_;
    GS_CHECK_ARG(n >= 0, "gs_bin_tiles: n = %d < 0", n);
    GS_CHECK_ARG(width > 0 && height > 0 && width <= kMaxDim && height <= kMaxDim,
                 "gs_bin_tiles: image size %d x %d outside 1..%d", width, height, kMaxDim);
    GS_CHECK_ARG(capacity >= 0, "gs_bin_tiles: capacity %lld < 0", (long long)capacity);
    GS_CHECK_ARG(n_isect != nullptr, "gs_bin_tiles: n_isect is NULL");
    GS_CHECK_ARG(tile_ranges != nullptr, "gs_bin_tiles: tile_ranges is NULL");
    GS_CHECK_ARG(splat_offsets != nullptr, "gs_bin_tiles: splat_offsets is NULL");
    GS_CHECK_ARG(n == 0 || (means2d && radii && depths), "gs_bin_tiles: NULL splat array");
    GS_CHECK_ARG(capacity == 0 || sorted_ids != nullptr, "gs_bin_tiles: sorted_ids is NULL");
    const BinLayout L = bin_layout(n, capacity);
    GS_CHECK_ARG(workspace != nullptr && workspace_bytes >= L.bytes,
                 "gs_bin_tiles: workspace %zu bytes, need %zu", workspace_bytes, L.bytes);
    GS_CHECK_ARG(((uintptr_t)workspace & 255) == 0, "gs_bin_tiles: workspace not 256-byte aligned");

    const int GX = grid_x(width), GY = grid_y(height);
    const int tiles = GX * GY;
    char* ws = (char*)workspace;
    auto* counts = (unsigned long long*)(ws + L.counts);
    auto* offsets = (unsigned long long*)(ws + L.offsets);
    auto* part = (unsigned long long*)(ws + L.part);
    auto* total = (unsigned long long*)(ws + L.total);

    unsigned long long h_total = 0;
    if (n > 0) {
        count_kernel<<<(n + 255) / 256, 256, 0, st>>>(n, (const float2*)means2d, radii, depths, GX, GY, counts);
        GS_HIP(hipGetLastError());
        GS_HIP((exclusive_scan<unsigned long long, unsigned long long>(counts, offsets, n, part, total, st)));
        GS_HIP(hipMemcpyAsync(&h_total, total, sizeof(h_total), hipMemcpyDeviceToHost, st));
        GS_HIP(hipStreamSynchronize(st));
    }
    *n_isect = (int64_t)h_total;
    if (h_total > 0x7fffffffull) {
        set_error("gs_bin_tiles: %llu intersections exceed the int32 index range", h_total);
        return GS_ERR_UNSUPPORTED;
    }
    if ((long long)h_total > capacity) {
        set_error("gs_bin_tiles: capacity %lld < %llu intersections", (long long)capacity, h_total);
        return GS_ERR_CAPACITY;
    }
    const long long I = (long long)h_total;
    GS_HIP(hipMemsetAsync(tile_ranges, 0, sizeof(int) * 2 * (size_t)tiles, st));
    if (n > 0) {
        offsets_kernel<<<(n + 1 + 255) / 256, 256, 0, st>>>(n, offsets, total, splat_offsets);
        GS_HIP(hipGetLastError());
    } else {
        GS_HIP(hipMemsetAsync(splat_offsets, 0, sizeof(int), st));
    }
    if (I == 0) return GS_OK;

    auto* keys_a = (unsigned long long*)(ws + L.keys_a);
    auto* keys_b = (unsigned long long*)(ws + L.keys_b);
    auto* vals_t = (int*)(ws + L.vals_tmp);
    auto* hist = (unsigned*)(ws + L.hist);

    // Digit passes: depth bits 0..30, then tile bits 32..32+tb-1.
    const int tb = bits_for(tiles);
    int shifts[8];
    int np = 0;
    for (int s = 0; s < 31; s += kRadixBits) shifts[np++] = s;
    for (int s = 32; s < 32 + tb; s += kRadixBits) shifts[np++] = s;

    // Ping-pong so that the last pass writes its values into sorted_ids.
    unsigned long long* kin = keys_a;
    unsigned long long* kout = keys_b;
    int* vin = (np % 2 == 0) ? sorted_ids : vals_t;
    int* vout = (np % 2 == 0) ? vals_t : sorted_ids;

    emit_kernel<<<(n + 255) / 256, 256, 0, st>>>(n, (const float2*)means2d, radii, depths, GX, GY, offsets, kin,
                                                 vin);
    GS_HIP(hipGetLastError());

    const int nwg = (int)((I + kSortTile - 1) / kSortTile);
    for (int p = 0; p < np; ++p) {
        radix_hist_kernel<<<nwg, kSortThreads, 0, st>>>(kin, I, shifts[p], nwg, hist);
        GS_HIP(hipGetLastError());
        GS_HIP((exclusive_scan<unsigned, unsigned>(hist, hist, (long long)kRadix * nwg, part, total, st)));
        radix_scatter_kernel<<<nwg, kSortThreads, 0, st>>>(kin, vin, I, shifts[p], nwg, hist, kout, vout);
        GS_HIP(hipGetLastError());
        unsigned long long* tk = kin; kin = kout; kout = tk;
        int* tv = vin; vin = vout; vout = tv;
    }
    ranges_kernel<<<(unsigned)((I + 255) / 256), 256, 0, st>>>(kin, I, (int2*)tile_ranges);
    GS_HIP(hipGetLastError());
    return GS_OK;
}
