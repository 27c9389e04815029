// gs_probe.hip -- measurement kernels for libgsprobe.so (not part of libgsraster).
//
// * gsp_walk_stats   exact algorithmic counts of a backward pass: walked
//                    (pixel, entry) pairs, composited pairs, (splat, tile) and
//                    (splat, 8x8 quadrant) groups with a composited pixel, and
//                    how many (entry, quadrant) pairs the culling keeps. Uses
//                    the library's own alpha evaluation and culling test.
// * gsp_copy         plain float4 copy: the reference kernel for scaling
//                    hardware byte counters.
// * gsp_copy_stream  unrolled non-temporal float4 copy: the HBM ceiling.
// * gsp_lds_peak     LDS ceilings: wave-uniform (broadcast) 16-byte reads and
//                    per-lane 16-byte writes.
// * gsp_atomic_replay the backward's flush stream replayed alone: one thread
//                    per (splat, tile) group that receives gradient, one float
//                    atomic per field, same addresses and order of issue.
// * gsp_valu_peak / gsp_exp_peak  issue-rate probes (independent FMA chains,
//                    independent v_exp_f32 chains).
// * gsp_fold_selftest the wave reduction used by the backward applied to known
//                    lane values.
#include "gs_common.hpp"

namespace gs {
namespace {

struct ProbeStage {
    float4 a[kBlock];
    float4 b[kBlock];
};

__global__ __launch_bounds__(kBlock) void walk_stats_kernel(
    int W, int H, int GX, int tiles, const int2* __restrict__ ranges, const int* __restrict__ ids,
    const float2* __restrict__ means, const float* __restrict__ conics, const float* __restrict__ opac,
    const int* __restrict__ n_contrib, unsigned long long* __restrict__ cnt, unsigned char* __restrict__ flags)
{
    __shared__ ProbeStage S;
    __shared__ int wave_max[4];
    __shared__ int entry_any[kBlock];
    const int tile = blockIdx.x;
    if (tile >= tiles) return;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int x = (tile % GX) * kTile + (wv & 1) * 8 + (lane & 7);
    const int y = (tile / GX) * kTile + (wv >> 1) * 8 + (lane >> 3);
    const float ox = (float)((tile % GX) * kTile) + 0.5f, oy = (float)((tile / GX) * kTile) + 0.5f;
    const bool inside = x < W && y < H;
    const int2 rg = ranges[tile];
    int nc = inside ? min(max(n_contrib[y * W + x], 0), rg.y - rg.x) : 0;
    const int wmax = wave_max_i32(nc);
    if (lane == 0) wave_max[wv] = wmax;
    __syncthreads();
    const int tmax = max(max(wave_max[0], wave_max[1]), max(wave_max[2], wave_max[3]));
    unsigned long long c_walk = nc, c_contrib = 0, c_swave = 0, c_keep = 0, c_stile = 0;
    // finer groups inside the quadrant: 8x4 halves (lanes 0-31, 32-63) and 4x4 blocks
    unsigned long long c_half = 0, c_blk = 0, c_half_max = 0, c_blk_max = 0;
    for (int bs = 0; bs < tmax; bs += kBlock) {
        __syncthreads();
        const int k = bs + (int)threadIdx.x;
        entry_any[threadIdx.x] = 0;
        if (k < tmax) {
            const int id = ids[rg.x + k];
            const float2 m = means[id];
            const float a = conics[3 * id], b = conics[3 * id + 1], c = conics[3 * id + 2], o = opac[id];
            const AlphaCoef kf = make_alpha_coef(m.x, m.y, a, b, c, o);
            S.a[threadIdx.x] = make_float4(kf.mx, kf.my, kf.l11, kf.l21);
            S.b[threadIdx.x] = make_float4(kf.l22, kf.lo, 0.0f, 0.0f);
            const float tau = cull_tau(o);
            for (int q = 0; q < 4; ++q) {
                const float x0 = ox + (float)((q & 1) * 8) - m.x, y0 = oy + (float)((q >> 1) * 8) - m.y;
                if (k < wave_max[q] && rect_min_q(a, b, c, x0, x0 + 7.0f, y0, y0 + 7.0f) <= tau) ++c_keep;
            }
        }
        __syncthreads();
        const int jend = min(kBlock, wmax - bs);
        unsigned h0 = 0, h1 = 0, b0 = 0, b1 = 0, b2 = 0, b3 = 0;
        for (int j = 0; j < jend; ++j) {
            const float4 A = S.a[j], B = S.b[j];
            const AlphaCoef kf{A.x, A.y, A.z, A.w, B.x, B.y};
            float dx, dy;
            const float al = fminf(kAlphaMax, alpha_raw(kf, (float)x + 0.5f, (float)y + 0.5f, dx, dy));
            const bool contrib = (bs + j < nc) && (al >= kAlphaMin);
            const unsigned long long bal = __ballot(contrib);
            c_contrib += contrib ? 1 : 0;
            h0 += (bal & 0xffffffffull) != 0;
            h1 += (bal >> 32) != 0;
            b0 += (bal & 0x0f0f0f0f0f0f0f0full & 0x00000000ffffffffull) != 0;  // x 0-3, y 0-3
            b1 += (bal & 0xf0f0f0f0f0f0f0f0ull & 0x00000000ffffffffull) != 0;  // x 4-7, y 0-3
            b2 += (bal & 0x0f0f0f0f0f0f0f0full & 0xffffffff00000000ull) != 0;  // x 0-3, y 4-7
            b3 += (bal & 0xf0f0f0f0f0f0f0f0ull & 0xffffffff00000000ull) != 0;  // x 4-7, y 4-7
            if (bal != 0) {
                if (lane == 0) {
                    ++c_swave;
                    entry_any[j] = 1;
                }
            }
        }
        if (lane == 0) {
            c_half += h0 + h1;
            c_half_max += max(h0, h1);
            c_blk += b0 + b1 + b2 + b3;
            c_blk_max += max(max(b0, b1), max(b2, b3));
        }
        __syncthreads();
        if (k < tmax && entry_any[threadIdx.x]) {
            ++c_stile;
            if (flags) flags[rg.x + k] = 1;
        }
    }
    // block totals
    for (int off = 32; off > 0; off >>= 1) {
        c_walk += __shfl_xor(c_walk, off, 64);
        c_contrib += __shfl_xor(c_contrib, off, 64);
        c_swave += __shfl_xor(c_swave, off, 64);
        c_keep += __shfl_xor(c_keep, off, 64);
        c_stile += __shfl_xor(c_stile, off, 64);
    }
    if (lane == 0) {
        atomicAdd(&cnt[7], c_half);
        atomicAdd(&cnt[8], c_blk);
        atomicAdd(&cnt[9], c_half_max);
        atomicAdd(&cnt[10], c_blk_max);
    }
    if (lane == 0) {
        atomicAdd(&cnt[0], c_walk);
        atomicAdd(&cnt[1], c_contrib);
        atomicAdd(&cnt[3], c_stile);
        atomicAdd(&cnt[4], c_swave);
        atomicAdd(&cnt[5], (unsigned long long)wmax);
        atomicAdd(&cnt[6], c_keep);
        if (wv == 0) atomicAdd(&cnt[2], (unsigned long long)tmax);
    }
}

__global__ __launch_bounds__(256) void copy_kernel(const float4* __restrict__ in, float4* __restrict__ out,
                                                   long long n)
{
    const long long stride = (long long)gridDim.x * blockDim.x;
    for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) out[i] = in[i];
}

// Streaming copy for the HBM ceiling: each thread moves four float4 per
// iteration (all four loads issued before the stores), non-temporal loads and
// stores (the data is touched once), grid-stride over the buffer.
typedef float v4f __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void copy_stream_kernel(const v4f* __restrict__ in, v4f* __restrict__ out,
                                                          long long n)
{
    const long long stride = (long long)gridDim.x * blockDim.x;
    long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + 3 * stride < n; i += 4 * stride) {
        const v4f a = __builtin_nontemporal_load(in + i);
        const v4f b = __builtin_nontemporal_load(in + i + stride);
        const v4f c = __builtin_nontemporal_load(in + i + 2 * stride);
        const v4f d = __builtin_nontemporal_load(in + i + 3 * stride);
        __builtin_nontemporal_store(a, out + i);
        __builtin_nontemporal_store(b, out + i + stride);
        __builtin_nontemporal_store(c, out + i + 2 * stride);
        __builtin_nontemporal_store(d, out + i + 3 * stride);
    }
    for (; i < n; i += stride) __builtin_nontemporal_store(__builtin_nontemporal_load(in + i), out + i);
}

// LDS ceilings, one 256-thread workgroup per CU slot, 32 KB of LDS each.
//  mode 0 (broadcast read): every lane of a wave reads the same 16 bytes
//         (wave-uniform address), eight independent reads in flight; counts
//         16 bytes per wave instruction, the way the walk's record reads are
//         counted.
//  mode 1 (write): every lane writes 16 bytes to its own address (1 KB per
//         wave instruction, no bank conflicts).
// iters * 8 instructions per wave; the result is kept live through out.
__global__ __launch_bounds__(256) void lds_peak_kernel(float* out, int iters, int mode)
{
    __shared__ float4 buf[2048];
    const int t = threadIdx.x, wv = t >> 6;
    for (int k = t; k < 2048; k += 256) buf[k] = make_float4((float)k, 1.0f, 2.0f, 3.0f);
    __syncthreads();
    float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if (mode == 0) {
        int base = __builtin_amdgcn_readfirstlane(wv * 64);
        for (int i = 0; i < iters; ++i) {
            float4 v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = buf[(base + 8 * j + (i & 7)) & 2047];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                acc.x += v[j].x;
                acc.y += v[j].y;
            }
            base = __builtin_amdgcn_readfirstlane((base + 97) & 1023);
        }
    } else {
        for (int i = 0; i < iters; ++i) {
            const float f = (float)i;
#pragma unroll
            for (int j = 0; j < 8; ++j) buf[(j * 256 + t) & 2047] = make_float4(f, f, f, f);
        }
        __syncthreads();
        acc = buf[t];
    }
    if (acc.x == 123.456f) out[blockIdx.x] = acc.y;  // keeps the reads live
}

template <int NF>
__global__ __launch_bounds__(256) void atomic_replay_kernel(const unsigned char* __restrict__ flags,
                                                            const int* __restrict__ ids, long long n,
                                                            float* __restrict__ d_means,
                                                            float* __restrict__ d_conics,
                                                            float* __restrict__ d_colors,
                                                            float* __restrict__ d_opac, float* __restrict__ aw)
{
    const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n || !flags[i]) return;
    const int id = ids[i];
    unsafeAtomicAdd(&d_means[2 * id + 0], 1.0f);
    unsafeAtomicAdd(&d_means[2 * id + 1], 1.0f);
    unsafeAtomicAdd(&d_conics[3 * id + 0], 1.0f);
    unsafeAtomicAdd(&d_conics[3 * id + 1], 1.0f);
    unsafeAtomicAdd(&d_conics[3 * id + 2], 1.0f);
    unsafeAtomicAdd(&d_colors[3 * id + 0], 1.0f);
    unsafeAtomicAdd(&d_colors[3 * id + 1], 1.0f);
    unsafeAtomicAdd(&d_colors[3 * id + 2], 1.0f);
    unsafeAtomicAdd(&d_opac[id], 1.0f);
    if (NF == 10) unsafeAtomicAdd(&aw[id], 1.0f);
}

// 8 independent FMA chains per lane; iters * 8 FMAs per lane.
__global__ __launch_bounds__(256) void valu_peak_kernel(float* out, int iters, float s)
{
    float a0 = threadIdx.x * 1e-3f, a1 = a0 + 1, a2 = a0 + 2, a3 = a0 + 3, a4 = a0 + 4, a5 = a0 + 5, a6 = a0 + 6,
          a7 = a0 + 7;
    for (int i = 0; i < iters; ++i) {
        a0 = __builtin_fmaf(a0, s, 0.5f); a1 = __builtin_fmaf(a1, s, 0.5f);
        a2 = __builtin_fmaf(a2, s, 0.5f); a3 = __builtin_fmaf(a3, s, 0.5f);
        a4 = __builtin_fmaf(a4, s, 0.5f); a5 = __builtin_fmaf(a5, s, 0.5f);
        a6 = __builtin_fmaf(a6, s, 0.5f); a7 = __builtin_fmaf(a7, s, 0.5f);
    }
    const float r = a0 + a1 + a2 + a3 + a4 + a5 + a6 + a7;
    if (r == 123.456f) out[blockIdx.x] = r;  // keeps the chains live
}

__global__ __launch_bounds__(256) void exp_peak_kernel(float* out, int iters)
{
    float a0 = -threadIdx.x * 1e-3f, a1 = a0 - 1, a2 = a0 - 2, a3 = a0 - 3;
    for (int i = 0; i < iters; ++i) {
        a0 = __builtin_amdgcn_exp2f(a0) - 1.0f; a1 = __builtin_amdgcn_exp2f(a1) - 1.0f;
        a2 = __builtin_amdgcn_exp2f(a2) - 1.0f; a3 = __builtin_amdgcn_exp2f(a3) - 1.0f;
    }
    const float r = a0 + a1 + a2 + a3;
    if (r == 123.456f) out[blockIdx.x] = r;
}

// One wave: field f at lane l holds in[f * 64 + l]; writes the 4 row-leader
// lanes' three results (out[row * 3 + reg]), exactly as the backward does.
__global__ void fold_selftest_kernel(const float* __restrict__ in, float* __restrict__ out)
{
    const int l = threadIdx.x;
    float f[10];
    for (int i = 0; i < 10; ++i) f[i] = in[i * 64 + l];
    const float r0 = fold32(f[0], f[1]);
    const float r1 = fold32(f[2], f[3]);
    const float r2 = fold32(f[4], f[5]);
    const float r3 = fold32(f[6], f[7]);
    const float r4 = fold32(f[8], f[9]);
    const float q0 = row_sum16(fold16(r0, r1));
    const float q1 = row_sum16(fold16(r2, r3));
    const float q2 = row_sum16(fold16(r4, r4));
    if ((l & 15) == 15) {
        out[(l >> 4) * 3 + 0] = q0;
        out[(l >> 4) * 3 + 1] = q1;
        out[(l >> 4) * 3 + 2] = q2;
    }
}

}  // namespace
}  // namespace gs

using namespace gs;

// counts[11] (uint64, zeroed by the caller): 0 walked pairs, 1 composited pairs,
// 2 walked entries (sum over tiles of the tile's largest n_contrib),
// 3 (splat, tile) groups with a composited pixel, 4 (splat, quadrant) groups
// with a composited pixel, 5 (entry, quadrant) pairs walked without culling,
// 6 (entry, quadrant) pairs the culling keeps, 7 (splat, 8x4 half) and
// 8 (splat, 4x4 block) groups with a composited pixel, 9 and 10 the same
// counted as the largest of the halves (blocks) per wave and batch, i.e. the
// wave iterations a lockstep walk over per-half (per-block) lists would need
// at perfect culling. flags [n_isect] (optional,
// zeroed by the caller) marks the (splat, tile) entries of count 3.
extern "C" int gsp_walk_stats(int32_t n, const float* means2d, const float* conics, const float* opacities,
                              int32_t width, int32_t height, const int32_t* tile_ranges,
                              const int32_t* sorted_ids, const int32_t* n_contrib, unsigned long long* counts,
                              unsigned char* flags, gs_stream_t stream)
{
    (void)n;
    const int GX = grid_x(width), tiles = GX * grid_y(height);
    walk_stats_kernel<<<tiles, kBlock, 0, (hipStream_t)stream>>>(width, height, GX, tiles,
                                                                 (const int2*)tile_ranges, sorted_ids,
                                                                 (const float2*)means2d, conics, opacities,
                                                                 n_contrib, counts, flags);
    return hipGetLastError() == hipSuccess ? 0 : 3;
}

extern "C" int gsp_copy(const void* in, void* out, long long n_float4, int blocks, gs_stream_t stream)
{
    copy_kernel<<<blocks, 256, 0, (hipStream_t)stream>>>((const float4*)in, (float4*)out, n_float4);
    return hipGetLastError() == hipSuccess ? 0 : 3;
}

extern "C" int gsp_copy_stream(const void* in, void* out, long long n_float4, int blocks, gs_stream_t stream)
{
    copy_stream_kernel<<<blocks, 256, 0, (hipStream_t)stream>>>((const v4f*)in, (v4f*)out, n_float4);
    return hipGetLastError() == hipSuccess ? 0 : 3;
}

extern "C" int gsp_lds_peak(float* out, int blocks, int iters, int mode, gs_stream_t stream)
{
    lds_peak_kernel<<<blocks, 256, 0, (hipStream_t)stream>>>(out, iters, mode);
    return hipGetLastError() == hipSuccess ? 0 : 3;
}

extern "C" int gsp_atomic_replay(const unsigned char* flags, const int32_t* sorted_ids, long long n_isect,
                                 float* d_means, float* d_conics, float* d_colors, float* d_opac, float* aw,
                                 gs_stream_t stream)
{
    const unsigned blocks = (unsigned)((n_isect + 255) / 256);
    if (blocks == 0) return 0;
    if (aw)
        atomic_replay_kernel<10><<<blocks, 256, 0, (hipStream_t)stream>>>(flags, sorted_ids, n_isect, d_means,
                                                                          d_conics, d_colors, d_opac, aw);
    else
        atomic_replay_kernel<9><<<blocks, 256, 0, (hipStream_t)stream>>>(flags, sorted_ids, n_isect, d_means,
                                                                         d_conics, d_colors, d_opac, aw);
    return hipGetLastError() == hipSuccess ? 0 : 3;
}

extern "C" int gsp_valu_peak(float* out, int blocks, int iters, gs_stream_t stream)
{
    valu_peak_kernel<<<blocks, 256, 0, (hipStream_t)stream>>>(out, iters, 0.999f);
    return hipGetLastError() == hipSuccess ? 0 : 3;
}

extern "C" int gsp_exp_peak(float* out, int blocks, int iters, gs_stream_t stream)
{
    exp_peak_kernel<<<blocks, 256, 0, (hipStream_t)stream>>>(out, iters);
    return hipGetLastError() == hipSuccess ? 0 : 3;
}

extern "C" int gsp_fold_selftest(const float* in, float* out, gs_stream_t stream)
{
    fold_selftest_kernel<<<1, 64, 0, (hipStream_t)stream>>>(in, out);
    return hipGetLastError() == hipSuccess ? 0 : 3;
}
