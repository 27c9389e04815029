// gs_common.hpp -- definitions shared by the libgsraster HIP sources (gfx950).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstring>

#include "gsraster.h"

namespace gs {

constexpr int kTile = 16;            // tile edge in pixels
constexpr int kBlock = 256;          // threads per raster workgroup = pixels per tile
constexpr int kWave = 64;            // gfx950 wavefront
constexpr int kMaxDim = 32768;       // largest accepted width / height

// Compositing constants of the rule documented in gsraster.h.
constexpr float kAlphaMax = 0.99f;
constexpr float kAlphaMin = 1.0f / 255.0f;
constexpr float kTMin = 1e-4f;

// ---------------------------------------------------------------------------
// Host-side error plumbing (thread-local message behind gs_last_error).
// ---------------------------------------------------------------------------
void set_error(const char* fmt, ...);
gs_status hip_fail(hipError_t e, const char* what);

#define GS_CHECK_ARG(cond, ...)                              \
    do {                                                     \
        if (!(cond)) {                                       \
            ::gs::set_error(__VA_ARGS__);                    \
            return GS_ERR_INVALID_ARG;                       \
        }                                                    \
    } while (0)

#define GS_HIP(call)                                         \
    do {                                                     \
        hipError_t e_ = (call);                              \
        if (e_ != hipSuccess) return ::gs::hip_fail(e_, #call); \
    } while (0)

inline int grid_x(int width) { return (width + kTile - 1) / kTile; }
inline int grid_y(int height) { return (height + kTile - 1) / kTile; }

// ---------------------------------------------------------------------------
// Workgroup -> tile mapping. Consecutive workgroups are dispatched round-robin
// over the 8 XCDs, each with its own L2. Neighbouring tiles share most of their
// splats, so give each XCD a contiguous run of tile ids: workgroup w runs tile
// (w % 8) * ceil(T / 8) + w / 8, skipping ids past the end. The grid is padded
// to 8 * ceil(T / 8) workgroups; the padding workgroups exit at once.
// ---------------------------------------------------------------------------
constexpr int kXcds = 8;

inline int xcd_grid(int tiles) { return kXcds * ((tiles + kXcds - 1) / kXcds); }

__device__ inline int xcd_tile(int wg, int tiles)
{
    const int per = (tiles + kXcds - 1) / kXcds;
    return (wg % kXcds) * per + wg / kXcds;
}

// ---------------------------------------------------------------------------
// Per-splat alpha evaluation, shared by the forward and backward kernels so
// that both take exactly the same float32 decisions.
//
// The conic Q = [[a, b], [b, c]] is factored once per staged splat as
// Q = L L^T, L = [[l11, 0], [l21, l22]], and scaled by s = sqrt(log2(e) / 2):
//     sigma * log2(e) = -(v1^2 + v2^2),   v1 = s (l11 dx + l21 dy),  v2 = s l22 dy
//     alpha_raw = exp2(log2(opacity) - v1^2 - v2^2)
// Forming sigma from a dx^2, b dx dy and c dy^2 separately loses up to
// |a| dx^2 * 2^-24 to cancellation for elongated splats; the factored form
// keeps the float32 error about ten times smaller at the same cost per pixel.
// The factor is computed with a compensated determinant so it is accurate to
// a few ulp even when a c ~ b^2.
// ---------------------------------------------------------------------------
struct AlphaCoef {
    float mx, my;        // mean
    float l11, l21, l22; // scaled Cholesky factor
    float lo;            // log2(opacity)
};

__device__ inline AlphaCoef make_alpha_coef(float mx, float my, float a, float b, float c, float o)
{
    constexpr float s = 0.84932180028801907f;   // sqrt(log2(e) / 2)
    AlphaCoef k;
    k.mx = mx;
    k.my = my;
    const float p = b * b;
    const float pe = __builtin_fmaf(b, b, -p);          // exact b*b = p + pe
    const float det = __builtin_fmaf(a, c, -p) - pe;    // a c - b^2, one rounding + small
    const float sa = __builtin_sqrtf(a);
    k.l11 = s * sa;
    k.l21 = s * (b / sa);
    k.l22 = s * __builtin_sqrtf(det / a);
    k.lo = log2f(o);
    return k;
}

// Returns alpha_raw = opacity * exp(sigma) (unclamped) and dx, dy.
__device__ __forceinline__ float alpha_raw(const AlphaCoef& k, float px, float py, float& dx, float& dy)
{
    dx = px - k.mx;
    dy = py - k.my;
    const float v1 = __builtin_fmaf(k.l11, dx, k.l21 * dy);
    const float v2 = k.l22 * dy;
    const float q = __builtin_fmaf(v1, v1, v2 * v2);
    return __builtin_amdgcn_exp2f(k.lo - q);
}

// ---------------------------------------------------------------------------
// Wave64 helpers.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp0(float x)
{
    // DPP move with zero fill for lanes whose source is outside the row.
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// Sum over each 16-lane row; the total lands in the row's last lane (15).
__device__ __forceinline__ float row_sum16(float x)
{
    x += dpp0<0x111>(x);   // row_shr:1
    x += dpp0<0x112>(x);   // row_shr:2
    x += dpp0<0x114>(x);   // row_shr:4
    x += dpp0<0x118>(x);   // row_shr:8
    return x;
}

// v_permlane32_swap: x.hi <-> y.lo.  Returns x' + y', i.e. lanes 0..31 hold
// x[l] + x[l+32] and lanes 32..63 hold y[l-32] + y[l].
__device__ __forceinline__ float fold32(float x, float y)
{
    // Copy both lanes of the result to scalars before reinterpreting them:
    // bit-casting the vector elements in place makes clang read element 0 twice.
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
    const unsigned u0 = r[0], u1 = r[1];
    return __uint_as_float(u0) + __uint_as_float(u1);
}

// v_permlane16_swap: odd rows of x <-> even rows of y.  Returns x' + y':
// row0 = x.r0 + x.r1, row1 = y.r0 + y.r1, row2 = x.r2 + x.r3, row3 = y.r2 + y.r3.
__device__ __forceinline__ float fold16(float x, float y)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
    const unsigned u0 = r[0], u1 = r[1];
    return __uint_as_float(u0) + __uint_as_float(u1);
}

__device__ __forceinline__ int wave_max_i32(int v)
{
    for (int off = 32; off > 0; off >>= 1) v = max(v, __shfl_xor(v, off, 64));
    return v;
}

}  // namespace gs
