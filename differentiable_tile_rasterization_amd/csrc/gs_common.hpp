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
// largest accepted splat count: per-splat offsets such as 3 i (colour, conic)
// and block counts such as (n + 255) / 256 stay within int32
constexpr int kMaxSplats = 1 << 29;

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

// A tile's [start, end) range of the sorted pair list, clamped to
// 0 <= start <= end <= n_pairs, so that ranges that did not come from one
// binning of these splats never index outside the list.
__device__ __forceinline__ int2 clamp_range(int2 rg, long long n_pairs)
{
    const long long x = min(max((long long)rg.x, 0ll), n_pairs);
    const long long y = min(max((long long)rg.y, x), n_pairs);
    return make_int2((int)x, (int)y);
}

// ---------------------------------------------------------------------------
// Tile rectangle [tx0, tx1) x [ty0, ty1) of a splat (the rule in gsraster.h):
// plain float32 sub, multiply by 1/16 and floor, then clamp to the grid. No
// contraction is possible in these expressions, so every evaluation -- the
// binning's and the backward's, which recomputes it to find a (splat, tile)
// pair's slot -- gets the same rectangle.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void tile_rect(float mx, float my, int r, int GX, int GY, int& tx0, int& tx1, int& ty0,
                                          int& ty1)
{
    const float rf = (float)r;
    const float x0 = floorf((mx - rf) * 0.0625f);
    const float x1 = floorf((mx + rf) * 0.0625f) + 1.0f;
    const float y0 = floorf((my - rf) * 0.0625f);
    const float y1 = floorf((my + rf) * 0.0625f) + 1.0f;
    tx0 = (int)fminf(fmaxf(x0, 0.0f), (float)GX);
    tx1 = (int)fminf(fmaxf(x1, 0.0f), (float)GX);
    ty0 = (int)fminf(fmaxf(y0, 0.0f), (float)GY);
    ty1 = (int)fminf(fmaxf(y1, 0.0f), (float)GY);
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

// Returns alpha_raw = opacity * exp(sigma) (unclamped) and dx, dy. The
// exponent log2(opacity) - v2^2 - v1^2 is two FMAs (two roundings): each
// subtracts a non-negative square from a value that is at most log2(opacity),
// so the exponent never exceeds log2(opacity) and alpha_raw never exceeds
// exp2(log2(opacity)) (v_exp_f32 is monotone).
__device__ __forceinline__ float alpha_raw(const AlphaCoef& k, float px, float py, float& dx, float& dy)
{
    dx = px - k.mx;
    dy = py - k.my;
    const float v1 = __builtin_fmaf(k.l11, dx, k.l21 * dy);
    const float v2 = k.l22 * dy;
    return __builtin_amdgcn_exp2f(__builtin_fmaf(-v1, v1, __builtin_fmaf(-v2, v2, k.lo)));
}

// ---------------------------------------------------------------------------
// Culling test of a splat against a rectangle of pixel centres.
//
// A pixel can take the splat only if alpha >= 1/255, i.e. if the quadratic
// form q(d) = d^T Q d stays within tau = 2 ln(255 opacity). Over a rectangle
// dx in [x0, x1], dy in [y0, y1] (d = pixel - mean) the minimum of this convex
// form is 0 if the rectangle holds the mean, and otherwise lies on an edge, at
// the edge's stationary point clamped to the edge. The test adds a relative
// and an absolute margin far above the float32 error of either evaluation, so
// it never drops a pair whose alpha reaches 1/255.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float qform(float a, float b, float c, float dx, float dy)
{
    return __builtin_fmaf(dx, __builtin_fmaf(a, dx, 2.0f * b * dy), c * dy * dy);
}

__device__ __forceinline__ float rect_min_q(float a, float b, float c, float x0, float x1, float y0, float y1)
{
    if (x0 <= 0.0f && 0.0f <= x1 && y0 <= 0.0f && 0.0f <= y1) return 0.0f;
    const float ia = 1.0f / a, ic = 1.0f / c;
    float m = qform(a, b, c, x0, fminf(fmaxf(-b * x0 * ic, y0), y1));
    m = fminf(m, qform(a, b, c, x1, fminf(fmaxf(-b * x1 * ic, y0), y1)));
    m = fminf(m, qform(a, b, c, fminf(fmaxf(-b * y0 * ia, x0), x1), y0));
    m = fminf(m, qform(a, b, c, fminf(fmaxf(-b * y1 * ia, x0), x1), y1));
    return m;
}

// tau with its safety margin; negative when the splat can never reach 1/255
// (opacity clearly below it), so that no pixel passes q <= tau.
__device__ __forceinline__ float cull_tau(float o)
{
    const float t = 2.0f * logf(255.0f * o);
    return __builtin_fmaf(t, 1.0f / 512.0f, t) + 1.0f / 512.0f;
}

// ---------------------------------------------------------------------------
// Wave64 helpers.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp0(float x)
{
    // DPP move; lanes whose source lies outside the row read zero.
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// Sum over each 16-lane row, left in every lane of the row: four rotations
// within the row (row_ror:8, 4, 2, 1), each fused into one v_add_f32_dpp.
__device__ __forceinline__ float row_sum16(float x)
{
    x += dpp0<0x128>(x);   // row_ror:8
    x += dpp0<0x124>(x);   // row_ror:4
    x += dpp0<0x122>(x);   // row_ror:2
    x += dpp0<0x121>(x);   // row_ror:1
    // pin the total in a VGPR here: left alone, the compiler moves the last
    // add under the caller's lane mask, where it costs a mov, a DPP mov and
    // an add instead of one fused DPP add
    asm volatile("" : "+v"(x));
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

// ---------------------------------------------------------------------------
// Register-merging row reductions. A DPP add with a bank mask writes only the
// 4-lane banks it names and leaves the others as they were, so two registers
// that each still need a pairwise step can be folded into one:
//     z = y + perm(y)            on every lane
//     z = x + perm(x)            on the masked banks only
// The builtin DPP move has no way to keep the destination's old lanes while
// fusing the add, so these two use inline assembly; the s_nop covers the
// two wait states a DPP read needs after a VALU write of its source.
// Permutations (all stay inside a 16-lane row):
//   row_ror:8        lane i <-> i + 8      (pairs the two 8-lane halves)
//   row_half_mirror  lane i <-> 7 - i      (inside each 8-lane half)
//   quad_perm        inside each 4-lane group
// ---------------------------------------------------------------------------
__device__ __forceinline__ float dpp_add_ror8(float x) { return x + dpp0<0x128>(x); }
__device__ __forceinline__ float dpp_add_half_mirror(float x) { return x + dpp0<0x141>(x); }
__device__ __forceinline__ float dpp_add_quad_xor2(float x) { return x + dpp0<0x4E>(x); }  // quad_perm [2,3,0,1]
__device__ __forceinline__ float dpp_add_quad_xor1(float x) { return x + dpp0<0xB1>(x); }  // quad_perm [1,0,3,2]

// rows 1 and 3: x + (lane 15 of the row before); rows 0 and 2 keep x. With a
// row total in every lane, rows 1 and 3 then hold the total of rows (0, 1)
// and (2, 3).
__device__ __forceinline__ float dpp_add_prev_row_odd(float x)
{
    asm volatile("s_nop 1\n\tv_add_f32_dpp %0, %0, %0 row_bcast:15 row_mask:0xa bank_mask:0xf" : "+v"(x));
    return x;
}

// Maxima of two values over each 32-lane half, for non-negative floats as
// their bit patterns (whose unsigned order is the order of the values).
// v_permlane16_swap folds the two rows of each half lane-wise, x's into rows 0
// and 2 and y's into rows 1 and 3; four DPP rotations (each fused into one
// v_max_u32_dpp) finish each row. Row 0 holds half 0's max of x, row 1 half
// 0's max of y, rows 2 and 3 the same for half 1, in every lane of the row.
template <int CTRL>
__device__ __forceinline__ unsigned dpp0u(unsigned x)
{
    return (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xf, 0xf, false);
}

__device__ __forceinline__ unsigned half_umax_pair(unsigned x, unsigned y)
{
    const auto r = __builtin_amdgcn_permlane16_swap(x, y, false, false);
    const unsigned u0 = r[0], u1 = r[1];
    unsigned m = max(u0, u1);
    m = max(m, dpp0u<0x128>(m));  // row_ror:8
    m = max(m, dpp0u<0x124>(m));  // row_ror:4
    m = max(m, dpp0u<0x122>(m));  // row_ror:2
    m = max(m, dpp0u<0x121>(m));  // row_ror:1
    asm volatile("" : "+v"(m));   // keep the last level fused, outside the caller's lane mask
    return m;
}

// lanes 0-7 of each row: x + ror8(x); lanes 8-15: y + ror8(y)
__device__ __forceinline__ float merge_ror8(float x, float y)
{
    float z = dpp_add_ror8(y);
    asm volatile("s_nop 1\n\tv_add_f32_dpp %0, %1, %1 row_ror:8 row_mask:0xf bank_mask:0x3"
                 : "+v"(z) : "v"(x));
    return z;
}

// banks 0 and 2 (lanes 0-3, 8-11) of each row: x + half_mirror(x); banks 1
// and 3: y + half_mirror(y)
__device__ __forceinline__ float merge_half_mirror(float x, float y)
{
    float z = dpp_add_half_mirror(y);
    asm volatile("s_nop 1\n\tv_add_f32_dpp %0, %1, %1 row_half_mirror row_mask:0xf bank_mask:0x5"
                 : "+v"(z) : "v"(x));
    return z;
}

__device__ __forceinline__ int wave_max_i32(int v)
{
    for (int off = 32; off > 0; off >>= 1) v = max(v, __shfl_xor(v, off, 64));
    return v;
}

}  // namespace gs
