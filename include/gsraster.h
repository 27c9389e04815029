/*
 * gsraster.h -- C ABI of libgsraster: tile-based Gaussian-splat rasterization
 * (binning, forward, backward) for AMD Instinct MI355X (gfx950).
 *
 * What the three calls compute
 * ----------------------------
 * The pages this library follows are the Spirula Studio article on the
 * rasterize_bwd_2d kernel ("从 8.6 KB 到 4.2 KB ...", sections 机制拆解 and
 * 亲手验证: the 2D screen-space backward pass, run once per training
 * iteration, with an optional per-splat accumulated-weight output; a fixed
 * benchmark load of 2,000,000 splats at 1237x822 with raster fwd / raster bwd
 * / tile isect timings) and the 3dgs-rs log "Phase 5 step 30b — kernel-by-
 * kernel timing" (section 計測結果: the per-iteration kernels emit_pairs,
 * radix_hist / radix_scatter, extract_offsets, rasterize_f32 and
 * rasterize_backwards; section ホットスポット ranking item 1: the backward
 * accumulates nine per-splat gradient fields -- 2D mean, conic, RGB, opacity
 * -- over all pixels; section 結論と次着手: a 16x16 tile of 256 pixels per
 * workgroup). The pages give no formula. The compositing rule implemented is
 * the standard one of tile-based 3D Gaussian splatting:
 *
 *   pixel (x, y) has centre p = (x + 0.5, y + 0.5); d = p - mean
 *   sigma = -1/2 (a dx^2 + c dy^2) - b dx dy  with conic (a, b, c) the upper
 *           triangle of the inverse 2D covariance (b is the off-diagonal entry)
 *   alpha = min(0.99, opacity * exp(sigma))
 *   each pixel walks its tile's list front to back:
 *     alpha < 1/255              -> skip the splat
 *     T * (1 - alpha) < 1e-4     -> stop; this splat is not composited
 *     otherwise                  -> C += colour * alpha * T;  T *= 1 - alpha
 *   image = C + T * background;  final_T = T;
 *   n_contrib = 1 + list position of the last composited splat (0 if none)
 *
 * The backward returns dL/dparam for L = sum_p <dL_dimage_p, image_p>, with
 * every skip / stop / clamp decision held as the forward took it (a clamped
 * alpha passes no gradient to opacity, conic or mean).
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Pointers marked "device" are caller-owned device memory (hipMalloc or a
 *    torch tensor), contiguous, float32 / int32 as stated. The library never
 *    allocates or frees device memory; scratch comes in as `workspace`.
 *  - All work is enqueued on `stream` (0 = the null stream) in stream order;
 *    calls return before the work finishes, except gs_bin_tiles, which waits
 *    once to read the intersection count back to the host.
 *    gs_rasterize_bwd and gs_rasterize_bwd_noalloc enqueue kernel launches
 *    only (no allocation, copy, memset or synchronisation), so a caller may
 *    capture them in a HIP graph; the binning cannot be captured (its
 *    read-back).
 *  - Outputs are overwritten, never accumulated into.
 *  - Tiles are 16x16 pixels; tile ids are row-major: ty * GX + tx with
 *    GX = ceil(width / 16), GY = ceil(height / 16).
 *  - Images are HWC, row-major, y pointing down: image[(y * width + x) * 3 + ch].
 *  - Errors: arguments the host can check (NULL where a pointer is required,
 *    n outside 0 .. 2^29, width or height <= 0 or too large, unknown flags) return
 *    GS_ERR_INVALID_ARG before any work is enqueued. A failing HIP call
 *    returns GS_ERR_HIP. gs_last_error() then describes the failure (a
 *    thread-local string, valid until the thread's next call). Faults inside
 *    kernels surface at the caller's next synchronisation.
 *  - Data preconditions (the caller's duty, not checked): finite values,
 *    positive-definite conics, opacity in [0, 1], radii from a conservative
 *    projection. Splats with radius <= 0, depth not > 0 or a non-finite mean
 *    are culled by the binning.
 *  - Binning outputs passed on: tile_ranges, sorted_ids and splat_offsets
 *    should come from one gs_bin_tiles call on the same splats and image
 *    size. The kernels still bound what they read: a sorted_ids entry
 *    outside [0, n) is no entry, both rasterizers clamp every tile range to
 *    [0, n_isect], the pair count the caller passes with sorted_ids (which
 *    must hold at least n_isect entries), and the backward clamps every
 *    splat offset to [0, n_slots].
 *  - Calls are re-entrant; the only global mutable state is the thread-local
 *    error string and the fixed per-device scratch of
 *    gs_rasterize_bwd_noalloc (calls of it that overlap on one GPU race).
 */
#ifndef GSRASTER_H
#define GSRASTER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* hipStream_t without pulling in the HIP headers: an opaque stream handle. */
typedef struct ihipStream_t* gs_stream_t;
typedef struct ihipEvent_t* gs_event_t;

typedef enum {
    GS_OK = 0,
    GS_ERR_INVALID_ARG = 1,
    GS_ERR_CAPACITY = 2,
    GS_ERR_HIP = 3,
    GS_ERR_UNSUPPORTED = 4
} gs_status;

enum { GS_TILE = 16 };

/* gs_rasterize_bwd flags */
enum {
    /* Also write accum_weight[i] = sum over composited (pixel, splat i) pairs of
     * alpha * T: the "accum weight" optional feature of the Spirula Studio
     * page (section 机制拆解). The weight is a template parameter of the
     * kernels: without the flag no instruction, register or global store is
     * spent on it. The LDS-add walk keeps an 80-byte LDS slot per staged
     * entry in both instances (16-byte aligned records at an odd multiple of
     * 16 bytes); the records of the deferred and stored-partials walks are 36
     * bytes without the weight and 40 with it. */
    GS_FLAG_ACCUM_WEIGHT = 1u << 0,
    /* Force one of the three reverse walks (same results up to the order of
     * float additions); setting more than one is an invalid argument.
     * Without any, the call takes the deferred walk.
     *   WALK_DEFER: each lockstep step only recovers alpha, T and the colour
     *               behind and parks each lane's (w = alpha T, s = dL/dsigma)
     *               in a per-wave buffer; every four steps the lanes sum the
     *               (half-list, position) records of those steps in registers
     *               (moments of s and w over their pixels) and store them;
     *               each entry's records are summed once per batch (no LDS
     *               float adds). Batches of 191 entries, or 127 when the
     *               splats average more than 16 listed tiles each.
     *   WALK_ADD:   each step reduces its ten sums across the half-wave and
     *               adds them into the entry's LDS partial sums (float LDS
     *               adds; 255-entry batches);
     *   WALK_STORE: each (half-list, position) step reduces and stores its
     *               totals into a record of its own (no adds; batches of at
     *               most 127 entries, cut further if their records would not
     *               fit). */
    GS_FLAG_WALK_ADD = 1u << 1,
    GS_FLAG_WALK_STORE = 1u << 2,
    GS_FLAG_WALK_DEFER = 1u << 3
};

/* Thread-local description of the last non-OK status returned on this thread. */
const char* gs_last_error(void);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int gs_version(void);

/*
 * Binning: the per-iteration tile-binning, sort and tile-range stages
 * (emit_pairs, radix_hist, radix_scatter, extract_offsets in the timing
 * table of "Phase 5 step 30b — kernel-by-kernel timing", section 計測結果;
 * the "tile isect" line of raster_bench on the Spirula Studio page, section
 * 亲手验证).
 *
 * Each live splat covers the tile rectangle [tx0, tx1) x [ty0, ty1) computed
 * in float32 as
 *     tx0 = clamp(floor((mean_x - r) * 0.0625),       0, GX)
 *     tx1 = clamp(floor((mean_x + r) * 0.0625) + 1,   0, GX)
 * (and likewise in y), r = (float)radii[i]. Within its rectangle a splat is
 * listed only in the tiles that its alpha >= 1/255 ellipse can reach: the
 * compositing skips alpha < 1/255, so a tile whose pixel centres all lie
 * outside {Q <= 2 ln(255 o)} (Q the splat's quadratic form) gets nothing from
 * it. The test takes, in float32 with every operation rounded once in a fixed
 * order, an upper bound T on 2 ln(255 o) (with a small margin) and, per tile
 * row, the ellipse {Q <= T}'s x-extent over the row's band of pixel centres;
 * a splat with 255 o < 1 is listed nowhere, one with a conic that is not
 * positive definite keeps its whole rectangle. Each tile's list holds the
 * splats kept there, ordered by the float32 bit pattern of depth, ties broken
 * by ascending splat id (so the result is unique). Lists are concatenated in
 * tile-id order into sorted_ids; tile_ranges[t] = [start, end) into it
 * ({0, 0} for an empty tile).
 *
 *   n            number of splats, 0 .. 2^29 (536,870,912), else
 *                GS_ERR_INVALID_ARG
 *   means2d      device float [n][2], pixels
 *   conics       device float [n][3] = (a, b, c) of the inverse covariance
 *   opacities    device float [n]
 *   radii        device int32 [n], screen radius in pixels (<= 0: culled)
 *   depths       device float [n] (not > 0: culled)
 *   width,height image size in pixels, 1 .. 32768 each
 *   capacity     number of int32 slots in sorted_ids
 *   sorted_ids   device int32 [capacity] (out)
 *   tile_ranges  device int32 [GX*GY][2] (out)
 *   splat_offsets device int32 [n + 1] (out): the tiles of splat i's whole
 *                rectangle (kept or not), in row-major order, are numbered
 *                splat_offsets[i] .. splat_offsets[i+1]-1; [n] = n_slots. The
 *                backward uses this numbering to give each (splat, tile) pair
 *                its own accumulation slot.
 *   n_isect      host int64 (out): number of listed (splat, tile) pairs, the
 *                length of sorted_ids
 *   n_slots      host int64 (out), or NULL: number of rectangle pairs
 *                (>= n_isect), the backward's slot count
 *   workspace    device scratch of at least gs_bin_tiles_workspace_size(...)
 *                bytes, 256-byte aligned
 *
 * Waits once on the host for both counts (an asynchronous copy into a small
 * pinned host buffer that each calling thread keeps from its first call; the
 * stages that do not need the counts are enqueued before the wait, so the GPU
 * does not idle meanwhile). If capacity < *n_isect it returns GS_ERR_CAPACITY
 * with *n_isect (and *n_slots) set and sorted_ids / tile_ranges /
 * splat_offsets untouched: allocate *n_isect entries (and the matching
 * workspace) and call again. A rectangle total above 2^31 - 1 returns
 * GS_ERR_UNSUPPORTED.
 */
size_t gs_bin_tiles_workspace_size(int32_t n, int64_t capacity, int32_t width, int32_t height);

gs_status gs_bin_tiles(int32_t n, const float* means2d, const float* conics, const float* opacities,
                       const int32_t* radii, const float* depths, int32_t width, int32_t height, int64_t capacity,
                       int32_t* sorted_ids, int32_t* tile_ranges, int32_t* splat_offsets, int64_t* n_isect,
                       int64_t* n_slots, void* workspace, size_t workspace_bytes, gs_stream_t stream);

/*
 * Forward composite (rasterize_f32 in the timing table of "Phase 5 step 30b —
 * kernel-by-kernel timing", section 計測結果; the "raster fwd" line of
 * raster_bench). One workgroup of 256 threads per 16x16 tile. Each splat is
 * first packed into a 48-byte record in the workspace (alpha coefficients,
 * colour, culling threshold, radius); each half of a wave (an 8x4 block of
 * pixels) then walks only the list entries whose alpha >= 1/255 ellipse
 * reaches it.
 *
 * Optionally also the per-splat max weight (the "max wt" line of raster_bench
 * on the Spirula Studio page, section 亲手验证, which names the statistic
 * without a formula; read here as the largest compositing weight alpha T the
 * splat receives over the pixels that composite it, 0 if none). The result
 * does not depend on scheduling.
 *
 *   n                 number of splats, 0 .. 2^29, else GS_ERR_INVALID_ARG
 *   means2d           device float [n][2]
 *   conics            device float [n][3] = (a, b, c) of the inverse covariance
 *   colors            device float [n][3]
 *   opacities         device float [n]
 *   background        device float [3], or NULL for black
 *   width, height     image size
 *   tile_ranges       device int32 [GX*GY][2], from gs_bin_tiles; each range is
 *                     clamped to [0, n_isect] before use
 *   sorted_ids        device int32 [n_isect], from gs_bin_tiles
 *   n_isect           number of entries of sorted_ids (the binning's pair
 *                     count); 0 .. 2^31 - 1, else GS_ERR_INVALID_ARG
 *   image             device float [height][width][3] (out)
 *   final_T           device float [height][width]    (out)
 *   n_contrib         device int32 [height][width]    (out)
 *   max_weight        device float [n] (out), or NULL to skip it; every entry is
 *                     written (0 for a splat no pixel composites)
 *   workspace         device scratch of at least gs_rasterize_fwd_workspace_size(n)
 *                     bytes (48 per splat), 256-byte aligned; contents on entry do
 *                     not matter
 */
size_t gs_rasterize_fwd_workspace_size(int32_t n);

gs_status gs_rasterize_fwd(int32_t n, const float* means2d, const float* conics, const float* colors,
                           const float* opacities, const float* background, int32_t width,
                           int32_t height, const int32_t* tile_ranges, const int32_t* sorted_ids,
                           int64_t n_isect, float* image, float* final_T, int32_t* n_contrib, float* max_weight,
                           void* workspace, size_t workspace_bytes, gs_stream_t stream);

/*
 * gs_rasterize_fwd with the depth outputs: the distortion and median-depth
 * options of rasterize_bwd_2d that the Spirula Studio page lists (section
 * 机制拆解: a per-pixel float4 of "distortion totals" and a median output)
 * without defining them. Read as
 *
 *   median      the depth of the last composited splat whose transmittance
 *               before it is still > 1/2, 0 when nothing composites; and its
 *               list position (within the tile's list) plus one, 0 for none
 *   distortion  D = sum over composited pairs i < j of w_i w_j (z_i - z_j)^2,
 *               w = alpha T, z = the splat's depth
 *   totals      (A, B, C, D): A = sum w, B = sum w (z - median),
 *               C = sum w (z - median)^2, and D (which equals A C - B^2)
 *
 * Same arguments, outputs and errors as gs_rasterize_fwd, and:
 *   depths        device float [n], the depths given to gs_bin_tiles; required
 *                 when any depth output is asked for
 *   dist_totals   device float [height][width][4] (out), or NULL
 *   median_depth  device float [height][width] (out), or NULL
 *   median_pos    device int32 [height][width] (out), or NULL
 * With all three NULL the call is gs_rasterize_fwd. Each combination of the
 * optional outputs runs its own kernel instance; without dist_totals no
 * instruction or register is spent on the sums.
 */
gs_status gs_rasterize_fwd_depth(int32_t n, const float* means2d, const float* conics, const float* colors,
                                 const float* opacities, const float* depths, const float* background,
                                 int32_t width, int32_t height, const int32_t* tile_ranges,
                                 const int32_t* sorted_ids, int64_t n_isect, float* image, float* final_T,
                                 int32_t* n_contrib, float* max_weight, float* dist_totals, float* median_depth,
                                 int32_t* median_pos, void* workspace, size_t workspace_bytes, gs_stream_t stream);

/*
 * Backward (rasterize_backwards in "Phase 5 step 30b — kernel-by-kernel
 * timing", sections 計測結果 and ホットスポット ranking; rasterize_bwd_2d on the
 * Spirula Studio page). One workgroup (4 wave64) per tile walks the tile's
 * list in reverse from the largest n_contrib of its pixels, recovers T by
 * division, and accumulates the nine gradient fields per splat. Partial sums
 * are reduced inside each wave and across the workgroup, stored once per
 * (splat, tile) pair into that pair's own workspace slot, and summed per
 * splat by a second kernel in a fixed order. With the deferred walk (the
 * default) and the stored-partials walk every sum runs in a fixed order, so
 * a call gives the same bits on every run; the LDS-add walk adds inside a
 * workgroup with LDS float atomics, whose order (and so the last bits) may
 * vary from run to run. No walk uses global floating-point atomics.
 *
 *   n .. opacities       as gs_rasterize_fwd
 *   radii                device int32 [n], the radii given to gs_bin_tiles
 *   background           device float [3] or NULL (black)
 *   tile_ranges, sorted_ids, splat_offsets, n_isect, n_slots
 *                        as returned by gs_bin_tiles for the same splats;
 *                        n_isect <= n_slots <= 2^31 - 1, else
 *                        GS_ERR_INVALID_ARG
 *   final_T, n_contrib   device, as written by gs_rasterize_fwd for the same
 *                        scene; n_contrib is clamped to each tile's list length
 *   dL_dimage            device float [height][width][3]
 *   dL_dmeans2d          device float [n][2] (out)
 *   dL_dconics           device float [n][3] (out): partials w.r.t. the stored
 *                        scalars a, b, c (b enters sigma as -b dx dy)
 *   dL_dcolors           device float [n][3] (out)
 *   dL_dopacities        device float [n]    (out)
 *   accum_weight         device float [n] (out), required iff
 *                        GS_FLAG_ACCUM_WEIGHT, else ignored (may be NULL)
 *   flags                bitwise OR of GS_FLAG_*
 *   workspace            device scratch of at least
 *                        gs_rasterize_bwd_workspace_size(n, n_slots, width,
 *                        height) bytes (48 per splat + 49 per slot + 8 per
 *                        tile), 256-byte aligned; contents on entry do not
 *                        matter
 *
 * Every output element is written; splats that no pixel takes get exact
 * zeros. Inputs that do not come from one binning of the same splats are
 * not detected; the kernels never write outside the outputs and workspace.
 */
/* 0 for n outside 0 .. 2^29, n_slots < 0 or a width / height outside 1..32768 */
size_t gs_rasterize_bwd_workspace_size(int32_t n, int64_t n_slots, int32_t width, int32_t height);

gs_status gs_rasterize_bwd(int32_t n, const float* means2d, const float* conics, const float* colors,
                           const float* opacities, const int32_t* radii, const float* background,
                           int32_t width, int32_t height, const int32_t* tile_ranges,
                           const int32_t* sorted_ids, const int32_t* splat_offsets, int64_t n_isect,
                           int64_t n_slots, const float* final_T, const int32_t* n_contrib, const float* dL_dimage,
                           float* dL_dmeans2d, float* dL_dconics, float* dL_dcolors,
                           float* dL_dopacities, float* accum_weight, uint32_t flags, void* workspace,
                           size_t workspace_bytes, gs_stream_t stream);

/*
 * gs_rasterize_bwd with the depth terms of gs_rasterize_fwd_depth: the
 * gradients of L = sum_p <dL_dimage_p, image_p> + dL_ddist_p D_p +
 * dL_dmedian_p median_p, every discrete decision (skip, stop, clamp, the
 * median's splat) held as the forward took it. The distortion reaches each
 * composited splat through its alpha (hence mean, conic and opacity) and its
 * depth, dD/dz_k = 2 w_k (A (z_k - median) - B); the median reaches only the
 * depth of its splat (dmedian/dz = 1).
 *
 * Same arguments, outputs and errors as gs_rasterize_bwd, and:
 *   depths        device float [n]; required with a depth term
 *   dist_totals   device float [height][width][4], as gs_rasterize_fwd_depth
 *                 wrote it; required with dL_ddist
 *   median_pos    device int32 [height][width], as gs_rasterize_fwd_depth
 *                 wrote it (clamped to [0, n_contrib]); required with a depth
 *                 term (the totals are taken about the median's depth)
 *   dL_ddist      device float [height][width], or NULL: no distortion term
 *   dL_dmedian    device float [height][width], or NULL: no median term
 *   dL_ddepths    device float [n] (out): required with a depth term; with
 *                 neither term it may be NULL, else it is zero-filled
 * The depth terms run on the deferred walk: with GS_FLAG_WALK_ADD or
 * GS_FLAG_WALK_STORE and a depth term the call returns GS_ERR_UNSUPPORTED.
 * Each combination of the terms is its own kernel instance (one more partial
 * sum per record and a per-wave LDS pad of one float per lane and step).
 */
gs_status gs_rasterize_bwd_depth(int32_t n, const float* means2d, const float* conics, const float* colors,
                                 const float* opacities, const float* depths, const int32_t* radii,
                                 const float* background, int32_t width, int32_t height,
                                 const int32_t* tile_ranges, const int32_t* sorted_ids,
                                 const int32_t* splat_offsets, int64_t n_isect, int64_t n_slots,
                                 const float* final_T, const int32_t* n_contrib, const float* dist_totals, const int32_t* median_pos,
                                 const float* dL_dimage, const float* dL_ddist, const float* dL_dmedian,
                                 float* dL_dmeans2d, float* dL_dconics, float* dL_dcolors, float* dL_dopacities,
                                 float* dL_ddepths, float* accum_weight, uint32_t flags, void* workspace,
                                 size_t workspace_bytes, gs_stream_t stream);

/*
 * gs_rasterize_bwd with its stages timed: the same work, arguments and errors,
 * and in addition a HIP event (created by the caller) recorded on `stream`
 * at each stage boundary, for measurement tools:
 *   events[0]  before the setup (splat records, per-tile walk lengths and the
 *              tiles' launch order, cleared slot flags)
 *   events[1]  before the reverse walk (the per-tile backward kernel)
 *   events[2]  after the reverse walk, before the per-splat gather
 *   events[3]  after the gather
 * NULL entries are skipped. With n == 0 or n_isect == 0 the walk is not
 * launched and events[1] and events[2] are recorded back to back.
 */
gs_status gs_rasterize_bwd_timed(int32_t n, const float* means2d, const float* conics, const float* colors,
                                 const float* opacities, const int32_t* radii, const float* background,
                                 int32_t width, int32_t height, const int32_t* tile_ranges,
                                 const int32_t* sorted_ids, const int32_t* splat_offsets, int64_t n_isect,
                                 int64_t n_slots, const float* final_T, const int32_t* n_contrib,
                                 const float* dL_dimage, float* dL_dmeans2d, float* dL_dconics, float* dL_dcolors,
                                 float* dL_dopacities, float* accum_weight, uint32_t flags, void* workspace,
                                 size_t workspace_bytes, gs_stream_t stream, const gs_event_t events[4]);

/*
 * gs_rasterize_bwd without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). Same arguments, results and errors as
 * gs_rasterize_bwd, less workspace / workspace_bytes; the caller still passes
 * every input and output.
 *
 * The workspace gs_rasterize_bwd would take lives in a fixed device array of
 * the library, gs_rasterize_bwd_noalloc_capacity() bytes (64 MiB), which each
 * GPU the library runs on holds from its first call until the process ends
 * (enough for about a million (splat, tile) slots: gs_rasterize_bwd_workspace_size
 * tells what a scene needs). A scene that needs more returns GS_ERR_CAPACITY
 * before anything is enqueued. The call allocates nothing: no hipMalloc, no
 * hipFree, no allocating library routine; its first call on a device looks up
 * that device's address of the array (hipGetSymbolAddress) and keeps it.
 * Every call on one GPU shares that GPU's array: calls that overlap on one GPU
 * (on different streams, or from different threads without ordering) race and
 * give wrong results. The kernels clear what must start at zero on every
 * call, so nothing carries over from the previous call.
 */
size_t gs_rasterize_bwd_noalloc_capacity(void);

gs_status gs_rasterize_bwd_noalloc(int32_t n, const float* means2d, const float* conics, const float* colors,
                                   const float* opacities, const int32_t* radii, const float* background,
                                   int32_t width, int32_t height, const int32_t* tile_ranges,
                                   const int32_t* sorted_ids, const int32_t* splat_offsets, int64_t n_isect,
                                   int64_t n_slots, const float* final_T, const int32_t* n_contrib, const float* dL_dimage,
                                   float* dL_dmeans2d, float* dL_dconics, float* dL_dcolors,
                                   float* dL_dopacities, float* accum_weight, uint32_t flags,
                                   gs_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* GSRASTER_H */
