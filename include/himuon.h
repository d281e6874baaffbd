/*
 * himuon.h - C ABI of the MI355X (gfx950) tiled Newton-Schulz library.
 *
 * What the library computes
 * -------------------------
 * HiMuon ("Hierarchical Muon: Tiled Newton-Schulz Updates for Efficient Muon
 * Optimization", arXiv 2606.27216, abstract): every H x W momentum matrix is
 * cut into T x T tiles anchored at (0, 0) (the last tile row and column hold
 * the remainder, processed at their own h x w size), the same finite
 * Newton-Schulz map is applied to every tile independently, and the results
 * are written back in place.
 *
 * The per-tile map is Algorithm 1 of the "Gram Newton-Schulz" summary page
 * (section 3, standard Newton-Schulz): X = Y / (||Y||_F + eps), then for
 * t = 1..K:  A = X X^T,  B = b_t A + c_t A^2,  X = a_t X + B X.
 * (The page's transpose of tall blocks only changes the cost: each step is an
 * odd matrix polynomial, so the result is the same either way.)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Matrices are row-major in device memory: element (i, j) of a descriptor
 *   sits at ptr + i * ld + j (in elements).  rows >= 1, cols >= 1, ld >= cols.
 *   All matrices of one call share one dtype.  Pointers must be aligned to the
 *   element size; no other alignment is required (16-byte aligned rows take a
 *   vector fast path).
 * - The caller owns all device memory.  The library allocates no device memory
 *   and keeps no device state between calls (himuon_tiled_ns_noalloc aside,
 *   which uses a fixed scratch array the library holds on each device).  The descriptor array and the
 *   coefficient array are read during the call only.  A call issues kernel
 *   launches only (no memsets or copies), so it may be captured in a HIP graph,
 *   and calls on different streams may run at once on disjoint matrices and
 *   workspaces.
 * - Work is enqueued on `stream` (a hipStream_t; NULL is the null stream) and
 *   the call returns without waiting.  Results are valid once the stream has
 *   reached that point.  The workspace must stay allocated until then.
 * - Validation is all-or-nothing: when a call returns anything but HIMUON_OK,
 *   nothing was enqueued and no memory was touched (HIMUON_ERR_HIP excepted: it
 *   reports a launch failure from the HIP runtime; himuon_last_hip_error()
 *   returns the hipError_t).
 * - Matrices of one call must not overlap in memory (they are written in
 *   place).  No exception crosses this interface.
 * - Non-finite inputs are not an error: a NaN or Inf stays inside its tile.
 * - bf16 tiles with both sides from 48 to 256 or from 32 to 128 (and tiles
 *   with both sides at most 64) stay resident on chip for all K steps and
 *   need no workspace: one kernel launch per group of up to 256 tile classes (a class
 *   is one matrix's interior, right-edge, bottom-edge or corner tiles), plus
 *   one for a partly filled last round of 128-tiles.  fp32 tiles with both
 *   sides at most 64 stay on chip too (fp32 MFMA, one launch per group).
 *   Larger tiles, thin tiles, larger fp32 tiles, and the full-matrix map
 *   (T >= max(rows, cols)) run step by step through the caller's workspace,
 *   in chunks of tiles that each fit in `workspace_bytes`; that workspace is
 *   bf16 for bf16 tiles whose sides are both at least 64, fp32 otherwise.
 *   HIMUON_BF16_PRECISE runs every tile on the step-by-step path with an
 *   fp32 workspace.
 */
#ifndef HIMUON_H
#define HIMUON_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Largest K accepted by any entry point. */
#define HIMUON_MAX_STEPS 16

/* One matrix: device pointer to element (0, 0), its size and row stride. */
typedef struct himuon_matrix {
    void*   ptr;   /* device pointer, aligned to the element size           */
    int64_t rows;  /* H >= 1                                                 */
    int64_t cols;  /* W >= 1                                                 */
    int64_t ld;    /* row stride in elements, ld >= cols                     */
} himuon_matrix_t;

/*
 * Storage and arithmetic.  The pages cast the normalised block to bf16 and
 * leave later precision open ("Gram Newton-Schulz" page, section 3,
 * Algorithm 1; section 6 notes on low-precision Gram iterations).
 *
 * Accuracy contract: the error of a tile is ||out - ref||_F / ||ref||_F with
 * ref the exact (fp64) map of the stored input; the bound is on the worst tile.
 *  - HIMUON_FP32: <= 1e-4 (measured at most a few 1e-6).
 *  - HIMUON_BF16: <= 3e-2 (measured 1.1e-2 to 2.0e-2 on the worst of 10^4 to
 *    10^6 random full-rank tiles per kernel size) for
 *      * K <= 5 steps (the quintic (3.4445, -4.7750, 2.0315) every step, or
 *        per-step mixes with cubic steps); tiles of up to 32 also for longer
 *        runs of converging steps, such as five quintic then eleven cubic
 *        (1.5, -0.5, 0) steps, which larger tiles exceed on a tail of tiles
 *        (1-3 % of random tiles, worst 0.15-0.25);
 *      * tiles without near-zero singular values (relative to the largest);
 *      * entries of magnitude about 1e-15 to 1e15 (tested at 2^-50 and
 *        2^50, with eps scaled to the data): the Frobenius reduction, and at
 *        kernel tile 128 the product X X^T of the raw tile, run in fp32 and
 *        underflow below about 1e-18 or overflow above about 1e17.
 *    It does NOT hold for tiles of low numerical rank (rank 1 to 16 of a
 *    128-tile: 0.17-0.29 measured), because the iterate is rounded to bf16
 *    every step and each step multiplies its small singular values by about
 *    a_t; nor for 16 quintic steps in a row (0.04-0.18 measured, by kernel
 *    size; the quintic keeps singular values where its slope exceeds 1, so
 *    every rounding grows from step to step).
 *  - HIMUON_BF16_PRECISE: bf16 storage, fp32 arithmetic throughout (the
 *    fp32 step-by-step path, fp32 MFMA); the result is rounded to bf16 once.
 *    <= 3e-2 also on the cases above (measured 1.7e-3 to 2.0e-3, mostly the
 *    final rounding), at a much lower throughput.  For calls whose tiles may
 *    be of low rank or that run many quintic steps.
 */
typedef enum himuon_dtype {
    HIMUON_BF16 = 0,          /* bfloat16 storage; bf16 MFMA with fp32 accumulation */
    HIMUON_FP32 = 1,          /* float32 storage; fp32 arithmetic throughout        */
    HIMUON_BF16_PRECISE = 2   /* bfloat16 storage; fp32 arithmetic throughout       */
} himuon_dtype_t;

typedef enum himuon_status {
    HIMUON_OK = 0,
    HIMUON_ERR_INVALID_ARGUMENT = 1, /* null pointer, size < 1, ld < cols, K or eps out of range, non-finite coefficient */
    HIMUON_ERR_UNSUPPORTED = 2,      /* dtype or option the library does not provide                                  */
    HIMUON_ERR_LAYOUT = 3,           /* pointer not aligned to the element size, or an index that overflows int64   */
    HIMUON_ERR_OVERLAP = 4,          /* two matrices that are written share memory                                  */
    HIMUON_ERR_WORKSPACE = 5,        /* workspace too small for one tile of the step-by-step path, or NULL with bytes > 0 */
    HIMUON_ERR_HIP = 6               /* the HIP runtime refused a launch                                            */
} himuon_status_t;

/* Summary of how a call would be carried out (host-side planning only). */
typedef struct himuon_plan_info {
    int64_t tiles;            /* tiles over all matrices                              */
    int64_t resident_launches;/* launch groups of the on-chip kernels (tiles <= 256, bf16) */
    int64_t chunks;           /* chunks of the step-by-step path (0 if not used)      */
    int64_t launches;         /* total kernel launches one call enqueues              */
    int64_t kernel_tile;      /* largest on-chip kernel size (32, 64, 128 or 256), or 0 */
    size_t  workspace_full;   /* bytes the step-by-step path needs for one chunk      */
    size_t  workspace_min;    /* bytes it needs for its largest single tile           */
    int64_t tail_tiles;       /* 128-tiles of the partial last round, run eight waves
                                 per tile by a second launch on the current device
                                 (0 when no device is visible)                        */
} himuon_plan_info_t;

/*
 * himuon_plan - describe how himuon_tiled_ns(m, n, T, K, ..., dt, ...,
 * workspace_bytes) would run, without touching the GPU.  workspace_bytes is
 * the cap the chunking must respect (ignored when no workspace is needed).
 * Returns the same validation status the call would return (pointers are not
 * dereferenced).
 */
himuon_status_t himuon_plan(const himuon_matrix_t* m, int32_t n, int32_t T, int32_t K,
                            himuon_dtype_t dt, size_t workspace_bytes,
                            himuon_plan_info_t* info);

/*
 * himuon_workspace_size - bytes of device workspace himuon_tiled_ns needs to
 * run all tiles of these matrices in a single chunk (*full) and the least it
 * accepts (*min, one tile).  Both are 0 when the call needs no workspace.
 * Either output pointer may be NULL.
 */
himuon_status_t himuon_workspace_size(const himuon_matrix_t* m, int32_t n, int32_t T,
                                      himuon_dtype_t dt, size_t* full, size_t* min);

/*
 * himuon_tiled_ns - HiMuon tiled Newton-Schulz, in place, on n matrices.
 *
 * m, n       : n >= 0 matrix descriptors (n == 0 is a no-op).
 * T          : tile edge, T >= 1.  Tiles are T x T anchored at (0, 0); edge
 *              tiles are h x w with h, w <= T.  T >= max(rows, cols) gives the
 *              full-matrix Newton-Schulz map of each matrix.
 * K          : number of Newton-Schulz steps, 0 <= K <= HIMUON_MAX_STEPS
 *              (K = 0 writes the Frobenius-normalised tiles).
 * abc        : 3*K floats, step t uses (a_t, b_t, c_t) = abc[3t .. 3t+2];
 *              may be NULL when K == 0.  Must be finite.
 * dt         : storage dtype of every matrix.
 * eps        : added to each tile's Frobenius norm (>= 0, finite); 1e-7 in
 *              the page's Algorithm 1.
 * workspace, workspace_bytes : device scratch for the step-by-step path; the
 *              tiles are processed in chunks that fit.  May be NULL / 0 when
 *              himuon_workspace_size reports 0.
 * stream     : hipStream_t to enqueue on.
 */
himuon_status_t himuon_tiled_ns(const himuon_matrix_t* m, int32_t n, int32_t T, int32_t K,
                                const float* abc, himuon_dtype_t dt, float eps,
                                void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device scratch the library holds for himuon_tiled_ns_noalloc. */
#define HIMUON_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)

/*
 * himuon_tiled_ns_noalloc - himuon_tiled_ns for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, and
 * harnesses that forbid hipMalloc.  It computes exactly what himuon_tiled_ns
 * computes (same kernels, same per-tile arithmetic, so the same bits) and
 * allocates nothing: the step-by-step path runs through a fixed scratch array
 * of HIMUON_NOALLOC_SCRATCH_BYTES (128 MiB) that the library holds on every
 * device it runs on, from the first use there until the process ends.  Tiles
 * are processed in chunks that fit it.
 *
 * Arguments as for himuon_tiled_ns, without the workspace.
 * Errors: as for himuon_tiled_ns; HIMUON_ERR_WORKSPACE when one tile of the
 * step-by-step path needs more than HIMUON_NOALLOC_SCRATCH_BYTES on its own
 * (for example a full-matrix map above about 64 M bf16 elements), reported
 * before the device is touched; HIMUON_ERR_HIP if the scratch address cannot
 * be obtained on the current device.
 * Every call on one device shares that device's scratch, which keeps the last
 * call's contents (nothing in it needs to start at zero).  Calls whose work
 * overlaps in time on one device (other streams, other threads) race on it:
 * order them on one stream, or use himuon_tiled_ns with separate workspaces.
 */
himuon_status_t himuon_tiled_ns_noalloc(const himuon_matrix_t* m, int32_t n, int32_t T, int32_t K,
                                        const float* abc, himuon_dtype_t dt, float eps, void* stream);

/*
 * himuon_tiled_ns_schedule - K Newton-Schulz steps with a tile size per step:
 * step k works on the T[k] x T[k] tiles (HiMuon abstract, "runtime tile-size
 * schedules", read as a per-step tile size).  Each tile of the first size is
 * normalised once (eps added to its Frobenius norm); later steps use the
 * tiles as they stand.  The sizes must not increase and each must divide the
 * one before, so a finer tile lies inside one coarser tile; the step count of
 * a size and its coefficients are taken in order from abc (3 K floats, host).
 * Steps of one size run as one himuon_tiled_ns pass; between passes the
 * matrices hold the current iterate in their own dtype.
 *
 * Arguments as for himuon_tiled_ns, with T a host array of K tile sizes.
 * workspace_bytes caps every pass; the workspace must fit the largest need of
 * any pass (himuon_workspace_size for that pass's tile size).
 * Errors: HIMUON_ERR_INVALID_ARGUMENT for K < 1 or > HIMUON_MAX_STEPS, a
 * null T, a size < 1, or sizes that increase or do not nest; otherwise as for
 * himuon_tiled_ns.  Every pass is validated before the first is enqueued.
 */
himuon_status_t himuon_tiled_ns_schedule(const himuon_matrix_t* m, int32_t n, const int32_t* T, int32_t K,
                                         const float* abc, himuon_dtype_t dt, float eps, void* workspace,
                                         size_t workspace_bytes, void* stream);

/*
 * himuon_muon_step - fused Muon update with the tiled map in place of polar()
 * ("Gram Newton-Schulz" summary page, section 3, the Muon update rule):
 *     M <- mu M + G            (stored back into M, rounded to dt)
 *     W <- W - eta * tiledNS(M)
 * W[i], M[i], G[i] must have equal rows and cols (their ld may differ).  W and
 * M are written; G is read only.  No W, M or G may overlap any written matrix.
 * Other arguments as for himuon_tiled_ns; mu and eta must be finite.
 */
himuon_status_t himuon_muon_step(const himuon_matrix_t* W, const himuon_matrix_t* M,
                                 const himuon_matrix_t* G, int32_t n, int32_t T, int32_t K,
                                 const float* abc, float mu, float eta, himuon_dtype_t dt,
                                 float eps, void* workspace, size_t workspace_bytes, void* stream);

/*
 * himuon_gram_ns - the full-matrix Newton-Schulz map of each matrix, in place,
 * computed through its Gram matrix ("Gram Newton-Schulz" summary page,
 * section 6, Algorithm 3, stabilised Gram Newton-Schulz with a restart).
 *
 * Each matrix Y is normalised, X = Y / (||Y||_F + eps), and oriented so that
 * X is r x s with r <= s (a tall matrix is worked on transposed).  The steps
 * then run on r x r matrices:
 *     R = X X^T,  Q = I;   for t = 1..K:
 *         P = a_t I + b_t R + c_t R^2,   Q <- P Q,   R <- P R P
 * and the result Q X is written back (in the matrix's own orientation).  In
 * exact arithmetic this equals himuon_tiled_ns with T >= max(rows, cols); the
 * iteration costs about 4 r^3 flops a step instead of 4 r^2 s + 2 r^3, so it
 * pays for wide matrices (s well above r).  Before step restart + 1 the
 * iteration restarts (the page restarts before its third step, restart = 2):
 * X <- Q X,  R <- X X^T,  Q <- I, which removes the rounding R has gathered.
 *
 * m, n       : n >= 0 matrix descriptors, as for himuon_tiled_ns.
 * K, abc     : steps and coefficients, as for himuon_tiled_ns.
 * restart    : >= 0; 0 (or >= K) never restarts (the page's Algorithm 2).
 * dt, eps    : as for himuon_tiled_ns.
 * workspace, workspace_bytes : device scratch, at least the *min of
 *              himuon_gram_ns_workspace; matrices are processed in chunks
 *              that fit (every matrix runs on the step-by-step path; K = 0
 *              writes the normalised matrices as himuon_tiled_ns does).
 * stream     : hipStream_t to enqueue on.
 * The workspace holds the iterates in bf16 when dt is bf16 and both sides of
 * the matrix are at least 96, else in fp32 (smaller Gram matrices lose too
 * much accuracy to bf16 rounding).
 * Errors: HIMUON_ERR_INVALID_ARGUMENT for restart < 0, otherwise as for
 * himuon_tiled_ns (HIMUON_ERR_LAYOUT also for a side above INT32_MAX).
 */
himuon_status_t himuon_gram_ns(const himuon_matrix_t* m, int32_t n, int32_t K, const float* abc,
                               int32_t restart, himuon_dtype_t dt, float eps, void* workspace,
                               size_t workspace_bytes, void* stream);

/* Bytes of workspace himuon_gram_ns needs for these matrices in one chunk
 * (*full) and for its largest single matrix (*min).  Host-side only; either
 * output pointer may be NULL. */
himuon_status_t himuon_gram_ns_workspace(const himuon_matrix_t* m, int32_t n, himuon_dtype_t dt,
                                         size_t* full, size_t* min);

/*
 * himuon_pair_stats - for n pairs of equal-shaped matrices (a[i], b[i]) the
 * three sums  sum a*b,  sum a*a,  sum b*b  over all elements, in fp64.
 *
 * They measure how far a tiled Newton-Schulz output lies from the
 * full-matrix map of the same input (HiMuon abstract: the tiled map acts on
 * each tile alone, where the full map couples all rows and columns; the pages
 * give no measure of that gap).  With g = tiled, f = full:
 *     ||g - f||_F / ||f||_F = sqrt(gg + ff - 2 gf) / sqrt(ff),
 *     cosine = gf / sqrt(gg ff).
 *
 * a, b     : n descriptors each (host arrays, read during the call); a[i] and
 *            b[i] must have equal rows and cols (their ld may differ).  Read
 *            only; they may overlap each other.
 * dt       : element type of every matrix.
 * out      : device array of 3 n doubles, written (out[3i .. 3i+2] =
 *            sum a*b, sum a*a, sum b*b of pair i); 8-byte aligned.
 * workspace, workspace_bytes : device scratch for per-workgroup partial sums,
 *            at least himuon_pair_stats_workspace(a, n) bytes, 8-byte aligned.
 * stream   : hipStream_t to enqueue on.
 * Products are exact in fp64 and summed in fp64 in a fixed order: the same
 * inputs give the same bits on every run.
 * Errors: HIMUON_ERR_INVALID_ARGUMENT (null pointer, size < 1, ld < cols,
 * shapes that differ), HIMUON_ERR_UNSUPPORTED (dtype), HIMUON_ERR_LAYOUT
 * (misaligned pointer), HIMUON_ERR_WORKSPACE (workspace NULL or too small),
 * HIMUON_ERR_HIP (launch refused).  n == 0 is a no-op.
 */
himuon_status_t himuon_pair_stats(const himuon_matrix_t* a, const himuon_matrix_t* b, int32_t n,
                                  himuon_dtype_t dt, double* out, void* workspace, size_t workspace_bytes,
                                  void* stream);

/* Bytes of workspace himuon_pair_stats needs for pairs of these shapes (the
 * shapes of `a`; pointers are not read).  Host-side only. */
himuon_status_t himuon_pair_stats_workspace(const himuon_matrix_t* a, int32_t n, size_t* bytes);

/* Static description of a status code (never NULL). */
const char* himuon_status_string(himuon_status_t s);

/* hipError_t of the most recent HIMUON_ERR_HIP on this thread (0 if none). */
int32_t himuon_last_hip_error(void);

/* Library version as major * 10000 + minor * 100 + patch. */
int32_t himuon_version(void);

#ifdef __cplusplus
}
#endif

#endif /* HIMUON_H */
