// Step path (stepwise.hip): the arguments of one chunk's kernels, the
// workspace layout and the launchers.  Kept apart from common.h, which the
// on-chip kernels share.
#pragma once

#include "common.h"

namespace himuon {

// Arguments of the step-by-step path kernels for one chunk of tiles.
struct StepArgs {
    MatEntry mats[kGroup];
    float abc[3 * kMaxSteps];
    int32_t nmats;
    int32_t T;
    int32_t tile_begin;         // chunk = tiles [tile_begin, tile_end) of the group
    int32_t tile_end;
    int64_t xbase, abase;       // area offsets of tile_begin (subtracted from the class offsets)
    int32_t step;               // Newton-Schulz step this launch runs
    int32_t K;
    int32_t nb_max;             // 128-row macro blocks along r of the largest tile
    int32_t ns_max;             // 128-column macro blocks along s of the largest tile
    int32_t wg_norm;            // workgroups per tile in the normalisation kernels
    int32_t grid_blocks;        // workgroups launched (multiple of 8)
    int32_t io_dtype;           // matrices: 0 bf16, 1 fp32
    int32_t wk_dtype;           // workspace: 0 bf16, 1 fp32
    int32_t muon;
    float eps, mu, eta;
    int32_t normalize;          // 0: the tiles are used as they are (later runs of a tile-size schedule)
    int32_t slab;               // 1: the bf16 workspace is laid out in column slabs (ws_off) for the
                                // direct-to-LDS GEMMs; 0: row-major
    int32_t x_raw;              // 1: X holds the tiles as loaded, not yet scaled; the Gram product and
                                // the apply product that read it scale their result by the tile's
                                // 1 / (|X|_F + eps) (squared for X X^T), from the partial sums
    void* Xc;                   // oriented tiles, current step
    void* Xn;                   // oriented tiles, next step
    void* A;                    // Gram matrices A = X X^T
    void* B;                    // B' = a I + b A + c A^2
    float* partial;             // wg_norm partial sums of squares per tile
    // product of two r x r matrices with a symmetric result, O = L M^T (Gram
    // iteration); same layout and offsets as A
    const void* L;
    const void* M;
    void* O;
};

// Element offset of (row, col) in an r-row workspace matrix of ld8-element
// rows (ld8 a multiple of 8).  Row-major, or in slabs of 32 columns, each slab
// holding its r row pieces one after another (the last slab is ld8 mod 32
// wide when that is not 0).  A GEMM's k chunk of 32 columns over a run of rows
// is then one contiguous range, whole 128-byte lines, where row-major rows of
// a 512-wide tile give each row's 64-byte piece half a line (measured on
// MI355X: T = 512 on the dense 8192 layer 9.9 -> 9.0-9.3 ms, identical results).
// A 16-byte piece at a column that is a multiple of 8 never crosses a slab.
__host__ __device__ inline int64_t ws_off(int64_t row, int64_t col, int64_t r, int64_t ld8, bool slab) {
    if (!slab) return row * ld8 + col;
    const int64_t c0 = col & ~int64_t(31);
    const int64_t wd = ld8 - c0 < 32 ? ld8 - c0 : 32;
    return c0 * r + row * wd + (col - c0);
}

// K >= 1: one pass that takes the partial sums of squares and writes the
// oriented tiles unscaled (the caller then sets x_raw for the first Gram and
// apply products); K = 0: the sums, then the normalised tiles in place.
hipError_t launch_step_norm(const StepArgs& a, hipStream_t s);
// Whether the step GEMMs of a chunk run the direct-to-LDS kernels (bf16
// workspace addressed with 32-bit offsets): their workspace is in slabs.
bool step_slab_layout(const StepArgs& a);
hipError_t launch_step_gram(const StepArgs& a, hipStream_t s);
hipError_t launch_step_poly(const StepArgs& a, hipStream_t s);
hipError_t launch_step_apply(const StepArgs& a, hipStream_t s);
hipError_t launch_step_product(const StepArgs& a, hipStream_t s);

}  // namespace himuon
