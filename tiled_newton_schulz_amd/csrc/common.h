// Internal declarations shared by the host planner and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace himuon {

constexpr int kMaxSteps = 16;     // largest K (matches HIMUON_MAX_STEPS)
constexpr int kGroup = 256;       // tile classes per launch (kernel-argument table, ~25 KB)

// One tile class of one matrix in a launch: a rectangular block of the
// matrix's tile grid whose tiles all have the same size th x tw (the interior
// T x T tiles, the right-edge column, the bottom-edge row, or the corner).
// For the plain map only `m`/`m_ld` are used; the fused Muon step also reads G
// and updates W.
struct MatEntry {
    void* m;             // matrix the map runs on (momentum for the Muon step)
    void* w;             // Muon step: weights
    const void* g;       // Muon step: gradient
    int64_t m_ld, w_ld, g_ld;
    int64_t xoff, aoff;  // step path: element offsets of the class's first tile
    int32_t ti0, tj0;    // first tile row and column of the class
    int32_t n_tj;        // tiles per row of the class
    int32_t th, tw;      // tile height and width
    int32_t tile_base;   // index of the class's first tile in the launch
};

// Arguments of the on-chip kernel (tiles up to 128 x 128, bf16): every tile
// runs all K steps in one wavefront.
struct ResidentArgs {
    MatEntry mats[kGroup];
    float abc[3 * kMaxSteps];
    int32_t nmats;
    int32_t total_tiles;  // tiles of the launch table
    int32_t tile_begin;   // this launch runs tiles [tile_begin, tile_end)
    int32_t tile_end;
    int32_t T;           // grid tile size: tile (i, j) starts at (i T, j T)
    int32_t K;
    float eps;
    float mu, eta;       // Muon step only
    int32_t normalize;   // 0: the tiles are used as they are (later runs of a tile-size schedule)
};

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

// Index of the class holding tile t: the last entry with tile_base <= t
// (binary search over the launch table; the search is uniform per wave).
__host__ __device__ inline int find_class(const MatEntry* mats, int n, int t) {
    int lo = 0, hi = n - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (mats[mid].tile_base <= t) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// ---- tile geometry ---------------------------------------------------------
// On the step path every tile is stored oriented (r = min(h, w) rows,
// s = max(h, w) columns) with rows padded to a multiple of 8 elements; the
// tiles of a class follow one another, and so do their r x round8(r) Gram
// buffers.
__host__ __device__ inline int64_t round8(int64_t x) { return (x + 7) & ~int64_t(7); }

struct TileGeom {
    int32_t r0, c0, h, w;   // position and size in the matrix
    int32_t r, s;           // oriented size, r <= s
    int32_t tr;             // 1 if the tile is tall (stored transposed)
    int64_t xoff, aoff;     // element offsets in the X and A areas
};

__host__ __device__ inline TileGeom class_tile(const MatEntry& e, int32_t T, int32_t local) {
    TileGeom g;
    const int32_t i = local / e.n_tj, j = local - i * e.n_tj;
    g.r0 = (e.ti0 + i) * T;
    g.c0 = (e.tj0 + j) * T;
    g.h = e.th;
    g.w = e.tw;
    g.tr = g.h > g.w;
    g.r = g.tr ? g.w : g.h;
    g.s = g.tr ? g.h : g.w;
    g.xoff = e.xoff + int64_t(local) * g.r * round8(g.s);
    g.aoff = e.aoff + int64_t(local) * g.r * round8(g.r);
    return g;
}

// Host-side launchers (defined in the .hip files).
// narrow: kernel tile 256 with the shorter tile side <= 128
hipError_t launch_resident(const ResidentArgs& a, int kernel_tile, bool muon, bool precise, bool narrow,
                           hipStream_t s);
hipError_t launch_resident_coop(const ResidentArgs& a, bool muon, hipStream_t s);
hipError_t launch_resident256(const ResidentArgs& a, bool muon, bool narrow, hipStream_t s);
int resident_slots(int kernel_tile, bool muon, bool precise);   // tiles the device holds at once (0 on error)
int device_cus();
hipError_t launch_step_norm(const StepArgs& a, hipStream_t s);
hipError_t launch_step_gram(const StepArgs& a, hipStream_t s);
hipError_t launch_step_poly(const StepArgs& a, hipStream_t s);
hipError_t launch_step_apply(const StepArgs& a, hipStream_t s);
hipError_t launch_step_product(const StepArgs& a, hipStream_t s);

}  // namespace himuon
