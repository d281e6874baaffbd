// Internal declarations shared by the host planner and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace himuon {

constexpr int kMaxSteps = 16;     // largest K (matches HIMUON_MAX_STEPS)
constexpr int kGroup = 256;       // tile classes per launch (kernel-argument table, ~25 KB)
// Bytes of the library's own device scratch (himuon_tiled_ns_noalloc; matches
// HIMUON_NOALLOC_SCRATCH_BYTES).
constexpr size_t kStaticScratchBytes = size_t(128) << 20;

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
    // Kernel tiles 64 and 128 (not the split-precision variants): steps with
    // bit k of sq_mask set run in square form, Z = A + sq_mu I rounded,
    // B' = Z^2 + sq_d I, on an iterate the host has scaled (abc then holds the
    // other steps' coefficients for that scaling; sym_schedule in resident.hip).
    float sq_mu[kMaxSteps], sq_d[kMaxSteps];
    int32_t sq_mask;
};

// Constants of the 32-tile kernel, which carries the iterate scaled, Y = g X
// (resident32.hip).
//  square = 1 (every step the same (a, b, c), c > 0; g = c^(1/4)):
//    fp32 steps Y' = ra Y + Ab bf16(beta Y + Ab Y) with Ab = bf16(A), bf16
//    steps Y' = ((A + mu I)^2 + d I) Y, with A = Y Y^T; the result is Y_K
//    times rlast = 1 / g.
//  square = 0: fp32 step k computes Y' = ra_k Y + Ab Z with Ab =
//    bf16(kap_k A) and Z = bf16(cb_k Y +- Ab Y) (the sign of c_k; c_k = 0:
//    Y' = ra_k Y + Ab Y); bf16 step k computes Y' = ra_k Y + (k1 A + k2 A^2) Y,
//    the identity entering the A^2 accumulator as dinit on the diagonal
//    (quad clear: that accumulator is dinit I alone, k2 = 1).
struct Consts32 {
    float g0;                 // scale of the normalised tile
    int32_t n_master;         // steps 0 .. n_master - 1 keep Y in fp32
    int32_t square;
    float beta, mu, d, ra, rlast;
    float k1[kMaxSteps];      // linear coefficient; exactly -1 or +1 within a run of equal b
    float k2[kMaxSteps];      // quadratic coefficient
    float ra_k[kMaxSteps];    // coefficient of Y
    float dinit[kMaxSteps];   // identity term over k2 (bf16 steps)
    float kap[kMaxSteps];     // fp32 steps: scale of the Gram matrix before its rounding
    float cb[kMaxSteps];      // fp32 steps: coefficient of Y in the inner factor
    int32_t quad;             // bit k: c_k != 0
    int32_t neg;              // bit k: c_k < 0
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
// fp32 tiles of up to 64 x 64: one four-wave workgroup per tile, fp32 MFMA
// (resident_f32.hip).
hipError_t launch_resident_f32(const ResidentArgs& a, bool muon, hipStream_t s);
hipError_t launch_resident_coop(const ResidentArgs& a, bool muon, hipStream_t s);
hipError_t launch_resident32(const ResidentArgs& a, bool muon, hipStream_t s);   // kernel tile 32, bf16 arithmetic
Consts32 consts32(const float* abc, int K);
hipError_t launch_resident256(const ResidentArgs& a, bool muon, bool narrow, hipStream_t s);
int resident_slots(int kernel_tile, bool muon, bool precise);   // tiles the device holds at once (0 on error)
int device_cus();
// Device address of the library's scratch array on the current device
// (static_scratch.hip); looked up once per device.
hipError_t static_scratch(void** out);

}  // namespace himuon
