// Step-by-step tiled Newton-Schulz on gfx950: tile sizes above 128, fp32
// data, and the full-matrix map (T >= max(rows, cols)).
//
// The map per tile is Algorithm 1 of the "Gram Newton-Schulz" summary page
// (section 3): normalise by ||X||_F + eps, orient so the Gram matrix is the
// short side, then K steps of A = X X^T, B = b A + c A^2, X = a X + B X.  Each
// step is three batched launches over the chunk's tiles, all on MFMA:
//   gram : A  = X X^T            lower 128x128 blocks, stored with their mirror
//   poly : B' = a I + b A + c A A lower blocks (A symmetric, so A A = A A^T)
//   apply: X' = B' X             (equal to a X + B X in exact arithmetic)
// The last apply writes the result in place in the input dtype, undoing the
// orientation.  One launch before the steps takes the per-tile partial sums of
// squares (fixed partition and order, so the result is deterministic) and
// writes the oriented tiles unscaled; the first gram and apply launches scale
// their results by the tile's 1 / (||X||_F + eps) (twice for X X^T), so the
// tiles are read once and the first products see them unrounded.
//
// bf16 workspaces use step_gemm_async (global -> LDS by buffer_load ... lds,
// epilogue through LDS); fp32 workspaces and operands of 2 GiB or more use
// step_gemm_kernel (register-staged loads, element-wise stores).
//
// Workgroup -> (tile, block) ids are remapped so that the blocks of one tile
// run on one XCD and share its L2.

#include <algorithm>

#include "device_util.h"
#include "stepargs.h"

namespace himuon {

namespace {

// Element access for the two storage types.
template <int DT> struct Elem;
template <> struct Elem<0> {
    using T = unsigned short;
    __device__ static float ld(const T* p) { return bf2f(*p); }
    __device__ static T cv(float f) { return f2bf(f); }
};
template <> struct Elem<1> {
    using T = float;
    __device__ static float ld(const T* p) { return *p; }
    __device__ static T cv(float f) { return f; }
};

struct TileRef {
    TileGeom g;
    int32_t mi;
};

__device__ __forceinline__ TileRef find_tile(const StepArgs& a, int t) {
    const int mi = find_class(a.mats, a.nmats, t);
    const MatEntry& me = a.mats[mi];
    TileRef r;
    r.mi = mi;
    r.g = class_tile(me, a.T, t - me.tile_base);
    r.g.xoff -= a.xbase;
    r.g.aoff -= a.abase;
    return r;
}

// Scale of chunk tile tl, 1 / (|X|_F + eps), from the normalisation pass's
// partial sums (summed in the same order wherever it is taken)
__device__ __forceinline__ float tile_scale(const StepArgs& a, int tl) {
    float tot = 0.f;
    for (int i = 0; i < a.wg_norm; ++i) tot += a.partial[(int64_t)tl * a.wg_norm + i];
    return a.normalize ? 1.0f / (sqrtf(tot) + a.eps) : 1.0f;
}

__device__ __forceinline__ float block_sum(float v, float* red) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    __syncthreads();
    float s = 0.f;
    for (int i = 0; i < (int)(blockDim.x >> 6); ++i) s += red[i];
    __syncthreads();
    return s;
}

}  // namespace

// ---------------------------------------------------------------------------
// Normalisation.  Grid: wg_norm workgroups per tile; workgroup k of a tile
// handles the tile's 64x64 sub-blocks k, k + wg_norm, ...
// Pass 2 (K >= 1): Muon prologue M <- mu M + G (stored), partial sum of
// squares, and the tile written oriented and unscaled into Xc.
// K == 0: pass 0 (the prologue and the partial sums), then pass 1: scale =
// 1 / (sqrt(sum of the tile's partials) + eps) and the scaled tile written
// straight back in place (Muon: W <- W - eta X).
// ---------------------------------------------------------------------------
template <int IO, int WK, int PASS>
__global__ __launch_bounds__(256) void step_norm_kernel(const StepArgs a) {
    using E = Elem<IO>;
    using ET = typename E::T;
    using EW = Elem<WK>;
    using WT = typename EW::T;
    __shared__ float red[4];
    __shared__ float tileT[64][65];

    const int tl = blockIdx.x / a.wg_norm, k = blockIdx.x % a.wg_norm;
    const int t = a.tile_begin + tl;
    if (t >= a.tile_end) return;
    const TileRef tr = find_tile(a, t);
    const TileGeom& g = tr.g;
    const MatEntry& me = a.mats[tr.mi];
    ET* mbase = reinterpret_cast<ET*>(me.m) + (int64_t)g.r0 * me.m_ld + g.c0;
    const int sbw = (g.w + 63) / 64, sbh = (g.h + 63) / 64;
    const int tid = threadIdx.x;
    // each thread moves runs of 8 consecutive elements: row tid/8 (+32), columns 8 (tid%8) ..
    const int rr = tid >> 3, cc8 = (tid & 7) * 8;

    // 8 elements of row i starting at column j of a matrix, masked to w columns
    auto load8 = [&](const ET* base, int64_t ld, int i, int j, int w, float (&v)[8]) {
        const ET* p = base + (int64_t)i * ld + j;
        if (j + 8 <= w && ((reinterpret_cast<uintptr_t>(p) & (8 * sizeof(ET) - 1)) == 0)) {
            if constexpr (IO == 0) {
                const u16x8 u = *reinterpret_cast<const u16x8*>(p);
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = bf2f(u[e]);
            } else {
                const float4 u0 = *reinterpret_cast<const float4*>(p);
                const float4 u1 = *reinterpret_cast<const float4*>(p + 4);
                v[0] = u0.x; v[1] = u0.y; v[2] = u0.z; v[3] = u0.w;
                v[4] = u1.x; v[5] = u1.y; v[6] = u1.z; v[7] = u1.w;
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = (j + e < w) ? E::ld(p + e) : 0.f;
        }
    };
    auto store8 = [&](ET* base, int64_t ld, int i, int j, int w, const float (&v)[8]) {
        ET* p = base + (int64_t)i * ld + j;
        if (j + 8 <= w && ((reinterpret_cast<uintptr_t>(p) & (8 * sizeof(ET) - 1)) == 0)) {
            if constexpr (IO == 0) {
                u16x8 u;
#pragma unroll
                for (int e = 0; e < 8; ++e) u[e] = f2bf(v[e]);
                *reinterpret_cast<u16x8*>(p) = u;
            } else {
                *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
                *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (j + e < w) p[e] = E::cv(v[e]);
        }
    };
    // 8 workspace elements (rows padded to a multiple of 8, so always whole)
    auto wstore8 = [&](WT* p, const float (&v)[8]) {
        if constexpr (WK == 0) {
            u16x8 u;
#pragma unroll
            for (int e = 0; e < 8; ++e) u[e] = f2bf(v[e]);
            *reinterpret_cast<u16x8*>(p) = u;
        } else {
            *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
            *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
        }
    };

    if (PASS == 0 || PASS == 2) {
        // sums of squares of this workgroup's 64 x 64 sub-blocks (Muon: of the
        // new momentum, stored); PASS 2 also writes the oriented tile unscaled
        const ET* gbase = a.muon ? reinterpret_cast<const ET*>(me.g) + (int64_t)g.r0 * me.g_ld + g.c0 : nullptr;
        WT* xo = reinterpret_cast<WT*>(a.Xc) + g.xoff;
        const int64_t xld = round8(g.s);
        float ss = 0.f;
        for (int sb = k; sb < sbw * sbh; sb += a.wg_norm) {
            const int i0 = (sb / sbw) * 64, j0 = (sb % sbw) * 64;
            float vk[2][8];   // the two runs of 8 this thread holds (zero outside the tile)
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int i = i0 + rr + 32 * half, j = j0 + cc8;
                float (&v)[8] = vk[half];
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = 0.f;
                if (i >= g.h || j >= g.w) continue;
                load8(mbase, me.m_ld, i, j, g.w, v);
                if (a.muon) {
                    float gv[8];
                    load8(gbase, me.g_ld, i, j, g.w, gv);
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const ET nv = E::cv(a.mu * v[e] + gv[e]);
                        v[e] = E::ld(&nv);
                    }
                    store8(mbase, me.m_ld, i, j, g.w, v);
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) ss = __builtin_fmaf(v[e], v[e], ss);
                // row i of the tile, 8 elements; past w they are zero, so the
                // row's padding up to round8(w) is written as zeros
                if (PASS == 2 && !g.tr) wstore8(xo + ws_off(i, j, g.r, xld, a.slab != 0), v);
            }
            if (PASS == 2 && g.tr) {
                // tall tile: stored transposed, through LDS so both sides move
                // whole runs
#pragma unroll
                for (int half = 0; half < 2; ++half)
#pragma unroll
                    for (int e = 0; e < 8; ++e) tileT[rr + 32 * half][cc8 + e] = vk[half][e];
                __syncthreads();
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    const int j = rr + 32 * half;   // oriented row (original column j0 + j)
                    if (j0 + j < g.w && i0 + cc8 < g.h) {
                        float v[8];
#pragma unroll
                        for (int e = 0; e < 8; ++e) v[e] = tileT[cc8 + e][j];
                        // 8 elements; past h they are zero (padding up to round8(h))
                        wstore8(xo + ws_off(j0 + j, i0 + cc8, g.r, xld, a.slab != 0), v);
                    }
                }
                __syncthreads();
            }
        }
        ss = block_sum(ss, red);
        if (tid == 0) a.partial[(int64_t)tl * a.wg_norm + k] = ss;
        return;
    }

    // pass 1 (K == 0): the normalised tile, in place (Muon: W -= eta * it)
    const float scale = tile_scale(a, tl);
    ET* wbase = a.muon ? reinterpret_cast<ET*>(me.w) + (int64_t)g.r0 * me.w_ld + g.c0 : nullptr;
    for (int sb = k; sb < sbw * sbh; sb += a.wg_norm) {
        const int i0 = (sb / sbw) * 64, j0 = (sb % sbw) * 64;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int i = i0 + rr + 32 * half, j = j0 + cc8;
            if (i >= g.h || j >= g.w) continue;
            float v[8];
            load8(mbase, me.m_ld, i, j, g.w, v);
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] *= scale;
            if (a.muon) {
                float wv[8];
                load8(wbase, me.w_ld, i, j, g.w, wv);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const ET r = E::cv(v[e]);
                    wv[e] = wv[e] - a.eta * E::ld(&r);
                }
                store8(wbase, me.w_ld, i, j, g.w, wv);
            } else {
                store8(mbase, me.m_ld, i, j, g.w, v);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Batched MFMA GEMM over the chunk's tiles.  128x128 output block per
// workgroup of 4 waves (2x2, 64x64 each as 2x2 blocks of 32x32).
// MODE 0 gram:  C = X X^T          (r x r, contraction over s), lower blocks
// MODE 1 poly:  C = A A, B' = a I + b A + c C                   lower blocks
// MODE 2 apply: C = B' X           (r x s, contraction over r)
// MODE 3 product: C = L M^T        (r x r, contraction over r), lower blocks;
//                 for results known to be symmetric (products of matrices
//                 that commute, as in the Gram iteration); the diagonal
//                 blocks keep their lower triangle, so C is exactly symmetric
// bf16: v_mfma_f32_32x32x16_bf16, k chunk 64; fp32: v_mfma_f32_32x32x2f32,
// k chunk 32; two LDS stages.  Row operands are read from LDS along k; the X
// operand of apply (k along rows of X) uses ds_read_tr16_b64 for bf16.
// ---------------------------------------------------------------------------
// Final result element (i, j) of a tile, in place in the matrix dtype (Muon:
// W <- W - eta * result, with the result rounded to the dtype first, as the
// plain map would store it).
template <int IO>
__device__ __forceinline__ void store_out(const StepArgs& a, const MatEntry& me, const TileGeom& g, int oi, int oj,
                                          float v) {
    using E = Elem<IO>;
    using ET = typename E::T;
    const ET rv = E::cv(v);
    if (a.muon) {
        ET* wp = reinterpret_cast<ET*>(me.w) + (int64_t)(g.r0 + oi) * me.w_ld + g.c0 + oj;
        *wp = E::cv(E::ld(wp) - a.eta * E::ld(&rv));
    } else {
        ET* op = reinterpret_cast<ET*>(me.m) + (int64_t)(g.r0 + oi) * me.m_ld + g.c0 + oj;
        *op = rv;
    }
}

// k chunk of the DMA GEMMs (elements): one workspace slab
constexpr int kAsyncBK = 32;

// ws_off in the slab layout with 32-bit arithmetic: the direct-to-LDS GEMMs
// run only where a tile's areas stay below 2 GiB
__device__ __forceinline__ uint32_t slab_off(int row, int col, int r, int ld8) {
    const int c0 = col & ~31;
    const int wd = ld8 - c0 < 32 ? ld8 - c0 : 32;
    return (uint32_t)c0 * (uint32_t)r + (uint32_t)(row * wd + (col - c0));
}
// Chunks whose largest tile has at least this many 128-row blocks run the
// 256 x 256 block shape (measured on MI355X: the symmetric products are level
// at r = 2048 and gain 38 % for X X^T of an 8192 x 28672 matrix; at r = 1024
// the 128 x 128 shape is 3 % faster on the slab workspace (it was 13 % slower
// on row-major rows); the apply product is level at r = s = 2048, 8 % faster
// at 2048 x 5632 and 16 % at 8192 x 28672, and 6 % slower at r = s = 1024)
constexpr int kBigNbSym = 16;
constexpr int kBigNbApply = 16;
template <int DT> struct GemmCfg;
template <> struct GemmCfg<0> {
    static constexpr int BK = 64, EPC = 8;         // k chunk, elements per 16-byte chunk
    static constexpr int LDP = BK + 8;             // row-panel stride (elements)
    static constexpr int LDN = 128 + 16;           // X-panel stride for apply
};
template <> struct GemmCfg<1> {
    static constexpr int BK = 32, EPC = 4;
    static constexpr int LDP = BK + 1;
    static constexpr int LDN = 128 + 4;
};

// Epilogue of the step GEMMs: lane l, register q of block (i,j) holds
// C[m0 + wm*64 + i*32 + rho(l,q)][n0 + wn*64 + j*32 + l%32]; the four registers
// 4m..4m+3 are four consecutive rows, so a transposed (mirrored) store writes
// them as one run.  aval (poly only) holds A over the same positions.
template <int DT, int MODE>
__device__ __forceinline__ void gemm_epilogue(const StepArgs& a, const TileRef& tref, int bm, int bn, int m0,
                                              int n0, int wm, int wn, int l32, int gl, const f32x16 (&acc)[2][2],
                                              const float (&aval)[2][2][16], float xs) {
    using E = Elem<DT>;
    using ET = typename E::T;
    const TileGeom& g = tref.g;
    const float ca = a.abc[3 * a.step], cb = a.abc[3 * a.step + 1], cc = a.abc[3 * a.step + 2];
    const bool last = (MODE == 2) && (a.step == a.K - 1);
    const MatEntry& me = a.mats[tref.mi];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int row0 = m0 + wm * 64 + i * 32 + m * 8 + gl * 4;   // rows row0 .. row0+3
                const int col = n0 + wn * 64 + j * 32 + l32;
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[e] = acc[i][j][4 * m + e];
                    // X read unscaled: X X^T takes the scale twice, B' X once
                    if (MODE == 0) v[e] = (v[e] * xs) * xs;
                    if (MODE == 2) v[e] *= xs;
                }
                if (MODE != 2) {
                    // columns up to the padded row length are written: past r
                    // the product is exactly zero (zero operand rows), which
                    // keeps the padding of A and B' zero for readers that do not
                    // mask it
                    const int64_t ld = round8(g.r);
                    if (col >= ld) continue;
                    ET* Out = reinterpret_cast<ET*>(MODE == 0 ? a.A : MODE == 1 ? a.B : a.O) + g.aoff;
                    if (MODE == 1) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            if (row0 + e < g.r) {
                                float bv = __builtin_fmaf(cc, v[e], cb * aval[i][j][4 * m + e]);
                                if (row0 + e == col && col < g.r) bv += ca;
                                v[e] = bv;
                            }
                        }
                    }
                    ET o[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) o[e] = E::cv(v[e]);
                    if (MODE == 3 && bm == bn) {
                        // diagonal block of a product of two different
                        // matrices: its two triangles differ by rounding, so
                        // the lower one is kept and mirrored and the stored
                        // result is exactly symmetric (padding columns get
                        // their zeros directly)
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int rr = row0 + e;
                            if (rr >= g.r) continue;
                            if (rr >= col || col >= g.r) Out[(int64_t)rr * ld + col] = o[e];
                            if (rr > col) Out[(int64_t)col * ld + rr] = o[e];
                        }
                        continue;
                    }
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (row0 + e < g.r) Out[(int64_t)(row0 + e) * ld + col] = o[e];
                    if (bm != bn && col < g.r) {
                        // mirror: row col, columns row0 .. row0+3 (rows are
                        // padded to 8 elements, so a run is whole or outside)
                        ET* mp = Out + (int64_t)col * ld + row0;
                        if (row0 + 4 <= ld) {
                            if constexpr (DT == 0) {
                                u32x2 pk = {(unsigned)__builtin_bit_cast(unsigned short, o[0]) |
                                                ((unsigned)__builtin_bit_cast(unsigned short, o[1]) << 16),
                                            (unsigned)__builtin_bit_cast(unsigned short, o[2]) |
                                                ((unsigned)__builtin_bit_cast(unsigned short, o[3]) << 16)};
                                *reinterpret_cast<u32x2*>(mp) = pk;
                            } else {
                                *reinterpret_cast<float4*>(mp) = make_float4(o[0], o[1], o[2], o[3]);
                            }
                        } else {
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                if (row0 + e < g.r) mp[e] = o[e];
                        }
                    }
                } else {
                    if (col >= (last ? g.s : round8(g.s))) continue;
                    if (!last) {
                        ET* Xo = reinterpret_cast<ET*>(a.Xn) + g.xoff;
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (row0 + e < g.r) Xo[(int64_t)(row0 + e) * round8(g.s) + col] = E::cv(v[e]);
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            if (row0 + e >= g.r) continue;
                            const int oi = g.tr ? col : row0 + e, oj = g.tr ? row0 + e : col;
                            if (a.io_dtype == 0) store_out<0>(a, me, g, oi, oj, v[e]);
                            else store_out<1>(a, me, g, oi, oj, v[e]);
                        }
                    }
                }
            }
}

template <int DT, int MODE>
__global__ __launch_bounds__(256) void step_gemm_kernel(const StepArgs a) {
    using E = Elem<DT>;           // workspace element
    using ET = typename E::T;
    using C = GemmCfg<DT>;
    constexpr int BK = C::BK, EPC = C::EPC, LDP = C::LDP, LDN = C::LDN;
    constexpr bool NN = MODE == 2;
    // two stages of the row panel P and of the second operand Q
    constexpr int PSZ = 128 * LDP, QSZ = NN ? BK * LDN : 128 * LDP;
    __shared__ __attribute__((aligned(16))) ET sP2[2 * PSZ];
    __shared__ __attribute__((aligned(16))) ET sQ2[2 * QSZ];

    // ---- workgroup -> (tile, block), blocks of one tile on one XCD ----
    const int nwg = a.grid_blocks;
    const int L = (blockIdx.x & 7) * (nwg >> 3) + (blockIdx.x >> 3);
    const int bpt = NN ? a.nb_max * a.ns_max : a.nb_max * (a.nb_max + 1) / 2;
    const int tl = L / bpt, b = L - tl * bpt;
    const int t = a.tile_begin + tl;
    if (t >= a.tile_end) return;
    const TileRef tref = find_tile(a, t);
    const TileGeom& g = tref.g;
    const int nb = (g.r + 127) / 128, ns = (g.s + 127) / 128;
    int bm, bn;
    if (NN) {
        bm = b / a.ns_max;
        bn = b - bm * a.ns_max;
        if (bm >= nb || bn >= ns) return;
    } else {
        bm = (int)((sqrtf(8.f * b + 1.f) - 1.f) * 0.5f);
        while ((bm + 1) * (bm + 2) / 2 <= b) ++bm;
        while (bm * (bm + 1) / 2 > b) --bm;
        bn = b - bm * (bm + 1) / 2;
        if (bm >= nb) return;
    }
    const int m0 = bm * 128, n0 = bn * 128;

    // operands: P (rows m0.., k contiguous), Q (NT: rows n0.., k contiguous;
    // NN: rows k.., columns n0..)
    const ET* P;
    const ET* Q;
    int64_t ldp, ldq;
    int prow, kdim, qrow, qcol;
    if (MODE == 0) {
        P = reinterpret_cast<const ET*>(a.Xc) + g.xoff; ldp = round8(g.s);
        Q = P; ldq = ldp;
        prow = g.r; kdim = g.s; qrow = g.r; qcol = 0;
    } else if (MODE == 1) {
        P = reinterpret_cast<const ET*>(a.A) + g.aoff; ldp = round8(g.r);
        Q = P; ldq = ldp;
        prow = g.r; kdim = g.r; qrow = g.r; qcol = 0;
    } else if (MODE == 3) {
        P = reinterpret_cast<const ET*>(a.L) + g.aoff; ldp = round8(g.r);
        Q = reinterpret_cast<const ET*>(a.M) + g.aoff; ldq = ldp;
        prow = g.r; kdim = g.r; qrow = g.r; qcol = 0;
    } else {
        P = reinterpret_cast<const ET*>(a.B) + g.aoff; ldp = round8(g.r);
        Q = reinterpret_cast<const ET*>(a.Xc) + g.xoff; ldq = round8(g.s);
        prow = g.r; kdim = g.r; qrow = g.r; qcol = g.s;
    }

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int l32 = lane & 31, gl = lane >> 5;

    // global -> register staging: NCP chunks of 16 bytes per panel per thread
    constexpr int NCP = 128 * BK / EPC / 256;
    static_assert(NCP * 256 * EPC == 128 * BK, "panel chunks must cover the panel");
    u32x4 rp[NCP], rq[NCP];
    // a diagonal block of X X^T or A A has the same row panel as both operands:
    // it is loaded and stored once
    const bool one_panel = (MODE == 0 || MODE == 1) && bm == bn;
    auto load_panels = [&](int k0) {
#pragma unroll
        for (int p = 0; p < NCP; ++p) {
            const int c = tid + 256 * p;
            {   // P: 128 rows x BK
                const int row = c / (BK / EPC), kc = (c % (BK / EPC)) * EPC;
                u32x4 v = {0, 0, 0, 0};
                const int gr = m0 + row, gk = k0 + kc;
                if (gr < prow && gk < kdim) {
                    v = *reinterpret_cast<const u32x4*>(P + (int64_t)gr * ldp + gk);
                    if (gk + EPC > kdim) {
                        ET* e = reinterpret_cast<ET*>(&v);
#pragma unroll
                        for (int q = 0; q < EPC; ++q) if (gk + q >= kdim) e[q] = ET(0);
                    }
                }
                rp[p] = v;
            }
            if (!NN && !one_panel) {
                const int row = c / (BK / EPC), kc = (c % (BK / EPC)) * EPC;
                u32x4 v = {0, 0, 0, 0};
                const int gr = n0 + row, gk = k0 + kc;
                if (gr < qrow && gk < kdim) {
                    v = *reinterpret_cast<const u32x4*>(Q + (int64_t)gr * ldq + gk);
                    if (gk + EPC > kdim) {
                        ET* e = reinterpret_cast<ET*>(&v);
#pragma unroll
                        for (int q = 0; q < EPC; ++q) if (gk + q >= kdim) e[q] = ET(0);
                    }
                }
                rq[p] = v;
            } else {
                constexpr int CPR = 128 / EPC;
                const int row = c / CPR, cc = (c % CPR) * EPC;
                u32x4 v = {0, 0, 0, 0};
                const int gk = k0 + row, gc = n0 + cc;
                if (gk < kdim && gc < qcol) {
                    v = *reinterpret_cast<const u32x4*>(Q + (int64_t)gk * ldq + gc);
                    if (gc + EPC > qcol) {
                        ET* e = reinterpret_cast<ET*>(&v);
#pragma unroll
                        for (int q = 0; q < EPC; ++q) if (gc + q >= qcol) e[q] = ET(0);
                    }
                }
                rq[p] = v;
            }
        }
    };
    auto store_panels = [&](int stage) {
        ET* sP = sP2 + stage * PSZ;
        ET* sQ = sQ2 + stage * QSZ;
#pragma unroll
        for (int p = 0; p < NCP; ++p) {
            const int c = tid + 256 * p;
            const int row = c / (BK / EPC), kc = (c % (BK / EPC)) * EPC;
            if (DT == 0) {
                *reinterpret_cast<u32x4*>(&sP[row * LDP + kc]) = rp[p];
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q) reinterpret_cast<unsigned*>(sP)[row * LDP + kc + q] = rp[p][q];
            }
            if (!NN) {
                if (one_panel) {
                    // compute reads the P stage for both operands
                } else if (DT == 0) {
                    *reinterpret_cast<u32x4*>(&sQ[row * LDP + kc]) = rq[p];
                } else {
#pragma unroll
                    for (int q = 0; q < 4; ++q) reinterpret_cast<unsigned*>(sQ)[row * LDP + kc + q] = rq[p][q];
                }
            } else {
                constexpr int CPR = 128 / EPC;
                const int nrow = c / CPR, cc = (c % CPR) * EPC;
                *reinterpret_cast<u32x4*>(&sQ[nrow * LDN + cc]) = rq[p];
            }
        }
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

    auto compute = [&](int stage) {
        const ET* sP = sP2 + stage * PSZ;
        const ET* sQ = one_panel ? sP : sQ2 + stage * QSZ;
        if constexpr (DT == 0) {
#pragma unroll
            for (int kk = 0; kk < BK / 16; ++kk) {
                bf16x8 av[2], bv[2];
#pragma unroll
                for (int i = 0; i < 2; ++i)
                    av[i] = *reinterpret_cast<const bf16x8*>(&sP[(wm * 64 + i * 32 + l32) * LDP + kk * 16 + gl * 8]);
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    if (!NN) {
                        bv[j] = *reinterpret_cast<const bf16x8*>(&sQ[(wn * 64 + j * 32 + l32) * LDP + kk * 16 + gl * 8]);
                    } else {
                        const int G = lane >> 4, i16 = lane & 15;
                        const int col = wn * 64 + j * 32 + 16 * (G & 1) + 4 * (i16 & 3);
                        const int row = kk * 16 + 8 * gl + (i16 >> 2);
                        bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(&sQ[row * LDN + col]));
                        bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(&sQ[(row + 4) * LDN + col]));
                        bv[j] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                    }
                }
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[j], acc[i][j], 0, 0, 0);
            }
        } else {
            const float* fP = reinterpret_cast<const float*>(sP);
            const float* fQ = reinterpret_cast<const float*>(sQ);
#pragma unroll
            for (int kk = 0; kk < BK / 2; ++kk) {
                float av[2], bv[2];
#pragma unroll
                for (int i = 0; i < 2; ++i) av[i] = fP[(wm * 64 + i * 32 + l32) * LDP + kk * 2 + gl];
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    bv[j] = NN ? fQ[(kk * 2 + gl) * LDN + wn * 64 + j * 32 + l32]
                               : fQ[(wn * 64 + j * 32 + l32) * LDP + kk * 2 + gl];
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[i], bv[j], acc[i][j], 0, 0, 0);
            }
        }
    };

    // pipeline: the next k chunk is loaded to registers while the current one
    // is multiplied from LDS; one barrier per chunk
    const int nk = (kdim + BK - 1) / BK;
    load_panels(0);
    store_panels(0);
    __syncthreads();
    // poly: the epilogue needs A over this output block, which (A being
    // symmetric) is the k range [n0 + wn 64 + j 32, +32) of the row panel, so it
    // is taken from LDS while that chunk is resident
    float aval[2][2][16];
    for (int kt = 0; kt < nk; ++kt) {
        if (kt + 1 < nk) load_panels((kt + 1) * BK);
        compute(kt & 1);
        if constexpr (MODE == 1) {
            const ET* sP = sP2 + (kt & 1) * PSZ;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int c0 = n0 + wn * 64 + j * 32;
                if (kt == c0 / BK) {
                    const int cl = c0 - kt * BK + l32;
#pragma unroll
                    for (int i = 0; i < 2; ++i)
#pragma unroll
                        for (int q = 0; q < 16; ++q) {
                            const int rl = wm * 64 + i * 32 + (q >> 2) * 8 + gl * 4 + (q & 3);
                            aval[i][j][q] = E::ld(&sP[rl * LDP + cl]);
                        }
                }
            }
        }
        if (kt + 1 < nk) store_panels((kt + 1) & 1);
        __syncthreads();
    }

    const float xs = ((MODE == 0 || MODE == 2) && a.x_raw) ? tile_scale(a, tl) : 1.0f;
    gemm_epilogue<DT, MODE>(a, tref, bm, bn, m0, n0, wm, wn, l32, gl, acc, aval, xs);
}

// ---------------------------------------------------------------------------
// bf16 step GEMMs with direct global -> LDS loads (buffer_load ... lds), in two
// block shapes that share the code:
//   128 x 128 output block: 4 waves of 64 x 64, 32 KB of LDS, several
//     workgroups per CU;
//   256 x 256 output block: 8 waves of 128 x 64, 64 KB of LDS, one workgroup
//     per CU.  It moves half the bytes per flop from L2 into LDS (the CU's L1
//     waiting on L2 is what bounds these GEMMs) and reads 0.75 KB of LDS
//     operands per MFMA instead of 1 KB.
// Both run k chunks of 32 in two LDS stages, the next chunk in flight while one
// is multiplied, and accumulate every output element over k in the same
// order, so they give the same bits.  Loads are masked through the buffer
// range: a lane whose 16-byte chunk lies outside the operand (rows past the
// tile, columns past the row) gets an offset past the buffer's end and reads
// zeros.  The workspace's row padding (up to a multiple of 8 elements) is kept
// zero by every writer, so a chunk is either wholly valid or wholly outside.
// Stage layouts (dense, 16-byte chunks XOR-swizzled by row, so that both the
// lane-contiguous DMA writes and the MFMA operand reads are conflict free):
//   row panels (block rows x 32): chunk c of row r at position c ^ ((r >> 2) & 3)
//   X panel of apply (32 rows, in sub-panels of 128 columns): chunk c of row r
//                                 at position c ^ ((r & 3) * 4)
// The result goes out through LDS, 128 block rows at a time (rows padded by 8
// elements, so each lane's stores are a base plus constant offsets and the
// half-waves fall on different banks), as whole 16-byte row chunks; the
// mirrored block of a symmetric product goes the same way from the transposed
// rows.
// ---------------------------------------------------------------------------
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_of(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Output block (bm, bn) of linear block b within a tile, in groups of GM block
// rows walked column by column, so that the workgroups that run at once share
// both operands' k chunks in L2 (row-major order, GM = 1, shares only the row
// panel and streams one column panel per workgroup: with long k that re-reads
// every column panel from memory once per block row).  sym: the lower blocks
// bn <= bm of an nbm x nbm grid; else the full nbm x nsm grid.
__device__ __forceinline__ void grouped_block(int b, int nbm, int nsm, bool sym, int GM, int& bm, int& bn) {
    if (!sym) {
        const int per = GM * nsm;
        const int grp = b / per, o = b - grp * per;
        const int first = grp * GM, gm = min(GM, nbm - first);
        bm = first + o % gm;
        bn = o / gm;
        return;
    }
    // group g holds rows [g GM, g GM + gm); the lower blocks of rows < r number
    // r (r + 1) / 2
    int first = 0;
    while (first + GM < nbm && (first + GM) * (first + GM + 1) / 2 <= b) first += GM;
    const int gm = min(GM, nbm - first);
    int o = b - first * (first + 1) / 2;
    if (o < first * gm) {   // columns left of the group's diagonal square: gm blocks each
        bn = o / gm;
        bm = first + o % gm;
        return;
    }
    o -= first * gm;
    // the group's diagonal square, column c holding rows c .. gm - 1
    int c = 0;
    while (o >= gm - c) {
        o -= gm - c;
        ++c;
    }
    bn = first + c;
    bm = first + c + o;
}

template <bool BIG> struct AsyncShape;
template <> struct AsyncShape<false> {
    static constexpr int NT = 256, BE = 128, WNW = 2, FM = 2;
};
template <> struct AsyncShape<true> {
    static constexpr int NT = 512, BE = 256, WNW = 4, FM = 4;
};

template <int MODE, bool BIG>
__global__ __launch_bounds__(AsyncShape<BIG>::NT) void step_gemm_async(const StepArgs a) {
    using ET = unsigned short;
    using S = AsyncShape<BIG>;
    constexpr int NT = S::NT;                        // threads
    constexpr int BE = S::BE;                        // output block edge
    constexpr int WNW = S::WNW;                      // waves along n (two along m)
    constexpr int FM = S::FM, FN = 2;                // 32 x 32 MFMA blocks of a wave along m and n
    constexpr int WR = 32 * FM;                      // rows of a wave's tile (its columns: 64)
    constexpr int BK = kAsyncBK;
    constexpr int STAGE = BE * BK;                   // elements per operand and stage
    constexpr int CPR = BK / 8;                      // 16-byte chunks per panel row
    constexpr int NPI = BE * CPR / NT;               // DMA instructions per thread and operand
    constexpr int SH = CPR == 4 ? 2 : 1;             // row-panel swizzle: chunk ^ ((r >> SH) & (CPR - 1))
    constexpr int PR = 128;                          // block rows per epilogue pass
    constexpr int NPASS = BE / PR;
    constexpr int CH = BE / 8;                       // 16-byte chunks per block row
    constexpr int U = BE / 128;                      // 128-blocks per block edge
    static_assert(CPR == 4 || CPR == 8, "k chunk of 32 or 64");
    static_assert(NPI * NT == BE * CPR, "the DMA instructions cover a panel");
    constexpr int LDC = BE + 8;                      // LDS stride of the C rows of a pass
    constexpr int LDT = PR + 8;                      // LDS stride of the transposed rows
    constexpr int LDS_E = 4 * STAGE > PR * LDC ? (4 * STAGE > BE * LDT ? 4 * STAGE : BE * LDT)
                                               : (PR * LDC > BE * LDT ? PR * LDC : BE * LDT);
    constexpr bool NN = MODE == 2;
    constexpr bool SYM = MODE != 2;
    __shared__ __attribute__((aligned(16))) ET sbuf[LDS_E];   // two stages of P and Q; the C rows
    ET* const sP0 = sbuf;
    ET* const sP1 = sbuf + STAGE;
    ET* const sQ0 = sbuf + 2 * STAGE;
    ET* const sQ1 = sbuf + 3 * STAGE;

    // ---- workgroup -> (tile, block), blocks of one tile on one XCD ----
    const int nwg = a.grid_blocks;
    const int L = (blockIdx.x & 7) * (nwg >> 3) + (blockIdx.x >> 3);
    const int nbm = (a.nb_max + U - 1) / U, nsm = (a.ns_max + U - 1) / U;
    const int bpt = NN ? nbm * nsm : nbm * (nbm + 1) / 2;
    const int tl = L / bpt, b = L - tl * bpt;
    const int t = a.tile_begin + tl;
    if (t >= a.tile_end) return;
    const TileRef tref = find_tile(a, t);
    const TileGeom& g = tref.g;
    const int nb = (g.r + BE - 1) / BE, ns = (g.s + BE - 1) / BE;
    // groups pay where k is long (measured: the full map of an 8192 x 28672
    // matrix fetches 2.8 times less past L2 and runs 8 % faster; with k = 2048
    // row-major order is 6 % faster)
    const int klen = MODE == 0 ? g.s : g.r;
    int bm, bn;
    grouped_block(b, nbm, nsm, !NN, klen >= 4096 ? (BIG ? 4 : 8) : 1, bm, bn);
    if (bm >= nb || bn >= ns) return;
    const int m0 = bm * BE, n0 = bn * BE;

    const ET* P;
    const ET* Q;
    int ldp, ldq, prow, kdim, qrows, qcol;
    if (MODE == 0) {
        P = reinterpret_cast<const ET*>(a.Xc) + g.xoff; ldp = (int)round8(g.s);
        Q = P; ldq = ldp;
        prow = g.r; kdim = g.s; qrows = g.r; qcol = 0;
    } else if (MODE == 1) {
        P = reinterpret_cast<const ET*>(a.A) + g.aoff; ldp = (int)round8(g.r);
        Q = P; ldq = ldp;
        prow = g.r; kdim = g.r; qrows = g.r; qcol = 0;
    } else if (MODE == 3) {
        P = reinterpret_cast<const ET*>(a.L) + g.aoff; ldp = (int)round8(g.r);
        Q = reinterpret_cast<const ET*>(a.M) + g.aoff; ldq = ldp;
        prow = g.r; kdim = g.r; qrows = g.r; qcol = 0;
    } else {
        P = reinterpret_cast<const ET*>(a.B) + g.aoff; ldp = (int)round8(g.r);
        Q = reinterpret_cast<const ET*>(a.Xc) + g.xoff; ldq = (int)round8(g.s);
        prow = g.r; kdim = g.r; qrows = g.r; qcol = g.s;
    }
    const uint32_t pbytes = (uint32_t)prow * (uint32_t)ldp * 2u;
    const uint32_t qbytes = (uint32_t)qrows * (uint32_t)ldq * 2u;
    const __amdgpu_buffer_rsrc_t rP = rsrc_of(P, pbytes);
    const __amdgpu_buffer_rsrc_t rQ = rsrc_of(Q, qbytes);

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WNW, wn = wave % WNW;
    const int l32 = lane & 31, gl = lane >> 5;

    // DMA source of instruction j of this thread (LDS chunk (wave NPI + j) 64 + lane)
    int prow_j[NPI], pcol_j[NPI], qrow_j[NPI], qcol_j[NPI];
#pragma unroll
    for (int j = 0; j < NPI; ++j) {
        const int pos = (wave * NPI + j) * 64 + lane;
        const int r = pos / CPR;
        prow_j[j] = r;
        pcol_j[j] = ((pos % CPR) ^ ((r >> SH) & (CPR - 1))) * 8;
        if (!NN) {
            qrow_j[j] = r;
            qcol_j[j] = pcol_j[j];
        } else {
            const int sub = pos / (BK * 16), pp = pos - sub * (BK * 16);
            const int rn = pp >> 4;
            qrow_j[j] = rn;
            qcol_j[j] = sub * 128 + ((pp & 15) ^ ((rn & 3) * 4)) * 8;
        }
    }
    // a diagonal block of X X^T or A A has the same row panel as both operands:
    // it is loaded once (at r = 512, 4 of the 10 lower blocks, a fifth of the
    // launch's loads from L2 into LDS)
    const bool one_panel = (MODE == 0 || MODE == 1) && bm == bn;
    auto issue = [&](int kt, ET* dP, ET* dQ) __attribute__((always_inline)) {
        const int k0 = kt * BK;
#pragma unroll
        for (int j = 0; j < NPI; ++j) {
            const int pr = m0 + prow_j[j], pk = k0 + pcol_j[j];
            const uint32_t po = (pr < prow && pk < kdim) ? slab_off(pr, pk, prow, ldp) * 2u : pbytes;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rP, (LDS_AS void*)(dP + (wave * NPI + j) * 512), 16, po, 0, 0, 0);
            uint32_t qo;
            if (!NN) {
                const int qr = n0 + qrow_j[j], qk = k0 + qcol_j[j];
                qo = (qr < qrows && qk < kdim) ? slab_off(qr, qk, qrows, ldq) * 2u : qbytes;
            } else {
                const int qr = k0 + qrow_j[j], qc = n0 + qcol_j[j];
                qo = (qr < kdim && qc < qcol) ? slab_off(qr, qc, kdim, ldq) * 2u : qbytes;
            }
            if (!one_panel)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rQ, (LDS_AS void*)(dQ + (wave * NPI + j) * 512), 16, qo, 0, 0, 0);
        }
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};

    // symmetric products: both operands are row panels
    auto compute = [&](int kt, const ET* cP, const ET* cQ) __attribute__((always_inline)) {
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            bf16x8 av[FM], bv[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int r = wm * WR + i * 32 + l32;
                const int pc = (kk * 2 + gl) ^ ((r >> SH) & (CPR - 1));
                av[i] = *reinterpret_cast<const bf16x8*>(&cP[r * BK + pc * 8]);
            }
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int r = wn * 64 + j * 32 + l32;
                const int pc = (kk * 2 + gl) ^ ((r >> SH) & (CPR - 1));
                bv[j] = *reinterpret_cast<const bf16x8*>(&cQ[r * BK + pc * 8]);
            }
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[j], acc[i][j], 0, 0, 0);
        }
    };

    // apply: the chunk's operands are read from LDS before the next chunk's
    // loads are issued.  The compiler makes a transposed LDS read wait for
    // every LDS load in flight (vmcnt 0), so reading after the issue would
    // hold the products until the next chunk had landed.
    auto read_nn = [&](const ET* cP, const ET* cQ, bf16x8 (&av)[BK / 16][FM], bf16x8 (&bv)[BK / 16][FN])
        __attribute__((always_inline)) {
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int r = wm * WR + i * 32 + l32;
                const int pc = (kk * 2 + gl) ^ ((r >> SH) & (CPR - 1));
                av[kk][i] = *reinterpret_cast<const bf16x8*>(&cP[r * BK + pc * 8]);
            }
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int G = lane >> 4, i16 = lane & 15;
                const int col = wn * 64 + j * 32 + 16 * (G & 1) + 4 * (i16 & 3);
                const int row = kk * 16 + 8 * gl + (i16 >> 2);
                const int sub = col >> 7, cl = col & 127;
                const int off = sub * (BK * 128) + row * 128 + (((cl >> 3) ^ ((row & 3) * 4)) * 8) + (cl & 7);
                bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(&cQ[off]));
                bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(&cQ[off + 4 * 128]));
                bv[kk][j] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            }
        }
    };

    // ---- pipeline: chunk kt + 1 in flight while kt is multiplied; one barrier
    //      per chunk (the barrier also tells that every wave is done with the
    //      stage the next loads overwrite) ----
    const int nk = (kdim + BK - 1) / BK;
    issue(0, sP0, sQ0);
    for (int kt = 0; kt < nk; ++kt) {
        // every load issued so far (chunk kt) has landed once vmcnt is 0
        const int cur = kt & 1;
        __builtin_amdgcn_s_waitcnt(0u | (7u << 4) | (15u << 8));
        __syncthreads();
        if constexpr (NN) {
            bf16x8 av[BK / 16][FM], bv[BK / 16][FN];
            read_nn(cur ? sP1 : sP0, cur ? sQ1 : sQ0, av, bv);
            if (kt + 1 < nk) issue(kt + 1, cur ? sP0 : sP1, cur ? sQ0 : sQ1);
#pragma unroll
            for (int kk = 0; kk < BK / 16; ++kk)
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[kk][i], bv[kk][j], acc[i][j], 0, 0, 0);
        } else {
            if (kt + 1 < nk) issue(kt + 1, cur ? sP0 : sP1, cur ? sQ0 : sQ1);
            const ET* cP = cur ? sP1 : sP0;
            compute(kt, cP, one_panel ? cP : (cur ? sQ1 : sQ0));
        }
    }

    const bool last = (MODE == 2) && (a.step == a.K - 1);

    // ---- epilogue through LDS, one pass per 128 block rows: the rows (bf16,
    //      padded stride), then whole 16-byte row chunks to the workspace; a
    //      symmetric product's mirrored part goes the same way from the
    //      transposed rows ----
    const float ca = a.abc[3 * a.step], cb = a.abc[3 * a.step + 1], cc = a.abc[3 * a.step + 2];
    auto sw = [](int row, int col) { return row * LDC + col; };
    auto swt = [](int row, int col) { return row * LDT + col; };
    // poly: A over the output block, bf16 pairs in the MFMA's register order,
    // read from the workspace once the products are done.  A is symmetric, so
    // the lane's four consecutive rows of column c are the four consecutive
    // elements of row c: one 8-byte load each.  (Taken from the row panel
    // while its k chunk was in LDS, they held 32 registers through the loop,
    // which left room for three workgroups per CU instead of four.)
    unsigned avp[FM][FN][8];
    if constexpr (MODE == 1) {
        const ET* Ag = reinterpret_cast<const ET*>(a.A) + g.aoff;
        const int ld8 = (int)round8(g.r);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const int col = n0 + wn * 64 + j * 32 + l32;
                    const int row0 = m0 + wm * WR + i * 32 + m * 8 + gl * 4;
                    u32x2 v = {0u, 0u};
                    if (col < g.r && row0 < ld8) v = *reinterpret_cast<const u32x2*>(Ag + slab_off(col, row0, g.r, ld8));
                    avp[i][j][2 * m] = v[0];
                    avp[i][j][2 * m + 1] = v[1];
                }
    }
    // X read unscaled (the first Gram and apply products after the
    // normalisation pass): X X^T takes the tile's scale twice, B' X once
    const float xs = ((MODE == 0 || MODE == 2) && a.x_raw) ? tile_scale(a, tl) : 1.0f;
    // the result rounded to bf16, two rows a register: cvp[i][j][p] holds rows
    // 2p and 2p + 1 of the lane's 16 (the MFMA's register order)
    unsigned cvp[FM][FN][8];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                float v = acc[i][j][q];
                if constexpr (MODE == 0) v = (v * xs) * xs;
                if constexpr (MODE == 2) v *= xs;
                if constexpr (MODE == 1) {
                    const float av = (q & 1) ? hi_f(avp[i][j][q >> 1]) : lo_f(avp[i][j][q >> 1]);
                    v = __builtin_fmaf(cc, v, cb * av);
                    const int row = m0 + wm * WR + i * 32 + (q >> 2) * 8 + gl * 4 + (q & 3);
                    const int col = n0 + wn * 64 + j * 32 + l32;
                    if (row == col && col < g.r) v += ca;
                }
                const unsigned u = f2bf(v);
                cvp[i][j][q >> 1] = (q & 1) ? (cvp[i][j][q >> 1] | (u << 16)) : u;
            }
    // the waves whose rows lie in pass h write them (transposed when tr)
    auto put_rows = [&](int h, bool tr) __attribute__((always_inline)) {
        if (wm * WR < h * PR || wm * WR >= (h + 1) * PR) return;
        const int rb = wm * WR - h * PR;
        if (!tr) {
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int q = 0; q < 16; ++q)
                        sbuf[sw(rb + i * 32 + (q >> 2) * 8 + gl * 4 + (q & 3), wn * 64 + j * 32 + l32)] =
                            (unsigned short)((q & 1) ? (cvp[i][j][q >> 1] >> 16) : (cvp[i][j][q >> 1] & 0xffffu));
        } else {
            // lane l holds rows rho .. rho+3 of column l%32: 4 consecutive
            // elements of one transposed row (8-byte stores)
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        const int Rt = wn * 64 + j * 32 + l32;
                        const int Ct = rb + i * 32 + m * 8 + gl * 4;
                        const u32x2 pk = {cvp[i][j][2 * m], cvp[i][j][2 * m + 1]};
                        *reinterpret_cast<u32x2*>(&sbuf[swt(Rt, Ct)]) = pk;
                    }
        }
    };

    if (MODE == 2 && last) {
        // the result goes in place into the matrix (bf16), oriented back: a
        // tall tile was stored transposed, so its transposed rows are
        // written; the Muon variant updates W <- W - eta X instead
        const MatEntry& me = a.mats[tref.mi];
        ET* base = reinterpret_cast<ET*>(a.muon ? me.w : me.m);
        const int64_t ld = a.muon ? me.w_ld : me.m_ld;
        const bool vec = vec_ok(base, ld, g.c0);
        auto put = [&](int orow, int ocol, u16x8 v) __attribute__((always_inline)) {
            if (orow >= g.h || ocol >= g.w) return;
            ET* op = base + (int64_t)(g.r0 + orow) * ld + g.c0 + ocol;
            if (vec && ocol + 8 <= g.w) {
                if (a.muon) {
                    const u16x8 w0 = *reinterpret_cast<const u16x8*>(op);
#pragma unroll
                    for (int e = 0; e < 8; ++e) v[e] = f2bf(bf2f(w0[e]) - a.eta * bf2f(v[e]));
                }
                *reinterpret_cast<u16x8*>(op) = v;
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    if (ocol + e >= g.w) break;
                    op[e] = a.muon ? f2bf(bf2f(op[e]) - a.eta * bf2f(v[e])) : v[e];
                }
            }
        };
#pragma unroll
        for (int h = 0; h < NPASS; ++h) {
            __syncthreads();   // the k stages, or the previous pass, are done with
            put_rows(h, g.tr != 0);
            __syncthreads();
            if (!g.tr) {
                // LDS row R = tile row m0 + h PR + R
#pragma unroll
                for (int it = 0; it < PR * CH / NT; ++it) {
                    const int id = it * NT + tid;
                    const int R = id / CH, ch = id % CH;
                    put(m0 + h * PR + R, n0 + ch * 8, *reinterpret_cast<const u16x8*>(&sbuf[sw(R, ch * 8)]));
                }
            } else {
                // transposed LDS row R = tile column n0 + R
#pragma unroll
                for (int it = 0; it < BE * 16 / NT; ++it) {
                    const int id = it * NT + tid;
                    const int R = id >> 4, ch = id & 15;
                    put(n0 + R, m0 + h * PR + ch * 8, *reinterpret_cast<const u16x8*>(&sbuf[swt(R, ch * 8)]));
                }
            }
        }
        return;
    }

    ET* Out;
    int64_t ldo;
    int rows_ok, cols_ok;
    if (MODE == 2) {
        Out = reinterpret_cast<ET*>(a.Xn) + g.xoff;
        ldo = round8(g.s);
        rows_ok = g.r;
        cols_ok = (int)round8(g.s);
    } else {
        Out = reinterpret_cast<ET*>(MODE == 0 ? a.A : MODE == 1 ? a.B : a.O) + g.aoff;
        ldo = round8(g.r);
        rows_ok = g.r;
        cols_ok = (int)round8(g.r);   // past r the values are zero: the padding stays zero
    }
    const bool diag = SYM && bm == bn;
#pragma unroll
    for (int h = 0; h < NPASS; ++h) {
        __syncthreads();   // the k stages, or the previous pass, are done with
        put_rows(h, false);
        __syncthreads();
        if (MODE == 3 && diag) {
            // the diagonal 128-block of this pass: the two triangles of a
            // product of two different matrices differ by rounding, so the
            // lower one is copied over the upper one and the stored result is
            // exactly symmetric (the Gram iteration amplifies any asymmetry);
            // reads are strictly below the diagonal, writes strictly above
#pragma unroll 4
            for (int it = 0; it < PR * PR / NT; ++it) {
                const int id = it * NT + tid;
                const int R = id >> 7, c = id & 127;
                if (c > R) sbuf[sw(R, h * PR + c)] = sbuf[sw(c, h * PR + R)];
            }
            __syncthreads();
        }
        // in a diagonal block, columns past this pass's diagonal 128-block are
        // strictly above the diagonal: a later pass mirrors them
        const int cmax = diag ? (h + 1) * PR : BE;
#pragma unroll
        for (int it = 0; it < PR * CH / NT; ++it) {
            const int id = it * NT + tid;
            const int R = id / CH, ch = id % CH;
            const u32x4 v = *reinterpret_cast<const u32x4*>(&sbuf[sw(R, ch * 8)]);
            if (m0 + h * PR + R < rows_ok && n0 + ch * 8 < cols_ok && ch * 8 < cmax)
                *reinterpret_cast<u32x4*>(Out + slab_off(m0 + h * PR + R, n0 + ch * 8, rows_ok, ldo)) = v;
        }
        if (!SYM) continue;
        // mirror: transposed row c of this pass goes to row n0 + c, columns
        // m0 + h PR ..; in a diagonal block only the columns left of this
        // pass's diagonal 128-block (none in the first pass)
        const int tmax = diag ? h * PR : BE;
        if (tmax == 0) continue;
        __syncthreads();
        put_rows(h, true);
        __syncthreads();
#pragma unroll
        for (int it = 0; it < BE * 16 / NT; ++it) {
            const int id = it * NT + tid;
            const int R = id >> 4, ch = id & 15;
            const u32x4 v = *reinterpret_cast<const u32x4*>(&sbuf[swt(R, ch * 8)]);
            if (R < tmax && n0 + R < rows_ok && m0 + h * PR + ch * 8 < cols_ok)
                *reinterpret_cast<u32x4*>(Out + slab_off(n0 + R, m0 + h * PR + ch * 8, rows_ok, ldo)) = v;
        }
    }
}

template <int IO, int WK, int PASS>
static hipError_t launch_norm_dt(const StepArgs& a, hipStream_t s) {
    const int n = (a.tile_end - a.tile_begin) * a.wg_norm;
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL((step_norm_kernel<IO, WK, PASS>), dim3(n), dim3(256), 0, s, a);
    return hipGetLastError();
}

template <int PASS>
static hipError_t launch_norm_pass(const StepArgs& a, hipStream_t s) {
    if (a.io_dtype == 0) return a.wk_dtype == 0 ? launch_norm_dt<0, 0, PASS>(a, s) : launch_norm_dt<0, 1, PASS>(a, s);
    return launch_norm_dt<1, 1, PASS>(a, s);
}

hipError_t launch_step_norm(const StepArgs& a, hipStream_t s) {
    if (a.K > 0) return launch_norm_pass<2>(a, s);
    hipError_t e = launch_norm_pass<0>(a, s);
    if (e != hipSuccess) return e;
    return launch_norm_pass<1>(a, s);
}

template <int MODE>
static hipError_t launch_gemm(const StepArgs& a, hipStream_t s) {
    if (a.grid_blocks <= 0) return hipSuccess;
    // the workspace layout (written by the normalisation pass) decides the kernel
    const bool dma = a.slab != 0;
    const int big_nb = MODE == 2 ? kBigNbApply : kBigNbSym;
    if (dma && a.nb_max >= big_nb) {
        // 256 x 256 blocks: the grid counts blocks of that size
        StepArgs b = a;
        const int64_t nt = a.tile_end - a.tile_begin;
        const int64_t nbm = (a.nb_max + 1) / 2, nsm = (a.ns_max + 1) / 2;
        const int64_t bpt = MODE == 2 ? nbm * nsm : nbm * (nbm + 1) / 2;
        b.grid_blocks = (int32_t)((nt * bpt + 7) / 8 * 8);
        hipLaunchKernelGGL((step_gemm_async<MODE, true>), dim3(b.grid_blocks), dim3(512), 0, s, b);
    } else if (dma)
        hipLaunchKernelGGL((step_gemm_async<MODE, false>), dim3(a.grid_blocks), dim3(256), 0, s, a);
    else if (a.wk_dtype == 0)
        hipLaunchKernelGGL((step_gemm_kernel<0, MODE>), dim3(a.grid_blocks), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((step_gemm_kernel<1, MODE>), dim3(a.grid_blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

bool step_slab_layout(const StepArgs& a) {
    // the direct-to-LDS kernel addresses an operand with 32-bit byte offsets
    const int64_t rmax = 128LL * a.nb_max, smax = 128LL * a.ns_max;
    return a.wk_dtype == 0 && rmax * std::max(rmax, smax) * 2 < (1LL << 31);
}

hipError_t launch_step_gram(const StepArgs& a, hipStream_t s) { return launch_gemm<0>(a, s); }
hipError_t launch_step_poly(const StepArgs& a, hipStream_t s) { return launch_gemm<1>(a, s); }
hipError_t launch_step_apply(const StepArgs& a, hipStream_t s) { return launch_gemm<2>(a, s); }
hipError_t launch_step_product(const StepArgs& a, hipStream_t s) { return launch_gemm<3>(a, s); }

}  // namespace himuon
