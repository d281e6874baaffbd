// On-chip tiled Newton-Schulz for bf16 tiles whose larger side is 129..256,
// on gfx950.
//
// One workgroup of eight waves owns one tile (zero padded to 256 x 256) for
// all K steps; a CU holds one tile.  The map is the per-tile Newton-Schulz
// iteration of the HiMuon abstract, written as in the Gram Newton-Schulz page
// (Algorithm 1): A = X X^T, B = b A + c A^2, X <- a X + B X.  Padding is exact:
// the padded Gram matrix is block diagonal, so padded rows and columns stay 0.
//
// The LDS (160 KB) holds one 256 x 256 bf16 matrix at a time (140 KB with
// row padding), in turn X, A and B' = a I + b A + c A^2:
//   1. A = X X^T: the 36 lower 32x32 blocks, four or five per wave, from
//      16-byte row fragments of X.  Each wave also copies its column block of
//      X (32 columns) into registers, as the MFMA operand of step 3.
//   2. A is written over X: each lower block transposed as the upper block,
//      then read back from there with transposing reads and written as the
//      lower block, so the stored A is exactly symmetric.
//   3. A^2 = A A^T (A symmetric), same blocks and reads as 1; the epilogue
//      forms B' from the same rounded A, and B' is written over A.
//   4. X'^T(w, I) = sum_K X(K, w)^T B'(K, I): a operand = the wave's column
//      block of X (registers), b operand = row fragments of B' (B' symmetric,
//      so column I of B'(K, I) is row I of B'(I, K)).  The result lands in the
//      row layout of X'(I, w) and is written with 8-byte stores over B'.
// Waves w and w + 4 share a SIMD; the block lists give each SIMD nine of the
// 36 lower blocks.
//
// Narrow tiles (the shorter side 32..128, the longer 129..256) run the same
// code with NR = 4 row blocks: the tile is oriented so that X has r <= 128
// rows (a tall tile is transposed on the way into LDS and back on the way out),
// A and B' are 128 x 128 (10 lower blocks) and X' is r x s; this does about a
// quarter of the padded 256 x 256 work.
//
// Register layouts as in the kernel-tile-128 kernel: AL (accumulator layout)
// lane l, register q holds M[rho(l,q)][l % 32], rho = (q/4)*8 + (l/32)*4 + q%4;
// RL = AL of the transpose.

#include "device_util.h"

namespace himuon {

namespace {

// LDS row stride: 280 elements (560 bytes).  Measured against 264 (1-2 % slower
// on every T = 256 workload), 272 (5 % slower), 296 and 312 (level).
constexpr int kT = 256, kLD = kT + 24;

// Lower 32x32 blocks (i, j), i >= j, of a symmetric product with NR x NR
// blocks, per wave (at most five).
template <int NR> struct Blocks;
template <> struct Blocks<8> {
    static constexpr int n[8] = {4, 4, 4, 4, 5, 5, 5, 5};
    static constexpr int i[8][5] = {{2, 2, 3, 3, 0}, {4, 4, 5, 5, 0}, {6, 6, 7, 7, 0}, {4, 4, 5, 5, 0},
                                    {6, 6, 7, 7, 0}, {6, 6, 7, 7, 1}, {1, 2, 3, 3, 4}, {5, 5, 6, 7, 7}};
    static constexpr int j[8][5] = {{0, 1, 0, 1, 0}, {0, 1, 0, 1, 0}, {0, 1, 0, 1, 0}, {2, 3, 2, 3, 0},
                                    {2, 3, 2, 3, 0}, {4, 5, 4, 5, 1}, {0, 2, 2, 3, 4}, {4, 5, 6, 6, 7}};
};
template <> struct Blocks<4> {
    static constexpr int n[8] = {2, 2, 2, 2, 1, 1, 0, 0};
    static constexpr int i[8][5] = {{1, 0}, {2, 1}, {3, 2}, {2, 3}, {3}, {3}, {}, {}};
    static constexpr int j[8][5] = {{0, 0}, {0, 1}, {0, 2}, {1, 3}, {1}, {2}, {}, {}};
};

template <int NR>
constexpr bool uses_row(int w, int r) {
    for (int b = 0; b < Blocks<NR>::n[w]; ++b)
        if (Blocks<NR>::i[w][b] == r || Blocks<NR>::j[w][b] == r) return true;
    return false;
}

template <int N> struct IC { static constexpr int value = N; };
// Runs f(IC<w>) for the wave index w (uniform, in a scalar register).
template <class F>
__device__ __forceinline__ void per_wave(int w, F&& f) {
    switch (w) {
        case 0: f(IC<0>{}); break;
        case 1: f(IC<1>{}); break;
        case 2: f(IC<2>{}); break;
        case 3: f(IC<3>{}); break;
        case 4: f(IC<4>{}); break;
        case 5: f(IC<5>{}); break;
        case 6: f(IC<6>{}); break;
        default: f(IC<7>{}); break;
    }
}

// LDS pointers with the lane-dependent part of each access pattern folded in,
// so that every access below is one of these plus a constant.
struct LdsLanes {
    const unsigned short* rf;   // row fragments:   (l%32) row, 8 (l/32) column
    const unsigned short* cf;   // column fragments (transposing reads)
    unsigned short* rl;         // row-layout runs:  (l%32) row, 4 (l/32) column
};

// 16-byte row fragment: row R*32 + l%32, columns k0 + 8 (l/32) .. +7.
__device__ __forceinline__ u32x4 row_frag(const LdsLanes& L, int R, int k0) {
    return *reinterpret_cast<const u32x4*>(&L.rf[R * 32 * kLD + k0]);
}

// Column fragment in natural k order: lane l gets rows k0 + 8 (l/32) .. +7 of
// column c0 + l%32 (two transposing 8-byte reads).
__device__ __forceinline__ u32x4 col_frag(const LdsLanes& L, int k0, int c0) {
    bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(&L.cf[k0 * kLD + c0]));
    bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(&L.cf[(k0 + 4) * kLD + c0]));
    return __builtin_bit_cast(u32x4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Lower blocks of M M^T (M the LDS matrix, KC k chunks of 16) for wave W,
// accumulated in AL.
template <int NR, int KC, int W>
__device__ __forceinline__ void gram_lower(const LdsLanes& L, f32x16 (&acc)[5]) {
    using B = Blocks<NR>;
#pragma unroll
    for (int b = 0; b < 5; ++b) acc[b] = f32x16{};
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
        u32x4 rf[NR];
#pragma unroll
        for (int r = 0; r < NR; ++r)
            if (uses_row<NR>(W, r)) rf[r] = row_frag(L, r, kc * 16);
#pragma unroll
        for (int b = 0; b < B::n[W]; ++b) acc[b] = mfma32w(rf[B::i[W][b]], rf[B::j[W][b]], acc[b]);
    }
}

// Writes the wave's lower blocks (bf16 AL in p) into the LDS matrix as a full
// symmetric matrix.  Block (j, i) takes the transpose, written from the AL
// registers as row-layout runs (8-byte stores).  For i != j, block (i, j) is
// then read back from (j, i) column by column with transposing reads (a column
// of the stored transpose is a row of the block) and written as 16-byte row
// fragments.  The same bits land as with one 2-byte store per element, in a
// quarter of the LDS instructions.
template <int NR, int W>
__device__ __forceinline__ void store_sym(const LdsLanes& L, const u32x4 (&p)[5][2]) {
    using B = Blocks<NR>;
    unsigned short* wf = const_cast<unsigned short*>(L.rf);   // row-fragment positions, for writing
#pragma unroll
    for (int b = 0; b < B::n[W]; ++b) {
        const int i = B::i[W][b], j = B::j[W][b];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            u32x2 v = {p[b][m >> 1][2 * (m & 1)], p[b][m >> 1][2 * (m & 1) + 1]};
            *reinterpret_cast<u32x2*>(&L.rl[j * 32 * kLD + i * 32 + 8 * m]) = v;
        }
    }
#pragma unroll
    for (int b = 0; b < B::n[W]; ++b) {
        const int i = B::i[W][b], j = B::j[W][b];
        if (i != j) {
            // lane l: row i*32 + l%32 of the block, columns 8 (l/32) .. +7 and
            // 16 + 8 (l/32) .. +7, from column i*32 + l%32 of block (j, i)
            const u32x4 r0 = col_frag(L, j * 32, i * 32);
            const u32x4 r1 = col_frag(L, j * 32 + 16, i * 32);
            *reinterpret_cast<u32x4*>(&wf[i * 32 * kLD + j * 32]) = r0;
            *reinterpret_cast<u32x4*>(&wf[i * 32 * kLD + j * 32 + 16]) = r1;
        }
    }
}

// B' = c A^2 + b A (+ a on the diagonal), in place of the rounded A in p.
template <int NR, int W>
__device__ __forceinline__ void combine(f32x16 (&acc)[5], u32x4 (&p)[5][2], float ca, float cb, float cc,
                                        int l32, int g) {
    using B = Blocks<NR>;
#pragma unroll
    for (int b = 0; b < B::n[W]; ++b) {
        const bool dg = B::i[W][b] == B::j[W][b];
#pragma unroll
        for (int f = 0; f < 2; ++f)
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int e = 8 * f + 2 * k;
                const float l0 = lo_f(p[b][f][k]), l1 = hi_f(p[b][f][k]);
                // linear term b A, with a on the diagonal of a diagonal block
                acc[b][e] = __builtin_fmaf(cc, acc[b][e], dg ? __builtin_fmaf(cb, l0, diag_term(e, l32, g, ca)) : cb * l0);
                acc[b][e + 1] =
                    __builtin_fmaf(cc, acc[b][e + 1], dg ? __builtin_fmaf(cb, l1, diag_term(e + 1, l32, g, ca)) : cb * l1);
            }
        p[b][0] = cvt8(acc[b], 0);
        p[b][1] = cvt8(acc[b], 8);
    }
}

}  // namespace

template <bool MUON, int NR>
__global__ __launch_bounds__(512) void resident256_kernel(const ResidentArgs args) {
    constexpr int XR = NR * 32;                     // rows of X in LDS
    __shared__ __attribute__((aligned(16))) unsigned short sX[XR * kLD];
    __shared__ float red[8];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, g = lane >> 5;

    const int t = args.tile_begin + blockIdx.x;
    const MatEntry& me = args.mats[find_class(args.mats, args.nmats, t)];
    const TileGeom tg = class_tile(me, args.T, t - me.tile_base);
    const int h = tg.h, wd = tg.w;
    // X is the tile itself, or (a tall narrow tile) its transpose
    const bool tr = NR == 4 && h > wd;
    unsigned short* mbase = reinterpret_cast<unsigned short*>(me.m) + (int64_t)tg.r0 * me.m_ld + tg.c0;
    const bool mvec = vec_ok(me.m, me.m_ld, tg.c0);
    using IO = TileIO<kT>;
    // 16-byte chunks of the tile per thread: XR rows of 32 chunks, or (tall)
    // 256 rows of 16
    constexpr int NCH = XR * 32 / 512;
    const int cpr = tr ? 16 : 32;

    // ---- load (Muon: M <- mu M + G, stored), sum of squares, scaled tile
    //      into LDS.  Every load of the thread is issued before the first one
    //      is waited for, and the tile stays in registers until the scale is
    //      known, so it is written to LDS once. ----
    {
        const unsigned short* gbase = nullptr;
        bool gvec = false;
        if constexpr (MUON) {
            gbase = reinterpret_cast<const unsigned short*>(me.g) + (int64_t)tg.r0 * me.g_ld + tg.c0;
            gvec = vec_ok(me.g, me.g_ld, tg.c0);
        }
        u16x8 chunk[NCH];
        // a whole tile in its own layout: XR rows of 256 (wide or square) or
        // 256 rows of XR = 128 (tall)
        if (MUON && (tr ? (h == kT && wd == XR) : (h == XR && wd == kT)) && mvec && gvec) {
            const int rpi = 512 / cpr;   // rows per chunk round
            muon_prologue_whole<NCH, 8>(mbase + (int64_t)(tid / cpr) * me.m_ld + (tid % cpr) * 8,
                                        (int64_t)rpi * me.m_ld,
                                        gbase + (int64_t)(tid / cpr) * me.g_ld + (tid % cpr) * 8,
                                        (int64_t)rpi * me.g_ld, args.mu, chunk);
        } else {
#pragma unroll
            for (int it = 0; it < NCH; ++it) {
                const int idx = it * 512 + tid;
                const int r = idx / cpr, col = (idx % cpr) * 8;
                u16x8 v = IO::load(mbase, me.m_ld, r, col, h, wd, mvec);
                if constexpr (MUON) {
                    u16x8 gv = IO::load(gbase, me.g_ld, r, col, h, wd, gvec);
#pragma unroll
                    for (int e = 0; e < 8; ++e) v[e] = f2bf(args.mu * bf2f(v[e]) + bf2f(gv[e]));
                    IO::store(mbase, me.m_ld, r, col, h, wd, mvec, v);
                }
                chunk[it] = v;
            }
        }
        float ss = 0.f;
#pragma unroll
        for (int it = 0; it < NCH; ++it)
#pragma unroll
            for (int e = 0; e < 8; ++e) { const float x = bf2f(chunk[it][e]); ss = __builtin_fmaf(x, x, ss); }
        ss = wave_sum(ss);
        if (lane == 0) red[w] = ss;
        __syncthreads();
        float tot = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) tot += red[i];
        const float scale = args.normalize ? 1.0f / (sqrtf(tot) + args.eps) : 1.0f;
#pragma unroll
        for (int it = 0; it < NCH; ++it) {
            const int idx = it * 512 + tid;
            const int r = idx / cpr, col = (idx % cpr) * 8;
            u16x8 v;
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = f2bf(bf2f(chunk[it][e]) * scale);
            if (!tr) {
                *reinterpret_cast<u16x8*>(&sX[r * kLD + col]) = v;
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) sX[(col + e) * kLD + r] = v[e];
            }
        }
        __syncthreads();
    }

    for (int step = 0; step < args.K; ++step) {
        const float ca = args.abc[3 * step], cb = args.abc[3 * step + 1], cc = args.abc[3 * step + 2];
        // The lane parts of the LDS addresses pass through an empty asm every
        // step; otherwise the compiler hoists the few hundred distinct LDS
        // addresses of a step out of the loop and spills them.
        int o_rf = l32 * kLD + g * 8;
        int o_cf = (8 * g + ((lane & 15) >> 2)) * kLD + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
        int o_rl = l32 * kLD + 4 * g;
        asm volatile("" : "+v"(o_rf), "+v"(o_cf), "+v"(o_rl));
        const LdsLanes L{sX + o_rf, sX + o_cf, sX + o_rl};
        f32x16 acc[5];
        u32x4 p[5][2];
        // 1. lower blocks of A = X X^T (k over the 256 columns); this wave's
        //    column block of X
        per_wave(w, [&](auto W) { gram_lower<NR, kT / 16, decltype(W)::value>(L, acc); });
        u32x4 xf[NR][2];
#pragma unroll
        for (int K = 0; K < NR; ++K)
#pragma unroll
            for (int kc = 0; kc < 2; ++kc) xf[K][kc] = col_frag(L, K * 32 + kc * 16, w * 32);
#pragma unroll
        for (int b = 0; b < 5; ++b) {
            p[b][0] = cvt8(acc[b], 0);
            p[b][1] = cvt8(acc[b], 8);
        }
        __syncthreads();
        // 2. A over X
        per_wave(w, [&](auto W) { store_sym<NR, decltype(W)::value>(L, p); });
        __syncthreads();
        // 3. A^2 = A A^T (k over the XR columns of A), B' = a I + b A + c A^2,
        //    B' over A
        per_wave(w, [&](auto W) {
            gram_lower<NR, XR / 16, decltype(W)::value>(L, acc);
            combine<NR, decltype(W)::value>(acc, p, ca, cb, cc, l32, g);
        });
        __syncthreads();
        per_wave(w, [&](auto W) { store_sym<NR, decltype(W)::value>(L, p); });
        __syncthreads();
        // 4. X'^T(w, I) = sum_K X(K, w)^T B'(K, I), two row blocks I at a time
        u32x4 xo[NR][2];
#pragma unroll
        for (int I = 0; I < NR; I += 2) {
            f32x16 c0 = {}, c1 = {};
#pragma unroll
            for (int K = 0; K < NR; ++K)
#pragma unroll
                for (int kc = 0; kc < 2; ++kc) {
                    const int k0 = K * 32 + kc * 16;
                    c0 = mfma32w(xf[K][kc], row_frag(L, I, k0), c0);
                    c1 = mfma32w(xf[K][kc], row_frag(L, I + 1, k0), c1);
                }
            xo[I][0] = cvt8(c0, 0);
            xo[I][1] = cvt8(c0, 8);
            xo[I + 1][0] = cvt8(c1, 0);
            xo[I + 1][1] = cvt8(c1, 8);
        }
        __syncthreads();
        // X' over B': RL(X'(I, w)) -> row I*32 + l%32, columns w*32 + rho
#pragma unroll
        for (int I = 0; I < NR; ++I)
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                u32x2 v = {xo[I][m >> 1][2 * (m & 1)], xo[I][m >> 1][2 * (m & 1) + 1]};
                *reinterpret_cast<u32x2*>(&L.rl[I * 32 * kLD + w * 32 + 8 * m]) = v;
            }
        __syncthreads();
    }

    // ---- write back in place (Muon: W <- W - eta X), transposed back for a
    //      tall tile ----
    unsigned short* obase = mbase;
    int64_t old = me.m_ld;
    bool ovec = mvec;
    if constexpr (MUON) {
        obase = reinterpret_cast<unsigned short*>(me.w) + (int64_t)tg.r0 * me.w_ld + tg.c0;
        old = me.w_ld;
        ovec = vec_ok(me.w, me.w_ld, tg.c0);
    }
    if (MUON && (tr ? (h == kT && wd == XR) : (h == XR && wd == kT)) && ovec) {
        // the result's chunks from LDS, then W updated in batches
        u16x8 x[NCH];
#pragma unroll
        for (int it = 0; it < NCH; ++it) {
            const int idx = it * 512 + tid;
            const int r = idx / cpr, col = (idx % cpr) * 8;
            if (!tr) {
                x[it] = *reinterpret_cast<const u16x8*>(&sX[r * kLD + col]);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) x[it][e] = sX[(col + e) * kLD + r];
            }
        }
        const int rpi = 512 / cpr;
        muon_update_whole<NCH, 8>(obase + (int64_t)(tid / cpr) * old + (tid % cpr) * 8, (int64_t)rpi * old, args.eta, x);
        return;
    }
#pragma unroll
    for (int it = 0; it < NCH; ++it) {
        const int idx = it * 512 + tid;
        const int r = idx / cpr, col = (idx % cpr) * 8;
        u16x8 v;
        if (!tr) {
            v = *reinterpret_cast<const u16x8*>(&sX[r * kLD + col]);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = sX[(col + e) * kLD + r];
        }
        if constexpr (MUON) {
            u16x8 wv = IO::load(obase, old, r, col, h, wd, ovec);
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = f2bf(bf2f(wv[e]) - args.eta * bf2f(v[e]));
        }
        IO::store(obase, old, r, col, h, wd, ovec, v);
    }
}

hipError_t launch_resident256(const ResidentArgs& a, bool muon, bool narrow, hipStream_t s) {
    const int n = a.tile_end - a.tile_begin;
    if (n <= 0) return hipSuccess;
    if (narrow) {
        if (muon)
            hipLaunchKernelGGL((resident256_kernel<true, 4>), dim3(n), dim3(512), 0, s, a);
        else
            hipLaunchKernelGGL((resident256_kernel<false, 4>), dim3(n), dim3(512), 0, s, a);
    } else {
        if (muon)
            hipLaunchKernelGGL((resident256_kernel<true, 8>), dim3(n), dim3(512), 0, s, a);
        else
            hipLaunchKernelGGL((resident256_kernel<false, 8>), dim3(n), dim3(512), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace himuon
