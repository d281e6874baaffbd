// On-chip tiled Newton-Schulz for bf16 tiles of up to 32 x 32 on gfx950.
//
// One wavefront owns one tile for all K steps (HiMuon abstract: the same
// finite Newton-Schulz map on every tile independently; Gram Newton-Schulz
// page, Algorithm 1, for the map) and walks tiles with a grid stride.  A
// 32-tile is one 32 x 32 MFMA block, so a step is a handful of
// v_mfma_f32_32x32x16_bf16 and the kernel's cost is the vector work around
// them; it is laid out to keep that work small.
//
// Scaled iterate.  The wave carries Y = g X.  One step with A = X X^T is
// X' = (a I + b A + c A^2) X; with A_Y = Y Y^T = g^2 A it reads
//     Y' = r (a I + (b / g^2) A_Y + (c / g^4) A_Y^2) Y,    r = g' / g,
// and the last step has g' = 1, so that it writes X itself.  The host
// computes the constants in double precision (Consts32).
//  * Square form (every step the same (a, b, c) with c > 0): g = c^(1/4) on
//    every step, so the quadratic coefficient is 1 and, with beta = b / g^2,
//        a I + beta A_Y + A_Y^2 = (A_Y + mu I)^2 + d I,
//        mu = beta / 2,  d = a - beta^2 / 4.
//    Both identity terms enter as the starting value of an MFMA accumulator
//    (a constant diagonal), so a bf16 step does no arithmetic of its own
//    besides the three roundings to bf16.  Every step keeps g; the final
//    factor 1 / g is applied with the last rounding.
//  * General form (any coefficients): g = sqrt(|b|) (1 when b = 0); the
//    linear coefficient is then exactly -1 or +1 within a run of equal b
//    (a sign modifier on the fma).  Its fp32 steps scale the Gram matrix
//    by kap before rounding it, kap^2 = r |c| / g^4, so that the quadratic
//    coefficient is +-1 there too.
//
// Precision.  The first n_master steps keep Y in fp32 registers and take
// the step in nested form, Y' = r a Y + Ab Z with Z = bf16(cb Y + Ab Y) and
// Ab = bf16(A_Y) (the square form's cb is beta): every bf16 rounding but
// that of the Gram matrix lands in a factor that Ab multiplies from the
// left, which scales it down by the small singular values in their
// directions, and the step is an exact polynomial of the one rounded Ab.
// It takes six MFMAs and no unpacking of bf16 values.  The later steps keep
// Y in bf16 with the identity folded into the product.  Rounding noise that
// a bf16 step puts into directions of small singular values is multiplied by
// roughly a_t by every later step, so the host makes the bf16 steps only a
// final run whose product of |a_t| stays at most 41 (three quintic steps).
// CPU emulation of these roundings over 200k random 32-tiles, five quintic
// steps: worst 1.41e-2 (n_master 2), against 1.52e-2 for the earlier fp32
// step B = beta Ab + Ab^2 split into a bf16 hi/lo pair.
//
// Layouts (one 32 x 32 block per wave, v_mfma_f32_32x32x16_bf16):
//   accumulator layout AL: lane l, register q holds M[rho(l,q)][l % 32],
//     rho(l,q) = (q/4)*8 + (l/32)*4 + q%4;
//   row layout RL = AL of the transpose.  Registers 8f..8f+7 are one MFMA
//   operand with a permuted k order, the same on both operands.
// A_Y = Y Y^T takes RL(Y) as both operands; A_Y^2 takes AL(A_Y) (A_Y
// symmetric) for both; Y'^T = Y^T B takes AL(Y), read from LDS with
// ds_read_tr16_b64, and AL(B), and lands in RL(Y').
//
// Measured on MI355X (24 transformer layers, 1.2 M tiles, K = 5): 1.65 ms per
// call.  Steps: 2.46 ms with every step in fp32 and one workgroup per tile;
// 2.00 ms with the hi/lo fp32 step, the tile pairing below (HBM reads
// halved) and four waves per SIMD; 1.72 ms with the nested fp32 step and the
// two step loops; 1.66 ms with five waves per SIMD (at most 96 registers);
// 1.65 ms with the sum of squares taken from the unpacked row fragments.
// Six waves would spill.  Loading the next tile during the current one was
// slower both into registers (5-8 %) and straight into LDS with
// global_load_lds (7 %).  LDS row strides of 48 and 56 elements were 1-2 %
// slower than 40.
//
// Workgroups go round-robin to the eight XCDs.  A 32-tile row is 64 bytes,
// half a cache line, so horizontally adjacent tiles are given to workgroups
// on the same XCD at about the same time (w and w + 8 of each group of 16),
// and the line is fetched from HBM once.

#include <atomic>
#include <cmath>
#include <type_traits>

#include "device_util.h"

namespace himuon {

namespace {

constexpr int kLD32 = 40;   // LDS row stride (elements): 80 bytes

// Sum over the 64 lanes: butterflies inside each row of 16 lanes with DPP
// (quad permutations, then rotations by 4 and 8), then the four row sums.
__device__ __forceinline__ float wave_sum_dpp(float v) {
    auto mv = [](float x, auto ctrl) {
        return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), decltype(ctrl)::value,
                                                                   0xf, 0xf, false));
    };
    v += mv(v, std::integral_constant<int, 0xb1>{});    // quad_perm [1, 0, 3, 2]
    v += mv(v, std::integral_constant<int, 0x4e>{});    // quad_perm [2, 3, 0, 1]
    v += mv(v, std::integral_constant<int, 0x124>{});   // row_ror:4
    v += mv(v, std::integral_constant<int, 0x128>{});   // row_ror:8
    const int b = __builtin_bit_cast(int, v);
    return (__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0)) +
            __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16))) +
           (__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32)) +
            __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48)));
}

template <bool MUON, bool SQUARE>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(MUON ? 4 : 5))) void resident32_kernel(
    const ResidentArgs args, const Consts32 cs) {
    __shared__ __attribute__((aligned(16))) unsigned short sX[32 * kLD32];
    __shared__ __attribute__((aligned(16))) unsigned short sZ[32 * kLD32];

    const int lane = threadIdx.x;
    const int l32 = lane & 31, g = lane >> 5;
    using IO = TileIO<32>;   // two 16-byte chunks per lane: rows lane / 4 and 16 + lane / 4
    const int crow = lane >> 2, ccol = (lane & 3) * 8;

    // RL run m (= q / 4) of a lane: row l32, columns 8m + 4g .. + 3
    auto rl_off = [&](int m) { return l32 * kLD32 + 8 * m + 4 * g; };
    auto put_rl = [&](unsigned short* buf, const u32x4 (&fr)[2]) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            u32x2 v = {fr[m >> 1][2 * (m & 1)], fr[m >> 1][2 * (m & 1) + 1]};
            *reinterpret_cast<u32x2*>(&buf[rl_off(m)]) = v;
        }
    };
    // AL operand f of the stored (row-major) matrix: two transposed 8-byte reads
    auto tr_frag = [&](const unsigned short* buf, int f) {
        const int G = lane >> 4, i16 = lane & 15;
        const int col = 16 * (G & 1) + 4 * (i16 & 3);
        const int rowb = 16 * f + 4 * g + (i16 >> 2);
        bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(&buf[rowb * kLD32 + col]));
        bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(&buf[(rowb + 8) * kLD32 + col]));
        return __builtin_bit_cast(u32x4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    // constant diagonals of the square form
    f32x16 CiMu = {}, CiD = {};
    if constexpr (SQUARE) {
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            CiMu[q] = diag_term(q, l32, g, cs.mu);
            CiD[q] = diag_term(q, l32, g, cs.d);
        }
    }
    // general form: identity term of the bf16 steps (rebuilt when it changes)
    f32x16 Ci = {};
    float d_cur = 0.f;
    auto set_diag = [&](float d) {
        if (d != d_cur) {
#pragma unroll
            for (int q = 0; q < 16; ++q) Ci[q] = diag_term(q, l32, g, d);
            d_cur = d;
        }
    };

    const int n = args.tile_end - args.tile_begin;
    const int K = args.K;
    const int p = blockIdx.x;
    // tile of this workgroup in the round starting at base: adjacent tiles to
    // workgroups w and w + 8 of a full group of 16
    auto tile_at = [&](int base) {
        const int o = base + (p | 15) < n ? ((p & ~15) | ((p & 7) << 1) | ((p >> 3) & 1)) : p;
        return args.tile_begin + base + o;
    };
    // class of the previous tile and its tile range: consecutive tiles of a
    // wave mostly fall in the same class, which then needs no search
    int cls = 0, cls_lo = 1, cls_hi = 0;
    for (int base = 0; base < n; base += gridDim.x) {
        if (base + p >= n) break;
        const int t = tile_at(base);
        if (t < cls_lo || t >= cls_hi) {
            cls = find_class(args.mats, args.nmats, t);
            cls_lo = args.mats[cls].tile_base;
            cls_hi = cls + 1 < args.nmats ? args.mats[cls + 1].tile_base : 0x7fffffff;
        }

        const MatEntry& me = args.mats[cls];
        const TileGeom tg = class_tile(me, args.T, t - me.tile_base);
        const int h = tg.h, wd = tg.w;
        unsigned short* mbase = reinterpret_cast<unsigned short*>(me.m) + (int64_t)tg.r0 * me.m_ld + tg.c0;
        const bool mvec = vec_ok(me.m, me.m_ld, tg.c0);
        const bool full = h == 32 && wd == 32 && mvec;

        // ---- load (Muon: M <- mu M + G, stored), sum of squares ----
        u16x8 chunk[IO::NCH];
        if (full && !MUON) {
            const unsigned short* p0 = mbase + (int64_t)crow * me.m_ld + ccol;
            chunk[0] = *reinterpret_cast<const u16x8*>(p0);
            chunk[1] = *reinterpret_cast<const u16x8*>(p0 + 16 * me.m_ld);
        } else if (MUON && full && vec_ok(me.g, me.g_ld, tg.c0)) {
            const unsigned short* g0 = reinterpret_cast<const unsigned short*>(me.g) + (int64_t)tg.r0 * me.g_ld + tg.c0;
            muon_prologue_whole<IO::NCH, IO::NCH>(mbase + (int64_t)crow * me.m_ld + ccol, 16 * me.m_ld,
                                                  g0 + (int64_t)crow * me.g_ld + ccol, 16 * me.g_ld, args.mu, chunk);
        } else {
            const unsigned short* gbase = nullptr;
            bool gvec = false;
            if constexpr (MUON) {
                gbase = reinterpret_cast<const unsigned short*>(me.g) + (int64_t)tg.r0 * me.g_ld + tg.c0;
                gvec = vec_ok(me.g, me.g_ld, tg.c0);
            }
#pragma unroll
            for (int it = 0; it < IO::NCH; ++it) {
                const int r = crow + 16 * it;
                u16x8 v = IO::load(mbase, me.m_ld, r, ccol, h, wd, mvec);
                if constexpr (MUON) {
                    u16x8 gv = IO::load(gbase, me.g_ld, r, ccol, h, wd, gvec);
#pragma unroll
                    for (int e = 0; e < 8; ++e) v[e] = f2bf(args.mu * bf2f(v[e]) + bf2f(gv[e]));
                    IO::store(mbase, me.m_ld, r, ccol, h, wd, mvec, v);
                }
                chunk[it] = v;
            }
        }
#pragma unroll
        for (int it = 0; it < IO::NCH; ++it)
            *reinterpret_cast<u16x8*>(&sX[(crow + 16 * it) * kLD32 + ccol]) = chunk[it];
        __syncthreads();
        // Ym: the iterate in fp32 (RL), read back once; the sum of squares is
        // taken from the same values (the lanes' row fragments cover the tile
        // once), so the bf16 values are unpacked only here
        f32x16 Ym;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const u16x4 v = *reinterpret_cast<const u16x4*>(&sX[rl_off(m)]);
#pragma unroll
            for (int e = 0; e < 4; ++e) Ym[4 * m + e] = bf2f(v[e]);
        }
        float ss = 0.f;
#pragma unroll
        for (int q = 0; q < 16; ++q) ss = __builtin_fmaf(Ym[q], Ym[q], ss);
        ss = wave_sum_dpp(ss);
        // v_sqrt_f32 and v_rcp_f32 (1 ulp each): the scale is a per-tile
        // constant whose relative error of a few 1e-7 is far below the bf16
        // rounding
        const float scale =
            (args.normalize ? __builtin_amdgcn_rcpf(__builtin_amdgcn_sqrtf(ss) + args.eps) : 1.0f) * cs.g0;
        Ym = Ym * scale;
        u32x4 XR[2];
        __syncthreads();
        // fp32 step (k < n_master): with Ab = bf16(kappa A_Y) and s = +-1,
        //     Y' = ca Y + Ab Z,   Z = bf16(cb Y + s Ab Y),
        // the iterate accumulated in fp32.  Both products put their bf16
        // rounding into a factor that Ab multiplies from the left, so in the
        // directions of small singular values it arrives scaled by them; the
        // map is an exact polynomial of the one rounded Gram matrix.  lin:
        // c = 0, Y' = ca Y + Ab Y.
        auto m_step = [&](float ca, float cb, float kap, bool lin, bool neg) __attribute__((always_inline)) {
            XR[0] = cvt8(Ym, 0);
            XR[1] = cvt8(Ym, 8);
            put_rl(sX, XR);
            f32x16 a = mfma32w(XR[0], XR[0], f32x16{});
            a = mfma32w(XR[1], XR[1], a);
            if (kap != 1.0f) a = a * kap;
            const u32x4 Ab[2] = {cvt8(a, 0), cvt8(a, 8)};
            __syncthreads();
            u32x4 op0 = tr_frag(sX, 0), op1 = tr_frag(sX, 1);
            if (!lin) {
                // Z^T = cb Y^T + Yb^T Ab lands in the row layout
                f32x16 z = Ym * cb;
                z = mfma32w(op0, Ab[0], z);
                z = mfma32w(op1, Ab[1], z);
                u32x4 ZR[2] = {cvt8(z, 0), cvt8(z, 8)};
                if (neg) {
                    // c < 0: Y' = ca Y - Ab (-cb Y + Ab Y), the sign on Z
                    ZR[0] ^= 0x80008000u;
                    ZR[1] ^= 0x80008000u;
                }
                put_rl(sZ, ZR);
                __syncthreads();
                op0 = tr_frag(sZ, 0);
                op1 = tr_frag(sZ, 1);
            }
            f32x16 y = Ym * ca;
            y = mfma32w(op0, Ab[0], y);
            y = mfma32w(op1, Ab[1], y);
            Ym = y;
            __syncthreads();
        };
        // bf16 step (k >= n_master): B' from the packed A by form_b,
        // Y' = B' Y rounded to bf16 in XR
        auto f_step = [&](auto make_b) __attribute__((always_inline)) {
            put_rl(sX, XR);
            u32x4 Bb[2];
            make_b(Bb);
            __syncthreads();
            const u32x4 op0 = tr_frag(sX, 0), op1 = tr_frag(sX, 1);
            f32x16 y = mfma32w(op0, Bb[0], f32x16{});
            y = mfma32w(op1, Bb[1], y);
            XR[0] = cvt8(y, 0);
            XR[1] = cvt8(y, 8);
            Ym = y;
            __syncthreads();
        };
        // A^2 from the packed A
        auto square_of = [](const u32x4 (&Ab)[2], const f32x16& c0) __attribute__((always_inline)) {
            f32x16 acc = mfma32w(Ab[0], Ab[0], c0);
            return mfma32w(Ab[1], Ab[1], acc);
        };

        // The fp32 steps, then the bf16 steps, as two loops: one loop with
        // both kinds of step made the compiler copy the iterate between
        // registers on every step.
        const int km = K < cs.n_master ? K : cs.n_master;
        if constexpr (SQUARE) {
            // ---- square form: constant coefficients, c > 0 ----
            // (the factor 1 / g that brings the last iterate back to X is
            // applied with the final rounding, below)
            for (int k = 0; k < km; ++k) m_step(cs.ra, cs.beta, 1.0f, false, false);
            if (km < K) {
                XR[0] = cvt8(Ym, 0);
                XR[1] = cvt8(Ym, 8);
            }
            for (int k = km; k < K; ++k) {
                {
                    // (A_Y + mu I)^2 + d I: both diagonals start the accumulators
                    f_step([&](u32x4 (&Bb)[2]) __attribute__((always_inline)) {
                        f32x16 z = mfma32w(XR[0], XR[0], CiMu);
                        z = mfma32w(XR[1], XR[1], z);
                        const u32x4 Zb[2] = {cvt8(z, 0), cvt8(z, 8)};
                        const f32x16 acc = square_of(Zb, CiD);
                        Bb[0] = cvt8(acc, 0);
                        Bb[1] = cvt8(acc, 8);
                    });
                }
            }
        } else {
            // ---- general form ----
            for (int k = 0; k < km; ++k)
                m_step(cs.ra_k[k], cs.cb[k], cs.kap[k], !((cs.quad >> k) & 1), (cs.neg >> k) & 1);
            if (km < K) {
                XR[0] = cvt8(Ym, 0);
                XR[1] = cvt8(Ym, 8);
            }
            for (int k = km; k < K; ++k) {
                const float k1 = cs.k1[k], k2 = cs.k2[k];
                const bool quad = (cs.quad >> k) & 1;
                // B = kq acc + k1 A from the packed A
                auto lin_b = [&](const f32x16& acc, const u32x4 (&Ab)[2], float kq, f32x16& B) __attribute__((always_inline)) {
#pragma unroll
                    for (int f = 0; f < 2; ++f)
#pragma unroll
                        for (int kk = 0; kk < 4; ++kk) {
                            const int e = 8 * f + 2 * kk;
                            B[e] = __builtin_fmaf(kq, acc[e], k1 * lo_f(Ab[f][kk]));
                            B[e + 1] = __builtin_fmaf(kq, acc[e + 1], k1 * hi_f(Ab[f][kk]));
                        }
                };
                {
                    // B' = r a I + k1 A + k2 A^2: the identity as the diagonal
                    // of the A^2 accumulator's start (dinit = r a / k2), or
                    // alone when c = 0 (k2 = 1, dinit = r a)
                    f_step([&](u32x4 (&Bb)[2]) __attribute__((always_inline)) {
                        f32x16 a = mfma32w(XR[0], XR[0], f32x16{});
                        a = mfma32w(XR[1], XR[1], a);
                        const u32x4 Ab[2] = {cvt8(a, 0), cvt8(a, 8)};
                        set_diag(cs.dinit[k]);
                        f32x16 B;
                        if (quad) lin_b(square_of(Ab, Ci), Ab, k2, B);
                        else lin_b(Ci, Ab, 1.f, B);
                        Bb[0] = cvt8(B, 0);
                        Bb[1] = cvt8(B, 8);
                    });
                }
            }
        }
        // the last iterate in fp32 (Ym), times 1 / g in the square form,
        // rounded once
        // (the square form always has K >= 1: consts32 picks it only then, so
        // no per-element select on K is needed here)
        if constexpr (SQUARE) Ym = Ym * cs.rlast;
        if (SQUARE || K <= cs.n_master) {
            XR[0] = cvt8(Ym, 0);
            XR[1] = cvt8(Ym, 8);
        }

        // ---- write back in place (Muon: W <- W - eta X) ----
        put_rl(sX, XR);
        __syncthreads();
        u16x8 out[IO::NCH];
#pragma unroll
        for (int it = 0; it < IO::NCH; ++it)
            out[it] = *reinterpret_cast<const u16x8*>(&sX[(crow + 16 * it) * kLD32 + ccol]);
        if (full && !MUON) {
            unsigned short* p0 = mbase + (int64_t)crow * me.m_ld + ccol;
            *reinterpret_cast<u16x8*>(p0) = out[0];
            *reinterpret_cast<u16x8*>(p0 + 16 * me.m_ld) = out[1];
        } else {
            unsigned short* obase = mbase;
            int64_t old = me.m_ld;
            bool ovec = mvec;
            if constexpr (MUON) {
                obase = reinterpret_cast<unsigned short*>(me.w) + (int64_t)tg.r0 * me.w_ld + tg.c0;
                old = me.w_ld;
                ovec = vec_ok(me.w, me.w_ld, tg.c0);
            }
            if (MUON && h == 32 && wd == 32 && ovec) {
                muon_update_whole<IO::NCH, IO::NCH>(obase + (int64_t)crow * old + ccol, 16 * old, args.eta, out);
            } else {
#pragma unroll
            for (int it = 0; it < IO::NCH; ++it) {
                const int r = crow + 16 * it;
                u16x8 v = out[it];
                if constexpr (MUON) {
                    u16x8 wv = IO::load(obase, old, r, ccol, h, wd, ovec);
#pragma unroll
                    for (int e = 0; e < 8; ++e) v[e] = f2bf(bf2f(wv[e]) - args.eta * bf2f(v[e]));
                }
                IO::store(obase, old, r, ccol, h, wd, ovec, v);
            }
            }
        }
        __syncthreads();
    }
}

}  // namespace

// Constants of the scaled iterate, in double precision.
Consts32 consts32(const float* abc, int K) {
    Consts32 c{};
    c.g0 = 1.0f;
    // bf16 steps only as a final run whose amplification of small singular
    // values (the product of |a_t|) stays at most that of three quintic steps
    int m = K < 2 ? K : 2;
    for (;;) {
        double prod = 1.0;
        for (int k = m; k < K; ++k) prod *= std::fabs((double)abc[3 * k]);
        if (prod <= 41.0 || m >= K) break;
        ++m;
    }
    c.n_master = m;
    if (K == 0) return c;
    bool same = true;
    for (int k = 1; k < K; ++k)
        for (int i = 0; i < 3; ++i) same = same && abc[3 * k + i] == abc[i];
    const double a = abc[0], b = abc[1], cc = abc[2];
    if (same && cc > 0.0) {
        // square form: g^4 = c, so the quadratic coefficient is 1
        c.square = 1;
        const float gf = (float)std::pow(cc, 0.25);
        const double g = gf;
        c.g0 = gf;
        const double beta = b / (g * g);
        c.beta = (float)beta;
        c.mu = (float)(beta / 2.0);
        c.d = (float)(a - beta * beta / 4.0);
        c.ra = (float)a;
        c.rlast = (float)(1.0 / g);
        return c;
    }
    // general form: g_k = sqrt(|b_k|) (1 when b_k = 0), g_K = 1
    double gk[kMaxSteps + 1];
    for (int k = 0; k < K; ++k) {
        const double bk = abc[3 * k + 1];
        gk[k] = bk != 0.0 ? (double)(float)std::sqrt(std::fabs(bk)) : 1.0;
    }
    gk[K] = 1.0;
    c.g0 = (float)gk[0];
    c.quad = 0;
    c.neg = 0;
    for (int k = 0; k < K; ++k) {
        const double ak = abc[3 * k], bk = abc[3 * k + 1], ck = abc[3 * k + 2];
        const double r = gk[k + 1] / gk[k];
        const double g2 = gk[k] * gk[k];
        c.k1[k] = (float)(r * bk / g2);
        if (bk != 0.0 && gk[k + 1] == gk[k]) c.k1[k] = bk < 0 ? -1.0f : 1.0f;
        c.ra_k[k] = (float)(r * ak);
        if (ck != 0.0) {
            c.quad |= 1 << k;
            const double k2 = r * ck / (g2 * g2);
            c.k2[k] = (float)k2;
            c.dinit[k] = (float)(r * ak / k2);
            // fp32 step: kap^2 = r |c| / g^4, kap cb = r b / g^2; for c < 0
            // the kernel forms -Z = -cb Y + Ab Y and negates its rounding
            const double kap = std::sqrt(r * std::fabs(ck)) / g2;
            const double cb = r * bk / (g2 * kap);
            c.kap[k] = (float)kap;
            c.cb[k] = (float)(ck < 0.0 ? -cb : cb);
            if (ck < 0.0) c.neg |= 1 << k;
        } else {
            c.k2[k] = 1.0f;
            c.dinit[k] = (float)(r * ak);
            c.kap[k] = (float)(r * bk / g2);   // fp32 step: Y' = r a Y + Ab Y
        }
    }
    return c;
}

// Resident slots of the 32-tile kernel on the current device, rounded down to
// a multiple of 16 (the adjacent-tile groups), cached per device and variant.
template <bool MUON, bool SQUARE>
static int slots32() {
    static std::atomic<int> cache[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        int per_cu = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, resident32_kernel<MUON, SQUARE>, 64, 0) != hipSuccess)
            return 0;
        v = (per_cu * device_cus()) & ~15;
        cache[dev].store(v, std::memory_order_relaxed);
    }
    return v;
}

hipError_t launch_resident32(const ResidentArgs& a, bool muon, hipStream_t s) {
    const int n = a.tile_end - a.tile_begin;
    if (n <= 0) return hipSuccess;
    const Consts32 c = consts32(a.abc, a.K);
    const int slots = muon ? (c.square ? slots32<true, true>() : slots32<true, false>())
                           : (c.square ? slots32<false, true>() : slots32<false, false>());
    int grid = (n + 15) & ~15;
    if (slots >= 16 && slots < grid) grid = slots;
    if (muon) {
        if (c.square) hipLaunchKernelGGL((resident32_kernel<true, true>), dim3(grid), dim3(64), 0, s, a, c);
        else hipLaunchKernelGGL((resident32_kernel<true, false>), dim3(grid), dim3(64), 0, s, a, c);
    } else {
        if (c.square) hipLaunchKernelGGL((resident32_kernel<false, true>), dim3(grid), dim3(64), 0, s, a, c);
        else hipLaunchKernelGGL((resident32_kernel<false, false>), dim3(grid), dim3(64), 0, s, a, c);
    }
    return hipGetLastError();
}

}  // namespace himuon
