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
//    (a sign modifier on the fma).
//
// Precision.  The first n_master steps keep Y in fp32 registers, Y' = r a Y
// accumulated in fp32, B = r (beta A_Y + A_Y^2) (square form: no shift, which
// would round the small early A_Y around a large diagonal) as a bf16 hi/lo
// pair (B Y = B_hi Y + B_lo Y).  The later steps keep Y in bf16 with the
// identity folded into the product.  Rounding noise that a bf16 step puts
// into directions of small singular values is multiplied by roughly a_t by
// every later step, so the host makes the bf16 steps only a final run whose
// product of |a_t| stays at most 41 (three quintic steps).  CPU emulation of
// these roundings over 200k random 32-tiles, five quintic steps: worst 1.52e-2
// (square form, n_master 2), 1.62e-2 (general form), against 1.79e-2 with
// every step in fp32 and no split of the shifted square; five quintic plus
// eleven cubic steps keep every step in fp32 by that rule: 7.9e-3.
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
// Measured on MI355X (24 transformer layers, 1.2 M tiles, K = 5): 2.00 ms per
// call against 2.46 ms for the earlier form (every step in fp32, one
// workgroup per tile), with the HBM reads halved by the tile pairing below.
// At 108-128 registers a SIMD holds four waves, and the waves' dependent
// chains (MFMA, conversion, MFMA) rather than the vector issue now set the
// time: loading the next tile during the current one was 5-8 % slower, LDS
// row strides of 48 and 56 elements 1-2 % slower than 40.
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
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(4))) void resident32_kernel(
    const ResidentArgs args, const Consts32 cs) {
    __shared__ __attribute__((aligned(16))) unsigned short sX[32 * kLD32];

    const int lane = threadIdx.x;
    const int l32 = lane & 31, g = lane >> 5;
    using IO = TileIO<32>;   // two 16-byte chunks per lane: rows lane / 4 and 16 + lane / 4
    const int crow = lane >> 2, ccol = (lane & 3) * 8;

    // RL run m (= q / 4) of a lane: row l32, columns 8m + 4g .. + 3
    auto rl_off = [&](int m) { return l32 * kLD32 + 8 * m + 4 * g; };
    auto put_rl = [&](const u32x4 (&fr)[2]) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            u32x2 v = {fr[m >> 1][2 * (m & 1)], fr[m >> 1][2 * (m & 1) + 1]};
            *reinterpret_cast<u32x2*>(&sX[rl_off(m)]) = v;
        }
    };
    // AL operand f of the stored (row-major) matrix: two transposed 8-byte reads
    auto tr_frag = [&](int f) {
        const int G = lane >> 4, i16 = lane & 15;
        const int col = 16 * (G & 1) + 4 * (i16 & 3);
        const int rowb = 16 * f + 4 * g + (i16 >> 2);
        bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(&sX[rowb * kLD32 + col]));
        bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(&sX[(rowb + 8) * kLD32 + col]));
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
    for (int base = 0; base < n; base += gridDim.x) {
        if (base + p >= n) break;
        const int t = tile_at(base);

        const MatEntry& me = args.mats[find_class(args.mats, args.nmats, t)];
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
        float ss = 0.f;
#pragma unroll
        for (int it = 0; it < IO::NCH; ++it)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float x = bf2f(chunk[it][e]);
                ss = __builtin_fmaf(x, x, ss);
            }
        ss = wave_sum_dpp(ss);
        // v_sqrt_f32 and v_rcp_f32 (1 ulp each): the scale is a per-tile
        // constant whose relative error of a few 1e-7 is far below the bf16
        // rounding
        const float scale =
            (args.normalize ? __builtin_amdgcn_rcpf(__builtin_amdgcn_sqrtf(ss) + args.eps) : 1.0f) * cs.g0;
#pragma unroll
        for (int it = 0; it < IO::NCH; ++it)
            *reinterpret_cast<u16x8*>(&sX[(crow + 16 * it) * kLD32 + ccol]) = chunk[it];
        __syncthreads();
        // Ym: the iterate in fp32 (RL); XR: its bf16 operand (RL)
        f32x16 Ym;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const u16x4 v = *reinterpret_cast<const u16x4*>(&sX[rl_off(m)]);
#pragma unroll
            for (int e = 0; e < 4; ++e) Ym[4 * m + e] = bf2f(v[e]) * scale;
        }
        u32x4 XR[2];
        __syncthreads();
        // fp32 step (k < n_master): B = r beta' A + r' A^2 as a hi/lo pair,
        // Y' = ra Y + B_hi Y + B_lo Y.  form_b writes B from the A^2
        // accumulator and the packed A.
        auto m_step = [&](float ra, auto form_b) __attribute__((always_inline)) {
            XR[0] = cvt8(Ym, 0);
            XR[1] = cvt8(Ym, 8);
            put_rl(XR);
            f32x16 a = mfma32w(XR[0], XR[0], f32x16{});
            a = mfma32w(XR[1], XR[1], a);
            const u32x4 Ab[2] = {cvt8(a, 0), cvt8(a, 8)};
            f32x16 B;
            form_b(Ab, B);
            const u32x4 Bh[2] = {cvt8(B, 0), cvt8(B, 8)};
            // B - B_hi (exact in fp32), rounded: the low part of the pair.
            // (v_dot2_f32_bf16 against (-1, 0) would save the unpacking, but
            // on gfx950 its result is not the exact fp32 value: measured, it
            // put a 1.7 % error into a 32-term sum of squares.)
            const u32x4 Bl[2] = {cvt8_lo(B, 0, Bh[0]), cvt8_lo(B, 8, Bh[1])};
            __syncthreads();
            const u32x4 op0 = tr_frag(0), op1 = tr_frag(1);
            f32x16 y = Ym * ra;
            y = mfma32w(op0, Bh[0], y);
            y = mfma32w(op0, Bl[0], y);
            y = mfma32w(op1, Bh[1], y);
            y = mfma32w(op1, Bl[1], y);
            Ym = y;
            __syncthreads();
        };
        // bf16 step (k >= n_master): B' from the packed A by form_b,
        // Y' = B' Y rounded to bf16 in XR
        auto f_step = [&](bool first, auto make_b) __attribute__((always_inline)) {
            if (first) {
                XR[0] = cvt8(Ym, 0);
                XR[1] = cvt8(Ym, 8);
            }
            put_rl(XR);
            u32x4 Bb[2];
            make_b(Bb);
            __syncthreads();
            const u32x4 op0 = tr_frag(0), op1 = tr_frag(1);
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

        if constexpr (SQUARE) {
            // ---- square form: constant coefficients, c > 0 ----
            // (the factor 1 / g that brings the last iterate back to X is
            // applied with the final rounding, below)
            const float beta = cs.beta;
            for (int k = 0; k < K; ++k) {
                if (k < cs.n_master) {
                    m_step(cs.ra, [&](const u32x4 (&Ab)[2], f32x16& B) __attribute__((always_inline)) {
                        const f32x16 acc = square_of(Ab, f32x16{});
#pragma unroll
                        for (int f = 0; f < 2; ++f)
#pragma unroll
                            for (int kk = 0; kk < 4; ++kk) {
                                const int e = 8 * f + 2 * kk;
                                B[e] = __builtin_fmaf(beta, lo_f(Ab[f][kk]), acc[e]);
                                B[e + 1] = __builtin_fmaf(beta, hi_f(Ab[f][kk]), acc[e + 1]);
                            }
                    });
                } else {
                    // (A_Y + mu I)^2 + d I: both diagonals start the accumulators
                    f_step(k == cs.n_master, [&](u32x4 (&Bb)[2]) __attribute__((always_inline)) {
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
            for (int k = 0; k < K; ++k) {
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
                if (k < cs.n_master) {
                    m_step(cs.ra_k[k], [&](const u32x4 (&Ab)[2], f32x16& B) __attribute__((always_inline)) {
                        if (quad) lin_b(square_of(Ab, f32x16{}), Ab, k2, B);
                        else lin_b(f32x16{}, Ab, 0.f, B);
                    });
                } else {
                    // B' = r a I + k1 A + k2 A^2: the identity as the diagonal
                    // of the A^2 accumulator's start (dinit = r a / k2), or
                    // alone when c = 0 (k2 = 1, dinit = r a)
                    f_step(k == cs.n_master, [&](u32x4 (&Bb)[2]) __attribute__((always_inline)) {
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
        if (SQUARE && K > 0) Ym = Ym * cs.rlast;
        if (SQUARE || K <= cs.n_master) {
            XR[0] = cvt8(Ym, 0);
            XR[1] = cvt8(Ym, 8);
        }

        // ---- write back in place (Muon: W <- W - eta X) ----
        put_rl(XR);
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
        } else {
            c.k2[k] = 1.0f;
            c.dinit[k] = (float)(r * ak);
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
