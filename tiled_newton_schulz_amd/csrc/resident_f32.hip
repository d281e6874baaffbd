// On-chip tiled Newton-Schulz for fp32 tiles of up to 64 x 64 on gfx950.
//
// One workgroup of four waves owns one tile for all K steps (HiMuon abstract:
// the same finite Newton-Schulz map on every tile independently; Gram
// Newton-Schulz page, Algorithm 1, for the map).  The tile, zero padded to
// 64 x 64, stays in LDS as fp32: the padded Gram matrix is block diagonal, so
// the padding stays zero and the real block evolves as its own map.  Per step
// wave w computes the 32 x 32 block (I, J) = (w / 2, w % 2) of
//     A = X X^T,   B' = a I + b A + c A^2,   X' = B' X
// with v_mfma_f32_32x32x2_f32 (fp32 operands and accumulation), A and then B'
// passing through a second LDS area.  Nothing is rounded below fp32, so the
// result matches the fp64 map to a few 1e-6.
//
// MFMA operands (32x32x2 fp32): lane l gives P[i = l % 32][k] of the left
// factor and Q[k][j = l % 32] of the right one, k = k0 + (l / 32); the result
// lands in the accumulator layout, lane l, register q holding
// C[(q / 4) * 8 + (l / 32) * 4 + q % 4][l % 32].  MFMA 2j + e of a product
// takes k = 4j + 2 (l / 32) + e on both factors, so that a lane reads the two
// k of a left-factor row with one 8-byte LDS read.
//
// The step path did this work in 3K + 2 launches over a global workspace;
// for the 32 tiles of a 256 x 512 matrix that was launch bound.

#include "common.h"

namespace himuon {

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kLDF = 66;   // LDS row stride (floats): 8-byte aligned rows, 32 rows on 64 distinct banks

__device__ __forceinline__ f32x16 mfma_f32(float a, float b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int al_row(int q, int g) { return (q >> 2) * 8 + g * 4 + (q & 3); }

template <bool MUON>
__global__ __launch_bounds__(256) void resident_f32_kernel(const ResidentArgs args) {
    __shared__ __attribute__((aligned(16))) float sX[64 * kLDF];
    __shared__ __attribute__((aligned(16))) float sA[64 * kLDF];
    __shared__ float red[4];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int I = w >> 1, J = w & 1;
    const int l32 = lane & 31, g = lane >> 5;

    const int t = args.tile_begin + blockIdx.x;
    const MatEntry& me = args.mats[find_class(args.mats, args.nmats, t)];
    const TileGeom tg = class_tile(me, args.T, t - me.tile_base);
    const int h = tg.h, wd = tg.w;
    float* mbase = reinterpret_cast<float*>(me.m) + (int64_t)tg.r0 * me.m_ld + tg.c0;

    // ---- load (Muon: M <- mu M + G, stored), sum of squares ----
    // thread tid: row tid / 4, columns 16 (tid % 4) .. + 15
    const int lr = tid >> 2, lc = (tid & 3) * 16;
    float v[16];
    {
        const bool row_in = lr < h;
        const bool vec = ((reinterpret_cast<uintptr_t>(mbase) & 15) == 0) && (me.m_ld % 4 == 0) && lc + 16 <= wd;
        const float* gbase = nullptr;
        bool gvec = false;
        if constexpr (MUON) {
            gbase = reinterpret_cast<const float*>(me.g) + (int64_t)tg.r0 * me.g_ld + tg.c0;
            gvec = ((reinterpret_cast<uintptr_t>(gbase) & 15) == 0) && (me.g_ld % 4 == 0) && lc + 16 <= wd;
        }
        float* mrow = mbase + (int64_t)lr * me.m_ld + lc;
        if (row_in && vec) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x4 x = *reinterpret_cast<const f32x4*>(mrow + 4 * q);
                v[4 * q] = x[0]; v[4 * q + 1] = x[1]; v[4 * q + 2] = x[2]; v[4 * q + 3] = x[3];
            }
        } else {
#pragma unroll
            for (int e = 0; e < 16; ++e) v[e] = (row_in && lc + e < wd) ? mrow[e] : 0.f;
        }
        if constexpr (MUON) {
            const float* grow = gbase + (int64_t)lr * me.g_ld + lc;
            float gv[16];
            if (row_in && gvec) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f32x4 x = *reinterpret_cast<const f32x4*>(grow + 4 * q);
                    gv[4 * q] = x[0]; gv[4 * q + 1] = x[1]; gv[4 * q + 2] = x[2]; gv[4 * q + 3] = x[3];
                }
            } else {
#pragma unroll
                for (int e = 0; e < 16; ++e) gv[e] = (row_in && lc + e < wd) ? grow[e] : 0.f;
            }
#pragma unroll
            for (int e = 0; e < 16; ++e) v[e] = __builtin_fmaf(args.mu, v[e], gv[e]);
            if (row_in && vec) {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    *reinterpret_cast<f32x4*>(mrow + 4 * q) = f32x4{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
            } else {
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    if (row_in && lc + e < wd) mrow[e] = v[e];
            }
        }
    }
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) ss = __builtin_fmaf(v[e], v[e], ss);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, 64);
    if (lane == 0) red[w] = ss;
    __syncthreads();
    const float tot = (red[0] + red[1]) + (red[2] + red[3]);
    const float scale = args.normalize ? 1.0f / (sqrtf(tot) + args.eps) : 1.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q)
        *reinterpret_cast<f32x4*>(&sX[lr * kLDF + lc + 4 * q]) =
            f32x4{v[4 * q] * scale, v[4 * q + 1] * scale, v[4 * q + 2] * scale, v[4 * q + 3] * scale};
    __syncthreads();

    // C(I, J) = sum_k P(I, k) Q(k, J): P read by rows (8-byte reads of two k),
    // Q by rows (q_rows: Q(k, J) = R(J, k) for a symmetric or transposed
    // right factor) or by columns
    auto product = [&](const float* P, const float* Q, bool q_rows) __attribute__((always_inline)) {
        f32x16 acc = {};
        const float* prow = P + (I * 32 + l32) * kLDF + 2 * g;
#pragma unroll 4
        for (int j = 0; j < 16; ++j) {
            const f32x2 p = *reinterpret_cast<const f32x2*>(prow + 4 * j);
            f32x2 q;
            if (q_rows) {
                q = *reinterpret_cast<const f32x2*>(Q + (J * 32 + l32) * kLDF + 4 * j + 2 * g);
            } else {
                q[0] = Q[(4 * j + 2 * g) * kLDF + J * 32 + l32];
                q[1] = Q[(4 * j + 2 * g + 1) * kLDF + J * 32 + l32];
            }
            acc = mfma_f32(p[0], q[0], acc);
            acc = mfma_f32(p[1], q[1], acc);
        }
        return acc;
    };
    auto put = [&](float* D, const f32x16& c) __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < 16; ++q) D[(I * 32 + al_row(q, g)) * kLDF + J * 32 + l32] = c[q];
    };

    for (int step = 0; step < args.K; ++step) {
        const float ca = args.abc[3 * step], cb = args.abc[3 * step + 1], cc = args.abc[3 * step + 2];
        const f32x16 a = product(sX, sX, true);                // A = X X^T
        put(sA, a);
        __syncthreads();
        f32x16 b = product(sA, sA, true);                      // A^2 (A symmetric)
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const float lin = (I == J && I * 32 + al_row(q, g) == J * 32 + l32) ? __builtin_fmaf(cb, a[q], ca)
                                                                               : cb * a[q];
            b[q] = __builtin_fmaf(cc, b[q], lin);
        }
        __syncthreads();                                       // every wave has read A
        put(sA, b);
        __syncthreads();
        const f32x16 x = product(sA, sX, false);               // X' = B' X
        __syncthreads();                                       // every wave has read X
        put(sX, x);
        __syncthreads();
    }

    // ---- write back in place (Muon: W <- W - eta X) ----
    float* obase = mbase;
    int64_t old = me.m_ld;
    if constexpr (MUON) {
        obase = reinterpret_cast<float*>(me.w) + (int64_t)tg.r0 * me.w_ld + tg.c0;
        old = me.w_ld;
    }
    const bool row_in = lr < h;
    const bool vec = ((reinterpret_cast<uintptr_t>(obase) & 15) == 0) && (old % 4 == 0) && lc + 16 <= wd;
    float* orow = obase + (int64_t)lr * old + lc;
    float o[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(&sX[lr * kLDF + lc + 4 * q]);
        o[4 * q] = x[0]; o[4 * q + 1] = x[1]; o[4 * q + 2] = x[2]; o[4 * q + 3] = x[3];
    }
    if constexpr (MUON) {
        if (row_in && vec) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x4 x = *reinterpret_cast<const f32x4*>(orow + 4 * q);
#pragma unroll
                for (int e = 0; e < 4; ++e) o[4 * q + e] = __builtin_fmaf(-args.eta, o[4 * q + e], x[e]);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 16; ++e)
                if (row_in && lc + e < wd) o[e] = __builtin_fmaf(-args.eta, o[e], orow[e]);
        }
    }
    if (row_in && vec) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            *reinterpret_cast<f32x4*>(orow + 4 * q) = f32x4{o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]};
    } else {
#pragma unroll
        for (int e = 0; e < 16; ++e)
            if (row_in && lc + e < wd) orow[e] = o[e];
    }
}

}  // namespace

hipError_t launch_resident_f32(const ResidentArgs& a, bool muon, hipStream_t s) {
    const int n = a.tile_end - a.tile_begin;
    if (n <= 0) return hipSuccess;
    if (muon)
        hipLaunchKernelGGL((resident_f32_kernel<true>), dim3(n), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((resident_f32_kernel<false>), dim3(n), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace himuon
