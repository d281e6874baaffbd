// Pair statistics of equal-shaped matrices on gfx950: for each pair (a, b)
// the sums  sum a*b,  sum a*a,  sum b*b  in fp64.  They give the relative
// Frobenius distance and the cosine similarity between a tiled Newton-Schulz
// output and the full-matrix map of the same input (HiMuon abstract: the tiled
// map stands in locally for the full one; the pages give no measure of the
// gap, so these plain ones are used).
//
// The work is a stream over both matrices (HBM bound, 4 or 8 bytes per
// element pair), so there are no MFMA or LDS tiles: each 256-thread workgroup
// reads a band of whole rows in 16-byte chunks, several chunks in flight per
// thread, and accumulates with fp64 fmas (the products of bf16 or fp32 values
// are exact in fp64).  The workgroup's three sums go to the caller's
// workspace; a second launch adds each pair's partials in a fixed order, so
// the result does not depend on scheduling.

#include "pair_stats.h"

namespace himuon {
namespace {

typedef unsigned short u16x8p __attribute__((ext_vector_type(8)));
typedef float f32x4p __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kUnroll = 4;   // 16-byte chunks per operand in flight per thread

__device__ __forceinline__ float bf16_to_f(unsigned short u) { return __uint_as_float(((unsigned)u) << 16); }

// Eight consecutive elements (c .. c+7) of row r, zero past the row's end.
template <int DT>
__device__ __forceinline__ void load8(const void* base, int64_t ld, int r, int c, int cols, bool vec, float (&v)[8]) {
    if constexpr (DT == 0) {
        const unsigned short* p = reinterpret_cast<const unsigned short*>(base) + (int64_t)r * ld + c;
        if (vec && c + 8 <= cols) {
            const u16x8p x = *reinterpret_cast<const u16x8p*>(p);
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = bf16_to_f(x[e]);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = c + e < cols ? bf16_to_f(p[e]) : 0.f;
        }
    } else {
        const float* p = reinterpret_cast<const float*>(base) + (int64_t)r * ld + c;
        if (vec && c + 8 <= cols) {
            const f32x4p x0 = *reinterpret_cast<const f32x4p*>(p);
            const f32x4p x1 = *reinterpret_cast<const f32x4p*>(p + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) { v[e] = x0[e]; v[4 + e] = x1[e]; }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = c + e < cols ? p[e] : 0.f;
        }
    }
}

__device__ __forceinline__ bool aligned16(const void* p, int64_t ld, int es) {
    return (reinterpret_cast<uintptr_t>(p) & 15) == 0 && ((ld * es) & 15) == 0;
}

__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

template <int DT>
__global__ __launch_bounds__(kThreads) void pair_partial_kernel(const PairArgs args) {
    constexpr int ES = DT == 0 ? 2 : 4;
    const int blk = blockIdx.x;
    // the pair of this workgroup: the last one whose first workgroup is <= blk
    // (binary search over the increasing block_base; pair 0 starts at 0)
    int lo = 0, hi = args.n - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (args.e[mid].block_base <= blk) lo = mid;
        else hi = mid - 1;
    }
    const int i = lo;
    const PairEntry& E = args.e[i];
    const int lb = blk - E.block_base;
    const int r0 = lb * E.rows_per_block;
    const int r1 = min(E.rows, r0 + E.rows_per_block);
    const int cpr = (E.cols + 7) / 8;             // 8-element chunks per row
    const int nch = (r1 - r0) * cpr;              // chunks of this band
    const bool vec = aligned16(E.a, E.lda, ES) && aligned16(E.b, E.ldb, ES);

    double dot = 0.0, aa = 0.0, bb = 0.0;
    for (int base = 0; base < nch; base += kThreads * kUnroll) {
        float av[kUnroll][8], bv[kUnroll][8];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int idx = base + u * kThreads + (int)threadIdx.x;
            if (idx < nch) {
                const int r = r0 + idx / cpr, c = (idx % cpr) * 8;
                load8<DT>(E.a, E.lda, r, c, E.cols, vec, av[u]);
                load8<DT>(E.b, E.ldb, r, c, E.cols, vec, bv[u]);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) av[u][e] = bv[u][e] = 0.f;
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const double x = av[u][e], y = bv[u][e];
                dot = __builtin_fma(x, y, dot);
                aa = __builtin_fma(x, x, aa);
                bb = __builtin_fma(y, y, bb);
            }
    }

    __shared__ double red[3][kThreads / 64];
    dot = wave_sum_d(dot);
    aa = wave_sum_d(aa);
    bb = wave_sum_d(bb);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (lane == 0) {
        red[0][w] = dot;
        red[1][w] = aa;
        red[2][w] = bb;
    }
    __syncthreads();
    if (threadIdx.x < 3) {
        double s = 0.0;
#pragma unroll
        for (int k = 0; k < kThreads / 64; ++k) s += red[threadIdx.x][k];
        args.partial[(int64_t)(E.part_base + lb) * 3 + threadIdx.x] = s;
    }
}

// One wave per pair: partials strided over the lanes, then the same butterfly
// in every run.
__global__ __launch_bounds__(64) void pair_final_kernel(const PairArgs args) {
    const PairEntry& E = args.e[blockIdx.x];
    const int lane = threadIdx.x;
    double s0 = 0.0, s1 = 0.0, s2 = 0.0;
    for (int k = lane; k < E.nblocks; k += 64) {
        const double* p = args.partial + (int64_t)(E.part_base + k) * 3;
        s0 += p[0];
        s1 += p[1];
        s2 += p[2];
    }
    s0 = wave_sum_d(s0);
    s1 = wave_sum_d(s1);
    s2 = wave_sum_d(s2);
    if (lane == 0) {
        args.out[3 * blockIdx.x + 0] = s0;
        args.out[3 * blockIdx.x + 1] = s1;
        args.out[3 * blockIdx.x + 2] = s2;
    }
}

}  // namespace

hipError_t launch_pair_stats(const PairArgs& a, hipStream_t s) {
    if (a.n <= 0) return hipSuccess;
    if (a.dtype == 0)
        hipLaunchKernelGGL((pair_partial_kernel<0>), dim3(a.total_blocks), dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL((pair_partial_kernel<1>), dim3(a.total_blocks), dim3(kThreads), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(pair_final_kernel, dim3(a.n), dim3(64), 0, s, a);
    return hipGetLastError();
}

}  // namespace himuon
