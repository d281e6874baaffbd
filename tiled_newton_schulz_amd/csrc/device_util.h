// Device helpers shared by the on-chip kernels: bf16 packing, the MFMA
// operand wrapper, wave reductions and masked 16-byte tile movement.
#pragma once

#include "common.h"

namespace himuon {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));

#define LDS_AS __attribute__((address_space(3)))

namespace {


__device__ __forceinline__ float bf2f(unsigned short u) { return __uint_as_float(((unsigned)u) << 16); }
__device__ __forceinline__ unsigned short f2bf(float f) {
    __bf16 b = (__bf16)f;
    return __builtin_bit_cast(unsigned short, b);
}
// Two floats -> one word of two bf16 (round to nearest even), low half first.
__device__ __forceinline__ unsigned pack2(float a, float b) {
    bf16x2 v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(unsigned, v);
}
__device__ __forceinline__ float lo_f(unsigned u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float hi_f(unsigned u) { return __uint_as_float(u & 0xffff0000u); }

// Registers off..off+7 of an accumulator block as one bf16 MFMA operand.
// The packed words are made opaque to the optimiser: otherwise it rewrites a
// later lo_f(word) (a shift of the word) as a fresh one-element conversion
// plus a shift, one extra VALU instruction per unpacked element.
__device__ __forceinline__ u32x4 cvt8(const f32x16& v, int off) {
    u32x4 r;
#pragma unroll
    for (int k = 0; k < 4; ++k) r[k] = pack2(v[off + 2 * k], v[off + 2 * k + 1]);
    asm("" : "+v"(r));
    return r;
}
// The bf16 rounding error of those registers, itself rounded to bf16.
__device__ __forceinline__ u32x4 cvt8_lo(const f32x16& v, int off, u32x4 hi) {
    u32x4 r;
#pragma unroll
    for (int k = 0; k < 4; ++k)
        r[k] = pack2(v[off + 2 * k] - lo_f(hi[k]), v[off + 2 * k + 1] - hi_f(hi[k]));
    return r;
}
__device__ __forceinline__ f32x16 mfma32w(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                   c, 0, 0, 0);
}

// a_t on the diagonal of a diagonal AL block: element q of lane (l32, g) sits
// at row (q/4) 8 + 4 g + q%4 and column l32.  B' = a I + b A + c A^2 is formed
// as fma(c, A^2, fma(b, A, this)), so the identity costs no extra instruction.
__device__ __forceinline__ float diag_term(int q, int l32, int g, float ca) {
    return ((q >> 2) * 8 + g * 4 + (q & 3) == l32) ? ca : 0.f;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// Global <-> LDS tile movement in 16-byte chunks, masked to the h x w tile.
template <int TK>
struct TileIO {
    static constexpr int CPR = TK / 8;            // chunks per row
    static constexpr int NCH = TK * CPR / 64;     // chunks per lane

    __device__ static u16x8 load(const unsigned short* base, int64_t ld, int r, int col, int h, int w, bool vec) {
        u16x8 v = {0, 0, 0, 0, 0, 0, 0, 0};
        if (r < h) {
            const unsigned short* p = base + (int64_t)r * ld + col;
            if (vec && col + 8 <= w) {
                v = *reinterpret_cast<const u16x8*>(p);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (col + e < w) v[e] = p[e];
            }
        }
        return v;
    }
    __device__ static void store(unsigned short* base, int64_t ld, int r, int col, int h, int w, bool vec, u16x8 v) {
        if (r < h) {
            unsigned short* p = base + (int64_t)r * ld + col;
            if (vec && col + 8 <= w) {
                *reinterpret_cast<u16x8*>(p) = v;
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (col + e < w) p[e] = v[e];
            }
        }
    }
};

__device__ __forceinline__ bool vec_ok(const void* base, int64_t ld, int c0) {
    return ((reinterpret_cast<uintptr_t>(base) & 15) == 0) && ((ld & 7) == 0) && ((c0 & 7) == 0);
}

// Muon prologue M <- mu M + G (rounded to bf16, stored) over NCH 16-byte
// chunks of a whole, aligned tile: chunk it of this thread sits it * mstride
// (M) and it * gstride (G) elements past pm and pg.  The loads of a batch of BT
// chunks of M and of G are all issued before any is waited for (one chunk at
// a time, each store would hold back the next chunk's loads); the new M is
// returned in chunk.
template <int NCH, int BT>
__device__ __forceinline__ void muon_prologue_whole(unsigned short* pm, int64_t mstride, const unsigned short* pg,
                                                    int64_t gstride, float mu, u16x8 (&chunk)[NCH]) {
    static_assert(NCH % BT == 0, "whole batches");
#pragma unroll
    for (int it0 = 0; it0 < NCH; it0 += BT) {
        u16x8 mv[BT], gv[BT];
#pragma unroll
        for (int u = 0; u < BT; ++u) mv[u] = *reinterpret_cast<const u16x8*>(pm + (it0 + u) * mstride);
#pragma unroll
        for (int u = 0; u < BT; ++u) gv[u] = *reinterpret_cast<const u16x8*>(pg + (it0 + u) * gstride);
#pragma unroll
        for (int u = 0; u < BT; ++u) {
            u16x8 v;
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = f2bf(mu * bf2f(mv[u][e]) + bf2f(gv[u][e]));
            chunk[it0 + u] = v;
            *reinterpret_cast<u16x8*>(pm + (it0 + u) * mstride) = v;
        }
    }
}

// Muon update W <- W - eta X (X rounded to bf16 first, as stored) over NCH
// chunks of a whole, aligned tile laid out as in muon_prologue_whole, the W
// loads of a batch of BT chunks issued together.
template <int NCH, int BT>
__device__ __forceinline__ void muon_update_whole(unsigned short* pw, int64_t wstride, float eta,
                                                  const u16x8 (&x)[NCH]) {
    static_assert(NCH % BT == 0, "whole batches");
#pragma unroll
    for (int it0 = 0; it0 < NCH; it0 += BT) {
        u16x8 wv[BT];
#pragma unroll
        for (int u = 0; u < BT; ++u) wv[u] = *reinterpret_cast<const u16x8*>(pw + (it0 + u) * wstride);
#pragma unroll
        for (int u = 0; u < BT; ++u) {
            u16x8 v;
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = f2bf(bf2f(wv[u][e]) - eta * bf2f(x[it0 + u][e]));
            *reinterpret_cast<u16x8*>(pw + (it0 + u) * wstride) = v;
        }
    }
}

}  // namespace

}  // namespace himuon
