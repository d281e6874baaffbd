// C ABI of the tiled Newton-Schulz library: argument validation, the tile
// planner (launch groups, on-chip kernel choice, workspace chunks) and
// dispatch.  See include/himuon.h for the contract.
#include "himuon.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

#include "common.h"
#include "stepargs.h"
#include "pair_stats.h"

using namespace himuon;

namespace {

thread_local int32_t g_last_hip = 0;

constexpr int kWgNormMax = 32;
constexpr size_t kAlign = 256;

size_t elem_size(himuon_dtype_t dt) { return dt == HIMUON_FP32 ? 4 : 2; }
// Storage is bf16 for HIMUON_BF16 and HIMUON_BF16_PRECISE.
bool bf16_storage(himuon_dtype_t dt) { return dt != HIMUON_FP32; }
size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

struct MatSpec {
    void* m;
    void* w;
    const void* g;
    int64_t rows, cols, m_ld, w_ld, g_ld;
    int64_t tiles;   // tiles of this matrix
};

// ---- validation --------------------------------------------------------
himuon_status_t check_matrix(const himuon_matrix_t& d, size_t es) {
    if (d.ptr == nullptr) return HIMUON_ERR_INVALID_ARGUMENT;
    if (d.rows < 1 || d.cols < 1 || d.ld < d.cols) return HIMUON_ERR_INVALID_ARGUMENT;
    if (d.rows > INT32_MAX || d.cols > INT32_MAX) return HIMUON_ERR_LAYOUT;
    if ((reinterpret_cast<uintptr_t>(d.ptr) % es) != 0) return HIMUON_ERR_LAYOUT;
    // extent in bytes must fit in int64
    const double ext = ((double)(d.rows - 1) * (double)d.ld + (double)d.cols) * (double)es;
    if (ext > 9.0e18) return HIMUON_ERR_LAYOUT;
    return HIMUON_OK;
}

struct Extent {
    uintptr_t lo, hi;  // [lo, hi) bytes
    int64_t ld, cols;
    int64_t rows;
    size_t es;
    int id;
};

// True if two matrices share an element.  Byte ranges that overlap can still
// be disjoint when both use the same row stride and occupy different column
// ranges of the same rows (column blocks of one fused tensor).
bool share_element(const Extent& a, const Extent& b) {
    if (a.hi <= b.lo || b.hi <= a.lo) return false;
    if (a.ld != b.ld || a.es != b.es) return true;
    const Extent& x = a.lo <= b.lo ? a : b;
    const Extent& y = a.lo <= b.lo ? b : a;
    const uintptr_t d = y.lo - x.lo;
    const uintptr_t row_bytes = (uintptr_t)x.ld * x.es;
    if (d % x.es != 0) return true;
    const int64_t dc = (int64_t)((d % row_bytes) / x.es);   // column offset of y inside x's rows
    // y's columns [dc, dc + y.cols) must avoid x's [0, x.cols) in every row both touch,
    // including y rows that wrap past ld.
    if (dc < x.cols) return true;
    if (dc + y.cols > x.ld) return true;   // wraps into x's next row
    return false;
}

himuon_status_t check_overlap(std::vector<Extent>& ex) {
    std::sort(ex.begin(), ex.end(), [](const Extent& a, const Extent& b) { return a.lo < b.lo; });
    for (size_t i = 0; i < ex.size(); ++i)
        for (size_t j = i + 1; j < ex.size() && ex[j].lo < ex[i].hi; ++j)
            if (share_element(ex[i], ex[j])) return HIMUON_ERR_OVERLAP;
    return HIMUON_OK;
}

Extent extent_of(const himuon_matrix_t& d, size_t es, int id) {
    Extent e;
    e.lo = reinterpret_cast<uintptr_t>(d.ptr);
    e.hi = e.lo + (uintptr_t)(((d.rows - 1) * d.ld + d.cols) * (int64_t)es);
    e.ld = d.ld;
    e.cols = d.cols;
    e.rows = d.rows;
    e.es = es;
    e.id = id;
    return e;
}

himuon_status_t check_common(int32_t n, int32_t T, int32_t K, himuon_dtype_t dt, float eps) {
    if (n < 0 || T < 1) return HIMUON_ERR_INVALID_ARGUMENT;
    if (K < 0 || K > HIMUON_MAX_STEPS) return HIMUON_ERR_INVALID_ARGUMENT;
    if (dt != HIMUON_BF16 && dt != HIMUON_FP32 && dt != HIMUON_BF16_PRECISE) return HIMUON_ERR_UNSUPPORTED;
    if (!(eps >= 0.f) || !std::isfinite(eps)) return HIMUON_ERR_INVALID_ARGUMENT;
    return HIMUON_OK;
}

himuon_status_t check_abc(int32_t K, const float* abc) {
    if (K > 0) {
        if (abc == nullptr) return HIMUON_ERR_INVALID_ARGUMENT;
        for (int i = 0; i < 3 * K; ++i)
            if (!std::isfinite(abc[i])) return HIMUON_ERR_INVALID_ARGUMENT;
    }
    return HIMUON_OK;
}

// ---- planning ------------------------------------------------------------
// Each matrix is cut into up to four tile classes (interior T x T tiles, the
// right-edge column, the bottom-edge row and the corner); all tiles of a class
// share one shape, and each class is routed by that shape:
//   bf16, both sides 48..256, or both 32..128
//                                     -> on-chip kernel (kernel tile 32/64/128/256)
//   bf16, a side < 32, both <= 64     -> on-chip kernel, hi/lo split precision
//   bf16, both sides >= 64, one > 256 -> step path, bf16 workspace
//   bf16, other thin tiles            -> step path, fp32 workspace
//   fp32, and bf16 with fp32 math     -> step path, fp32 workspace
// A bf16 iterate of a tile whose short side r is small and whose long side s
// is long loses accuracy.  Emulated worst errors, with a 3e-2 bound:
//   on chip:   2.6e-2 at r = 32, s = 256; 2.1e-2 at r = 32, s = 128 and at
//              r = 48, s = 256;
//   step path: 2.5-2.9e-2 for r = 32..40 and s = 600..2000; 1.3e-2 at r = 64.
struct TileClass {
    int spec;                 // matrix index
    int32_t ti0, tj0, n_ti, n_tj, th, tw;
    int64_t tiles() const { return (int64_t)n_ti * n_tj; }
};

enum class Route { OnChip, OnChipPrecise, OnChipF32, StepBf16, StepFp32 };

Route route_of(himuon_dtype_t dt, int32_t th, int32_t tw) {
    const int32_t mn = std::min(th, tw), mx = std::max(th, tw);
    if (dt == HIMUON_FP32 && mx <= 64) return Route::OnChipF32;
    if (dt == HIMUON_FP32 || dt == HIMUON_BF16_PRECISE) return Route::StepFp32;
    if (mx <= 256 && (mn >= 48 || (mn >= 32 && mx <= 128))) return Route::OnChip;
    if (mx <= 64) return Route::OnChipPrecise;
    if (mn >= 64) return Route::StepBf16;
    return Route::StepFp32;
}
int kernel_tile_for(int32_t th, int32_t tw) {
    const int32_t e = std::max(th, tw);
    return e <= 32 ? 32 : e <= 64 ? 64 : e <= 128 ? 128 : 256;
}
int64_t tiles_of(int64_t rows, int64_t cols, int32_t T) {
    return ((rows + T - 1) / T) * ((cols + T - 1) / T);
}

void classes_of(const MatSpec& s, int idx, int32_t T, std::vector<TileClass>& out) {
    const int32_t fh = (int32_t)(s.rows / T), fw = (int32_t)(s.cols / T);
    const int32_t rh = (int32_t)(s.rows % T), rw = (int32_t)(s.cols % T);
    if (fh > 0 && fw > 0) out.push_back({idx, 0, 0, fh, fw, T, T});
    if (fh > 0 && rw > 0) out.push_back({idx, 0, fw, fh, 1, T, rw});
    if (rh > 0 && fw > 0) out.push_back({idx, fh, 0, 1, fw, rh, T});
    if (rh > 0 && rw > 0) out.push_back({idx, fh, fw, 1, 1, rh, rw});
}

struct Chunk {
    int group;          // index into step groups
    int32_t tb, te;     // tile range within the group
    int64_t xbase, abase, xel, ael;
    int32_t rmax, smax, sbmax;
};

struct Group {
    std::vector<TileClass> cls;
    std::vector<int64_t> tile_base, xoff, aoff;
    int kernel_tile = 0;         // on-chip groups
    bool precise = false;        // on-chip groups
    bool f32 = false;            // on-chip groups: fp32 data (kernel tile 64)
    bool narrow = false;         // on-chip kernel tile 256: shorter side <= 128
    int wk = 0;                  // step groups: workspace dtype (0 bf16, 1 fp32)
    int64_t tiles = 0;
};

struct Plan {
    std::vector<Group> rgroups;  // on-chip launches
    std::vector<Group> sgroups;  // step-by-step groups
    std::vector<Chunk> chunks;
    size_t ws_full = 0, ws_min = 0;
    int64_t tiles = 0;
    int64_t launches = 0;
};

// Workspace of one chunk: the current and next oriented tiles, `sq` areas of
// r x r matrices (the standard step keeps A and B'; the Gram iteration keeps
// R, its step polynomial, the running product and a spare) and the norm
// partials.
size_t chunk_bytes(int64_t xel, int64_t ael, int64_t tiles, size_t es, int sq) {
    return align_up((size_t)xel * es) * 2 + align_up((size_t)ael * es) * sq + align_up((size_t)tiles * kWgNormMax * 4);
}

// Kernel launches of the Gram iteration for one chunk: two norm passes,
// R = X X^T, per step the polynomial, the running product (not on the first
// step after a start or restart, where it is the polynomial itself) and the
// two products of the R update (not after the last step, nor before a
// restart, which rebuilds R); a restart applies Q and rebuilds R; at the end
// Q is applied once.
int64_t gram_launches(int32_t K, int32_t restart) {
    int64_t n = 4;
    bool ident = true;
    for (int32_t t = 1; t <= K; ++t) {
        if (restart > 0 && t == restart + 1) {
            n += 2;
            ident = true;
        }
        n += ident ? 1 : 2;
        ident = false;
        if (t < K && !(restart > 0 && t == restart)) n += 2;
    }
    return n;
}

void oriented(const TileClass& c, int32_t& r, int32_t& sd) {
    r = std::min(c.th, c.tw);
    sd = std::max(c.th, c.tw);
}

// Builds the plan.  With enforce_cap, every chunk's workspace stays within
// `cap` (HIMUON_ERR_WORKSPACE if one tile alone does not fit).  gram: every
// tile runs the Gram iteration on the step path (restart as for
// himuon_gram_ns); bf16 tiles with both sides >= 96 keep a bf16 workspace,
// the others fp32 (the r x r iterates of a bf16 Gram iteration lose accuracy
// for small r: emulated worst errors of 3.3e-2 at r = 32, 2.9e-2 at 48,
// 2.0e-2 at 64 and at most 1.3e-2 from 96 on, with a 3e-2 bound).
himuon_status_t build_plan(const std::vector<MatSpec>& specs, int32_t T, int32_t K, himuon_dtype_t dt,
                           size_t cap, bool enforce_cap, Plan& plan, bool gram = false, int32_t restart = 0) {
    plan = Plan();
    std::vector<TileClass> all;
    for (size_t i = 0; i < specs.size(); ++i) {
        plan.tiles += specs[i].tiles;
        classes_of(specs[i], (int)i, T, all);
    }

    // step path workspace dtype of a class: 0 bf16, 1 fp32, -1 on chip
    auto step_wk = [&](const TileClass& c) {
        if (gram) return (dt != HIMUON_BF16 || std::min(c.th, c.tw) < 96) ? 1 : 0;
        const Route r = route_of(dt, c.th, c.tw);
        return r == Route::StepBf16 ? 0 : r == Route::StepFp32 ? 1 : -1;
    };
    const int sq = gram ? 4 : 2;

    // on-chip launches, keyed by (kernel tile, kind): kind 0 bf16, 1 split
    // precision, 2 fp32 data (every such tile in the kernel of tile 64)
    for (int kind = 0; kind < (gram ? 0 : 3); ++kind)
        for (int kt : {32, 64, 128, 256})
          for (int narrow = 0; narrow < (kt == 256 ? 2 : 1); ++narrow) {
            if (kind == 2 && kt != 64) continue;
            Group cur;
            cur.kernel_tile = kt;
            cur.precise = kind == 1;
            cur.f32 = kind == 2;
            cur.narrow = narrow != 0;
            for (const TileClass& c : all) {
                const Route r = route_of(dt, c.th, c.tw);
                const bool on = r == (kind == 0 ? Route::OnChip : kind == 1 ? Route::OnChipPrecise : Route::OnChipF32);
                if (!on || (kind != 2 && kernel_tile_for(c.th, c.tw) != kt)) continue;
                if (kt == 256 && (std::min(c.th, c.tw) <= 128) != (narrow != 0)) continue;
                if ((int)cur.cls.size() == kGroup || cur.tiles + c.tiles() > INT32_MAX) {
                    plan.rgroups.push_back(cur);
                    cur = Group();
                    cur.kernel_tile = kt;
                    cur.precise = kind == 1;
                    cur.f32 = kind == 2;
                    cur.narrow = narrow != 0;
                }
                cur.cls.push_back(c);
                cur.tile_base.push_back(cur.tiles);
                cur.tiles += c.tiles();
            }
            if (!cur.cls.empty()) plan.rgroups.push_back(cur);
        }
    plan.launches = (int64_t)plan.rgroups.size();

    // step groups, keyed by workspace dtype
    for (int wk = 0; wk < 2; ++wk) {
        Group cur;
        cur.wk = wk;
        int64_t xo = 0, ao = 0;
        for (const TileClass& c : all) {
            if (step_wk(c) != wk) continue;
            if ((int)cur.cls.size() == kGroup || cur.tiles + c.tiles() > INT32_MAX / 64) {
                plan.sgroups.push_back(cur);
                cur = Group();
                cur.wk = wk;
                xo = ao = 0;
            }
            int32_t rr, ss;
            oriented(c, rr, ss);
            cur.cls.push_back(c);
            cur.tile_base.push_back(cur.tiles);
            cur.xoff.push_back(xo);
            cur.aoff.push_back(ao);
            cur.tiles += c.tiles();
            xo += c.tiles() * rr * round8(ss);
            ao += c.tiles() * rr * round8(rr);
        }
        if (!cur.cls.empty()) plan.sgroups.push_back(cur);
    }
    for (size_t gi = 0; gi < plan.sgroups.size(); ++gi) {
        const Group& G = plan.sgroups[gi];
        const size_t es = G.wk == 0 ? 2 : 4;
        Chunk ch{};
        bool open = false;
        for (size_t k = 0; k < G.cls.size(); ++k) {
            const TileClass& c = G.cls[k];
            int32_t rr, ss;
            oriented(c, rr, ss);
            const int64_t xe = (int64_t)rr * round8(ss), ae = (int64_t)rr * round8(rr);
            const int32_t sb = ((c.th + 63) / 64) * ((c.tw + 63) / 64);
            const size_t one = chunk_bytes(xe, ae, 1, es, sq);
            plan.ws_min = std::max(plan.ws_min, one);
            for (int64_t lt = 0; lt < c.tiles(); ++lt) {
                const int32_t t = (int32_t)(G.tile_base[k] + lt);
                if (open && enforce_cap && chunk_bytes(ch.xel + xe, ch.ael + ae, t + 1 - ch.tb, es, sq) > cap) {
                    plan.chunks.push_back(ch);
                    open = false;
                }
                if (!open) {
                    if (enforce_cap && one > cap) return HIMUON_ERR_WORKSPACE;
                    ch = Chunk{};
                    ch.group = (int)gi;
                    ch.tb = t;
                    ch.xbase = G.xoff[k] + lt * xe;
                    ch.abase = G.aoff[k] + lt * ae;
                    open = true;
                }
                ch.te = t + 1;
                ch.xel += xe;
                ch.ael += ae;
                ch.rmax = std::max(ch.rmax, rr);
                ch.smax = std::max(ch.smax, ss);
                ch.sbmax = std::max(ch.sbmax, sb);
            }
        }
        if (open) plan.chunks.push_back(ch);
    }
    for (const auto& c : plan.chunks) {
        const size_t es = plan.sgroups[c.group].wk == 0 ? 2 : 4;
        plan.ws_full = std::max(plan.ws_full, chunk_bytes(c.xel, c.ael, c.te - c.tb, es, sq));
        plan.launches += gram ? gram_launches(K, restart) : 2 + 3LL * K;
    }
    return HIMUON_OK;
}

himuon_status_t gather(const himuon_matrix_t* W, const himuon_matrix_t* M, const himuon_matrix_t* G,
                       int32_t n, int32_t T, himuon_dtype_t dt, std::vector<MatSpec>& specs) {
    const size_t es = elem_size(dt);
    specs.clear();
    if (n > 0 && M == nullptr) return HIMUON_ERR_INVALID_ARGUMENT;
    const bool muon = W != nullptr || G != nullptr;
    if (muon && (W == nullptr || G == nullptr)) return HIMUON_ERR_INVALID_ARGUMENT;
    std::vector<Extent> written, read;
    for (int i = 0; i < n; ++i) {
        himuon_status_t st = check_matrix(M[i], es);
        if (st != HIMUON_OK) return st;
        MatSpec s{};
        s.m = M[i].ptr;
        s.rows = M[i].rows;
        s.cols = M[i].cols;
        s.m_ld = M[i].ld;
        written.push_back(extent_of(M[i], es, i));
        if (muon) {
            if ((st = check_matrix(W[i], es)) != HIMUON_OK) return st;
            if ((st = check_matrix(G[i], es)) != HIMUON_OK) return st;
            if (W[i].rows != M[i].rows || W[i].cols != M[i].cols || G[i].rows != M[i].rows ||
                G[i].cols != M[i].cols)
                return HIMUON_ERR_INVALID_ARGUMENT;
            s.w = W[i].ptr;
            s.w_ld = W[i].ld;
            s.g = G[i].ptr;
            s.g_ld = G[i].ld;
            written.push_back(extent_of(W[i], es, n + i));
            read.push_back(extent_of(G[i], es, 2 * n + i));
        }
        s.tiles = tiles_of(s.rows, s.cols, T);
        if (s.tiles > INT32_MAX / 64) return HIMUON_ERR_LAYOUT;
        specs.push_back(s);
    }
    std::vector<Extent> all = written;
    if (check_overlap(all) != HIMUON_OK) return HIMUON_ERR_OVERLAP;
    // a read-only gradient may alias nothing that is written
    for (const auto& r : read)
        for (const auto& w : written)
            if (share_element(r, w)) return HIMUON_ERR_OVERLAP;
    return HIMUON_OK;
}

MatEntry entry_of(const MatSpec& s, const TileClass& c, int64_t tile_base, int64_t xoff, int64_t aoff) {
    MatEntry e{};
    e.m = s.m;
    e.w = s.w;
    e.g = s.g;
    e.m_ld = s.m_ld;
    e.w_ld = s.w_ld;
    e.g_ld = s.g_ld;
    e.xoff = xoff;
    e.aoff = aoff;
    e.ti0 = c.ti0;
    e.tj0 = c.tj0;
    e.n_tj = c.n_tj;
    e.th = c.th;
    e.tw = c.tw;
    e.tile_base = (int32_t)tile_base;
    return e;
}

// One-wave kernel-tile-128 slots and CU count of the current device, queried
// once per device.
struct SlotInfo {
    int slots, cus;
};
// Cached per device and kernel; both figures are fixed for a device, so
// threads that race to fill an entry store the same values.
SlotInfo slot_info(bool muon) {
    static std::atomic<int> slots[2][64] = {};
    static std::atomic<int> cus[2][64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return SlotInfo{0, 0};
    const int k = muon ? 1 : 0;
    int c = cus[k][dev].load(std::memory_order_acquire);
    if (c == 0) {
        slots[k][dev].store(resident_slots(128, muon, false), std::memory_order_relaxed);
        c = device_cus();
        cus[k][dev].store(c, std::memory_order_release);
    }
    return SlotInfo{slots[k][dev].load(std::memory_order_relaxed), c};
}

// First tile of a group's partial last round, which goes to the eight-waves-
// per-tile kernel (kernel tile 128 only; a round is the number of tiles the
// device holds at once).  Returns the group's tile count when there is none.
int32_t tail_split(const Group& G, bool muon) {
    const int32_t total = (int32_t)G.tiles;
    if (G.kernel_tile != 128 || G.precise || G.f32) return total;
    const SlotInfo si = slot_info(muon);
    if (si.slots <= 0 || si.cus <= 0) return total;
    const int32_t rem = total % si.slots;
    return (rem > 0 && rem <= 2 * si.cus) ? total - rem : total;
}

himuon_status_t hip_fail(hipError_t e) {
    g_last_hip = (int32_t)e;
    return HIMUON_ERR_HIP;
}

// Step path arguments of one chunk, with its workspace laid out as
// [X current | X next | nsq r x r areas | norm partials]; sq receives the r x r
// area bases.
void chunk_args(const std::vector<MatSpec>& specs, const Plan& plan, const Chunk& c, int32_t T, int32_t K,
                const float* abc, himuon_dtype_t dt, float eps, float mu, float eta, bool muon, bool normalize,
                void* ws, int nsq, StepArgs& a, char** sq) {
    const Group& G = plan.sgroups[c.group];
    const size_t es = G.wk == 0 ? 2 : 4;
    a.nmats = (int32_t)G.cls.size();
    for (size_t k = 0; k < G.cls.size(); ++k)
        a.mats[k] = entry_of(specs[G.cls[k].spec], G.cls[k], G.tile_base[k], G.xoff[k], G.aoff[k]);
    for (int i = 0; i < 3 * K; ++i) a.abc[i] = abc[i];
    a.T = T;
    a.K = K;
    a.tile_begin = c.tb;
    a.tile_end = c.te;
    a.xbase = c.xbase;
    a.abase = c.abase;
    a.nb_max = (c.rmax + 127) / 128;
    a.ns_max = (c.smax + 127) / 128;
    a.wg_norm = std::min(kWgNormMax, std::max(1, c.sbmax));
    a.io_dtype = bf16_storage(dt) ? 0 : 1;
    a.wk_dtype = G.wk;
    a.slab = step_slab_layout(a) ? 1 : 0;
    a.muon = muon ? 1 : 0;
    a.eps = eps;
    a.normalize = normalize ? 1 : 0;
    a.mu = mu;
    a.eta = eta;
    char* base = reinterpret_cast<char*>(ws);
    const size_t xb = align_up((size_t)c.xel * es), ab = align_up((size_t)c.ael * es);
    a.Xc = base;
    a.Xn = base + xb;
    for (int i = 0; i < nsq; ++i) sq[i] = base + 2 * xb + i * ab;
    a.partial = reinterpret_cast<float*>(base + 2 * xb + nsq * ab);
}

himuon_status_t run(const std::vector<MatSpec>& specs, int32_t T, int32_t K, const float* abc,
                    himuon_dtype_t dt, float eps, float mu, float eta, bool muon, void* ws, size_t ws_bytes,
                    void* stream, bool normalize = true) {
    if (specs.empty()) return HIMUON_OK;
    if (ws_bytes > 0 && ws == nullptr) return HIMUON_ERR_WORKSPACE;
    Plan plan;
    himuon_status_t st = build_plan(specs, T, K, dt, ws_bytes, true, plan);
    if (st != HIMUON_OK) return st;
    if (!plan.chunks.empty() && ws == nullptr) return HIMUON_ERR_WORKSPACE;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);

    for (const Group& G : plan.rgroups) {
        ResidentArgs a{};
        a.nmats = (int32_t)G.cls.size();
        for (size_t k = 0; k < G.cls.size(); ++k)
            a.mats[k] = entry_of(specs[G.cls[k].spec], G.cls[k], G.tile_base[k], 0, 0);
        for (int i = 0; i < 3 * K; ++i) a.abc[i] = abc[i];
        a.total_tiles = (int32_t)G.tiles;
        a.T = T;
        a.K = K;
        a.eps = eps;
        a.normalize = normalize ? 1 : 0;
        a.mu = mu;
        a.eta = eta;
        // Tiles beyond the last full round of one-wave tiles go to the
        // eight-waves-per-tile kernel (kernel tile 128), which finishes a
        // partial round in about a third of a tile time.
        const int32_t split = tail_split(G, muon);
        a.tile_begin = 0;
        a.tile_end = split;
        hipError_t e = G.f32 ? launch_resident_f32(a, muon, s)
                             : launch_resident(a, G.kernel_tile, muon, G.precise, G.narrow, s);
        if (e != hipSuccess) return hip_fail(e);
        if (split < a.total_tiles) {
            a.tile_begin = split;
            a.tile_end = a.total_tiles;
            if ((e = launch_resident_coop(a, muon, s)) != hipSuccess) return hip_fail(e);
        }
    }

    for (const Chunk& c : plan.chunks) {
        StepArgs a{};
        char* sq[2];
        chunk_args(specs, plan, c, T, K, abc, dt, eps, mu, eta, muon, normalize, ws, 2, a, sq);
        a.A = sq[0];
        a.B = sq[1];
        const int64_t nt = c.te - c.tb;
        hipError_t e = launch_step_norm(a, s);
        if (e != hipSuccess) return hip_fail(e);
        // the pass wrote the tiles unscaled: the first Gram and apply products
        // take each tile's scale in their epilogue
        a.x_raw = 1;
        for (int step = 0; step < K; ++step) {
            a.step = step;
            const int64_t tri = (int64_t)a.nb_max * (a.nb_max + 1) / 2;
            a.grid_blocks = (int32_t)(((nt * tri) + 7) / 8 * 8);
            if ((e = launch_step_gram(a, s)) != hipSuccess) return hip_fail(e);
            if ((e = launch_step_poly(a, s)) != hipSuccess) return hip_fail(e);
            a.grid_blocks = (int32_t)(((nt * a.nb_max * a.ns_max) + 7) / 8 * 8);
            if ((e = launch_step_apply(a, s)) != hipSuccess) return hip_fail(e);
            a.x_raw = 0;
            std::swap(a.Xc, a.Xn);
        }
    }
    return HIMUON_OK;
}

// Tile edge that makes every matrix one tile: the largest side of the batch
// (1 when there is nothing to look at; gather reports bad descriptors).  0 if
// a side does not fit the int32 tile grid.
int32_t whole_tile(const himuon_matrix_t* m, int32_t n) {
    int64_t T = 1;
    for (int32_t i = 0; m != nullptr && i < n; ++i) T = std::max({T, m[i].rows, m[i].cols});
    return T > INT32_MAX ? 0 : (int32_t)T;
}

// Gram Newton-Schulz ("Gram Newton-Schulz" summary page, section 6,
// Algorithm 3) on every matrix as one tile, oriented so that r <= s.  The
// iteration runs on r x r matrices: R = X X^T, per step t
//     P = a_t I + b_t R + c_t R^2,  Q <- P Q,  R <- P R P,
// which is the page's Z, Q, RZ and R update with the identity terms folded
// into P (every matrix here is a polynomial in the same symmetric R, so the
// products commute and each result is symmetric: only lower blocks are
// computed and mirrored).  A restart before step restart + 1 applies Q to X,
// rebuilds R from it and starts Q again from I; at the end X <- Q X is
// written in place.  Four r x r areas rotate: R, P, Q and a spare.
himuon_status_t run_gram(const std::vector<MatSpec>& specs, int32_t T, int32_t K, const float* abc,
                         int32_t restart, himuon_dtype_t dt, float eps, void* ws, size_t ws_bytes, void* stream) {
    if (specs.empty()) return HIMUON_OK;
    if (ws_bytes > 0 && ws == nullptr) return HIMUON_ERR_WORKSPACE;
    Plan plan;
    himuon_status_t st = build_plan(specs, T, K, dt, ws_bytes, true, plan, true, restart);
    if (st != HIMUON_OK) return st;
    if (!plan.chunks.empty() && ws == nullptr) return HIMUON_ERR_WORKSPACE;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    for (const Chunk& c : plan.chunks) {
        StepArgs a{};
        char* sq[4];
        chunk_args(specs, plan, c, T, K, abc, dt, eps, 0.f, 0.f, false, true, ws, 4, a, sq);
        const int64_t nt = c.te - c.tb;
        const int64_t tri = (int64_t)a.nb_max * (a.nb_max + 1) / 2;
        const int32_t sym_grid = (int32_t)(((nt * tri) + 7) / 8 * 8);
        const int32_t apply_grid = (int32_t)(((nt * a.nb_max * a.ns_max) + 7) / 8 * 8);
        void* const R = sq[0];
        // one of the other three areas that holds neither x nor y
        auto other = [&](const void* x, const void* y) -> void* {
            for (int i = 1; i < 4; ++i)
                if (sq[i] != x && sq[i] != y) return sq[i];
            return nullptr;
        };
        auto product = [&](const void* L, const void* M, void* O) {   // O = L M^T
            a.L = L;
            a.M = M;
            a.O = O;
            a.grid_blocks = sym_grid;
            return launch_step_product(a, s);
        };
        auto gram_of_x = [&]() {   // R = X X^T
            a.A = R;
            a.grid_blocks = sym_grid;
            return launch_step_gram(a, s);
        };
        auto apply_q = [&](void* Q, int32_t step) {   // X <- Q X (written in place when step == K - 1)
            a.B = Q;
            a.step = step;
            a.grid_blocks = apply_grid;
            hipError_t e = launch_step_apply(a, s);
            a.x_raw = 0;   // X now holds the scaled product
            std::swap(a.Xc, a.Xn);
            return e;
        };
        hipError_t e = launch_step_norm(a, s);
        // the pass wrote the tiles unscaled (K >= 1): the first X X^T and the
        // first apply of Q take each tile's scale in their epilogue
        a.x_raw = K > 0 ? 1 : 0;
        if (e == hipSuccess) e = gram_of_x();
        void* Q = nullptr;   // nullptr: the identity
        for (int32_t t = 1; t <= K && e == hipSuccess; ++t) {
            if (restart > 0 && t == restart + 1) {
                if ((e = apply_q(Q, t - 2)) != hipSuccess) break;
                if ((e = gram_of_x()) != hipSuccess) break;
                Q = nullptr;
            }
            // P = a I + b R + c R^2 (step t's coefficients)
            void* P = other(Q, nullptr);
            a.A = R;
            a.B = P;
            a.step = t - 1;
            a.grid_blocks = sym_grid;
            if ((e = launch_step_poly(a, s)) != hipSuccess) break;
            if (Q == nullptr) {
                Q = P;
            } else {
                void* Qn = other(P, Q);
                if ((e = product(P, Q, Qn)) != hipSuccess) break;
                Q = Qn;
            }
            if (t < K && !(restart > 0 && t == restart)) {
                void* Tm = other(P, Q);   // R P, then R <- P (R P)
                if ((e = product(R, P, Tm)) != hipSuccess) break;
                if ((e = product(P, Tm, R)) != hipSuccess) break;
            }
        }
        if (e == hipSuccess) e = apply_q(Q, K - 1);
        if (e != hipSuccess) return hip_fail(e);
    }
    return HIMUON_OK;
}

// ---- pair statistics ----------------------------------------------------
constexpr int64_t kPairBandElems = 65536;   // elements one workgroup reduces (about)

int32_t pair_rows_per_block(int64_t rows, int64_t cols) {
    const int64_t r = (kPairBandElems + cols - 1) / cols;
    return (int32_t)std::max<int64_t>(1, std::min<int64_t>(r, rows));
}

// Workgroups (one partial each) over all pairs, from the shapes of `a`.
himuon_status_t pair_blocks(const himuon_matrix_t* a, int32_t n, int64_t* total) {
    if (n < 0 || (n > 0 && a == nullptr)) return HIMUON_ERR_INVALID_ARGUMENT;
    int64_t t = 0;
    for (int32_t i = 0; i < n; ++i) {
        if (a[i].rows < 1 || a[i].cols < 1) return HIMUON_ERR_INVALID_ARGUMENT;
        if (a[i].rows > INT32_MAX || a[i].cols > INT32_MAX) return HIMUON_ERR_LAYOUT;
        const int32_t R = pair_rows_per_block(a[i].rows, a[i].cols);
        t += (a[i].rows + R - 1) / R;
    }
    if (t > INT32_MAX) return HIMUON_ERR_LAYOUT;
    *total = t;
    return HIMUON_OK;
}

}  // namespace

extern "C" {

himuon_status_t himuon_plan(const himuon_matrix_t* m, int32_t n, int32_t T, int32_t K, himuon_dtype_t dt,
                            size_t workspace_bytes, himuon_plan_info_t* info) {
    if (info == nullptr) return HIMUON_ERR_INVALID_ARGUMENT;
    std::memset(info, 0, sizeof(*info));
    himuon_status_t st = check_common(n, T, K, dt, 0.f);
    if (st != HIMUON_OK) return st;
    std::vector<MatSpec> specs;
    if ((st = gather(nullptr, m, nullptr, n, T, dt, specs)) != HIMUON_OK) return st;
    Plan plan;
    if ((st = build_plan(specs, T, K, dt, workspace_bytes, true, plan)) != HIMUON_OK) return st;
    info->tiles = plan.tiles;
    info->resident_launches = (int64_t)plan.rgroups.size();
    info->chunks = (int64_t)plan.chunks.size();
    info->launches = plan.launches;
    for (const auto& g : plan.rgroups) {
        info->kernel_tile = std::max<int64_t>(info->kernel_tile, g.kernel_tile);
        const int32_t split = tail_split(g, false);
        if (split < g.tiles) {
            info->tail_tiles += g.tiles - split;
            info->launches += 1;
        }
    }
    info->workspace_full = plan.ws_full;
    info->workspace_min = plan.ws_min;
    return HIMUON_OK;
}

himuon_status_t himuon_workspace_size(const himuon_matrix_t* m, int32_t n, int32_t T, himuon_dtype_t dt,
                                      size_t* full, size_t* min) {
    if (full) *full = 0;
    if (min) *min = 0;
    himuon_status_t st = check_common(n, T, 0, dt, 0.f);
    if (st != HIMUON_OK) return st;
    std::vector<MatSpec> specs;
    if ((st = gather(nullptr, m, nullptr, n, T, dt, specs)) != HIMUON_OK) return st;
    Plan plan;
    if ((st = build_plan(specs, T, 0, dt, 0, false, plan)) != HIMUON_OK) return st;
    if (full) *full = plan.ws_full;
    if (min) *min = plan.ws_min;
    return HIMUON_OK;
}

himuon_status_t himuon_tiled_ns(const himuon_matrix_t* m, int32_t n, int32_t T, int32_t K, const float* abc,
                                himuon_dtype_t dt, float eps, void* workspace, size_t workspace_bytes,
                                void* stream) {
    himuon_status_t st = check_common(n, T, K, dt, eps);
    if (st != HIMUON_OK) return st;
    if ((st = check_abc(K, abc)) != HIMUON_OK) return st;
    std::vector<MatSpec> specs;
    if ((st = gather(nullptr, m, nullptr, n, T, dt, specs)) != HIMUON_OK) return st;
    return run(specs, T, K, abc, dt, eps, 0.f, 0.f, false, workspace, workspace_bytes, stream);
}

himuon_status_t himuon_tiled_ns_noalloc(const himuon_matrix_t* m, int32_t n, int32_t T, int32_t K,
                                        const float* abc, himuon_dtype_t dt, float eps, void* stream) {
    static_assert(HIMUON_NOALLOC_SCRATCH_BYTES == kStaticScratchBytes, "scratch size");
    himuon_status_t st = check_common(n, T, K, dt, eps);
    if (st != HIMUON_OK) return st;
    if ((st = check_abc(K, abc)) != HIMUON_OK) return st;
    std::vector<MatSpec> specs;
    if ((st = gather(nullptr, m, nullptr, n, T, dt, specs)) != HIMUON_OK) return st;
    // Size check before the device is touched: every tile of the step path
    // must fit the scratch on its own (run() repeats this plan).
    Plan plan;
    if ((st = build_plan(specs, T, K, dt, kStaticScratchBytes, true, plan)) != HIMUON_OK) return st;
    if (specs.empty()) return HIMUON_OK;
    void* scratch = nullptr;
    const hipError_t e = static_scratch(&scratch);
    if (e != hipSuccess) return hip_fail(e);
    return run(specs, T, K, abc, dt, eps, 0.f, 0.f, false, scratch, kStaticScratchBytes, stream);
}

himuon_status_t himuon_tiled_ns_schedule(const himuon_matrix_t* m, int32_t n, const int32_t* T, int32_t K,
                                         const float* abc, himuon_dtype_t dt, float eps, void* workspace,
                                         size_t workspace_bytes, void* stream) {
    if (K < 1 || K > HIMUON_MAX_STEPS || T == nullptr) return HIMUON_ERR_INVALID_ARGUMENT;
    for (int k = 0; k < K; ++k) {
        if (T[k] < 1) return HIMUON_ERR_INVALID_ARGUMENT;
        if (k > 0 && (T[k] > T[k - 1] || T[k - 1] % T[k] != 0)) return HIMUON_ERR_INVALID_ARGUMENT;
    }
    himuon_status_t st = check_common(n, T[0], K, dt, eps);
    if (st != HIMUON_OK) return st;
    if ((st = check_abc(K, abc)) != HIMUON_OK) return st;
    // validate every run (tile size) before enqueueing anything
    std::vector<std::vector<MatSpec>> runs;
    std::vector<int32_t> run_T, run_k0, run_K;
    for (int k = 0; k < K;) {
        int k1 = k;
        while (k1 < K && T[k1] == T[k]) ++k1;
        std::vector<MatSpec> specs;
        if ((st = check_common(n, T[k], k1 - k, dt, eps)) != HIMUON_OK) return st;
        if ((st = gather(nullptr, m, nullptr, n, T[k], dt, specs)) != HIMUON_OK) return st;
        Plan plan;
        if ((st = build_plan(specs, T[k], k1 - k, dt, workspace_bytes, true, plan)) != HIMUON_OK) return st;
        if (!plan.chunks.empty() && workspace == nullptr) return HIMUON_ERR_WORKSPACE;
        runs.push_back(std::move(specs));
        run_T.push_back(T[k]);
        run_k0.push_back(k);
        run_K.push_back(k1 - k);
        k = k1;
    }
    for (size_t i = 0; i < runs.size(); ++i) {
        st = run(runs[i], run_T[i], run_K[i], abc + 3 * run_k0[i], dt, eps, 0.f, 0.f, false, workspace,
                 workspace_bytes, stream, i == 0);
        if (st != HIMUON_OK) return st;
    }
    return HIMUON_OK;
}

himuon_status_t himuon_muon_step(const himuon_matrix_t* W, const himuon_matrix_t* M, const himuon_matrix_t* G,
                                 int32_t n, int32_t T, int32_t K, const float* abc, float mu, float eta,
                                 himuon_dtype_t dt, float eps, void* workspace, size_t workspace_bytes,
                                 void* stream) {
    himuon_status_t st = check_common(n, T, K, dt, eps);
    if (st != HIMUON_OK) return st;
    if ((st = check_abc(K, abc)) != HIMUON_OK) return st;
    if (!std::isfinite(mu) || !std::isfinite(eta)) return HIMUON_ERR_INVALID_ARGUMENT;
    if (n > 0 && (W == nullptr || G == nullptr || M == nullptr)) return HIMUON_ERR_INVALID_ARGUMENT;
    std::vector<MatSpec> specs;
    if ((st = gather(n > 0 ? W : nullptr, M, n > 0 ? G : nullptr, n, T, dt, specs)) != HIMUON_OK) return st;
    return run(specs, T, K, abc, dt, eps, mu, eta, true, workspace, workspace_bytes, stream);
}

himuon_status_t himuon_gram_ns_workspace(const himuon_matrix_t* m, int32_t n, himuon_dtype_t dt, size_t* full,
                                         size_t* min) {
    if (full) *full = 0;
    if (min) *min = 0;
    himuon_status_t st = check_common(n, 1, 0, dt, 0.f);
    if (st != HIMUON_OK) return st;
    std::vector<MatSpec> specs;
    const int32_t T = whole_tile(m, n);
    if (T == 0) return HIMUON_ERR_LAYOUT;
    if ((st = gather(nullptr, m, nullptr, n, T, dt, specs)) != HIMUON_OK) return st;
    Plan plan;
    if ((st = build_plan(specs, T, 1, dt, 0, false, plan, true, 0)) != HIMUON_OK) return st;
    if (full) *full = plan.ws_full;
    if (min) *min = plan.ws_min;
    return HIMUON_OK;
}

himuon_status_t himuon_gram_ns(const himuon_matrix_t* m, int32_t n, int32_t K, const float* abc, int32_t restart,
                               himuon_dtype_t dt, float eps, void* workspace, size_t workspace_bytes,
                               void* stream) {
    if (restart < 0) return HIMUON_ERR_INVALID_ARGUMENT;
    himuon_status_t st = check_common(n, 1, K, dt, eps);
    if (st != HIMUON_OK) return st;
    if ((st = check_abc(K, abc)) != HIMUON_OK) return st;
    std::vector<MatSpec> specs;
    const int32_t T = whole_tile(m, n);
    if (T == 0) return HIMUON_ERR_LAYOUT;
    if ((st = gather(nullptr, m, nullptr, n, T, dt, specs)) != HIMUON_OK) return st;
    // K = 0 is the normalisation alone, which the standard path writes
    if (K == 0) return run(specs, T, 0, abc, dt, eps, 0.f, 0.f, false, workspace, workspace_bytes, stream);
    return run_gram(specs, T, K, abc, restart >= K ? 0 : restart, dt, eps, workspace, workspace_bytes, stream);
}

himuon_status_t himuon_pair_stats_workspace(const himuon_matrix_t* a, int32_t n, size_t* bytes) {
    if (bytes == nullptr) return HIMUON_ERR_INVALID_ARGUMENT;
    int64_t total = 0;
    himuon_status_t st = pair_blocks(a, n, &total);
    if (st != HIMUON_OK) return st;
    *bytes = (size_t)total * 3 * sizeof(double);
    return HIMUON_OK;
}

himuon_status_t himuon_pair_stats(const himuon_matrix_t* a, const himuon_matrix_t* b, int32_t n, himuon_dtype_t dt,
                                  double* out, void* workspace, size_t workspace_bytes, void* stream) {
    if (dt != HIMUON_BF16 && dt != HIMUON_FP32 && dt != HIMUON_BF16_PRECISE) return HIMUON_ERR_UNSUPPORTED;
    if (n < 0) return HIMUON_ERR_INVALID_ARGUMENT;
    if (n == 0) return HIMUON_OK;
    if (a == nullptr || b == nullptr || out == nullptr) return HIMUON_ERR_INVALID_ARGUMENT;
    if ((reinterpret_cast<uintptr_t>(out) % sizeof(double)) != 0) return HIMUON_ERR_LAYOUT;
    const size_t es = elem_size(dt);
    for (int32_t i = 0; i < n; ++i) {
        himuon_status_t st = check_matrix(a[i], es);
        if (st != HIMUON_OK) return st;
        if ((st = check_matrix(b[i], es)) != HIMUON_OK) return st;
        if (a[i].rows != b[i].rows || a[i].cols != b[i].cols) return HIMUON_ERR_INVALID_ARGUMENT;
    }
    int64_t total = 0;
    himuon_status_t st = pair_blocks(a, n, &total);
    if (st != HIMUON_OK) return st;
    const size_t need = (size_t)total * 3 * sizeof(double);
    if (workspace == nullptr || workspace_bytes < need) return HIMUON_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) % sizeof(double)) != 0) return HIMUON_ERR_LAYOUT;

    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    int32_t part = 0;
    for (int32_t g0 = 0; g0 < n; g0 += kPairGroup) {
        PairArgs pa{};
        pa.n = std::min<int32_t>(kPairGroup, n - g0);
        pa.dtype = bf16_storage(dt) ? 0 : 1;
        pa.partial = reinterpret_cast<double*>(workspace);
        pa.out = out + 3 * (int64_t)g0;
        int32_t blocks = 0;
        for (int32_t k = 0; k < pa.n; ++k) {
            const himuon_matrix_t& x = a[g0 + k];
            const himuon_matrix_t& y = b[g0 + k];
            PairEntry& e = pa.e[k];
            e.a = x.ptr;
            e.b = y.ptr;
            e.lda = x.ld;
            e.ldb = y.ld;
            e.rows = (int32_t)x.rows;
            e.cols = (int32_t)x.cols;
            e.rows_per_block = pair_rows_per_block(x.rows, x.cols);
            e.nblocks = (int32_t)((x.rows + e.rows_per_block - 1) / e.rows_per_block);
            e.block_base = blocks;
            e.part_base = part;
            blocks += e.nblocks;
            part += e.nblocks;
        }
        pa.total_blocks = blocks;
        hipError_t e = launch_pair_stats(pa, s);
        if (e != hipSuccess) return hip_fail(e);
    }
    return HIMUON_OK;
}

const char* himuon_status_string(himuon_status_t s) {
    switch (s) {
        case HIMUON_OK: return "ok";
        case HIMUON_ERR_INVALID_ARGUMENT: return "invalid argument";
        case HIMUON_ERR_UNSUPPORTED: return "unsupported dtype or option";
        case HIMUON_ERR_LAYOUT: return "bad layout (alignment or size)";
        case HIMUON_ERR_OVERLAP: return "matrices overlap in memory";
        case HIMUON_ERR_WORKSPACE: return "workspace too small or missing";
        case HIMUON_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

int32_t himuon_last_hip_error(void) { return g_last_hip; }

int32_t himuon_version(void) { return 10300; }

}  // extern "C"
