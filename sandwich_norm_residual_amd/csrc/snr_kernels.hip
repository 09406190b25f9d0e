// snr_kernels.hip - gfx950 (CDNA4) kernels for row-wise RMSNorm, the fused
// dual-epsilon sandwich tail, and the tail's two halves.
//
// What is computed ("RMSNorm and the dual-epsilon sandwich", Muser book
// chapter 12, and Hesper's "RMSNorm Layer" page):
//   plain (Muser 12.1):      y = x / sqrt(mean(x^2) + eps) * gamma
//   tail (Muser 12.2, 12.4.3):
//       h = r + a / sqrt(mean(a^2) + eps_post) * gamma_post
//       y = h / sqrt(mean(h^2) + eps_pre) * gamma_pre
//   norm_then_add (Hesper rmsNormThenAdd[ThenBroadcastScale]Kernel):
//       out = (a / sqrt(mean(a^2) + eps) * gamma + r) * scale
//   add_then_norm (Hesper residualAddRmsNormKernel):
//       s = a + b;  y = s / sqrt(mean(s^2) + eps) * gamma   (writes s and y)
// An intermediate that a later norm reads (the tail's h, add_then_norm's s)
// is stored rounded to the storage type, and the later norm works from its
// f32 value, so y carries one rounding (normalising the rounded copy would
// add the rounding of the row's largest element to every output). For f32
// storage the two are the same.
//
// Design (HBM-bound, no contraction, so no MFMA):
// * Each row is read from HBM exactly once: every lane loads its share of the
//   row into registers with coalesced 128-bit loads (the n % W elements past
//   the last whole vector one at a time), the sum of squares is reduced, and
//   the normalise pass works from those registers. The tail also keeps h in
//   registers for its second reduction, so a and r are read once and h and y
//   written once.
// * Sums of squares accumulate in f32. Inside a wavefront the reduction uses
//   DPP lane moves (quad permutes and row mirrors) and one ds_swizzle, then a
//   readlane pair across the two 32-lane halves; across wavefronts of one
//   row there is a single LDS exchange with one barrier. The summation order
//   is fixed, so results are bit-reproducible.
// * Row-tile kernel: G lanes per row. G <= 64 packs 64/G rows into each
//   wavefront (small rows, no LDS and no barrier); G > 64 spans G/64
//   wavefronts of one workgroup.
// * Split-row kernels for very wide rows (one workgroup per chunk of a row,
//   partial sums combined through device memory) are in snr_split.hip.
// * Multi-pass kernels for rows so wide that their chunks cannot all be
//   co-resident: partial sums through device memory (rows read twice).
// * Stores of outputs and loads of row data are non-temporal (each byte is
//   touched once); gains use ordinary cached loads (every row re-reads them).
#include "snr_device.h"

namespace snr {
namespace {

// ---------------------------------------------------------------------------
// One row, shared by the row-tile and several-segment kernels.
//
// The lane holds vectors vbase + k*vstride (k < VPT) of the row and, when
// `sown`, the remainder elements sbase + q*sstride (q < EX) that follow the
// last whole vector. `reduce(s, which)` turns this lane's partial sum of
// squares into the row total (which = 0 for the first norm, 1 for the
// second); every lane of the row must call it.
//
// LATE (tail and norm_then_add): r is loaded while forming the output
// instead of together with a, so only one row stream is held in registers.
// add_then_norm always holds only the sum s = a + b.
// EARLY: the gains are loaded with the row (see below).
// ---------------------------------------------------------------------------
template <int OP, int ST, int VPT, int EX, bool LATE, bool EARLY, class Reduce>
__device__ __forceinline__ void process_row(const RowArgs &p, int64_t off,
                                            bool live, int vbase, int vstride,
                                            int sbase, int sstride, bool sown,
                                            Reduce reduce) {
    using C = Codec<ST>;
    using T = typename C::T;
    constexpr int W = C::W;
    constexpr bool HOLD_R = (OP == OP_TAIL || OP == OP_NORM_ADD) && !LATE;
    const int nv = p.nv;
    const int rem = p.rem;
    const int tail0 = nv * W;  // first remainder element of the row

    float v0[VPT][W], e0[EX];
    float v1[HOLD_R ? VPT : 1][W], e1[HOLD_R ? EX : 1];
    (void)v1;
    (void)e1;

    const T *x0 = static_cast<const T *>(p.x0) + off;
    const T *x1 = static_cast<const T *>(p.x1) + off;
    (void)x1;
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        const int i = vbase + k * vstride;
        if (live && i < nv) C::load_nt(x0, i, v0[k]); else zero(v0[k]);
    }
#pragma unroll
    for (int q = 0; q < EX; ++q) {
        const int j = sbase + q * sstride;
        e0[q] = (live && sown && j < rem) ? C::load1_nt(x0, tail0 + j) : 0.0f;
    }
    if constexpr (HOLD_R) {
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            const int i = vbase + k * vstride;
            if (live && i < nv) C::load_nt(x1, i, v1[k]); else zero(v1[k]);
        }
#pragma unroll
        for (int q = 0; q < EX; ++q) {
            const int j = sbase + q * sstride;
            e1[q] = (live && sown && j < rem) ? C::load1_nt(x1, tail0 + j)
                                              : 0.0f;
        }
    }
    // Gains are loaded one vector just before its use, or with the row (PRE)
    // where registers allow: always for norm_then_add (measured 53.5 ->
    // 52.6 us at 4096 x 6656 f32), and for the other operations when the
    // launch asks for it (EARLY). The vector memory counter retires in issue
    // order and counts stores too, so a gain loaded between two stores is
    // waited for together with the first store. For a few rows the step is
    // one memory round trip after another and loading the gains with the
    // row takes one of them away (1 row x 6656 f32: tail 3.38 -> 3.24 us,
    // plain 2.36 -> 2.26 us); over many rows the late loads measured faster
    // (4096 rows: tail 73.0 -> 75.7 us with the gains loaded with the row).
    using V = typename C::vec;
    constexpr bool PRE = (OP == OP_NORM_ADD || EARLY) && !LATE && VPT <= 4;
    constexpr int NG = OP == OP_TAIL ? 2 : 1;
    const T *gp[2] = {static_cast<const T *>(p.g0),
                      static_cast<const T *>(OP == OP_TAIL ? p.g1 : p.g0)};
    V gq[NG][PRE ? VPT : 1];   // as stored, decoded where used
    float ge[NG][PRE ? EX : 1];
    (void)gq;
    (void)ge;
    if constexpr (PRE) {
#pragma unroll
        for (int w = 0; w < NG; ++w) {
#pragma unroll
            for (int k = 0; k < VPT; ++k) {
                const int i = vbase + k * vstride;
                gq[w][k] = (live && i < nv) ? C::load_raw(gp[w], i) : V{};
            }
#pragma unroll
            for (int q = 0; q < EX; ++q) {
                const int j = sbase + q * sstride;
                ge[w][q] = (live && sown && j < rem) ? C::load1(gp[w], tail0 + j)
                                                     : 0.0f;
            }
        }
    }
    // gain w's values at vector slot k (index i) and remainder slot q (j)
    auto gain = [&](int w, int k, int i, float(&g)[W]) {
        if constexpr (PRE) C::decode(gq[w][k], g);
        else C::load(gp[w], i, g);
    };
    auto gain1 = [&](int w, int q, int j) {
        if constexpr (PRE) return ge[w][q];
        else return C::load1(gp[w], tail0 + j);
    };

    T *out0 = static_cast<T *>(p.out0) + off;
    if constexpr (OP == OP_ADD_NORM) {
        // s = a + b: stored rounded to storage, kept in f32 for the norm.
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            const int i = vbase + k * vstride;
            if (live && i < nv) {
                float b[W];
                C::load_nt(x1, i, b);
#pragma unroll
                for (int e = 0; e < W; ++e) v0[k][e] = v0[k][e] + b[e];
                C::store_nt(out0, i, v0[k]);
            }
        }
#pragma unroll
        for (int q = 0; q < EX; ++q) {
            const int j = sbase + q * sstride;
            if (live && sown && j < rem) {
                e0[q] = e0[q] + C::load1_nt(x1, tail0 + j);
                C::store1_nt(out0, tail0 + j, e0[q]);
            }
        }
    }

    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < VPT; ++k) s += sumsq<W>(v0[k]);
#pragma unroll
    for (int q = 0; q < EX; ++q) s = fmaf(e0[q], e0[q], s);
    const float inv0 = inv_rms(reduce(s, 0), p.n, p.eps0);

    if constexpr (OP == OP_PLAIN || OP == OP_ADD_NORM) {
        // y = x * inv * gamma (add_then_norm: x is the stored sum)
        T *y = static_cast<T *>(OP == OP_PLAIN ? p.out0 : p.out1) + off;
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            const int i = vbase + k * vstride;
            if (live && i < nv) {
                float g[W], o[W];
                gain(0, k, i, g);
#pragma unroll
                for (int e = 0; e < W; ++e) o[e] = v0[k][e] * inv0 * g[e];
                C::store_nt(y, i, o);
            }
        }
#pragma unroll
        for (int q = 0; q < EX; ++q) {
            const int j = sbase + q * sstride;
            if (live && sown && j < rem)
                C::store1_nt(y, tail0 + j, e0[q] * inv0 * gain1(0, q, j));
        }
    } else {
        // h = r + a * inv * gamma0, stored rounded and kept in f32 registers
        // (v1/e1, or v0/e0 once a is consumed when r is late) for the second
        // norm. norm_then_add stores h * scale.
        const float scale = (OP == OP_NORM_ADD && p.scale) ? *p.scale : 1.0f;
        float(*hv)[W] = LATE ? v0 : v1;
        float *he = LATE ? e0 : e1;
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            const int i = vbase + k * vstride;
            if (live && i < nv) {
                float g[W], rr[W];
                gain(0, k, i, g);
                if constexpr (LATE) {
                    C::load_nt(x1, i, rr);
                } else {
#pragma unroll
                    for (int e = 0; e < W; ++e) rr[e] = v1[k][e];
                }
                if constexpr (OP == OP_TAIL) {
#pragma unroll
                    for (int e = 0; e < W; ++e)
                        hv[k][e] = fmaf(v0[k][e] * inv0, g[e], rr[e]);
                    C::store_nt(out0, i, hv[k]);
                } else {
                    float o[W];
#pragma unroll
                    for (int e = 0; e < W; ++e)
                        o[e] = fmaf(v0[k][e] * inv0, g[e], rr[e]) * scale;
                    C::store_nt(out0, i, o);
                }
            }
        }
#pragma unroll
        for (int q = 0; q < EX; ++q) {
            const int j = sbase + q * sstride;
            if (live && sown && j < rem) {
                const float rr = LATE ? C::load1_nt(x1, tail0 + j) : e1[q];
                const float h = fmaf(e0[q] * inv0, gain1(0, q, j), rr);
                if constexpr (OP == OP_TAIL) {
                    he[q] = h;
                    C::store1_nt(out0, tail0 + j, he[q]);
                } else {
                    C::store1_nt(out0, tail0 + j, h * scale);
                }
            }
        }
        if constexpr (OP == OP_TAIL) {
            float sh = 0.0f;
#pragma unroll
            for (int k = 0; k < VPT; ++k) sh += sumsq<W>(hv[k]);
#pragma unroll
            for (int q = 0; q < EX; ++q) sh = fmaf(he[q], he[q], sh);
            const float inv1 = inv_rms(reduce(sh, 1), p.n, p.eps1);

            T *out1 = static_cast<T *>(p.out1) + off;
#pragma unroll
            for (int k = 0; k < VPT; ++k) {
                const int i = vbase + k * vstride;
                if (live && i < nv) {
                    float g[W], o[W];
                    gain(1, k, i, g);
#pragma unroll
                    for (int e = 0; e < W; ++e) o[e] = hv[k][e] * inv1 * g[e];
                    C::store_nt(out1, i, o);
                }
            }
#pragma unroll
            for (int q = 0; q < EX; ++q) {
                const int j = sbase + q * sstride;
                if (live && sown && j < rem)
                    C::store1_nt(out1, tail0 + j, he[q] * inv1 * gain1(1, q, j));
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Row-tile kernel: G lanes per row, VPT vectors per lane. G <= 64 packs
// 64/G rows into each wavefront; G > 64 is one row per workgroup.
// ---------------------------------------------------------------------------
// Remainder elements each lane may hold: a row has at most W - 1 of them.
template <int ST, int G>
constexpr int rowtile_extra() {
    return (Codec<ST>::W - 1 + G - 1) / G;
}

// r is loaded late where holding two row streams would not fit the 128
// registers a lane of a 1024-lane workgroup may use.
template <int OP, int ST, int G, int VPT>
constexpr bool rowtile_late() {
    return (OP == OP_TAIL || OP == OP_NORM_ADD) && G == 1024 &&
           VPT * Codec<ST>::W >= 64;
}

// The row tiles that also have a form with the gains loaded with the row:
// a register tile that leaves room for the gains, and an operation that does
// not load them with the row already.
template <int OP, int ST, int G, int VPT>
constexpr bool rowtile_has_early() {
    return OP != OP_NORM_ADD && VPT <= 4 && !rowtile_late<OP, ST, G, VPT>();
}

template <int OP, int ST, int G, int VPT, bool EARLY>
__global__ void __launch_bounds__(rowtile_block<G>())
rowtile_kernel(RowArgs p, int64_t row0, int64_t row_end) {
    constexpr int BLOCK = rowtile_block<G>();
    constexpr int RPB = BLOCK / G;
    constexpr int WPR = G > 64 ? G / 64 : 1;
    __shared__ float red[2][WPR];

    const int sub = threadIdx.x & (G - 1);
    const int64_t row = row0 + (int64_t)blockIdx.x * RPB + threadIdx.x / G;
    const bool live = row < row_end;
    const int64_t off = live ? row * (int64_t)p.n : 0;
    process_row<OP, ST, VPT, rowtile_extra<ST, G>(),
                rowtile_late<OP, ST, G, VPT>(), EARLY>(
        p, off, live, sub, G, sub, G, true,
        [&](float s, int which) { return row_total<G>(s, red[which]); });
}

// Several RMSNorms in one launch (the same row tile as above): each row
// finds its segment in the table and normalises with that segment's
// tensors and epsilon.
template <int ST, int G, int VPT, bool EARLY>
__global__ void __launch_bounds__(rowtile_block<G>())
multi_kernel(MultiArgs m, int64_t row0, int64_t row_end) {
    constexpr int BLOCK = rowtile_block<G>();
    constexpr int RPB = BLOCK / G;
    constexpr int WPR = G > 64 ? G / 64 : 1;
    __shared__ float red[2][WPR];

    const int sub = threadIdx.x & (G - 1);
    const int64_t row = row0 + (int64_t)blockIdx.x * RPB + threadIdx.x / G;
    const bool live = row < row_end;
    int seg = 0;
    while (seg + 1 < m.count && row >= m.row_start[seg + 1]) ++seg;
    RowArgs p{};
    p.x0 = m.x[seg];
    p.g0 = m.g[seg];
    p.out0 = m.y[seg];
    p.eps0 = m.eps[seg];
    p.n = m.n;
    p.nv = m.nv;
    p.rem = m.rem;
    const int64_t off = live ? (row - m.row_start[seg]) * (int64_t)m.n : 0;
    process_row<OP_PLAIN, ST, VPT, rowtile_extra<ST, G>(), false, EARLY>(
        p, off, live, sub, G, sub, G, true,
        [&](float s, int which) { return row_total<G>(s, red[which]); });
}

// ---------------------------------------------------------------------------
// Multi-pass kernels for rows too wide to keep on chip (more chunks than
// co-resident workgroups). Each pass is a plain grid; partial sums go
// through device memory and are added in chunk order, so results stay
// deterministic. These passes read a row more than once:
//   plain:         partial(x) -> combine -> y = x * inv * g          (x twice)
//   tail:          partial(a) -> combine -> h = r + a*inv*gp, partial(h)
//                  -> combine -> y = h * inv_h * gq          (a and h twice)
//   norm_then_add: partial(a) -> combine -> out = (a*inv*g + r) * scale
//   add_then_norm: s = a + b, partial(s) -> combine -> y = s * inv * g
// ---------------------------------------------------------------------------
// dst = src * inv * gain.
template <int ST>
__global__ void __launch_bounds__(MB)
pass_scale(RowArgs p, const void *src, const void *gain, void *dst,
           int64_t row0, int chunks, const float *inv) {
    using C = Codec<ST>;
    using T = typename C::T;
    constexpr int W = C::W;
    const int chunk = (int)(blockIdx.x % (unsigned)chunks);
    const int64_t rl = blockIdx.x / (unsigned)chunks;
    const int64_t off = (row0 + rl) * (int64_t)p.n;
    const T *x = static_cast<const T *>(src) + off;
    const T *g = static_cast<const T *>(gain);
    T *y = static_cast<T *>(dst) + off;
    const float r = inv[rl];
    for_chunk<ST>(
        p, chunk, chunks,
        [&](int i) {
            float v[W], gv[W], o[W];
            C::load_nt(x, i, v);
            C::load(g, i, gv);
#pragma unroll
            for (int e = 0; e < W; ++e) o[e] = v[e] * r * gv[e];
            C::store_nt(y, i, o);
        },
        [&](int j) { C::store1_nt(y, j, C::load1_nt(x, j) * r * C::load1(g, j)); });
}

// The elementwise middle pass, with the chunk's sum of squares in
// part[rl * chunks + c] when a later norm needs it:
//   tail:          h = r + a * inv * gamma0                        (+ part)
//   norm_then_add: out = (a * inv * gamma0 + r) * scale
//   add_then_norm: s = a + b                                       (+ part)
// The sums of squares are of the f32 values; the stored copies are rounded
// to storage. The last pass reads those stored copies, so in 16-bit storage
// y = (stored h) * (1/rms of the f32 h) * gain carries two roundings here,
// against one in the register-resident kernels.
template <int OP, int ST>
__global__ void __launch_bounds__(MB)
pass_fuse(RowArgs p, int64_t row0, int chunks, const float *inv, float *part) {
    using C = Codec<ST>;
    using T = typename C::T;
    constexpr int W = C::W;
    __shared__ float red[MB / 64];
    const int chunk = (int)(blockIdx.x % (unsigned)chunks);
    const int64_t rl = blockIdx.x / (unsigned)chunks;
    const int64_t off = (row0 + rl) * (int64_t)p.n;
    const T *a = static_cast<const T *>(p.x0) + off;
    const T *r = static_cast<const T *>(p.x1) + off;
    const T *g = static_cast<const T *>(p.g0);
    T *o = static_cast<T *>(p.out0) + off;
    const float ia = OP == OP_ADD_NORM ? 0.0f : inv[rl];
    const float scale = (OP == OP_NORM_ADD && p.scale) ? *p.scale : 1.0f;
    auto fuse = [&](float av, float rv, float gv) {
        if constexpr (OP == OP_ADD_NORM) return av + rv;
        else if constexpr (OP == OP_TAIL) return fmaf(av * ia, gv, rv);
        else return fmaf(av * ia, gv, rv) * scale;
    };
    float s = 0.0f;
    for_chunk<ST>(
        p, chunk, chunks,
        [&](int i) {
            float av[W], rv[W], gv[W], hv[W];
            C::load_nt(a, i, av);
            C::load_nt(r, i, rv);
            if constexpr (OP != OP_ADD_NORM) C::load(g, i, gv);
            else zero(gv);
#pragma unroll
            for (int e = 0; e < W; ++e) hv[e] = fuse(av[e], rv[e], gv[e]);
            C::store_nt(o, i, hv);
            s += sumsq<W>(hv);
        },
        [&](int j) {
            const float gv = OP == OP_ADD_NORM ? 0.0f : C::load1(g, j);
            const float hv = fuse(C::load1_nt(a, j), C::load1_nt(r, j), gv);
            C::store1_nt(o, j, hv);
            s = fmaf(hv, hv, s);
        });
    if constexpr (OP != OP_NORM_ADD) {
        const float t = block_total(s, red);
        if (threadIdx.x == 0) part[rl * chunks + chunk] = t;
    }
}

__global__ void fill_kernel(unsigned int *p, int64_t words, unsigned int v) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
         i < words; i += stride)
        p[i] = v;
}

// ---------------------------------------------------------------------------
// Launchers and the kernel table
// ---------------------------------------------------------------------------
// Launches of at most kEarlyBlocks workgroups use the form with the gains
// loaded with the row where there is one. Measured over 1 to 256 rows of
// 6656 f32 (one row per workgroup; steps replayed from a HIP graph): faster
// for every operation up to 16 rows (the tail 3.60 -> 3.47 us at 16 rows),
// even at 32 (4.16 -> 4.10 us in one run, 4.04 -> 4.11 us in another),
// slower for the tail and the plain norm from 64 rows on (4.55 -> 4.81 us,
// 3.17 -> 3.27 us). With several rows per workgroup the count that matters
// is the same: the per-head query and key norms of one token (52 + 8 rows
// of 128 f32, two workgroups) took 2.60 -> 2.26 us in one several-segment
// launch and 4.19 -> 3.55 us in two launches.
template <int OP, int ST, int G, int VPT>
hipError_t launch_rowtile(const RowArgs &p, int64_t row0, int64_t nrows,
                          hipStream_t stream) {
    constexpr int BLOCK = rowtile_block<G>();
    constexpr int RPB = BLOCK / G;
    const int64_t blocks = (nrows + RPB - 1) / RPB;
    const dim3 grid((unsigned int)blocks);
    if constexpr (rowtile_has_early<OP, ST, G, VPT>()) {
        if (blocks <= kEarlyBlocks) {
            hipLaunchKernelGGL((rowtile_kernel<OP, ST, G, VPT, true>), grid,
                               dim3(BLOCK), 0, stream, p, row0, row0 + nrows);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((rowtile_kernel<OP, ST, G, VPT, false>), grid,
                       dim3(BLOCK), 0, stream, p, row0, row0 + nrows);
    return hipGetLastError();
}

template <int OP, int ST, int G, int VPT>
int64_t resident_rowtile() {
    return resident_blocks<&rowtile_kernel<OP, ST, G, VPT, false>>(
        rowtile_block<G>());
}

template <int OP, int ST, int G, int VPT>
hipError_t occupancy_rowtile(int *blocks_per_cu) {
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(
        blocks_per_cu, rowtile_kernel<OP, ST, G, VPT, false>,
        rowtile_block<G>(), 0);
}

template <int ST, int G, int VPT>
hipError_t launch_multi(const MultiArgs &m, int64_t row0, int64_t nrows,
                        hipStream_t stream) {
    constexpr int BLOCK = rowtile_block<G>();
    constexpr int RPB = BLOCK / G;
    const int64_t blocks = (nrows + RPB - 1) / RPB;
    const dim3 grid((unsigned int)blocks);
    if constexpr (rowtile_has_early<OP_PLAIN, ST, G, VPT>()) {
        if (blocks <= kEarlyBlocks) {
            hipLaunchKernelGGL((multi_kernel<ST, G, VPT, true>), grid,
                               dim3(BLOCK), 0, stream, m, row0, row0 + nrows);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((multi_kernel<ST, G, VPT, false>), grid, dim3(BLOCK), 0,
                       stream, m, row0, row0 + nrows);
    return hipGetLastError();
}

template <int OP, int ST, int G, int VPT>
constexpr MultiLaunch multi_for() {
    if constexpr (OP == OP_PLAIN) return &launch_multi<ST, G, VPT>;
    else return nullptr;
}

// Multi-pass launch over rows [row0, row0 + nrows): scratch holds
// nrows * chunks partial sums followed by nrows inverse norms.
template <int OP, int ST>
hipError_t launch_multipass(const RowArgs &p, float *scratch, int64_t row0,
                            int64_t nrows, int chunks, hipStream_t stream) {
    float *part = scratch;
    float *inv = scratch + nrows * (int64_t)chunks;
    const dim3 grid((unsigned int)(nrows * chunks));
    const dim3 rows_grid((unsigned int)nrows);
    const float *cinv = inv;
    if constexpr (OP == OP_ADD_NORM) {
        hipLaunchKernelGGL((pass_fuse<OP, ST>), grid, dim3(MB), 0, stream, p,
                           row0, chunks, cinv, part);
        hipLaunchKernelGGL(pass_combine, rows_grid, dim3(MB), 0, stream,
                           (const float *)part, chunks, p.n, p.eps0, inv);
        hipLaunchKernelGGL(pass_scale<ST>, grid, dim3(MB), 0, stream, p,
                           (const void *)p.out0, p.g0, p.out1, row0, chunks,
                           cinv);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(pass_sumsq<ST>, grid, dim3(MB), 0, stream, p, p.x0,
                       row0, chunks, part);
    hipLaunchKernelGGL(pass_combine, rows_grid, dim3(MB), 0, stream,
                       (const float *)part, chunks, p.n, p.eps0, inv);
    if constexpr (OP == OP_PLAIN) {
        hipLaunchKernelGGL(pass_scale<ST>, grid, dim3(MB), 0, stream, p, p.x0,
                           p.g0, p.out0, row0, chunks, cinv);
    } else {
        hipLaunchKernelGGL((pass_fuse<OP, ST>), grid, dim3(MB), 0, stream, p,
                           row0, chunks, cinv, part);
        if constexpr (OP == OP_TAIL) {
            hipLaunchKernelGGL(pass_combine, rows_grid, dim3(MB), 0, stream,
                               (const float *)part, chunks, p.n, p.eps1, inv);
            hipLaunchKernelGGL(pass_scale<ST>, grid, dim3(MB), 0, stream, p,
                               (const void *)p.out0, p.g1, p.out1, row0,
                               chunks, cinv);
        }
    }
    return hipGetLastError();
}

// Plain row tiles on the automatic menu also get the several-segment
// launcher; the sweep-only shapes do not.
#define SNR_RT_M(OP, ST, G, VPT, M)                                         \
    KernelEntry{OP, ST, Codec<ST>::W, KIND_ROWTILE, G, VPT,                 \
                rowtile_block<G>(), &launch_rowtile<OP, ST, G, VPT>,        \
                nullptr, &occupancy_rowtile<OP, ST, G, VPT>, nullptr, M,    \
                &resident_rowtile<OP, ST, G, VPT>}
#define SNR_RT(OP, ST, G, VPT) SNR_RT_M(OP, ST, G, VPT, nullptr)
#define SNR_RT_A(OP, ST, G, VPT)                                            \
    SNR_RT_M(OP, ST, G, VPT, (multi_for<OP, ST, G, VPT>()))
#define SNR_MULTI(OP, ST)                                                   \
    KernelEntry{OP, ST, Codec<ST>::W, KIND_MULTIPASS, MB, MVPT, MB, nullptr, \
                nullptr, nullptr, &launch_multipass<OP, ST>, nullptr}

// The shapes the automatic choice can reach for one (operation, storage):
// sub-wavefront groups with 4 vectors per lane, then one row per workgroup
// with the smallest register tile that holds about two vectors per lane
// (registers are allocated for every slot of a tile, used or not, and
// occupancy follows them), then multi-pass (the split-row kernels have a
// table of their own, snr_split.hip).
#define SNR_AUTO_SHAPES(OP, ST)                                             \
    SNR_RT_A(OP, ST, 1, 4), SNR_RT_A(OP, ST, 2, 4), SNR_RT_A(OP, ST, 4, 4), \
    SNR_RT_A(OP, ST, 8, 4), SNR_RT_A(OP, ST, 16, 4),                        \
    SNR_RT_A(OP, ST, 32, 4), SNR_RT_A(OP, ST, 128, 2),                      \
    SNR_RT_A(OP, ST, 128, 8), SNR_RT_A(OP, ST, 256, 2),                     \
    SNR_RT_A(OP, ST, 256, 4), SNR_RT_A(OP, ST, 512, 2),                     \
    SNR_RT_A(OP, ST, 512, 4), SNR_RT_A(OP, ST, 1024, 1),                    \
    SNR_RT_A(OP, ST, 1024, 2), SNR_RT_A(OP, ST, 1024, 4),                   \
    SNR_RT_A(OP, ST, 1024, 8), SNR_MULTI(OP, ST)

// Further shapes, reachable only by forcing (shape sweeps and tests).
#define SNR_SWEEP_SHAPES(OP, ST)                                            \
    SNR_RT(OP, ST, 64, 2), SNR_RT(OP, ST, 64, 4), SNR_RT(OP, ST, 64, 8),    \
    SNR_RT(OP, ST, 64, 16), SNR_RT(OP, ST, 128, 13), SNR_RT(OP, ST, 128, 16), \
    SNR_RT(OP, ST, 256, 7), SNR_RT(OP, ST, 256, 8), SNR_RT(OP, ST, 256, 16), \
    SNR_RT(OP, ST, 512, 8), SNR_RT(OP, ST, 512, 16)

// 1024 lanes x 16 vectors only for 4-wide f32 rows: 8-wide 16-bit rows would
// need 128 registers for the row alone (the tail and norm_then_add hold a/h
// only, with r loaded late).
const KernelEntry kTable[] = {
    SNR_AUTO_SHAPES(OP_PLAIN, ST_F32),    SNR_SWEEP_SHAPES(OP_PLAIN, ST_F32),
    SNR_RT_A(OP_PLAIN, ST_F32, 1024, 16),
    SNR_AUTO_SHAPES(OP_PLAIN, ST_BF16),   SNR_SWEEP_SHAPES(OP_PLAIN, ST_BF16),
    SNR_AUTO_SHAPES(OP_PLAIN, ST_F16),
    SNR_AUTO_SHAPES(OP_TAIL, ST_F32),     SNR_SWEEP_SHAPES(OP_TAIL, ST_F32),
    SNR_RT(OP_TAIL, ST_F32, 1024, 16),
    SNR_AUTO_SHAPES(OP_TAIL, ST_BF16),    SNR_AUTO_SHAPES(OP_TAIL, ST_F16),
    SNR_AUTO_SHAPES(OP_NORM_ADD, ST_F32), SNR_RT(OP_NORM_ADD, ST_F32, 1024, 16),
    SNR_AUTO_SHAPES(OP_NORM_ADD, ST_BF16), SNR_AUTO_SHAPES(OP_NORM_ADD, ST_F16),
    SNR_AUTO_SHAPES(OP_ADD_NORM, ST_F32), SNR_RT(OP_ADD_NORM, ST_F32, 1024, 16),
    SNR_AUTO_SHAPES(OP_ADD_NORM, ST_BF16), SNR_AUTO_SHAPES(OP_ADD_NORM, ST_F16),
};

}  // namespace

const KernelEntry *kernel_table(int *count) {
    *count = (int)(sizeof(kTable) / sizeof(kTable[0]));
    return kTable;
}

hipError_t fill_words(void *p, int64_t words, unsigned int value,
                      hipStream_t stream) {
    if (words <= 0) return hipSuccess;
    int64_t blocks = (words + 255) / 256;
    if (blocks > 1024) blocks = 1024;
    hipLaunchKernelGGL(fill_kernel, dim3((unsigned int)blocks), dim3(256), 0,
                       stream, static_cast<unsigned int *>(p), words, value);
    return hipGetLastError();
}

}  // namespace snr
