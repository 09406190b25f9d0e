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
// is normalised as it is stored: rounded to the storage type first (the
// identity for f32).
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
// * Split-row kernel for very wide rows: one workgroup per chunk of a row. A
//   workgroup publishes its chunk's partial sum to device memory, waits for
//   the other chunks of its row, adds the partials in chunk order and
//   normalises its chunk from registers (no second read of the row). The
//   grid is a cooperative launch (every workgroup co-resident) of `groups`
//   x `chunks` workgroups; workgroup (g, c) handles chunk c of rows g,
//   g + groups, g + 2 groups, ... in order, so a wait only ever depends on
//   resident workgroups that are working on the same row.
// * Multi-pass kernels for rows so wide that their chunks cannot all be
//   co-resident: partial sums through device memory (rows read twice).
// * Stores of outputs and loads of row data are non-temporal (each byte is
//   touched once); gains use ordinary cached loads (every row re-reads them).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <type_traits>

#include "snr_internal.h"

namespace snr {
namespace {

// ---------------------------------------------------------------------------
// Storage codecs. Rows are moved with 128-bit accesses: W elements per
// vector (4 f32, or 8 bf16/f16). The vector types carry only element
// alignment: gfx950 performs dwordx4 accesses at any 4-byte (f32) or 2-byte
// (16-bit types) boundary, so rows whose start is not 16-byte aligned (odd
// n, offset views) still use 128-bit accesses. The n % W elements after a
// row's last whole vector are moved one at a time.
// `round` rounds an f32 value to the storage type and back (exact decode).
// ---------------------------------------------------------------------------
template <int ST>
struct Codec;

template <>
struct Codec<ST_F32> {
    using T = float;
    static constexpr int W = 4;
    typedef float vec __attribute__((ext_vector_type(4), aligned(4)));
    // one 128-bit vector as stored, and its values
    __device__ static vec load_raw_nt(const T *row, int i) {
        return __builtin_nontemporal_load(reinterpret_cast<const vec *>(row) + i);
    }
    __device__ static void decode(const vec q, float (&v)[4]) {
        v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
    }
    __device__ static void load_nt(const T *row, int i, float (&v)[4]) {
        const vec q = __builtin_nontemporal_load(
            reinterpret_cast<const vec *>(row) + i);
        v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
    }
    __device__ static void load(const T *base, int i, float (&v)[4]) {
        const vec q = reinterpret_cast<const vec *>(base)[i];
        v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
    }
    __device__ static void store_nt(T *row, int i, const float (&v)[4]) {
        const vec q = {v[0], v[1], v[2], v[3]};
        __builtin_nontemporal_store(q, reinterpret_cast<vec *>(row) + i);
    }
    __device__ static float load1_nt(const T *row, int j) {
        return __builtin_nontemporal_load(row + j);
    }
    __device__ static float load1(const T *base, int j) { return base[j]; }
    __device__ static void store1_nt(T *row, int j, float v) {
        __builtin_nontemporal_store(v, row + j);
    }
    __device__ static float round(float v) { return v; }
};

// Two 16-bit values per 32-bit word, element 2k in the low half.
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// bf16 -> f32 is exact (a bf16 is the upper half of an f32); f32 -> bf16
// rounds to nearest even (gfx950's v_cvt_pk_bf16_f32).
struct BF16Bits {
    __device__ static float lo(unsigned int w) {
        return __uint_as_float(w << 16);
    }
    __device__ static float hi(unsigned int w) {
        return __uint_as_float(w & 0xFFFF0000u);
    }
    __device__ static unsigned int pack(float a, float b) {
        const f32x2 f = {a, b};
        return __builtin_bit_cast(unsigned int,
                                  __builtin_convertvector(f, bf16x2));
    }
    __device__ static float one(unsigned short b) {
        return __uint_as_float((unsigned int)b << 16);
    }
    __device__ static unsigned short enc(float v) {
        return __builtin_bit_cast(unsigned short, (__bf16)v);
    }
};

// f16 -> f32 is exact; f32 -> f16 rounds to nearest even.
struct F16Bits {
    __device__ static float lo(unsigned int w) {
        return (float)__builtin_bit_cast(f16x2, w).x;
    }
    __device__ static float hi(unsigned int w) {
        return (float)__builtin_bit_cast(f16x2, w).y;
    }
    __device__ static unsigned int pack(float a, float b) {
        const f32x2 f = {a, b};
        return __builtin_bit_cast(unsigned int,
                                  __builtin_convertvector(f, f16x2));
    }
    __device__ static float one(unsigned short b) {
        return (float)__builtin_bit_cast(_Float16, b);
    }
    __device__ static unsigned short enc(float v) {
        return __builtin_bit_cast(unsigned short, (_Float16)v);
    }
};

template <class B>
struct Codec16 {
    using T = unsigned short;
    static constexpr int W = 8;
    typedef unsigned int vec __attribute__((ext_vector_type(4), aligned(2)));
    __device__ static void unpack(const vec q, float (&v)[8]) {
        v[0] = B::lo(q.x); v[1] = B::hi(q.x);
        v[2] = B::lo(q.y); v[3] = B::hi(q.y);
        v[4] = B::lo(q.z); v[5] = B::hi(q.z);
        v[6] = B::lo(q.w); v[7] = B::hi(q.w);
    }
    __device__ static void load_nt(const T *row, int i, float (&v)[8]) {
        unpack(__builtin_nontemporal_load(reinterpret_cast<const vec *>(row) + i),
               v);
    }
    // one 128-bit vector as stored, and its values
    __device__ static vec load_raw_nt(const T *row, int i) {
        return __builtin_nontemporal_load(reinterpret_cast<const vec *>(row) + i);
    }
    __device__ static void decode(const vec q, float (&v)[8]) { unpack(q, v); }
    __device__ static void load(const T *base, int i, float (&v)[8]) {
        unpack(reinterpret_cast<const vec *>(base)[i], v);
    }
    __device__ static void store_nt(T *row, int i, const float (&v)[8]) {
        const vec q = {B::pack(v[0], v[1]), B::pack(v[2], v[3]),
                       B::pack(v[4], v[5]), B::pack(v[6], v[7])};
        __builtin_nontemporal_store(q, reinterpret_cast<vec *>(row) + i);
    }
    __device__ static float load1_nt(const T *row, int j) {
        return B::one(__builtin_nontemporal_load(row + j));
    }
    __device__ static float load1(const T *base, int j) {
        return B::one(base[j]);
    }
    __device__ static void store1_nt(T *row, int j, float v) {
        __builtin_nontemporal_store(B::enc(v), row + j);
    }
    __device__ static float round(float v) { return B::one(B::enc(v)); }
};

template <>
struct Codec<ST_BF16> : Codec16<BF16Bits> {};
template <>
struct Codec<ST_F16> : Codec16<F16Bits> {};

// ---------------------------------------------------------------------------
// Reductions
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(
        0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of G lanes (G a power of two, 1..64). Every lane of
// a group ends with the same bits: each step adds a value and its partner's,
// and f32 addition is commutative. Must be called with all 64 lanes active.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
    if constexpr (G >= 2) v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]: lane ^ 1
    if constexpr (G >= 4) v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]: lane ^ 2
    if constexpr (G >= 8) v += dpp<0x141>(v);  // row_half_mirror: 8-lane halves
    if constexpr (G >= 16) v += dpp<0x140>(v); // row_mirror: 16-lane rows
    if constexpr (G >= 32)                     // swap 16-lane rows in each 32
        v += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v),
                                                         0x401F));
    if constexpr (G >= 64)                     // the two 32-lane halves
        v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0)) +
            __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    return v;
}

// Row total for the row-tile kernel. G <= 64: the row lives in one
// wavefront. G > 64 (one row per workgroup): wavefront totals meet in LDS
// behind one barrier and every lane adds them in wavefront order. `slot`
// must differ between consecutive reductions of one workgroup so that no
// barrier is needed after the reads.
template <int G>
__device__ __forceinline__ float row_total(float s, float *slot) {
    if constexpr (G <= 64) {
        return group_sum<G>(s);
    } else {
        constexpr int WPR = G / 64;
        const float w = group_sum<64>(s);
        if ((threadIdx.x & 63) == 0) slot[threadIdx.x >> 6] = w;
        __syncthreads();
        float t = slot[0];
#pragma unroll
        for (int j = 1; j < WPR; ++j) t += slot[j];
        return t;
    }
}

template <int W>
__device__ __forceinline__ float sumsq(const float (&v)[W]) {
    float p[W / 2];
#pragma unroll
    for (int e = 0; e < W / 2; ++e)
        p[e] = fmaf(v[2 * e], v[2 * e], v[2 * e + 1] * v[2 * e + 1]);
#pragma unroll
    for (int w = W / 4; w >= 1; w /= 2)
#pragma unroll
        for (int e = 0; e < w; ++e) p[e] += p[e + w];
    return p[0];
}

__device__ __forceinline__ float inv_rms(float total, int n, float eps) {
    // 1/sqrt(mean + eps) with IEEE division and square root.
    return 1.0f / sqrtf(total / (float)n + eps);
}

template <int W>
__device__ __forceinline__ void zero(float (&v)[W]) {
#pragma unroll
    for (int e = 0; e < W; ++e) v[e] = 0.0f;
}

// ---------------------------------------------------------------------------
// One row (or one chunk of a row), shared by the row-tile and split kernels.
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
// ---------------------------------------------------------------------------
template <int OP, int ST, int VPT, int EX, bool LATE, class Reduce>
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
    T *out0 = static_cast<T *>(p.out0) + off;
    if constexpr (OP == OP_ADD_NORM) {
        // s = a + b, rounded to storage, stored, and kept for the norm.
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            const int i = vbase + k * vstride;
            if (live && i < nv) {
                float b[W];
                C::load_nt(x1, i, b);
#pragma unroll
                for (int e = 0; e < W; ++e) v0[k][e] = C::round(v0[k][e] + b[e]);
                C::store_nt(out0, i, v0[k]);
            }
        }
#pragma unroll
        for (int q = 0; q < EX; ++q) {
            const int j = sbase + q * sstride;
            if (live && sown && j < rem) {
                e0[q] = C::round(e0[q] + C::load1_nt(x1, tail0 + j));
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
    const T *g0 = static_cast<const T *>(p.g0);

    if constexpr (OP == OP_PLAIN || OP == OP_ADD_NORM) {
        // y = x * inv * gamma (add_then_norm: x is the stored sum)
        T *y = static_cast<T *>(OP == OP_PLAIN ? p.out0 : p.out1) + off;
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            const int i = vbase + k * vstride;
            if (live && i < nv) {
                float g[W], o[W];
                C::load(g0, i, g);
#pragma unroll
                for (int e = 0; e < W; ++e) o[e] = v0[k][e] * inv0 * g[e];
                C::store_nt(y, i, o);
            }
        }
#pragma unroll
        for (int q = 0; q < EX; ++q) {
            const int j = sbase + q * sstride;
            if (live && sown && j < rem)
                C::store1_nt(y, tail0 + j,
                             e0[q] * inv0 * C::load1(g0, tail0 + j));
        }
    } else {
        // h = r + a * inv * gamma0, kept in registers (v1/e1, or v0/e0 once
        // a is consumed when r is late). norm_then_add stores h * scale.
        const float scale = (OP == OP_NORM_ADD && p.scale) ? *p.scale : 1.0f;
        float(*hv)[W] = LATE ? v0 : v1;
        float *he = LATE ? e0 : e1;
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            const int i = vbase + k * vstride;
            if (live && i < nv) {
                float g[W], rr[W];
                C::load(g0, i, g);
                if constexpr (LATE) {
                    C::load_nt(x1, i, rr);
                } else {
#pragma unroll
                    for (int e = 0; e < W; ++e) rr[e] = v1[k][e];
                }
                if constexpr (OP == OP_TAIL) {
#pragma unroll
                    for (int e = 0; e < W; ++e)
                        hv[k][e] = C::round(fmaf(v0[k][e] * inv0, g[e], rr[e]));
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
                const float h =
                    fmaf(e0[q] * inv0, C::load1(g0, tail0 + j), rr);
                if constexpr (OP == OP_TAIL) {
                    he[q] = C::round(h);
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

            const T *g1 = static_cast<const T *>(p.g1);
            T *out1 = static_cast<T *>(p.out1) + off;
#pragma unroll
            for (int k = 0; k < VPT; ++k) {
                const int i = vbase + k * vstride;
                if (live && i < nv) {
                    float g[W], o[W];
                    C::load(g1, i, g);
#pragma unroll
                    for (int e = 0; e < W; ++e) o[e] = hv[k][e] * inv1 * g[e];
                    C::store_nt(out1, i, o);
                }
            }
#pragma unroll
            for (int q = 0; q < EX; ++q) {
                const int j = sbase + q * sstride;
                if (live && sown && j < rem)
                    C::store1_nt(out1, tail0 + j,
                                 he[q] * inv1 * C::load1(g1, tail0 + j));
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Row-tile kernel: G lanes per row, VPT vectors per lane. G <= 64 packs
// 64/G rows into each wavefront; G > 64 is one row per workgroup.
// ---------------------------------------------------------------------------
template <int G>
constexpr int rowtile_block() { return G >= 128 ? G : 256; }

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

template <int OP, int ST, int G, int VPT>
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
                rowtile_late<OP, ST, G, VPT>()>(
        p, off, live, sub, G, sub, G, true,
        [&](float s, int which) { return row_total<G>(s, red[which]); });
}

// Several RMSNorms in one launch (the same row tile as above): each row
// finds its segment in the table and normalises with that segment's
// tensors and epsilon.
template <int ST, int G, int VPT>
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
    process_row<OP_PLAIN, ST, VPT, rowtile_extra<ST, G>(), false>(
        p, off, live, sub, G, sub, G, true,
        [&](float s, int which) { return row_total<G>(s, red[which]); });
}

// ---------------------------------------------------------------------------
// RMSNorm followed by Q8_1 quantisation (Hesper "RMSNorm Layer", fused
// RMSNorm + Q8_1): each block of 32 normalised values y becomes a 36-byte
// record {f16 d, f16 s = 0, int8 q[32]} with d = max|y| / 127 and
// q = round-half-even(y / d) (a zero block: d = 0, q = 0). Codes are packed
// four per 32-bit word, element 4k in the low byte. n is a multiple of 32,
// so a block is BV = 32 / W consecutive vectors, held by BV consecutive
// lanes of one row group (G a multiple of BV).
//
// With y = x * inv * gamma, the row's 1 / rms cancels from the codes:
// y / d = 127 z / max|z| for z = x * gamma. So the codes are computed from z
// alone, before (and without waiting for) the row's reduction, and only the
// header needs inv: d = inv * max|z| / 127.
// ---------------------------------------------------------------------------

// Max over aligned groups of Q lanes of non-negative f32 bit patterns (which
// order as unsigned integers).
template <int Q>
__device__ __forceinline__ unsigned int group_max_bits(unsigned int v) {
    auto dpp_u = [](unsigned int x, auto ctrl) {
        return (unsigned int)__builtin_amdgcn_update_dpp(
            0, (int)x, decltype(ctrl)::value, 0xF, 0xF, false);
    };
    if constexpr (Q >= 2)
        v = max(v, dpp_u(v, std::integral_constant<int, 0xB1>{}));   // lane ^ 1
    if constexpr (Q >= 4)
        v = max(v, dpp_u(v, std::integral_constant<int, 0x4E>{}));   // lane ^ 2
    if constexpr (Q >= 8)
        v = max(v, dpp_u(v, std::integral_constant<int, 0x141>{}));  // 8-lane halves
    return v;
}

// The codes of one lane's W values z = x * gamma (all lanes of the wavefront
// call it: the block's max|z| is a cross-lane max), packed into W / 4 words;
// returns the block's max|z|.
// t = 127 z / max|z| is formed as (z 2^-e) * (127 / (max|z| 2^-e)) with e
// the binary exponent of max|z|: the power-of-two scalings are exact, the
// reciprocal is of a value in [0.5, 1) (so nothing overflows for any
// max|z| > 0, subnormal included), and t is within a few f32 units of the
// exact quotient, which moves a code only next to a rounding tie. Adding
// 1.5 * 2^23 in the same fused multiply-add rounds t to the nearest integer,
// ties to even, and leaves it in the sum's low bits (|t| <= 127 up to
// rounding, so the int8 clamp never binds); the code is the low byte.
template <int W>
__device__ __forceinline__ float q8_codes(const float (&z)[W],
                                          unsigned int (&words)[W / 4]) {
    constexpr int BV = 32 / W;
    unsigned int m = 0u;
#pragma unroll
    for (int e = 0; e < W; ++e) m = max(m, __float_as_uint(fabsf(z[e])));
    const float amax = __uint_as_float(group_max_bits<BV>(m));
    const int ex = __builtin_amdgcn_frexp_expf(amax);
    const float s =
        amax > 0.0f ? 127.0f * __builtin_amdgcn_rcpf(ldexpf(amax, -ex)) : 0.0f;
    unsigned int c[W];
#pragma unroll
    for (int e = 0; e < W; ++e)
        c[e] = __float_as_uint(fmaf(ldexpf(z[e], -ex), s, 12582912.0f));
#pragma unroll
    for (int w = 0; w < W / 4; ++w)
        words[w] = __builtin_amdgcn_perm(c[4 * w + 1], c[4 * w], 0x0c0c0400u) |
                   __builtin_amdgcn_perm(c[4 * w + 3], c[4 * w + 2], 0x04000c0cu);
    return amax;
}

// Header word {f16 d, s = 0} of a block from its max|z| and the row's 1/rms:
// d = inv * max|z| / 127 (within an f32 unit or two before the f16
// rounding, which is to nearest even).
__device__ __forceinline__ unsigned int q8_header(float amax, float inv) {
    const float d = inv * amax * (1.0f / 127.0f);
    return (unsigned int)__builtin_bit_cast(unsigned short, (_Float16)d);
}

// Codes and header of one lane's vector z (vector index i of a row whose
// records start at `rec`), stored through plain pointers; `valid` masks the
// stores.
template <int W>
__device__ __forceinline__ void q8_vector(const float (&z)[W], float inv,
                                          int i, bool valid,
                                          unsigned char *rec) {
    constexpr int BV = 32 / W;
    unsigned int words[W / 4];
    const float amax = q8_codes<W>(z, words);
    if (!valid) return;
    unsigned char *blk = rec + (int64_t)(i / BV) * 36;
    unsigned int *qw = reinterpret_cast<unsigned int *>(blk + 4) +
                       (i % BV) * (W / 4);
#pragma unroll
    for (int w = 0; w < W / 4; ++w) __builtin_nontemporal_store(words[w], qw + w);
    if (i % BV == 0)
        __builtin_nontemporal_store(q8_header(amax, inv),
                                    reinterpret_cast<unsigned int *>(blk));
}

// Raw buffer access (gfx9 buffer descriptor: 32-bit data format, no
// stride). A lane whose offset is at or past the descriptor's byte count
// loads zeros and its stores are dropped, so edge lanes need no branch.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x3 __attribute__((ext_vector_type(3)));
constexpr int kBufferFormat = 0x00020000;
constexpr unsigned int kOutOfRange = 0x80000000u;
constexpr int kNonTemporal = 2;   // cache policy bit: nt

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_of(const void *base,
                                                           int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0,
                                             (int)bytes, kBufferFormat);
}

constexpr bool q8_persistent(int values_per_lane) { return values_per_lane <= 16; }
// Row blocks in flight per workgroup of the persistent form.
constexpr int q8_prefetch(int values_per_lane) { return 2; }

// Row tile. Where registers allow (PF: at most 16 values per lane) it is
// persistent: workgroup b takes rows b*RPB, b*RPB + stride, ... (stride =
// grid * RPB), issues the next row's loads before the current row is
// reduced and quantised, so HBM reads continue through the arithmetic, and
// keeps the gains in registers. Otherwise each workgroup takes one tile.
template <int ST, int G, int VPT>
__global__ void __launch_bounds__(rowtile_block<G>())
q8_kernel(RowArgs p, int64_t row0, int64_t row_end) {
    using C = Codec<ST>;
    using T = typename C::T;
    constexpr int W = C::W;
    constexpr int BLOCK = rowtile_block<G>();
    constexpr int RPB = BLOCK / G;
    constexpr int WPR = G > 64 ? G / 64 : 1;
    constexpr bool PF = q8_persistent(VPT * W);
    constexpr int PD = q8_prefetch(VPT * W);
    constexpr int BV = 32 / W;
    static_assert(G % BV == 0, "a Q8_1 block must lie in one lane group");
    __shared__ float red[2][WPR];
    // Record staging (persistent form, G >= 64): for each vector slot a
    // wavefront holds 64 consecutive vectors of one row, i.e. RW = 64 / BV
    // whole records forming one contiguous range of the output. They are
    // assembled in LDS, one 16-byte slot per 12-byte third of a record, and
    // leave as one contiguous 12-bytes-per-lane store (a third never
    // straddles a record, so a partly valid range ends on a lane boundary).
    constexpr bool STAGE = PF && G >= 64;
    constexpr int RW = 64 / BV;
    constexpr int WAVES = BLOCK / 64;
    __shared__ unsigned int stage[STAGE ? VPT * WAVES * RW * 12 : 1];

    const int sub = threadIdx.x & (G - 1);
    const int nv = p.nv;
    const int64_t stride = (int64_t)gridDim.x * RPB;
    const int64_t first = row0 + (int64_t)blockIdx.x * RPB;   // block-uniform
    const T *x = static_cast<const T *>(p.x0);
    const T *g = static_cast<const T *>(p.g0);
    unsigned char *out = static_cast<unsigned char *>(p.out0);
    const int64_t rec_row = (int64_t)(p.n / 32) * 36;

    // 1 / rms of the row(s) held in v
    // Only the f16 header uses 1/rms, so the hardware reciprocal square root
    // (about one f32 unit) replaces IEEE square root and division: a shorter
    // chain between a row's reduction and its stores.
    const float inv_n = 1.0f / (float)p.n;
    auto inverse_rms = [&](const float (&v)[VPT][W], float *slot) {
        float s = 0.0f;
#pragma unroll
        for (int k = 0; k < VPT; ++k) s += sumsq<W>(v[k]);
        return __builtin_amdgcn_rsqf(fmaf(row_total<G>(s, slot), inv_n, p.eps0));
    };

    const int lrow = threadIdx.x / G;
    if constexpr (PF) {
        // Persistent, through raw buffers: one descriptor per trip covers
        // the workgroup's RPB rows (bytes of the live ones only), so a dead
        // row or a lane past the row's end reads zeros and writes nothing
        // without a branch. With no branch around any load or store the
        // compiler counts the memory operations in flight exactly and waits
        // for a row's loads without waiting for the previous row's stores
        // (loads and stores share one counter on this architecture).
        const int64_t row_bytes = (int64_t)p.n * (int64_t)sizeof(T);
        const int lane = threadIdx.x & 63;
        unsigned int off_x[VPT], off_q[VPT], off_h[VPT];
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            const int i = k * G + sub;
            const unsigned int rec = (unsigned int)(lrow * rec_row) +
                                     (unsigned int)(i / BV) * 36u;
            off_x[k] = i < nv ? (unsigned int)(lrow * row_bytes) + 16u * i
                              : kOutOfRange;
            if constexpr (STAGE) {
                // this lane's third of a record: record lane / 3 of the
                // wavefront's range, which starts at vector k*G + (sub & ~63)
                const int first_rec = (k * G + (sub & ~63)) / BV;
                const int r3 = first_rec + lane / 3;
                off_q[k] = lane < 3 * RW && r3 < nv / BV
                               ? (unsigned int)(lrow * rec_row) + 36u * r3 +
                                     12u * (lane % 3)
                               : kOutOfRange;
                off_h[k] = 0;
            } else {
                off_q[k] = i < nv ? rec + 4u + (unsigned int)((i % BV) * W)
                                  : kOutOfRange;
                off_h[k] = i < nv && i % BV == 0 ? rec : kOutOfRange;
            }
        }
        // LDS dword of word w (0 = header) of local record j: thirds of a
        // record sit in 16-byte slots
        auto stage_at = [&](int k, int j, int w) {
            return ((k * WAVES + (int)(threadIdx.x >> 6)) * RW + j) * 12 +
                   (w / 3) * 4 + w % 3;
        };
        auto live_rows = [&](int64_t b) {
            const int64_t l = row_end - b;
            return l <= 0 ? (int64_t)0 : (l < RPB ? l : (int64_t)RPB);
        };
        auto load_rows = [&](u32x4 (&raw)[VPT], int64_t b) {
            const auto rs = buffer_of(x + (b < row_end ? b : first) * (int64_t)p.n,
                                      live_rows(b) * row_bytes);
#pragma unroll
            for (int k = 0; k < VPT; ++k)
                raw[k] = __builtin_amdgcn_raw_buffer_load_b128(rs, off_x[k], 0,
                                                              kNonTemporal);
        };
        auto quant_rows = [&](const u32x4 (&raw)[VPT], const float (&gv)[VPT][W],
                              int64_t b, float *slot) {
            float v[VPT][W], amax[VPT];
#pragma unroll
            for (int k = 0; k < VPT; ++k)
                C::decode(__builtin_bit_cast(typename C::vec, raw[k]), v[k]);
            const auto rs = buffer_of(out + (b < row_end ? b : first) * rec_row,
                                      live_rows(b) * rec_row);
            // The codes do not depend on the row's reduction, so they are
            // computed while it is under way; a record's codes and header
            // are stored together afterwards (written apart, the two parts
            // of a record's cache line leave the cache separately).
            unsigned int words[VPT][W / 4];
#pragma unroll
            for (int k = 0; k < VPT; ++k) {
                float z[W];
#pragma unroll
                for (int e = 0; e < W; ++e) z[e] = v[k][e] * gv[k][e];
                amax[k] = q8_codes<W>(z, words[k]);
            }
            const float inv = inverse_rms(v, slot);
            if constexpr (STAGE) {
                // every lane of a record writes its header (the same value)
                const int j = lane / BV;
#pragma unroll
                for (int k = 0; k < VPT; ++k) {
                    stage[stage_at(k, j, 0)] = q8_header(amax[k], inv);
#pragma unroll
                    for (int w = 0; w < W / 4; ++w)
                        stage[stage_at(k, j, 1 + (lane % BV) * (W / 4) + w)] =
                            words[k][w];
                }
                // LDS operations of one wavefront complete in order; the
                // fences only keep the compiler from moving them
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
                for (int k = 0; k < VPT; ++k) {
                    const int l = lane < 3 * RW ? lane : 0;
                    const u32x3 third = *reinterpret_cast<const u32x3 *>(
                        &stage[stage_at(k, l / 3, 3 * (l % 3))]);
                    __builtin_amdgcn_raw_buffer_store_b96(third, rs, off_q[k], 0,
                                                          kNonTemporal);
                }
                return;
            }
#pragma unroll
            for (int k = 0; k < VPT; ++k) {
                if constexpr (W == 4) {
                    __builtin_amdgcn_raw_buffer_store_b32(words[k][0], rs,
                                                          off_q[k], 0,
                                                          kNonTemporal);
                } else {
                    const u32x2 w2 = {words[k][0], words[k][1]};
                    __builtin_amdgcn_raw_buffer_store_b64(w2, rs, off_q[k], 0,
                                                          kNonTemporal);
                }
                __builtin_amdgcn_raw_buffer_store_b32(q8_header(amax[k], inv), rs,
                                                      off_h[k], 0, kNonTemporal);
            }
        };

        // Row blocks b_r = first + r * stride, r < trips, go through NB =
        // PD + 1 buffers in fixed registers: the loads of block r + PD are
        // issued before block r is quantised, so PD blocks are in flight
        // through the arithmetic. The first PD steps are peeled and the loop
        // body is NB steps, unrolled, so the memory operations in flight at
        // the loop's top are the same on entry and on every return (the
        // loads of blocks r .. r + PD - 1 interleaved with the stores of the
        // PD blocks before r); the compiler then waits for block r's loads
        // alone. Prefetches past the last block read nothing and are issued
        // unconditionally inside the loop: a conditional one would leave
        // paths on which the compiler cannot tell which loads are in flight,
        // and it then waits for all of them.
        constexpr int NB = PD + 1;
        const int64_t trips = (row_end - first + stride - 1) / stride;
        float gv[VPT][W];
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            const int i = k * G + sub;
            C::load(g, i < nv ? i : nv - 1, gv[k]);
        }
        u32x4 buf[NB][VPT];
#pragma unroll
        for (int r = 0; r < PD; ++r) load_rows(buf[r], first + r * stride);
        // (the peeled steps run even for a dead block, which reads zeros and
        // stores nothing: skipping them would again leave the loop's top
        // with two different sets of operations in flight)
#pragma unroll
        for (int r = 0; r < PD; ++r) {
            load_rows(buf[(r + PD) % NB], first + (r + PD) * stride);
            quant_rows(buf[r % NB], gv, first + r * stride, red[r & 1]);
        }
        int64_t r = PD;
        for (; r + NB <= trips; r += NB) {
#pragma unroll
            for (int u = 0; u < NB; ++u) {
                // r = PD (mod NB), so block r + u sits in buffer (PD + u) % NB
                const int64_t b = first + (r + u) * stride;
                // the scheduling barriers keep each step's prefetch ahead of
                // its wait and the steps' memory operations in program order
                __builtin_amdgcn_sched_barrier(0);
                load_rows(buf[(2 * PD + u) % NB], b + PD * stride);
                __builtin_amdgcn_sched_barrier(0);
                quant_rows(buf[(PD + u) % NB], gv, b, red[(PD + u) & 1]);
            }
        }
        // at most NB - 1 blocks remain, all already loaded
#pragma unroll
        for (int u = 0; u < NB - 1; ++u)
            if (r + u < trips)
                quant_rows(buf[(PD + u) % NB], gv, first + (r + u) * stride,
                           red[(PD + u) & 1]);
    } else {
        // One row tile per workgroup (a loop would hoist the gain loads and
        // hold a second row's worth of registers); nothing to overlap.
        const int64_t row = first + lrow;
        const bool live = row < row_end;
        const T *xr = x + (live ? row : 0) * (int64_t)p.n;
        float v[VPT][W];
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            const int i = k * G + sub;
            if (live && i < nv) C::load_nt(xr, i, v[k]); else zero(v[k]);
        }
        const float inv = inverse_rms(v, red[0]);
        unsigned char *rec = out + (live ? row : 0) * rec_row;
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            const int i = k * G + sub;
            const bool valid = live && i < nv;
            float gk[W], z[W];
            if (valid) C::load(g, i, gk); else zero(gk);
#pragma unroll
            for (int e = 0; e < W; ++e) z[e] = v[k][e] * gk[e];
            q8_vector<W>(z, inv, i, valid, rec);
        }
    }
}

// ---------------------------------------------------------------------------
// Split-row kernel: chunk c of rows g, g + groups, ... for workgroup
// (g, c) of a cooperative grid of groups x chunks workgroups.
// ---------------------------------------------------------------------------
constexpr int SB = kSplitBlock;
constexpr int SNW = SB / 64;

// Workgroup total of a per-lane value (all lanes receive the same bits).
__device__ __forceinline__ float block_total(float s, float *slot) {
    const float w = group_sum<64>(s);
    if ((threadIdx.x & 63) == 0) slot[threadIdx.x >> 6] = w;
    __syncthreads();
    float t = slot[0];
#pragma unroll
    for (int j = 1; j < SNW; ++j) t += slot[j];
    return t;
}

// Publish this chunk's partial, gather the partials of every chunk of the
// row in chunk order, and leave the row's slots at zero once every chunk has
// read them. `set` selects one of two independent slot sets (the tail's two
// reductions). Each slot is one 64-bit word (flag in the high half, the f32
// partial in the low half), so no fence is needed between value and flag.
__device__ float cross_chunk_total(float partial, const SplitState &st,
                                   int set, int64_t row_local, int chunk,
                                   int chunks, float *part) {
    const int tid = threadIdx.x;
    unsigned long long *slots = st.slots + set * st.slot_cap +
                                row_local * (int64_t)chunks;
    unsigned int *depart = st.depart + set * st.row_cap + row_local;
    if (tid == 0) {
        const unsigned long long word =
            (1ull << 32) | (unsigned long long)__float_as_uint(partial);
        __hip_atomic_store(slots + chunk, word, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
    for (int j = tid; j < chunks; j += SB) {
        unsigned long long v;
        uint32_t polls = 0;
        while (((v = __hip_atomic_load(slots + j, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT)) >> 32) == 0) {
            if (++polls >= st.spin_limit) {
                __hip_atomic_fetch_add(st.timeouts, 1u, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        part[j] = __uint_as_float((unsigned int)v);
    }
    __syncthreads();
    if (tid == 0) {
        const unsigned int done = __hip_atomic_fetch_add(
            depart, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (done == (unsigned int)chunks - 1) {
            for (int j = 0; j < chunks; ++j)
                __hip_atomic_store(slots + j, 0ull, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(depart, 0u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    float t = part[0];
    for (int j = 1; j < chunks; ++j) t += part[j];
    return t;
}

template <int OP, int ST, int VPT>
__global__ void __launch_bounds__(SB)
split_kernel(RowArgs p, SplitState st, int64_t row0, int64_t nrows,
             int chunks, int groups) {
    __shared__ float red[2][SNW];
    __shared__ float part[kSplitMaxChunks];

    const int tid = threadIdx.x;
    const int chunk = (int)(blockIdx.x % (unsigned)chunks);
    const int group = (int)(blockIdx.x / (unsigned)chunks);
    const int vbase = chunk * (SB * VPT) + tid;
    const bool last = chunk == chunks - 1;  // the last chunk owns the remainder

    for (int64_t rl = group; rl < nrows; rl += groups) {
        const int64_t off = (row0 + rl) * (int64_t)p.n;
        process_row<OP, ST, VPT, 1, false>(
            p, off, true, vbase, SB, tid, SB, last,
            [&](float s, int which) {
                return cross_chunk_total(block_total(s, red[which]), st, which,
                                         rl, chunk, chunks, part);
            });
        // The next row rewrites `part` and `red`: every lane must have
        // finished reading them first.
        __syncthreads();
    }
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
constexpr int MB = kMultiBlock;   // threads per workgroup
constexpr int MVPT = kMultiVpt;   // vectors per thread per chunk

// Lane-strided chunk walk: vectors c*MB*MVPT + k*MB + tid, and in the last
// chunk the remainder element tid.
template <int ST, class F, class G>
__device__ __forceinline__ void for_chunk(const RowArgs &p, int chunk,
                                          int chunks, F vec_fn, G rem_fn) {
    const int tid = threadIdx.x;
    const int base = chunk * (MB * MVPT) + tid;
#pragma unroll
    for (int k = 0; k < MVPT; ++k) {
        const int i = base + k * MB;
        if (i < p.nv) vec_fn(i);
    }
    if (chunk == chunks - 1 && tid < p.rem) rem_fn(p.nv * Codec<ST>::W + tid);
}

// part[rl * chunks + c] = sum of squares of chunk c of row row0 + rl of `src`.
template <int ST>
__global__ void __launch_bounds__(MB)
pass_sumsq(RowArgs p, const void *src, int64_t row0, int chunks, float *part) {
    using C = Codec<ST>;
    using T = typename C::T;
    constexpr int W = C::W;
    __shared__ float red[MB / 64];
    const int chunk = (int)(blockIdx.x % (unsigned)chunks);
    const int64_t rl = blockIdx.x / (unsigned)chunks;
    const T *x = static_cast<const T *>(src) + (row0 + rl) * (int64_t)p.n;
    float s = 0.0f;
    for_chunk<ST>(
        p, chunk, chunks,
        [&](int i) { float v[W]; C::load_nt(x, i, v); s += sumsq<W>(v); },
        [&](int j) { const float v = C::load1_nt(x, j); s = fmaf(v, v, s); });
    const float t = block_total(s, red);
    if (threadIdx.x == 0) part[rl * chunks + chunk] = t;
}

// inv[rl] = 1/sqrt(sum_c part[rl * chunks + c] / n + eps), one workgroup per
// row; lane l adds chunks l, l + 256, ... in order, then the lanes' sums are
// added in a fixed order.
__global__ void __launch_bounds__(MB)
pass_combine(const float *part, int chunks, int n, float eps, float *inv) {
    __shared__ float red[MB / 64];
    const int64_t rl = blockIdx.x;
    float s = 0.0f;
    for (int c = threadIdx.x; c < chunks; c += MB) s += part[rl * chunks + c];
    const float t = block_total(s, red);
    if (threadIdx.x == 0) inv[rl] = inv_rms(t, n, eps);
}

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

// The elementwise middle pass, with the chunk's sum of squares of what it
// stores in part[rl * chunks + c] when a later norm needs it:
//   tail:          h = round(r + a * inv * gamma0)                 (+ part)
//   norm_then_add: out = (a * inv * gamma0 + r) * scale
//   add_then_norm: s = round(a + b)                                (+ part)
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
        if constexpr (OP == OP_ADD_NORM) return C::round(av + rv);
        else if constexpr (OP == OP_TAIL) return C::round(fmaf(av * ia, gv, rv));
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

// Q8_1 records of the normalised rows (rows too wide for one register
// tile): codes from z = x * gain, headers from the row's inv. Consecutive
// lanes hold consecutive vectors, so a block is BV consecutive lanes of one
// wavefront.
template <int ST>
__global__ void __launch_bounds__(MB)
pass_q8(RowArgs p, int64_t row0, int chunks, const float *inv) {
    using C = Codec<ST>;
    using T = typename C::T;
    constexpr int W = C::W;
    const int chunk = (int)(blockIdx.x % (unsigned)chunks);
    const int64_t rl = blockIdx.x / (unsigned)chunks;
    const int64_t row = row0 + rl;
    const T *x = static_cast<const T *>(p.x0) + row * (int64_t)p.n;
    const T *g = static_cast<const T *>(p.g0);
    unsigned char *rec = static_cast<unsigned char *>(p.out0) +
                         row * (int64_t)(p.n / 32) * 36;
    const float r = inv[rl];
    const int base = chunk * (MB * MVPT) + threadIdx.x;
#pragma unroll
    for (int k = 0; k < MVPT; ++k) {
        const int i = base + k * MB;
        const bool valid = i < p.nv;
        float v[W], gv[W], z[W];
        if (valid) {
            C::load_nt(x, i, v);
            C::load(g, i, gv);
        } else {
            zero(v);
            zero(gv);
        }
#pragma unroll
        for (int e = 0; e < W; ++e) z[e] = v[e] * gv[e];
        q8_vector<W>(z, r, i, valid, rec);
    }
}

__global__ void zero_kernel(unsigned int *p, int64_t words) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
         i < words; i += stride)
        p[i] = 0u;
}

// ---------------------------------------------------------------------------
// Launchers and the kernel table
// ---------------------------------------------------------------------------
template <int OP, int ST, int G, int VPT>
hipError_t launch_rowtile(const RowArgs &p, int64_t row0, int64_t nrows,
                          hipStream_t stream) {
    constexpr int BLOCK = rowtile_block<G>();
    constexpr int RPB = BLOCK / G;
    const int64_t blocks = (nrows + RPB - 1) / RPB;
    hipLaunchKernelGGL((rowtile_kernel<OP, ST, G, VPT>),
                       dim3((unsigned int)blocks), dim3(BLOCK), 0, stream, p,
                       row0, row0 + nrows);
    return hipGetLastError();
}

template <int OP, int ST, int G, int VPT>
hipError_t occupancy_rowtile(int *blocks_per_cu) {
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(
        blocks_per_cu, rowtile_kernel<OP, ST, G, VPT>, rowtile_block<G>(), 0);
}

template <int ST, int G, int VPT>
hipError_t launch_multi(const MultiArgs &m, int64_t row0, int64_t nrows,
                        hipStream_t stream) {
    constexpr int BLOCK = rowtile_block<G>();
    constexpr int RPB = BLOCK / G;
    const int64_t blocks = (nrows + RPB - 1) / RPB;
    hipLaunchKernelGGL((multi_kernel<ST, G, VPT>), dim3((unsigned int)blocks),
                       dim3(BLOCK), 0, stream, m, row0, row0 + nrows);
    return hipGetLastError();
}

template <int OP, int ST, int G, int VPT>
constexpr MultiLaunch multi_for() {
    if constexpr (OP == OP_PLAIN) return &launch_multi<ST, G, VPT>;
    else return nullptr;
}

template <int OP, int ST, int VPT>
hipError_t launch_split(const RowArgs &p, const SplitState &st, int64_t row0,
                        int64_t nrows, int chunks, int groups,
                        hipStream_t stream) {
    RowArgs pa = p;
    SplitState sa = st;
    int c = chunks, g = groups;
    void *args[] = {&pa, &sa, &row0, &nrows, &c, &g};
    return hipLaunchCooperativeKernel(
        reinterpret_cast<const void *>(&split_kernel<OP, ST, VPT>),
        dim3((unsigned int)(groups * chunks)), dim3(SB), args, 0, stream);
}

template <int OP, int ST, int VPT>
hipError_t occupancy_split(int *blocks_per_cu) {
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(
        blocks_per_cu, split_kernel<OP, ST, VPT>, SB, 0);
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
constexpr int kMaxDevices = 64;

// Workgroups of `kernel` that the current device holds at once (cached per
// device; 0 when the runtime cannot say).
template <typename K>
int64_t resident_blocks(K kernel, int block) {
    static std::atomic<int64_t> cache[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return 0;
    int64_t n = cache[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block,
                                                     0) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount,
                              dev) != hipSuccess)
        return 0;
    n = (int64_t)per_cu * cus;
    cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

template <int ST, int G, int VPT>
hipError_t launch_q8(const RowArgs &p, int64_t row0, int64_t nrows,
                     hipStream_t stream) {
    constexpr int BLOCK = rowtile_block<G>();
    constexpr int RPB = BLOCK / G;
    int64_t blocks = (nrows + RPB - 1) / RPB;
    if constexpr (q8_persistent(VPT * Codec<ST>::W)) {
        const int64_t resident = resident_blocks(q8_kernel<ST, G, VPT>, BLOCK);
        if (resident > 0 && blocks > resident) blocks = resident;
    }
    hipLaunchKernelGGL((q8_kernel<ST, G, VPT>), dim3((unsigned int)blocks),
                       dim3(BLOCK), 0, stream, p, row0, row0 + nrows);
    return hipGetLastError();
}

template <int ST, int G, int VPT>
hipError_t occupancy_q8(int *blocks_per_cu) {
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(
        blocks_per_cu, q8_kernel<ST, G, VPT>, rowtile_block<G>(), 0);
}

template <int ST>
hipError_t launch_multipass_q8(const RowArgs &p, float *scratch, int64_t row0,
                               int64_t nrows, int chunks, hipStream_t stream) {
    float *part = scratch;
    float *inv = scratch + nrows * (int64_t)chunks;
    const dim3 grid((unsigned int)(nrows * chunks));
    hipLaunchKernelGGL(pass_sumsq<ST>, grid, dim3(MB), 0, stream, p, p.x0,
                       row0, chunks, part);
    hipLaunchKernelGGL(pass_combine, dim3((unsigned int)nrows), dim3(MB), 0,
                       stream, (const float *)part, chunks, p.n, p.eps0, inv);
    hipLaunchKernelGGL(pass_q8<ST>, grid, dim3(MB), 0, stream, p, row0, chunks,
                       (const float *)inv);
    return hipGetLastError();
}

#define SNR_Q8(ST, G, VPT)                                                  \
    KernelEntry{OP_NORM_Q8, ST, Codec<ST>::W, KIND_ROWTILE, G, VPT,         \
                rowtile_block<G>(), &launch_q8<ST, G, VPT>, nullptr,        \
                &occupancy_q8<ST, G, VPT>, nullptr, nullptr}
#define SNR_Q8_MULTI(ST)                                                    \
    KernelEntry{OP_NORM_Q8, ST, Codec<ST>::W, KIND_MULTIPASS, MB, MVPT, MB, \
                nullptr, nullptr, nullptr, &launch_multipass_q8<ST>, nullptr}
// Q8_1 shapes: row groups of at least one block (8 lanes for f32, 4 for
// 16-bit storage).
#define SNR_Q8_SHAPES(ST)                                                   \
    SNR_Q8(ST, 8, 4), SNR_Q8(ST, 16, 4), SNR_Q8(ST, 32, 4),                 \
    SNR_Q8(ST, 128, 2), SNR_Q8(ST, 128, 8), SNR_Q8(ST, 256, 2),             \
    SNR_Q8(ST, 256, 4), SNR_Q8(ST, 512, 2), SNR_Q8(ST, 512, 4),             \
    SNR_Q8(ST, 1024, 1), SNR_Q8(ST, 1024, 2), SNR_Q8(ST, 1024, 4),          \
    SNR_Q8(ST, 1024, 8), SNR_Q8_MULTI(ST)

#define SNR_RT_M(OP, ST, G, VPT, M)                                         \
    KernelEntry{OP, ST, Codec<ST>::W, KIND_ROWTILE, G, VPT,                 \
                rowtile_block<G>(), &launch_rowtile<OP, ST, G, VPT>,        \
                nullptr, &occupancy_rowtile<OP, ST, G, VPT>, nullptr, M}
#define SNR_RT(OP, ST, G, VPT) SNR_RT_M(OP, ST, G, VPT, nullptr)
#define SNR_RT_A(OP, ST, G, VPT)                                            \
    SNR_RT_M(OP, ST, G, VPT, (multi_for<OP, ST, G, VPT>()))
#define SNR_SPLIT(OP, ST)                                                   \
    KernelEntry{OP, ST, Codec<ST>::W, KIND_SPLIT, SB, 8, SB, nullptr,        \
                &launch_split<OP, ST, 8>, &occupancy_split<OP, ST, 8>,      \
                nullptr, nullptr}
#define SNR_MULTI(OP, ST)                                                   \
    KernelEntry{OP, ST, Codec<ST>::W, KIND_MULTIPASS, MB, MVPT, MB, nullptr, \
                nullptr, nullptr, &launch_multipass<OP, ST>, nullptr}

// The shapes the automatic choice can reach for one (operation, storage):
// sub-wavefront groups with 4 vectors per lane, then one row per workgroup
// with the smallest register tile that holds about two vectors per lane
// (registers are allocated for every slot of a tile, used or not, and
// occupancy follows them), then split and multi-pass.
#define SNR_AUTO_SHAPES(OP, ST)                                             \
    SNR_RT_A(OP, ST, 1, 4), SNR_RT_A(OP, ST, 2, 4), SNR_RT_A(OP, ST, 4, 4), \
    SNR_RT_A(OP, ST, 8, 4), SNR_RT_A(OP, ST, 16, 4),                        \
    SNR_RT_A(OP, ST, 32, 4), SNR_RT_A(OP, ST, 128, 2),                      \
    SNR_RT_A(OP, ST, 128, 8), SNR_RT_A(OP, ST, 256, 2),                     \
    SNR_RT_A(OP, ST, 256, 4), SNR_RT_A(OP, ST, 512, 2),                     \
    SNR_RT_A(OP, ST, 512, 4), SNR_RT_A(OP, ST, 1024, 1),                    \
    SNR_RT_A(OP, ST, 1024, 2), SNR_RT_A(OP, ST, 1024, 4),                   \
    SNR_RT_A(OP, ST, 1024, 8), SNR_SPLIT(OP, ST), SNR_MULTI(OP, ST)

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
    SNR_Q8_SHAPES(ST_F32),               SNR_Q8(ST_F32, 1024, 16),
    SNR_Q8_SHAPES(ST_BF16),              SNR_Q8(ST_BF16, 4, 4),
    SNR_Q8_SHAPES(ST_F16),               SNR_Q8(ST_F16, 4, 4),
};

}  // namespace

const KernelEntry *kernel_table(int *count) {
    *count = (int)(sizeof(kTable) / sizeof(kTable[0]));
    return kTable;
}

hipError_t zero_words(void *p, int64_t words, hipStream_t stream) {
    if (words <= 0) return hipSuccess;
    int64_t blocks = (words + 255) / 256;
    if (blocks > 1024) blocks = 1024;
    hipLaunchKernelGGL(zero_kernel, dim3((unsigned int)blocks), dim3(256), 0,
                       stream, static_cast<unsigned int *>(p), words);
    return hipGetLastError();
}

}  // namespace snr
