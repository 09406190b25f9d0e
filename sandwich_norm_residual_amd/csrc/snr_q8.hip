// snr_q8.hip - RMSNorm into Q8_1 records for gfx950: the persistent
// row-tile kernel, its one-tile-per-workgroup form for wide register tiles,
// the multi-pass form, and their entries in the dispatch table.
//
// Definition: Hesper's "RMSNorm Layer" page, "Fused RMSNorm + Q8_1
// quantize" (fusedRMSNormQ8_1Kernel): the normalised row is cut into blocks
// of 32 values, each stored as a scale d = amax / 127 (f16), a second f16
// field s (always 0 here) and 32 codes round(value / d) in int8.
#include "snr_device.h"

namespace snr {
namespace {

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

// 127 / m for m in [0.5, 1): the hardware reciprocal refined by one Newton
// step, then the quotient corrected by its remainder, which a fused
// multiply-add computes exactly (Markstein's scheme). With the reciprocal
// anywhere within one unit of 1/m this gives the correctly rounded quotient
// (checked in exact arithmetic by the host tests), and the exact quotient
// where it is representable (m = 1/2 and 127/128), so an exact tie stays a
// tie. With m bounded away from zero, infinity and the subnormals, none of
// the scaling and special-case steps of a general division apply.
__device__ __forceinline__ float q8_quotient127(float m) {
    float r = __builtin_amdgcn_rcpf(m);
    r = fmaf(fmaf(-m, r, 1.0f), r, r);
    const float q = 127.0f * r;
    return fmaf(fmaf(-m, q, 127.0f), r, q);
}

// The codes of one lane's W values z = x * gamma (all lanes of the wavefront
// call it: the block's max|z| is a cross-lane max), packed into W / 4 words;
// returns the block's max|z|.
// t = 127 z / max|z| is formed as (z 2^-e) * (127 / (max|z| 2^-e)) with e
// the binary exponent of max|z|: the power-of-two scalings are exact, the
// divisor lies in [0.5, 1) (so nothing overflows for any max|z| > 0,
// subnormal included), and the quotient 127 / m is correctly rounded. The
// fused multiply-add with 1.5 * 2^23 then rounds the exact product to the
// nearest integer, ties to even, leaving it in the sum's low bits (|t| <=
// 127 up to rounding, so the int8 clamp never binds); the code is the low
// byte. So a code is round-half-even of the exact quotient whenever 127 / m
// is exact (an exact tie stays a tie), and otherwise differs from it only
// within about 127 * 2^-24 of a tie.
template <int W>
__device__ __forceinline__ float q8_codes(const float (&z)[W],
                                          unsigned int (&words)[W / 4]) {
    constexpr int BV = 32 / W;
    unsigned int m = 0u;
#pragma unroll
    for (int e = 0; e < W; ++e) m = max(m, __float_as_uint(fabsf(z[e])));
    const float amax = __uint_as_float(group_max_bits<BV>(m));
    const int ex = __builtin_amdgcn_frexp_expf(amax);
    const float s = amax > 0.0f ? q8_quotient127(ldexpf(amax, -ex)) : 0.0f;
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

constexpr bool q8_persistent(int values_per_lane) { return values_per_lane <= 16; }
// Row blocks in flight per workgroup of the persistent form.
constexpr int q8_prefetch(int values_per_lane) { return 1; }

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
    // v_rsq_f32 takes a subnormal input as zero. The input is below the
    // smallest normal only when epsilon is subnormal; it is then scaled by
    // 2^24 and the result by 2^12, both exact, so a zero row still gets a
    // finite 1/rms (and d = 0).
    const float inv_n = 1.0f / (float)p.n;
    auto inverse_rms = [&](float s, float *slot) {
        const float v = fmaf(row_total<G>(s, slot), inv_n, p.eps0);
        const bool tiny = v < 0x1p-126f;
        const float r = __builtin_amdgcn_rsqf(tiny ? v * 0x1p24f : v);
        return tiny ? r * 0x1p12f : r;
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
        auto quant_rows = [&](const u32x4 (&raw)[VPT], const u32x4 (&graw)[VPT],
                              int64_t b, float *slot) {
            const auto rs = buffer_of(out + (b < row_end ? b : first) * rec_row,
                                      live_rows(b) * rec_row);
            // The codes do not depend on the row's reduction, so one pass
            // over the vectors forms each vector's codes and its share of
            // the sum of squares (the decoded row is never held whole); a
            // record's codes and header are stored together after the
            // reduction (written apart, the two parts of a record's cache
            // line leave the cache separately).
            unsigned int words[VPT][W / 4];
            float amax[VPT], s = 0.0f;
#pragma unroll
            for (int k = 0; k < VPT; ++k) {
                float v[W], gk[W], z[W];
                C::decode(__builtin_bit_cast(typename C::vec, raw[k]), v);
                C::decode(__builtin_bit_cast(typename C::vec, graw[k]), gk);
                s += sumsq<W>(v);
#pragma unroll
                for (int e = 0; e < W; ++e) z[e] = v[e] * gk[e];
                amax[k] = q8_codes<W>(z, words[k]);
            }
            const float inv = inverse_rms(s, slot);
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
        // the gains stay in registers as stored (half the registers for
        // 16-bit storage) and are decoded where used
        u32x4 gv[VPT];
        const auto rg = buffer_of(g, row_bytes);
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            const int i = k * G + sub;
            gv[k] = __builtin_amdgcn_raw_buffer_load_b128(
                rg, i < nv ? 16u * i : kOutOfRange, 0, 0);
        }
        u32x4 buf[NB][VPT];
        if (trips == 1) {
            // one row block for this workgroup: nothing to prefetch
            load_rows(buf[0], first);
            quant_rows(buf[0], gv, first, red[0]);
            return;
        }
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
        float s = 0.0f;
#pragma unroll
        for (int k = 0; k < VPT; ++k) s += sumsq<W>(v[k]);
        const float inv = inverse_rms(s, red[0]);
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

template <int ST, int G, int VPT>
hipError_t launch_q8(const RowArgs &p, int64_t row0, int64_t nrows,
                     hipStream_t stream) {
    constexpr int BLOCK = rowtile_block<G>();
    constexpr int RPB = BLOCK / G;
    int64_t blocks = (nrows + RPB - 1) / RPB;
    if constexpr (q8_persistent(VPT * Codec<ST>::W)) {
        const int64_t resident = resident_blocks<&q8_kernel<ST, G, VPT>>(BLOCK);
        if (resident > 0 && blocks > resident) blocks = resident;
        const int64_t cap = forced_grid_cap();
        if (cap > 0 && blocks > cap) blocks = cap;
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

const KernelEntry kQ8Table[] = {
    SNR_Q8_SHAPES(ST_F32),  SNR_Q8(ST_F32, 1024, 16),
    SNR_Q8_SHAPES(ST_BF16), SNR_Q8(ST_BF16, 4, 4),
    SNR_Q8_SHAPES(ST_F16),  SNR_Q8(ST_F16, 4, 4),
};

}  // namespace

const KernelEntry *q8_kernel_table(int *count) {
    *count = (int)(sizeof(kQ8Table) / sizeof(kQ8Table[0]));
    return kQ8Table;
}

}  // namespace snr
