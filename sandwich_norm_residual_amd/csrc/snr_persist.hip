// snr_persist.hip - persistent, pipelined row-tile kernels for RMSNorm, the
// dual-epsilon tail and its two halves (gfx950), and their dispatch table.
//
// The same arithmetic as the row-tile kernel (snr_kernels.hip, process_row)
// with the same G and VPT, so results are bit-identical to it; what changes
// is how rows reach the registers. The grid is the resident workgroup count
// and workgroup b walks rows b, b + grid, ...; the next row's input streams
// are loaded (raw buffer loads) before the current row is reduced, so HBM
// reads continue through both reductions and their barriers. Used for rows
// with no elements past the last whole 128-bit vector and G >= 128 (one row
// per workgroup).
//
// Definitions: "RMSNorm and the dual-epsilon sandwich" (Muser book ch. 12,
// sections 12.1, 12.2, 12.4.3) and Hesper's "RMSNorm Layer" page
// (rmsNormThenAdd[ThenBroadcastScale]Kernel, residualAddRmsNormKernel).
#include "snr_device.h"

namespace snr {
namespace {

template <int OP, int ST, int G, int VPT>
__global__ void __launch_bounds__(G)
persist_kernel(RowArgs p, int64_t row0, int64_t row_end) {
    static_assert(G >= 128, "one row per workgroup");
    using C = Codec<ST>;
    using T = typename C::T;
    constexpr int W = C::W;
    constexpr int NI = OP == OP_PLAIN ? 1 : 2;    // input row streams
    constexpr int WPR = G / 64;
    __shared__ float red[2][WPR];

    const int sub = threadIdx.x;
    const int nv = p.nv;
    const int n = p.n;
    const int64_t stride = gridDim.x;
    const int64_t first = row0 + blockIdx.x;       // block-uniform
    const int64_t row_bytes = (int64_t)n * (int64_t)sizeof(T);
    unsigned int off[VPT];
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        const int i = k * G + sub;
        off[k] = i < nv ? 16u * (unsigned int)i : kOutOfRange;
    }
    // the gains stay in registers as stored and are decoded where used
    u32x4 g0[VPT], g1[VPT];
    {
        const auto r0 = buffer_of(p.g0, row_bytes);
        const auto r1 = buffer_of(OP == OP_TAIL ? p.g1 : p.g0, row_bytes);
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            g0[k] = __builtin_amdgcn_raw_buffer_load_b128(r0, off[k], 0, 0);
            g1[k] = OP == OP_TAIL
                        ? __builtin_amdgcn_raw_buffer_load_b128(r1, off[k], 0, 0)
                        : g0[k];
        }
    }
    const float scale = (OP == OP_NORM_ADD && p.scale) ? *p.scale : 1.0f;

    // descriptor of row `row` of a [rows, n] tensor (no bytes past the end)
    auto row_buf = [&](const void *base, int64_t row) {
        const bool live = row < row_end;
        return buffer_of(static_cast<const T *>(base) + (live ? row : first) * (int64_t)n,
                         live ? row_bytes : 0);
    };
    auto load_rows = [&](u32x4 (&x0)[VPT], u32x4 (&x1)[VPT], int64_t row) {
        const auto r0 = row_buf(p.x0, row);
#pragma unroll
        for (int k = 0; k < VPT; ++k)
            x0[k] = __builtin_amdgcn_raw_buffer_load_b128(r0, off[k], 0, kNonTemporal);
        if constexpr (NI == 2) {
            const auto r1 = row_buf(p.x1, row);
#pragma unroll
            for (int k = 0; k < VPT; ++k)
                x1[k] = __builtin_amdgcn_raw_buffer_load_b128(r1, off[k], 0,
                                                             kNonTemporal);
        }
    };
    auto dec = [&](const u32x4 q, float (&v)[W]) {
        C::decode(__builtin_bit_cast(typename C::vec, q), v);
    };
    auto enc = [&](const float (&v)[W]) {
        return __builtin_bit_cast(u32x4, C::encode(v));
    };
    auto store = [&](const __amdgpu_buffer_rsrc_t rs, int k, const float (&v)[W]) {
        __builtin_amdgcn_raw_buffer_store_b128(enc(v), rs, off[k], 0, kNonTemporal);
    };

    // `slot` is the LDS slot of the row's first reduction: single-reduction
    // operations alternate it between consecutive rows (only that row's
    // barrier separates two of them); the tail's two reductions use slots 0
    // and 1 in every row, so its next first reduction is separated from
    // this one's reads by the second's barrier.
    auto process = [&](const u32x4 (&x0)[VPT], const u32x4 (&x1)[VPT],
                       int64_t row, int slot) {
        float v0[VPT][W];
        const auto o0 = row_buf(p.out0, row);
#pragma unroll
        for (int k = 0; k < VPT; ++k) dec(x0[k], v0[k]);
        if constexpr (OP == OP_ADD_NORM) {
            // s = a + b: stored rounded to storage, kept in f32 for the norm
#pragma unroll
            for (int k = 0; k < VPT; ++k) {
                float b[W];
                dec(x1[k], b);
#pragma unroll
                for (int e = 0; e < W; ++e) v0[k][e] = v0[k][e] + b[e];
                store(o0, k, v0[k]);
            }
        }
        float s = 0.0f;
#pragma unroll
        for (int k = 0; k < VPT; ++k) s += sumsq<W>(v0[k]);
        const float inv0 =
            inv_rms(row_total<G>(s, red[OP == OP_TAIL ? 0 : slot]), n, p.eps0);

        if constexpr (OP == OP_PLAIN || OP == OP_ADD_NORM) {
            const auto oy = row_buf(OP == OP_PLAIN ? p.out0 : p.out1, row);
#pragma unroll
            for (int k = 0; k < VPT; ++k) {
                float g[W], o[W];
                dec(g0[k], g);
#pragma unroll
                for (int e = 0; e < W; ++e) o[e] = v0[k][e] * inv0 * g[e];
                store(oy, k, o);
            }
        } else {
            float h[VPT][W];
#pragma unroll
            for (int k = 0; k < VPT; ++k) {
                float g[W], rr[W];
                dec(g0[k], g);
                dec(x1[k], rr);
                if constexpr (OP == OP_TAIL) {
#pragma unroll
                    for (int e = 0; e < W; ++e)
                        h[k][e] = fmaf(v0[k][e] * inv0, g[e], rr[e]);
                    store(o0, k, h[k]);
                } else {
                    float o[W];
#pragma unroll
                    for (int e = 0; e < W; ++e)
                        o[e] = fmaf(v0[k][e] * inv0, g[e], rr[e]) * scale;
                    store(o0, k, o);
                }
            }
            if constexpr (OP == OP_TAIL) {
                float sh = 0.0f;
#pragma unroll
                for (int k = 0; k < VPT; ++k) sh += sumsq<W>(h[k]);
                const float inv1 = inv_rms(row_total<G>(sh, red[1]), n, p.eps1);
                const auto oy = row_buf(p.out1, row);
#pragma unroll
                for (int k = 0; k < VPT; ++k) {
                    float g[W], o[W];
                    dec(g1[k], g);
#pragma unroll
                    for (int e = 0; e < W; ++e) o[e] = h[k][e] * inv1 * g[e];
                    store(oy, k, o);
                }
            }
        }
    };
    // Rows r = first + t * stride, t < trips, alternate between two buffer
    // sets in fixed registers; the loop is peeled and unrolled so that the
    // same memory operations are in flight at its top on entry and on every
    // return, and prefetches past the end read nothing (see the Q8_1 kernel
    // for why both matter to the compiler's waits).
    const int64_t trips = (row_end - first + stride - 1) / stride;
    u32x4 a0[VPT], b0[VPT], a1[VPT], b1[VPT];
    if (first + stride >= row_end) {
        // one row for this workgroup: nothing to prefetch
        load_rows(a0, b0, first);
        process(a0, b0, first, 0);
        return;
    }
    load_rows(a0, b0, first);
    load_rows(a1, b1, first + stride);
    process(a0, b0, first, 0);
    load_rows(a0, b0, first + 2 * stride);
    int64_t t = 1;
    for (; t + 1 < trips; t += 2) {
        const int64_t row = first + t * stride;
        __builtin_amdgcn_sched_barrier(0);
        process(a1, b1, row, 1);
        __builtin_amdgcn_sched_barrier(0);
        load_rows(a1, b1, row + 2 * stride);
        __builtin_amdgcn_sched_barrier(0);
        process(a0, b0, row + stride, 0);
        __builtin_amdgcn_sched_barrier(0);
        load_rows(a0, b0, row + 3 * stride);
    }
    if (t < trips) process(a1, b1, first + t * stride, 1);
}

template <int OP, int ST, int G, int VPT>
hipError_t launch_persist(const RowArgs &p, int64_t row0, int64_t nrows,
                          hipStream_t stream) {
    int64_t blocks = nrows;
    const int64_t resident = resident_blocks<&persist_kernel<OP, ST, G, VPT>>(G);
    if (resident > 0 && blocks > resident) blocks = resident;
    const int64_t cap = forced_grid_cap();
    if (cap > 0 && blocks > cap) blocks = cap;
    hipLaunchKernelGGL((persist_kernel<OP, ST, G, VPT>), dim3((unsigned int)blocks),
                       dim3(G), 0, stream, p, row0, row0 + nrows);
    return hipGetLastError();
}

template <int OP, int ST, int G, int VPT>
int64_t resident_persist() {
    return resident_blocks<&persist_kernel<OP, ST, G, VPT>>(G);
}

#define SNR_PERSIST(OP, ST, G, VPT)                                          \
    KernelEntry{OP, ST, Codec<ST>::W, KIND_PERSIST, G, VPT, G,               \
                &launch_persist<OP, ST, G, VPT>, nullptr, nullptr, nullptr,  \
                nullptr, &resident_persist<OP, ST, G, VPT>}
#define SNR_PERSIST_SHAPES(OP, ST)                                           \
    SNR_PERSIST(OP, ST, 128, 2), SNR_PERSIST(OP, ST, 256, 2),                \
    SNR_PERSIST(OP, ST, 512, 2), SNR_PERSIST(OP, ST, 1024, 1),               \
    SNR_PERSIST(OP, ST, 1024, 2)

// 1024 x 4 only for the plain norm: one input stream double-buffered and
// one gain fit a 1024-lane workgroup's registers; the tail's two streams and
// two gains would not.
const KernelEntry kPersistTable[] = {
    SNR_PERSIST_SHAPES(OP_PLAIN, ST_F32),    SNR_PERSIST(OP_PLAIN, ST_F32, 1024, 4),
    SNR_PERSIST_SHAPES(OP_PLAIN, ST_BF16),   SNR_PERSIST(OP_PLAIN, ST_BF16, 1024, 4),
    SNR_PERSIST_SHAPES(OP_PLAIN, ST_F16),    SNR_PERSIST(OP_PLAIN, ST_F16, 1024, 4),
    SNR_PERSIST_SHAPES(OP_TAIL, ST_F32),
    SNR_PERSIST_SHAPES(OP_TAIL, ST_BF16),    SNR_PERSIST_SHAPES(OP_TAIL, ST_F16),
    SNR_PERSIST_SHAPES(OP_NORM_ADD, ST_F32), SNR_PERSIST_SHAPES(OP_NORM_ADD, ST_BF16),
    SNR_PERSIST_SHAPES(OP_NORM_ADD, ST_F16), SNR_PERSIST_SHAPES(OP_ADD_NORM, ST_F32),
    SNR_PERSIST_SHAPES(OP_ADD_NORM, ST_BF16), SNR_PERSIST_SHAPES(OP_ADD_NORM, ST_F16),
};

}  // namespace

const KernelEntry *persist_kernel_table(int *count) {
    *count = (int)(sizeof(kPersistTable) / sizeof(kPersistTable[0]));
    return kPersistTable;
}

}  // namespace snr
