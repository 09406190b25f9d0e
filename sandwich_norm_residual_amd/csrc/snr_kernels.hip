// snr_kernels.hip - gfx950 (CDNA4) kernels for row-wise RMSNorm and the fused
// dual-epsilon sandwich tail.
//
// What is computed ("RMSNorm and the dual-epsilon sandwich", Muser book
// chapter 12):
//   plain (section 12.1):  y = x / sqrt(mean(x^2) + eps) * gamma
//   tail (sections 12.2 and 12.4.3):
//       h = r + a / sqrt(mean(a^2) + eps_post) * gamma_post
//       y = h / sqrt(mean(h^2) + eps_pre) * gamma_pre
//
// Design (HBM-bound, no contraction, so no MFMA):
// * Each row is read from HBM exactly once: every lane loads its share of the
//   row into registers with coalesced loads (128-bit when the row layout
//   allows, element-wide otherwise), the sum of squares is reduced, and the
//   normalise pass works from those registers. The tail also keeps h in
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
// * Stores of outputs and loads of row data are non-temporal (each byte is
//   touched once); gains use ordinary cached loads (every row re-reads them).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "snr_internal.h"

namespace snr {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// Storage codecs: W elements per load, converted to f32 registers.
// ---------------------------------------------------------------------------
template <int ST, int W>
struct Access;

template <>
struct Access<ST_F32, 4> {
    using T = float;
    __device__ static void load_nt(const T *row, int i, float (&v)[4]) {
        const f32x4 q = __builtin_nontemporal_load(
            reinterpret_cast<const f32x4 *>(row) + i);
        v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
    }
    __device__ static void load(const T *base, int i, float (&v)[4]) {
        const f32x4 q = reinterpret_cast<const f32x4 *>(base)[i];
        v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
    }
    __device__ static void store_nt(T *row, int i, const float (&v)[4]) {
        const f32x4 q = {v[0], v[1], v[2], v[3]};
        __builtin_nontemporal_store(q, reinterpret_cast<f32x4 *>(row) + i);
    }
};

template <>
struct Access<ST_F32, 1> {
    using T = float;
    __device__ static void load_nt(const T *row, int i, float (&v)[1]) {
        v[0] = __builtin_nontemporal_load(row + i);
    }
    __device__ static void load(const T *base, int i, float (&v)[1]) {
        v[0] = base[i];
    }
    __device__ static void store_nt(T *row, int i, const float (&v)[1]) {
        __builtin_nontemporal_store(v[0], row + i);
    }
};

// bf16 -> f32 is exact (a bf16 is the upper half of an f32); f32 -> bf16
// rounds to nearest even (gfx950's v_cvt_pk_bf16_f32).
__device__ __forceinline__ float bf16_lo(unsigned int w) {
    return __uint_as_float(w << 16);
}
__device__ __forceinline__ float bf16_hi(unsigned int w) {
    return __uint_as_float(w & 0xFFFF0000u);
}
__device__ __forceinline__ unsigned int bf16_pack(float lo, float hi) {
    const f32x2 f = {lo, hi};
    return __builtin_bit_cast(unsigned int, __builtin_convertvector(f, bf16x2));
}

template <>
struct Access<ST_BF16, 8> {
    using T = unsigned short;
    __device__ static void unpack(const u32x4 q, float (&v)[8]) {
        v[0] = bf16_lo(q.x); v[1] = bf16_hi(q.x);
        v[2] = bf16_lo(q.y); v[3] = bf16_hi(q.y);
        v[4] = bf16_lo(q.z); v[5] = bf16_hi(q.z);
        v[6] = bf16_lo(q.w); v[7] = bf16_hi(q.w);
    }
    __device__ static void load_nt(const T *row, int i, float (&v)[8]) {
        unpack(__builtin_nontemporal_load(
                   reinterpret_cast<const u32x4 *>(row) + i), v);
    }
    __device__ static void load(const T *base, int i, float (&v)[8]) {
        unpack(reinterpret_cast<const u32x4 *>(base)[i], v);
    }
    __device__ static void store_nt(T *row, int i, const float (&v)[8]) {
        const u32x4 q = {bf16_pack(v[0], v[1]), bf16_pack(v[2], v[3]),
                         bf16_pack(v[4], v[5]), bf16_pack(v[6], v[7])};
        __builtin_nontemporal_store(q, reinterpret_cast<u32x4 *>(row) + i);
    }
};

template <>
struct Access<ST_BF16, 1> {
    using T = unsigned short;
    __device__ static void load_nt(const T *row, int i, float (&v)[1]) {
        v[0] = __uint_as_float(
            (unsigned int)__builtin_nontemporal_load(row + i) << 16);
    }
    __device__ static void load(const T *base, int i, float (&v)[1]) {
        v[0] = __uint_as_float((unsigned int)base[i] << 16);
    }
    __device__ static void store_nt(T *row, int i, const float (&v)[1]) {
        const unsigned short b =
            __builtin_bit_cast(unsigned short, (__bf16)v[0]);
        __builtin_nontemporal_store(b, row + i);
    }
};

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
    if constexpr (W == 1) {
        return v[0] * v[0];
    } else {
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
// Row-tile kernel
// ---------------------------------------------------------------------------
template <int G>
constexpr int rowtile_block() { return G >= 128 ? G : 256; }

template <int OP, int ST, int W, int G, int VPT>
__global__ void __launch_bounds__(rowtile_block<G>())
rowtile_kernel(RowArgs p, int64_t row0, int64_t row_end) {
    using A = Access<ST, W>;
    using T = typename A::T;
    constexpr int BLOCK = rowtile_block<G>();
    constexpr int RPB = BLOCK / G;
    constexpr int WPR = G > 64 ? G / 64 : 1;
    __shared__ float red[2][WPR];

    const int tid = threadIdx.x;
    const int sub = tid & (G - 1);
    const int64_t row = row0 + (int64_t)blockIdx.x * RPB + tid / G;
    const bool live = row < row_end;
    const int64_t off = live ? row * (int64_t)p.n : 0;
    const int nv = p.nv;

    float v0[VPT][W];
    float v1[OP == OP_TAIL ? VPT : 1][W];
    (void)v1;

    const T *x0 = static_cast<const T *>(p.x0) + off;
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        const int i = k * G + sub;
        if (live && i < nv) A::load_nt(x0, i, v0[k]); else zero(v0[k]);
    }
    if constexpr (OP == OP_TAIL) {
        const T *x1 = static_cast<const T *>(p.x1) + off;
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            const int i = k * G + sub;
            if (live && i < nv) A::load_nt(x1, i, v1[k]); else zero(v1[k]);
        }
    }

    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < VPT; ++k) s += sumsq<W>(v0[k]);
    const float inv0 = inv_rms(row_total<G>(s, red[0]), p.n, p.eps0);

    const T *g0 = static_cast<const T *>(p.g0);
    T *out0 = static_cast<T *>(p.out0) + off;
    if constexpr (OP == OP_PLAIN) {
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            const int i = k * G + sub;
            if (live && i < nv) {
                float g[W], o[W];
                A::load(g0, i, g);
#pragma unroll
                for (int e = 0; e < W; ++e) o[e] = v0[k][e] * inv0 * g[e];
                A::store_nt(out0, i, o);
            }
        }
    } else {
        // h = r + a * inv_a * gamma_post, kept in v1 for the second norm.
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            const int i = k * G + sub;
            if (live && i < nv) {
                float g[W];
                A::load(g0, i, g);
#pragma unroll
                for (int e = 0; e < W; ++e)
                    v1[k][e] = fmaf(v0[k][e] * inv0, g[e], v1[k][e]);
                A::store_nt(out0, i, v1[k]);
            }
        }
        float sh = 0.0f;
#pragma unroll
        for (int k = 0; k < VPT; ++k) sh += sumsq<W>(v1[k]);
        const float inv1 = inv_rms(row_total<G>(sh, red[1]), p.n, p.eps1);
        const T *g1 = static_cast<const T *>(p.g1);
        T *out1 = static_cast<T *>(p.out1) + off;
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            const int i = k * G + sub;
            if (live && i < nv) {
                float g[W], o[W];
                A::load(g1, i, g);
#pragma unroll
                for (int e = 0; e < W; ++e) o[e] = v1[k][e] * inv1 * g[e];
                A::store_nt(out1, i, o);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Split-row kernel
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
// reductions).
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

template <int OP, int ST, int W, int VPT>
__global__ void __launch_bounds__(SB)
split_kernel(RowArgs p, SplitState st, int64_t row0, int64_t nrows,
             int chunks, int groups) {
    using A = Access<ST, W>;
    using T = typename A::T;
    __shared__ float red[2][SNW];
    __shared__ float part[kSplitMaxChunks];

    const int tid = threadIdx.x;
    const int chunk = (int)(blockIdx.x % (unsigned)chunks);
    const int group = (int)(blockIdx.x / (unsigned)chunks);
    const int first = chunk * (SB * VPT) + tid;
    const int nv = p.nv;
    const T *g0 = static_cast<const T *>(p.g0);
    const T *g1 = static_cast<const T *>(p.g1);

    for (int64_t rl = group; rl < nrows; rl += groups) {
        const int64_t off = (row0 + rl) * (int64_t)p.n;
        float v0[VPT][W];
        float v1[OP == OP_TAIL ? VPT : 1][W];
        (void)v1;
        const T *x0 = static_cast<const T *>(p.x0) + off;
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            const int i = first + k * SB;
            if (i < nv) A::load_nt(x0, i, v0[k]); else zero(v0[k]);
        }
        if constexpr (OP == OP_TAIL) {
            const T *x1 = static_cast<const T *>(p.x1) + off;
#pragma unroll
            for (int k = 0; k < VPT; ++k) {
                const int i = first + k * SB;
                if (i < nv) A::load_nt(x1, i, v1[k]); else zero(v1[k]);
            }
        }
        float s = 0.0f;
#pragma unroll
        for (int k = 0; k < VPT; ++k) s += sumsq<W>(v0[k]);
        const float tot0 = cross_chunk_total(block_total(s, red[0]), st, 0, rl,
                                             chunk, chunks, part);
        const float inv0 = inv_rms(tot0, p.n, p.eps0);

        T *out0 = static_cast<T *>(p.out0) + off;
        if constexpr (OP == OP_PLAIN) {
#pragma unroll
            for (int k = 0; k < VPT; ++k) {
                const int i = first + k * SB;
                if (i < nv) {
                    float g[W], o[W];
                    A::load(g0, i, g);
#pragma unroll
                    for (int e = 0; e < W; ++e) o[e] = v0[k][e] * inv0 * g[e];
                    A::store_nt(out0, i, o);
                }
            }
        } else {
#pragma unroll
            for (int k = 0; k < VPT; ++k) {
                const int i = first + k * SB;
                if (i < nv) {
                    float g[W];
                    A::load(g0, i, g);
#pragma unroll
                    for (int e = 0; e < W; ++e)
                        v1[k][e] = fmaf(v0[k][e] * inv0, g[e], v1[k][e]);
                    A::store_nt(out0, i, v1[k]);
                }
            }
            float sh = 0.0f;
#pragma unroll
            for (int k = 0; k < VPT; ++k) sh += sumsq<W>(v1[k]);
            const float tot1 = cross_chunk_total(block_total(sh, red[1]), st,
                                                 1, rl, chunk, chunks, part);
            const float inv1 = inv_rms(tot1, p.n, p.eps1);
            T *out1 = static_cast<T *>(p.out1) + off;
#pragma unroll
            for (int k = 0; k < VPT; ++k) {
                const int i = first + k * SB;
                if (i < nv) {
                    float g[W], o[W];
                    A::load(g1, i, g);
#pragma unroll
                    for (int e = 0; e < W; ++e) o[e] = v1[k][e] * inv1 * g[e];
                    A::store_nt(out1, i, o);
                }
            }
        }
        // The next row reuses `part` and `red`: every lane must have finished
        // reading them (cross_chunk_total's sums) before they are rewritten.
        __syncthreads();
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
template <int OP, int ST, int W, int G, int VPT>
hipError_t launch_rowtile(const RowArgs &p, int64_t row0, int64_t nrows,
                          hipStream_t stream) {
    constexpr int BLOCK = rowtile_block<G>();
    constexpr int RPB = BLOCK / G;
    const int64_t blocks = (nrows + RPB - 1) / RPB;
    hipLaunchKernelGGL((rowtile_kernel<OP, ST, W, G, VPT>),
                       dim3((unsigned int)blocks), dim3(BLOCK), 0, stream, p,
                       row0, row0 + nrows);
    return hipGetLastError();
}

template <int OP, int ST, int W, int G, int VPT>
hipError_t occupancy_rowtile(int *blocks_per_cu) {
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(
        blocks_per_cu, rowtile_kernel<OP, ST, W, G, VPT>, rowtile_block<G>(),
        0);
}

template <int OP, int ST, int W, int VPT>
hipError_t launch_split(const RowArgs &p, const SplitState &st, int64_t row0,
                        int64_t nrows, int chunks, int groups,
                        hipStream_t stream) {
    RowArgs pa = p;
    SplitState sa = st;
    int c = chunks, g = groups;
    void *args[] = {&pa, &sa, &row0, &nrows, &c, &g};
    return hipLaunchCooperativeKernel(
        reinterpret_cast<const void *>(&split_kernel<OP, ST, W, VPT>),
        dim3((unsigned int)(groups * chunks)), dim3(SB), args, 0, stream);
}

template <int OP, int ST, int W, int VPT>
hipError_t occupancy_split(int *blocks_per_cu) {
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(
        blocks_per_cu, split_kernel<OP, ST, W, VPT>, SB, 0);
}

#define SNR_RT(OP, ST, W, G, VPT)                                         \
    KernelEntry{OP, ST, W, KIND_ROWTILE, G, VPT, rowtile_block<G>(),      \
                &launch_rowtile<OP, ST, W, G, VPT>, nullptr,              \
                &occupancy_rowtile<OP, ST, W, G, VPT>}
#define SNR_SPLIT(OP, ST, W, VPT)                                         \
    KernelEntry{OP, ST, W, KIND_SPLIT, SB, VPT, SB, nullptr,              \
                &launch_split<OP, ST, W, VPT>, &occupancy_split<OP, ST, W, VPT>}

// The shapes compiled for one (operation, storage, load width). Sub-wavefront
// groups hold 4 loads per lane; whole wavefronts and workgroups hold up to 16.
#define SNR_SHAPES(OP, ST, W)                                              \
    SNR_RT(OP, ST, W, 1, 4), SNR_RT(OP, ST, W, 2, 4),                      \
    SNR_RT(OP, ST, W, 4, 4), SNR_RT(OP, ST, W, 8, 4),                      \
    SNR_RT(OP, ST, W, 16, 4), SNR_RT(OP, ST, W, 32, 4),                    \
    SNR_RT(OP, ST, W, 64, 2), SNR_RT(OP, ST, W, 64, 4),                    \
    SNR_RT(OP, ST, W, 64, 8), SNR_RT(OP, ST, W, 64, 16),                   \
    SNR_RT(OP, ST, W, 128, 8), SNR_RT(OP, ST, W, 128, 13),                 \
    SNR_RT(OP, ST, W, 128, 16), SNR_RT(OP, ST, W, 256, 4),                 \
    SNR_RT(OP, ST, W, 256, 7), SNR_RT(OP, ST, W, 256, 8),                  \
    SNR_RT(OP, ST, W, 256, 16), SNR_RT(OP, ST, W, 512, 4),                 \
    SNR_RT(OP, ST, W, 512, 8), SNR_RT(OP, ST, W, 512, 16),                 \
    SNR_RT(OP, ST, W, 1024, 2), SNR_RT(OP, ST, W, 1024, 4),                \
    SNR_RT(OP, ST, W, 1024, 8), SNR_SPLIT(OP, ST, W, 8)

// 1024 lanes x 16 loads only where the row fits in the 128 registers a lane
// of a 1024-lane workgroup may use (it spills for 8-wide bf16 and the tail's
// two 4-wide streams).
const KernelEntry kTable[] = {
    SNR_SHAPES(OP_PLAIN, ST_F32, 4),  SNR_RT(OP_PLAIN, ST_F32, 4, 1024, 16),
    SNR_SHAPES(OP_PLAIN, ST_F32, 1),  SNR_RT(OP_PLAIN, ST_F32, 1, 1024, 16),
    SNR_SHAPES(OP_PLAIN, ST_BF16, 8),
    SNR_SHAPES(OP_PLAIN, ST_BF16, 1), SNR_RT(OP_PLAIN, ST_BF16, 1, 1024, 16),
    SNR_SHAPES(OP_TAIL, ST_F32, 4),
    SNR_SHAPES(OP_TAIL, ST_F32, 1),   SNR_RT(OP_TAIL, ST_F32, 1, 1024, 16),
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
