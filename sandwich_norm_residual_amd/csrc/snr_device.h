// snr_device.h - device building blocks shared by the kernel sources of
// libsnr (internal; included only by the .hip files): storage codecs, the
// cross-lane and workgroup reductions, raw buffer access, the multi-pass
// sum-of-squares passes, and the resident-workgroup query.
#pragma once

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
    __device__ static vec encode(const float (&v)[4]) {
        return vec{v[0], v[1], v[2], v[3]};
    }
    __device__ static void load_nt(const T *row, int i, float (&v)[4]) {
        const vec q = __builtin_nontemporal_load(
            reinterpret_cast<const vec *>(row) + i);
        v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
    }
    __device__ static vec load_raw(const T *base, int i) {
        return reinterpret_cast<const vec *>(base)[i];
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
    // A stored value is the f16 rounding of the f32 result. The empty asm
    // makes the f32 value opaque, so the compiler cannot fuse the operation
    // that produced it with the conversion (v_fma_mix*/v_mad_mix* round once,
    // straight to f16); otherwise kernels would round differently wherever
    // it happened to fuse.
    __device__ static float settle(float v) {
        __asm__("" : "+v"(v));
        return v;
    }
    __device__ static unsigned int pack(float a, float b) {
        const f32x2 f = {settle(a), settle(b)};
        return __builtin_bit_cast(unsigned int,
                                  __builtin_convertvector(f, f16x2));
    }
    __device__ static float one(unsigned short b) {
        return (float)__builtin_bit_cast(_Float16, b);
    }
    __device__ static unsigned short enc(float v) {
        return __builtin_bit_cast(unsigned short, (_Float16)settle(v));
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
    __device__ static vec encode(const float (&v)[8]) {
        return vec{B::pack(v[0], v[1]), B::pack(v[2], v[3]),
                   B::pack(v[4], v[5]), B::pack(v[6], v[7])};
    }
    __device__ static vec load_raw(const T *base, int i) {
        return reinterpret_cast<const vec *>(base)[i];
    }
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

// Workgroup size of the row-tile kernels: G > 64 lanes per row is one row
// per workgroup of G lanes; smaller groups share 256-lane workgroups.
template <int G>
constexpr int rowtile_block() { return G >= 128 ? G : 256; }

static_assert(kSplitBlock == kMultiBlock,
              "block_total serves split and multi-pass workgroups alike");
constexpr int SNW = kSplitBlock / 64;

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

// ---------------------------------------------------------------------------
// Multi-pass building blocks (rows too wide to keep on chip): per-chunk sums
// of squares and their per-row combination, shared by every operation's
// multi-pass form.
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
[[maybe_unused]] __global__ void __launch_bounds__(MB)
pass_combine(const float *part, int chunks, int n, float eps, float *inv) {
    __shared__ float red[MB / 64];
    const int64_t rl = blockIdx.x;
    // each thread adds its chunks (c, c + MB, ...) in blocks of 32, then the
    // block sums: chains of at most 32 + chunks / (32 MB) additions
    float s = 0.0f, blk = 0.0f;
    int cnt = 0;
    for (int c = threadIdx.x; c < chunks; c += MB) {
        blk += part[rl * chunks + c];
        if (++cnt == 32) {
            s += blk;
            blk = 0.0f;
            cnt = 0;
        }
    }
    s += blk;
    const float t = block_total(s, red);
    if (threadIdx.x == 0) inv[rl] = inv_rms(t, n, eps);
}

constexpr int kMaxDevices = 64;

// Workgroups of kernel K (launched with `block` threads) that the current
// device holds at once; 0 when the runtime cannot say. Cached per kernel and
// device: K is a template argument, so every kernel has a cache of its own
// (kernels of one signature must not share one).
template <auto K>
int64_t resident_blocks(int block) {
    static std::atomic<int64_t> cache[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return 0;
    int64_t n = cache[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, K, block, 0) !=
            hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount,
                              dev) != hipSuccess)
        return 0;
    n = (int64_t)per_cu * cus;
    cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

}  // namespace
}  // namespace snr
