// Streaming kernels that the benchmark times beside the hot path, to state
// what this GPU's HBM sustains for the same bytes with no arithmetic and no
// reduction:
// * plain reads, plain writes and plain copies (stream_probe). Reads alone
//   and writes alone each stream faster than any mix of the two (an HBM
//   channel turns its bus around between them), so a step's floor is a
//   plain copy of its written bytes plus its remaining reads at the
//   read-only rate;
// * the access pattern of a row operation (stream_probe_rows): one or two
//   input rows and one or two output rows per workgroup, as the row-tile
//   kernels lay them out, loads then stores, nothing computed.
//
// Not part of the library: built into bench_stream.so, loaded by bench.py
// only.
//
// stream_probe's access pattern: a flat grid-stride loop over 16-byte
// vectors, 256 lanes per workgroup, U vectors per lane per trip spaced 256
// vectors apart, so that a workgroup touches 256*U consecutive vectors per
// trip and consecutive workgroups touch consecutive ranges. Every access is
// guarded by i < total.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <initializer_list>

typedef float f4 __attribute__((ext_vector_type(4)));
typedef unsigned u4 __attribute__((ext_vector_type(4)));

namespace {

constexpr int kLanes = 256;

template <bool NT> __device__ __forceinline__ f4 load(const f4 *p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}
template <bool NT> __device__ __forceinline__ void store(f4 v, f4 *p) {
    if constexpr (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}

// Reads every vector and folds its bits into one word, which is stored only
// if it equals a constant no fill used here produces: the loads stay, and
// nothing is written.
template <bool NT, int U>
__global__ void __launch_bounds__(kLanes) read_kernel(const f4 *src, int64_t total, unsigned *sink) {
    unsigned acc = 0;
    const int64_t stride = (int64_t)gridDim.x * kLanes * U;
    for (int64_t base = (int64_t)blockIdx.x * kLanes * U + threadIdx.x; base < total; base += stride) {
        f4 v[U];
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int64_t i = base + (int64_t)k * kLanes;
            v[k] = i < total ? load<NT>(src + i) : f4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const u4 b = __builtin_bit_cast(u4, v[k]);
            acc ^= b.x ^ b.y ^ b.z ^ b.w;
        }
    }
    if (acc == 0x9e3779b9u) sink[0] = acc;
}

template <bool NT, int U>
__global__ void __launch_bounds__(kLanes) write_kernel(f4 *dst, int64_t total) {
    const f4 v = {(float)threadIdx.x, 1.f, 2.f, 3.f};
    const int64_t stride = (int64_t)gridDim.x * kLanes * U;
    for (int64_t base = (int64_t)blockIdx.x * kLanes * U + threadIdx.x; base < total; base += stride) {
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int64_t i = base + (int64_t)k * kLanes;
            if (i < total) store<NT>(v, dst + i);
        }
    }
}

template <bool NT, int U>
__global__ void __launch_bounds__(kLanes) copy_kernel(const f4 *src, f4 *dst, int64_t total) {
    const int64_t stride = (int64_t)gridDim.x * kLanes * U;
    for (int64_t base = (int64_t)blockIdx.x * kLanes * U + threadIdx.x; base < total; base += stride) {
        f4 v[U];
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int64_t i = base + (int64_t)k * kLanes;
            if (i < total) v[k] = load<NT>(src + i);
        }
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int64_t i = base + (int64_t)k * kLanes;
            if (i < total) store<NT>(v[k], dst + i);
        }
    }
}

// The access pattern of a row operation with no arithmetic: one row per
// workgroup of LANES lanes, VPT vectors per lane of each stream, consecutive
// lanes on consecutive vectors; the input rows (a, and r when TWO_IN) are
// loaded, then the outputs (h, and y when TWO_OUT) are stored.
template <int LANES, int VPT, bool TWO_IN, bool TWO_OUT>
__global__ void __launch_bounds__(LANES) rows_kernel(const f4 *a, const f4 *r, f4 *h, f4 *y, int nvec) {
    const int64_t o = (int64_t)blockIdx.x * nvec;
    f4 va[VPT], vr[VPT];
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        const int i = k * LANES + (int)threadIdx.x;
        if (i < nvec) {
            va[k] = load<true>(a + o + i);
            vr[k] = TWO_IN ? load<true>(r + o + i) : va[k];
        }
    }
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        const int i = k * LANES + (int)threadIdx.x;
        if (i < nvec) store<true>(va[k] + vr[k], h + o + i);
    }
    if constexpr (TWO_OUT) {
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            const int i = k * LANES + (int)threadIdx.x;
            if (i < nvec) store<true>(va[k] - vr[k], y + o + i);
        }
    }
}

template <bool TWO_IN, bool TWO_OUT>
int launch_rows(const f4 *a, const f4 *r, f4 *h, f4 *y, unsigned rows, int nvec, int lanes, int vpt,
                hipStream_t stream) {
    if (lanes == 1024 && vpt == 1) rows_kernel<1024, 1, TWO_IN, TWO_OUT><<<rows, 1024, 0, stream>>>(a, r, h, y, nvec);
    else if (lanes == 1024 && vpt == 2) rows_kernel<1024, 2, TWO_IN, TWO_OUT><<<rows, 1024, 0, stream>>>(a, r, h, y, nvec);
    else if (lanes == 512 && vpt == 2) rows_kernel<512, 2, TWO_IN, TWO_OUT><<<rows, 512, 0, stream>>>(a, r, h, y, nvec);
    else if (lanes == 512 && vpt == 4) rows_kernel<512, 4, TWO_IN, TWO_OUT><<<rows, 512, 0, stream>>>(a, r, h, y, nvec);
    else if (lanes == 256 && vpt == 2) rows_kernel<256, 2, TWO_IN, TWO_OUT><<<rows, 256, 0, stream>>>(a, r, h, y, nvec);
    else if (lanes == 256 && vpt == 4) rows_kernel<256, 4, TWO_IN, TWO_OUT><<<rows, 256, 0, stream>>>(a, r, h, y, nvec);
    else if (lanes == 256 && vpt == 8) rows_kernel<256, 8, TWO_IN, TWO_OUT><<<rows, 256, 0, stream>>>(a, r, h, y, nvec);
    else return -1;
    return (int)hipGetLastError();
}

}  // namespace

extern "C" {

// The variants, by index:
//   0 read,  non-temporal loads, 8 vectors per lane per trip
//   1 write, default-policy stores, 1 vector per lane per trip
//   2 write, non-temporal stores, 1 vector per lane per trip
//   3 copy,  non-temporal loads and stores, 4 vectors per lane per trip
int stream_probe_variants(void) { return 4; }

// Enqueues variant `variant` on `stream` over `bytes` bytes (a multiple of 16)
// of `src` (read and copy) and `dst` (write and copy), device pointers
// aligned to 16 bytes; `sink` is a device word the read variant may write.
// grid <= 0 launches one workgroup per 256*U vectors (a single trip).
// Returns 0, -1 for an invalid argument (nothing enqueued) or the HIP error
// of the launch.
int stream_probe(int variant, const void *src, void *dst, unsigned *sink, int64_t bytes, int grid,
                 hipStream_t stream) {
    if (bytes <= 0 || bytes % 16 != 0 || variant < 0 || variant > 3) return -1;
    if ((variant != 1 && variant != 2 && (!src || (uintptr_t)src % 16)) ||
        (variant != 0 && (!dst || (uintptr_t)dst % 16)) || (variant == 0 && !sink))
        return -1;
    const int64_t total = bytes / 16;
    const int u = variant == 0 ? 8 : variant == 3 ? 4 : 1;
    const int64_t one_trip = (total + (int64_t)kLanes * u - 1) / ((int64_t)kLanes * u);
    const int64_t g = grid > 0 ? (grid < one_trip ? grid : one_trip) : one_trip;
    if (g > 0x7fffffff) return -1;
    const f4 *s = static_cast<const f4 *>(src);
    f4 *d = static_cast<f4 *>(dst);
    switch (variant) {
    case 0: read_kernel<true, 8><<<(unsigned)g, kLanes, 0, stream>>>(s, total, sink); break;
    case 1: write_kernel<false, 1><<<(unsigned)g, kLanes, 0, stream>>>(d, total); break;
    case 2: write_kernel<true, 1><<<(unsigned)g, kLanes, 0, stream>>>(d, total); break;
    default: copy_kernel<true, 4><<<(unsigned)g, kLanes, 0, stream>>>(s, d, total); break;
    }
    return (int)hipGetLastError();
}

// Enqueues a row operation's access pattern with no arithmetic on `stream`:
// rows of `nvec` 16-byte vectors, read from a (and r, if not NULL) and
// written to h (and y, if not NULL), one workgroup of `lanes` lanes per row
// with `vpt` vectors per lane of each stream. (lanes, vpt) is one of
// (1024, 1), (1024, 2), (512, 2), (512, 4), (256, 2), (256, 4), (256, 8), and
// lanes * vpt must cover nvec. Pointers are device pointers aligned to 16
// bytes. Returns 0, -1 for an invalid argument (nothing enqueued) or the HIP
// error of the launch.
int stream_probe_rows(const void *a, const void *r, void *h, void *y, int64_t rows, int64_t nvec, int lanes,
                      int vpt, hipStream_t stream) {
    if (rows <= 0 || rows > 0x7fffffff || nvec <= 0 || nvec > (int64_t)lanes * vpt) return -1;
    if (!a || !h) return -1;
    for (const void *p : {a, (const void *)r, (const void *)h, (const void *)y})
        if ((uintptr_t)p % 16) return -1;
    const f4 *fa = static_cast<const f4 *>(a), *fr = static_cast<const f4 *>(r);
    f4 *fh = static_cast<f4 *>(h), *fy = static_cast<f4 *>(y);
    const int nv = (int)nvec;
    const unsigned g = (unsigned)rows;
    if (r && y) return launch_rows<true, true>(fa, fr, fh, fy, g, nv, lanes, vpt, stream);
    if (r) return launch_rows<true, false>(fa, fr, fh, fy, g, nv, lanes, vpt, stream);
    if (y) return launch_rows<false, true>(fa, fr, fh, fy, g, nv, lanes, vpt, stream);
    return launch_rows<false, false>(fa, fr, fh, fy, g, nv, lanes, vpt, stream);
}

}  // extern "C"
