// snr_internal.h - types shared by the kernel translation unit and the host
// dispatch layer of libsnr. Not part of the public ABI (include/snr.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace snr {

enum Op : int {
    OP_PLAIN = 0,
    OP_TAIL = 1,
    OP_NORM_ADD = 2,
    OP_ADD_NORM = 3,
    OP_NORM_Q8 = 4  // RMSNorm, then Q8_1 records of the normalised row
};
enum Storage : int { ST_F32 = 0, ST_BF16 = 1, ST_F16 = 2 };
enum Kind : int {
    KIND_ROWTILE = 1,
    KIND_SPLIT = 2,
    KIND_MULTIPASS = 3,
    KIND_PERSIST = 4   // persistent row tile: same launcher signature
};

// Everything a row kernel needs.
//   OP_PLAIN:    x0 = x, g0 = gamma, out0 = y, eps0
//   OP_TAIL:     x0 = a, x1 = r, g0 = gamma_post, g1 = gamma_pre, out0 = h,
//                out1 = y, eps0 = eps_post, eps1 = eps_pre
//   OP_NORM_ADD: x0 = a, x1 = r, g0 = gamma, out0 = out, eps0, scale (device
//                pointer to one f32, or null for 1)
//   OP_ADD_NORM: x0 = a, x1 = b, g0 = gamma, out0 = s, out1 = y, eps0
struct RowArgs {
    const void *x0;
    const void *x1;
    const void *g0;
    const void *g1;
    void *out0;
    void *out1;
    const float *scale;
    float eps0;
    float eps1;
    int64_t rows;  // rows in the whole tensor
    int32_t n;     // elements per row
    int32_t nv;    // whole 128-bit vectors per row (n / W)
    int32_t rem;   // elements after the last whole vector (n % W)
};

// Several independent RMSNorms in one launch: segment s covers global rows
// [row_start[s], row_start[s + 1]) with its own tensors and epsilon; all
// segments share the row width and storage type.
constexpr int kMaxSegments = 8;
struct MultiArgs {
    const void *x[kMaxSegments];
    const void *g[kMaxSegments];
    void *y[kMaxSegments];
    float eps[kMaxSegments];
    int64_t row_start[kMaxSegments + 1];
    int32_t count;
    int32_t n;
    int32_t nv;
    int32_t rem;
};

// Cross-workgroup state of a split-row launch (see snr_split.hip for the
// protocol): slots[] in a workspace's device memory holds one tagged partial
// sum per (row of a launch, reduction, chunk); hdr[kHdrTimeouts] counts the
// waits that gave up; `tag` is the launch's tag (never 0).
constexpr int kHdrTimeouts = 0;
struct SplitState {
    unsigned long long *slots;  // [slot_cap] (tag << 32) | f32 partial
    unsigned int *hdr;          // hdr[kHdrTimeouts]: wait overruns
    int64_t slot_cap;           // slots available to one launch
    uint32_t spin_limit;        // polls before a wait gives up
    uint32_t tag;               // this launch's tag
};

// Row-tile launches of at most this many workgroups load the gains with the
// row (one memory round trip fewer per step; slower over many rows).
constexpr int64_t kEarlyBlocks = 16;

// Chunk geometry of the split-row kernels: 256 threads per workgroup and
// 4096 elements per chunk (4 vectors per lane in f32, 2 in 16-bit storage).
constexpr int kSplitBlock = 256;
constexpr int kSplitChunkElems = 4096;
constexpr int kSplitMaxChunks = 1024;

using RowtileLaunch = hipError_t (*)(const RowArgs &, int64_t row0,
                                     int64_t nrows, hipStream_t);
using SplitLaunch = hipError_t (*)(const RowArgs &, const SplitState &,
                                   int64_t row0, int64_t nrows, int chunks,
                                   int groups, bool cooperative, hipStream_t);
using OccupancyQuery = hipError_t (*)(int *blocks_per_cu);
// Workgroups the current device holds at once (cached; 0 when unknown).
using ResidentQuery = int64_t (*)();
using MultiLaunch = hipError_t (*)(const MultiArgs &, int64_t row0,
                                   int64_t nrows, hipStream_t);
using MultipassLaunch = hipError_t (*)(const RowArgs &, float *scratch,
                                       int64_t row0, int64_t nrows,
                                       int chunks, hipStream_t);

// Geometry of the multi-pass kernels: 256 threads x 16 vectors per chunk
// (16384 f32 or 32768 16-bit elements).
constexpr int kMultiBlock = 256;
constexpr int kMultiVpt = 16;

struct KernelEntry {
    int op;        // Op
    int storage;   // Storage
    int width;     // elements per 128-bit vector (4 f32, 8 bf16/f16)
    int kind;      // Kind
    int g;         // lanes per row (rowtile) / workgroup size (split)
    int vpt;       // loads held per lane
    int block;     // threads per workgroup
    RowtileLaunch rowtile;
    SplitLaunch split;
    OccupancyQuery occupancy;
    MultipassLaunch multipass;
    MultiLaunch multi;   // several segments in one launch (row tile only)
    ResidentQuery resident = nullptr;  // row tiles and persistent tiles
};

// The tables of compiled kernels: RMSNorm, the tail and its halves
// (snr_kernels.hip), and RMSNorm into Q8_1 records (snr_q8.hip).
const KernelEntry *kernel_table(int *count);
const KernelEntry *q8_kernel_table(int *count);
const KernelEntry *persist_kernel_table(int *count);   // snr_persist.hip
const KernelEntry *split_kernel_table(int *count);     // snr_split.hip

// The calling thread's cap on rows in flight (snr_force_grid; 0: none): the
// persistent tiles launch at most this many workgroups.
int64_t forced_grid_cap();

// Set `words` 32-bit words to `value` with a kernel (used instead of a
// memset so that the call can also be recorded into a HIP graph).
hipError_t fill_words(void *p, int64_t words, unsigned int value,
                      hipStream_t stream);

}  // namespace snr
