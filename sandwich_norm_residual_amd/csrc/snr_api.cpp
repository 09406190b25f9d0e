// snr_api.cpp - the C ABI of libsnr (declared in include/snr.h): argument
// validation, dispatch-shape selection, the split-row workspace and the
// kernel launches. Host code only; the kernels live in snr_kernels.hip (row
// tiles, multi-pass), snr_persist.hip (persistent row tiles), snr_split.hip
// (split rows) and snr_q8.hip (RMSNorm into Q8_1 records).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <initializer_list>
#include <map>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "snr.h"
#include "snr_internal.h"

namespace snr {
namespace {

thread_local int t_last_hip_error = 0;
thread_local int t_force_kind = SNR_SHAPE_AUTO;
thread_local int t_force_g = 0;
thread_local int t_force_vpt = 0;
thread_local int64_t t_force_grid = 0;   // snr_force_grid; 0: no cap
thread_local char t_last_shape[64] = "";

int hip_fail(hipError_t e) {
    t_last_hip_error = (int)e;
    return SNR_ERR_HIP;
}

}  // namespace

int64_t forced_grid_cap() { return t_force_grid; }

namespace {

bool debug_enabled() {
    static const bool on = [] {
        const char *v = std::getenv("SNR_DEBUG");
        return v && *v && std::strcmp(v, "0") != 0;
    }();
    return on;
}

// ---------------------------------------------------------------------------
// Device facts (cached per device ordinal)
// ---------------------------------------------------------------------------
struct DeviceInfo {
    bool ok = false;   // gfx950
    int cus = 0;
};

std::mutex g_dev_mu;
std::map<int, DeviceInfo> g_dev;

// The current device, which must be a gfx950 and own `stream`: the
// workspace, the occupancy figures and the device check all follow the
// current device, while HIP runs the kernels on the stream's device.
int current_device(hipStream_t stream, int *dev, DeviceInfo *info) {
    hipError_t e = hipGetDevice(dev);
    if (e != hipSuccess) return hip_fail(e);
    if (stream) {
        hipDevice_t owner = 0;
        e = hipStreamGetDevice(stream, &owner);
        if (e != hipSuccess) return hip_fail(e);
        if (owner != *dev) return SNR_ERR_DEVICE;
    }
    std::lock_guard<std::mutex> lk(g_dev_mu);
    auto it = g_dev.find(*dev);
    if (it == g_dev.end()) {
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, *dev);
        if (e != hipSuccess) return hip_fail(e);
        DeviceInfo d;
        d.ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
        d.cus = prop.multiProcessorCount;
        it = g_dev.emplace(*dev, d).first;
    }
    *info = it->second;
    return info->ok ? SNR_OK : SNR_ERR_DEVICE;
}

// ---------------------------------------------------------------------------
// Workspaces: the split-row kernels' tagged partial-sum slots and the
// multi-pass kernels' scratch, 1 MiB of device memory each:
//   [0, 256)                 header: the count of waits that gave up
//   [256, 256 + 256 KiB)     32768 slots of 8 bytes (split-row kernels)
//   [256 + 256 KiB, 1 MiB)   196544 floats (multi-pass partial sums and
//                            inverse norms)
// A device has at most kMaxWorkspaces of them, each bound to one stream at a
// time. Every use of a workspace on an eagerly running stream is enqueued
// after a wait on the event recorded after its previous use (on whichever
// stream that was) and followed by a new record, all under g_ws_mu, so two
// uses of one workspace never overlap on the GPU. A new stream takes a free
// workspace, or the least recently used one that no captured graph holds.
// A stream that is being captured into a HIP graph may use only the
// workspace it already holds (allocation and cross-stream waits cannot be
// captured); that workspace is then pinned to it for the life of the
// process, because the graph may be replayed at any time.
// ---------------------------------------------------------------------------
constexpr int64_t kWorkspaceBytes = int64_t(1) << 20;
constexpr int64_t kHeaderBytes = 256;
constexpr int64_t kSlotWords = 32768;
constexpr int64_t kMultiOffset = kHeaderBytes + kSlotWords * 8;
constexpr int64_t kMultiFloats = (kWorkspaceBytes - kMultiOffset) / 4;
constexpr uint32_t kSpinLimit = 1u << 22;   // polls before a wait gives up
constexpr int kMaxWorkspaces = 8;           // per device
// The library's events only order work on one device: a device-scope
// release on record (the default, a system-scope one, writes back caches
// between back-to-back wide-row calls).
constexpr unsigned kEventFlags = hipEventDisableTiming | hipEventReleaseToDevice;

struct Workspace {
    void *base = nullptr;
    hipEvent_t last_use = nullptr;  // recorded after each eager use
    hipStream_t stream = nullptr;   // the stream it is bound to
    uint64_t stamp = 0;             // last use, for eviction
    bool pinned = false;            // captured into a graph
    uint32_t next_tag = 1;          // the next split-row launch's tag
    bool uncleared = false;         // static scratch not yet cleared eagerly
};

std::mutex g_ws_mu;   // guards g_ws, g_ws_clock and every workspace use
std::map<int, std::vector<Workspace>> g_ws;
uint64_t g_ws_clock = 0;

SplitState split_state(void *base) {
    char *b = static_cast<char *>(base);
    SplitState st{};
    st.hdr = reinterpret_cast<unsigned int *>(b);
    st.slots = reinterpret_cast<unsigned long long *>(b + kHeaderBytes);
    st.slot_cap = kSlotWords;
    st.spin_limit = kSpinLimit;
    // Test hook: a small poll budget (0: none) forces the bounded-wait path.
    if (const char *lim = std::getenv("SNR_SPLIT_SPIN_LIMIT")) {
        char *end = nullptr;
        const long v = std::strtol(lim, &end, 10);
        if (end != lim && v >= 0 && v <= (long)UINT32_MAX)
            st.spin_limit = (uint32_t)v;
    }
    return st;
}

float *multi_scratch(void *base) {
    return reinterpret_cast<float *>(static_cast<char *>(base) + kMultiOffset);
}

bool capturing(hipStream_t stream) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    return hipStreamIsCapturing(stream, &cs) == hipSuccess &&
           cs != hipStreamCaptureStatusNone;
}

// A zeroed workspace. Its first tag is 1, or SNR_SPLIT_EPOCH + 1 when that
// is given (a test hook: a value near 2^31 - 1 makes the next launches wrap
// the tags).
int new_workspace(hipStream_t stream, Workspace *w) {
    hipError_t e = hipMalloc(&w->base, (size_t)kWorkspaceBytes);
    if (e != hipSuccess) {
        t_last_hip_error = (int)e;
        w->base = nullptr;
        return SNR_ERR_WORKSPACE;
    }
    e = hipEventCreateWithFlags(&w->last_use, kEventFlags);
    if (e == hipSuccess)
        e = fill_words(w->base, kWorkspaceBytes / 4, 0u, stream);
    if (e != hipSuccess) {
        if (w->last_use) (void)hipEventDestroy(w->last_use);
        (void)hipFree(w->base);
        *w = Workspace{};
        return hip_fail(e);
    }
    if (const char *ep = std::getenv("SNR_SPLIT_EPOCH"))
        w->next_tag = (uint32_t)std::strtoul(ep, nullptr, 10) + 1u;
    return SNR_OK;
}

// The tag of the next split-row launch on a workspace whose slots are at
// `slots` (caller holds g_ws_mu). Eager launches take 1, 2, ...,
// 2^31 - 1; before these wrap to 1 again, every slot is cleared on the
// stream (after every earlier use of the workspace, which the caller's
// stream is ordered after). Launches recorded into a graph all take
// kCapturedTag, outside that range, and the caller records a clear of the
// launch's slots before each of them: a replay's leftovers never carry an
// eager launch's tag, and every replay starts from cleared slots.
constexpr uint32_t kCapturedTag = 0x80000000u;

hipError_t take_tag(Workspace *w, unsigned long long *slots, bool eager,
                    hipStream_t stream, uint32_t *tag) {
    if (!eager) {
        *tag = kCapturedTag;
        return hipSuccess;
    }
    if (w->next_tag == 0 || w->next_tag >= kCapturedTag) {
        const hipError_t e = fill_words(slots, kSlotWords * 2, 0u, stream);
        if (e != hipSuccess) return e;
        w->next_tag = 1;
    }
    *tag = w->next_tag++;
    return hipSuccess;
}

// The workspace `stream` uses on device `dev` (caller holds g_ws_mu). Sets
// *eager to whether the stream runs eagerly (not under capture); for an
// eager stream the caller waits on w->last_use before its launches and
// records it after them.
int acquire_workspace(int dev, hipStream_t stream, Workspace **out,
                      bool *eager) {
    const bool cap = capturing(stream);
    *eager = !cap;
    std::vector<Workspace> &pool = g_ws[dev];
    for (Workspace &w : pool)
        if (w.base && w.stream == stream) {
            if (cap) w.pinned = true;
            w.stamp = ++g_ws_clock;
            *out = &w;
            return SNR_OK;
        }
    if (cap) return SNR_ERR_CAPTURE;
    // a slot released by snr_release_workspaces, a new slot, or else the
    // least recently used workspace
    Workspace *w = nullptr;
    for (Workspace &c : pool)
        if (!c.base) {
            w = &c;
            break;
        }
    if (!w && (int)pool.size() < kMaxWorkspaces) {
        pool.reserve(kMaxWorkspaces);   // pointers into the pool stay valid
        pool.push_back(Workspace{});
        w = &pool.back();
    }
    if (w) {
        Workspace fresh;
        const int rc = new_workspace(stream, &fresh);
        if (rc != SNR_OK) return rc;
        *w = fresh;
    } else {
        for (Workspace &c : pool)
            if (!c.pinned && (!w || c.stamp < w->stamp)) w = &c;
        if (!w) return SNR_ERR_WORKSPACE;   // every workspace is pinned
    }
    w->stream = stream;
    w->stamp = ++g_ws_clock;
    *out = w;
    return SNR_OK;
}

// Cooperative launches of the split-row kernels (SNR_SPLIT_COOPERATIVE set
// and not "0"): the runtime then checks and guarantees that the whole grid
// is resident, at a cost of about 14 us per launch on MI355X. By default the
// launch is ordinary, with the grid sized to the occupancy-derived resident
// count and split-row launches serialised per device.
bool split_cooperative() {
    const char *v = std::getenv("SNR_SPLIT_COOPERATIVE");
    return v && *v && std::strcmp(v, "0") != 0;
}

// The workspace whose last_use event marks the latest eager split-row launch
// on a device (caller holds g_ws_mu). One record per call serves both
// orders: each record costs about 3.5 us between back-to-back calls.
std::map<int, Workspace *> g_split_last;

// Order `stream` after the work an event marks. (Also when the event was
// recorded on `stream` itself: a destroyed stream's handle can come back as
// a new stream's while the old stream's work still runs.)
hipError_t wait_for(hipStream_t stream, hipEvent_t ev) {
    return hipStreamWaitEvent(stream, ev, 0);
}

// ---------------------------------------------------------------------------
// Validation helpers
// ---------------------------------------------------------------------------
bool overlaps(const void *p, int64_t pb, const void *q, int64_t qb) {
    if (!p || !q || pb <= 0 || qb <= 0) return false;
    const uintptr_t a = (uintptr_t)p, b = (uintptr_t)q;
    return a < b + (uintptr_t)qb && b < a + (uintptr_t)pb;
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

bool eps_ok(float e) { return std::isfinite(e) && e > 0.0f; }

int check_shape(int64_t rows, int64_t n, int64_t esize) {
    if (rows < 0 || n < 1 || n > INT32_MAX) return SNR_ERR_SHAPE;
    if (rows > 0 && rows > (INT64_MAX / esize) / n) return SNR_ERR_SHAPE;
    return SNR_OK;
}

// ---------------------------------------------------------------------------
// Shape selection
// ---------------------------------------------------------------------------
struct Choice {
    const KernelEntry *k = nullptr;
    int chunks = 0;  // split only
};

// The compiled kernels of an operation and kind: RMSNorm into Q8_1 records
// and the persistent row tiles have their own sources and tables.
const KernelEntry *table_for(int op, int kind, int *count) {
    if (op == OP_NORM_Q8) return q8_kernel_table(count);
    if (kind == KIND_PERSIST) return persist_kernel_table(count);
    if (kind == KIND_SPLIT) return split_kernel_table(count);
    return kernel_table(count);
}

const KernelEntry *find_entry(int op, int st, int w, int kind, int g,
                              int vpt) {
    int count = 0;
    const KernelEntry *t = table_for(op, kind, &count);
    // the split-row kernels have one geometry per storage type
    const bool by_g = kind == KIND_ROWTILE || kind == KIND_PERSIST;
    const bool by_vpt = kind != KIND_SPLIT;
    for (int i = 0; i < count; ++i)
        if (t[i].op == op && t[i].storage == st && t[i].width == w &&
            t[i].kind == kind && (!by_g || t[i].g == g) &&
            (!by_vpt || t[i].vpt == vpt))
            return &t[i];
    return nullptr;
}

int split_chunks(const KernelEntry *k, int64_t nv) {
    const int64_t per = (int64_t)kSplitBlock * k->vpt;
    const int64_t c = (nv + per - 1) / per;
    return (int)(c > 0 ? c : 1);  // a row of only remainder elements
}

// `rows` is the launch's row count (0 where the caller needs a row tile:
// the several-segment launch).
int choose(int op, int st, int w, int64_t nv, int rem, int64_t rows,
           Choice *c) {
    if (t_force_kind == SNR_SHAPE_PERSIST) {
        if (op == OP_NORM_Q8 || rem != 0) return SNR_ERR_SHAPE;
        c->k = find_entry(op, st, w, KIND_PERSIST, t_force_g, t_force_vpt);
        if (!c->k || (int64_t)c->k->g * c->k->vpt < nv) return SNR_ERR_SHAPE;
        return SNR_OK;
    }
    if (t_force_kind == SNR_SHAPE_ROWTILE) {
        c->k = find_entry(op, st, w, KIND_ROWTILE, t_force_g, t_force_vpt);
        if (!c->k || (int64_t)c->k->g * c->k->vpt < nv) return SNR_ERR_SHAPE;
        return SNR_OK;
    }
    if (t_force_kind == SNR_SHAPE_SPLIT) {
        c->k = find_entry(op, st, w, KIND_SPLIT, 0, t_force_vpt);
        if (!c->k) return SNR_ERR_SHAPE;
        c->chunks = split_chunks(c->k, nv);
        return SNR_OK;
    }
    if (t_force_kind == SNR_SHAPE_MULTIPASS) {
        c->k = find_entry(op, st, w, KIND_MULTIPASS, 0, kMultiVpt);
        if (!c->k) return SNR_ERR_SHAPE;
        c->chunks = split_chunks(c->k, nv);
        return SNR_OK;
    }
    if (op == OP_NORM_Q8 && nv <= 128) {
        // Q8_1 records need each 32-element block inside one lane group.
        // About two vectors per lane measured best for short rows (at
        // least 8 lanes unless the row is a single block; at most 32):
        // 65536 x 512 bf16 took 25.8 us at 32 x 4 against 31.5 us at 16 x 4.
        int g = 32 / w;
        while (2 * g < nv) g *= 2;
        if (g < 8 && nv > g) g = 8;
        if (g > 32) g = 32;
        c->k = find_entry(op, st, w, KIND_ROWTILE, g, 4);
        return c->k ? SNR_OK : SNR_ERR_SHAPE;
    }
    if (nv <= 128) {
        // several rows per wavefront: 4 vectors per lane
        int g = 1;
        while (g * 4 < nv) g *= 2;
        c->k = find_entry(op, st, w, KIND_ROWTILE, g, 4);
        return c->k ? SNR_OK : SNR_ERR_SHAPE;
    }
    // Wider rows: about two loads per lane, so each row is fetched by as
    // many lanes as possible (G = nv/2 rounded up to a power of two, 64 to
    // 1024 lanes), with the smallest compiled register tile that holds it.
    int g = 64;
    while (g < 1024 && 2LL * g < nv) g *= 2;
    int count = 0;
    const KernelEntry *t = table_for(op, KIND_ROWTILE, &count);
    const KernelEntry *best = nullptr;
    for (int i = 0; i < count; ++i) {
        const KernelEntry &e = t[i];
        if (e.op != op || e.storage != st || e.width != w ||
            e.kind != KIND_ROWTILE || e.g != g || (int64_t)e.g * e.vpt < nv)
            continue;
        if (!best || e.vpt < best->vpt) best = &e;
    }
    if (!best) {
        // no register tile holds the row: split it across workgroups (or,
        // for an operation without a split kernel, use the multi-pass one)
        c->k = find_entry(op, st, w, KIND_SPLIT, 0, 0);
        if (!c->k) c->k = find_entry(op, st, w, KIND_MULTIPASS, 0, kMultiVpt);
        if (!c->k) return SNR_ERR_SHAPE;
        c->chunks = split_chunks(c->k, nv);
        return SNR_OK;
    }
    // Launches of a few rows are a chain of dependent memory round trips.
    // There the 512 x 4 tile measured faster than 1024 x 2 in f32 for the
    // tail, the plain norm and norm_then_add (1 to 16 rows of 4608, 6656
    // and 8192: tail 3.25 -> 3.12 us at one row of 6656, plain 2.28 ->
    // 2.21, norm_then_add 2.49 -> 2.41), and slower for add_then_norm (2.78
    // -> 2.93), whose first phase also stores the sum. What helps is leaving
    // the 16-wavefront workgroup: halving 512 x 2 into 256 x 4 was 5-15%
    // slower for every operation (one row of 4096: tail 2.68 -> 2.85 us).
    // RMSNorm into Q8_1 records was not measured this way and keeps its
    // tile.
    if (st == ST_F32 && op != OP_ADD_NORM && op != OP_NORM_Q8 &&
        best->g == 1024 &&
        best->vpt == 2 && rows > 0 && rows <= kEarlyBlocks) {
        const KernelEntry *half = find_entry(op, st, w, KIND_ROWTILE, 512, 4);
        if (half && 512LL * 4 >= nv) best = half;
    }
    c->k = best;
    // The persistent form of the same tile (loads of the next row in flight
    // through this row's reductions) measured faster for:
    // * the 16-bit tail and its halves with 512 or more lanes per row
    //   (4096 x 6656: bf16 tail 43.1 -> 40.9 us, norm_then_add 32.4 -> 30.0);
    // * the 16-bit plain norm with 1024 lanes per row over 256 rows or more
    //   (n = 16384 bf16: 1024 rows 14.6 -> 12.5 us, 8192 rows 93.8 -> 88.7;
    //   n = 24576: 1024 rows 19.2 -> 17.7 us);
    // * the f32 plain norm at 1024 x 4 over 1024 rows or more (n = 16384:
    //   1024 rows 24.9 -> 22.1 us, 4096 rows 93.9 -> 85.3), and at 1024 x 2
    //   when the row fills the tile (n = 8192: 1024 rows 13.7 -> 12.9 us,
    //   16384 rows 186.4 -> 181.1).
    // It measured slower or no faster for the f32 tail and its halves, for
    // the f32 plain norm with fewer rows (256 x 16384: 6.97 -> 7.30 us) or
    // a partly filled 1024 x 2 tile (n = 6656 and 7168: within 1.5% either
    // way), for the plain norm with 512 lanes (slower at 1024 and 16384 rows
    // of 6656 bf16, faster between), and for smaller groups, whose rows are
    // shorter than the loop's fixed cost. It needs rows without a ragged
    // end.
    const bool halves = st != ST_F32 && best->g >= 512 &&
                        (op == OP_TAIL || op == OP_NORM_ADD || op == OP_ADD_NORM);
    const bool f32_tile = best->vpt == 4 || (best->vpt == 2 && nv == 2048);
    const bool wide_plain =
        op == OP_PLAIN && best->g == 1024 &&
        (st != ST_F32 ? rows >= 256 : f32_tile && rows >= 1024);
    if (rem == 0 && (halves || wide_plain)) {
        const KernelEntry *pk =
            find_entry(op, st, w, KIND_PERSIST, best->g, best->vpt);
        // Not where the row tile holds every row at once and the persistent
        // grid, whose larger register tile fits fewer workgroups, would take
        // them in two or more rounds with little to overlap. At 6656 bf16
        // (row tile 1024 resident; persistent 512 for the tail, 768 for its
        // halves), persistent against row tile: the tail 8.63 -> 7.68 us at
        // 640 rows and 11.27 -> 10.01 at 1024, norm_then_add 9.13 -> 7.84
        // and add_then_norm 11.43 -> 10.34 at 1024 rows; f16 plain at 12288
        // (512 against 256 resident) 5.65 -> 4.89 us at 300 rows. At 1024
        // lanes (16384 bf16) it is mixed: the tail 10.30 -> 9.43 us at 300
        // rows but 10.87 -> 11.33 at 512, add_then_norm 2-5% slower.
        const int64_t rt = best->resident ? best->resident() : 0;
        const int64_t pr = pk && pk->resident ? pk->resident() : 0;
        const bool one_round = rt > 0 && pr > 0 && rows > pr && rows <= rt;
        // Nor for a few rows at 1024 lanes, where the row tile with its gains
        // loaded with the row is as fast or faster (one row of 12288 bf16:
        // tail 4.25 -> 3.70 us; of 16384 within 2%), while at 512 lanes the
        // persistent tile is (one row of 6656 bf16: 2.92 against 3.32 us).
        const bool few_wide = best->g == 1024 && rows > 0 && rows <= kEarlyBlocks;
        if (pk && !one_round && !few_wide) c->k = pk;
    }
    return SNR_OK;
}

// ---------------------------------------------------------------------------
// The allocation-free entry point's scratch (sandwich_tail_noalloc): the
// file-scope device array `scratch` (one copy per device, laid out as a
// workspace), whose device address is looked up once per device at that
// entry point's first call there. Its tag counter lives with the address.
// ---------------------------------------------------------------------------
constexpr int kMaxScratchDevices = 64;
Workspace g_scratch_ws[kMaxScratchDevices];   // base == nullptr: not set up

}  // namespace
}  // namespace snr

static __device__ __align__(256) unsigned char scratch[snr::kWorkspaceBytes];

namespace snr {
namespace {

// The device address of `scratch` on device `dev`, looked up on the first
// call there, and the array cleared by the first eager call: its slots and
// overrun count start at zero before an eager launch takes tag 1. (A call
// recorded into a graph clears the slots its launch uses inside the graph,
// and the multi-pass scratch is written before it is read.) Caller holds
// g_ws_mu; `dev` is the current device.
int setup_scratch(int dev, hipStream_t stream) {
    if (dev < 0 || dev >= kMaxScratchDevices) return SNR_ERR_DEVICE;
    Workspace &w = g_scratch_ws[dev];
    if (!w.base) {
        void *ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e);
        w.base = ptr;
        w.next_tag = 1;
        w.uncleared = true;
    }
    if (w.uncleared && !capturing(stream)) {
        const hipError_t e = fill_words(w.base, kWorkspaceBytes / 4, 0u, stream);
        if (e != hipSuccess) return hip_fail(e);
        w.uncleared = false;
        w.next_tag = 1;
    }
    return SNR_OK;
}

int scratch_workspace(int dev, Workspace **out) {
    if (dev < 0 || dev >= kMaxScratchDevices || !g_scratch_ws[dev].base)
        return SNR_ERR_WORKSPACE;
    *out = &g_scratch_ws[dev];
    return SNR_OK;
}

// ---------------------------------------------------------------------------
// Launch
// ---------------------------------------------------------------------------
int launch(int op, int st, int64_t esize, const RowArgs &args_in,
           hipStream_t stream, bool use_scratch = false) {
    int dev = 0;
    DeviceInfo info;
    int rc = current_device(stream, &dev, &info);
    if (rc != SNR_OK) return rc;

    // 128-bit vectors need only element alignment on gfx950; the n % w
    // elements after a row's last whole vector are handled one by one.
    const int w = (int)(16 / esize);
    RowArgs a = args_in;
    a.nv = (int32_t)(a.n / w);
    a.rem = (int32_t)(a.n % w);
    Choice c;
    rc = choose(op, st, w, a.nv, a.rem, a.rows, &c);
    if (rc != SNR_OK) return rc;
    const KernelEntry *k = c.k;

    if (k->kind == KIND_SPLIT) {
        // The split grid needs every chunk of a row co-resident; rows
        // wider than that go through the multi-pass kernels instead (unless
        // the split shape was forced, which then fails).
        int per_cu = 0;
        hipError_t e = k->occupancy(&per_cu);
        if (e != hipSuccess) return hip_fail(e);
        const bool fits = c.chunks <= kSplitMaxChunks &&
                          (int64_t)per_cu * info.cus >= c.chunks;
        if (!fits) {
            if (t_force_kind == SNR_SHAPE_SPLIT) return SNR_ERR_WORKSPACE;
            k = find_entry(op, st, w, KIND_MULTIPASS, 0, kMultiVpt);
            if (!k) return SNR_ERR_SHAPE;
            c.chunks = split_chunks(k, a.nv);
        }
    }

    if (k->kind == KIND_ROWTILE || k->kind == KIND_PERSIST) {
        const int rpb = k->block / k->g;
        const int64_t max_blocks = (int64_t)(UINT32_MAX / (uint32_t)k->block);
        const int64_t step = max_blocks * rpb;
        for (int64_t r0 = 0; r0 < a.rows; r0 += step) {
            const int64_t nr = a.rows - r0 < step ? a.rows - r0 : step;
            hipError_t e = k->rowtile(a, r0, nr, stream);
            if (e != hipSuccess) return hip_fail(e);
        }
    } else {
        // Split-row and multi-pass launches use a workspace: the whole
        // sequence is enqueued under the workspace lock, after the wait on
        // its previous use and before the record of this one (which also
        // marks the device's latest split-row launch).
        // The allocation-free entry point uses its device's static scratch
        // instead, with no events (its calls must not overlap on a device).
        std::lock_guard<std::mutex> lk(g_ws_mu);
        Workspace *ws = nullptr;
        bool eager = !capturing(stream);
        bool events = false;
        if (use_scratch) {
            rc = scratch_workspace(dev, &ws);
        } else {
            rc = acquire_workspace(dev, stream, &ws, &eager);
            events = eager;
        }
        if (rc != SNR_OK) return rc;
        if (events) {
            hipError_t e = wait_for(stream, ws->last_use);
            if (e != hipSuccess) return hip_fail(e);
        }
        hipError_t e = hipSuccess;
        if (k->kind == KIND_MULTIPASS) {
            // partial sums (rows x chunks) and inverse norms (rows) must fit
            // the scratch; each pass's grid (rows x chunks workgroups) must
            // fit a launch
            int64_t step = kMultiFloats / (c.chunks + 1);
            const int64_t max_grid = (int64_t)(UINT32_MAX / (uint32_t)k->block);
            if (step * c.chunks > max_grid) step = max_grid / c.chunks;
            if (step < 1) return use_scratch ? SNR_ERR_WORKSPACE : SNR_ERR_SHAPE;
            float *scratch = multi_scratch(ws->base);
            for (int64_t r0 = 0; r0 < a.rows && e == hipSuccess; r0 += step) {
                const int64_t nr = a.rows - r0 < step ? a.rows - r0 : step;
                e = k->multipass(a, scratch, r0, nr, c.chunks, stream);
            }
        } else {
            int per_cu = 0;
            e = k->occupancy(&per_cu);
            if (e != hipSuccess) return hip_fail(e);
            // Every workgroup of the grid must be resident at once: at most
            // floor(capacity / chunks) rows are in flight (fewer under
            // snr_force_grid: each workgroup then walks more rows).
            int64_t max_groups = (int64_t)per_cu * info.cus / c.chunks;
            if (max_groups < 1) return SNR_ERR_WORKSPACE;
            if (t_force_grid > 0 && t_force_grid < max_groups)
                max_groups = t_force_grid;
            const SplitState st = split_state(ws->base);
            // each launch's rows x reductions x chunks slots fit the slots
            const int64_t nph = op == OP_TAIL ? 2 : 1;
            const int64_t step = st.slot_cap / (c.chunks * nph);
            if (step < 1) return use_scratch ? SNR_ERR_WORKSPACE : SNR_ERR_SHAPE;
            // Split-row launches never overlap one another on a device, on
            // any stream: two grids that each fill the device could then
            // each be partly resident, waiting for workgroups the other
            // keeps out. (Under capture the graph's stream order is the
            // caller's to keep.)
            if (events) {
                Workspace *prev = g_split_last[dev];
                if (prev && prev != ws) {
                    e = wait_for(stream, prev->last_use);
                    if (e != hipSuccess) return hip_fail(e);
                }
                g_split_last[dev] = ws;   // its record below marks this launch
            }
            const bool coop = split_cooperative();
            for (int64_t r0 = 0; r0 < a.rows && e == hipSuccess; r0 += step) {
                const int64_t nr = a.rows - r0 < step ? a.rows - r0 : step;
                const int groups = (int)(nr < max_groups ? nr : max_groups);
                SplitState sl = st;
                e = take_tag(ws, st.slots, eager, stream, &sl.tag);
                // a replay repeats the captured tag: clear the slots this
                // launch uses first (a kernel, recorded with it)
                if (e == hipSuccess && !eager)
                    e = fill_words(st.slots, nr * nph * c.chunks * 2, 0u,
                                   stream);
                if (e == hipSuccess)
                    e = k->split(a, sl, r0, nr, c.chunks, groups, coop, stream);
            }
        }
        if (e == hipSuccess && events) e = hipEventRecord(ws->last_use, stream);
        if (e != hipSuccess) return hip_fail(e);
    }
    if (k->kind == KIND_ROWTILE || k->kind == KIND_PERSIST)
        std::snprintf(t_last_shape, sizeof t_last_shape, "%s:%d:%d:%d",
                      k->kind == KIND_ROWTILE ? "rowtile" : "persist", k->g,
                      k->vpt, w);
    else
        std::snprintf(t_last_shape, sizeof t_last_shape, "%s:%d:%d:%d:%d",
                      k->kind == KIND_SPLIT ? "split" : "multipass", k->g,
                      k->vpt, w, c.chunks);
    if (debug_enabled())
        std::fprintf(stderr, "[snr] %s rows=%lld n=%d -> %s\n",
                     op == OP_TAIL       ? "sandwich_tail"
                     : op == OP_NORM_ADD ? "norm_then_add"
                     : op == OP_ADD_NORM ? "add_then_norm"
                     : op == OP_NORM_Q8  ? "rmsnorm_q8_1"
                                         : "rmsnorm_fwd",
                     (long long)a.rows, a.n, t_last_shape);
    t_last_hip_error = 0;
    return SNR_OK;
}

// Storage of a dtype code and its element size (0 when the code is invalid).
int storage_of(int dtype, int64_t *esize) {
    switch (dtype) {
    case SNR_F32: *esize = 4; return ST_F32;
    case SNR_BF16: *esize = 2; return ST_BF16;
    case SNR_F16: *esize = 2; return ST_F16;
    default: *esize = 0; return -1;
    }
}

// Common front of the two-input operations: shape, epsilons, nulls,
// element alignment. Returns SNR_OK, an error, or -1 for "rows == 0, done".
int check_common(int64_t rows, int64_t n, int64_t es,
                 std::initializer_list<float> eps,
                 std::initializer_list<const void *> ptrs) {
    int rc = check_shape(rows, n, es);
    if (rc != SNR_OK) return rc;
    for (float e : eps)
        if (!eps_ok(e)) return SNR_ERR_EPS;
    if (rows == 0) return -1;
    for (const void *p : ptrs)
        if (!p) return SNR_ERR_NULL;
    for (const void *p : ptrs)
        if (!aligned(p, (uintptr_t)es)) return SNR_ERR_ALIGN;
    return SNR_OK;
}

int tail_impl(const void *a, const void *r, const void *gamma_post,
              float eps_post, const void *gamma_pre, float eps_pre,
              void *h_out, void *y_out, int64_t rows, int64_t n, int dtype,
              hipStream_t stream, bool use_scratch = false) {
    int64_t es = 0;
    const int st = storage_of(dtype, &es);
    if (st < 0) return SNR_ERR_DTYPE;
    int rc = check_common(rows, n, es, {eps_post, eps_pre},
                          {a, r, gamma_post, gamma_pre, h_out, y_out});
    if (rc != SNR_OK) return rc < 0 ? SNR_OK : rc;
    const int64_t tb = rows * n * es, gb = n * es;
    // y_out may overlap nothing; h_out may only coincide exactly with r.
    if (overlaps(y_out, tb, a, tb) || overlaps(y_out, tb, r, tb) ||
        overlaps(y_out, tb, h_out, tb) || overlaps(y_out, tb, gamma_post, gb) ||
        overlaps(y_out, tb, gamma_pre, gb))
        return SNR_ERR_ALIAS;
    if (overlaps(h_out, tb, a, tb) || overlaps(h_out, tb, gamma_post, gb) ||
        overlaps(h_out, tb, gamma_pre, gb))
        return SNR_ERR_ALIAS;
    if (h_out != r && overlaps(h_out, tb, r, tb)) return SNR_ERR_ALIAS;

    RowArgs args{};
    args.x0 = a;
    args.x1 = r;
    args.g0 = gamma_post;
    args.g1 = gamma_pre;
    args.out0 = h_out;
    args.out1 = y_out;
    args.eps0 = eps_post;
    args.eps1 = eps_pre;
    args.rows = rows;
    args.n = (int32_t)n;
    if (use_scratch) {
        int dev = 0;
        DeviceInfo info;
        rc = current_device(stream, &dev, &info);
        if (rc != SNR_OK) return rc;
        std::lock_guard<std::mutex> lk(g_ws_mu);
        rc = setup_scratch(dev, stream);
        if (rc != SNR_OK) return rc;
    }
    return launch(OP_TAIL, st, es, args, stream, use_scratch);
}

}  // namespace
}  // namespace snr

using namespace snr;

static_assert(SNR_MAX_SEGMENTS == kMaxSegments,
              "segment table size differs between the ABI and the kernels");

extern "C" {

int rmsnorm_fwd(const void *x, const void *gamma, float eps, int64_t rows,
                int64_t n, int dtype, void *y, hipStream_t stream) {
    int64_t es = 0;
    const int st = storage_of(dtype, &es);
    if (st < 0) return SNR_ERR_DTYPE;
    int rc = check_common(rows, n, es, {eps}, {x, gamma, y});
    if (rc != SNR_OK) return rc < 0 ? SNR_OK : rc;
    const int64_t tb = rows * n * es, gb = n * es;
    if (y != x && overlaps(y, tb, x, tb)) return SNR_ERR_ALIAS;
    if (overlaps(y, tb, gamma, gb)) return SNR_ERR_ALIAS;

    RowArgs a{};
    a.x0 = x;
    a.g0 = gamma;
    a.out0 = y;
    a.eps0 = eps;
    a.rows = rows;
    a.n = (int32_t)n;
    return launch(OP_PLAIN, st, es, a, stream);
}

int sandwich_tail(const float *a, const float *r, const float *gamma_post,
                  float eps_post, const float *gamma_pre, float eps_pre,
                  float *h_out, float *y_out, int64_t rows, int64_t n,
                  hipStream_t stream) {
    return tail_impl(a, r, gamma_post, eps_post, gamma_pre, eps_pre, h_out,
                     y_out, rows, n, SNR_F32, stream);
}

int sandwich_tail_noalloc(const float *a, const float *r,
                          const float *gamma_post, float eps_post,
                          const float *gamma_pre, float eps_pre, float *h_out,
                          float *y_out, int64_t rows, int64_t n,
                          hipStream_t stream) {
    return tail_impl(a, r, gamma_post, eps_post, gamma_pre, eps_pre, h_out,
                     y_out, rows, n, SNR_F32, stream, true);
}

int sandwich_tail_typed(const void *a, const void *r, const void *gamma_post,
                        float eps_post, const void *gamma_pre, float eps_pre,
                        void *h_out, void *y_out, int64_t rows, int64_t n,
                        int dtype, hipStream_t stream) {
    return tail_impl(a, r, gamma_post, eps_post, gamma_pre, eps_pre, h_out,
                     y_out, rows, n, dtype, stream);
}

int sandwich_tail_inplace(const void *a, void *residual,
                          const void *gamma_post, float eps_post,
                          const void *gamma_pre, float eps_pre, void *y_out,
                          int64_t rows, int64_t n, int dtype,
                          hipStream_t stream) {
    return tail_impl(a, residual, gamma_post, eps_post, gamma_pre, eps_pre,
                     residual, y_out, rows, n, dtype, stream);
}

int norm_then_add(const void *a, const void *r, const void *gamma, float eps,
                  const float *out_scale, void *out, int64_t rows, int64_t n,
                  int dtype, hipStream_t stream) {
    int64_t es = 0;
    const int st = storage_of(dtype, &es);
    if (st < 0) return SNR_ERR_DTYPE;
    int rc = check_common(rows, n, es, {eps}, {a, r, gamma, out});
    if (rc != SNR_OK) return rc < 0 ? SNR_OK : rc;
    if (out_scale && !aligned(out_scale, 4)) return SNR_ERR_ALIGN;
    const int64_t tb = rows * n * es, gb = n * es;
    // out may coincide exactly with r (the residual updated in place).
    if (overlaps(out, tb, a, tb) || overlaps(out, tb, gamma, gb) ||
        overlaps(out, tb, out_scale, 4))
        return SNR_ERR_ALIAS;
    if (out != r && overlaps(out, tb, r, tb)) return SNR_ERR_ALIAS;

    RowArgs args{};
    args.x0 = a;
    args.x1 = r;
    args.g0 = gamma;
    args.out0 = out;
    args.scale = out_scale;
    args.eps0 = eps;
    args.rows = rows;
    args.n = (int32_t)n;
    return launch(OP_NORM_ADD, st, es, args, stream);
}

int add_then_norm(const void *a, const void *b, const void *gamma, float eps,
                  void *sum_out, void *y_out, int64_t rows, int64_t n,
                  int dtype, hipStream_t stream) {
    int64_t es = 0;
    const int st = storage_of(dtype, &es);
    if (st < 0) return SNR_ERR_DTYPE;
    int rc = check_common(rows, n, es, {eps}, {a, b, gamma, sum_out, y_out});
    if (rc != SNR_OK) return rc < 0 ? SNR_OK : rc;
    const int64_t tb = rows * n * es, gb = n * es;
    if (overlaps(y_out, tb, a, tb) || overlaps(y_out, tb, b, tb) ||
        overlaps(y_out, tb, sum_out, tb) || overlaps(y_out, tb, gamma, gb))
        return SNR_ERR_ALIAS;
    // sum_out may coincide exactly with a or with b.
    if (overlaps(sum_out, tb, gamma, gb)) return SNR_ERR_ALIAS;
    if (sum_out != a && overlaps(sum_out, tb, a, tb)) return SNR_ERR_ALIAS;
    if (sum_out != b && overlaps(sum_out, tb, b, tb)) return SNR_ERR_ALIAS;

    RowArgs args{};
    args.x0 = a;
    args.x1 = b;
    args.g0 = gamma;
    args.out0 = sum_out;
    args.out1 = y_out;
    args.eps0 = eps;
    args.rows = rows;
    args.n = (int32_t)n;
    return launch(OP_ADD_NORM, st, es, args, stream);
}

int rmsnorm_q8_1(const void *x, const void *gamma, float eps, int64_t rows,
                 int64_t n, int dtype, void *out, hipStream_t stream) {
    int64_t es = 0;
    const int st = storage_of(dtype, &es);
    if (st < 0) return SNR_ERR_DTYPE;
    if (n % 32 != 0) return SNR_ERR_SHAPE;
    int rc = check_common(rows, n, es, {eps}, {x, gamma, out});
    if (rc != SNR_OK) return rc < 0 ? SNR_OK : rc;
    if (reinterpret_cast<uintptr_t>(out) % 4 != 0) return SNR_ERR_ALIGN;
    const int64_t ob = rows * (n / 32) * 36, tb = rows * n * es, gb = n * es;
    if (overlaps(out, ob, x, tb) || overlaps(out, ob, gamma, gb))
        return SNR_ERR_ALIAS;

    RowArgs a{};
    a.x0 = x;
    a.g0 = gamma;
    a.out0 = out;
    a.eps0 = eps;
    a.rows = rows;
    a.n = (int32_t)n;
    return launch(OP_NORM_Q8, st, es, a, stream);
}

int rmsnorm_fwd_multi(const snr_segment *segs, int count, int64_t n,
                      int dtype, hipStream_t stream) {
    int64_t es = 0;
    const int st = storage_of(dtype, &es);
    if (st < 0) return SNR_ERR_DTYPE;
    if (!segs) return SNR_ERR_NULL;
    if (count < 1 || count > kMaxSegments) return SNR_ERR_SHAPE;
    int64_t total = 0;
    for (int s = 0; s < count; ++s) {
        const snr_segment &g = segs[s];
        int rc = check_common(g.rows, n, es, {g.eps}, {g.x, g.gamma, g.y});
        if (rc > 0) return rc;
        if (g.rows > INT64_MAX - total) return SNR_ERR_SHAPE;
        total += g.rows;
    }
    if (total == 0) return SNR_OK;
    const int64_t gb = n * es;
    for (int s = 0; s < count; ++s) {
        const snr_segment &a = segs[s];
        if (a.rows == 0) continue;
        const int64_t ta = a.rows * n * es;
        if (a.y != a.x && overlaps(a.y, ta, a.x, ta)) return SNR_ERR_ALIAS;
        for (int t = 0; t < count; ++t) {
            const snr_segment &b = segs[t];
            if (b.rows == 0) continue;
            const int64_t tb = b.rows * n * es;
            if (overlaps(a.y, ta, b.gamma, gb)) return SNR_ERR_ALIAS;
            if (t != s && (overlaps(a.y, ta, b.x, tb) ||
                           overlaps(a.y, ta, b.y, tb)))
                return SNR_ERR_ALIAS;
        }
    }

    int dev = 0;
    DeviceInfo info;
    int rc = current_device(stream, &dev, &info);
    if (rc != SNR_OK) return rc;
    const int w = (int)(16 / es);
    Choice c;
    rc = choose(OP_PLAIN, st, w, n / w, (int)(n % w), 0, &c);
    if (rc != SNR_OK) return rc;
    if (c.k->kind != KIND_ROWTILE || !c.k->multi) {
        // rows too wide for one register tile (or a forced shape without a
        // several-segment kernel): one ordinary launch per segment
        for (int s = 0; s < count; ++s) {
            if (segs[s].rows == 0) continue;
            rc = rmsnorm_fwd(segs[s].x, segs[s].gamma, segs[s].eps,
                             segs[s].rows, n, dtype, segs[s].y, stream);
            if (rc != SNR_OK) return rc;
        }
        return SNR_OK;
    }
    MultiArgs m{};
    m.count = count;
    m.n = (int32_t)n;
    m.nv = (int32_t)(n / w);
    m.rem = (int32_t)(n % w);
    m.row_start[0] = 0;
    for (int s = 0; s < count; ++s) {
        m.x[s] = segs[s].x;
        m.g[s] = segs[s].gamma;
        m.y[s] = segs[s].y;
        m.eps[s] = segs[s].eps;
        m.row_start[s + 1] = m.row_start[s] + segs[s].rows;
    }
    const KernelEntry *k = c.k;
    const int rpb = k->block / k->g;
    const int64_t step = (int64_t)(UINT32_MAX / (uint32_t)k->block) * rpb;
    for (int64_t r0 = 0; r0 < total; r0 += step) {
        const int64_t nr = total - r0 < step ? total - r0 : step;
        hipError_t e = k->multi(m, r0, nr, stream);
        if (e != hipSuccess) return hip_fail(e);
    }
    std::snprintf(t_last_shape, sizeof t_last_shape, "multi:%d:%d:%d:%d",
                  k->g, k->vpt, w, count);
    t_last_hip_error = 0;
    return SNR_OK;
}

const char *snr_strerror(int code) {
    switch (code) {
    case SNR_OK: return "success";
    case SNR_ERR_NULL: return "a required pointer is NULL";
    case SNR_ERR_SHAPE:
        return "invalid shape (n < 1, n > 2^31-1, rows < 0, size overflow, "
               "or a forced dispatch shape that cannot hold the row)";
    case SNR_ERR_DTYPE: return "unsupported dtype (SNR_F32, SNR_BF16 or SNR_F16)";
    case SNR_ERR_EPS: return "epsilon must be finite and > 0";
    case SNR_ERR_ALIAS: return "output buffers overlap inputs or each other";
    case SNR_ERR_ALIGN: return "pointer not aligned to its element size";
    case SNR_ERR_WORKSPACE:
        return "workspace unavailable (allocation failed or every workspace "
               "held by a captured graph), or a forced split shape whose "
               "chunks cannot all be co-resident";
    case SNR_ERR_HIP: return "HIP runtime call failed";
    case SNR_ERR_DEVICE:
        return "current device is not a gfx950 GPU, or the stream belongs to "
               "another device";
    case SNR_ERR_CAPTURE:
        return "rows wider than 65536 elements under graph capture need a "
               "workspace: make one such call on the stream before capturing";
    default: return "unknown error code";
    }
}

int snr_last_hip_error(void) { return t_last_hip_error; }

int snr_force_shape(int kind, int g, int vpt) {
    if (kind != SNR_SHAPE_AUTO && kind != SNR_SHAPE_ROWTILE &&
        kind != SNR_SHAPE_SPLIT && kind != SNR_SHAPE_MULTIPASS &&
        kind != SNR_SHAPE_PERSIST)
        return SNR_ERR_SHAPE;
    t_force_kind = kind;
    t_force_g = g;
    t_force_vpt = vpt;
    return SNR_OK;
}

int snr_force_grid(int64_t max_groups) {
    if (max_groups < 0) return SNR_ERR_SHAPE;
    t_force_grid = max_groups;
    return SNR_OK;
}

int snr_last_shape(char *buf, int len) {
    if (!buf || len <= 0) return SNR_ERR_NULL;
    std::snprintf(buf, (size_t)len, "%s", t_last_shape);
    return SNR_OK;
}

int snr_release_workspaces(void) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e);
    std::lock_guard<std::mutex> lk(g_ws_mu);
    auto it = g_ws.find(dev);
    if (it == g_ws.end()) return SNR_OK;
    for (Workspace &w : it->second)
        if (w.base && !w.pinned && capturing(w.stream)) return SNR_ERR_CAPTURE;
    for (Workspace &w : it->second) {
        if (!w.base || w.pinned) continue;
        // the last use recorded on its stream; no later use is enqueued
        // while the lock is held
        e = hipEventSynchronize(w.last_use);
        if (e != hipSuccess) return hip_fail(e);
        (void)hipEventDestroy(w.last_use);
        e = hipFree(w.base);
        if (g_split_last[dev] == &w) g_split_last[dev] = nullptr;
        w = Workspace{};   // an empty slot, taken again by the next need
        if (e != hipSuccess) return hip_fail(e);
    }
    return SNR_OK;
}

int snr_split_timeouts(hipStream_t stream, int64_t *count) {
    if (!count) return SNR_ERR_NULL;
    *count = 0;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e);
    std::lock_guard<std::mutex> lk(g_ws_mu);
    auto it = g_ws.find(dev);
    if (it == g_ws.end()) return SNR_OK;
    for (Workspace &w : it->second) {
        if (!w.base || w.stream != stream) continue;
        // every eager use of the workspace is recorded in last_use; graph
        // replays on the stream are covered by synchronising it
        e = hipEventSynchronize(w.last_use);
        if (e == hipSuccess) e = hipStreamSynchronize(stream);
        if (e != hipSuccess) return hip_fail(e);
        unsigned int *word = split_state(w.base).hdr + kHdrTimeouts;
        unsigned int host = 0;
        e = hipMemcpy(&host, word, sizeof host, hipMemcpyDeviceToHost);
        if (e != hipSuccess) return hip_fail(e);
        *count = host;
        if (host != 0) {
            // Tags keep later launches from taking anything left behind by
            // a wait that gave up, so only the count is reset.
            static const unsigned int zero = 0;
            e = hipMemcpy(word, &zero, sizeof zero, hipMemcpyHostToDevice);
            if (e != hipSuccess) return hip_fail(e);
        }
        break;
    }
    return SNR_OK;
}

}  // extern "C"
