// snr_split.hip - split-row kernels for RMSNorm, the dual-epsilon tail and
// its two halves (gfx950): rows too wide for one workgroup's registers are
// cut into chunks of 4096 elements, one workgroup per chunk, and the chunks
// of a row combine their sums of squares through device memory.
//
// What is computed is the row operation of snr_kernels.hip ("RMSNorm and
// the dual-epsilon sandwich", Muser book ch. 12, sections 12.1, 12.2 and
// 12.4.3; Hesper's "RMSNorm Layer" page for the two halves). The mechanism
// for rows too wide for one workgroup is Hesper's "GPU Kernel
// Implementation" (several workgroups per row for large dimensions) and its
// two-pass kernel, re-designed: each chunk stays in registers through the
// cross-workgroup combine, so a row is read from HBM once.
//
// Grid: groups x chunks workgroups, every one resident at once (the grid is
// at most the kernel's resident-workgroup count); workgroup (g, c) holds
// chunk c of rows g, g + groups, g + 2 groups, ... of the launch. It is
// persistent and software-pipelined over those rows. At step t it
//   A. reduces its chunk of row t and publishes the partial sum,
//   issues the loads of row t + 1 (and the second input stream as that
//      stream's schedule needs it), then
//   B. gathers the total of a row published two steps earlier and writes
//      that row's outputs (the tail: forms h of row t - 1 and publishes its
//      partial sum, then
//   C. gathers that second total for row t - 2 and writes its y).
// A row's partial is published one or two steps before any workgroup waits
// for its total, so the other chunks' partials have arrived when it is
// gathered, and the handoff's latency (several microseconds through device
// memory under full HBM load) is spent on other rows. A row's chunk stays in
// a ring of four register buffers from its load to its last use. The
// chunk's gains are loaded once.
//
// The cross-workgroup handoff:
// * Slots. Each (row of the launch, reduction, chunk) has its own 64-bit
//   slot in the workspace, written once per launch: the high half holds the
//   launch's tag, the low half the chunk's f32 partial. Writer and readers
//   exchange only that word (one relaxed agent-scope atomic store, read by
//   relaxed agent-scope atomic loads), and a 64-bit atomic is read whole, so
//   a reader that sees the tag sees the partial stored with it; nothing else
//   is communicated through the handoff (each workgroup normalises its own
//   chunk from its own registers), so no fence is needed. No slot is
//   written twice within a launch, so no reader can see a later value than
//   the one it waits for.
// * Tags. The host gives every eager launch on a workspace a tag no earlier
//   launch on it used since its slots were last cleared (a counter per
//   workspace, 1 .. 2^31 - 1; before it wraps, the slots are cleared on the
//   stream). Launches recorded into a HIP graph carry a tag of their own
//   (2^31), which their replays repeat, and each is preceded in the graph by
//   a kernel that clears the slots it uses. So slot words left by an
//   earlier launch, including a wait that gave up, never carry the current
//   tag, and a later launch never takes them for its own.
// * Row totals are the chunks' partials added in a fixed order (lane j
//   takes chunks j, j + 256, ... in order, then a fixed tree), the same in
//   every workgroup and every launch: results are deterministic.
// * Waits are bounded (spin_limit polls; 0 makes every wait give up at once,
//   a test hook). A wait that gives up is counted in the header (the
//   watchdog count), and its row's total is NaN, so every output of that
//   row is NaN rather than a plausible wrong value; the kernel still
//   finishes.
#include <type_traits>

#include "snr_device.h"

namespace snr {
namespace {

constexpr int SB = kSplitBlock;         // threads per workgroup
constexpr int CE = kSplitChunkElems;    // elements per chunk
constexpr int RING = 4;                 // register buffers per row stream
static_assert(SNW == SB / 64, "block_total's wavefront count");

template <int ST>
constexpr int split_vpt() { return CE / (SB * Codec<ST>::W); }
// reductions per row
template <int OP>
constexpr int split_phases() { return OP == OP_TAIL ? 2 : 1; }

template <int I>
using IC = std::integral_constant<int, I>;

// One chunk of one input stream as stored: VPT 128-bit vectors per lane
// and, in the last chunk, one remainder element for lanes tid < n % W.
template <int VPT>
struct Chunk {
    u32x4 v[VPT];
    unsigned int e;
};
// The same in f32 values.
template <int VPT, int W>
struct FChunk {
    float v[VPT][W];
    float e;
};

// Remainder element codecs (raw bits as stored -> f32).
template <int ST>
__device__ __forceinline__ float dec1(unsigned int raw) {
    if constexpr (ST == ST_F32) return __uint_as_float(raw);
    else if constexpr (ST == ST_BF16) return BF16Bits::one((unsigned short)raw);
    else return F16Bits::one((unsigned short)raw);
}

template <int OP, int ST>
__global__ void __launch_bounds__(SB)
split_kernel(RowArgs p, SplitState st, int64_t row0, int64_t nrows,
             int chunks, int groups) {
    using C = Codec<ST>;
    using T = typename C::T;
    constexpr int W = C::W;
    constexpr int VPT = split_vpt<ST>();
    constexpr int NPH = split_phases<OP>();
    constexpr bool F32 = ST == ST_F32;
    // second input stream ring: r (tail, norm_then_add) is loaded one step
    // before its use; b (add_then_norm) with a, and kept to the output step
    // in 16-bit storage (the f32 sum is formed again there)
    constexpr int NY = OP == OP_PLAIN ? 1 : (OP == OP_ADD_NORM && !F32) ? 4 : 2;
    __shared__ float red[8][SNW];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int chunk = (int)(blockIdx.x % (unsigned)chunks);
    const int group = (int)(blockIdx.x / (unsigned)chunks);
    const int n = p.n;
    const unsigned int tag = st.tag;

    // This chunk: vectors v0 .. v0 + SB*VPT - 1 of the row (lane tid holds
    // v0 + k*SB + tid), and for the last chunk the n % W elements after the
    // row's last whole vector. Offsets are relative to the chunk's first
    // element; a slot past the chunk's end gets an offset the buffer
    // descriptor's range check drops (loads read zeros, stores are dropped).
    const int64_t v0 = (int64_t)chunk * SB * VPT;
    const bool last = chunk == chunks - 1;
    const int64_t celems = last ? (int64_t)n - v0 * W : (int64_t)SB * VPT * W;
    const int cbytes = (int)(celems * (int64_t)sizeof(T));
    unsigned int off[VPT];
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        const int64_t i = (int64_t)k * SB + tid;
        off[k] = v0 + i < p.nv ? 16u * (unsigned int)i : kOutOfRange;
    }
    const unsigned int eoff =
        last && tid < p.rem
            ? (unsigned int)(((int64_t)p.nv - v0) * W + tid) * sizeof(T)
            : kOutOfRange;

    // This workgroup's rows: launch row group + t * groups for t < trips
    // (group < groups <= nrows, so trips >= 1).
    const int64_t trips = (nrows - group + groups - 1) / groups;
    auto live = [&](int64_t t) { return t >= 0 && t < trips; };
    auto buf = [&](const void *base, int64_t t) {
        const bool ok = live(t);
        const int64_t rl = group + (ok ? t : 0) * (int64_t)groups;
        const T *q = static_cast<const T *>(base) + (row0 + rl) * (int64_t)n +
                     v0 * W;
        return buffer_of(q, ok ? cbytes : 0);
    };
    // row streams are loaded non-temporally (each byte is used once), the
    // gains with the default policy
    auto load = [&](Chunk<VPT> &c, const __amdgpu_buffer_rsrc_t r, auto pol) {
        constexpr int P = decltype(pol)::value;
#pragma unroll
        for (int k = 0; k < VPT; ++k)
            c.v[k] = __builtin_amdgcn_raw_buffer_load_b128(r, off[k], 0, P);
        if constexpr (F32)
            c.e = __builtin_amdgcn_raw_buffer_load_b32(r, eoff, 0, P);
        else
            c.e = __builtin_amdgcn_raw_buffer_load_b16(r, eoff, 0, P);
    };
    const IC<kNonTemporal> NT;
    const IC<0> CACHED;
    auto dec = [&](const Chunk<VPT> &c, FChunk<VPT, W> &f) {
#pragma unroll
        for (int k = 0; k < VPT; ++k)
            C::decode(__builtin_bit_cast(typename C::vec, c.v[k]), f.v[k]);
        f.e = dec1<ST>(c.e);
    };
    auto store = [&](const __amdgpu_buffer_rsrc_t r, const FChunk<VPT, W> &f) {
#pragma unroll
        for (int k = 0; k < VPT; ++k)
            __builtin_amdgcn_raw_buffer_store_b128(
                __builtin_bit_cast(u32x4, C::encode(f.v[k])), r, off[k], 0,
                kNonTemporal);
        if constexpr (F32)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(f.e), r,
                                                  eoff, 0, kNonTemporal);
        else if constexpr (ST == ST_BF16)
            __builtin_amdgcn_raw_buffer_store_b16(BF16Bits::enc(f.e), r, eoff,
                                                  0, kNonTemporal);
        else
            __builtin_amdgcn_raw_buffer_store_b16(F16Bits::enc(f.e), r, eoff,
                                                  0, kNonTemporal);
    };
    auto sumsq_chunk = [&](const FChunk<VPT, W> &f) {
        float s = 0.0f;
#pragma unroll
        for (int k = 0; k < VPT; ++k) s += sumsq<W>(f.v[k]);
        return fmaf(f.e, f.e, s);
    };
    // f32 values kept in a raw buffer (f32 storage only: same bits)
    auto keep = [&](Chunk<VPT> &c, const FChunk<VPT, W> &f) {
#pragma unroll
        for (int k = 0; k < VPT; ++k)
#pragma unroll
            for (int e = 0; e < W; ++e) c.v[k][e] = __float_as_uint(f.v[k][e]);
        c.e = __float_as_uint(f.e);
    };

    // The gains of this chunk, as stored, for every row.
    Chunk<VPT> g0, g1;
    load(g0, buffer_of(static_cast<const T *>(p.g0) + v0 * W, cbytes), CACHED);
    if constexpr (OP == OP_TAIL)
        load(g1, buffer_of(static_cast<const T *>(p.g1) + v0 * W, cbytes),
             CACHED);
    const float scale = (OP == OP_NORM_ADD && p.scale) ? *p.scale : 1.0f;

    // Workgroup sum of a per-lane value (every lane gets the same bits).
    // The LDS slot cycles through eight, so two uses of one slot are eight
    // reductions apart, each with its barrier, and no barrier is needed
    // after the reads.
    int rc = 0;
    auto block_sum = [&](float s) {
        float *slot = red[rc++ & 7];
        const float w = group_sum<64>(s);
        if (lane == 0) slot[tid >> 6] = w;
        __syncthreads();
        float t = slot[0];
#pragma unroll
        for (int j = 1; j < SNW; ++j) t += slot[j];
        return t;
    };
    auto slots_of = [&](int64_t t, int ph) {
        return st.slots + ((group + t * (int64_t)groups) * NPH + ph) *
                              (int64_t)chunks;
    };
    auto publish = [&](int64_t t, int ph, float partial) {
        if (tid == 0)
            __hip_atomic_store(
                slots_of(t, ph) + chunk,
                ((unsigned long long)tag << 32) | __float_as_uint(partial),
                __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    // The total of reduction `ph` of row t: lane j waits for chunks j,
    // j + SB, ... and adds them in that order, then the workgroup sum.
    auto gather = [&](int64_t t, int ph) {
        const unsigned long long *s = slots_of(t, ph);
        float mine = 0.0f;
        for (int j = tid; j < chunks; j += SB) {
            unsigned long long w = 0;
            float v;
            for (uint32_t polls = 0; polls < st.spin_limit; ++polls) {
                w = __hip_atomic_load(s + j, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
                if ((unsigned int)(w >> 32) == tag) break;
                __builtin_amdgcn_s_sleep(1);
            }
            if ((unsigned int)(w >> 32) == tag) {
                v = __uint_as_float((unsigned int)w);
            } else {
                __hip_atomic_fetch_add(st.hdr + kHdrTimeouts, 1u,
                                       __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                v = __builtin_nanf("");
            }
            mine = j == tid ? v : mine + v;
        }
        return block_sum(mine);
    };

    Chunk<VPT> X[RING];          // first stream (x / a), and h or s in f32
    Chunk<VPT> Y[NY];            // second stream (r / b)
    FChunk<VPT, W> H[2];         // h in f32 (16-bit tail)
    (void)Y;
    (void)H;

    // Step t of the schedule, with S = t % RING known at compile time.
    auto step = [&](auto sc, int64_t t) {
        constexpr int S = decltype(sc)::value;
        constexpr int S1 = (S + 1) % RING;   // row t + 1
        constexpr int SP1 = (S + RING - 1) % RING;   // row t - 1
        constexpr int SP2 = (S + RING - 2) % RING;   // row t - 2
        // A. row t: first reduction
        if (live(t)) {
            FChunk<VPT, W> v;
            dec(X[S], v);
            if constexpr (OP == OP_ADD_NORM) {
                // s = a + b: stored rounded to storage, kept in f32
                FChunk<VPT, W> b;
                dec(Y[S % NY], b);
#pragma unroll
                for (int k = 0; k < VPT; ++k)
#pragma unroll
                    for (int e = 0; e < W; ++e) v.v[k][e] = v.v[k][e] + b.v[k][e];
                v.e = v.e + b.e;
                store(buf(p.out0, t), v);
                if constexpr (F32) keep(X[S], v);
            }
            publish(t, 0, block_sum(sumsq_chunk(v)));
        }
        // loads of later rows
        load(X[S1], buf(p.x0, t + 1), NT);
        if constexpr (OP == OP_ADD_NORM) load(Y[S1 % NY], buf(p.x1, t + 1), NT);
        if constexpr (OP == OP_TAIL) load(Y[S % 2], buf(p.x1, t), NT);
        if constexpr (OP == OP_NORM_ADD) load(Y[SP1 % 2], buf(p.x1, t - 1), NT);

        if constexpr (OP == OP_TAIL) {
            // B. row t - 1: h = r + a * inv_a * gamma_post, stored, reduced
            if (live(t - 1)) {
                const float inv0 = inv_rms(gather(t - 1, 0), n, p.eps0);
                FChunk<VPT, W> a, r, g;
                FChunk<VPT, W> &h = H[SP1 % 2];
                dec(X[SP1], a);
                dec(Y[SP1 % 2], r);
                dec(g0, g);
#pragma unroll
                for (int k = 0; k < VPT; ++k)
#pragma unroll
                    for (int e = 0; e < W; ++e)
                        h.v[k][e] = fmaf(a.v[k][e] * inv0, g.v[k][e], r.v[k][e]);
                h.e = fmaf(a.e * inv0, g.e, r.e);
                store(buf(p.out0, t - 1), h);
                if constexpr (F32) keep(X[SP1], h);
                publish(t - 1, 1, block_sum(sumsq_chunk(h)));
            }
            // C. row t - 2: y = h * inv_h * gamma_pre
            if (live(t - 2)) {
                const float inv1 = inv_rms(gather(t - 2, 1), n, p.eps1);
                FChunk<VPT, W> h, g, y;
                if constexpr (F32) dec(X[SP2], h);
                else h = H[SP2 % 2];
                dec(g1, g);
#pragma unroll
                for (int k = 0; k < VPT; ++k)
#pragma unroll
                    for (int e = 0; e < W; ++e)
                        y.v[k][e] = h.v[k][e] * inv1 * g.v[k][e];
                y.e = h.e * inv1 * g.e;
                store(buf(p.out1, t - 2), y);
            }
        } else {
            // B. row t - 2: its outputs
            if (live(t - 2)) {
                const float inv0 = inv_rms(gather(t - 2, 0), n, p.eps0);
                FChunk<VPT, W> x, g, o;
                dec(X[SP2], x);
                if constexpr (OP == OP_ADD_NORM && !F32) {
                    FChunk<VPT, W> b;
                    dec(Y[SP2 % NY], b);
#pragma unroll
                    for (int k = 0; k < VPT; ++k)
#pragma unroll
                        for (int e = 0; e < W; ++e)
                            x.v[k][e] = x.v[k][e] + b.v[k][e];
                    x.e = x.e + b.e;
                }
                dec(g0, g);
                if constexpr (OP == OP_NORM_ADD) {
                    FChunk<VPT, W> r;
                    dec(Y[SP2 % 2], r);
#pragma unroll
                    for (int k = 0; k < VPT; ++k)
#pragma unroll
                        for (int e = 0; e < W; ++e)
                            o.v[k][e] =
                                fmaf(x.v[k][e] * inv0, g.v[k][e], r.v[k][e]) *
                                scale;
                    o.e = fmaf(x.e * inv0, g.e, r.e) * scale;
                    store(buf(p.out0, t - 2), o);
                } else {
#pragma unroll
                    for (int k = 0; k < VPT; ++k)
#pragma unroll
                        for (int e = 0; e < W; ++e)
                            o.v[k][e] = x.v[k][e] * inv0 * g.v[k][e];
                    o.e = x.e * inv0 * g.e;
                    store(buf(OP == OP_PLAIN ? p.out0 : p.out1, t - 2), o);
                }
            }
        }
    };

    load(X[0], buf(p.x0, 0), NT);
    if constexpr (OP == OP_ADD_NORM) load(Y[0], buf(p.x1, 0), NT);
    // the last row's last step is trips + 1
    for (int64_t t = 0; t < trips + 2; t += RING) {
        step(IC<0>{}, t);
        step(IC<1>{}, t + 1);
        step(IC<2>{}, t + 2);
        step(IC<3>{}, t + 3);
    }

}

// An ordinary launch, or a cooperative one (which the runtime accepts only
// if every workgroup can be resident, and then guarantees it) when
// `cooperative` is set.
template <int OP, int ST>
hipError_t launch_split(const RowArgs &p, const SplitState &st, int64_t row0,
                        int64_t nrows, int chunks, int groups, bool cooperative,
                        hipStream_t stream) {
    const dim3 grid((unsigned int)(groups * chunks));
    if (!cooperative) {
        hipLaunchKernelGGL((split_kernel<OP, ST>), grid, dim3(SB), 0, stream, p,
                           st, row0, nrows, chunks, groups);
        return hipGetLastError();
    }
    RowArgs pa = p;
    SplitState sa = st;
    int c = chunks, g = groups;
    void *args[] = {&pa, &sa, &row0, &nrows, &c, &g};
    return hipLaunchCooperativeKernel(
        reinterpret_cast<const void *>(&split_kernel<OP, ST>), grid, dim3(SB),
        args, 0, stream);
}

template <int OP, int ST>
hipError_t occupancy_split(int *blocks_per_cu) {
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(
        blocks_per_cu, reinterpret_cast<const void *>(&split_kernel<OP, ST>),
        SB, 0);
}

#define SNR_SPLIT(OP, ST)                                                    \
    KernelEntry{OP, ST, Codec<ST>::W, KIND_SPLIT, SB, split_vpt<ST>(), SB,   \
                nullptr, &launch_split<OP, ST>, &occupancy_split<OP, ST>,    \
                nullptr, nullptr}
#define SNR_SPLIT_ALL(OP)                                                    \
    SNR_SPLIT(OP, ST_F32), SNR_SPLIT(OP, ST_BF16), SNR_SPLIT(OP, ST_F16)

const KernelEntry kSplitTable[] = {
    SNR_SPLIT_ALL(OP_PLAIN), SNR_SPLIT_ALL(OP_TAIL),
    SNR_SPLIT_ALL(OP_NORM_ADD), SNR_SPLIT_ALL(OP_ADD_NORM),
};

}  // namespace

const KernelEntry *split_kernel_table(int *count) {
    *count = (int)(sizeof(kSplitTable) / sizeof(kSplitTable[0]));
    return kSplitTable;
}

}  // namespace snr
