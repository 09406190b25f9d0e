/*
 * snr.h - C ABI of libsnr: row-wise RMSNorm and the fused dual-epsilon
 * sandwich tail on AMD Instinct MI355X (gfx950), hand-written HIP kernels.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Tensors are dense, contiguous, row-major [rows, n] arrays in device
 *   memory (row i starts at element i*n); gains are dense [n] vectors shared
 *   by all rows. There is no stride argument.
 * - All pointers are device pointers owned by the caller. The library never
 *   frees or retains them. It owns only workspaces of 1 MiB of device
 *   memory each, for the partial sums of the split-row and multi-pass
 *   kernels (rows wider than 65536 elements): at most 8 per device, each
 *   bound to one stream at a time, allocated by the first such call on a
 *   stream that finds none free, kept until snr_release_workspaces or the
 *   end of the process (so at most 8 MiB per device however many streams
 *   are used). When a ninth stream
 *   needs one, it takes the least recently used workspace, and its launches
 *   wait on the GPU for that workspace's last use on the other stream to
 *   finish (the library records an event after each use), so uses of one
 *   workspace never overlap. Every other shape allocates nothing.
 * - Calls are asynchronous: they validate the arguments, enqueue kernels on
 *   `stream` (NULL = the legacy default stream of the current device; any
 *   other stream must belong to the current device) and return. Execution faults surface at the caller's next synchronisation.
 *   Arguments are validated before anything is enqueued: a call that rejects
 *   its arguments has enqueued nothing. (SNR_ERR_HIP from a failed launch
 *   can follow earlier launches of the same call, e.g. of other row
 *   batches.)
 * - HIP graphs: calls on rows that a register tile holds (up to 65536
 *   elements) enqueue only kernels, so they can be recorded into a graph,
 *   the first call of a process included (the host-side device and
 *   occupancy queries it makes enqueue nothing). Wider rows use a
 *   workspace: under capture a call may use only the workspace its stream
 *   already holds (make one call on that stream outside the capture first;
 *   otherwise the call returns SNR_ERR_CAPTURE and enqueues nothing), and
 *   that workspace then stays with the stream for the life of the process.
 *   Replays of such a graph must not overlap one another or wide-row calls
 *   on the capture stream (replay them on that stream, or order them).
 * - Reductions are deterministic: for a given (rows, n, dtype, dispatch
 *   shape) the result is bit-identical from run to run (fixed summation
 *   order, no floating-point atomics).
 * - Every n >= 1 is computed; there is no refusal by row width. rows == 0 is
 *   a successful no-op. n is limited to 2^31 - 1 elements per row.
 * - Return value: SNR_OK (0) or one of the SNR_ERR_* codes below.
 */
#ifndef SNR_H
#define SNR_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define SNR_API __attribute__((visibility("default")))
#else
#define SNR_API
#endif

/* An opaque HIP stream handle (identical to HIP's own hipStream_t). */
typedef struct ihipStream_t *hipStream_t;

typedef enum {
    SNR_F32 = 0,  /* IEEE binary32 storage */
    SNR_BF16 = 1, /* bfloat16 storage */
    SNR_F16 = 2   /* IEEE binary16 storage */
} snr_dtype;
/* Every operation reads its storage type exactly into f32, accumulates and
 * computes in f32, and rounds its outputs to the storage type to nearest
 * even. An intermediate that a later norm of the same call reads (the
 * tail's h, add_then_norm's sum) is stored rounded to the storage type,
 * and the later norm works from its f32 value, so y carries one rounding. */

enum {
    SNR_OK = 0,
    SNR_ERR_NULL = 1,      /* a required pointer is NULL while rows > 0 */
    SNR_ERR_SHAPE = 2,     /* n < 1, n > 2^31 - 1, rows < 0, or rows*n
                              overflows */
    SNR_ERR_DTYPE = 3,     /* dtype is not an snr_dtype value */
    SNR_ERR_EPS = 4,       /* an epsilon is not finite or not > 0 */
    SNR_ERR_ALIAS = 5,     /* buffers overlap other than in an allowed way */
    SNR_ERR_ALIGN = 6,     /* a pointer is not aligned to its element size */
    SNR_ERR_WORKSPACE = 7, /* a workspace could not be allocated, every
                              workspace of the device is held by a captured
                              graph, or a forced split shape cannot keep
                              every chunk of a row co-resident */
    SNR_ERR_HIP = 8,       /* a HIP runtime call failed; see
                              snr_last_hip_error() */
    SNR_ERR_DEVICE = 9,    /* the current device is not a gfx950 GPU, or
                              `stream` belongs to another device */
    SNR_ERR_CAPTURE = 10   /* rows wider than 65536 elements under HIP
                              graph capture on a stream that holds no
                              workspace yet (see "HIP graphs" above) */
};

/*
 * rmsnorm_fwd - row-wise RMSNorm.
 *
 * Defined in "RMSNorm and the dual-epsilon sandwich" (Muser book, chapter
 * 12), section 12.1 "What it computes": for each row i
 *     y[i, j] = x[i, j] / sqrt( (1/n) * sum_k x[i, k]^2 + eps ) * gamma[j]
 * with epsilon inside the root (the same three steps Hesper's RMSNorm layer
 * documents for rmsNormKernel).
 *
 *   x      [rows, n] input, dtype `dtype`, device memory
 *   gamma  [n] per-channel gain, same dtype as x
 *   eps    epsilon added to the mean of squares; finite and > 0.
 *          Sums of squares are f32: a row's n * mean(x^2) must stay below
 *          3.4e38, and mean(x^2) + eps too (else 1/rms = 0). A subnormal
 *          epsilon is computed, but squares below 2^-126 lose precision and
 *          below 2^-150 vanish, so with such an epsilon rows whose mean
 *          square is itself below about 1e-37 are not accurate; any normal
 *          epsilon outweighs what those squares lose.
 *   rows   number of rows (>= 0)
 *   n      row width (>= 1)
 *   dtype  SNR_F32, SNR_BF16 or SNR_F16 (storage of x, gamma and y)
 *   y      [rows, n] output, dtype `dtype`. y == x (exactly the same
 *          pointer) is allowed and computes in place; any other overlap of y
 *          with x or gamma is SNR_ERR_ALIAS.
 *   stream HIP stream to enqueue on (NULL = default stream)
 *
 * Pointers need only element alignment (4 B for f32, 2 B for 16-bit types).
 * Rows are moved with 128-bit accesses whatever their alignment; the n % 4
 * (f32) or n % 8 (16-bit) elements after a row's last whole vector one at a
 * time.
 */
SNR_API int rmsnorm_fwd(const void *x, const void *gamma, float eps, int64_t rows,
                int64_t n, int dtype, void *y, hipStream_t stream);

/*
 * sandwich_tail - the fused dual-epsilon sandwich tail, f32 storage.
 *
 * Defined in "RMSNorm and the dual-epsilon sandwich" (Muser book, chapter
 * 12): section 12.2 gives the layer order (each sub-block's output goes
 * through its post-norm and then into the residual stream, whose pre-norm
 * feeds the next sub-block) and section 12.4.3 the fused tail that does the
 * post-norm, the residual add and the next pre-norm in a single launch, each
 * norm with its own epsilon. Per row:
 *     h = r + gamma_post * a / sqrt(mean(a^2) + eps_post)
 *     y = gamma_pre * h / sqrt(mean(h^2) + eps_pre)
 * The model the book describes uses eps_post = 1e-8 and eps_pre = 1e-5; both
 * are arguments here. y is computed from the f32 value of h that is stored.
 * Hesper's residualAddRmsNormKernel ("Hesper.Layers.RMSNorm") writes both the
 * updated stream and its norm the same way.
 *
 *   a          [rows, n] sub-block output (e.g. the attention or FFN result)
 *   r          [rows, n] residual stream before the add
 *   gamma_post [n] post-norm gain;  eps_post its epsilon (finite, > 0)
 *   gamma_pre  [n] pre-norm gain;   eps_pre its epsilon (finite, > 0)
 *   h_out      [rows, n] updated residual stream. h_out == r (exactly) is
 *              allowed and updates the stream in place.
 *   y_out      [rows, n] normalised input of the next sub-block
 *   rows, n    as for rmsnorm_fwd
 *   stream     HIP stream (NULL = default stream)
 *
 * SNR_ERR_ALIAS: y_out overlapping any other buffer, h_out overlapping a or
 * a gain, or h_out partially overlapping r.
 */
SNR_API int sandwich_tail(const float *a, const float *r, const float *gamma_post,
                  float eps_post, const float *gamma_pre, float eps_pre,
                  float *h_out, float *y_out, int64_t rows, int64_t n,
                  hipStream_t stream);

/*
 * sandwich_tail_noalloc - sandwich_tail for callers that cannot allocate
 * device memory: code recorded into HIP graphs whose capture must not
 * allocate, tight serving loops, harnesses that forbid hipMalloc.
 *
 * Same arguments, results and errors as sandwich_tail (the same kernels, so
 * the outputs are bit-identical). Where sandwich_tail would use an allocated
 * workspace (rows wider than 65536 elements), this uses instead a 1 MiB
 * array in the library's own device memory (a file-scope __device__ array;
 * each GPU the library runs on holds one copy until the process ends). It
 * calls no allocating routine. Rows are processed in batches sized to that
 * array, so every row width the ABI accepts fits; a row that needed more
 * would be refused with SNR_ERR_WORKSPACE.
 *
 * Every call on a GPU shares that GPU's array and no events order them:
 * calls of this entry point that overlap on one GPU race (and so does one
 * that overlaps another wide-row call there). Serialise them, e.g. on one
 * stream. The array's slots carry per-call tags, so what an earlier call
 * left there is never taken for a later call's. The first call on a device
 * looks up the array's device address; the first call there that is not
 * being captured into a graph clears the array with a kernel on `stream`
 * (a captured call clears, inside the graph, the slots its launch uses).
 */
SNR_API int sandwich_tail_noalloc(const float *a, const float *r,
                                  const float *gamma_post, float eps_post,
                                  const float *gamma_pre, float eps_pre,
                                  float *h_out, float *y_out, int64_t rows,
                                  int64_t n, hipStream_t stream);

/*
 * sandwich_tail_typed - the same tail for any snr_dtype storage: a, r, both
 * gains, h_out and y_out all of type `dtype`. With bf16 or f16 storage, h is
 * stored rounded to the storage type, and y is the norm of its f32 value
 * (one rounding in y; normalising the rounded copy would add the rounding
 * of the row's largest element to every output). Rows too wide for the
 * split-row kernel (beyond about 4.2 million elements: 1024 chunks of 4096) go through multi-pass
 * kernels whose last pass re-reads the stored h: there y carries two.
 * Same aliasing rules as sandwich_tail.
 *
 * sandwich_tail_inplace - the tail with the residual stream updated in place
 * (the Muser kernel's form, where `hidden` is read and written, and Hesper's
 * forwardNormThenAddBatchInPlace): residual <- residual + post-norm(a), and
 * y_out <- pre-norm of the updated residual. y_out may not overlap any other
 * buffer; residual may not overlap a or the gains.
 */
SNR_API int sandwich_tail_typed(const void *a, const void *r,
                                const void *gamma_post, float eps_post,
                                const void *gamma_pre, float eps_pre,
                                void *h_out, void *y_out, int64_t rows,
                                int64_t n, int dtype, hipStream_t stream);
SNR_API int sandwich_tail_inplace(const void *a, void *residual,
                                  const void *gamma_post, float eps_post,
                                  const void *gamma_pre, float eps_pre,
                                  void *y_out, int64_t rows, int64_t n,
                                  int dtype, hipStream_t stream);

/*
 * norm_then_add - the first half of the tail on its own: post-norm of a
 * sub-block's output, added to the residual, optionally times a broadcast
 * scalar. Defined on Hesper's "RMSNorm Layer" page (rmsNormThenAddKernel,
 * the Gemma-4 post-norm shape, its batched row-major form
 * rmsNormAddBatchRowsKernel, and rmsNormThenAddThenBroadcastScaleKernel):
 *     out = (a / sqrt(mean(a^2) + eps) * gamma + r) * out_scale[0]
 *   a, r      [rows, n] of `dtype`;  gamma [n] of `dtype`
 *   out_scale device pointer to one f32 value, or NULL for 1
 *   out       [rows, n] of `dtype`; out == r (exactly) updates the residual
 *             in place; any other overlap with a, r, gamma or out_scale is
 *             SNR_ERR_ALIAS.
 */
SNR_API int norm_then_add(const void *a, const void *r, const void *gamma,
                          float eps, const float *out_scale, void *out,
                          int64_t rows, int64_t n, int dtype,
                          hipStream_t stream);

/*
 * add_then_norm - the second half on its own: residual add, then RMSNorm of
 * the sum, writing both. Hesper's "RMSNorm Layer" page,
 * residualAddRmsNormKernel:
 *     sum = a + b;  y = sum / sqrt(mean(sum^2) + eps) * gamma
 *   a, b      [rows, n] of `dtype`;  gamma [n] of `dtype`
 *   sum_out   [rows, n]; may coincide exactly with a or with b
 *   y_out     [rows, n]; may overlap no other buffer
 * With bf16 or f16 storage, the sum is stored rounded and y is the norm
 * of its f32 value.
 */
SNR_API int add_then_norm(const void *a, const void *b, const void *gamma,
                          float eps, void *sum_out, void *y_out, int64_t rows,
                          int64_t n, int dtype, hipStream_t stream);

/*
 * rmsnorm_q8_1 - RMSNorm whose output goes straight into Q8_1 records, for a
 * following 8-bit matmul. Hesper's "RMSNorm Layer" page, "Fused RMSNorm +
 * Q8_1 quantize" (fusedRMSNormQ8_1Kernel): each row is normalised as in
 * rmsnorm_fwd, then every block of 32 consecutive normalised values v[0..31]
 * is encoded as
 *     d    = max_k |v[k]| / 127              (f32, stored as f16)
 *     q[k] = round(v[k] / d), ties to even, clamped to [-128, 127]
 * and a block whose values are all zero encodes as d = 0, q = 0.
 *   x      [rows, n] of `dtype`; n must be a multiple of 32 (else
 *          SNR_ERR_SHAPE);  gamma [n] of `dtype`
 *   out    rows * (n / 32) records of 36 bytes, row-major, block b of row i
 *          at byte (i * n / 32 + b) * 36:
 *            bytes 0-1  d as IEEE binary16 (round to nearest even)
 *            bytes 2-3  s, always 0 (a consumer that reads s gets 0)
 *            bytes 4-35 q[0..31] as int8
 *          4-byte aligned (else SNR_ERR_ALIGN); may overlap neither x nor
 *          gamma (SNR_ERR_ALIAS).
 * The codes are computed with the f32 scale d, before its rounding to f16.
 */
SNR_API int rmsnorm_q8_1(const void *x, const void *gamma, float eps,
                         int64_t rows, int64_t n, int dtype, void *out,
                         hipStream_t stream);

/*
 * rmsnorm_fwd_multi - several independent RMSNorms of one row width in one
 * launch, e.g. the per-head query and key norms of a layer. The Muser book's
 * per-token accounting ("RMSNorm and the dual-epsilon sandwich", section
 * 12.5) counts these per-head norms at head_dim 128 as the second-largest
 * family of norm dispatches (two per layer); one launch here replaces two.
 * Each segment is an ordinary rmsnorm_fwd problem:
 *     y[i, j] = x[i, j] / sqrt(mean_k x[i, k]^2 + eps) * gamma[j]
 *   segments  host array of `count` (1..SNR_MAX_SEGMENTS) descriptors, read
 *             during the call only
 *   n, dtype  shared row width and storage type
 * Within a segment y == x is allowed; a segment's y may not overlap any
 * other segment's x or y, nor any gain. Segments with rows == 0 are skipped.
 * Rows too wide for one register tile (over 65536 f32 elements) fall back to
 * one rmsnorm_fwd launch per segment.
 */
#define SNR_MAX_SEGMENTS 8
typedef struct {
    const void *x;     /* [rows, n] input */
    const void *gamma; /* [n] gain */
    void *y;           /* [rows, n] output */
    int64_t rows;
    float eps;
} snr_segment;
SNR_API int rmsnorm_fwd_multi(const snr_segment *segments, int count,
                              int64_t n, int dtype, hipStream_t stream);

/* Human-readable text for an SNR_* code (static storage, never NULL). */
SNR_API const char *snr_strerror(int code);

/* The hipError_t of the most recent failing HIP call made by this library on
 * the calling thread (0 if none since the last successful call). */
SNR_API int snr_last_hip_error(void);

/*
 * Dispatch-shape introspection and override (diagnostics and tests).
 *
 * Shapes:  SNR_SHAPE_AUTO     choose by n, rows, dtype and alignment
 *          SNR_SHAPE_ROWTILE  g lanes per row (g a power of two, 1..1024),
 *                             each lane holding `vpt` loads of the row in
 *                             registers; g <= 64 packs several rows in one
 *                             wavefront, g > 64 spans g/64 wavefronts joined
 *                             by one LDS step. A launch of at most 16
 *                             workgroups loads the gains together with the
 *                             row (one memory round trip fewer; the same
 *                             results bit for bit)
 *          SNR_SHAPE_SPLIT    the row is cut into chunks of 4096 elements
 *                             (256 lanes x 4 vectors f32, x 2 vectors
 *                             16-bit), one workgroup per chunk, joined by a
 *                             cross-workgroup reduction through device
 *                             memory; every chunk of a row must be
 *                             co-resident (g and vpt are ignored)
 *          SNR_SHAPE_MULTIPASS rows wider than that: per-chunk partial sums,
 *                             a per-row combine and an apply pass through
 *                             device memory (reads the row twice; the tail
 *                             also re-reads h). Chosen automatically only
 *                             when the split shape cannot hold the row.
 *          SNR_SHAPE_PERSIST  the row tile (g >= 128 lanes, one row per
 *                             workgroup) on a persistent grid that loads the
 *                             next row while reducing the current one; same
 *                             arithmetic and results as SNR_SHAPE_ROWTILE
 *                             with the same g and vpt. Only for rows with n
 *                             a multiple of the vector width (4 f32, 8
 *                             16-bit), and not for rmsnorm_q8_1 (whose row
 *                             tiles are persistent already).
 * snr_force_shape applies to subsequent calls on the calling thread until it
 * is called again with SNR_SHAPE_AUTO. A forced shape that cannot hold the
 * row (g * vpt loads < row length) or that has no compiled kernel returns
 * SNR_ERR_SHAPE from the call. snr_last_shape writes "rowtile:g:vpt:width",
 * "persist:g:vpt:width", "split:256:vpt:width:chunks" or
 * "multipass:256:16:width:chunks" (width =
 * elements per 128-bit vector) of
 * the calling thread's most recent successful launch into buf
 * (NUL-terminated).
 */
enum {
    SNR_SHAPE_AUTO = 0,
    SNR_SHAPE_ROWTILE = 1,
    SNR_SHAPE_SPLIT = 2,
    SNR_SHAPE_MULTIPASS = 3,
    SNR_SHAPE_PERSIST = 4
};
SNR_API int snr_force_shape(int kind, int g, int vpt);
/*
 * snr_force_grid - diagnostics: caps the rows in flight of the kernels that
 * walk several rows per workgroup, for subsequent calls on the calling
 * thread: the persistent row tiles (SNR_SHAPE_PERSIST, and rmsnorm_q8_1's
 * persistent tiles) launch at most `max_groups` workgroups, and the
 * split-row kernels at most `max_groups` workgroups per chunk. Each
 * workgroup then walks more rows, which exercises the kernels' pipelined
 * loops on small inputs; results are unchanged. 0 restores the default
 * (as many as the device holds at once); a negative value returns
 * SNR_ERR_SHAPE.
 */
SNR_API int snr_force_grid(int64_t max_groups);
SNR_API int snr_last_shape(char *buf, int len);

/*
 * Split-row kernels and their wait watchdog. Rows wider than any register
 * tile (65536 elements) are cut into chunks of 4096 elements, one
 * workgroup per chunk, whose partial sums meet through the workspace. The
 * grid is at most the number of workgroups the device holds at once, and
 * the library never lets two split-row launches overlap on a device (it
 * orders each one after the previous one, on any stream, with an event);
 * the kernels assume every workgroup of their grid becomes resident. By
 * default they are ordinary launches; with the environment variable
 * SNR_SPLIT_COOPERATIVE set (not "0") they are cooperative launches, which
 * the runtime admits only when the whole grid fits and then keeps resident,
 * at a cost of about 14 us per launch. A workgroup waits for the partial
 * sums of the other chunks of its row with a bounded spin; if the bound is
 * ever exceeded (only if some workgroups of the grid could not become
 * resident for seconds), the kernel stops waiting, counts the event in the
 * workspace, writes NaN to every output of that row, and finishes. Later
 * calls are not affected: each launch tags its partial sums with a number
 * no earlier launch left in the workspace, so nothing an earlier launch
 * left behind is ever taken for a later launch's. This returns the number
 * of such events counted in the workspace (current device, stream) holds,
 * and clears the count. It synchronises the stream and the workspace's last
 * use. 0 means every wait completed normally (or the stream holds no
 * workspace). Overruns of sandwich_tail_noalloc's calls are counted in its
 * static array, which this does not read; their rows' outputs are NaN all
 * the same.
 * The environment variable SNR_SPLIT_SPIN_LIMIT (an integer >= 0, read at
 * each split-row launch) replaces the default bound of 2^22 polls; tests use
 * 0 to make every wait give up at once. SNR_SPLIT_EPOCH (read when a
 * workspace is created) sets its starting tag number; tests use a value
 * near 2^31 - 1 to exercise the wrap of the tag numbers.
 */
SNR_API int snr_split_timeouts(hipStream_t stream, int64_t *count);

/*
 * snr_release_workspaces - frees the current device's workspaces (the 1 MiB
 * blocks of device memory the split-row and multi-pass kernels use for rows
 * wider than 65536 elements), for a caller that wants that memory back or
 * is about to unload the library. It waits on the host for each
 * workspace's last use, then frees it; the next wide-row call on a stream
 * allocates one again. A workspace recorded into a HIP graph is kept (the
 * graph may still be replayed). Returns SNR_ERR_CAPTURE, freeing nothing,
 * if a stream that holds a workspace is being captured; do not call it
 * while any other stream of the device is being captured either (freeing
 * device memory is not allowed during a capture). Overrun counts not yet
 * read with snr_split_timeouts are dropped. The allocation-free entry
 * point's static array is not affected.
 */
SNR_API int snr_release_workspaces(void);

#ifdef __cplusplus
}
#endif

#endif /* SNR_H */
