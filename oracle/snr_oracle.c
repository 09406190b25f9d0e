/*
 * snr_oracle.c - scalar double-precision reference for row-wise RMSNorm and
 * the fused dual-epsilon sandwich tail.
 *
 * TEST INFRASTRUCTURE ONLY. The library's compute path never links, loads or
 * calls this file: only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg do. It includes no header of the HIP library and shares no
 * source, table or helper with it.
 *
 * Every quantity is evaluated in IEEE-754 double precision by plain loops in
 * index order, with no blocking, fusion or reordering, so that each function
 * can be checked against the definitions by eye. Inputs arrive as f32 values
 * (or bf16 bit patterns) and are widened to double exactly; epsilon arrives as
 * the f32 value the GPU library receives and is widened exactly as well.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -shared -fPIC
 * (no FMA contraction, so every product and sum is rounded once, as written).
 *
 * Every function here is pinned by tests/test_oracle_pins.py against values
 * the pages print, closed forms, invariants, library routines and exact
 * rational arithmetic; tests/test_oracle_mutants.py shows that plausible
 * mistakes planted in a copy of this file fail those pins.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_EBADARG 1

/* Exact bf16 -> f32 widening: a bf16 value is the top half of an f32. */
static float bf16_bits_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/*
 * One row of RMSNorm, following "RMSNorm and the dual-epsilon sandwich"
 * (Muser book ch. 12), section 12.1 "What it computes":
 *   mean(x^2) = (1/n) * sum_j x_j^2
 *   rms       = sqrt(mean(x^2) + eps)        (eps inside the root)
 *   y_i       = x_i / rms * gamma_i
 * The same three steps are the algorithm listed for Hesper's rmsNormKernel
 * ("Hesper.Layers.RMSNorm", GPU Kernel Implementation: RMS = sqrt(sum/n + eps),
 * then y = x / RMS * scale).
 * Returns rms (the denominator) so callers can inspect it.
 */
static double rms_row(const double *x, const double *gamma, double eps,
                      int64_t n, double *y)
{
    double sum_sq = 0.0;
    for (int64_t j = 0; j < n; ++j)
        sum_sq += x[j] * x[j];
    const double mean_sq = sum_sq / (double)n;
    const double rms = sqrt(mean_sq + eps);
    for (int64_t j = 0; j < n; ++j)
        y[j] = x[j] / rms * gamma[j];
    return rms;
}

/*
 * Plain RMSNorm over `rows` contiguous rows of length n, f32 inputs.
 * y: rows*n doubles. rms_out: optional (NULL) array of `rows` denominators.
 * Scratch for the widened row and gamma is provided by the caller through
 * `work` (2*n doubles) so that this file performs no allocation.
 */
int snr_oracle_rmsnorm_f32(const float *x, const float *gamma, float eps,
                           int64_t rows, int64_t n, double *y,
                           double *rms_out, double *work)
{
    if (n < 1 || rows < 0 || !x || !gamma || !y || !work)
        return ORACLE_EBADARG;
    double *xr = work, *gr = work + n;
    for (int64_t j = 0; j < n; ++j)
        gr[j] = (double)gamma[j];
    for (int64_t i = 0; i < rows; ++i) {
        for (int64_t j = 0; j < n; ++j)
            xr[j] = (double)x[i * n + j];
        const double rms = rms_row(xr, gr, (double)eps, n, y + i * n);
        if (rms_out)
            rms_out[i] = rms;
    }
    return ORACLE_OK;
}

/*
 * Plain RMSNorm with bf16 storage: x and gamma are bf16 bit patterns, decoded
 * exactly to f32 and then to double; the result is the exact-input definition
 * in double (no output rounding, which is the GPU's business).
 */
int snr_oracle_rmsnorm_bf16(const uint16_t *x, const uint16_t *gamma,
                            float eps, int64_t rows, int64_t n, double *y,
                            double *rms_out, double *work)
{
    if (n < 1 || rows < 0 || !x || !gamma || !y || !work)
        return ORACLE_EBADARG;
    double *xr = work, *gr = work + n;
    for (int64_t j = 0; j < n; ++j)
        gr[j] = (double)bf16_bits_to_f32(gamma[j]);
    for (int64_t i = 0; i < rows; ++i) {
        for (int64_t j = 0; j < n; ++j)
            xr[j] = (double)bf16_bits_to_f32(x[i * n + j]);
        const double rms = rms_row(xr, gr, (double)eps, n, y + i * n);
        if (rms_out)
            rms_out[i] = rms;
    }
    return ORACLE_OK;
}

/*
 * The dual-epsilon sandwich tail, one row at a time. It follows the sandwich
 * order of "RMSNorm and the dual-epsilon sandwich", section 12.2 (post-norm on
 * the sub-block output before the residual add, then the next pre-norm on the
 * updated stream), and the fused tail of section 12.4.3, which adds the
 * post-normed sub-block output into the residual stream in place and then
 * pre-norms the updated stream with the second epsilon and gain. With a =
 * the sub-block output and r = the residual stream before the add:
 *   d_a = sqrt(mean(a^2) + eps_post)
 *   p_j = a_j / d_a * gamma_post_j           (post-norm output)
 *   h_j = r_j + p_j                          (residual add; updated stream)
 *   d_h = sqrt(mean(h^2) + eps_pre)
 *   y_j = h_j / d_h * gamma_pre_j            (next block's pre-normed input)
 * Hesper's residualAddRmsNormKernel (write both the sum and its norm) is the
 * second half of the same chain. h is kept in double: it is NOT rounded to f32
 * before the second norm.
 *
 * Outputs (all rows*n or rows doubles): h, y; optional p (post-norm term),
 * d_a, d_h (the two denominators). `work` holds 4*n doubles.
 */
int snr_oracle_sandwich_tail(const float *a, const float *r,
                             const float *gamma_post, float eps_post,
                             const float *gamma_pre, float eps_pre,
                             int64_t rows, int64_t n, double *h, double *y,
                             double *p_out, double *d_a_out, double *d_h_out,
                             double *work)
{
    if (n < 1 || rows < 0 || !a || !r || !gamma_post || !gamma_pre || !h ||
        !y || !work)
        return ORACLE_EBADARG;
    double *ar = work, *p = work + n, *gp = work + 2 * n, *gq = work + 3 * n;
    for (int64_t j = 0; j < n; ++j) {
        gp[j] = (double)gamma_post[j];
        gq[j] = (double)gamma_pre[j];
    }
    for (int64_t i = 0; i < rows; ++i) {
        for (int64_t j = 0; j < n; ++j)
            ar[j] = (double)a[i * n + j];
        /* post-norm of the sub-block output, epsilon eps_post */
        const double d_a = rms_row(ar, gp, (double)eps_post, n, p);
        /* residual add */
        double *hi = h + i * n;
        for (int64_t j = 0; j < n; ++j)
            hi[j] = (double)r[i * n + j] + p[j];
        /* next pre-norm of the updated stream, epsilon eps_pre */
        const double d_h = rms_row(hi, gq, (double)eps_pre, n, y + i * n);
        if (p_out)
            memcpy(p_out + i * n, p, (size_t)n * sizeof(double));
        if (d_a_out)
            d_a_out[i] = d_a;
        if (d_h_out)
            d_h_out[i] = d_h;
    }
    return ORACLE_OK;
}

/*
 * The first half of the tail on its own: post-norm of a sub-block's output
 * added to the residual, optionally times a broadcast scalar. Hesper's
 * "RMSNorm Layer" page (rmsNormThenAddKernel, the Gemma-4 post-norm shape,
 * and rmsNormThenAddThenBroadcastScaleKernel): normalise the block output
 * first, then add the residual, then multiply by out_scale:
 *   d   = sqrt(mean(a^2) + eps)
 *   out = (a / d * gamma + r) * scale        (scale = 1 when absent)
 * Inputs f32 (callers decode other storage exactly); out in double.
 * work: 2*n doubles.
 */
int snr_oracle_norm_then_add(const float *a, const float *r,
                             const float *gamma, float eps, double scale,
                             int64_t rows, int64_t n, double *out,
                             double *d_out, double *work)
{
    if (n < 1 || rows < 0 || !a || !r || !gamma || !out || !work)
        return ORACLE_EBADARG;
    double *ar = work, *gr = work + n;
    for (int64_t j = 0; j < n; ++j)
        gr[j] = (double)gamma[j];
    for (int64_t i = 0; i < rows; ++i) {
        for (int64_t j = 0; j < n; ++j)
            ar[j] = (double)a[i * n + j];
        double *oi = out + i * n;
        const double d = rms_row(ar, gr, (double)eps, n, oi);
        for (int64_t j = 0; j < n; ++j)
            oi[j] = (oi[j] + (double)r[i * n + j]) * scale;
        if (d_out)
            d_out[i] = d;
    }
    return ORACLE_OK;
}

/*
 * The second half on its own: residual add, then RMSNorm of the sum, writing
 * both. Hesper's "RMSNorm Layer" page, residualAddRmsNormKernel: each row
 * forms residualOut = a + b, reduces it, and writes residualOut and
 * output = RMSNorm(residualOut) * scale.
 *   s = a + b;  y = s / sqrt(mean(s^2) + eps) * gamma
 * s is kept in double. work: 2*n doubles.
 */
int snr_oracle_add_then_norm(const float *a, const float *b,
                             const float *gamma, float eps, int64_t rows,
                             int64_t n, double *sum, double *y,
                             double *d_out, double *work)
{
    if (n < 1 || rows < 0 || !a || !b || !gamma || !sum || !y || !work)
        return ORACLE_EBADARG;
    double *gr = work;
    for (int64_t j = 0; j < n; ++j)
        gr[j] = (double)gamma[j];
    for (int64_t i = 0; i < rows; ++i) {
        double *si = sum + i * n;
        for (int64_t j = 0; j < n; ++j)
            si[j] = (double)a[i * n + j] + (double)b[i * n + j];
        const double d = rms_row(si, gr, (double)eps, n, y + i * n);
        if (d_out)
            d_out[i] = d;
    }
    return ORACLE_OK;
}

/*
 * RMSNorm followed by Q8_1 quantisation of the normalised row, the fused
 * epilogue on Hesper's "RMSNorm Layer" page ("Fused RMSNorm + Q8_1
 * quantize", fusedRMSNormQ8_1Kernel). Phase 1 is the RMSNorm of section
 * 12.1 of the Muser chapter (x / rms * gamma). Phase 2 takes each block of
 * 32 consecutive normalised values and
 *   amax = max |x_normed|          over the block
 *   d    = amax / 127
 *   q    = round(x_normed / d)     to nearest, ties to even (WGSL round),
 *                                  clamped to [-128, 127]
 * A block whose amax is 0 has d = 0 and q = 0 (the division is undefined;
 * reading: a zero block encodes as zeros).
 * Everything in double; n must be a multiple of 32.
 * Outputs: y (rows*n normalised values), d (rows*n/32 block scales),
 * t (rows*n values x_normed / d, 0 where d = 0), q (rows*n codes).
 * work: 2*n doubles.
 */
int snr_oracle_rmsnorm_q8_1(const float *x, const float *gamma, float eps,
                            int64_t rows, int64_t n, double *y, double *d,
                            double *t, int8_t *q, double *work)
{
    if (n < 32 || n % 32 != 0 || rows < 0 || !x || !gamma || !y || !d ||
        !t || !q || !work)
        return ORACLE_EBADARG;
    double *xr = work, *gr = work + n;
    for (int64_t j = 0; j < n; ++j)
        gr[j] = (double)gamma[j];
    const int64_t nb = n / 32;
    for (int64_t i = 0; i < rows; ++i) {
        for (int64_t j = 0; j < n; ++j)
            xr[j] = (double)x[i * n + j];
        double *yi = y + i * n;
        rms_row(xr, gr, (double)eps, n, yi);
        for (int64_t b = 0; b < nb; ++b) {
            double amax = 0.0;
            for (int64_t l = 0; l < 32; ++l)
                if (fabs(yi[b * 32 + l]) > amax)
                    amax = fabs(yi[b * 32 + l]);
            const double db = amax / 127.0;
            d[i * nb + b] = db;
            for (int64_t l = 0; l < 32; ++l) {
                const int64_t j = i * n + b * 32 + l;
                if (db == 0.0) {
                    t[j] = 0.0;
                    q[j] = 0;
                    continue;
                }
                t[j] = yi[b * 32 + l] / db;
                double r = nearbyint(t[j]);   /* ties to even (default mode) */
                if (r > 127.0)
                    r = 127.0;
                if (r < -128.0)
                    r = -128.0;
                q[j] = (int8_t)r;
            }
        }
    }
    return ORACLE_OK;
}
