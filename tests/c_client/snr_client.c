/*
 * snr_client.c - a plain C program that uses libsnr through include/snr.h
 * and the HIP runtime API alone, with no PyTorch in the process.
 *
 * Test infrastructure: tests/test_gpu_c_client.py writes the inputs, runs
 * this program and compares its outputs with the oracle.
 *
 *   snr_client DIR ROWS N
 *
 * reads DIR/a.f32, DIR/r.f32 ([ROWS, N] f32), DIR/gp.f32, DIR/gq.f32 ([N]
 * f32) and DIR/eps.f32 (eps_post, eps_pre), then on a stream of its own:
 *   - sandwich_tail(a, r, gp, eps_post, gq, eps_pre) -> DIR/h.f32, DIR/y.f32
 *   - rmsnorm_fwd(a, gp, eps_pre) in f32 -> DIR/z.f32
 *   - the in-place tail on a copy of r -> DIR/hi.f32 (the updated residual)
 *     and DIR/yi.f32
 * and checks that invalid arguments come back as their error codes with
 * nothing enqueued. Prints "ok" and exits 0, or names the failing step and
 * exits 1.
 */
#include <hip/hip_runtime_api.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "snr.h"

static int fail(const char *what, int code) {
    fprintf(stderr, "snr_client: %s failed: %d (%s)\n", what, code,
            code > 0 && code < 100 ? snr_strerror(code) : "hip");
    return 1;
}

static float *read_file(const char *dir, const char *name, size_t count) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE *f = fopen(path, "rb");
    if (!f) return NULL;
    float *buf = (float *)malloc(count * sizeof(float));
    if (buf && fread(buf, sizeof(float), count, f) != count) {
        free(buf);
        buf = NULL;
    }
    fclose(f);
    return buf;
}

static int write_file(const char *dir, const char *name, const float *buf,
                      size_t count) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE *f = fopen(path, "wb");
    if (!f) return 0;
    const size_t wrote = fwrite(buf, sizeof(float), count, f);
    fclose(f);
    return wrote == count;
}

/* a device copy of a host array */
static float *upload(const float *host, size_t count) {
    void *d = NULL;
    if (hipMalloc(&d, count * sizeof(float)) != hipSuccess) return NULL;
    if (hipMemcpy(d, host, count * sizeof(float), hipMemcpyHostToDevice) !=
        hipSuccess)
        return NULL;
    return (float *)d;
}

static int download(const char *dir, const char *name, const float *dev,
                    size_t count) {
    float *host = (float *)malloc(count * sizeof(float));
    int ok = host &&
             hipMemcpy(host, dev, count * sizeof(float),
                       hipMemcpyDeviceToHost) == hipSuccess &&
             write_file(dir, name, host, count);
    free(host);
    return ok;
}

int main(int argc, char **argv) {
    if (argc != 4) {
        fprintf(stderr, "usage: snr_client DIR ROWS N\n");
        return 2;
    }
    const char *dir = argv[1];
    const int64_t rows = strtoll(argv[2], NULL, 10);
    const int64_t n = strtoll(argv[3], NULL, 10);
    if (rows < 1 || n < 1) return fail("arguments", 0);
    const size_t tn = (size_t)rows * (size_t)n;

    float *a = read_file(dir, "a.f32", tn), *r = read_file(dir, "r.f32", tn);
    float *gp = read_file(dir, "gp.f32", (size_t)n);
    float *gq = read_file(dir, "gq.f32", (size_t)n);
    float *eps = read_file(dir, "eps.f32", 2);
    if (!a || !r || !gp || !gq || !eps) return fail("reading inputs", 0);

    hipStream_t stream = NULL;
    if (hipStreamCreate(&stream) != hipSuccess)
        return fail("hipStreamCreate", 0);
    float *da = upload(a, tn), *dr = upload(r, tn), *dri = upload(r, tn);
    float *dgp = upload(gp, (size_t)n), *dgq = upload(gq, (size_t)n);
    float *dh = NULL, *dy = NULL, *dz = NULL, *dyi = NULL;
    if (!da || !dr || !dri || !dgp || !dgq ||
        hipMalloc((void **)&dh, tn * sizeof(float)) != hipSuccess ||
        hipMalloc((void **)&dy, tn * sizeof(float)) != hipSuccess ||
        hipMalloc((void **)&dz, tn * sizeof(float)) != hipSuccess ||
        hipMalloc((void **)&dyi, tn * sizeof(float)) != hipSuccess)
        return fail("device allocation", 0);

    /* invalid arguments: each is refused before anything is enqueued */
    int rc = sandwich_tail(NULL, dr, dgp, eps[0], dgq, eps[1], dh, dy, rows,
                           n, stream);
    if (rc != SNR_ERR_NULL) return fail("NULL input check", rc);
    rc = sandwich_tail(da, dr, dgp, 0.0f, dgq, eps[1], dh, dy, rows, n,
                       stream);
    if (rc != SNR_ERR_EPS) return fail("eps check", rc);
    rc = sandwich_tail(da, dr, dgp, eps[0], dgq, eps[1], dh, da, rows, n,
                       stream);
    if (rc != SNR_ERR_ALIAS) return fail("alias check", rc);
    rc = rmsnorm_fwd(da, dgp, eps[1], rows, n, 7, dz, stream);
    if (rc != SNR_ERR_DTYPE) return fail("dtype check", rc);
    rc = rmsnorm_fwd(da, dgp, eps[1], rows, 0, SNR_F32, dz, stream);
    if (rc != SNR_ERR_SHAPE) return fail("shape check", rc);
    rc = rmsnorm_fwd(da, dgp, eps[1], 0, n, SNR_F32, dz, stream);
    if (rc != SNR_OK) return fail("rows == 0 no-op", rc);

    rc = sandwich_tail(da, dr, dgp, eps[0], dgq, eps[1], dh, dy, rows, n,
                       stream);
    if (rc != SNR_OK) return fail("sandwich_tail", rc);
    rc = rmsnorm_fwd(da, dgp, eps[1], rows, n, SNR_F32, dz, stream);
    if (rc != SNR_OK) return fail("rmsnorm_fwd", rc);
    rc = sandwich_tail_inplace(da, dri, dgp, eps[0], dgq, eps[1], dyi, rows,
                               n, SNR_F32, stream);
    if (rc != SNR_OK) return fail("sandwich_tail_inplace", rc);
    if (hipStreamSynchronize(stream) != hipSuccess)
        return fail("hipStreamSynchronize", 0);
    if (snr_last_hip_error() != 0)
        return fail("snr_last_hip_error", snr_last_hip_error());

    if (!download(dir, "h.f32", dh, tn) || !download(dir, "y.f32", dy, tn) ||
        !download(dir, "z.f32", dz, tn) || !download(dir, "hi.f32", dri, tn) ||
        !download(dir, "yi.f32", dyi, tn))
        return fail("writing outputs", 0);

    (void)hipFree(da); (void)hipFree(dr); (void)hipFree(dri);
    (void)hipFree(dgp); (void)hipFree(dgq); (void)hipFree(dh);
    (void)hipFree(dy); (void)hipFree(dz); (void)hipFree(dyi);
    (void)hipStreamDestroy(stream);
    free(a); free(r); free(gp); free(gq); free(eps);
    printf("ok\n");
    return 0;
}
