/*
 * snr_client.c - a plain C program that uses libsnr through include/snr.h
 * and the HIP runtime API alone, with no PyTorch in the process.
 *
 * Test infrastructure: tests/test_gpu_c_client.py writes the inputs, runs
 * this program and compares its outputs with the oracle.
 *
 *   snr_client DIR ROWS N f32    f32 tail, plain norm and in-place tail
 *   snr_client DIR ROWS N bf16   every other entry point, bf16 storage
 *
 * Inputs (raw little-endian arrays; f32, or bf16 bit patterns): DIR/a, DIR/r
 * ([ROWS, N]), DIR/gp, DIR/gq ([N]) and DIR/eps (two f32: eps_post,
 * eps_pre). On a stream of its own it runs, for f32:
 *   sandwich_tail(a, r, gp, eps_post, gq, eps_pre)      -> DIR/h, DIR/y
 *   rmsnorm_fwd(a, gp, eps_pre)                          -> DIR/z
 *   sandwich_tail_inplace on a copy of r                 -> DIR/hi, DIR/yi
 *   sandwich_tail_noalloc(a, r, gp, eps_post, gq, eps_pre) -> DIR/hn, DIR/yn
 *   snr_release_workspaces() at the end
 * and for bf16:
 *   sandwich_tail_typed(a, r, gp, eps_post, gq, eps_pre) -> DIR/h, DIR/y
 *   norm_then_add(a, r, gp, eps_post, no scale)          -> DIR/na
 *   add_then_norm(r, a, gq, eps_pre)                     -> DIR/s, DIR/sy
 *   rmsnorm_fwd_multi({a, gp}, {r, gq}, eps_pre)         -> DIR/m0, DIR/m1
 *   rmsnorm_q8_1(a, gp, eps_pre) when N % 32 == 0        -> DIR/q8
 * after checking that invalid arguments come back as their error codes with
 * nothing enqueued. Prints "ok" and exits 0, or names the failing step and
 * exits 1.
 */
#include <hip/hip_runtime_api.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "snr.h"

static const char *g_dir;

static int fail(const char *what, int code) {
    fprintf(stderr, "snr_client: %s failed: %d (%s)\n", what, code,
            code > 0 && code < 100 ? snr_strerror(code) : "hip");
    return 1;
}

/* a device copy of DIR/name (exactly `bytes` long), or NULL */
static void *upload(const char *name, size_t bytes) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", g_dir, name);
    FILE *f = fopen(path, "rb");
    if (!f) return NULL;
    void *host = malloc(bytes), *dev = NULL;
    const int ok = host && fread(host, 1, bytes, f) == bytes &&
                   hipMalloc(&dev, bytes) == hipSuccess &&
                   hipMemcpy(dev, host, bytes, hipMemcpyHostToDevice) ==
                       hipSuccess;
    fclose(f);
    free(host);
    return ok ? dev : NULL;
}

static void *device(size_t bytes) {
    void *d = NULL;
    return hipMalloc(&d, bytes) == hipSuccess ? d : NULL;
}

/* write `bytes` of device memory to DIR/name */
static int download(const char *name, const void *dev, size_t bytes) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", g_dir, name);
    void *host = malloc(bytes);
    int ok = host != NULL &&
             hipMemcpy(host, dev, bytes, hipMemcpyDeviceToHost) == hipSuccess;
    if (ok) {
        FILE *f = fopen(path, "wb");
        ok = f != NULL && fwrite(host, 1, bytes, f) == bytes;
        if (f) fclose(f);
    }
    free(host);
    return ok;
}

static int run_f32(int64_t rows, int64_t n, const float *eps,
                   hipStream_t stream) {
    const size_t tb = (size_t)rows * (size_t)n * 4, gb = (size_t)n * 4;
    float *a = upload("a", tb), *r = upload("r", tb), *ri = upload("r", tb);
    float *gp = upload("gp", gb), *gq = upload("gq", gb);
    float *h = device(tb), *y = device(tb), *z = device(tb), *yi = device(tb);
    float *hn = device(tb), *yn = device(tb);
    if (!a || !r || !ri || !gp || !gq || !h || !y || !z || !yi || !hn || !yn)
        return fail("inputs or device allocation", 0);

    /* invalid arguments: each is refused before anything is enqueued */
    int rc = sandwich_tail(NULL, r, gp, eps[0], gq, eps[1], h, y, rows, n,
                           stream);
    if (rc != SNR_ERR_NULL) return fail("NULL input check", rc);
    rc = sandwich_tail(a, r, gp, 0.0f, gq, eps[1], h, y, rows, n, stream);
    if (rc != SNR_ERR_EPS) return fail("eps check", rc);
    rc = sandwich_tail(a, r, gp, eps[0], gq, eps[1], h, a, rows, n, stream);
    if (rc != SNR_ERR_ALIAS) return fail("alias check", rc);
    rc = rmsnorm_fwd(a, gp, eps[1], rows, n, 7, z, stream);
    if (rc != SNR_ERR_DTYPE) return fail("dtype check", rc);
    rc = rmsnorm_fwd(a, gp, eps[1], rows, 0, SNR_F32, z, stream);
    if (rc != SNR_ERR_SHAPE) return fail("shape check", rc);
    rc = rmsnorm_fwd(a, gp, eps[1], 0, n, SNR_F32, z, stream);
    if (rc != SNR_OK) return fail("rows == 0 no-op", rc);
    rc = sandwich_tail_noalloc(a, r, gp, eps[0], gq, eps[1], hn, a, rows, n,
                               stream);
    if (rc != SNR_ERR_ALIAS) return fail("no-alloc alias check", rc);
    rc = snr_force_grid(-1);
    if (rc != SNR_ERR_SHAPE) return fail("grid cap check", rc);

    rc = sandwich_tail(a, r, gp, eps[0], gq, eps[1], h, y, rows, n, stream);
    if (rc != SNR_OK) return fail("sandwich_tail", rc);
    rc = rmsnorm_fwd(a, gp, eps[1], rows, n, SNR_F32, z, stream);
    if (rc != SNR_OK) return fail("rmsnorm_fwd", rc);
    rc = sandwich_tail_inplace(a, ri, gp, eps[0], gq, eps[1], yi, rows, n,
                               SNR_F32, stream);
    if (rc != SNR_OK) return fail("sandwich_tail_inplace", rc);
    rc = sandwich_tail_noalloc(a, r, gp, eps[0], gq, eps[1], hn, yn, rows, n,
                               stream);
    if (rc != SNR_OK) return fail("sandwich_tail_noalloc", rc);
    if (hipStreamSynchronize(stream) != hipSuccess)
        return fail("hipStreamSynchronize", 0);
    if (!download("h", h, tb) || !download("y", y, tb) ||
        !download("z", z, tb) || !download("hi", ri, tb) ||
        !download("yi", yi, tb) || !download("hn", hn, tb) ||
        !download("yn", yn, tb))
        return fail("writing outputs", 0);
    rc = snr_release_workspaces();
    if (rc != SNR_OK) return fail("snr_release_workspaces", rc);
    void *all[] = {a, r, ri, gp, gq, h, y, z, yi, hn, yn};
    for (size_t i = 0; i < sizeof all / sizeof all[0]; ++i)
        (void)hipFree(all[i]);
    return 0;
}

static int run_bf16(int64_t rows, int64_t n, const float *eps,
                    hipStream_t stream) {
    const size_t tb = (size_t)rows * (size_t)n * 2, gb = (size_t)n * 2;
    const size_t qb = (size_t)rows * (size_t)(n / 32) * 36;
    void *a = upload("a", tb), *r = upload("r", tb);
    void *gp = upload("gp", gb), *gq = upload("gq", gb);
    void *h = device(tb), *y = device(tb), *na = device(tb), *s = device(tb);
    void *sy = device(tb), *m0 = device(tb), *m1 = device(tb);
    void *q8 = n % 32 == 0 ? device(qb) : NULL;
    if (!a || !r || !gp || !gq || !h || !y || !na || !s || !sy || !m0 ||
        !m1 || (n % 32 == 0 && !q8))
        return fail("inputs or device allocation", 0);

    int rc = sandwich_tail_typed(a, r, gp, eps[0], gq, eps[1], h, y, rows, n,
                                 3, stream);
    if (rc != SNR_ERR_DTYPE) return fail("dtype check", rc);
    rc = norm_then_add(a, r, gp, eps[0], NULL, a, rows, n, SNR_BF16, stream);
    if (rc != SNR_ERR_ALIAS) return fail("norm_then_add alias check", rc);
    rc = add_then_norm(r, a, gq, -1.0f, s, sy, rows, n, SNR_BF16, stream);
    if (rc != SNR_ERR_EPS) return fail("add_then_norm eps check", rc);
    if (n % 32 != 0) {
        rc = rmsnorm_q8_1(a, gp, eps[1], rows, n, SNR_BF16, s, stream);
        if (rc != SNR_ERR_SHAPE) return fail("q8 width check", rc);
    }
    snr_segment bad[1] = {{a, gp, a, rows, eps[1]}};
    bad[0].y = (char *)a + 2; /* overlaps x without coinciding */
    rc = rmsnorm_fwd_multi(bad, 1, n, SNR_BF16, stream);
    if (rc != SNR_ERR_ALIAS) return fail("multi alias check", rc);

    rc = sandwich_tail_typed(a, r, gp, eps[0], gq, eps[1], h, y, rows, n,
                             SNR_BF16, stream);
    if (rc != SNR_OK) return fail("sandwich_tail_typed", rc);
    rc = norm_then_add(a, r, gp, eps[0], NULL, na, rows, n, SNR_BF16,
                       stream);
    if (rc != SNR_OK) return fail("norm_then_add", rc);
    rc = add_then_norm(r, a, gq, eps[1], s, sy, rows, n, SNR_BF16, stream);
    if (rc != SNR_OK) return fail("add_then_norm", rc);
    snr_segment segs[2] = {{a, gp, m0, rows, eps[1]}, {r, gq, m1, rows, eps[1]}};
    rc = rmsnorm_fwd_multi(segs, 2, n, SNR_BF16, stream);
    if (rc != SNR_OK) return fail("rmsnorm_fwd_multi", rc);
    if (q8) {
        rc = rmsnorm_q8_1(a, gp, eps[1], rows, n, SNR_BF16, q8, stream);
        if (rc != SNR_OK) return fail("rmsnorm_q8_1", rc);
    }
    if (hipStreamSynchronize(stream) != hipSuccess)
        return fail("hipStreamSynchronize", 0);
    if (!download("h", h, tb) || !download("y", y, tb) ||
        !download("na", na, tb) || !download("s", s, tb) ||
        !download("sy", sy, tb) || !download("m0", m0, tb) ||
        !download("m1", m1, tb) || (q8 && !download("q8", q8, qb)))
        return fail("writing outputs", 0);
    void *all[] = {a, r, gp, gq, h, y, na, s, sy, m0, m1, q8};
    for (size_t i = 0; i < sizeof all / sizeof all[0]; ++i)
        if (all[i]) (void)hipFree(all[i]);
    return 0;
}

int main(int argc, char **argv) {
    if (argc != 5) {
        fprintf(stderr, "usage: snr_client DIR ROWS N f32|bf16\n");
        return 2;
    }
    g_dir = argv[1];
    const int64_t rows = strtoll(argv[2], NULL, 10);
    const int64_t n = strtoll(argv[3], NULL, 10);
    const int bf16 = strcmp(argv[4], "bf16") == 0;
    if (rows < 1 || n < 1 || (!bf16 && strcmp(argv[4], "f32") != 0))
        return fail("arguments", 0);

    float eps[2];
    {
        char path[4096];
        snprintf(path, sizeof path, "%s/eps", g_dir);
        FILE *f = fopen(path, "rb");
        const int ok = f && fread(eps, sizeof(float), 2, f) == 2;
        if (f) fclose(f);
        if (!ok) return fail("reading eps", 0);
    }
    hipStream_t stream = NULL;
    if (hipStreamCreate(&stream) != hipSuccess)
        return fail("hipStreamCreate", 0);
    const int rc = bf16 ? run_bf16(rows, n, eps, stream)
                        : run_f32(rows, n, eps, stream);
    if (rc != 0) return rc;
    if (snr_last_hip_error() != 0)
        return fail("snr_last_hip_error", snr_last_hip_error());
    (void)hipStreamDestroy(stream);
    printf("ok\n");
    return 0;
}
