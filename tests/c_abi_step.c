/*
 * One rank's share of a ZeRO-3 step driven from C through libzr's C ABI alone
 * (no Python, no torch): layout, pack of the rank's own gradient, mean of the
 * contributions, AdamW with the bf16 copy, unpack into tensor views, plus one
 * rejected call.  Test infrastructure: the GPU test writes the inputs, runs
 * this program and checks its outputs against the oracle.
 *
 * Usage: c_abi_step <dir>.  <dir> holds
 *   config.bin    int64: n_tensors, numels[n_tensors], n_d, rank, threshold,
 *                 n_contrib, step; then float64: lr, beta1, beta2, eps,
 *                 weight_decay
 *   grad_<t>.bin  bf16 [numel_t], the rank's own gradient of each partitioned
 *                 tensor
 *   contrib_<k>.bin  bf16 [S], contribution k = 1 .. n_contrib - 1
 *   state.bin     fp32 master [S], exp_avg [S], exp_avg_sq [S]
 * and receives reduced.bin (bf16 [S]), state_out.bin (fp32 3 x [S]) and
 * param_<t>.bin (bf16 [numel_t]: the tensor view after the unpack, zero
 * outside the rank's range).
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "zr.h"

#define MAX_TENSORS 64

static void die(const char *what)
{
    fprintf(stderr, "c_abi_step: %s (%s)\n", what, zr_last_error());
    exit(1);
}

static void hip_check(hipError_t e, const char *what)
{
    if (e != hipSuccess) {
        fprintf(stderr, "c_abi_step: %s: %s\n", what, hipGetErrorString(e));
        exit(1);
    }
}

static void zr_check(zr_status s, const char *what)
{
    if (s != ZR_OK)
        die(what);
}

static void *read_file(const char *dir, const char *name, size_t bytes)
{
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE *f = fopen(path, "rb");
    if (!f)
        die(path);
    void *buf = malloc(bytes ? bytes : 1);
    if (!buf || fread(buf, 1, bytes, f) != bytes)
        die(path);
    fclose(f);
    return buf;
}

static void write_file(const char *dir, const char *name, const void *buf, size_t bytes)
{
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE *f = fopen(path, "wb");
    if (!f || fwrite(buf, 1, bytes, f) != bytes)
        die(path);
    fclose(f);
}

/* host buffer -> new device buffer */
static void *upload(const void *host, size_t bytes)
{
    void *d = NULL;
    hip_check(hipMalloc(&d, bytes ? bytes : 16), "hipMalloc");
    if (bytes)
        hip_check(hipMemcpy(d, host, bytes, hipMemcpyHostToDevice), "hipMemcpy H2D");
    return d;
}

int main(int argc, char **argv)
{
    if (argc != 2) {
        fprintf(stderr, "usage: c_abi_step <dir>\n");
        return 2;
    }
    const char *dir = argv[1];
    hip_check(hipSetDevice(0), "hipSetDevice");

    /* configuration */
    FILE *f;
    char path[4096];
    snprintf(path, sizeof path, "%s/config.bin", dir);
    if (!(f = fopen(path, "rb")))
        die(path);
    int64_t n_tensors = 0, numels[MAX_TENSORS], n_d, rank, threshold, n_contrib, step;
    double hpd[5];
    if (fread(&n_tensors, 8, 1, f) != 1 || n_tensors < 1 || n_tensors > MAX_TENSORS ||
        fread(numels, 8, (size_t)n_tensors, f) != (size_t)n_tensors || fread(&n_d, 8, 1, f) != 1 ||
        fread(&rank, 8, 1, f) != 1 || fread(&threshold, 8, 1, f) != 1 || fread(&n_contrib, 8, 1, f) != 1 ||
        fread(&step, 8, 1, f) != 1 || fread(hpd, 8, 5, f) != 5)
        die("config.bin");
    fclose(f);
    if (n_contrib < 1 || n_contrib > 256)
        die("n_contrib");

    /* layout and this rank's range */
    zr_layout *L = NULL;
    zr_check(zr_layout_create(numels, (int32_t)n_tensors, (int32_t)n_d, threshold, &L), "zr_layout_create");
    int64_t b = 0, e = 0;
    zr_check(zr_layout_rank_range(L, (int32_t)rank, &b, &e), "zr_layout_rank_range");
    const int64_t S = e - b;

    /* per-tensor gradient views (whole tensors; persistent ones absent) */
    zr_view gviews[MAX_TENSORS], pviews[MAX_TENSORS];
    for (int64_t t = 0; t < n_tensors; ++t) {
        int32_t persistent = 0;
        int64_t off = 0;
        zr_check(zr_layout_tensor(L, (int32_t)t, &persistent, &off), "zr_layout_tensor");
        gviews[t].ptr = pviews[t].ptr = NULL;
        gviews[t].first = pviews[t].first = 0;
        gviews[t].count = pviews[t].count = numels[t];
        if (persistent)
            continue;
        char name[64];
        snprintf(name, sizeof name, "grad_%lld.bin", (long long)t);
        void *h = read_file(dir, name, (size_t)numels[t] * 2);
        gviews[t].ptr = upload(h, (size_t)numels[t] * 2);
        free(h);
        hip_check(hipMalloc(&pviews[t].ptr, (size_t)numels[t] * 2 + 16), "hipMalloc");
        hip_check(hipMemset(pviews[t].ptr, 0, (size_t)numels[t] * 2), "hipMemset");
    }

    /* contributions: 0 is this rank's own gradient packed over its slice */
    const void *contribs[256];
    void *c0 = NULL;
    hip_check(hipMalloc(&c0, (size_t)S * 2 + 16), "hipMalloc");
    zr_check(zr_pack(L, gviews, (int32_t)n_tensors, c0, b, e, NULL), "zr_pack");
    contribs[0] = c0;
    for (int64_t k = 1; k < n_contrib; ++k) {
        char name[64];
        snprintf(name, sizeof name, "contrib_%lld.bin", (long long)k);
        void *h = read_file(dir, name, (size_t)S * 2);
        contribs[k] = upload(h, (size_t)S * 2);
        free(h);
    }
    void *grad = NULL;
    hip_check(hipMalloc(&grad, (size_t)S * 2 + 16), "hipMalloc");
    zr_check(zr_reduce_slice(contribs, (int32_t)n_contrib, S, grad, NULL), "zr_reduce_slice");

    /* AdamW on the shard, bf16 copy into the rank's slot of the flat buffer */
    float *st_h = (float *)read_file(dir, "state.bin", (size_t)S * 12);
    float *st = (float *)upload(st_h, (size_t)S * 12);
    void *flat = NULL;
    hip_check(hipMalloc(&flat, (size_t)S * 2 + 16), "hipMalloc");
    zr_adamw_hparams hp;
    hp.lr = hpd[0];
    hp.beta1 = hpd[1];
    hp.beta2 = hpd[2];
    hp.eps = hpd[3];
    hp.weight_decay = hpd[4];
    hp.grad_scale = 1.0;
    hp.step = step;
    zr_check(zr_adamw_step(grad, st, st + S, st + 2 * S, flat, S, &hp, NULL), "zr_adamw_step");
    zr_check(zr_unpack(L, flat, b, e, pviews, (int32_t)n_tensors, NULL), "zr_unpack");

    /* a rejected call: no contributions */
    if (zr_reduce_slice(contribs, 0, S, grad, NULL) != ZR_EINVAL || zr_last_error()[0] == '\0')
        die("n = 0 was not rejected with ZR_EINVAL and a message");

    hip_check(hipDeviceSynchronize(), "hipDeviceSynchronize");

    /* outputs */
    void *h = malloc((size_t)S * 12 + 16);
    if (!h)
        die("malloc");
    hip_check(hipMemcpy(h, grad, (size_t)S * 2, hipMemcpyDeviceToHost), "hipMemcpy D2H");
    write_file(dir, "reduced.bin", h, (size_t)S * 2);
    hip_check(hipMemcpy(h, st, (size_t)S * 12, hipMemcpyDeviceToHost), "hipMemcpy D2H");
    write_file(dir, "state_out.bin", h, (size_t)S * 12);
    free(h);
    for (int64_t t = 0; t < n_tensors; ++t) {
        if (!pviews[t].ptr)
            continue;
        void *p = malloc((size_t)numels[t] * 2 + 16);
        if (!p)
            die("malloc");
        hip_check(hipMemcpy(p, pviews[t].ptr, (size_t)numels[t] * 2, hipMemcpyDeviceToHost), "hipMemcpy D2H");
        char name[64];
        snprintf(name, sizeof name, "param_%lld.bin", (long long)t);
        write_file(dir, name, p, (size_t)numels[t] * 2);
        free(p);
        hipFree(pviews[t].ptr);
        hipFree(gviews[t].ptr);
    }
    for (int64_t k = 0; k < n_contrib; ++k)
        hipFree((void *)contribs[k]);
    hipFree(grad);
    hipFree(st);
    hipFree(flat);
    free(st_h);
    zr_layout_destroy(L);
    printf("c_abi_step: shard [%lld, %lld) done\n", (long long)b, (long long)e);
    return 0;
}
