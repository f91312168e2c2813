/* moe_c_caller.c -- the layer driven from C through include/moe.h alone.
 *
 * Reads a layer config and its inputs from a binary file, runs moe_route
 * (with the logits written out), moe_forward and moe_balance_stats on the
 * current GPU, and writes the outputs to a second file.  The GPU tests use it
 * to show that a caller needs nothing beyond the header, the HIP runtime and
 * libmoe.so; `--host` runs only calls that need no device (status strings,
 * argument validation).
 *
 * Input file, little-endian:
 *   int32 magic 0x4D4F4531, then the moe_config fields in declaration order
 *   (13 x 32-bit), float alpha1, int32 has_offset, int32 has_bias; then
 *   x [T][d], w_gate [N'][d], offset [N'] f32 (if has_offset), bias [N'] f32
 *   (if has_bias), w13 [N'][2 d_ff][d], w2 [N'][d][d_ff],
 *   w13_shared [K_s][2 d_ff_s][d], w2_shared [K_s][d][d_ff_s] (elements of
 *   2 bytes for MOE_BF16, 4 for MOE_F32).
 * Output file: logits [T][N'] f32, topk_idx [T][K'] i32, topk_w [T][K'] f32,
 *   expert_counts [N'] i32, h [T][d] (element type of x), f [N'] f32,
 *   P [N'] f32, loss [2] f32.
 * Exit status 0 on success; otherwise a message naming the failing call. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "moe.h"

#define MAGIC 0x4D4F4531

static void fail(const char *what, const char *detail) {
    fprintf(stderr, "moe_c_caller: %s: %s\n", what, detail);
    exit(1);
}

static void check_hip(hipError_t e, const char *what) {
    if (e != hipSuccess) fail(what, hipGetErrorString(e));
}

static void check_moe(int rc, const char *what) {
    if (rc != MOE_OK) fail(what, moe_status_string(rc));
}

static void read_exact(FILE *f, void *p, size_t n, const char *what) {
    if (n && fread(p, 1, n, f) != n) fail("short input", what);
}

/* host copy of n bytes from the file, then a device copy of it */
static void *to_device(FILE *f, size_t n, const char *what) {
    void *h = malloc(n ? n : 1), *d = NULL;
    if (!h) fail("malloc", what);
    read_exact(f, h, n, what);
    check_hip(hipMalloc(&d, n ? n : 1), what);
    if (n) check_hip(hipMemcpy(d, h, n, hipMemcpyHostToDevice), what);
    free(h);
    return d;
}

static void *device_zeros(size_t n, const char *what) {
    void *d = NULL;
    check_hip(hipMalloc(&d, n ? n : 1), what);
    check_hip(hipMemset(d, 0, n ? n : 1), what);
    return d;
}

static void write_back(FILE *f, const void *d, size_t n, const char *what) {
    void *h = malloc(n ? n : 1);
    if (!h) fail("malloc", what);
    check_hip(hipMemcpy(h, d, n, hipMemcpyDeviceToHost), what);
    if (n && fwrite(h, 1, n, f) != n) fail("short write", what);
    free(h);
}

static int host_checks(void) {
    /* status strings, and argument errors caught before any device work */
    for (int s = MOE_ERR_HIP; s <= MOE_OK; ++s)
        if (!moe_status_string(s) || !moe_status_string(s)[0]) fail("moe_status_string", "empty");
    moe_config c;
    memset(&c, 0, sizeof c);
    c.T = 8;
    c.d_model = 64;
    c.n_routed = 4;
    c.top_k = 2;
    c.d_ff = 64;
    c.scoring = MOE_SCORE_SOFTMAX;
    c.dtype = MOE_F32;
    if (moe_workspace_bytes(&c, MOE_WS_FORWARD) == 0) fail("moe_workspace_bytes", "0 for a valid config");
    int32_t idx[16];
    float w[16];
    int32_t counts[4];
    if (moe_route(NULL, NULL, NULL, NULL, NULL, NULL, NULL, idx, w, counts, NULL, NULL, 0, NULL) !=
        MOE_ERR_INVALID_ARG)
        fail("moe_route", "a NULL config was accepted");
    c.top_k = 5; /* K' > N' */
    if (moe_workspace_bytes(&c, MOE_WS_FORWARD) != 0) fail("moe_workspace_bytes", "K' > N' accepted");
    printf("host checks ok\n");
    return 0;
}

int main(int argc, char **argv) {
    if (argc == 2 && strcmp(argv[1], "--host") == 0) return host_checks();
    if (argc != 3) {
        fprintf(stderr, "usage: moe_c_caller INPUT OUTPUT | --host\n");
        return 2;
    }
    FILE *in = fopen(argv[1], "rb");
    if (!in) fail("open", argv[1]);
    int32_t hdr[14];
    read_exact(in, hdr, sizeof hdr, "header");
    if (hdr[0] != MAGIC) fail("header", "bad magic");
    moe_config c;
    memset(&c, 0, sizeof c);
    c.T = hdr[1];
    c.d_model = hdr[2];
    c.n_routed = hdr[3];
    c.top_k = hdr[4];
    c.n_shared = hdr[5];
    c.d_ff = hdr[6];
    c.d_ff_shared = hdr[7];
    c.scoring = hdr[8];
    c.renorm = hdr[9];
    c.dtype = hdr[10];
    c.flags = (uint32_t)hdr[11];
    c.n_groups = hdr[12];
    c.topk_groups = hdr[13];
    float alpha1;
    int32_t has_offset, has_bias;
    read_exact(in, &alpha1, 4, "alpha1");
    read_exact(in, &has_offset, 4, "has_offset");
    read_exact(in, &has_bias, 4, "has_bias");
    const size_t eb = c.dtype == MOE_BF16 ? 2 : 4;
    const size_t T = (size_t)c.T, d = (size_t)c.d_model, N = (size_t)c.n_routed;
    const size_t K = (size_t)c.top_k, Ks = (size_t)c.n_shared, f = (size_t)c.d_ff;
    const size_t fs = (size_t)c.d_ff_shared;

    void *x = to_device(in, T * d * eb, "x");
    void *wg = to_device(in, N * d * eb, "w_gate");
    float *offset = has_offset ? (float *)to_device(in, N * 4, "offset") : NULL;
    float *bias = has_bias ? (float *)to_device(in, N * 4, "bias") : NULL;
    void *w13 = to_device(in, N * 2 * f * d * eb, "w13");
    void *w2 = to_device(in, N * d * f * eb, "w2");
    void *w13s = Ks ? to_device(in, Ks * 2 * fs * d * eb, "w13_shared") : NULL;
    void *w2s = Ks ? to_device(in, Ks * d * fs * eb, "w2_shared") : NULL;
    fclose(in);

    moe_config cr = c;
    cr.flags = MOE_LOGITS_OUT;
    c.flags = 0;
    const size_t ws_route = moe_workspace_bytes(&cr, MOE_WS_ROUTE);
    const size_t ws_fwd = moe_workspace_bytes(&c, MOE_WS_FORWARD);
    const size_t ws_pstat = moe_workspace_bytes(&c, MOE_WS_PSTAT);
    if (!ws_route || !ws_fwd || !ws_pstat) fail("moe_workspace_bytes", "0");
    float *logits = (float *)device_zeros(T * N * 4, "logits");
    int32_t *idx = (int32_t *)device_zeros(T * K * 4, "topk_idx");
    float *w = (float *)device_zeros(T * K * 4, "topk_w");
    int32_t *counts = (int32_t *)device_zeros(N * 4, "expert_counts");
    void *pstat = device_zeros(ws_pstat, "p_partial");
    void *wsr = device_zeros(ws_route, "route workspace");
    void *wsf = device_zeros(ws_fwd, "forward workspace");
    void *h = device_zeros(T * d * eb, "h");
    float *fo = (float *)device_zeros(N * 4, "f");
    float *P = (float *)device_zeros(N * 4, "P");
    float *loss = (float *)device_zeros(8, "loss");

    hipStream_t s;
    check_hip(hipStreamCreate(&s), "hipStreamCreate");
    check_moe(moe_route(&cr, x, wg, offset, bias, NULL, logits, idx, w, counts, pstat, wsr, ws_route,
                        (void *)s),
              "moe_route");
    check_moe(moe_forward(&c, x, idx, w, w13, w2, w13s, w2s, h, wsf, ws_fwd, (void *)s), "moe_forward");
    check_moe(moe_balance_stats(&c, counts, pstat, alpha1, fo, P, loss, (void *)s), "moe_balance_stats");
    check_hip(hipStreamSynchronize(s), "hipStreamSynchronize");

    FILE *out = fopen(argv[2], "wb");
    if (!out) fail("open", argv[2]);
    write_back(out, logits, T * N * 4, "logits");
    write_back(out, idx, T * K * 4, "topk_idx");
    write_back(out, w, T * K * 4, "topk_w");
    write_back(out, counts, N * 4, "expert_counts");
    write_back(out, h, T * d * eb, "h");
    write_back(out, fo, N * 4, "f");
    write_back(out, P, N * 4, "P");
    write_back(out, loss, 8, "loss");
    if (fclose(out) != 0) fail("close", argv[2]);
    check_hip(hipStreamDestroy(s), "hipStreamDestroy");
    printf("layer ok: T=%d d=%d N'=%d K'=%d\n", c.T, c.d_model, c.n_routed, c.top_k);
    return 0;
}
