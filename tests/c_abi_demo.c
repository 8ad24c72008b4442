/*
 * A plain C99 program against the library's C ABI (include/gdn.h), with no
 * Python or C++ in between.
 *
 *   c_abi_demo check
 *       Validation answers that need no GPU: version, status strings,
 *       workspace sizes, and the documented status of bad calls (returned
 *       before any launch).  Prints the workspace sizes it read.
 *
 *   c_abi_demo run DIR B T Hk Hv Dk Dv K q_scale k_scale
 *       One gdn_layer_core call on the GPU: reads the raw inputs from DIR
 *       (qkv, conv_w, conv_state, a, b, A_log, dt_bias, state: row-major
 *       little-endian bytes, shapes as the header states), copies them to
 *       device memory, runs the call on the null stream, and writes y,
 *       state_out and conv_state_out back to DIR.
 *
 * Exit status 0 on success; a message on stderr otherwise.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "gdn.h"

static int failures = 0;

static void expect_status(const char *what, gdn_status got, gdn_status want) {
    if (got != want) {
        fprintf(stderr, "%s: status %s, expected %s (%s)\n", what, gdn_status_string(got),
                gdn_status_string(want), gdn_last_error());
        ++failures;
    } else if (want != GDN_OK && gdn_last_error()[0] == '\0') {
        fprintf(stderr, "%s: no error description\n", what);
        ++failures;
    }
}

/* fake, distinct, 256-byte aligned addresses: validation never reads them */
static void *fake(int i) { return (void *)(uintptr_t)(((uint64_t)1 << 40) + (uint64_t)i * ((uint64_t)1 << 34)); }

static int check(void) {
    if (gdn_version() < 1) {
        fprintf(stderr, "gdn_version() = %d\n", gdn_version());
        ++failures;
    }
    if (strcmp(gdn_status_string(GDN_ERR_BAD_DIMS), "GDN_ERR_BAD_DIMS") != 0) {
        fprintf(stderr, "status string: %s\n", gdn_status_string(GDN_ERR_BAD_DIMS));
        ++failures;
    }
    const size_t ws_core = gdn_layer_core_workspace_bytes(1, 4096, 16, 32, 128, 128);
    const size_t ws_chunked = gdn_recurrent_chunked_workspace_bytes(1, 4096, 16, 32, 128, 128);
    const size_t ws_decode = gdn_layer_core_workspace_bytes(64, 1, 16, 32, 128, 128);
    printf("layer_core_workspace_bytes(1,4096,16,32,128,128) %zu\n", ws_core);
    printf("recurrent_chunked_workspace_bytes(1,4096,16,32,128,128) %zu\n", ws_chunked);
    printf("layer_core_workspace_bytes(64,1,16,32,128,128) %zu\n", ws_decode);
    if (ws_core == 0 || ws_chunked == 0) {
        fprintf(stderr, "zero workspace for the prefill sizes\n");
        ++failures;
    }

    const gdn_bf16 *q = fake(0), *k = fake(1), *v = fake(2);
    const float *g = fake(3), *beta = fake(4), *s_in = fake(5);
    float *s_out = fake(6);
    gdn_bf16 *y = fake(7);
    /* Hv not a multiple of Hk */
    expect_status("Hv % Hk", gdn_recurrent(q, k, v, g, beta, s_in, s_out, y, 1, 8, 3, 4, 64, 32, NULL),
                  GDN_ERR_BAD_DIMS);
    /* unsupported key size */
    expect_status("Dk = 48", gdn_recurrent(q, k, v, g, beta, s_in, s_out, y, 1, 8, 2, 4, 48, 32, NULL),
                  GDN_ERR_UNSUPPORTED);
    /* a missing input */
    expect_status("q = NULL", gdn_recurrent(NULL, k, v, g, beta, s_in, s_out, y, 1, 8, 2, 4, 64, 32, NULL),
                  GDN_ERR_NULL_POINTER);
    /* a pointer off 16-byte alignment */
    expect_status("misaligned k",
                  gdn_recurrent(q, (const gdn_bf16 *)((const char *)k + 2), v, g, beta, s_in, s_out, y, 1, 8, 2,
                                4, 64, 32, NULL),
                  GDN_ERR_MISALIGNED);
    /* y on top of v */
    expect_status("y overlaps v", gdn_recurrent(q, k, v, g, beta, s_in, s_out, (gdn_bf16 *)v, 1, 8, 2, 4, 64, 32, NULL),
                  GDN_ERR_OVERLAP);
    /* the chunked form without a workspace */
    expect_status("no workspace",
                  gdn_recurrent_chunked(q, k, v, g, beta, s_in, s_out, y, NULL, 0, 1, 64, 2, 4, 128, 32, NULL),
                  GDN_ERR_WORKSPACE);
    /* an empty batch is valid and does nothing */
    expect_status("B = 0", gdn_recurrent(q, k, v, g, beta, s_in, s_out, y, 0, 8, 2, 4, 64, 32, NULL), GDN_OK);
    if (failures == 0) printf("check ok\n");
    return failures ? 1 : 0;
}

#define HIP_OK(call)                                                                      \
    do {                                                                                  \
        hipError_t e_ = (call);                                                           \
        if (e_ != hipSuccess) {                                                           \
            fprintf(stderr, "%s: %s\n", #call, hipGetErrorString(e_));                    \
            return 1;                                                                     \
        }                                                                                 \
    } while (0)

/* reads DIR/name (exactly n bytes) into a new device buffer */
static int upload(const char *dir, const char *name, size_t n, void **dev) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE *f = fopen(path, "rb");
    if (!f) {
        fprintf(stderr, "cannot open %s\n", path);
        return 1;
    }
    void *host = malloc(n ? n : 1);
    const size_t got = host ? fread(host, 1, n, f) : 0;
    const int extra = fgetc(f) != EOF;
    fclose(f);
    if (!host || got != n || extra) {
        fprintf(stderr, "%s: expected %zu bytes\n", path, n);
        free(host);
        return 1;
    }
    HIP_OK(hipMalloc(dev, n ? n : 1));
    HIP_OK(hipMemcpy(*dev, host, n, hipMemcpyHostToDevice));
    free(host);
    return 0;
}

static int download(const char *dir, const char *name, const void *dev, size_t n) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    void *host = malloc(n ? n : 1);
    if (!host) return 1;
    HIP_OK(hipMemcpy(host, dev, n, hipMemcpyDeviceToHost));
    FILE *f = fopen(path, "wb");
    const size_t put = f ? fwrite(host, 1, n, f) : 0;
    if (f) fclose(f);
    free(host);
    if (put != n) {
        fprintf(stderr, "cannot write %s\n", path);
        return 1;
    }
    return 0;
}

static int run(int argc, char **argv) {
    if (argc != 12) {
        fprintf(stderr, "usage: c_abi_demo run DIR B T Hk Hv Dk Dv K q_scale k_scale\n");
        return 2;
    }
    const char *dir = argv[2];
    const int B = atoi(argv[3]), T = atoi(argv[4]), Hk = atoi(argv[5]), Hv = atoi(argv[6]);
    const int Dk = atoi(argv[7]), Dv = atoi(argv[8]), K = atoi(argv[9]);
    const float q_scale = (float)atof(argv[10]), k_scale = (float)atof(argv[11]);
    if (B < 1 || T < 1 || Hk < 1 || Hv < 1 || Dk < 1 || Dv < 1 || K < 2) {
        fprintf(stderr, "bad sizes\n");
        return 2;
    }
    const size_t C = (size_t)2 * Hk * Dk + (size_t)Hv * Dv;
    const size_t n_qkv = (size_t)B * T * C, n_cs = (size_t)B * (K - 1) * C, n_ab = (size_t)B * T * Hv;
    const size_t n_s = (size_t)B * Hv * Dv * Dk, n_y = (size_t)B * T * Hv * Dv;
    void *qkv, *conv_w, *cs_in, *a, *b, *A_log, *dt_bias, *s_in, *s_out, *y, *cs_out, *ws = NULL;
    if (upload(dir, "qkv", 2 * n_qkv, &qkv) || upload(dir, "conv_w", 2 * C * K, &conv_w) ||
        upload(dir, "conv_state", 2 * n_cs, &cs_in) || upload(dir, "a", 2 * n_ab, &a) ||
        upload(dir, "b", 2 * n_ab, &b) || upload(dir, "A_log", 4 * (size_t)Hv, &A_log) ||
        upload(dir, "dt_bias", 4 * (size_t)Hv, &dt_bias) || upload(dir, "state", 4 * n_s, &s_in))
        return 1;
    HIP_OK(hipMalloc(&s_out, 4 * n_s));
    HIP_OK(hipMalloc(&y, 2 * n_y));
    HIP_OK(hipMalloc(&cs_out, 2 * n_cs));
    const size_t nws = gdn_layer_core_workspace_bytes(B, T, Hk, Hv, Dk, Dv);
    if (nws) HIP_OK(hipMalloc(&ws, nws));
    const gdn_status st = gdn_layer_core(qkv, conv_w, cs_in, cs_out, a, b, A_log, dt_bias, s_in, s_out, y, ws, nws,
                                         B, T, Hk, Hv, Dk, Dv, K, q_scale, k_scale, 1e-6f, NULL);
    if (st != GDN_OK) {
        fprintf(stderr, "gdn_layer_core: %s (%s)\n", gdn_status_string(st), gdn_last_error());
        return 1;
    }
    HIP_OK(hipDeviceSynchronize());
    if (download(dir, "y", y, 2 * n_y) || download(dir, "state_out", s_out, 4 * n_s) ||
        download(dir, "conv_state_out", cs_out, 2 * n_cs))
        return 1;
    void *bufs[] = {qkv, conv_w, cs_in, a, b, A_log, dt_bias, s_in, s_out, y, cs_out, ws};
    for (size_t i = 0; i < sizeof bufs / sizeof bufs[0]; ++i)
        if (bufs[i]) HIP_OK(hipFree(bufs[i]));
    printf("run ok: B=%d T=%d workspace %zu bytes\n", B, T, nws);
    return 0;
}

int main(int argc, char **argv) {
    if (argc >= 2 && strcmp(argv[1], "check") == 0) return check();
    if (argc >= 2 && strcmp(argv[1], "run") == 0) return run(argc, argv);
    fprintf(stderr, "usage: c_abi_demo check | run DIR B T Hk Hv Dk Dv K q_scale k_scale\n");
    return 2;
}
