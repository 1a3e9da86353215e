/* A plain C11 user of libmoedx.so: only include/moedx.h and the HIP runtime
 * API, no C++ and no Python.
 *
 *   c_consumer validate          host-side argument checks (no GPU needed)
 *   c_consumer run IN OUT        one exact-mode step on device 0: layout,
 *                                prepare from the layout's outputs, first
 *                                dispatch, gate-weighted combine
 *
 * IN  (little-endian): int32 T, K, E, R, C, H; int64 topk_idx[T*K];
 *     uint16 x[T*H] (bf16 bits); float weights[T*K]
 * OUT: int32 N; int32 num_tokens_per_rank[R]; int32 num_tokens_per_expert[E];
 *      uint8 is_token_in_rank[T*R]; uint16 recv_x[N*H]; int64 recv_topk_idx[N*K];
 *      float recv_topk_weights[N*K]; uint16 combined[T*H]
 */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "moedx.h"

#define CHECK(call)                                                                  \
    do {                                                                             \
        int rc_ = (call);                                                            \
        if (rc_ != MOEDX_OK) {                                                       \
            fprintf(stderr, "%s failed: %d (%s)\n", #call, rc_, moedx_last_error()); \
            exit(1);                                                                 \
        }                                                                            \
    } while (0)
#define HIPCHECK(call)                                                   \
    do {                                                                 \
        hipError_t e_ = (call);                                          \
        if (e_ != hipSuccess) {                                          \
            fprintf(stderr, "%s failed: %d\n", #call, (int)e_);          \
            exit(1);                                                     \
        }                                                                \
    } while (0)

static int expect(int got, int want, const char* what) {
    if (got != want) {
        fprintf(stderr, "%s: got %d, want %d\n", what, got, want);
        return 1;
    }
    if (want != MOEDX_OK && moedx_last_error()[0] == '\0') {
        fprintf(stderr, "%s: no error message\n", what);
        return 1;
    }
    return 0;
}

static int validate(void) {
    int bad = 0;
    moedx_ctx* ctx = (moedx_ctx*)0x1;
    int64_t dummy[4];
    int32_t d32[4];
    uint8_t d8[4];
    bad |= expect(moedx_create(&ctx, 0, 16, 3, 2, 128, 0), MOEDX_EINVAL, "E % R != 0");
    bad |= expect(ctx == NULL ? 0 : 1, 0, "ctx cleared on error");
    bad |= expect(moedx_create(&ctx, 0, 16, 4, 0, 128, 0), MOEDX_EINVAL, "C < 1");
    bad |= expect(moedx_get_dispatch_layout_static(dummy, 10, 2, 16, 65, d32, d32, d8, NULL),
                  MOEDX_EINVAL, "static layout, R > 64");
    bad |= expect(moedx_get_dispatch_layout_static(NULL, 10, 2, 16, 4, d32, d32, d8, NULL),
                  MOEDX_EINVAL, "static layout, NULL topk_idx");
    bad |= expect(moedx_event_wait(NULL, NULL), MOEDX_EINVAL, "event_wait(NULL)");
    bad |= expect(moedx_destroy(NULL), MOEDX_OK, "destroy(NULL)");
    bad |= expect(moedx_handle_destroy(NULL), MOEDX_OK, "handle_destroy(NULL)");
    if (!bad) printf("validate ok\n");
    return bad;
}

static void* read_exact(FILE* f, size_t n) {
    void* p = malloc(n ? n : 1);
    if (!p || fread(p, 1, n, f) != n) {
        fprintf(stderr, "short input\n");
        exit(1);
    }
    return p;
}

static void* to_device(const void* h, size_t n) {
    void* d = NULL;
    HIPCHECK(hipMalloc(&d, n ? n : 16));
    if (n) HIPCHECK(hipMemcpy(d, h, n, hipMemcpyHostToDevice));
    return d;
}

static void write_back(FILE* f, const void* d, size_t n) {
    void* h = malloc(n ? n : 1);
    if (!h) exit(1);
    if (n) HIPCHECK(hipMemcpy(h, d, n, hipMemcpyDeviceToHost));
    if (fwrite(h, 1, n, f) != n) exit(1);
    free(h);
}

static int run(const char* in_path, const char* out_path) {
    FILE* in = fopen(in_path, "rb");
    if (!in) return 1;
    int32_t* dims = (int32_t*)read_exact(in, 6 * sizeof(int32_t));
    const int T = dims[0], K = dims[1], E = dims[2], R = dims[3], C = dims[4], H = dims[5];
    int64_t* idx = (int64_t*)read_exact(in, (size_t)T * K * 8);
    uint16_t* x = (uint16_t*)read_exact(in, (size_t)T * H * 2);
    float* w = (float*)read_exact(in, (size_t)T * K * 4);
    fclose(in);

    void* d_idx = to_device(idx, (size_t)T * K * 8);
    void* d_x = to_device(x, (size_t)T * H * 2);
    void* d_w = to_device(w, (size_t)T * K * 4);
    moedx_ctx* ctx = NULL;
    CHECK(moedx_create(&ctx, 0, E, R, C, T, 0));
    void *d_ntr, *d_nte, *d_itr;
    HIPCHECK(hipMalloc(&d_ntr, (size_t)R * 4));
    HIPCHECK(hipMalloc(&d_nte, (size_t)E * 4));
    HIPCHECK(hipMalloc(&d_itr, (size_t)T * R + 16));
    /* a NULL exec: the caller's null stream, blocking until done */
    CHECK(moedx_get_dispatch_layout(ctx, (const int64_t*)d_idx, T, K, (int32_t*)d_ntr,
                                    (int32_t*)d_nte, (uint8_t*)d_itr, NULL));
    size_t ws_bytes = 0;
    CHECK(moedx_handle_workspace_bytes(ctx, T, K, 0, &ws_bytes));
    void* d_ws = NULL;
    HIPCHECK(hipMalloc(&d_ws, ws_bytes));
    moedx_handle* h = NULL;
    CHECK(moedx_dispatch_prepare(ctx, (const int64_t*)d_idx, T, K, (const int32_t*)d_ntr,
                                 (const uint8_t*)d_itr, (const int32_t*)d_nte, d_ws, ws_bytes, 0,
                                 &h, NULL));
    int64_t N = 0;
    CHECK(moedx_handle_num_recv(h, &N));
    void *d_recv, *d_rti, *d_rtw, *d_out;
    HIPCHECK(hipMalloc(&d_recv, (size_t)(N > 0 ? N : 1) * H * 2));
    HIPCHECK(hipMalloc(&d_rti, (size_t)(N > 0 ? N : 1) * K * 8));
    HIPCHECK(hipMalloc(&d_rtw, (size_t)(N > 0 ? N : 1) * K * 4));
    HIPCHECK(hipMalloc(&d_out, (size_t)(T > 0 ? T : 1) * H * 2));
    CHECK(moedx_dispatch(ctx, h, d_x, T, H, MOEDX_QUANT_NONE, (const int64_t*)d_idx,
                         (const float*)d_w, d_recv, NULL, (int64_t*)d_rti, (float*)d_rtw, NULL));
    CHECK(moedx_combine(ctx, h, (const uint16_t*)d_recv, H, (const float*)d_w, NULL,
                        (uint16_t*)d_out, NULL, NULL));

    FILE* out = fopen(out_path, "wb");
    if (!out) return 1;
    const int32_t n32 = (int32_t)N;
    if (fwrite(&n32, 4, 1, out) != 1) return 1;
    write_back(out, d_ntr, (size_t)R * 4);
    write_back(out, d_nte, (size_t)E * 4);
    write_back(out, d_itr, (size_t)T * R);
    write_back(out, d_recv, (size_t)N * H * 2);
    write_back(out, d_rti, (size_t)N * K * 8);
    write_back(out, d_rtw, (size_t)N * K * 4);
    write_back(out, d_out, (size_t)T * H * 2);
    fclose(out);

    CHECK(moedx_handle_destroy(h));
    CHECK(moedx_destroy(ctx));
    void* bufs[] = {d_idx, d_x, d_w, d_ntr, d_nte, d_itr, d_ws, d_recv, d_rti, d_rtw, d_out};
    for (size_t i = 0; i < sizeof(bufs) / sizeof(bufs[0]); ++i) HIPCHECK(hipFree(bufs[i]));
    free(dims);
    free(idx);
    free(x);
    free(w);
    printf("run ok: N=%lld\n", (long long)N);
    return 0;
}

int main(int argc, char** argv) {
    if (argc >= 2 && strcmp(argv[1], "validate") == 0) return validate();
    if (argc >= 4 && strcmp(argv[1], "run") == 0) return run(argv[2], argv[3]);
    fprintf(stderr, "usage: %s validate | run IN OUT\n", argv[0]);
    return 2;
}
