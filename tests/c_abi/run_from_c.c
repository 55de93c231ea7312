/*
 * A C99 program that uses the library on the GPU with nothing but the HIP
 * runtime's C API and include/skinny.h: hipMalloc'd buffers, skinny_prepare
 * (which tunes the shape), skinny_run for every M = 1..64, a hipGraph that
 * captures a run and is replayed, and skinny_run_static with a K-split
 * tactic.  Inputs are small integers, so every sum is exact in fp32 and the
 * result must equal a plain int64 triple loop bit for bit (fp32 out) or its
 * nearest-even BF16 rounding (BF16 out); rows of out at and beyond M must
 * keep their sentinel.  Prints "c run ok <checks>" and exits 0, or names the
 * first failed check and exits 1.  Built by tests/c_abi/build.py.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "skinny.h"

enum { N = 1000, K = 1032, MAXM = 64 };

static long checks;

#define CHECK(cond, ...)                                                \
    do {                                                                \
        ++checks;                                                       \
        if (!(cond)) {                                                  \
            printf("check failed at line %d: %s: ", __LINE__, #cond);   \
            printf(__VA_ARGS__);                                        \
            printf(" (last error: %s)\n", skinny_last_error());         \
            return 1;                                                   \
        }                                                               \
    } while (0)

#define HIP(call)                                                              \
    do {                                                                       \
        hipError_t e_ = (call);                                                \
        if (e_ != hipSuccess) {                                                \
            printf("%s failed at line %d: %s\n", #call, __LINE__,              \
                   hipGetErrorString(e_));                                     \
            return 1;                                                          \
        }                                                                      \
    } while (0)

static uint16_t bf16_of_int(int v)
{
    float f = (float)v;   /* small integers: exact in BF16 */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

static uint16_t bf16_rne(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

static uint32_t f32_bits(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    return u;
}

/* out rows < m against the exact sums, rows >= m against the sentinel */
static int check_out(const void *host, int f32, int m, const int64_t *ref, const char *what)
{
    int r, n;
    for (r = 0; r < MAXM; ++r)
        for (n = 0; n < N; ++n) {
            uint32_t got = f32 ? ((const uint32_t *)host)[r * N + n] : ((const uint16_t *)host)[r * N + n];
            uint32_t want;
            if (r >= m)
                want = f32 ? 0x7FBFBFBFu : 0x7FBFu;
            else
                want = f32 ? f32_bits((float)ref[r * N + n]) : bf16_rne((float)ref[r * N + n]);
            CHECK(got == want, "%s M=%d row %d col %d: got %#x want %#x", what, m, r, n, got, want);
        }
    return 0;
}

static int fill_sentinel(void *dev, int f32, hipStream_t stream)
{
    static uint32_t pattern[MAXM * N];
    size_t i;
    for (i = 0; i < (size_t)MAXM * N; ++i)
        pattern[i] = f32 ? 0x7FBFBFBFu : 0x7FBF7FBFu;
    HIP(hipMemcpyAsync(dev, pattern, (size_t)MAXM * N * (f32 ? 4 : 2), hipMemcpyHostToDevice, stream));
    HIP(hipStreamSynchronize(stream));
    return 0;
}

int main(void)
{
    static uint16_t w_host[N * K], x_host[MAXM * K];
    static int64_t ref[MAXM * N];
    static uint32_t out_host[MAXM * N];
    uint32_t state = 12345u;
    void *w_dev = NULL, *x_dev = NULL, *out_dev = NULL;
    hipStream_t stream;
    int i, r, n, k, m, f32;

    for (i = 0; i < N * K; ++i) {
        state = state * 1664525u + 1013904223u;
        w_host[i] = bf16_of_int((int)(state >> 29) - 3);     /* -3..4 */
    }
    for (i = 0; i < MAXM * K; ++i) {
        state = state * 1664525u + 1013904223u;
        x_host[i] = bf16_of_int((int)((state >> 28) % 7u) - 3);   /* -3..3 */
    }
    for (r = 0; r < MAXM; ++r)
        for (n = 0; n < N; ++n) {
            int64_t acc = 0;
            for (k = 0; k < K; ++k) {
                float wf, xf;
                uint32_t wu = (uint32_t)w_host[n * K + k] << 16, xu = (uint32_t)x_host[r * K + k] << 16;
                memcpy(&wf, &wu, 4);
                memcpy(&xf, &xu, 4);
                acc += (int64_t)wf * (int64_t)xf;
            }
            ref[r * N + n] = acc;
        }

    HIP(hipSetDevice(0));
    HIP(hipStreamCreate(&stream));
    HIP(hipMalloc(&w_dev, sizeof w_host));
    HIP(hipMalloc(&x_dev, sizeof x_host));
    HIP(hipMalloc(&out_dev, sizeof out_host));
    HIP(hipMemcpy(w_dev, w_host, sizeof w_host, hipMemcpyHostToDevice));
    HIP(hipMemcpy(x_dev, x_host, sizeof x_host, hipMemcpyHostToDevice));

    for (f32 = 0; f32 < 2; ++f32) {
        skinny_plan *plan = NULL;
        hipGraph_t graph;
        hipGraphExec_t exec;
        skinny_tactic t;
        skinny_status st = skinny_prepare(w_dev, N, K, f32 ? SKINNY_OUT_F32 : SKINNY_OUT_BF16, &plan);
        CHECK(st == SKINNY_OK && plan != NULL, "prepare (%s)", skinny_status_string(st));
        for (m = 1; m <= MAXM; ++m) {
            if (fill_sentinel(out_dev, f32, stream))
                return 1;
            st = skinny_run(plan, x_dev, out_dev, m, stream);
            CHECK(st == SKINNY_OK, "run M=%d (%s)", m, skinny_status_string(st));
            HIP(hipMemcpyAsync(out_host, out_dev, (size_t)MAXM * N * (f32 ? 4 : 2), hipMemcpyDeviceToHost, stream));
            HIP(hipStreamSynchronize(stream));
            if (check_out(out_host, f32, m, ref, f32 ? "run f32" : "run bf16"))
                return 1;
        }
        CHECK(skinny_run(plan, x_dev, out_dev, 65, stream) == SKINNY_ERR_UNSUPPORTED_M, "M=65");
        CHECK(skinny_supports(plan, 64) == 1 && skinny_supports(plan, 0) == 0, "supports");

        /* one run captured in a graph, replayed three times */
        if (fill_sentinel(out_dev, f32, stream))
            return 1;
        HIP(hipStreamBeginCapture(stream, hipStreamCaptureModeThreadLocal));
        st = skinny_run(plan, x_dev, out_dev, 37, stream);
        HIP(hipStreamEndCapture(stream, &graph));
        CHECK(st == SKINNY_OK, "run under capture (%s)", skinny_status_string(st));
        HIP(hipGraphInstantiate(&exec, graph, NULL, NULL, 0));
        for (i = 0; i < 3; ++i) {
            HIP(hipGraphLaunch(exec, stream));
            HIP(hipMemcpyAsync(out_host, out_dev, (size_t)MAXM * N * (f32 ? 4 : 2), hipMemcpyDeviceToHost, stream));
            HIP(hipStreamSynchronize(stream));
            if (check_out(out_host, f32, 37, ref, "graph replay"))
                return 1;
        }
        HIP(hipGraphExecDestroy(exec));
        HIP(hipGraphDestroy(graph));

        /* the allocation-free entry point with a K-split MFMAW tactic */
        t.path = SKINNY_PATH_MFMAW;
        t.mt = 32;
        t.rows = 64;
        t.waves = 4;
        t.unroll = 3;
        t.split = 2;
        CHECK(skinny_tactic_check(&t, N, K) == SKINNY_OK, "static tactic");
        for (i = 0; i < 2; ++i) {
            if (fill_sentinel(out_dev, f32, stream))
                return 1;
            st = skinny_run_static(w_dev, N, K, K, SKINNY_IN_BF16, f32 ? SKINNY_OUT_F32 : SKINNY_OUT_BF16, &t,
                                   x_dev, K, NULL, 0, out_dev, N, 32 - 7 * i, stream);
            CHECK(st == SKINNY_OK, "run_static (%s)", skinny_status_string(st));
            HIP(hipMemcpyAsync(out_host, out_dev, (size_t)MAXM * N * (f32 ? 4 : 2), hipMemcpyDeviceToHost, stream));
            HIP(hipStreamSynchronize(stream));
            if (check_out(out_host, f32, 32 - 7 * i, ref, "run_static"))
                return 1;
        }
        skinny_destroy(plan);
    }
    HIP(hipFree(w_dev));
    HIP(hipFree(x_dev));
    HIP(hipFree(out_dev));
    HIP(hipStreamDestroy(stream));
    printf("c run ok %ld\n", checks);
    return 0;
}
