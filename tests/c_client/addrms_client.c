/*
 * A plain C client of libaddrms.so: the library used with nothing but the
 * HIP runtime (no PyTorch), as a C caller would.  GPU test infrastructure:
 * tests/test_gpu_c_client.py writes the inputs, runs this program and checks
 * what it writes against the oracle.
 *
 *   addrms_client IN OUT
 *   addrms_client --plan M N
 *
 * IN (little-endian): int64 M, int64 N, then bf16 arrays x [M][N], r [M][N],
 * w [N], dy [M][N], h [M][N] and float32 rstd [M] (h and rstd: the saved
 * forward values the backward takes).  OUT: bf16 y [M][N] and residual_out
 * [M][N], float32 rstd [M], bf16 dx [M][N], float32 dw [N], and bf16 y2
 * [M][N], the forward's y again from the second replay of a captured graph.
 *
 * Steps, on a stream of its own (hipStreamCreate):
 *   1. add_rmsnorm_fwd into device buffers from hipMalloc;
 *   2. rmsnorm_bwd with a workspace of rmsnorm_bwd_workspace_bytes(M, N);
 *   3. the forward captured into a HIP graph (hipStreamBeginCapture), the
 *      graph replayed twice, with y2 overwritten by a byte pattern before
 *      each replay (outside the graph), so that y2 comes from the replay;
 *   4. argument errors: a negative eps and a NULL x must return
 *      ADDRMS_ERR_EPS and ADDRMS_ERR_NULL, with a status string, and launch
 *      nothing.
 * Exit status 0 and "ok" on stdout when every step succeeded; otherwise a
 * message naming the step and a non-zero status.
 *
 * With --plan, no file and no HIP call: the launch plans (addrms_plan) of
 * the bf16 add_rmsnorm_fwd and rmsnorm_bwd of M x N on a 256-CU device, one
 * line each, as name key=value ...
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "addrms.h"

static int fail(const char *step, const char *what)
{
    fprintf(stderr, "addrms_client: %s: %s\n", step, what);
    return 1;
}

#define HIP_OK(step, call)                                                       \
    do {                                                                         \
        hipError_t e_ = (call);                                                  \
        if (e_ != hipSuccess)                                                    \
            return fail(step, hipGetErrorString(e_));                            \
    } while (0)

#define LIB_OK(step, call)                                                       \
    do {                                                                         \
        int s_ = (call);                                                         \
        if (s_ != ADDRMS_OK)                                                     \
            return fail(step, addrms_status_str(s_));                            \
    } while (0)

static int read_all(FILE *f, void *p, size_t n) { return fread(p, 1, n, f) == n; }

static int print_plans(const char *ms, const char *ns)
{
    char *end;
    const long long M = strtoll(ms, &end, 10);
    if (end == ms || *end)
        return fail("plan", "bad M");
    const long long N = strtoll(ns, &end, 10);
    if (end == ns || *end)
        return fail("plan", "bad N");
    static const struct {
        const char *name;
        int op, fused;
    } calls[] = {{"add_rmsnorm_fwd", ADDRMS_PLAN_FWD, 1}, {"rmsnorm_bwd", ADDRMS_PLAN_BWD, 0}};
    for (int i = 0; i < 2; ++i) {
        addrms_plan_t p;
        LIB_OK("plan", addrms_plan(calls[i].op, ADDRMS_PLAN_RMS, calls[i].fused, 0, 0, M, N,
                                   ADDRMS_BF16, ADDRMS_BF16, 256, &p));
        printf("%s vector=%d waves_per_row=%d vectors_per_lane=%d prefetch=%d wide=%d "
               "blocks_per_cu=%d\n",
               calls[i].name, p.vector, p.waves_per_row, p.vectors_per_lane, p.prefetch, p.wide,
               p.blocks_per_cu);
    }
    return 0;
}

int main(int argc, char **argv)
{
    if (argc == 4 && strcmp(argv[1], "--plan") == 0)
        return print_plans(argv[2], argv[3]);
    if (argc != 3)
        return fail("arguments", "usage: addrms_client IN OUT");
    FILE *in = fopen(argv[1], "rb");
    if (!in)
        return fail("input", "cannot open");
    int64_t M = 0, N = 0;
    if (!read_all(in, &M, 8) || !read_all(in, &N, 8) || M <= 0 || N <= 0 || M > (1 << 20) ||
        N > (1 << 20))
        return fail("input", "bad header");
    const size_t mat = (size_t)M * (size_t)N * 2, vec = (size_t)N * 2, rows = (size_t)M * 4;
    unsigned char *hx = malloc(mat), *hr = malloc(mat), *hw = malloc(vec), *hdy = malloc(mat),
                  *hh = malloc(mat), *hrs = malloc(rows);
    if (!hx || !hr || !hw || !hdy || !hh || !hrs)
        return fail("input", "out of host memory");
    if (!read_all(in, hx, mat) || !read_all(in, hr, mat) || !read_all(in, hw, vec) ||
        !read_all(in, hdy, mat) || !read_all(in, hh, mat) || !read_all(in, hrs, rows))
        return fail("input", "short file");
    fclose(in);

    HIP_OK("device", hipSetDevice(0));
    hipStream_t s;
    HIP_OK("stream", hipStreamCreate(&s));
    void *x, *r, *w, *y, *res, *dy, *h, *dx, *y2, *res2, *ws;
    float *rstd, *rstd_in, *dw;
    HIP_OK("alloc", hipMalloc(&x, mat));
    HIP_OK("alloc", hipMalloc(&r, mat));
    HIP_OK("alloc", hipMalloc(&w, vec));
    HIP_OK("alloc", hipMalloc(&y, mat));
    HIP_OK("alloc", hipMalloc(&res, mat));
    HIP_OK("alloc", hipMalloc((void **)&rstd, rows));
    HIP_OK("alloc", hipMalloc(&dy, mat));
    HIP_OK("alloc", hipMalloc(&h, mat));
    HIP_OK("alloc", hipMalloc((void **)&rstd_in, rows));
    HIP_OK("alloc", hipMalloc(&dx, mat));
    HIP_OK("alloc", hipMalloc((void **)&dw, (size_t)N * 4));
    HIP_OK("alloc", hipMalloc(&y2, mat));
    HIP_OK("alloc", hipMalloc(&res2, mat));
    const size_t ws_bytes = rmsnorm_bwd_workspace_bytes(M, N);
    HIP_OK("alloc", hipMalloc(&ws, ws_bytes > 0 ? ws_bytes : 1));
    HIP_OK("upload", hipMemcpy(x, hx, mat, hipMemcpyHostToDevice));
    HIP_OK("upload", hipMemcpy(r, hr, mat, hipMemcpyHostToDevice));
    HIP_OK("upload", hipMemcpy(w, hw, vec, hipMemcpyHostToDevice));
    HIP_OK("upload", hipMemcpy(dy, hdy, mat, hipMemcpyHostToDevice));
    HIP_OK("upload", hipMemcpy(h, hh, mat, hipMemcpyHostToDevice));
    HIP_OK("upload", hipMemcpy(rstd_in, hrs, rows, hipMemcpyHostToDevice));

    /* 1. forward, 2. backward */
    LIB_OK("add_rmsnorm_fwd", add_rmsnorm_fwd(x, r, w, y, res, rstd, M, N, 1e-6f, ADDRMS_BF16,
                                              ADDRMS_BF16, s));
    LIB_OK("rmsnorm_bwd", rmsnorm_bwd(dy, h, w, rstd_in, dx, dw, ws, ws_bytes, M, N, ADDRMS_BF16,
                                      ADDRMS_BF16, s));

    /* 3. the forward in a captured graph, replayed twice */
    hipGraph_t g;
    hipGraphExec_t ge;
    HIP_OK("capture", hipStreamBeginCapture(s, hipStreamCaptureModeGlobal));
    int st = add_rmsnorm_fwd(x, r, w, y2, res2, NULL, M, N, 1e-6f, ADDRMS_BF16, ADDRMS_BF16, s);
    HIP_OK("capture", hipStreamEndCapture(s, &g));
    if (st != ADDRMS_OK)
        return fail("captured add_rmsnorm_fwd", addrms_status_str(st));
    HIP_OK("instantiate", hipGraphInstantiate(&ge, g, NULL, NULL, 0));
    for (int rep = 0; rep < 2; ++rep) {
        HIP_OK("clear", hipMemsetAsync(y2, 0xA5, mat, s));
        HIP_OK("replay", hipGraphLaunch(ge, s));
    }

    /* 4. argument errors */
    if (add_rmsnorm_fwd(x, r, w, y, res, rstd, M, N, -1.0f, ADDRMS_BF16, ADDRMS_BF16, s) !=
        ADDRMS_ERR_EPS)
        return fail("negative eps", "not rejected with ADDRMS_ERR_EPS");
    if (add_rmsnorm_fwd(NULL, r, w, y, res, rstd, M, N, 1e-6f, ADDRMS_BF16, ADDRMS_BF16, s) !=
        ADDRMS_ERR_NULL)
        return fail("NULL x", "not rejected with ADDRMS_ERR_NULL");
    const char *msg = addrms_status_str(ADDRMS_ERR_EPS);
    if (!msg || !*msg)
        return fail("status string", "empty");

    HIP_OK("synchronise", hipStreamSynchronize(s));
    FILE *out = fopen(argv[2], "wb");
    if (!out)
        return fail("output", "cannot open");
    const struct { const void *p; size_t n; } outs[] = {
        {y, mat}, {res, mat}, {rstd, rows}, {dx, mat}, {dw, (size_t)N * 4}, {y2, mat}};
    size_t most = 0; /* the largest output (dw, 4 N bytes, exceeds 2 M N when M = 1) */
    for (size_t k = 0; k < sizeof(outs) / sizeof(outs[0]); ++k)
        most = outs[k].n > most ? outs[k].n : most;
    unsigned char *buf = malloc(most);
    if (!buf)
        return fail("output", "out of host memory");
    for (size_t k = 0; k < sizeof(outs) / sizeof(outs[0]); ++k) {
        HIP_OK("download", hipMemcpy(buf, outs[k].p, outs[k].n, hipMemcpyDeviceToHost));
        if (fwrite(buf, 1, outs[k].n, out) != outs[k].n)
            return fail("output", "short write");
    }
    fclose(out);
    HIP_OK("graph", hipGraphExecDestroy(ge));
    HIP_OK("graph", hipGraphDestroy(g));
    HIP_OK("stream", hipStreamDestroy(s));
    void *bufs[] = {x, r, w, y, res, rstd, dy, h, rstd_in, dx, dw, y2, res2, ws};
    for (size_t k = 0; k < sizeof(bufs) / sizeof(bufs[0]); ++k)
        HIP_OK("free", hipFree(bufs[k]));
    free(buf);
    free(hx);
    free(hr);
    free(hw);
    free(hdy);
    free(hh);
    free(hrs);
    printf("ok\n");
    return 0;
}
