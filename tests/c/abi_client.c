/*
 * A plain C client of libvwc: device memory from the HIP runtime, every
 * number through the C ABI only, checked against the fp64 oracle (test
 * infrastructure, linked here as a C library).
 *
 * Rows of bf16 logits (four segments, so the workspace and the merge launch
 * are used; an odd width and stride, so rows start off 16 bytes) go through
 * the forward with entropy, the backward into a bf16 gradient, and the same
 * rows as a row set; argument errors come back as status codes with a
 * message.  Exit status 0 means every
 * check held; the first failure is printed with its numbers.
 *
 * Inputs come from a fixed 64-bit LCG (Knuth's MMIX constants): logits
 * ~ U(-6, 6) rounded to bf16, targets uniform, grad_out ~ U(-1, 1) with every
 * fifth row 0.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "oracle.h"
#include "vwc.h"

#define N_ROWS 40
#define VOCAB 248321

static uint64_t lcg_state = 0x243F6A8885A308D3ull;

static double lcg_uniform(void) { /* [0, 1) */
    lcg_state = lcg_state * 6364136223846793005ull + 1442695040888963407ull;
    return (double)(lcg_state >> 11) * (1.0 / 9007199254740992.0);
}

static uint16_t to_bf16(float f) { /* round to nearest even; inputs are finite */
    uint32_t u;
    memcpy(&u, &f, 4);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

static int bf16_steps(uint16_t a, uint16_t b) { /* distance in bf16 steps, +0 == -0 */
    int32_t ia = (a & 0x8000u) ? -(int32_t)(a & 0x7fffu) : (int32_t)a;
    int32_t ib = (b & 0x8000u) ? -(int32_t)(b & 0x7fffu) : (int32_t)b;
    return abs(ia - ib);
}

#define HIP_OK(call)                                                               \
    do {                                                                           \
        hipError_t e_ = (call);                                                    \
        if (e_ != hipSuccess) {                                                    \
            fprintf(stderr, "%s: %s\n", #call, hipGetErrorString(e_));              \
            return 1;                                                              \
        }                                                                          \
    } while (0)

#define VWC_OK_(call)                                                              \
    do {                                                                           \
        vwc_status s_ = (call);                                                    \
        if (s_ != VWC_OK) {                                                        \
            fprintf(stderr, "%s: %s (%s)\n", #call, vwc_status_string(s_),         \
                    vwc_last_error());                                             \
            return 1;                                                              \
        }                                                                          \
    } while (0)

int main(void) {
    const int64_t n = N_ROWS, v = VOCAB, ld = VOCAB;
    const size_t nx = (size_t)(n * ld);
    uint16_t *x = malloc(nx * sizeof *x), *grad = malloc(nx * sizeof *grad);
    int32_t *t = malloc(n * sizeof *t);
    float *g = malloc(n * sizeof *g), lp[N_ROWS], lse[N_ROWS], ent[N_ROWS];
    double *gref = malloc((size_t)(n * v) * sizeof *gref);
    uint16_t *gref16 = malloc((size_t)(n * v) * sizeof *gref16);
    double rlp[N_ROWS], rlse[N_ROWS], rent[N_ROWS];
    if (!x || !grad || !t || !g || !gref || !gref16) return 1;
    for (size_t i = 0; i < nx; ++i) x[i] = to_bf16((float)(lcg_uniform() * 12.0 - 6.0));
    for (int64_t r = 0; r < n; ++r) {
        t[r] = (int32_t)(lcg_uniform() * (double)v);
        g[r] = r % 5 == 0 ? 0.0f : (float)(lcg_uniform() * 2.0 - 1.0);
    }
    printf("abi version %d, %lld x %lld bf16 rows\n", vwc_abi_version(), (long long)n,
           (long long)v);

    /* device buffers */
    void *dx, *dgrad, *dws = NULL;
    int32_t *dt, *didx;
    float *dg, *dlp, *dlse, *dent;
    const size_t ws = vwc_workspace_bytes(n, v, VWC_BF16);
    HIP_OK(hipMalloc(&dx, nx * 2));
    HIP_OK(hipMalloc(&dgrad, nx * 2));
    HIP_OK(hipMalloc((void **)&dt, n * 4));
    HIP_OK(hipMalloc((void **)&didx, n * 4));
    HIP_OK(hipMalloc((void **)&dg, n * 4));
    HIP_OK(hipMalloc((void **)&dlp, n * 4));
    HIP_OK(hipMalloc((void **)&dlse, n * 4));
    HIP_OK(hipMalloc((void **)&dent, n * 4));
    if (ws) HIP_OK(hipMalloc(&dws, ws));
    HIP_OK(hipMemcpy(dx, x, nx * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dt, t, n * 4, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dg, g, n * 4, hipMemcpyHostToDevice));
    hipStream_t s;
    HIP_OK(hipStreamCreate(&s));

    /* forward with entropy, then the backward, on one stream */
    VWC_OK_(vwc_selected_logprob_fwd(dx, VWC_BF16, n, v, ld, dt, 1.0f, dlp, dlse, dent, dws, ws,
                                     s));
    VWC_OK_(vwc_selected_logprob_bwd(dx, VWC_BF16, n, v, ld, dt, 1.0f, dlse, dg, dgrad, VWC_BF16,
                                     ld, s));
    HIP_OK(hipStreamSynchronize(s));
    HIP_OK(hipMemcpy(lp, dlp, n * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(lse, dlse, n * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(ent, dent, n * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(grad, dgrad, nx * 2, hipMemcpyDeviceToHost));

    /* the oracle: dtype 0 = bf16 bits */
    if (oracle_forward(x, 0, n, v, ld, t, NULL, n, 1.0, n, rlp, rlse, rent) != 0) return 1;
    if (oracle_backward(x, 0, n, v, ld, t, NULL, n, 1.0, g, gref) != 0) return 1;
    oracle_bf16_rne_array(gref, gref16, n * v);
    double worst = 0.0;
    for (int64_t r = 0; r < n; ++r) {
        const double e = fmax(fabs(lp[r] - rlp[r]), fmax(fabs(lse[r] - rlse[r]),
                                                         fabs(ent[r] - rent[r])));
        worst = fmax(worst, e);
    }
    if (!(worst <= 5e-5)) {
        fprintf(stderr, "forward: max error %.3g above 5e-5\n", worst);
        return 1;
    }
    int steps = 0;
    for (int64_t r = 0; r < n; ++r)
        for (int64_t j = 0; j < v; ++j) {
            const int d = bf16_steps(grad[r * ld + j], gref16[r * v + j]);
            if (d > steps) steps = d;
        }
    if (steps > 1) {
        fprintf(stderr, "backward: %d bf16 steps from the rounded oracle\n", steps);
        return 1;
    }
    printf("forward max error %.3g, backward within %d bf16 step(s)\n", worst, steps);

    /* a row set: rows 3, 0, 39 -- bitwise the dense rows' results */
    const int32_t idx[3] = {3, 0, 39};
    float clp[3], clse[3];
    HIP_OK(hipMemcpy(didx, idx, sizeof idx, hipMemcpyHostToDevice));
    VWC_OK_(vwc_selected_logprob_fwd_rows(dx, VWC_BF16, n, v, ld, dt, didx, 3, 1.0f, dlp, dlse,
                                          NULL, dws, ws, s));
    HIP_OK(hipStreamSynchronize(s));
    HIP_OK(hipMemcpy(clp, dlp, sizeof clp, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(clse, dlse, sizeof clse, hipMemcpyDeviceToHost));
    for (int i = 0; i < 3; ++i)
        if (memcmp(&clp[i], &lp[idx[i]], 4) || memcmp(&clse[i], &lse[idx[i]], 4)) {
            fprintf(stderr, "row set: output %d differs from dense row %d\n", i, idx[i]);
            return 1;
        }

    /* argument errors are status codes, with a message, and launch nothing */
    vwc_status st = vwc_selected_logprob_fwd(dx, VWC_BF16, n, v, v - 1, dt, 1.0f, dlp, dlse,
                                             NULL, dws, ws, s);
    if (st != VWC_ERR_INVALID_ARG || strstr(vwc_last_error(), "ld") == NULL) {
        fprintf(stderr, "ld < vocab: status %d, message '%s'\n", (int)st, vwc_last_error());
        return 1;
    }
    st = vwc_selected_logprob_fwd(dx, VWC_BF16, n, v, ld, dt, -1.0f, dlp, dlse, NULL, dws, ws, s);
    if (st != VWC_ERR_INVALID_ARG) {
        fprintf(stderr, "negative temperature: status %d\n", (int)st);
        return 1;
    }
    printf("row set bitwise equal to dense rows; argument errors reported\n");

    HIP_OK(hipStreamDestroy(s));
    hipFree(dx);
    hipFree(dgrad);
    hipFree(dt);
    hipFree(didx);
    hipFree(dg);
    hipFree(dlp);
    hipFree(dlse);
    hipFree(dent);
    if (dws) hipFree(dws);
    free(x);
    free(grad);
    free(t);
    free(g);
    free(gref);
    free(gref16);
    printf("ok\n");
    return 0;
}
