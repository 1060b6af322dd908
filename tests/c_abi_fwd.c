/* c_abi_fwd.c -- the forward through the C ABI from plain C, with the HIP runtime
 * and nothing else (no Python, no torch): inputs in device memory from hipMalloc,
 * bsattn_fwd on a stream of its own, the results against the fp64 oracle
 * (liboracle.so, test infrastructure).  Checked per dtype:
 *   bf16: max |out error| <= 1e-2, mean <= 1e-3, max |lse error| <= 1e-3;
 *   fp32: max |out error| <= 1e-4, max |lse error| <= 1e-5;
 * a query block with no active key block gets out = 0 and lse = -inf exactly, and
 * a NULL argument is refused with BSATTN_ERR_NULL before any device work.
 * Exit status 0 when every check holds.  Built by __graft_entry__.build(). */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "bsattn.h"

/* the oracle's forward (oracle/oracle.c): dtype 0 fp32, 1 bf16 */
int oracle_fwd(const void* q, const void* k, const void* v, int dtype, const uint8_t* mask, int64_t B,
               int64_t H, int64_t S, int64_t D, int64_t block_q, int64_t block_k, float scale, double* out,
               double* lse, int nthreads);

#define B 1
#define H 2
#define S 512
#define BQ 128
#define BK 128
#define NQ (S / BQ)
#define NK (S / BK)

static uint32_t rng = 12345u;
static float uniform_pm2(void) { /* xorshift32, uniform in [-2, 2) */
    rng ^= rng << 13;
    rng ^= rng >> 17;
    rng ^= rng << 5;
    return (float)(rng >> 8) * (4.0f / 16777216.0f) - 2.0f;
}

static uint16_t to_bf16(float x) { /* round to nearest even (finite x) */
    uint32_t u;
    memcpy(&u, &x, 4);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

static float from_bf16(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float x;
    memcpy(&x, &u, 4);
    return x;
}

#define HIP_OK(call)                                                             \
    do {                                                                         \
        hipError_t e_ = (call);                                                  \
        if (e_ != hipSuccess) {                                                  \
            fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));    \
            return 1;                                                            \
        }                                                                        \
    } while (0)

static int run(int D, int bf16) {
    const size_t n = (size_t)B * H * S * D, esz = bf16 ? 2 : 4, rows = (size_t)B * H * S;
    const float scale = 1.0f / sqrtf((float)D);
    void *hq = malloc(n * esz), *hk = malloc(n * esz), *hv = malloc(n * esz), *hout = malloc(n * esz);
    float* hlse = malloc(rows * 4);
    double *rout = malloc(n * 8), *rlse = malloc(rows * 8);
    uint8_t mask[B * H * NQ * NK];
    void* arrs[3] = {hq, hk, hv};
    for (int a = 0; a < 3; ++a)
        for (size_t i = 0; i < n; ++i) {
            const float x = uniform_pm2();
            if (bf16)
                ((uint16_t*)arrs[a])[i] = to_bf16(x);
            else
                ((float*)arrs[a])[i] = x;
        }
    /* head 0: causal blocks; head 1: query block 1 empty, the others every other key block */
    for (int h = 0; h < H; ++h)
        for (int i = 0; i < NQ; ++i)
            for (int j = 0; j < NK; ++j)
                mask[(h * NQ + i) * NK + j] = h == 0 ? (j <= i) : (i != 1 && (i + j) % 2 == 0);

    void *dq, *dk, *dv, *dout, *ws;
    float* dlse;
    uint8_t* dmask;
    size_t wsb = 0;
    if (bsattn_workspace_size(B, H, S, BQ, BK, &wsb) != BSATTN_OK) return 1;
    HIP_OK(hipMalloc(&dq, n * esz));
    HIP_OK(hipMalloc(&dk, n * esz));
    HIP_OK(hipMalloc(&dv, n * esz));
    HIP_OK(hipMalloc(&dout, n * esz));
    HIP_OK(hipMalloc((void**)&dlse, rows * 4));
    HIP_OK(hipMalloc((void**)&dmask, sizeof mask));
    HIP_OK(hipMalloc(&ws, wsb));
    HIP_OK(hipMemcpy(dq, hq, n * esz, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dk, hk, n * esz, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dv, hv, n * esz, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dmask, mask, sizeof mask, hipMemcpyHostToDevice));
    hipStream_t st;
    HIP_OK(hipStreamCreate(&st));
    const int dt = bf16 ? BSATTN_BF16 : BSATTN_F32;

    int rc = bsattn_fwd(NULL, dk, dv, dmask, dout, dlse, B, H, S, D, BQ, BK, scale, dt, ws, wsb, st);
    if (rc != BSATTN_ERR_NULL) {
        fprintf(stderr, "NULL q: status %d (%s), expected BSATTN_ERR_NULL\n", rc, bsattn_status_string(rc));
        return 1;
    }
    rc = bsattn_fwd(dq, dk, dv, dmask, dout, dlse, B, H, S, D, BQ, BK, scale, dt, ws, wsb, st);
    if (rc != BSATTN_OK) {
        fprintf(stderr, "bsattn_fwd: %s (HIP %d)\n", bsattn_status_string(rc), bsattn_last_hip_error());
        return 1;
    }
    HIP_OK(hipStreamSynchronize(st));
    HIP_OK(hipMemcpy(hout, dout, n * esz, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(hlse, dlse, rows * 4, hipMemcpyDeviceToHost));

    if (oracle_fwd(hq, hk, hv, bf16 ? 1 : 0, mask, B, H, S, D, BQ, BK, scale, rout, rlse, 0) != 0) return 1;
    double emax = 0, esum = 0, lmax = 0;
    int bad = 0;
    for (size_t r = 0; r < rows; ++r) {
        const int empty = isinf(rlse[r]) && rlse[r] < 0;
        if (empty) {
            if (!(isinf(hlse[r]) && hlse[r] < 0)) bad = 1;
        } else {
            const double e = fabs(hlse[r] - rlse[r]);
            if (!(e <= lmax)) lmax = e; /* (a NaN makes lmax NaN and fails below) */
        }
        for (int d = 0; d < D; ++d) {
            const size_t i = r * D + d;
            const double g = bf16 ? from_bf16(((uint16_t*)hout)[i]) : ((float*)hout)[i];
            if (empty && g != 0.0) bad = 1;
            const double e = fabs(g - rout[i]);
            if (!(e <= emax)) emax = e; /* (a NaN makes emax NaN and fails below) */
            esum += e;
        }
    }
    const double emean = esum / (double)n;
    const double tmax = bf16 ? 1e-2 : 1e-4, tmean = bf16 ? 1e-3 : 1e-4, tlse = bf16 ? 1e-3 : 1e-5;
    const int ok = !bad && emax <= tmax && emean <= tmean && lmax <= tlse;
    printf("C ABI %s D=%d: out max err %.3g mean %.3g, lse max err %.3g, empty rows %s: %s\n",
           bf16 ? "bf16" : "fp32", D, emax, emean, lmax, bad ? "WRONG" : "ok", ok ? "PASS" : "FAIL");
    HIP_OK(hipStreamDestroy(st));
    HIP_OK(hipFree(dq));
    HIP_OK(hipFree(dk));
    HIP_OK(hipFree(dv));
    HIP_OK(hipFree(dout));
    HIP_OK(hipFree(dlse));
    HIP_OK(hipFree(dmask));
    HIP_OK(hipFree(ws));
    free(hq);
    free(hk);
    free(hv);
    free(hout);
    free(hlse);
    free(rout);
    free(rlse);
    return ok ? 0 : 1;
}

int main(void) {
    printf("libbsattn version %d\n", bsattn_version());
    int fails = 0;
    fails += run(128, 1);
    fails += run(64, 1);
    fails += run(64, 0);
    return fails ? 1 : 0;
}
