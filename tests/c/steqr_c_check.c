/*
 * A C caller of the library's C ABI (include/steqr.h), without Python: it
 * allocates device memory with the HIP runtime, calls steqr_batched and
 * steqr_batched_ex, and checks the results on the host against closed
 * forms.
 *
 *  1. Discrete Laplacians T = tridiag(-1; 2; -1) of order n (double,
 *     eigenvectors): lambda_k = 2 - 2 cos(k pi / (n + 1)), Q orthogonal,
 *     T Q = Q Lambda, info 0; at n = 12 (chunked kernels), 37 (producer and
 *     consumer wavefronts) and 300 (rows of Q split over workgroups).
 *  2. Float random-sign couplings at n = 16: the 9-argument steqr_batched
 *     writes bit for bit what steqr_batched_ex with default params writes.
 *  3. Argument errors: -1 for a NULL d, -5 for n > STEQR_MAX_N, 0 for an
 *     empty batch.
 * Prints one line per check and "all ok"; returns 0 on success, 1 on a
 * failed check, 2 on a HIP error.
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "steqr.h"

#define HIP(call)                                                              \
    do {                                                                       \
        hipError_t err_ = (call);                                              \
        if (err_ != hipSuccess) {                                              \
            fprintf(stderr, "HIP error %d at %s:%d\n", (int)err_, __FILE__, __LINE__); \
            exit(2);                                                           \
        }                                                                      \
    } while (0)

static int laplacian(int n, int batch)
{
    const double pi = 3.14159265358979323846;
    size_t nd = (size_t)n * batch, ne = (size_t)(n - 1) * batch, nq = (size_t)n * n * batch;
    double *d = malloc(nd * sizeof(double)), *e = malloc(ne * sizeof(double));
    double *lam = malloc(nd * sizeof(double)), *q = malloc(nq * sizeof(double));
    int *info = malloc(batch * sizeof(int));
    for (size_t i = 0; i < nd; ++i) d[i] = 2.0;
    for (size_t i = 0; i < ne; ++i) e[i] = -1.0;
    void *dd, *de, *dl, *dq, *di;
    HIP(hipMalloc(&dd, nd * sizeof(double)));
    HIP(hipMalloc(&de, ne * sizeof(double)));
    HIP(hipMalloc(&dl, nd * sizeof(double)));
    HIP(hipMalloc(&dq, nq * sizeof(double)));
    HIP(hipMalloc(&di, batch * sizeof(int)));
    HIP(hipMemcpy(dd, d, nd * sizeof(double), hipMemcpyHostToDevice));
    HIP(hipMemcpy(de, e, ne * sizeof(double), hipMemcpyHostToDevice));
    int rc = steqr_batched_ex(dd, de, dl, dq, n, batch, STEQR_V, STEQR_F64, 0, (int *)di, NULL);
    if (rc != 0) {
        printf("laplacian n=%d: steqr_batched_ex returned %d\n", n, rc);
        return 1;
    }
    HIP(hipDeviceSynchronize());
    HIP(hipMemcpy(lam, dl, nd * sizeof(double), hipMemcpyDeviceToHost));
    HIP(hipMemcpy(q, dq, nq * sizeof(double), hipMemcpyDeviceToHost));
    HIP(hipMemcpy(info, di, batch * sizeof(int), hipMemcpyDeviceToHost));
    const double tol = 16.0 * n * 2.220446049250313e-16 * 4.0; /* 16 n eps ||T||_1 */
    double eig = 0, orth = 0, res = 0;
    int bad_info = 0;
    for (int b = 0; b < batch; ++b) {
        bad_info |= info[b] != 0;
        const double *l = lam + (size_t)b * n, *Q = q + (size_t)b * n * n;
        for (int k = 0; k < n; ++k) {
            double exact = 2.0 - 2.0 * cos((k + 1) * pi / (n + 1));
            double err = fabs(l[k] - exact);
            if (err > eig) eig = err;
        }
        if (b % 7 != 0) continue; /* orthogonality and residual on every 7th matrix */
        for (int i = 0; i < n; ++i)
            for (int j = 0; j < n; ++j) {
                double s = 0, r = 0;
                for (int k = 0; k < n; ++k) s += Q[k * n + i] * Q[k * n + j];
                s -= (i == j);
                if (fabs(s) > orth) orth = fabs(s);
                /* (T Q - Q Lambda)_{ij} */
                r = 2.0 * Q[i * n + j] - (i > 0 ? Q[(i - 1) * n + j] : 0.0)
                    - (i + 1 < n ? Q[(i + 1) * n + j] : 0.0) - Q[i * n + j] * l[j];
                if (fabs(r) > res) res = fabs(r);
            }
    }
    int ok = !bad_info && eig <= tol && orth <= tol && res <= tol;
    printf("laplacian n=%d batch=%d: eig %.2e orth %.2e residual %.2e (tol %.2e) info %s: %s\n",
           n, batch, eig, orth, res, tol, bad_info ? "bad" : "0", ok ? "ok" : "FAILED");
    hipFree(dd); hipFree(de); hipFree(dl); hipFree(dq); hipFree(di);
    free(d); free(e); free(lam); free(q); free(info);
    return ok ? 0 : 1;
}

static int plain_equals_ex(void)
{
    const int n = 16, batch = 1000;
    size_t nd = (size_t)n * batch, ne = (size_t)(n - 1) * batch, nq = (size_t)n * n * batch;
    float *d = malloc(nd * sizeof(float)), *e = malloc(ne * sizeof(float));
    unsigned s = 12345u;
    for (size_t i = 0; i < nd; ++i) { s = s * 1664525u + 1013904223u; d[i] = (float)((s >> 8) & 0xffff) / 65536.0f - 0.5f; }
    for (size_t i = 0; i < ne; ++i) { s = s * 1664525u + 1013904223u; e[i] = (s & 0x100) ? 1.0f : -1.0f; }
    void *dd, *de, *l1, *l2, *q1, *q2;
    HIP(hipMalloc(&dd, nd * sizeof(float)));
    HIP(hipMalloc(&de, ne * sizeof(float)));
    HIP(hipMalloc(&l1, nd * sizeof(float)));
    HIP(hipMalloc(&l2, nd * sizeof(float)));
    HIP(hipMalloc(&q1, nq * sizeof(float)));
    HIP(hipMalloc(&q2, nq * sizeof(float)));
    HIP(hipMemcpy(dd, d, nd * sizeof(float), hipMemcpyHostToDevice));
    HIP(hipMemcpy(de, e, ne * sizeof(float), hipMemcpyHostToDevice));
    int rc1 = steqr_batched(dd, de, l1, q1, n, batch, STEQR_V, STEQR_F32, 0);
    int rc2 = steqr_batched_ex(dd, de, l2, q2, n, batch, STEQR_V, STEQR_F32, 0, NULL, NULL);
    HIP(hipDeviceSynchronize());
    float *h1 = malloc(nq * sizeof(float)), *h2 = malloc(nq * sizeof(float));
    HIP(hipMemcpy(h1, l1, nd * sizeof(float), hipMemcpyDeviceToHost));
    HIP(hipMemcpy(h2, l2, nd * sizeof(float), hipMemcpyDeviceToHost));
    int same = memcmp(h1, h2, nd * sizeof(float)) == 0;
    HIP(hipMemcpy(h1, q1, nq * sizeof(float), hipMemcpyDeviceToHost));
    HIP(hipMemcpy(h2, q2, nq * sizeof(float), hipMemcpyDeviceToHost));
    same = same && memcmp(h1, h2, nq * sizeof(float)) == 0;
    int ok = rc1 == 0 && rc2 == 0 && same;
    printf("steqr_batched vs steqr_batched_ex (float, n=16, 1000 matrices): rc %d %d, %s: %s\n",
           rc1, rc2, same ? "bit-identical" : "different", ok ? "ok" : "FAILED");
    hipFree(dd); hipFree(de); hipFree(l1); hipFree(l2); hipFree(q1); hipFree(q2);
    free(d); free(e); free(h1); free(h2);
    return ok ? 0 : 1;
}

static int errors(void)
{
    void *p;
    HIP(hipMalloc(&p, 4096));
    int a = steqr_batched(NULL, p, p, p, 8, 4, STEQR_V, STEQR_F32, 0);
    int b = steqr_batched(p, p, p, p, STEQR_MAX_N + 1, 4, STEQR_V, STEQR_F32, 0);
    int c = steqr_batched(p, p, p, p, 8, 0, STEQR_V, STEQR_F32, 0);
    hipFree(p);
    int ok = a == -1 && b == -5 && c == 0;
    printf("argument errors: NULL d %d, n > STEQR_MAX_N %d, empty batch %d: %s\n", a, b, c,
           ok ? "ok" : "FAILED");
    return ok ? 0 : 1;
}

int main(void)
{
    printf("%s\n", steqr_version());
    int bad = 0;
    bad |= laplacian(12, 333);
    bad |= laplacian(37, 70);
    bad |= laplacian(300, 3);
    bad |= plain_equals_ex();
    bad |= errors();
    printf(bad ? "FAILED\n" : "all ok\n");
    return bad ? 1 : 0;
}
