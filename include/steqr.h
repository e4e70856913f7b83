/*
 * steqr.h -- C ABI of the MI355X (gfx950) batched symmetric tridiagonal
 * eigensolver.
 *
 * The operation (BatchLAS steqr algorithm page, problem statement at the top
 * of the page): for each matrix b of a batch, the symmetric tridiagonal
 *     T_b = tridiag(e_1..e_{n-1}; d_1..d_n; e_1..e_{n-1})
 * held as the vector d of its n diagonal entries and the vector e of
 * its n-1 couplings (band storage, same page), compute the eigenvalues Lambda and, on request, an orthogonal Q
 * with T_b = Q Lambda Q^T. The method is the implicit shifted QR/QL
 * iteration of that page: relative deflation, block scaling, a shift from
 * the end 2x2 block, a Givens bulge chase, analytic 2x2 blocks and a final
 * ascending sort that permutes Q's columns the same way.
 *
 * Memory layout (all arrays packed, no strides):
 *   d      [batch][n]       element type T, read only
 *   e      [batch][n-1]     element type T, read only (absent when n == 1)
 *   lambda [batch][n]       T, written: eigenvalues, ascending per matrix
 *   Q      [batch][n][n]    T, written: row-major per matrix, Q[b][i][j] is
 *                           Q_ij, so eigenvector k is column k (the column
 *                           for lambda[b][k])
 * T is float when dtype == STEQR_F32 and double when dtype == STEQR_F64.
 *
 * Ownership: every pointer is DEVICE memory owned by the caller (for
 * example torch tensors on the HIP device). The library keeps no pointer,
 * allocates nothing and holds no state between calls; calls are
 * thread-safe. d and e are never modified; Q is written only, except with
 * back-transformation (steqr_params.back_transform), where it is read on
 * entry and overwritten in place.
 *
 * Asynchrony: the call only enqueues work on `stream` (0 = the null
 * stream); results are valid once that stream is synchronised.
 *
 * Errors: 0 on success. A negative value -k names the first invalid
 * argument in the order of steqr_batched's parameter list (LAPACK style;
 * the array pointers are checked first, then n, batch, jobz, dtype and
 * finally the params of steqr_batched_ex):
 *   -1 d == NULL (n > 0, batch > 0)     -2 e == NULL (n > 1, batch > 0)
 *   -3 lambda == NULL                   -4 Q == NULL with jobz == STEQR_V
 *   -5 n < 0 or n > STEQR_MAX_N         -6 batch < 0
 *   -7 jobz not STEQR_N / STEQR_V       -8 dtype not STEQR_F32 / STEQR_F64
 *   -10 (steqr_batched_ex only) a params field out of range
 * A positive value is a hipError_t returned by the kernel launch (an error
 * pending from an earlier HIP call is cleared before the launch, so the
 * value is this launch's). n == 0 or batch == 0 returns 0 at once without
 * touching the GPU.
 */
#ifndef STEQR_H
#define STEQR_H

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define STEQR_MAX_N 512

enum { STEQR_N = 0, STEQR_V = 1 };     /* jobz: values only / values+vectors */
enum { STEQR_F32 = 0, STEQR_F64 = 1 }; /* dtype */
enum { STEQR_EXP = 0, STEQR_PG = 1 };  /* update_scheme */
enum { STEQR_SHIFT_LAPACK = 0, STEQR_SHIFT_CLOSED = 1 };  /* shift */
enum { STEQR_METHOD_QR = 0, STEQR_METHOD_BISECT = 1 };    /* method */

/* Options of steqr_batched_ex. Zero-initialised fields mean "default". */
typedef struct steqr_params {
    /* Sweep budget: max_sweeps_per_n * n implicit sweeps per matrix; the
     * pages time with thirty per eigenvalue (BatchLAS "STEQR: the CTA
     * tridiagonal solver" page, setup paragraph). 0 = 30; negative values
     * mean a budget of zero sweeps (every matrix that needs one fails). */
    int max_sweeps_per_n;
    /* 0 = sort eigenpairs ascending (default), 1 = keep converged order. */
    int no_sort;
    /* Lanes per problem P (problems per 64-lane wavefront = 64 / P). 0 =
     * tuned default, which depends on the order, dtype, jobz and band
     * storage and, at orders 8..32 (and 64, 128 in some cases), on the
     * batch: the fewest lanes whose launch still fills the SIMDs; otherwise
     * a power of two the build provides for this (dtype, n, jobz).
     * steqr_query() reports the choice for a given batch. Every P and band
     * storage gives the same results bit for bit. */
    int lanes_per_problem;
    /* Wavefronts per workgroup (1, 2 or 4); 0 = default (4, fewer when a
     * small batch would otherwise leave fewer than 256 workgroups). Launch
     * shape only: the arithmetic and results do not depend on it. */
    int waves_per_block;
    /* Where a chunked kernel keeps the band d, e during the solve:
     * 0 = tuned default, 1 = replicated in every lane's registers,
     * 2 = shared in LDS (frees registers for more rows of Q per lane),
     * 3 = (orders 33..512 with eigenvectors) shared in LDS by one producer
     *     wavefront per workgroup that runs the chase for one or several
     *     problems and logs its rotations, applied to Q by consumer
     *     wavefronts (one per problem up to order 64; at 65..128 two lanes
     *     per row, or whole rows in float; at 129..256 eight consumers per
     *     problem, two lanes per row in float, four in double with two
     *     workgroups sharing a problem; at 257..512 eight consumers per
     *     workgroup, eight lanes per row in float, sixteen in double, with
     *     eight or sixteen workgroups sharing a problem, each running the
     *     same chase); lanes_per_problem then counts producer lanes.
     * Orders above 32 always use LDS (1 means the default there); orders
     * 65..512 without eigenvectors run the producer's algorithm alone in
     * every wavefront (band storage 2). */
    int band_storage;
    /* Form of the implicit step (BatchLAS steqr algorithm page, "the two CTA
     * update schemes"): STEQR_EXP (0, default) writes each local similarity
     * G^T T G; STEQR_PG (1) is the Parlett-Gray form, which carries the
     * scalars (g, p, c, s) along the sweep. Both are the same implicit
     * step; results differ by rounding only. */
    int update_scheme;
    /* Shift of each implicit step from the trailing 2x2 block (BatchLAS
     * steqr algorithm page, shift section): STEQR_SHIFT_LAPACK (0, default)
     * mu = d1 - e1/(g + copysign(sqrt(g^2+1), g)), g = (d2-d1)/(2 e1);
     * STEQR_SHIFT_CLOSED (1) the closed form lambda+- of the block, the one
     * nearer d1. The same eigenvalue of the block up to rounding. */
    int shift;
    /* Eigenvector accumulation (BatchLAS steqr algorithm page, eigenvector
     * paragraph): 0 (default) Q is output only and the rotations accumulate
     * onto the identity; 1 = back-transformation: Q holds a basis Z
     * [batch][n][n] (row-major, as Q) on entry, the rotations right-multiply
     * it, and Q receives Z G_1 G_2 ... G_p with the sort's column
     * permutation. With Z the orthogonal factor of a reduction A = Z T Z^T,
     * the result is the eigenvectors of A. Needs jobz == STEQR_V (-10
     * otherwise). */
    int back_transform;
    /* Eigenvalue method. STEQR_METHOD_QR (0, default): the implicit QR/QL
     * iteration above. STEQR_METHOD_BISECT (1), values only (jobz ==
     * STEQR_N): Sturm-count bisection for every index 0..n-1, ascending
     * (BatchLAS syev routing and tuning page, the values-only stebz
     * solve): one lane per eigenvalue, each bisecting the Gershgorin
     * interval until it is within max(ulp ||T||, 2 ulp |lambda|), the
     * midpoint stops advancing or floor(log2((||T|| + pivmin)/pivmin)) + 2
     * halvings are spent (the band is first scaled by an exact power of
     * two to ||T|| in [0.5, 1)). info[b] is then the number of indices
     * that ran out of halvings (0 for any finite input in practice), n for
     * a band holding a NaN (all eigenvalues NaN). max_sweeps_per_n and
     * no_sort do not apply; update_scheme, shift, band_storage,
     * back_transform must be 0 (-10 otherwise). lanes_per_problem: 0
     * (default) or the lanes the kernel uses: the padded order up to 64;
     * from order 128 64, 128 or 256 (the problem's indices spread over one,
     * two or four wavefronts of a workgroup, at most the padded order; the
     * default takes the fewest whose launch has 2,048 wavefronts, and
     * waves_per_block then does not apply); -10 otherwise. Every choice
     * gives the same results bit for bit. */
    int method;
} steqr_params;

/* Eigenvalues (jobz = STEQR_N) or eigenpairs (jobz = STEQR_V) of a batch of
 * symmetric tridiagonal matrices, n <= STEQR_MAX_N, in the precision given
 * by dtype. Layout, ownership and error codes as described above. A matrix
 * whose sweep budget runs out keeps its current unsorted values; use
 * steqr_batched_ex to receive the per-matrix status. */
int steqr_batched(const void *d, const void *e, void *lambda, void *Q,
                  int n, int batch, int jobz, int dtype, hipStream_t stream);

/* As steqr_batched, plus:
 *   info    [batch] int, DEVICE memory, may be NULL. info[b] = 0 when matrix
 *           b converged; k > 0 when its sweep budget ran out, k being the
 *           number of nonzero off-diagonal entries left (LAPACK steqr
 *           convention); lambda[b] and Q[b] are then the current unsorted
 *           values, unscaled.
 *   params  may be NULL (all defaults). */
int steqr_batched_ex(const void *d, const void *e, void *lambda, void *Q,
                     int n, int batch, int jobz, int dtype, hipStream_t stream,
                     int *info, const steqr_params *params);

/* Describe the launch steqr_batched_ex would make, without launching:
 * padded order (the compile-time order the kernel runs at, >= n), lanes per
 * problem P, rows of Q held per lane, wavefronts per workgroup, workgroups
 * for `batch` matrices and band storage (1 registers, 2 LDS, 3 LDS with
 * producer and consumer wavefronts; for bisection 1 or 2). Returns 0 or
 * the same negative codes as steqr_batched_ex (-5/-7/-8/-10). Any output
 * pointer may be NULL. */
int steqr_query(int n, int batch, int jobz, int dtype, const steqr_params *params,
                int *padded_n, int *lanes_per_problem, int *rows_per_lane,
                int *waves_per_block, int *workgroups, int *band_storage);

/* ------------------------------------------------------------------------
 * Fused small-n dense symmetric eigensolver (BatchLAS syev routing and
 * tuning page, CTA-family paragraph: one problem resident from the load of
 * A to the store, reduction to tridiagonal form, the steqr solve above and
 * the back-transformation in one kernel; steqr algorithm page, eigenvector
 * paragraph, for the back-transformation). For each symmetric A_b it
 * computes the eigenvalues and, on request, orthonormal eigenvectors:
 * A_b = Q Lambda Q^T. The reduction is the Householder tridiagonalization
 * A = Z T Z^T (reflectors in the LAPACK larfg convention); T is then
 * solved exactly as by steqr_batched_ex with Z as the basis of the
 * back-transformation.
 *
 * Layout: A [batch][n][n] row-major, read only; only the lower triangle
 * (A[b][i][j], j <= i) is read, the strict upper triangle is ignored.
 * lambda [batch][n] ascending; Q [batch][n][n] row-major, eigenvector k in
 * column k (as for steqr_batched). Ownership, asynchrony and the meaning
 * of info as for steqr_batched_ex.
 *
 * Errors (0 on success; -k names the k-th argument):
 *   -1 A == NULL          -2 lambda == NULL      -3 Q == NULL with STEQR_V
 *   -4 n < 0 or n > SYEV_MAX_N (SYEV_MAX_N_F64_V for double with
 *      eigenvectors)                             -5 batch < 0
 *   -6 jobz invalid       -7 dtype invalid
 *   -10 (_ex) params: update_scheme other than STEQR_EXP, back_transform
 *       set, band_storage other than 0/1/2, or a lanes_per_problem /
 *       band_storage / waves_per_block the build does not provide
 *       (syev_query lists them)
 * A positive value is a hipError_t from the launch; n == 0 or batch == 0
 * returns 0 without touching the GPU. */
#define SYEV_MAX_N 32
/* Double precision with eigenvectors: the same limit. At order 32 the rows
 * of A and Q and the replicated band do not fit 256 registers per lane
 * together, so double at order 32 runs with the band in LDS by default
 * (band_storage 2; values only also with 1). */
#define SYEV_MAX_N_F64_V 32

int syev_batched(const void *A, void *lambda, void *Q, int n, int batch, int jobz, int dtype,
                 hipStream_t stream);

int syev_batched_ex(const void *A, void *lambda, void *Q, int n, int batch, int jobz,
                    int dtype, hipStream_t stream, int *info, const steqr_params *params);

/* The launch syev_batched_ex would make (outputs as for steqr_query). */
int syev_query(int n, int batch, int jobz, int dtype, const steqr_params *params,
               int *padded_n, int *lanes_per_problem, int *rows_per_lane,
               int *waves_per_block, int *workgroups, int *band_storage);

/* Library version string, e.g. "steqr-mi355x 0.1.0 gfx950". */
const char *steqr_version(void);

#ifdef __cplusplus
}
#endif

#endif /* STEQR_H */
