// Chunked batched steqr kernel for CDNA4 (gfx950, wave64).
//
// One problem per chunk of P consecutive lanes; a wavefront holds 64/P
// problems. Design (MI355X-first, not a port of the pages' CUDA-warp
// schedulers):
//
//  * Replicated band state. Every lane of a chunk holds the whole d[N], e[N]
//    of its problem in VGPRs and performs the (serial) chase itself, so the
//    rotation (c, s) is available in every lane without any cross-lane
//    broadcast. All lanes of a chunk compute identical values.
//  * Q rows in VGPRs. Lane r of a chunk holds rows r*R .. r*R+R-1 of Q
//    (R = ceil(N/P)); each rotation is a lane-parallel update of two columns
//    of those rows [algo, eigenvector accumulation].
//  * Static positions. N is a compile-time order (n <= N, padded with a
//    zero problem tail, as on the CTA page's set-up); every loop over
//    positions is fully unrolled, so d[p], e[p], q[i][p] are registers.
//  * Direction unification [cta, micro-structure list, QL versus QR: one
//    direction runs as the other on the reversed block]: a block that must
//    converge at its top is mirrored
//    (the whole order-N problem, Q's columns included, by a static register
//    reversal) so that every chunk always chases top to bottom and always
//    converges at the bottom of its block.
//  * Lockstep passes. The wavefront repeats: settle (each chunk opens blocks,
//    deflates converged eigenvalues with bit operations over a position
//    mask, and picks its next operation: a sweep on [s, m] or an analytic
//    2x2 solve at one position), then one chase pass over the static
//    positions in which every chunk with a sweep applies its rotation at p
//    when s <= p < m. Lanes whose chunk is idle at p are masked off (EXEC),
//    and positions where no chunk is active are skipped by the wave.
//    A 2x2 block is a one-step chase at its position, seeded with its
//    closed-form rotation. The step is written in the EXP form (local
//    similarity) or, with the PG template flag, in the Parlett-Gray form
//    [algo, update-scheme paragraph].
//  * Run-time positions (the shift inputs at the converging end, the block
//    ends, the sort keys) are read from a per-chunk copy of the band in LDS,
//    kept current after every change of the band (written by the chase's
//    steps with eigenvectors, republished after the pass without); register
//    arrays are only ever indexed by compile-time positions.
//
// The per-chunk sequence of operations is the one of the steqr algorithm
// page: split blocks at exact zeros, the left boundary moving right [algo,
// steqr_cta paragraph], scale each block [algo, scaling], converge the end
// of smaller |d| first [cta, micro-structure list], re-test deflation after
// every step and locate the last new zero from the converging end [algo],
// solve 2x2 blocks analytically [algo], shift from the trailing 2x2 block
// (LAPACK form) [algo, shift section], chase with Givens rotations as
// similarities [algo], count sweeps against a budget of
// max_sweeps_per_n * n [cta, setup paragraph], unscale, sort ascending and
// permute Q's columns [algo].
#pragma once

#include "steqr_device.hpp"
#include "syev_reduce.hpp"
#include "steqr_phase.hpp"

namespace steqr {

struct KernelArgs {
    const void* d;
    const void* e;
    void* lam;
    void* q;
    int* info;
    int n;
    int batch;
    int max_sweeps_per_n;
    int do_sort;
    int shift_kind;  // 0 = LAPACK-form shift, 1 = closed form lambda+-
    int back_transform;  // 1: q holds a basis on entry, right-multiplied
    const void* a;       // dense kernels: A [batch][n][n], lower triangle read
};

// Reverse the whole order-N problem in place (positions p <-> N-1-p for d
// and Q's columns, e_p <-> e_{N-2-p}) when `mir` holds.
template <typename T, int N, int RQ, bool WITHQ>
__device__ __forceinline__ void mirror_problem(bool mir, T (&d)[N], T (&e)[N], T (&q)[RQ][N]) {
    static_for<N / 2>([&](auto I) {
        constexpr int p = decltype(I)::value;
        const T a = d[p], b = d[N - 1 - p];
        d[p] = mir ? b : a;
        d[N - 1 - p] = mir ? a : b;
    });
    static_for<(N - 1) / 2>([&](auto I) {
        constexpr int p = decltype(I)::value;
        const T a = e[p], b = e[N - 2 - p];
        e[p] = mir ? b : a;
        e[N - 2 - p] = mir ? a : b;
    });
    if constexpr (WITHQ) {
        static_for<RQ>([&](auto II) {
            constexpr int i = decltype(II)::value;
            static_for<N / 2>([&](auto I) {
                constexpr int p = decltype(I)::value;
                const T a = q[i][p], b = q[i][N - 1 - p];
                q[i][p] = mir ? b : a;
                q[i][N - 1 - p] = mir ? a : b;
            });
        });
    }
}

// Copy `total` (<= MAXE) consecutive elements from src to dst with the 64
// lanes of a wavefront, consecutive lanes at consecutive addresses; `vec`
// (both ends 16-byte aligned, total a multiple of the piece) moves 16-byte
// pieces. Used between HBM and the LDS staging area of Q.
template <typename T, int MAXE>
__device__ __forceinline__ void copy_block(T* __restrict__ dst, const T* __restrict__ src,
                                           int total, int lane, bool vec) {
    if (vec) {
        constexpr int V = 16 / sizeof(T);
        static_for<(MAXE + 64 * V - 1) / (64 * V)>([&](auto K) {
            constexpr int k = decltype(K)::value;
            const int idx = (k * 64 + lane) * V;
            if (idx < total) {
                if constexpr (sizeof(T) == 4) {
                    *reinterpret_cast<float4*>(dst + idx) = *reinterpret_cast<const float4*>(src + idx);
                } else {
                    *reinterpret_cast<double2*>(dst + idx) = *reinterpret_cast<const double2*>(src + idx);
                }
            }
        });
    } else {
        static_for<(MAXE + 63) / 64>([&](auto K) {
            constexpr int k = decltype(K)::value;
            const int idx = k * 64 + lane;
            if (idx < total) dst[idx] = src[idx];
        });
    }
}

// LDS per wavefront: one band slot per chunk (d then e, padded to an odd
// number of elements against bank conflicts), for P > 1 one rank row per
// chunk for the final sort, and with eigenvectors a staging area holding the
// wavefront's Q blocks in their HBM layout, so that the store is one
// contiguous, fully coalesced copy (the dense kernels also stage A there).
template <typename T, int N, int P, bool WANTQ = false, bool DENSE = false>
struct Smem {
    static constexpr int CH = 64 / P;
    static constexpr int SLOT = 2 * N + 1;
    static constexpr int band_elems = CH * SLOT;
    static constexpr int rank_ints = (P > 1) ? CH * N : 0;
    static constexpr size_t band_bytes = ((band_elems * sizeof(T) + 15) / 16) * 16;
    static constexpr size_t rank_bytes = (((size_t)rank_ints * sizeof(int) + 15) / 16) * 16;
    static constexpr size_t stage_bytes = (WANTQ || DENSE) ? (size_t)CH * N * N * sizeof(T) : 0;
    static constexpr size_t bytes_per_wave = band_bytes + rank_bytes + stage_bytes;
};

// DENSE: the fused dense eigensolver. The chunk loads a dense symmetric
// matrix (args.a), reduces it to tridiagonal form with Q accumulated in the
// registers that otherwise start as the identity, and continues with the
// tridiagonal solve below, which then back-transforms that Q.
template <typename T, int N, int P, bool WANTQ, bool PG, bool DENSE = false>
__global__ void __launch_bounds__(256) steqr_chunk_kernel(KernelArgs args) {
    static_assert(P >= 1 && P <= 64 && (64 % P) == 0, "P must divide 64");
    static_assert(!DENSE || (N % P) == 0, "dense: the lanes hold whole rows");
    constexpr int CH = 64 / P;                       // problems per wavefront
    constexpr int R = WANTQ ? (N + P - 1) / P : 0;   // rows of Q per lane
    constexpr int RQ = R > 0 ? R : 1;
    constexpr int RJ = (N + P - 1) / P;              // sort keys ranked per lane
    using M = PosMask<N>;
    using F = Fp<T>;
    using S = Smem<T, N, P, WANTQ, DENSE>;
    enum { ST_OPEN = 0, ST_ITER = 1, ST_DONE = 2 };
    // split the deflation scan over the chunk's lanes from 4 lanes per
    // problem (DPP lane moves up to 16 lanes; 32-bit position masks); at 2
    // lanes the LDS reads cost more than the halved scan saves (measured)
    constexpr bool SPLIT_SCAN = P >= 4 && P <= 16 && N <= 32 && P <= N;

    extern __shared__ __align__(16) unsigned char smem_raw[];

    const T* __restrict__ gd = static_cast<const T*>(args.d);
    const T* __restrict__ ge = static_cast<const T*>(args.e);
    T* __restrict__ glam = static_cast<T*>(args.lam);
    T* __restrict__ gq = static_cast<T*>(args.q);
    const int n = args.n;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    // phase slots: 0 load, 5 settle up to the next operation (block open,
    // deflation scan, masks), 6 settle's closes and shift, 1 settle's 2x2
    // step setup, 2 chase, 3 epilogue, 4 passes
    STEQR_PHASE_START;
    const int chunk = lane / P;
    const int r = lane % P;
    const long prob = ((long)blockIdx.x * (blockDim.x >> 6) + wave) * CH + chunk;
    const bool live = prob < (long)args.batch;
    const long pb = live ? prob : (long)args.batch - 1;  // in-bounds address for dead chunks

    unsigned char* wave_smem = smem_raw + (size_t)wave * S::bytes_per_wave;
    T* const sd = reinterpret_cast<T*>(wave_smem) + chunk * S::SLOT;  // chunk's d copy
    T* const se = sd + N;                                              // chunk's e copy
    int* const srank = reinterpret_cast<int*>(wave_smem + S::band_bytes) + chunk * N;
    T* const stage = reinterpret_cast<T*>(wave_smem + S::band_bytes + S::rank_bytes);

    // ---------------------------------------------------------------- load
    T d[N], e[N];
    // The wavefront's problems are consecutive, and so are their Q blocks
    // (and dense matrices) in HBM: [first, first + nprob) holds the live ones.
    const long first = ((long)blockIdx.x * (blockDim.x >> 6) + wave) * CH;
    const int nprob = (long)args.batch - first < CH ? (int)((long)args.batch - first) : CH;
    const int nn = n * n;
    const bool qvec = ((nn & 3) == 0) & ((reinterpret_cast<uintptr_t>(gq) & 15) == 0);
    T q[RQ][N];
    if constexpr (DENSE) {
        // one coalesced copy of the wavefront's matrices into the staging
        // area, then each lane takes its rows, the strict upper triangle
        // mirrored from the lower one
        constexpr int RA = N / P;
        const T* __restrict__ ga = static_cast<const T*>(args.a);
        const bool avec = ((nn & 3) == 0) & ((reinterpret_cast<uintptr_t>(ga) & 15) == 0);
        copy_block<T, CH * N * N>(stage, ga + first * nn, nprob * nn, lane, avec);
        __builtin_amdgcn_wave_barrier();
        const T* const st = stage + chunk * nn;
        T a[RA][N];
        static_for<RA>([&](auto II) {
            constexpr int i = decltype(II)::value;
            const int row = r * RA + i;
            const bool in = live & (row < n);
            static_for<N>([&](auto J) {
                constexpr int j = decltype(J)::value;
                const bool use = in & (j < n);
                const int idx = use ? ((j <= row) ? row * n + j : j * n + row) : 0;
                const T v = st[idx];
                a[i][j] = use ? v : T(0);
            });
        });
        static_for<RQ>([&](auto II) {
            constexpr int i = decltype(II)::value;
            const int row = r * R + i;
            static_for<N>([&](auto J) {
                constexpr int j = decltype(J)::value;
                q[i][j] = (WANTQ & (row == j)) ? T(1) : T(0);
            });
        });
        householder_chunk<T, N, P, RA, WANTQ, RQ>(a, q, d, e, sd, se, nullptr, n, r);
    } else {
        static_for<N>([&](auto I) {
            constexpr int p = decltype(I)::value;
            const int pc = p < n ? p : n - 1;
            const T v = gd[pb * n + pc];
            d[p] = (live & (p < n)) ? v : T(0);
            e[p] = T(0);
        });
        if (n > 1) {
            static_for<N - 1>([&](auto I) {
                constexpr int p = decltype(I)::value;
                const int pc = p < n - 1 ? p : n - 2;
                const T v = ge[pb * (n - 1) + pc];
                e[p] = (live & (p < n - 1)) ? v : T(0);
            });
        }
        if (WANTQ && args.back_transform) {
            // back-transformation [algo, eigenvector accumulation]: the lane's
            // rows of the caller's basis, loaded straight into registers (the
            // loads overlap the first settle)
            const bool vec = (n == N) & ((reinterpret_cast<uintptr_t>(gq) & 15) == 0);
            static_for<RQ>([&](auto II) {
                constexpr int i = decltype(II)::value;
                load_basis_row<T, N>(gq + pb * nn, n, r * R + i, live, true, vec, q[i]);
            });
        } else {
            static_for<RQ>([&](auto II) {
                constexpr int i = decltype(II)::value;
                const int row = r * R + i;
                static_for<N>([&](auto J) {
                    constexpr int j = decltype(J)::value;
                    q[i][j] = (WANTQ & (row == j)) ? T(1) : T(0);
                });
            });
        }
    }
    // bit p set <=> e_p == 0 (positions >= n-1 are zero padding)
    M zeromask = 0;
    static_for<N>([&](auto I) {
        constexpr int p = N - 1 - decltype(I)::value;
        zeromask = zeromask + zeromask + ((e[p] == T(0)) ? (M)1 : (M)0);
    });

    // Publish the chunk's band to LDS (one lane per chunk writes; the
    // wavefront executes its LDS operations in order, so later reads by any
    // lane of the chunk see it).
    auto publish = [&]() __attribute__((always_inline)) {
        if (r == 0) {
            static_for<N>([&](auto I) {
                constexpr int p = decltype(I)::value;
                sd[p] = d[p];
                se[p] = e[p];
            });
        }
        __builtin_amdgcn_wave_barrier();
    };
    publish();

    // ---------------------------------------------------------------- state
    // ST_OPEN: the chunk's next block is to be opened; ST_ITER: a block is
    // being reduced; ST_DONE: nothing left to reduce (a converged last block
    // may still wait for its close, `pending`).
    int state = live ? ST_OPEN : ST_DONE;
    int l1 = 0;           // left boundary of the next split block (original coords)
    int bt = 0, bb = 0;   // current block [bt, bb] in current (possibly mirrored) coords
    int m = 0;            // converging (bottom) end of the active part
    int s = 0;            // top of the unreduced part [s, m]
    int jtot = 0;
    const int nmaxit = (args.max_sweeps_per_n > 0 ? args.max_sweeps_per_n : 0) * n;
    bool mir = false, failed = false;
    bool last = false;     // no block follows the current one
    bool pending = false;  // converged last block, closed after the loop
    int mode = 0;
    T anorm = T(0);
    M zeroed = 0;  // negligible e's found inside the current block
    int info = 0;

    // Close the current block: zero the negligible e's found in it, undo the
    // scaling (d always, e too when the block failed), undo the mirror.
    auto close_block = [&](bool fail) __attribute__((always_inline)) {
        static_for<N - 1>([&](auto I) {
            constexpr int p = decltype(I)::value;
            e[p] = ((zeroed >> p) & 1) ? T(0) : e[p];
        });
        if (mode != 0) {
            const T un = (mode == 1) ? anorm / F::ssfmax : anorm / F::ssfmin;
            static_for<N>([&](auto I) {
                constexpr int p = decltype(I)::value;
                d[p] = ((p >= bt) & (p <= bb)) ? d[p] * un : d[p];
                if constexpr (p < N - 1) e[p] = (fail & (p >= bt) & (p < bb)) ? e[p] * un : e[p];
            });
        }
        mirror_problem<T, N, RQ, WANTQ>(mir, d, e, q);
        mir = false;
        mode = 0;
        zeroed = 0;
    };

    // Open the next block of every chunk in ST_OPEN: skip 1x1 blocks (zero
    // e) and stop at the first zero e at or right of the block start [algo,
    // steqr_cta paragraph]; skip blocks of norm zero; scale [algo, scaling];
    // pick the converging end and mirror.
    auto open_blocks = [&]() __attribute__((always_inline)) {
        while (state == ST_OPEN) {
            const M avail = ~zeromask & ~bits_below<M>(l1) & bits_below<M>(n - 1);
            if (avail == 0) {
                state = ST_DONE;
                break;
            }
            const int lo = lsb(avail);
            const int hi = lsb((M)(zeromask & ~bits_below<M>(lo)));
            l1 = hi + 1;
            last = (avail & ~bits_below<M>(l1)) == 0;
            // block norm, NaN-propagating [algo, scaling]
            T an = T(0);
            bool hasnan = false;
            static_for<N>([&](auto I) {
                constexpr int p = decltype(I)::value;
                const bool ind = (p >= lo) & (p <= hi);
                const bool ine = (p >= lo) & (p < hi);
                an = ind ? F::max(an, F::abs(d[p])) : an;
                an = ine ? F::max(an, F::abs(e[p])) : an;
                hasnan = hasnan | (ind & (d[p] != d[p])) | (ine & (e[p] != e[p]));
            });
            anorm = hasnan ? F::qnan() : an;
            if (anorm == T(0)) continue;
            mode = (anorm > F::ssfmax) ? 1 : ((anorm < F::ssfmin) ? 2 : 0);
            const T sg = (mode == 0) ? T(1) : ((mode == 1) ? F::ssfmax : F::ssfmin) / anorm;
            if (mode != 0) {
                static_for<N>([&](auto I) {
                    constexpr int p = decltype(I)::value;
                    d[p] = ((p >= lo) & (p <= hi)) ? d[p] * sg : d[p];
                    e[p] = ((p >= lo) & (p < hi)) ? e[p] * sg : e[p];
                });
            }
            // converge the end of smaller magnitude first; a tie or NaN
            // converges the top end first, i.e. mirror. |sg*x| = sg*|x|
            // exactly, so this compares the scaled end values.
            const T dlo = F::abs(sd[lo]) * sg, dhi = F::abs(sd[hi]) * sg;
            mir = !(dhi < dlo);
            mirror_problem<T, N, RQ, WANTQ>(mir, d, e, q);
            bt = mir ? N - 1 - hi : lo;
            bb = mir ? N - 1 - lo : hi;
            m = bb;
            // the coupling above the block is zero; the chase may write
            // it and closing the block restores it
            zeroed = bt > 0 ? ((M)1 << (bt - 1)) : (M)0;
            state = ST_ITER;
        }
    };

    T x = T(0), y = T(0);  // running pair of the chase
    STEQR_PHASE_MARK(0);
    while (true) {
        // ------------------------------------------------------------ settle
        // Opening and closing blocks are rare (once per block); they run
        // behind wavefront-wide tests. The per-pass part is straight-line.
        if (__any(state == ST_OPEN)) {
            open_blocks();
            publish();
        }
        const bool iter = state == ST_ITER;
        if (!__any(iter)) break;
        // deflation test [algo, deflation] at every position; e's found
        // negligible earlier count too (the chase may overwrite them). With
        // several lanes per problem, lane r tests positions r*K .. r*K+K-1
        // of the chunk's band copy in LDS (current: it is republished after
        // every change) and the lanes OR their partial masks; the same
        // values and the same test as the register scan, so the same mask.
        M neg = 0;
        if constexpr (SPLIT_SCAN) {
            constexpr int K = (N - 1 + P - 1) / P;  // P*K <= N: reads stay in the slot
            const int p0 = r * K;
            unsigned loc = 0;
            static_for<K>([&](auto KK) {
                constexpr int k = decltype(KK)::value;
                const int p = p0 + k;
                loc |= negligible(se[p], sd[p], sd[p + 1]) ? (1u << k) : 0u;
            });
            neg = (M)chunk_or_dpp<P>(loc << p0) & bits_below<M>(N - 1);
        } else {
            static_for<N - 1>([&](auto I) {
                constexpr int p = N - 2 - decltype(I)::value;
                neg = neg + neg + (negligible(e[p], d[p], d[p + 1]) ? (M)1 : (M)0);
            });
        }
        neg |= zeroed;
        const M rng = bit_range<M>(bt, m - 1);
        const M nb = neg & rng;
        const M clr = rng & ~neg;
        // every remaining eigenvalue of the block has converged
        const bool conv = iter & (clr == 0);
        const bool go = iter & (clr != 0);
        // the bottom run of negligible e's deflates 1x1 eigenvalues (new
        // end t); the last negligible e above t bounds the unreduced part
        // [s, t] [algo]
        const int t = msb((M)(clr | (M)1));
        const M above = nb & bit_range<M>(bt, t - 1);
        const int s2 = above ? msb(above) + 1 : bt;
        const M znew = (nb & bit_range<M>(t + 1, m - 1)) | (above ? ((M)1 << (above ? s2 - 1 : 0)) : (M)0);
        zeroed |= conv ? nb : (go ? znew : (M)0);
        // next operation: an analytic 2x2 solve, a failure (budget spent)
        // or a sweep on [s, m]
        const bool jac = go & (t == s2);
        const bool fail = go & !jac & (jtot >= nmaxit);
        const bool sweep = go & !jac & !fail;
        const int jpos = s2;
        m = jac ? s2 - 1 : (go ? t + 1 : m);
        s = go ? s2 : s;
        jtot += sweep ? 1 : 0;
        STEQR_PHASE_MARK(5);
        // a failed block, or a converged block with another one after it
        const bool close_now = fail | (conv & !last);
        if (__any(close_now)) {
            if (close_now) {
                close_block(fail);
                if (fail) {
                    failed = true;
                    M nz = 0;
                    static_for<N - 1>([&](auto I) {
                        constexpr int p = N - 2 - decltype(I)::value;
                        nz = nz + nz + ((e[p] != T(0)) ? (M)1 : (M)0);
                    });
                    info = popc((M)(nz & bits_below<M>(n - 1)));
                    info = info > 0 ? info : 1;
                }
                state = fail ? ST_DONE : ST_OPEN;
            }
            publish();
        }
        // a converged last block is closed after the loop
        pending = pending | (conv & last);
        state = (conv & last) ? ST_DONE : state;
        // shift from the trailing 2x2 (LAPACK form) [algo, shift section];
        // running pair for the first rotation: (d_s - mu, e_s)
        const int mi = sweep ? m : (jac ? jpos + 1 : 1);
        const int si = sweep ? s : 0;
        const T dm = sd[mi], dm1 = sd[mi - 1], em1 = se[mi - 1];
        const T mu = sweep_shift(args.shift_kind != 0, dm, dm1, em1);
        // EXP carries the pair (x, y) the next rotation annihilates; PG
        // carries g in x and the previous sine in y (f = y e_p)
        x = sd[si] - mu;
        y = PG ? T(1) : se[si];
        STEQR_PHASE_MARK(6);
        // A 2x2 block at (jpos, jpos+1) [algo, 2x2 block paragraph]: its
        // closed-form Schur rotation becomes the running
        // pair of a one-step chase at jpos (lartg returns that rotation, for
        // PG from (cs e, -sj e), the same rotation up to sign), so it is
        // applied by the same similarity and Q update as the sweeps. The
        // leftover e_jpos (rounding size) joins `zeroed`.
        if (__any(jac)) {
            T rt1, rt2, cs, sj;
            sym2x2(dm1, em1, dm, rt1, rt2, cs, sj);
            x = jac ? (PG ? cs * em1 : cs) : x;
            y = jac ? -sj : y;
            zeroed |= jac ? ((M)1 << jpos) : (M)0;
        }

        // ------------------------------------------------------------ chase pass
        // Running pair (x, y), seeded in the settle. The update
        // e_{p+1} <- c_p e_{p+1} of step p is applied by step p itself in the
        // EXP form (the last step of a sweep scales the negligible or zero e
        // below the block, which stays negligible) and by step p+1 through
        // the previous cosine cp in the PG form. Step p writes r into
        // e_{p-1}; at the first step that position is a zero coupling or a
        // negligible e already in `zeroed`, which the next deflation test
        // keeps and closing the block restores.
        T cp = T(1);
        STEQR_PHASE_MARK(1);
        STEQR_PHASE_ADD(4, 1);
        // The chase runs at a raised issue priority and the settle at the
        // default one: with two wavefronts per SIMD the SIMD's arbiter then
        // prefers the chase's dense VALU stream over the other wavefront's
        // settle (measured: 2% faster than no priority change; raising the
        // settle's priority instead gains 1.4%).
        __builtin_amdgcn_s_setprio(1);
        // step p runs when s <= p < m: one unsigned compare of p - s with
        // the step count (0 when this chunk does not sweep)
        const unsigned steps = sweep ? (unsigned)(m - s) : (jac ? 1u : 0u);
        static_for<N - 1>([&](auto I) {
            constexpr int p = decltype(I)::value;
            if ((unsigned)(p - s) < steps) {
                T c, sn, rr;
                if constexpr (PG) {
                    // PG step [algo, update-scheme paragraph]: f = s' e_p,
                    // (c, s, r) = lartg(g, f), r* = (d_{p+1} - g*) s + 2 c c' e_p,
                    // d_p = g* + s r*, g = c r* - c' e_p (c', s' of the previous
                    // step). g* = d_p - s' r*' is folded into d_p by the
                    // previous step (d_{p+1} -= s r* below), which also leaves
                    // the sweep's final d_m -= p in place; e_p = g is the
                    // final e_{m-1} = g, and the next step overwrites it with r.
                    const T f = y * e[p];
                    const T b = cp * e[p];
                    lartg(x, f, c, sn, rr);
                    if constexpr (p > 0) e[p - 1] = rr;
                    const T gs = d[p];
                    const T rs = F::fma(d[p + 1] - gs, sn, (c + c) * b);
                    const T pk = sn * rs;
                    d[p] = gs + pk;
                    d[p + 1] = d[p + 1] - pk;
                    x = F::fma(c, rs, -b);
                    e[p] = x;
                    y = sn;
                    cp = c;
                } else {
                    // EXP step [algo]: first rotation from (d_s - mu, e_s),
                    // later ones from (e_{p-1}, bulge); apply G^T B G to the
                    // 2x2 at (p, p+1) (exp_step_w). e_p already carries the
                    // previous step's factor c (applied eagerly below); the
                    // new d_p, d_{p+1} and running x are written over the old
                    // values in place, so the lanes this step masks off keep
                    // theirs without a copy.
                    const T b = e[p];
                    lartg(x, y, c, sn, rr);
                    if constexpr (p > 0) e[p - 1] = rr;
                    const T w = exp_step_w(c, sn, d[p], b, d[p + 1]);
                    F::fma_acc(d[p], sn, w);
                    F::fma_acc_neg(d[p + 1], sn, w);
                    F::fma_over_neg(x, c, w, b);
                    e[p] = x;
                    if constexpr (p + 1 < N - 1) {
                        y = sn * e[p + 1];     // new bulge
                        e[p + 1] = c * e[p + 1];
                    }
                }
                // With eigenvectors the band copy in LDS follows the chase
                // (every lane of the chunk writes the same words): this
                // step's final d_p and e_{p-1}, and d_{p+1}, e_p, final after
                // the sweep's last step. The factor c the EXP step applies to
                // e_{p+1} at the last step is not copied: that e is zero or
                // already in `zeroed`. Without eigenvectors the shorter step
                // measured faster with one publish after the pass.
                if constexpr (WANTQ) {
                    if constexpr (p > 0) se[p - 1] = e[p - 1];
                    sd[p] = d[p];
                    sd[p + 1] = d[p + 1];
                    se[p] = e[p];
                }
                if constexpr (WANTQ) {
                    static_for<R>([&](auto II) {
                        constexpr int i = decltype(II)::value;
                        F::rot(q[i][p], q[i][p + 1], c, sn);
                    });
                }
            }
        });
        __builtin_amdgcn_s_setprio(0);
        if constexpr (WANTQ) __builtin_amdgcn_wave_barrier();
        else publish();
        STEQR_PHASE_MARK(2);
        // a NaN shift turns [s, m] into NaN, a fixed point of every further
        // sweep: spend the rest of the budget at once (same final state)
        jtot = (sweep & (mu != mu)) ? nmaxit : jtot;
    }
    STEQR_PHASE_MARK(1);
    // closes of converged last blocks, all at once
    if (__any(pending)) {
        if (pending) close_block(false);
        publish();
    }

    // ---------------------------------------------------------------- sort
    // rank_j = #{k < n : (d_k, k) precedes (d_j, j)}: ascending, ties by
    // index, NaN last [algo, sort paragraph]. Lane r of a chunk ranks keys
    // j = r, r+P, ... and shares the ranks through LDS.
    const bool sort_it = (args.do_sort != 0) & !failed;
    // with no NaN among the wavefront's keys (a wave-uniform test) the
    // comparison drops its NaN terms: (d_k, k) precedes (d_j, j) iff
    // d_k < d_j, or d_k = d_j and k < j (k = j then never counts)
    bool nan_here = false;
    static_for<N>([&](auto K) {
        constexpr int k = decltype(K)::value;
        nan_here = nan_here | ((k < n) & (d[k] != d[k]));
    });
    const bool nonan = !__any(nan_here);
    auto rank_of = [&](T dj, int j) __attribute__((always_inline)) {
        int rk = 0;
        if (nonan) {
            static_for<N>([&](auto K) {
                constexpr int k = decltype(K)::value;
                const T dk = d[k];
                rk += ((k < n) & ((dk < dj) | ((dk == dj) & (k < j)))) ? 1 : 0;
            });
        } else {
            const bool nanj = dj != dj;
            static_for<N>([&](auto K) {
                constexpr int k = decltype(K)::value;
                const T dk = d[k];
                const bool before =
                    (k < j) ? ((dk <= dj) | nanj) : ((dk < dj) | (nanj & (dk == dk)));
                rk += ((k < n) & (k != j) & before) ? 1 : 0;
            });
        }
        return sort_it ? rk : j;
    };
    int rank[N];
    T myd[RJ];
    int myrank[RJ];
    if constexpr (P == 1) {
        static_for<N>([&](auto J) {
            constexpr int j = decltype(J)::value;
            rank[j] = rank_of(d[j], j);
        });
    } else {
        static_for<RJ>([&](auto K) {
            constexpr int k = decltype(K)::value;
            const int j = r + k * P;
            const int jc = j < N ? j : N - 1;
            myd[k] = sd[jc];
            myrank[k] = rank_of(myd[k], j);
            if (j < N) srank[j] = myrank[k];
        });
        __builtin_amdgcn_wave_barrier();
        static_for<N>([&](auto J) {
            constexpr int j = decltype(J)::value;
            rank[j] = srank[j];
        });
    }

    // ---------------------------------------------------------------- store
    if (live) {
        if constexpr (P == 1) {
            static_for<N>([&](auto J) {
                constexpr int j = decltype(J)::value;
                if (j < n) glam[prob * n + rank[j]] = d[j];
            });
        } else {
            static_for<RJ>([&](auto K) {
                constexpr int k = decltype(K)::value;
                const int j = r + k * P;
                if (j < n) glam[prob * n + myrank[k]] = myd[k];
            });
        }
        if (args.info != nullptr && r == 0) args.info[prob] = info;
    }
    if constexpr (WANTQ) {
        // stage the wavefront's Q blocks (chunk c at c*n*n, row-major with
        // the sort's column permutation applied), then copy them to HBM as
        // one contiguous range: the wavefront's problems are consecutive.
        T* const myq = stage + chunk * nn;
        if (n == N) {
            // full order (uniform): the lane's rows r*R .. r*R+R-1 lie N
            // elements apart, so one address per column serves all of them
            // through the instruction's constant offset
            static_assert(!WANTQ || R * P == N, "the chunk's lanes hold exactly N rows");
            T* const base = myq + r * R * N;
            static_for<N>([&](auto J) {
                constexpr int j = decltype(J)::value;
                T* const col = base + rank[j];
                static_for<R>([&](auto II) {
                    constexpr int i = decltype(II)::value;
                    col[i * N] = q[i][j];
                });
            });
        } else {
            static_for<R>([&](auto II) {
                constexpr int i = decltype(II)::value;
                const int row = r * R + i;
                if (row < n) {
                    static_for<N>([&](auto J) {
                        constexpr int j = decltype(J)::value;
                        if (j < n) myq[row * n + rank[j]] = q[i][j];
                    });
                }
            });
        }
        __builtin_amdgcn_wave_barrier();
        copy_block<T, CH * N * N>(gq + first * nn, stage, nprob * nn, lane, qvec);
    }
    STEQR_PHASE_MARK(3);
    STEQR_PHASE_STORE(wave, lane);
}

}  // namespace steqr
