// Chunked steqr kernel with the band in LDS (gfx950, wave64).
//
// Same per-problem algorithm and lockstep pass structure as
// steqr_chunk.hpp (P lanes serve one problem, Q rows in VGPRs,
// mirrored blocks so every chunk chases top to bottom), but the band d, e of
// each chunk lives in LDS instead of being replicated in every lane's
// VGPRs. That frees 2N VGPRs per lane, which is what lets a lane hold more
// rows of Q (fewer lanes per problem, less repeated chase arithmetic) at a
// usable occupancy for N = 32, and it lets the lanes of a chunk share the
// settle-phase work:
//  * the deflation scan, the block norm, the scaling, the mirror and the
//    sort keys are split over the P lanes of the chunk (lane r handles
//    positions r, r+P, ..., or at 2 and 4 lanes a run of consecutive
//    positions for the scan) and combined with DPP lane moves (the ORs) or
//    butterfly shuffles (the block norm's maximum, once per block);
//  * the chase reads d_{p+2}, e_{p+2} at position p (a two-deep window), so
//    the LDS latency overlaps the rotation; every lane of the chunk writes
//    the same final d_p and e_{p-1} to the same word (no lane mask);
//  * Q is written through an LDS slice per row index: lane r of a chunk
//    holds rows r, r+P, ..., so each slice is P consecutive rows of every
//    chunk's Q, copied out in coalesced 16-byte pieces after the column
//    permutation of the sort.
// Citations as in steqr_chunk.hpp ([algo] = the steqr algorithm page,
// [cta] = "STEQR: the CTA tridiagonal solver").
#pragma once

#include "steqr_chunk.hpp"

namespace steqr {

template <typename T, int N, int P>
struct SmemL {
    static constexpr int CH = 64 / P;
    static constexpr int SLOT = 2 * N + 1;                 // d[N], e[N], pad
    static constexpr int STAGE_STRIDE = N + 1;             // staging row stride
    static constexpr size_t band_bytes = ((CH * SLOT * sizeof(T) + 15) / 16) * 16;
    static constexpr size_t rank_bytes = ((CH * N * sizeof(int) + 15) / 16) * 16;
    static constexpr size_t stage_bytes = ((64 * STAGE_STRIDE * sizeof(T) + 15) / 16) * 16;
    static constexpr size_t bytes_per_wave = band_bytes + rank_bytes + stage_bytes;
};

// OR / max over the P lanes of a chunk (every lane of the chunk must be
// active, which holds because a chunk's lanes share control flow). The OR
// takes DPP lane moves, whose partners never leave the chunk.
// With 64 lanes per problem the result is the same in every lane of the
// wavefront: read it into a scalar register, so that the masks and the
// per-problem state derived from them live in scalar registers.
template <int P>
__device__ __forceinline__ unsigned chunk_or(unsigned v) {
    v = chunk_or_dpp<P>(v);
    if constexpr (P == 64) v = (unsigned)__builtin_amdgcn_readfirstlane((int)v);
    return v;
}
// OR over the P lanes of a chunk for masks of 32 to 512 bits (DPP lane
// moves on each 32-bit word)
template <int P, typename M>
__device__ __forceinline__ M chunk_or_mask(M v) {
    if constexpr (sizeof(M) <= 16) {
        M out = 0;
        static_for<(int)(sizeof(M) / 4)>([&](auto WW) {
            constexpr int w = decltype(WW)::value;
            out |= (M)chunk_or<P>((unsigned)(v >> (32 * w))) << (32 * w);
        });
        return out;
    } else {
        M out;
        static_for<M::WORDS>([&](auto WW) {
            constexpr int w = decltype(WW)::value;
            const uint64_t lo = chunk_or<P>((unsigned)v.w[w]);
            const uint64_t hi = chunk_or<P>((unsigned)(v.w[w] >> 32));
            out.w[w] = lo | (hi << 32);
        });
        return out;
    }
}

// Deflation test [algo, deflation] of every position of a chunk's band copy
// in LDS (sd = d, se = e; the slot holds at least 2N values, so sd[N] reads
// se[0]), split over the chunk's P lanes with no branch; the partial masks
// are OR-ed and bit N-1 (no such off-diagonal) is cleared. With 8 to 32
// lanes, lane r tests positions r, r+P, r+2P, ... (consecutive lanes read
// consecutive words: no bank conflicts); its bits are gathered per 32-bit
// word of the mask at lane 0's places and shifted by r at the end (kP mod 32
// + r < 32 as P divides 32). With 2 or 4 lanes (at most 4-way bank
// conflicts) and with 64, lane r tests the consecutive positions r*K ..
// r*K+K-1, which take about half as many LDS reads (measured faster at 4
// lanes, slower at 16).
template <typename T, int N, int P, typename M>
__device__ __forceinline__ M scan_negligible(const T* sd, const T* se, int r) {
    constexpr int K = N / P;
    constexpr int WORDS = (int)(sizeof(M) / 4);
    static_assert(K * P == N && K <= 32 && sizeof(M) * 8 >= N, "P lanes per chunk");
    if constexpr (P <= 4 || P > 32) {
        unsigned loc = 0;
        static_for<K>([&](auto KK) {
            constexpr int k = decltype(KK)::value;
            const int p = r * K + k;
            loc |= negligible(se[p], sd[p], sd[p + 1]) ? (1u << k) : 0u;
        });
        return chunk_or_mask<P>((M)((M)loc << (r * K))) & bits_below<M>(N - 1);
    } else {
        unsigned word[WORDS];
        static_for<WORDS>([&](auto WW) { word[decltype(WW)::value] = 0u; });
        static_for<K>([&](auto KK) {
            constexpr int k = decltype(KK)::value;
            constexpr int bit = k * P;  // lane 0's position
            const int p = r + bit;
            word[bit / 32] |= negligible(se[p], sd[p], sd[p + 1]) ? (1u << (bit % 32)) : 0u;
        });
        M part = 0;
        static_for<WORDS>([&](auto WW) {
            constexpr int w = decltype(WW)::value;
            part |= (M)(word[w] << r) << (32 * w);
        });
        return chunk_or_mask<P>(part) & bits_below<M>(N - 1);
    }
}

template <int P, typename T>
__device__ __forceinline__ T chunk_max(T v) {
#pragma unroll
    for (int o = 1; o < P; o <<= 1) v = Fp<T>::max(v, __shfl_xor(v, o, 64));
    if constexpr (P == 64) {
        if constexpr (sizeof(T) == 4) {
            v = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
        } else {
            const long long b = __double_as_longlong(v);
            const int lo = __builtin_amdgcn_readfirstlane((int)b);
            const int hi = __builtin_amdgcn_readfirstlane((int)(b >> 32));
            v = __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
        }
    }
    return v;
}

// DENSE: the fused dense eigensolver, as in the chunked kernel with the band
// in registers: the wavefront's dense matrices are staged in LDS, each lane
// reduces its N/P consecutive rows of A with the identity rows of Q it
// holds, and the reduction leaves T's bands in the chunk's band slots, where
// the solve below starts from them.
template <typename T, int N, int P, bool WANTQ, bool PG, bool DENSE = false>
__global__ void __launch_bounds__(256) steqr_chunkl_kernel(KernelArgs args) {
    static_assert(P >= 2 && P <= N && (N % P) == 0 && (64 % P) == 0, "2 <= P <= N, P | N");
    static_assert(!DENSE || (64 / P) * N * N <= 64 * (N + 1),
                  "dense: the wavefront's matrices fit the staging area");
    static_assert(N <= 32, "position masks are 32 bits");
    constexpr int CH = 64 / P;
    constexpr int K = N / P;                       // positions per lane
    constexpr int R = WANTQ ? N / P : 0;           // rows of Q per lane
    constexpr int RQ = R > 0 ? R : 1;
    using M = uint32_t;
    using F = Fp<T>;
    using S = SmemL<T, N, P>;
    enum { ST_OPEN = 0, ST_ITER = 1, ST_DONE = 2 };

    extern __shared__ __align__(16) unsigned char smem_raw[];

    const T* __restrict__ gd = static_cast<const T*>(args.d);
    const T* __restrict__ ge = static_cast<const T*>(args.e);
    T* __restrict__ glam = static_cast<T*>(args.lam);
    T* __restrict__ gq = static_cast<T*>(args.q);
    const int n = args.n;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int chunk = lane / P;
    const int r = lane % P;
    const long prob = ((long)blockIdx.x * (blockDim.x >> 6) + wave) * CH + chunk;
    const bool live = prob < (long)args.batch;
    const long pb = live ? prob : (long)args.batch - 1;
    const bool writer = (r == 0);

    unsigned char* ws = smem_raw + (size_t)wave * S::bytes_per_wave;
    T* const sd = reinterpret_cast<T*>(ws) + chunk * S::SLOT;
    T* const se = sd + N;
    int* const srank = reinterpret_cast<int*>(ws + S::band_bytes) + chunk * N;
    T* const stage = reinterpret_cast<T*>(ws + S::band_bytes + S::rank_bytes);

    // ---------------------------------------------------------------- load
    // lane r of a chunk holds rows r, r+P, r+2P, ... of Q, so that the
    // chunk's lanes hold P consecutive rows in each row slice i
    T q[RQ][N];
    if constexpr (DENSE) {
        // one coalesced copy of the wavefront's matrices into the staging
        // area, each lane's rows of A (strict upper triangle mirrored from
        // the lower one) and identity rows of Q, then the reduction
        constexpr int RA = N / P;
        const T* __restrict__ ga = static_cast<const T*>(args.a);
        const int nn = n * n;
        const long first = ((long)blockIdx.x * (blockDim.x >> 6) + wave) * CH;
        const int nprob = (long)args.batch - first < CH ? (int)((long)args.batch - first) : CH;
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
            const int row = i * P + r;
            static_for<N>([&](auto J) {
                constexpr int j = decltype(J)::value;
                q[i][j] = (WANTQ & (row == j)) ? T(1) : T(0);
            });
        });
        // w goes through the chunk's e slot, e through its share of the
        // staging area (whose matrices are in registers now)
        T* const ez = stage + chunk * S::SLOT;
        T d0[N], e0[N];  // not used: the band stays in LDS
        householder_chunk<T, N, P, RA, WANTQ, RQ, true>(a, q, d0, e0, sd, se, ez, n, r);
        // the band in its slots, zero beyond the order as the tridiagonal
        // load leaves it
        static_for<K>([&](auto KK) {
            constexpr int k = decltype(KK)::value;
            const int p = r + k * P;
            const T dv = sd[p];
            sd[p] = (p < n) ? dv : T(0);
            se[p] = ez[p];
        });
    } else {
        static_for<K>([&](auto KK) {
            constexpr int k = decltype(KK)::value;
            const int p = r + k * P;
            const int pc = p < n ? p : n - 1;
            const T v = gd[pb * n + pc];
            sd[p] = (live & (p < n)) ? v : T(0);
            T w = T(0);
            if (n > 1) {
                const int ec = p < n - 1 ? p : n - 2;
                w = ge[pb * (n - 1) + ec];
            }
            se[p] = (live & (p < n - 1)) ? w : T(0);
        });
    }
    __builtin_amdgcn_wave_barrier();
    M zeromask;
    {
        M part = 0;
        static_for<K>([&](auto KK) {
            constexpr int k = decltype(KK)::value;
            const int p = r + k * P;
            part |= (se[p] == T(0)) ? ((M)1 << p) : (M)0;
        });
        zeromask = chunk_or<P>(part);
    }
    if constexpr (DENSE) {
        // Q holds the reduction's H_0 ... H_{n-2}
    } else if (WANTQ && args.back_transform) {
        // back-transformation [algo, eigenvector accumulation]: the rows of
        // the caller's basis instead of the identity
        const bool vec = (n == N) & ((reinterpret_cast<uintptr_t>(gq) & 15) == 0);
        static_for<RQ>([&](auto II) {
            constexpr int i = decltype(II)::value;
            load_basis_row<T, N>(gq + pb * n * n, n, i * P + r, live, true, vec, q[i]);
        });
    } else {
        static_for<RQ>([&](auto II) {
            constexpr int i = decltype(II)::value;
            const int row = i * P + r;
            static_for<N>([&](auto J) {
                constexpr int j = decltype(J)::value;
                q[i][j] = (WANTQ & (row == j)) ? T(1) : T(0);
            });
        });
    }

    // ST_OPEN: the chunk's next block is to be opened; ST_ITER: a block is
    // being reduced; ST_DONE: nothing left to reduce (a converged last block
    // may still wait for its close, `pending`). All lanes of a chunk hold
    // the same state, so chunk-wide shuffles inside these branches are safe.
    int state = live ? ST_OPEN : ST_DONE;
    int l1 = 0, bt = 0, bb = 0, m = 0, s = 0;
    int jtot = 0;
    const int nmaxit = (args.max_sweeps_per_n > 0 ? args.max_sweeps_per_n : 0) * n;
    bool mir = false, failed = false;
    bool last = false;     // no block follows the current one
    bool pending = false;  // converged last block, closed after the loop
    int mode = 0;
    T anorm = T(0);
    M zeroed = 0;
    int info = 0;

    // reverse the band of the chunk (lane-parallel) and Q's columns
    auto mirror_all = [&]() __attribute__((always_inline)) {
        T dv[K], ev[K];
        static_for<K>([&](auto KK) {
            constexpr int k = decltype(KK)::value;
            const int p = r + k * P;
            dv[k] = sd[N - 1 - p];
            ev[k] = se[p < N - 1 ? N - 2 - p : N - 1];
        });
        __builtin_amdgcn_wave_barrier();
        static_for<K>([&](auto KK) {
            constexpr int k = decltype(KK)::value;
            const int p = r + k * P;
            sd[p] = dv[k];
            se[p] = ev[k];
        });
        __builtin_amdgcn_wave_barrier();
        if constexpr (WANTQ) {
            static_for<RQ>([&](auto II) {
                constexpr int i = decltype(II)::value;
                static_for<N / 2>([&](auto I) {
                    constexpr int p = decltype(I)::value;
                    const T a = q[i][p];
                    q[i][p] = q[i][N - 1 - p];
                    q[i][N - 1 - p] = a;
                });
            });
        }
    };

    // Close the current block: zero the negligible e's found in it, undo the
    // scaling (d always, e too when the block failed), undo the mirror.
    auto close_block = [&](bool fail) __attribute__((always_inline)) {
        const T un = (mode == 1) ? anorm / F::ssfmax : ((mode == 2) ? anorm / F::ssfmin : T(1));
        static_for<K>([&](auto KK) {
            constexpr int k = decltype(KK)::value;
            const int p = r + k * P;
            T ev = se[p], dv = sd[p];
            ev = ((zeroed >> p) & 1) ? T(0) : ev;
            if (mode != 0) {
                dv = ((p >= bt) & (p <= bb)) ? dv * un : dv;
                ev = (fail & (p >= bt) & (p < bb)) ? ev * un : ev;
            }
            sd[p] = dv;
            se[p] = ev;
        });
        __builtin_amdgcn_wave_barrier();
        if (mir) mirror_all();
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
            T an = T(0);
            bool hasnan = false;
            static_for<K>([&](auto KK) {
                constexpr int k = decltype(KK)::value;
                const int p = r + k * P;
                const bool ind = (p >= lo) & (p <= hi);
                const bool ine = (p >= lo) & (p < hi);
                const T dv = sd[p], ev = se[p];
                an = ind ? F::max(an, F::abs(dv)) : an;
                an = ine ? F::max(an, F::abs(ev)) : an;
                hasnan = hasnan | (ind & (dv != dv)) | (ine & (ev != ev));
            });
            an = chunk_max<P>(an);
            hasnan = chunk_or<P>(hasnan ? 1u : 0u) != 0;
            anorm = hasnan ? F::qnan() : an;
            if (anorm == T(0)) continue;
            mode = (anorm > F::ssfmax) ? 1 : ((anorm < F::ssfmin) ? 2 : 0);
            if (mode != 0) {
                const T sg = ((mode == 1) ? F::ssfmax : F::ssfmin) / anorm;
                static_for<K>([&](auto KK) {
                    constexpr int k = decltype(KK)::value;
                    const int p = r + k * P;
                    const T dv = sd[p], ev = se[p];
                    sd[p] = ((p >= lo) & (p <= hi)) ? dv * sg : dv;
                    se[p] = ((p >= lo) & (p < hi)) ? ev * sg : ev;
                });
                __builtin_amdgcn_wave_barrier();
            }
            // converge the end of smaller magnitude first; a tie or NaN
            // converges the top end first, i.e. mirror
            mir = !(F::abs(sd[hi]) < F::abs(sd[lo]));
            if (mir) mirror_all();
            bt = mir ? N - 1 - hi : lo;
            bb = mir ? N - 1 - lo : hi;
            m = bb;
            zeroed = bt > 0 ? ((M)1 << (bt - 1)) : (M)0;  // zero coupling above
            state = ST_ITER;
        }
    };

    T x = T(0), y = T(0), dcur = T(0);  // running pair and current d_p of the chase
    while (true) {
        // ------------------------------------------------------------ settle
        // Opening and closing blocks are rare (once per block); they run
        // behind wavefront-wide tests. The per-pass part is straight-line.
        if (__any(state == ST_OPEN)) open_blocks();
        const bool iter = state == ST_ITER;
        if (!__any(iter)) break;
        // deflation test [algo, deflation], positions split over the chunk;
        // e's found negligible earlier count too
        const M neg = scan_negligible<T, N, P, M>(sd, se, r) | zeroed;
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
        // a failed block, or a converged block with another one after it
        const bool close_now = fail | (conv & !last);
        if (__any(close_now)) {
            if (close_now) {
                close_block(fail);
                if (fail) {
                    failed = true;
                    M part = 0;
                    static_for<K>([&](auto KK) {
                        constexpr int k = decltype(KK)::value;
                        const int p = r + k * P;
                        part |= ((p < n - 1) & (se[p] != T(0))) ? ((M)1 << p) : (M)0;
                    });
                    info = popc(chunk_or<P>(part));
                    info = info > 0 ? info : 1;
                }
                state = fail ? ST_DONE : ST_OPEN;
            }
        }
        // a converged last block is closed after the loop
        pending = pending | (conv & last);
        state = (conv & last) ? ST_DONE : state;
        // shift from the trailing 2x2 (LAPACK form) [algo, shift section];
        // running pair for the first rotation: (d_s - mu, e_s)
        const int mi = sweep ? m : (jac ? jpos + 1 : 1);
        const int si = sweep ? s : (jac ? jpos : 0);
        const T dm = sd[mi], dm1 = sd[mi - 1], em1 = se[mi - 1];
        const T mu = sweep_shift(args.shift_kind != 0, dm, dm1, em1);
        // EXP carries the pair (x, y) the next rotation annihilates; PG
        // carries g in x and the previous sine in y (f = y e_p)
        dcur = sd[si];
        x = dcur - mu;
        y = PG ? T(1) : se[si];
        // A 2x2 block at (jpos, jpos+1) [algo, 2x2 block
        // paragraph]: its closed-form Schur rotation becomes the running
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
        // window: (d0, e0) = original d_p, e_p; (d1, e1) = d_{p+1}, e_{p+1};
        // d_{p+2}, e_{p+2} are read at position p. No step writes a position
        // before the window has read it.
        T d0 = sd[0], e0 = se[0], d1 = sd[1], e1 = se[1];
        T cp = T(1);
        // chase at a raised issue priority, settle at the default one (as in
        // steqr_chunk.hpp)
        __builtin_amdgcn_s_setprio(1);
        // step p runs when s <= p < m: one unsigned compare of p - s with
        // the step count (0 when this chunk does not sweep)
        const unsigned steps = sweep ? (unsigned)(m - s) : (jac ? 1u : 0u);
        static_for<N - 1>([&](auto I) {
            constexpr int p = decltype(I)::value;
            T d2 = T(0), e2 = T(0);
            if constexpr (p + 2 < N) {
                d2 = sd[p + 2];
                e2 = se[p + 2];
            }
            if ((unsigned)(p - s) < steps) {
                // running pair and d_p seeded in the settle; r goes to
                // e_{p-1} (at the first step a zero coupling or an e already
                // in `zeroed`, restored when the block closes). Every lane of
                // the chunk writes the same value to the same word.
                T c, sn, rr;
                if constexpr (PG) {
                    // PG step [algo, update-scheme paragraph]; dcur holds
                    // g* = d_p - s' r*' (folded in by the previous step), and
                    // after the last step d_m - p and g are what the sweep's
                    // end writes back
                    const T f = y * e0;
                    const T b = cp * e0;
                    lartg(x, f, c, sn, rr);
                    const T gs = dcur;
                    const T rs = F::fma(d1 - gs, sn, (c + c) * b);
                    const T pk = sn * rs;
                    if constexpr (p > 0) se[p - 1] = rr;
                    sd[p] = gs + pk;
                    dcur = d1 - pk;
                    x = F::fma(c, rs, -b);
                    y = sn;
                    cp = c;
                } else {
                    // e0 already carries the factor c of the previous step
                    // (applied to the window below, so no cosine is carried)
                    const T a = dcur;
                    lartg(x, y, c, sn, rr);
                    const T b = e0;
                    const T w = exp_step_w(c, sn, a, b, d1);
                    if constexpr (p > 0) se[p - 1] = rr;
                    sd[p] = F::fma(sn, w, a);
                    dcur = F::fma(-sn, w, d1);
                    x = F::fma(c, w, -b);
                    y = sn * e1;
                    e1 = c * e1;
                }
                if constexpr (WANTQ) {
                    static_for<R>([&](auto II) {
                        constexpr int i = decltype(II)::value;
                        F::rot(q[i][p], q[i][p + 1], c, sn);
                    });
                }
            }
            d0 = d1;
            e0 = e1;
            d1 = d2;
            e1 = e2;
        });
        if (steps != 0u) {
            // the last step's d_{p+1} and e_p
            const int me = s + (int)steps;
            sd[me] = dcur;
            se[me - 1] = x;
        }
        __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_wave_barrier();
        // a NaN shift turns [s, m] into NaN, a fixed point of every further
        // sweep: spend the rest of the budget at once (same final state)
        jtot = (sweep & (mu != mu)) ? nmaxit : jtot;
    }
    // closes of converged last blocks, all at once
    if (__any(pending)) {
        if (pending) close_block(false);
    }

    // ---------------------------------------------------------------- sort
    __builtin_amdgcn_wave_barrier();
    const bool sort_it = (args.do_sort != 0) & !failed;
    // with no NaN among the wavefront's keys (a wave-uniform test) the
    // comparison drops its NaN terms, as in steqr_chunk.hpp
    bool nan_here = false;
    static_for<K>([&](auto KK) {
        constexpr int kk = decltype(KK)::value;
        const int j = r + kk * P;
        const T dj = sd[j];
        nan_here = nan_here | ((j < n) & (dj != dj));
    });
    const bool nonan = !__any(nan_here);
    T myd[K];
    int myrank[K];
    static_for<K>([&](auto KK) {
        constexpr int kk = decltype(KK)::value;
        const int j = r + kk * P;
        const T dj = sd[j];
        int rk = 0;
        if (nonan) {
            for (int k = 0; k < n; ++k) {
                const T dk = sd[k];
                rk += ((dk < dj) | ((dk == dj) & (k < j))) ? 1 : 0;
            }
        } else {
            const bool nanj = dj != dj;
            for (int k = 0; k < n; ++k) {
                const T dk = sd[k];
                const bool before =
                    (k < j) ? ((dk <= dj) | nanj) : ((dk < dj) | (nanj & (dk == dk)));
                rk += ((k != j) & before) ? 1 : 0;
            }
        }
        myd[kk] = dj;
        myrank[kk] = sort_it ? rk : j;
        srank[j] = myrank[kk];
    });
    __builtin_amdgcn_wave_barrier();

    // ---------------------------------------------------------------- store
    if (live) {
        static_for<K>([&](auto KK) {
            constexpr int kk = decltype(KK)::value;
            const int j = r + kk * P;
            if (j < n) glam[prob * n + myrank[kk]] = myd[kk];
        });
        if (args.info != nullptr && writer) args.info[prob] = info;
    }
    if constexpr (WANTQ) {
        // Row slice i: lane (chunk c, r) holds row i*P + r of its problem, so
        // the chunk's P rows are one contiguous range of its Q in HBM. Each
        // lane writes its row, columns permuted by rank, to its own LDS row
        // (stride N+1 against bank conflicts); then the wavefront copies the
        // slice out in 16-byte pieces, consecutive lanes at consecutive
        // addresses within each chunk's range.
        T* const myrow = stage + lane * S::STAGE_STRIDE;
        const long first = ((long)blockIdx.x * (blockDim.x >> 6) + wave) * CH;
        const bool vec = ((n & 3) == 0) & ((reinterpret_cast<uintptr_t>(gq) & 15) == 0);
        static_for<R>([&](auto II) {
            constexpr int i = decltype(II)::value;
            static_for<N>([&](auto J) {
                constexpr int j = decltype(J)::value;
                if (j < n) myrow[srank[j]] = q[i][j];
            });
            __builtin_amdgcn_wave_barrier();
            if (vec) {
                constexpr int V = 16 / sizeof(T);
                constexpr int PR = N / V;  // pieces per staged row
                static_for<PR>([&](auto KK) {
                    constexpr int k = decltype(KK)::value;
                    const int idx = k * 64 + lane;
                    const int L = idx / PR, c4 = idx % PR;  // source lane (row), piece
                    const int c = L / P, rr = L % P;
                    const long pr = first + c;
                    const int row = i * P + rr;
                    if ((pr < (long)args.batch) & (row < n) & (c4 * V < n)) {
                        const T* src = stage + L * S::STAGE_STRIDE + c4 * V;
                        T* dst = gq + (pr * n + row) * (long)n + c4 * V;
                        if constexpr (sizeof(T) == 4) {
                            *reinterpret_cast<float4*>(dst) = make_float4(src[0], src[1], src[2], src[3]);
                        } else {
                            *reinterpret_cast<double2*>(dst) = make_double2(src[0], src[1]);
                        }
                    }
                });
            } else {
                const int row = i * P + r;
                if (live & (row < n)) {
                    T* dst = gq + (prob * (long)n + row) * n;
                    static_for<N>([&](auto J) {
                        constexpr int j = decltype(J)::value;
                        if (j < n) dst[j] = myrow[j];
                    });
                }
            }
            __builtin_amdgcn_wave_barrier();
        });
    }
}

}  // namespace steqr
