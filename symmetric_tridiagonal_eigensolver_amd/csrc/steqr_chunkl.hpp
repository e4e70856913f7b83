// Chunked steqr kernel with the band in LDS (gfx950, wave64).
//
// Same per-problem algorithm and lockstep pass structure as
// steqr_chunk.hpp (one problem per chunk of P lanes, Q rows in VGPRs,
// mirrored blocks so every chunk chases top to bottom), but the band d, e of
// each chunk lives in LDS instead of being replicated in every lane's
// VGPRs. That frees 2N VGPRs per lane, which is what lets a lane hold more
// rows of Q (fewer lanes per problem, less repeated chase arithmetic) at a
// usable occupancy for N = 32, and it lets the lanes of a chunk share the
// settle-phase work:
//  * the deflation scan, the block norm, the scaling, the mirror and the
//    sort keys are split over the P lanes of the chunk (lane r handles
//    positions r, r+P, ...) and combined with butterfly shuffles;
//  * the chase reads d_{p+2}, e_{p+2} at position p (a two-deep window), so
//    the LDS latency overlaps the rotation; one lane per chunk writes back
//    the final d_p and e_{p-1};
//  * Q is written through an LDS slice per row index, so each output row is
//    written contiguously (a full cache line per row) after the column
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

// OR / max over the P lanes of a chunk (butterfly; every lane of the chunk
// must be active, which holds because a chunk's lanes share control flow).
template <int P>
__device__ __forceinline__ unsigned chunk_or(unsigned v) {
#pragma unroll
    for (int o = 1; o < P; o <<= 1) v |= (unsigned)__shfl_xor((int)v, o, 64);
    return v;
}
template <int P, typename T>
__device__ __forceinline__ T chunk_max(T v) {
#pragma unroll
    for (int o = 1; o < P; o <<= 1) v = Fp<T>::max(v, __shfl_xor(v, o, 64));
    return v;
}

template <typename T, int N, int P, bool WANTQ>
__global__ void __launch_bounds__(256) steqr_chunkl_kernel(KernelArgs args) {
    static_assert(P >= 2 && P <= N && (N % P) == 0 && (64 % P) == 0, "2 <= P <= N, P | N");
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
    T q[RQ][N];
    static_for<RQ>([&](auto II) {
        constexpr int i = decltype(II)::value;
        const int row = r * R + i;
        static_for<N>([&](auto J) {
            constexpr int j = decltype(J)::value;
            q[i][j] = (WANTQ & (row == j)) ? T(1) : T(0);
        });
    });

    int state = live ? ST_OPEN : ST_DONE;
    int l1 = 0, bt = 0, bb = 0, m = 0, s = 0, jpos = -1;
    int jtot = 0;
    const int nmaxit = (args.max_sweeps_per_n > 0 ? args.max_sweeps_per_n : 0) * n;
    bool mir = false, failed = false;
    int mode = 0;
    T anorm = T(0);
    M zeroed = 0;
    int info = 0;
    T mu = T(0);

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

    T x = T(0), y = T(0), dcur = T(0);  // running pair and current d_p of the chase
    while (state != ST_DONE) {
        bool sweep = false, jac = false;
        // ------------------------------------------------------------ settle
        while (true) {
            if (state == ST_OPEN) {
                const M avail = ~zeromask & ~bits_below<M>(l1) & bits_below<M>(n - 1);
                if (avail == 0) {
                    state = ST_DONE;
                    break;
                }
                const int lo = lsb(avail);
                const int hi = lsb((M)(zeromask & ~bits_below<M>(lo)));
                l1 = hi + 1;
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
                mir = !(F::abs(sd[hi]) < F::abs(sd[lo]));
                if (mir) mirror_all();
                bt = mir ? N - 1 - hi : lo;
                bb = mir ? N - 1 - lo : hi;
                m = bb;
                zeroed = bt > 0 ? ((M)1 << (bt - 1)) : (M)0;  // zero coupling above
                state = ST_ITER;
            }
            // deflation test [algo, deflation], positions split over the chunk
            M neg;
            {
                M part = 0;
                static_for<K>([&](auto KK) {
                    constexpr int k = decltype(KK)::value;
                    const int p = r + k * P;
                    if (p < N - 1)
                        part |= negligible(se[p], sd[p], sd[p + 1 < N ? p + 1 : N - 1])
                                    ? ((M)1 << p) : (M)0;
                });
                neg = chunk_or<P>(part) | zeroed;
            }
            const M rng = bit_range<M>(bt, m - 1);
            const M nb = neg & rng;
            const M clr = rng & ~neg;
            if (clr == 0) {
                zeroed |= nb;
                close_block(false);
                state = ST_OPEN;
                continue;
            }
            const int t = msb(clr);
            zeroed |= nb & bit_range<M>(t + 1, m - 1);
            m = t + 1;
            const M above = nb & bit_range<M>(bt, t - 1);
            s = above ? msb(above) + 1 : bt;
            if (above) zeroed |= (M)1 << (s - 1);
            if (m - s == 1) {
                jac = true;
                jpos = s;
                m = s - 1;
                break;
            }
            if (jtot >= nmaxit) {
                failed = true;
                close_block(true);
                M part = 0;
                static_for<K>([&](auto KK) {
                    constexpr int k = decltype(KK)::value;
                    const int p = r + k * P;
                    part |= ((p < n - 1) & (se[p] != T(0))) ? ((M)1 << p) : (M)0;
                });
                info = popc(chunk_or<P>(part));
                info = info > 0 ? info : 1;
                state = ST_DONE;
                break;
            }
            ++jtot;
            mu = lapack_shift(sd[m], sd[m - 1], se[m - 1]);
            dcur = sd[s];
            x = dcur - mu;
            y = se[s];
            sweep = true;
            break;
        }
        if (state == ST_DONE) break;

        // ------------------------------------------------------------ chase pass
        // window: (d0, e0) = original d_p, e_p; (d1, e1) = d_{p+1}, e_{p+1};
        // d_{p+2}, e_{p+2} are read at position p. No step writes a position
        // before the window has read it.
        T d0 = sd[0], e0 = se[0], d1 = sd[1], e1 = se[1];
        T cp = T(1);
        // step p runs when s <= p < m: one unsigned compare of p - s with
        // the step count (0 when this chunk does not sweep)
        const unsigned steps = sweep ? (unsigned)(m - s) : 0u;
        const int jat = jac ? jpos : -1;  // position of this chunk's 2x2 solve
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
                // in `zeroed`, restored when the block closes)
                const T a = dcur;
                T c, sn, rr;
                lartg(x, y, c, sn, rr);
                const T b = cp * e0;
                const T pp = c * a + sn * b;
                const T qq = c * b + sn * d1;
                const T an = pp * c + qq * sn;
                const T bn = qq * c - pp * sn;
                // every lane of the chunk writes the same value to the same word
                if constexpr (p > 0) se[p - 1] = rr;
                sd[p] = an;
                dcur = (a + d1) - an;
                x = bn;
                y = sn * e1;
                cp = c;
                if constexpr (WANTQ) {
                    static_for<R>([&](auto II) {
                        constexpr int i = decltype(II)::value;
                        F::rot(q[i][p], q[i][p + 1], c, sn);
                    });
                }
            }
            if (p == jat) {
                T rt1, rt2, cs, sj;
                sym2x2(d0, e0, d1, rt1, rt2, cs, sj);
                sd[p] = rt1;
                sd[p + 1] = rt2;
                se[p] = T(0);
                if constexpr (WANTQ) {
                    static_for<R>([&](auto II) {
                        constexpr int i = decltype(II)::value;
                        F::rot(q[i][p], q[i][p + 1], cs, -sj);
                    });
                }
            }
            d0 = d1;
            e0 = e1;
            d1 = d2;
            e1 = e2;
        });
        if (sweep & writer) {
            sd[m] = dcur;
            se[m - 1] = x;
        }
        __builtin_amdgcn_wave_barrier();
        if (sweep & (mu != mu)) jtot = nmaxit;
    }

    // ---------------------------------------------------------------- sort
    __builtin_amdgcn_wave_barrier();
    const bool sort_it = (args.do_sort != 0) & !failed;
    T myd[K];
    int myrank[K];
    static_for<K>([&](auto KK) {
        constexpr int kk = decltype(KK)::value;
        const int j = r + kk * P;
        const T dj = sd[j];
        const bool nanj = dj != dj;
        int rk = 0;
        for (int k = 0; k < n; ++k) {
            const T dk = sd[k];
            const bool before = (k < j) ? ((dk <= dj) | nanj) : ((dk < dj) | (nanj & (dk == dk)));
            rk += ((k != j) & before) ? 1 : 0;
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
        // slice i: row r*R + i of every chunk, columns permuted by rank,
        // staged in LDS then written row by row (a row is contiguous in HBM)
        T* const myrow = stage + lane * S::STAGE_STRIDE;
        const long qbase = prob * (long)n * n;
        static_for<R>([&](auto II) {
            constexpr int i = decltype(II)::value;
            const int row = r * R + i;
            static_for<N>([&](auto J) {
                constexpr int j = decltype(J)::value;
                if (j < n) myrow[srank[j]] = q[i][j];
            });
            __builtin_amdgcn_wave_barrier();
            if (live & (row < n)) {
                T* dst = gq + qbase + (long)row * n;
                static_for<N>([&](auto J) {
                    constexpr int j = decltype(J)::value;
                    if (j < n) dst[j] = myrow[j];
                });
            }
            __builtin_amdgcn_wave_barrier();
        });
    }
}

}  // namespace steqr
