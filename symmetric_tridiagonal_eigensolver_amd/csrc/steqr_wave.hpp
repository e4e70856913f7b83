// One-problem-per-wavefront steqr kernel for CDNA4 (gfx950, wave64): the
// P = 64 case, used for orders 33..64.
//
// With one problem per wavefront every decision of the solve is uniform
// across the wavefront, so the design differs from the chunked kernel:
//  * the band d, e lives in LDS (broadcast reads; every lane writes the
//    same words, so no lane mask); the chase reads the next position's
//    entries one step ahead, so the LDS latency overlaps the current
//    rotation;
//  * block bounds, the active part [s, m], the sweep counter and the status
//    are scalar (SGPR) values and every branch is a scalar branch;
//  * the deflation test runs on all lanes at once (lane i tests e_i) and one
//    ballot yields the whole position mask;
//  * lane i holds row i of Q in VGPRs; a rotation at position p updates
//    columns (p, p+1) of every row in one lane-parallel step.
// The per-problem operation sequence is the one of the chunked kernel and
// of the steqr algorithm page (see steqr_chunk.hpp for the citations).
#pragma once

#include "steqr_chunk.hpp"

namespace steqr {

template <typename T, int N>
struct WaveSmem {
    // d[N], e[N], then N ints of ranks
    static constexpr size_t bytes_per_wave = ((2 * N * sizeof(T) + N * sizeof(int) + 15) / 16) * 16;
};

__device__ __forceinline__ int uniform_int(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ unsigned long long wave_ballot(bool b) { return __ballot((int)b); }

template <typename T>
__device__ __forceinline__ T shfl_xor(T v, int mask) {
    const int lane = threadIdx.x & 63;
    const int src = ((lane ^ mask) & 63) << 2;
    if constexpr (sizeof(T) == 4) {
        return __builtin_bit_cast(T, __builtin_amdgcn_ds_bpermute(src, __builtin_bit_cast(int, v)));
    } else {
        const long long x = __builtin_bit_cast(long long, v);
        const int lo = __builtin_amdgcn_ds_bpermute(src, (int)(x & 0xffffffffll));
        const int hi = __builtin_amdgcn_ds_bpermute(src, (int)(x >> 32));
        return __builtin_bit_cast(T, ((long long)hi << 32) | (unsigned int)lo);
    }
}

template <typename T, int N, bool WANTQ, bool PG>
__global__ void __launch_bounds__(256) steqr_wave_kernel(KernelArgs args) {
    static_assert(N == 64, "one problem per wavefront needs N == 64");
    using F = Fp<T>;
    using M = uint64_t;

    const T* __restrict__ gd = static_cast<const T*>(args.d);
    const T* __restrict__ ge = static_cast<const T*>(args.e);
    T* __restrict__ glam = static_cast<T*>(args.lam);
    T* __restrict__ gq = static_cast<T*>(args.q);
    const int n = args.n;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const long prob = (long)blockIdx.x * (blockDim.x >> 6) + wave;
    if (prob >= (long)args.batch) return;  // whole wavefront leaves together

    extern __shared__ __align__(16) unsigned char smem_raw[];
    unsigned char* ws = smem_raw + (size_t)wave * WaveSmem<T, N>::bytes_per_wave;
    T* const sd = reinterpret_cast<T*>(ws);
    T* const se = sd + N;
    int* const srank = reinterpret_cast<int*>(se + N);

    // ---------------------------------------------------------------- load
    {
        const int lc = lane < n ? lane : n - 1;
        const T v = gd[prob * n + lc];
        sd[lane] = lane < n ? v : T(0);
        T w = T(0);
        if (n > 1) {
            const int ec = lane < n - 1 ? lane : n - 2;
            w = ge[prob * (n - 1) + ec];
        }
        se[lane] = lane < n - 1 ? w : T(0);
    }
    __builtin_amdgcn_wave_barrier();
    const M zeromask = wave_ballot(se[lane] == T(0));

    // lane = row of Q; the identity, or with back-transformation [algo,
    // eigenvector accumulation] the caller's basis
    T q[N];
    if (WANTQ && args.back_transform) {
        const bool vec = (n == N) & ((reinterpret_cast<uintptr_t>(args.q) & 15) == 0);
        load_basis_row<T, N>(static_cast<const T*>(args.q) + prob * n * n, n, lane, true, true,
                             vec, q);
    } else {
        static_for<N>([&](auto J) {
            constexpr int j = decltype(J)::value;
            q[j] = (WANTQ & (lane == j)) ? T(1) : T(0);
        });
    }

    enum { ST_OPEN = 0, ST_ITER = 1, ST_DONE = 2 };
    int state = ST_OPEN;
    int l1 = 0, bt = 0, bb = 0, m = 0, s = 0, jpos = -1;
    int jtot = 0;
    const int nmaxit = (args.max_sweeps_per_n > 0 ? args.max_sweeps_per_n : 0) * n;
    bool failed = false;
    int mir = 0, mode = 0;
    T anorm = T(0);
    M zeroed = 0;
    int info = 0;

    // reverse the band (positions p <-> N-1-p, e_p <-> e_{N-2-p}) and Q's
    // columns; uniform call
    auto mirror_all = [&]() __attribute__((always_inline)) {
        const T dv = sd[N - 1 - lane];
        const T ev = se[lane < N - 1 ? N - 2 - lane : N - 1];
        __builtin_amdgcn_wave_barrier();
        sd[lane] = dv;
        se[lane] = ev;
        __builtin_amdgcn_wave_barrier();
        if constexpr (WANTQ) {
            static_for<N / 2>([&](auto I) {
                constexpr int p = decltype(I)::value;
                const T a = q[p];
                q[p] = q[N - 1 - p];
                q[N - 1 - p] = a;
            });
        }
    };

    auto close_block = [&](bool fail) __attribute__((always_inline)) {
        // zero the negligible e's found in the block, undo scaling and mirror
        T ev = se[lane];
        ev = ((zeroed >> lane) & 1) ? T(0) : ev;
        T dv = sd[lane];
        if (mode != 0) {
            const T un = (mode == 1) ? anorm / F::ssfmax : anorm / F::ssfmin;
            dv = ((lane >= bt) & (lane <= bb)) ? dv * un : dv;
            ev = (fail & (lane >= bt) & (lane < bb)) ? ev * un : ev;
        }
        __builtin_amdgcn_wave_barrier();
        sd[lane] = dv;
        se[lane] = ev;
        __builtin_amdgcn_wave_barrier();
        if (mir) mirror_all();
        mir = 0;
        mode = 0;
        zeroed = 0;
    };

    while (true) {
        bool sweep = false, jac = false;
        T mu = T(0);
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
                const bool ind = (lane >= lo) & (lane <= hi);
                const bool ine = (lane >= lo) & (lane < hi);
                const T dv = sd[lane], ev = se[lane];
                T a = F::max(ind ? F::abs(dv) : T(0), ine ? F::abs(ev) : T(0));
                const bool nanl = (ind & (dv != dv)) | (ine & (ev != ev));
#pragma unroll
                for (int k = 1; k < 64; k <<= 1) a = F::max(a, shfl_xor(a, k));
                const bool anynan = wave_ballot(nanl) != 0;
                anorm = anynan ? F::qnan() : a;
                if (uniform_int(anorm == T(0))) continue;
                mode = uniform_int((anorm > F::ssfmax) ? 1 : ((anorm < F::ssfmin) ? 2 : 0));
                const T sg = (mode == 0) ? T(1) : ((mode == 1) ? F::ssfmax : F::ssfmin) / anorm;
                if (mode != 0) {
                    __builtin_amdgcn_wave_barrier();
                    sd[lane] = ind ? dv * sg : dv;
                    se[lane] = ine ? ev * sg : ev;
                    __builtin_amdgcn_wave_barrier();
                }
                mir = uniform_int(!(F::abs(sd[hi]) < F::abs(sd[lo])));
                if (mir) mirror_all();
                bt = mir ? N - 1 - hi : lo;
                bb = mir ? N - 1 - lo : hi;
                m = bb;
                zeroed = bt > 0 ? ((M)1 << (bt - 1)) : (M)0;  // zero coupling above
                state = ST_ITER;
            }
            // deflation test: lane i tests e_i between d_i and d_{i+1}
            const T di = sd[lane], ei = se[lane];
            const T dn = sd[lane < N - 1 ? lane + 1 : N - 1];
            const M neg = wave_ballot(negligible(ei, di, dn)) | zeroed;
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
                const M nz = wave_ballot(se[lane] != T(0));
                info = popc((M)(nz & bits_below<M>(n - 1)));
                info = info > 0 ? info : 1;
                state = ST_DONE;
                break;
            }
            ++jtot;
            mu = sweep_shift(args.shift_kind != 0, sd[m], sd[m - 1], se[m - 1]);
            sweep = true;
            break;
        }
        if (state == ST_DONE) break;

        if (sweep | jac) {
            // chase over [s, me - 1]. Carried: dcur = current d_p (updated by
            // the previous step), ecur = original e_p, cp = previous cosine
            // (the update e_p <- c_{p-1} e_p is applied here), (x, y) =
            // running pair. d_{p+1}, e_{p+1} are read one step ahead: no step
            // writes them before step p.
            T dcur = sd[s], ecur = se[s];
            T x, y;
            int me = m;
            if (jac) {
                // A 2x2 block at (jpos, jpos+1) [algo, 2x2 block paragraph],
                // as in the chunked kernels: its closed-form Schur rotation
                // seeds a one-step chase at jpos (lartg returns that rotation;
                // for PG from (cs e, -sj e)), so the similarity and the Q
                // update are those of the sweeps, and every kernel family
                // computes the same bits. The leftover e_jpos (rounding size)
                // joins `zeroed`; s == jpos here.
                T rt1, rt2, cs, sj;
                sym2x2(dcur, ecur, sd[jpos + 1], rt1, rt2, cs, sj);
                x = PG ? cs * ecur : cs;
                y = -sj;
                me = jpos + 1;
                zeroed |= (M)1 << jpos;
            } else {
                // running pair (d_s - mu, e_s) for the first rotation (PG: g
                // in x, the previous sine in y)
                x = dcur - mu;
                y = PG ? T(1) : ecur;
            }
            T cp = T(1);
            T dnext = sd[s + 1], enext = se[s + 1];
            // positions s .. me-1; the walk stops after me-1 (uniform branch)
            static_for_while<N - 1>([&](auto I) {
                constexpr int p = decltype(I)::value;
                if (p >= s) {
                    // r goes to e_{p-1}: at the first step a zero coupling or
                    // an e already in `zeroed`, restored when the block closes
                    const T dp1 = dnext, ep1 = enext;
                    if constexpr (p + 2 < N) {
                        dnext = sd[p + 2];
                        enext = se[p + 2];
                    }
                    const T ep = ecur;
                    T c, sn, rr;
                    if constexpr (PG) {
                        // PG step [algo, update-scheme paragraph]; dcur
                        // holds g* (see steqr_chunk.hpp)
                        const T f = y * ep;
                        const T b = cp * ep;
                        lartg<T, true>(x, f, c, sn, rr);
                        if constexpr (p > 0) se[p - 1] = rr;  // every lane writes the same word
                        const T gs = dcur;
                        const T rs = F::fma(dp1 - gs, sn, (c + c) * b);
                        const T pk = sn * rs;
                        sd[p] = gs + pk;
                        dcur = dp1 - pk;
                        x = F::fma(c, rs, -b);
                        y = sn;
                    } else {
                        const T a = dcur;
                        lartg<T, true>(x, y, c, sn, rr);
                        if constexpr (p > 0) se[p - 1] = rr;  // every lane writes the same word
                        const T b = cp * ep;
                        const T w = exp_step_w(c, sn, a, b, dp1);
                        sd[p] = F::fma(sn, w, a);
                        dcur = F::fma(-sn, w, dp1);
                        x = F::fma(c, w, -b);
                        y = sn * ep1;  // new bulge
                    }
                    cp = c;
                    ecur = ep1;
                    if constexpr (WANTQ) {
                        F::rot(q[p], q[p + 1], c, sn);
                    }
                }
                return p + 1 < me;
            });
            sd[me] = dcur;
            se[me - 1] = x;
            __builtin_amdgcn_wave_barrier();
            if (sweep && uniform_int(mu != mu)) jtot = nmaxit;
        }
    }

    // ---------------------------------------------------------------- sort
    const T dmine = sd[lane];
    const bool sort_it = (args.do_sort != 0) & !failed;
    int rk = 0;
    {
        const bool nanj = dmine != dmine;
        for (int k = 0; k < n; ++k) {
            const T dk = sd[k];
            const bool before = (k < lane) ? ((dk <= dmine) | nanj)
                                           : ((dk < dmine) | (nanj & (dk == dk)));
            rk += ((k != lane) & before) ? 1 : 0;
        }
    }
    rk = sort_it ? rk : lane;
    srank[lane] = rk;
    __builtin_amdgcn_wave_barrier();
    if (lane < n) glam[prob * n + rk] = dmine;
    if constexpr (WANTQ) {
        if (lane < n) {
            T* qrow = gq + prob * (long)n * n + (long)lane * n;
            static_for<N>([&](auto J) {
                constexpr int j = decltype(J)::value;
                if (j < n) qrow[srank[j]] = q[j];
            });
        }
    }
    if (args.info != nullptr && lane == 0) args.info[prob] = info;
}

}  // namespace steqr
