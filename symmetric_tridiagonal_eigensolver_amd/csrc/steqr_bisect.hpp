// Eigenvalue-only bisection kernel for CDNA4 (gfx950, wave64): the values
// mode of the pages' stebz (BatchLAS syev routing and tuning page: bisection
// for the indices 0..n-1 in ascending order, straight off the tridiagonal;
// exits on the tolerance, the halving budget or a stalled midpoint).
//
// Design (MI355X-first). One problem per chunk of N lanes (N = the padded
// order; from order 128 one problem per wavefront with N / 64 indices per
// lane, k, k + 64, ..., or spread over G wavefronts of one workgroup with
// N / (64 G) indices each), one eigenvalue index per lane: lane k of a chunk
// bisects the k-th smallest eigenvalue with Sturm counts of its own, so the
// 64 lanes of a wavefront run 64 independent bisections in lockstep with no
// exchange at all after the set-up. With G wavefronts per problem every
// wavefront repeats the (cheap) set-up over the whole band and bisects its
// own share of the indices; the status sums the shares through LDS. Every
// bisection takes about the same number of halvings (the interval starts
// as the Gershgorin interval and ends at a few ulps of ||T||), so lockstep
// costs little; a lane that has converged is masked off until every lane
// of the wavefront has.
//
// Set-up per chunk (lane k handles position k): the Gershgorin norm
// max |e_{k-1}| + |d_k| + |e_k| by a butterfly (NaN-propagating), the exact
// power-of-two prescaling 2^-ceil(log2 ||T||), the scaled band published to
// LDS, pivmin = safmin max(1, max e^2) and the Gershgorin interval widened
// by 2 n ulp ||T|| + 2 pivmin, the tolerance max(ulp ||T||, 2 ulp max(|lo|,
// |hi|)) and the budget floor(log2((||T|| + pivmin)/pivmin)) + 2 halvings.
// The count q_1 = d_1 - x, q_i = (d_i - x) - e_{i-1}^2 / q_{i-1} (|q_i| <
// pivmin replaced by -pivmin), count = #{q_i < 0}, uses the hardware
// reciprocal (one third-order step in double); the band sits in VGPRs, or in LDS
// for double at order 64. Status: the number of indices that ran out of
// halvings; a NaN gives NaN eigenvalues and status n; T = 0 gives zeros.
#pragma once

#include "steqr_chunk.hpp"

namespace steqr {

template <typename T, int N>
struct SmemB {
    static constexpr int CH = N < 64 ? 64 / N : 1;
    // the chunks' scaled bands, then one int (the wavefront's failed
    // indices, for G wavefronts per problem)
    static constexpr size_t bytes_per_wave = (size_t)CH * 2 * N * sizeof(T) + 16;
};

// Butterfly over the N lanes of a chunk.
template <int N, typename T>
__device__ __forceinline__ T chunk_maxf(T v) {
#pragma unroll
    for (int o = 1; o < N; o <<= 1) v = Fp<T>::max(v, __shfl_xor(v, o, 64));
    return v;
}
template <int N, typename T>
__device__ __forceinline__ T chunk_minf(T v) {
#pragma unroll
    for (int o = 1; o < N; o <<= 1) v = -Fp<T>::max(-v, -__shfl_xor(v, o, 64));
    return v;
}
template <int N>
__device__ __forceinline__ int chunk_sumi(int v) {
#pragma unroll
    for (int o = 1; o < N; o <<= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// 1/x for the Sturm count. Double: the hardware seed y (relative error
// below 2^-24.3, measured on MI355X over 4M inputs of either sign and
// exponents -900..900) and one third-order step y (1 + r + r^2) with
// r = 1 - x y, whose error is O(r^3) < 2^-72 plus rounding: three dependent
// operations where two Newton steps take four. Float: the hardware
// reciprocal alone.
template <typename T>
__device__ __forceinline__ T sturm_rcp(T x) {
    if constexpr (sizeof(T) == 4) {
        return Fp<T>::rcp(x);
    } else {
        const double y = __builtin_amdgcn_rcp(x);
        const double r = __builtin_fma(-x, y, 1.0);
        return __builtin_fma(y, __builtin_fma(r, r, r), y);
    }
}

template <typename T, int N, int G = 1>
__global__ void __launch_bounds__(G > 1 ? 64 * G : 256) steqr_bisect_kernel(KernelArgs args) {
    // L lanes per wavefront and problem, E = N / L positions per lane for
    // the set-up (k, k + L, ...): one up to order 64, two at 128, four at
    // 256, eight at 512; the G wavefronts of a problem bisect EB = E / G
    // indices per lane each (wavefront g: k0 + (g EB + j) L, j < EB)
    constexpr int L = N < 64 ? N : 64;
    constexpr int E = N / L;
    constexpr int EB = E / G;
    static_assert(N >= 2 && N <= 512 && (64 % L) == 0 && E * L == N, "lanes per position");
    static_assert(G >= 1 && EB * G == E && (G == 1 || L == 64), "wavefronts per problem");
    using F = Fp<T>;
    using S = SmemB<T, N>;
    constexpr int CH = 64 / L;
    // band in VGPRs unless it would take more than 128 of them
    constexpr bool REGS = 2 * N * (int)sizeof(T) / 4 <= 128;
    constexpr T ulp = sizeof(T) == 4 ? T(0x1p-23) : T(0x1p-52);

    extern __shared__ __align__(16) unsigned char smem_raw[];
    const T* __restrict__ gd = static_cast<const T*>(args.d);
    const T* __restrict__ ge = static_cast<const T*>(args.e);
    T* __restrict__ glam = static_cast<T*>(args.lam);
    const int n = args.n;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int chunk = lane / L;
    const int k0 = lane % L;  // first position / eigenvalue index of this lane
    const int grp = wave % G;  // this wavefront's share of the indices
    const long prob = ((long)blockIdx.x * ((blockDim.x >> 6) / G) + wave / G) * CH + chunk;
    const bool live = prob < (long)args.batch;
    const long pb = live ? prob : (long)args.batch - 1;
    T* const sdd = reinterpret_cast<T*>(smem_raw + (size_t)wave * S::bytes_per_wave) + chunk * 2 * N;
    T* const se2 = sdd + N;
    const T inf = T(__builtin_inff());

    // ------------------------------------------------------------ set-up
    T dk[E], ek[E], ekm[E];
    bool hasd[E];
    T rmax = T(0);
    int nan_here = 0;
    static_for<E>([&](auto J) {
        constexpr int j = decltype(J)::value;
        const int k = k0 + j * L;
        hasd[j] = live & (k < n);
        dk[j] = ek[j] = ekm[j] = T(0);
        if (hasd[j]) dk[j] = gd[pb * n + k];
        if (live & (k < n - 1)) ek[j] = ge[pb * (n - 1) + k];
        if (hasd[j] & (k >= 1)) ekm[j] = ge[pb * (n - 1) + k - 1];
        const T rk = F::abs(ekm[j]) + F::abs(dk[j]) + F::abs(ek[j]);
        nan_here |= (rk != rk) ? 1 : 0;
        rmax = F::max(rmax, rk);
    });
    // NaN anywhere in the band (the butterflies below use fmax, which
    // drops NaNs, so they are counted on their own)
    const int nnan = chunk_sumi<L>(nan_here);
    const T tn = chunk_maxf<L>(rmax);
    const bool zero = (nnan == 0) & (tn == T(0));
    const bool bad = nnan != 0;
    // exact power-of-two prescaling: tn * s in [0.5, 1)
    const int ex = (bad | zero) ? 0 : F::frexp_exp(tn);
    const T s = F::ldexp(T(1), -ex);
    T e2loc = T(0), gl_loc = inf, gu_loc = -inf, tn_loc = T(0);
    static_for<E>([&](auto J) {
        constexpr int j = decltype(J)::value;
        const int k = k0 + j * L;
        const T ds = dk[j] * s;
        const T es = ek[j] * s;
        const T esm = ekm[j] * s;
        const T e2 = es * es;
        sdd[k] = ds;
        se2[k] = e2;
        e2loc = F::max(e2loc, e2);
        // Gershgorin interval over positions 0..n-1 (padding neutral)
        const T rad = F::abs(esm) + F::abs(es);
        gl_loc = hasd[j] ? -F::max(-gl_loc, -(ds - rad)) : gl_loc;
        gu_loc = hasd[j] ? F::max(gu_loc, ds + rad) : gu_loc;
        tn_loc = hasd[j] ? F::max(tn_loc, F::abs(ds) + rad) : tn_loc;
    });
    __builtin_amdgcn_wave_barrier();
    const T e2max = chunk_maxf<L>(e2loc);
    const T pivmin = F::safmin * F::max(T(1), e2max);
    const T gl0 = chunk_minf<L>(gl_loc);
    const T gu0 = chunk_maxf<L>(gu_loc);
    const T tns = chunk_maxf<L>(tn_loc);
    const T widen = T(2) * T(n) * ulp * tns + T(2) * pivmin;
    const T atol = ulp * tns;
    // floor(log2(r)) = e - 1 for r = f 2^e, f in [0.5, 1): exact
    // (at most 1,024 for a finite band, whose norm is scaled to [0.5, 1);
    // an infinite entry makes the ratio infinite or NaN, and the bound keeps
    // the loop finite whatever the exponent instruction returns for those)
    const int itraw =
        __builtin_amdgcn_frexp_exp(((double)tns + (double)pivmin) / (double)pivmin) + 1;
    const int itmax = itraw < 1 ? 1 : (itraw > 1100 ? 1100 : itraw);

    T bd[REGS ? N : 1], be2[REGS ? N : 1];
    if constexpr (REGS) {
        static_for<N>([&](auto I) {
            constexpr int i = decltype(I)::value;
            bd[i] = sdd[i];
            be2[i] = se2[i];
        });
    }

    // Sturm counts of the scaled band below x[0..EB) in one traversal
    auto count = [&](const T (&x)[EB], int (&c)[EB]) __attribute__((always_inline)) {
        T q[EB];
        static_for<EB>([&](auto J) { c[decltype(J)::value] = 0; });
        static_for_while<N>([&](auto I) {
            constexpr int i = decltype(I)::value;
            const T di = REGS ? bd[i] : sdd[i];
            T ei = T(0);
            if constexpr (i > 0) ei = REGS ? be2[i - 1] : se2[i - 1];
            static_for<EB>([&](auto J) {
                constexpr int j = decltype(J)::value;
                if constexpr (i == 0) {
                    q[j] = di - x[j];
                } else {
                    q[j] = F::fma(-ei, sturm_rcp(q[j]), di - x[j]);
                }
                q[j] = (F::abs(q[j]) < pivmin) ? -pivmin : q[j];
                c[j] += (q[j] < T(0)) ? 1 : 0;
            });
            return i + 1 < n;  // uniform
        });
    };

    // ------------------------------------------------------------ bisection
    // index k0 + (grp EB + j) L of the lane's share
    bool mine[EB];
    static_for<EB>([&](auto J) {
        constexpr int j = decltype(J)::value;
        mine[j] = live & (k0 + (grp * EB + j) * L < n);
    });
    T lo[EB], hi[EB];
    bool done[EB];
    int fail = 0, it[EB];
    bool any_open = false;
    static_for<EB>([&](auto J) {
        constexpr int j = decltype(J)::value;
        lo[j] = gl0 - widen;
        hi[j] = gu0 + widen;
        done[j] = !mine[j] | bad | zero;
        it[j] = 0;
        any_open |= !done[j];
    });
    while (__builtin_amdgcn_ballot_w64(any_open)) {
        if (any_open) {
            T mid[EB];
            bool step[EB];
            static_for<EB>([&](auto J) {
                constexpr int j = decltype(J)::value;
                step[j] = false;
                mid[j] = (lo[j] + hi[j]) * T(0.5);
                if (!done[j]) {
                    const T big = F::max(F::abs(lo[j]), F::abs(hi[j]));
                    const T tol = F::max(T(2) * ulp * big, atol);
                    if (hi[j] - lo[j] <= tol) {
                        done[j] = true;
                    } else if (it[j] == itmax) {
                        done[j] = true;
                        fail += 1;
                    } else if ((mid[j] == lo[j]) | (mid[j] == hi[j])) {
                        done[j] = true;
                    } else {
                        step[j] = true;
                    }
                }
            });
            bool any_step = false;
            static_for<EB>([&](auto J) { any_step |= step[decltype(J)::value]; });
            if (any_step) {
                int c[EB];
                count(mid, c);
                static_for<EB>([&](auto J) {
                    constexpr int j = decltype(J)::value;
                    const int k = k0 + (grp * EB + j) * L;
                    if (step[j]) {
                        if (c[j] <= k)
                            lo[j] = mid[j];
                        else
                            hi[j] = mid[j];
                        ++it[j];
                    }
                });
            }
            any_open = false;
            static_for<EB>([&](auto J) { any_open |= !done[decltype(J)::value]; });
        }
    }

    // ------------------------------------------------------------ store
    const T us = F::ldexp(T(1), ex);
    static_for<EB>([&](auto J) {
        constexpr int j = decltype(J)::value;
        T lam = ((lo[j] + hi[j]) * T(0.5)) * us;
        lam = zero ? T(0) : lam;
        lam = bad ? F::qnan() : lam;
        if (mine[j]) glam[prob * n + k0 + (grp * EB + j) * L] = lam;
    });
    int nfail = chunk_sumi<L>(fail);
    if constexpr (G > 1) {
        // the G wavefronts of the problem (consecutive in the workgroup)
        // add their counts through LDS; every wavefront reaches the barrier
        int* const fl = reinterpret_cast<int*>(smem_raw + (size_t)(wave + 1) * S::bytes_per_wave) - 4;
        if (lane == 0) fl[0] = nfail;
        __syncthreads();
        nfail = 0;
        static_for<G>([&](auto GG) {
            constexpr int gg = decltype(GG)::value;
            nfail += reinterpret_cast<const int*>(
                smem_raw + (size_t)(wave - grp + gg + 1) * S::bytes_per_wave)[-4];
        });
    }
    if (live & (grp == 0) & (k0 == 0) & (args.info != nullptr)) args.info[prob] = bad ? n : nfail;
}

}  // namespace steqr
