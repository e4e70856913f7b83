// Eigenvalue-only bisection kernel for CDNA4 (gfx950, wave64): the values
// mode of the pages' stebz (BatchLAS syev routing and tuning page: bisection
// for the indices 0..n-1 in ascending order, straight off the tridiagonal;
// exits on the tolerance, the halving budget or a stalled midpoint).
//
// Design (MI355X-first). One problem per chunk of N lanes (N = the padded
// order), one eigenvalue index per lane: lane k of a chunk bisects the k-th
// smallest eigenvalue with Sturm counts of its own, so the 64 lanes of a
// wavefront run 64 independent bisections in lockstep with no exchange at
// all after the set-up. Every bisection takes about the same number of
// halvings (the interval starts as the Gershgorin interval and ends at a
// few ulps of ||T||), so lockstep costs little; a lane that has converged
// is masked off until every lane of the wavefront has.
//
// Set-up per chunk (lane k handles position k): the Gershgorin norm
// max |e_{k-1}| + |d_k| + |e_k| by a butterfly (NaN-propagating), the exact
// power-of-two prescaling 2^-ceil(log2 ||T||), the scaled band published to
// LDS, pivmin = safmin max(1, max e^2) and the Gershgorin interval widened
// by 2 n ulp ||T|| + 2 pivmin, the tolerance max(ulp ||T||, 2 ulp max(|lo|,
// |hi|)) and the budget floor(log2((||T|| + pivmin)/pivmin)) + 2 halvings.
// The count q_1 = d_1 - x, q_i = (d_i - x) - e_{i-1}^2 / q_{i-1} (|q_i| <
// pivmin replaced by -pivmin), count = #{q_i < 0}, uses the hardware
// reciprocal (Newton-refined in double); the band sits in VGPRs, or in LDS
// for double at order 64. Status: the number of indices that ran out of
// halvings; a NaN gives NaN eigenvalues and status n; T = 0 gives zeros.
#pragma once

#include "steqr_chunk.hpp"

namespace steqr {

template <typename T, int N>
struct SmemB {
    static constexpr int CH = 64 / N;
    static constexpr size_t bytes_per_wave = (size_t)CH * 2 * N * sizeof(T);
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

template <typename T, int N>
__global__ void __launch_bounds__(256) steqr_bisect_kernel(KernelArgs args) {
    static_assert(N >= 2 && N <= 64 && (64 % N) == 0, "one lane per position");
    using F = Fp<T>;
    using S = SmemB<T, N>;
    constexpr int CH = 64 / N;
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
    const int chunk = lane / N;
    const int k = lane % N;  // position / eigenvalue index of this lane
    const long prob = ((long)blockIdx.x * (blockDim.x >> 6) + wave) * CH + chunk;
    const bool live = prob < (long)args.batch;
    const long pb = live ? prob : (long)args.batch - 1;
    T* const sdd = reinterpret_cast<T*>(smem_raw + (size_t)wave * S::bytes_per_wave) + chunk * 2 * N;
    T* const se2 = sdd + N;

    // ------------------------------------------------------------ set-up
    const bool hasd = live & (k < n);
    const bool hase = live & (k < n - 1);
    T dk = T(0), ek = T(0), ekm = T(0);
    if (hasd) dk = gd[pb * n + k];
    if (hase) ek = ge[pb * (n - 1) + k];
    if (hasd & (k >= 1)) ekm = ge[pb * (n - 1) + k - 1];
    const T rk = F::abs(ekm) + F::abs(dk) + F::abs(ek);
    // NaN anywhere in the band (the butterflies below use fmax, which
    // drops NaNs, so they are counted on their own)
    const int nnan = chunk_sumi<N>((rk != rk) ? 1 : 0);
    const T tn = chunk_maxf<N>(rk);
    const bool zero = (nnan == 0) & (tn == T(0));
    const bool bad = nnan != 0;
    // exact power-of-two prescaling: tn * s in [0.5, 1)
    const int ex = (bad | zero) ? 0 : F::frexp_exp(tn);
    const T s = F::ldexp(T(1), -ex);
    const T ds = dk * s;
    const T es = ek * s;
    const T esm = ekm * s;
    const T e2 = es * es;
    sdd[k] = ds;
    se2[k] = e2;
    __builtin_amdgcn_wave_barrier();
    const T e2max = chunk_maxf<N>(e2);
    const T pivmin = F::safmin * F::max(T(1), e2max);
    // Gershgorin interval over positions 0..n-1 (padding lanes neutral)
    const T rad = F::abs(esm) + F::abs(es);
    const T inf = T(__builtin_inff());
    const T gl0 = chunk_minf<N>(hasd ? ds - rad : inf);
    const T gu0 = chunk_maxf<N>(hasd ? ds + rad : -inf);
    const T tns = chunk_maxf<N>(hasd ? F::abs(ds) + rad : T(0));
    const T widen = T(2) * T(n) * ulp * tns + T(2) * pivmin;
    T lo = gl0 - widen;
    T hi = gu0 + widen;
    const T atol = ulp * tns;
    // floor(log2(r)) = e - 1 for r = f 2^e, f in [0.5, 1): exact
    const int itmax =
        __builtin_amdgcn_frexp_exp(((double)tns + (double)pivmin) / (double)pivmin) + 1;

    T bd[REGS ? N : 1], be2[REGS ? N : 1];
    if constexpr (REGS) {
        static_for<N>([&](auto I) {
            constexpr int i = decltype(I)::value;
            bd[i] = sdd[i];
            be2[i] = se2[i];
        });
    }

    // Sturm count of the scaled band below x
    auto count = [&](T x) __attribute__((always_inline)) {
        int c = 0;
        T q = T(0);
        static_for_while<N>([&](auto I) {
            constexpr int i = decltype(I)::value;
            const T di = REGS ? bd[i] : sdd[i];
            if constexpr (i == 0) {
                q = di - x;
            } else {
                const T ei = REGS ? be2[i - 1] : se2[i - 1];
                q = F::fma(-ei, F::rcp(q), di - x);
            }
            q = (F::abs(q) < pivmin) ? -pivmin : q;
            c += (q < T(0)) ? 1 : 0;
            return i + 1 < n;  // uniform
        });
        return c;
    };

    // ------------------------------------------------------------ bisection
    bool done = !hasd | bad | zero;
    int fail = 0, it = 0;
    while (__builtin_amdgcn_ballot_w64(!done)) {
        if (!done) {
            const T big = F::max(F::abs(lo), F::abs(hi));
            const T tol = F::max(T(2) * ulp * big, atol);
            if (hi - lo <= tol) {
                done = true;
            } else if (it == itmax) {
                done = true;
                fail = 1;
            } else {
                const T mid = (lo + hi) * T(0.5);
                if ((mid == lo) | (mid == hi)) {
                    done = true;
                } else {
                    if (count(mid) <= k)
                        lo = mid;
                    else
                        hi = mid;
                    ++it;
                }
            }
        }
    }

    // ------------------------------------------------------------ store
    const T us = F::ldexp(T(1), ex);
    T lam = ((lo + hi) * T(0.5)) * us;
    lam = zero ? T(0) : lam;
    lam = bad ? F::qnan() : lam;
    if (hasd) glam[prob * n + k] = lam;
    const int nfail = chunk_sumi<N>(fail);
    if (live & (k == 0) & (args.info != nullptr)) args.info[prob] = bad ? n : nfail;
}

}  // namespace steqr
