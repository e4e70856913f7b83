// Dense front end of the fused small-n symmetric eigensolver: Householder
// reduction of one dense symmetric matrix per chunk of P lanes to
// tridiagonal form T = Q^T A Q, inside the chunked steqr kernel, so that
// the problem stays resident from the load of A to the store of lambda
// and Q (BatchLAS syev routing and tuning page, CTA-family paragraph: the
// fused kernel runs the reduction, the tridiagonal solve and the
// back-transformation with one read of A and one write).
//
// The pages give no arithmetic for the reduction; this is the textbook
// Householder tridiagonalization (Golub and Van Loan) with the reflector
// in the LAPACK larfg convention: for x = (alpha, x_2..x_m) below the
// diagonal of column k, H = I - tau v v^T, v = (1, v_2..v_m), H x =
// (beta, 0..0), beta = -sign(alpha) ||x||, tau = (beta - alpha)/beta,
// v_j = x_j/(alpha - beta); x_2..x_m = 0 gives H = I. The two-sided update
// of the trailing block is the symmetric rank-2 form p = tau A v,
// w = p - (tau p^T v / 2) v, A <- A - v w^T - w v^T, and Q = H_0 H_1 ...
// is accumulated from the identity by right-multiplication.
//
// Layout on chip (MI355X-first): lane r of a chunk holds full rows
// r*RA .. r*RA+RA-1 of A (both triangles) and the same rows of Q in VGPRs.
// Step k is fully unrolled (k, the column positions and the row slots are
// compile-time), so every register array is statically indexed. Per step
// the owner lane of row k publishes it to LDS (by symmetry it is column k),
// every lane of the chunk forms the reflector redundantly from it (no
// broadcast of v), each lane forms p for its own rows, a butterfly over the
// chunk's lanes sums p^T v, and the lanes exchange w through LDS for the
// rank-2 update. Rows at or beyond n are zero padding (their reflectors are
// the identity, their d and e zero). Reciprocals and the square root use
// the hardware instructions (about 1 ulp; Newton-refined in double), as the
// tridiagonal solve's shift does: the reduction is accurate to a few ulps
// of ||A|| either way.
#pragma once

#include "steqr_device.hpp"

namespace steqr {

// Sum over the P lanes of a chunk (butterfly). Every lane receives the same
// value bit for bit: each level adds the same two operands in both lanes of
// a pair, and floating-point addition is commutative. Up to 16 lanes the
// partner comes from a DPP lane move (swap neighbours, swap pairs, mirror 8,
// mirror 16; after each level the lanes of a group hold equal values, so a
// mirror pairs every lane with the other half), beyond that from a shuffle.
template <int CTRL, typename T>
__device__ __forceinline__ T dpp_partner(T v) {
    if constexpr (sizeof(T) == 4) {
        return __builtin_bit_cast(
            T, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
    } else {
        const unsigned long long u = __builtin_bit_cast(unsigned long long, v);
        const int lo = __builtin_amdgcn_update_dpp(0, (int)(unsigned)u, CTRL, 0xF, 0xF, false);
        const int hi = __builtin_amdgcn_update_dpp(0, (int)(unsigned)(u >> 32), CTRL, 0xF, 0xF, false);
        return __builtin_bit_cast(T, ((unsigned long long)(unsigned)hi << 32) | (unsigned)lo);
    }
}
template <int P, typename T>
__device__ __forceinline__ T chunk_sum(T v) {
    static_assert(P >= 1 && P <= 64 && (P & (P - 1)) == 0, "P a power of two");
    if constexpr (P >= 2) v = v + dpp_partner<0xB1>(v);
    if constexpr (P >= 4) v = v + dpp_partner<0x4E>(v);
    if constexpr (P >= 8) v = v + dpp_partner<0x141>(v);
    if constexpr (P >= 16) v = v + dpp_partner<0x140>(v);
    if constexpr (P >= 32) v = v + __shfl_xor(v, 16, 64);
    if constexpr (P >= 64) v = v + __shfl_xor(v, 32, 64);
    return v;
}

// Reduce the chunk's matrix (a: the lane's RA rows, row = r*RA + i) to
// tridiagonal form. With WANTQ the lane's rows of Q (the identity rows on
// entry, in any assignment of rows to lanes) receive H_0 H_1 ... H_{n-2}.
// sx and sw are two chunk-private LDS vectors of N elements. d[0..N) and
// e[0..N) receive T's bands (zero beyond n); with BAND_LDS they stay in LDS
// instead, so that they take no registers while the rows of A and Q do: sx
// then holds the diagonal on return (positions n.. unspecified; step k
// publishes row k from position k on, so sx[k] is never written again) and
// se, a third such vector, the subdiagonal (zero from position n-1 on),
// stored by the chunk's first lane; d and e are not touched. a is
// destroyed.
template <typename T, int N, int P, int RA, bool WANTQ, int RQ, bool BAND_LDS = false>
__device__ __forceinline__ void householder_chunk(T (&a)[RA][N], T (&q)[RQ][N], T (&d)[N],
                                                  T (&e)[N], T* sx, T* sw, T* se, int n, int r) {
    using F = Fp<T>;
    static_assert(RA * P == N, "the chunk's lanes hold exactly N rows");
    static_for<N>([&](auto K) {
        constexpr int k = decltype(K)::value;
        // publish row k (= column k by symmetry) from its owner lane
        if (r == k / RA) {
            static_for<N - k>([&](auto J) {
                constexpr int j = k + decltype(J)::value;
                sx[j] = a[k % RA][j];
            });
        }
        __builtin_amdgcn_wave_barrier();
        if constexpr (!BAND_LDS) {
            d[k] = (k < n) ? sx[k] : T(0);
            e[k] = T(0);
        }
        T ek = T(0);
        if constexpr (k + 1 < N) {
            if (k + 1 < n) {  // uniform: n is the same for every problem
                T x[N];
                static_for<N - k - 1>([&](auto J) {
                    constexpr int j = k + 1 + decltype(J)::value;
                    x[j] = sx[j];
                });
                // reflector of (alpha, x_{k+2..}): scaled 2-norm, NaN-propagating;
                // H = I exactly when the tail x_{k+2..} is zero (tested on the
                // unscaled entries: a tail far below |alpha|, or an infinite
                // alpha, scales to squares that vanish but still takes the
                // reflector, here as in the larfg convention)
                const T alpha = x[k + 1];
                T sc = F::abs(alpha);
                bool hasnan = alpha != alpha;
                bool tailnz = false;
                static_for<N - k - 2>([&](auto J) {
                    constexpr int j = k + 2 + decltype(J)::value;
                    sc = F::max(sc, F::abs(x[j]));
                    hasnan = hasnan | (x[j] != x[j]);
                    tailnz = tailnz | (x[j] != T(0));
                });
                sc = hasnan ? F::qnan() : sc;
                const T inv = (sc == T(0)) ? T(0) : F::rcp(sc);
                T ss = T(0);
                static_for<N - k - 2>([&](auto J) {
                    constexpr int j = k + 2 + decltype(J)::value;
                    const T y = x[j] * inv;
                    ss = F::fma(y, y, ss);
                });
                T tau = T(0), beta = alpha, scal = T(0);
                if (tailnz) {
                    const T ya = alpha * inv;
                    const T nrm = sc * F::sqrt_fast(F::fma(ya, ya, ss));
                    beta = -F::copysign(nrm, alpha);
                    tau = (beta - alpha) * F::rcp(beta);
                    scal = F::rcp(alpha - beta);
                }
                ek = beta;
                if constexpr (!BAND_LDS) e[k] = beta;
                if (tau != T(0)) {
                    // short of registers: double at order 32 with vectors
                    constexpr bool LIGHT = sizeof(T) == 8 && N >= 32 && WANTQ;
                    constexpr int WT = 8;
                    if constexpr (!LIGHT) {
                        T v[N];
                        v[k + 1] = T(1);
                        static_for<N - k - 2>([&](auto J) {
                            constexpr int j = k + 2 + decltype(J)::value;
                            v[j] = x[j] * scal;
                        });
                        // p = tau A v on the lane's rows (rows <= k are done: 0)
                        T p[RA], vr[RA];
                        T part = T(0);
                        static_for<RA>([&](auto II) {
                            constexpr int i = decltype(II)::value;
                            const int row = r * RA + i;
                            T s = a[i][k + 1];
                            static_for<N - k - 2>([&](auto J) {
                                constexpr int j = k + 2 + decltype(J)::value;
                                s = F::fma(a[i][j], v[j], s);
                            });
                            p[i] = (row > k) ? tau * s : T(0);
                            const T xr = sx[row];
                            vr[i] = (row == k + 1) ? T(1) : ((row > k + 1) ? xr * scal : T(0));
                            part = F::fma(p[i], vr[i], part);
                        });
                        const T pv = chunk_sum<P>(part);
                        const T half = tau * pv * T(0.5);
                        T w[RA];
                        static_for<RA>([&](auto II) {
                            constexpr int i = decltype(II)::value;
                            w[i] = F::fma(-half, vr[i], p[i]);
                            sw[r * RA + i] = w[i];
                        });
                        __builtin_amdgcn_wave_barrier();
                        T wv[N];
                        static_for<N - k - 1>([&](auto J) {
                            constexpr int j = k + 1 + decltype(J)::value;
                            wv[j] = sw[j];
                        });
                        // A <- A - v w^T - w v^T on the trailing columns
                        static_for<RA>([&](auto II) {
                            constexpr int i = decltype(II)::value;
                            static_for<N - k - 1>([&](auto J) {
                                constexpr int j = k + 1 + decltype(J)::value;
                                a[i][j] = F::fma(-w[i], v[j], F::fma(-vr[i], wv[j], a[i][j]));
                            });
                        });
                        // Q <- Q H_k, row by row
                        if constexpr (WANTQ) {
                            static_for<RQ>([&](auto II) {
                                constexpr int i = decltype(II)::value;
                                T t = q[i][k + 1];
                                static_for<N - k - 2>([&](auto J) {
                                    constexpr int j = k + 2 + decltype(J)::value;
                                    t = F::fma(q[i][j], v[j], t);
                                });
                                t = tau * t;
                                static_for<N - k - 1>([&](auto J) {
                                    constexpr int j = k + 1 + decltype(J)::value;
                                    q[i][j] = F::fma(-t, v[j], q[i][j]);
                                });
                            });
                        }
                    } else {
                        // The same arithmetic with v_j = x_j scal formed
                        // again from sx (row k stays published until the
                        // step ends) WT columns at a time, so that neither v
                        // nor w occupies N registers next to the rows of A
                        // and Q: the dot products a_i.v and q_i.v in one pass,
                        // the rank-2 update of A and Q <- Q H_k in a second.
                        constexpr int NT = (N - k - 1 + WT - 1) / WT;
                        T sa[RA], tq[RQ];
                        static_for<RA>([&](auto II) {
                            sa[decltype(II)::value] = a[decltype(II)::value][k + 1];
                        });
                        static_for<RQ>([&](auto II) {
                            tq[decltype(II)::value] = q[decltype(II)::value][k + 1];
                        });
                        static_for<NT>([&](auto TT) {
                            constexpr int j0 = k + 1 + decltype(TT)::value * WT;
                            constexpr int nj = (N - j0 < WT) ? N - j0 : WT;
                            T vt[WT];
                            static_for<nj>([&](auto J) {
                                constexpr int j = j0 + decltype(J)::value;
                                if constexpr (j > k + 1) vt[decltype(J)::value] = sx[j] * scal;
                            });
                            static_for<RA>([&](auto II) {
                                constexpr int i = decltype(II)::value;
                                static_for<nj>([&](auto J) {
                                    constexpr int j = j0 + decltype(J)::value;
                                    if constexpr (j > k + 1)
                                        sa[i] = F::fma(a[i][j], vt[decltype(J)::value], sa[i]);
                                });
                            });
                            if constexpr (WANTQ) {
                                static_for<RQ>([&](auto II) {
                                    constexpr int i = decltype(II)::value;
                                    static_for<nj>([&](auto J) {
                                        constexpr int j = j0 + decltype(J)::value;
                                        if constexpr (j > k + 1)
                                            tq[i] = F::fma(q[i][j], vt[decltype(J)::value], tq[i]);
                                    });
                                });
                            }
                            __builtin_amdgcn_wave_barrier();
                        });
                        T p[RA], vr[RA];
                        T part = T(0);
                        static_for<RA>([&](auto II) {
                            constexpr int i = decltype(II)::value;
                            const int row = r * RA + i;
                            p[i] = (row > k) ? tau * sa[i] : T(0);
                            const T xr = sx[row];
                            vr[i] = (row == k + 1) ? T(1) : ((row > k + 1) ? xr * scal : T(0));
                            part = F::fma(p[i], vr[i], part);
                        });
                        const T pv = chunk_sum<P>(part);
                        const T half = tau * pv * T(0.5);
                        T w[RA];
                        static_for<RA>([&](auto II) {
                            constexpr int i = decltype(II)::value;
                            w[i] = F::fma(-half, vr[i], p[i]);
                            sw[r * RA + i] = w[i];
                        });
                        T t[RQ];
                        static_for<RQ>([&](auto II) {
                            t[decltype(II)::value] = tau * tq[decltype(II)::value];
                        });
                        __builtin_amdgcn_wave_barrier();
                        static_for<NT>([&](auto TT) {
                            constexpr int j0 = k + 1 + decltype(TT)::value * WT;
                            constexpr int nj = (N - j0 < WT) ? N - j0 : WT;
                            T vt[WT], wv[WT];
                            static_for<nj>([&](auto J) {
                                constexpr int j = j0 + decltype(J)::value;
                                vt[decltype(J)::value] = (j == k + 1) ? T(1) : sx[j] * scal;
                                wv[decltype(J)::value] = sw[j];
                            });
                            static_for<RA>([&](auto II) {
                                constexpr int i = decltype(II)::value;
                                static_for<nj>([&](auto J) {
                                    constexpr int jj = decltype(J)::value;
                                    a[i][j0 + jj] = F::fma(-w[i], vt[jj],
                                                           F::fma(-vr[i], wv[jj], a[i][j0 + jj]));
                                });
                            });
                            if constexpr (WANTQ) {
                                static_for<RQ>([&](auto II) {
                                    constexpr int i = decltype(II)::value;
                                    static_for<nj>([&](auto J) {
                                        constexpr int jj = decltype(J)::value;
                                        q[i][j0 + jj] = F::fma(-t[i], vt[jj], q[i][j0 + jj]);
                                    });
                                });
                            }
                            __builtin_amdgcn_wave_barrier();
                        });
                    }
                }
            }
        }
        if constexpr (BAND_LDS) {
            if (r == 0) se[k] = ek;
        }
        // the next step's publish overwrites sx: keep this step's reads first
        __builtin_amdgcn_wave_barrier();
    });
}

}  // namespace steqr
