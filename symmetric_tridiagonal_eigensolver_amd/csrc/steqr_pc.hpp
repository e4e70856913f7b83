// Producer-consumer steqr kernel for orders 33..512 with eigenvectors (and
// values only at 65..512)
// (gfx950, wave64).
//
// At these orders a problem's Q fills much of a wavefront's registers (at
// order 64 lane i holds row i: 64 values), so a kernel that keeps both the
// band chase and the rows of Q in one wavefront either runs the serial
// chase on many lanes for few problems or runs out of registers; the
// chase, not the Q update, sets its time. Here a workgroup splits the two
// parts of the step [algo, Givens/similarity paragraphs and eigenvector
// accumulation]:
//  * one producer wavefront holds the bands of NP problems in LDS, one chunk
//    of P lanes per problem, and runs the whole per-problem algorithm of
//    steqr_chunkl.hpp (settle, shift, chase, 2x2 blocks as one-step chases)
//    without Q. Each chase step writes its rotation (c, s) to a rotation
//    log in LDS; each pass writes, per problem, the part of Q it touches
//    (first position, step count) and whether the problem was mirrored
//    (block direction) before the pass;
//  * W consumer wavefronts each hold the Q of 64/N problems (lane = row) and apply
//    the logged rotations of the previous pass while the producer computes
//    the next one (two log slots, one workgroup barrier per pass).
// From order 128 a row of Q is split over RS lanes of one wavefront (at
// order 128 two: columns 0..63 and 64..127 in lanes l and l^32; at 256 two
// or four, at 512 eight or sixteen), so a consumer wavefront holds 64/RS
// rows; the unrolled pass applies the rotations in position order, so the
// lanes of the part a rotation falls in run it while the others are masked,
// and a rotation that straddles two parts swaps the two boundary values
// across the lane pair. When a problem needs more consumers than a
// workgroup holds, several workgroups share it, each with its own producer. Without eigenvectors
// (WANTQ false) every wavefront is a producer of its own problems and no
// log is written.
// The consumers' column updates are the same as the other kernels' and
// their order of application is the producer's, so the results equal the
// chunked kernels' up to the same rounding. The bands, the sort keys and
// all control decisions stay with the producer; the consumers only read
// the log, the ranks of the final sort and the final mirror flag.
// Citations as in steqr_chunk.hpp.
#pragma once

#include "steqr_chunkl.hpp"

namespace steqr {

// W consumer wavefronts. RS lanes hold one row of Q (at order 128 by
// default two half rows; at order 256 halves in float, quarters in double,
// 128 registers per lane either way; at order 512 eighths in float and
// sixteenths in double, 64 registers per lane, which keeps the kernel
// within the 168 registers per lane of three wavefronts per SIMD without
// spilling), so a consumer holds RPW = 64/RS
// rows: CQ = RPW/N problems when N <= RPW, else WPP = N/RPW consumers per
// problem. When one problem needs more consumers than a workgroup holds
// (double at order 256: 16; at 512: 64 in float, 128 in double), GPP = WPP/W
// workgroups share it, each with its
// own producer (the producers compute the same rotations) and a slice of
// the rows. NP = W * CQ / WPP problems per workgroup (1 when shared).
template <typename T, int N>
constexpr int pc_default_rs() {
    return N <= 64 ? 1 : (N == 128 ? 2 : (N == 256 ? (sizeof(T) == 4 ? 2 : 4)
                                                    : (sizeof(T) == 4 ? 8 : 16)));
}

template <typename T, int N, int W, int P, int RS = pc_default_rs<T, N>()>
struct SmemPC {
    static constexpr int RPW = 64 / RS;                   // rows per consumer
    static constexpr int CQ = N <= RPW ? RPW / N : 1;     // problems per consumer
    static constexpr int WPP = N <= RPW ? 1 : N / RPW;    // consumers per problem
    static constexpr int GPP = (W > 0 && WPP > W) ? WPP / W : 1;  // workgroups per problem
    static constexpr int NP = GPP > 1 ? 1 : W * CQ / WPP; // problems per workgroup
    static constexpr int CH = 64 / P;                     // producer chunks (>= NP)
    static constexpr int SLOT = 2 * N + 1;                // d[N], e[N], pad
    static constexpr size_t band_bytes = ((CH * SLOT * sizeof(T) + 15) / 16) * 16;
    // rotation log: [slot 0/1][problem][position] -> (c, s); row NP of each
    // slot is a sink for the producer's unused chunks
    static constexpr size_t rot_bytes = (size_t)2 * (NP + 1) * (N - 1) * 2 * sizeof(T);
    // per slot: control word, then per problem (flip, first position, steps)
    static constexpr int HDR = 1 + 3 * NP;
    static constexpr size_t hdr_bytes = ((2 * HDR * sizeof(int) + 15) / 16) * 16;
    static constexpr size_t rank_bytes = ((CH * N * sizeof(int) + 15) / 16) * 16;
    static constexpr size_t fin_bytes = ((NP * sizeof(int) + 15) / 16) * 16;
    // store staging: each consumer writes GROUP of its rows at a time, with
    // the sort's column permutation, into a GROUP x N tile and copies the
    // tile to HBM as contiguous 16-byte pieces (about 4 KiB per consumer)
    static constexpr int ROWS = N <= RPW ? N : RPW;  // rows a consumer holds
    static constexpr int GROUP_ = (int)(4096 / (N * sizeof(T)));
    static constexpr int GROUP = GROUP_ < 2 ? 2 : (GROUP_ > ROWS ? ROWS : GROUP_);
    static constexpr size_t stage_bytes = (size_t)W * GROUP * N * sizeof(T);
    static constexpr size_t bytes =
        band_bytes + rot_bytes + hdr_bytes + rank_bytes + fin_bytes + stage_bytes;
};

// Values-only form (WANTQ false): the producer's algorithm alone, every
// wavefront of the workgroup a producer of its own 64/P problems.
template <typename T, int N, int P>
struct SmemPV {
    static constexpr int CH = 64 / P;
    static constexpr int SLOT = 2 * N + 1;
    static constexpr size_t band_bytes = ((CH * SLOT * sizeof(T) + 15) / 16) * 16;
    static constexpr size_t rank_bytes = ((CH * N * sizeof(int) + 15) / 16) * 16;
    static constexpr size_t bytes_per_wave = band_bytes + rank_bytes;
};

enum { PC_CTRL_PASS = 1, PC_CTRL_END = 2 };

// Consumer wavefront: hold rows of Q (lane = row; with RS lanes per row,
// lane row + RPW*k holds columns kQW .. kQW+QW-1 of the row) and apply the
// producer's logged rotations pass by pass; at the end store the rows with
// the sort's column permutation.
template <typename T, int N, int W, int P, int RS>
__device__ __forceinline__ void consume(const KernelArgs& args, int lane, int wave, long first,
                                        const T* rot, const int* hdr, const int* ranks,
                                        const int* fin) {
    // slots: 0 load, 1 waiting for a pass, 2 applying a pass, 3 epilogue,
    // 5 passes
    STEQR_PHASE_START;
    using S = SmemPC<T, N, W, P, RS>;
    using F = Fp<T>;
    constexpr int NP = S::NP;
    constexpr int QW = N / RS;  // columns held per lane
    T* __restrict__ gq = static_cast<T*>(args.q);
    const int n = args.n;
    constexpr int RPW = S::RPW;
    constexpr int WL = S::WPP / S::GPP;  // this workgroup's consumers of a problem
    const int pi = (N <= RPW) ? wave * S::CQ + lane / N : wave / WL;
    const int part = RS > 1 ? lane / RPW : 0;  // which QW columns of the row
    const int slice = S::GPP > 1 ? (int)(blockIdx.x % S::GPP) : 0;
    const int row = (N <= RPW) ? lane % N : ((wave % WL) + slice * WL) * RPW + lane % RPW;
    const int c0 = part * QW;
    const long prob = first + pi;
    const bool live = prob < (long)args.batch;
    // the identity, or with back-transformation [algo, eigenvector
    // accumulation] the caller's basis
    T q[QW];
    {
        const bool vec = (n == N) & ((reinterpret_cast<uintptr_t>(gq) & 15) == 0);
        const long pc = live ? prob : (long)args.batch - 1;
        load_basis_cols<T, QW>(gq + pc * n * n, n, row, c0, live, args.back_transform != 0, vec,
                               q);
    }
    // The rotation straddling parts j and j+1 of a row (columns (j+1)QW - 1
    // and (j+1)QW): the two lanes swap their boundary values (every lane of
    // the wavefront takes part in the shuffle); `lead_upper` says whether
    // part j+1 holds the rotation's first operand.
    auto straddle = [&](int j, bool lead_upper, T c, T sn) __attribute__((always_inline)) {
        const bool lower = part == j, upper = part == j + 1;
        const T mine = upper ? q[0] : q[QW - 1];
        const T other = __shfl(mine, (upper ? lane - RPW : lane + RPW) & 63, 64);
        const bool lead = lead_upper ? upper : lower;
        const T upd = lead ? F::fma(c, mine, sn * other) : F::fma(c, mine, -(sn * other));
        if (lower) q[QW - 1] = upd;
        if (upper) q[0] = upd;
    };
    // The producer mirrors a problem (positions p <-> N-1-p, Q's columns
    // included) while a block that converges at its top is reduced.
    // Instead of reversing its registers, the consumer tracks the
    // orientation and applies a rotation at mirrored position p to the
    // columns (N-1-p, N-2-p), which is the same update.
    int orient = 0;
    int slot = 0;
    STEQR_PHASE_MARK(0);
    while (true) {
        __syncthreads();
        STEQR_PHASE_MARK(1);
        const int* h = hdr + slot * S::HDR;
        if (h[0] == PC_CTRL_END) break;
        STEQR_PHASE_ADD(5, 1);
        if constexpr (RS == 1) {
            orient ^= h[1 + 3 * pi];
        } else if (h[1 + 3 * pi]) {
            // with a row split over RS lanes the mirror is applied to the
            // registers (column j of part k <-> column QW-1-j of part
            // RS-1-k, pairwise through lane shuffles; a problem's blocks
            // open and close a few times), so that the passes below need
            // only the one orientation
            const int src = (lane % RPW) + RPW * (RS - 1 - part);
            static_for<QW / 2>([&](auto J) {
                constexpr int j = decltype(J)::value;
                const T a = __shfl(q[QW - 1 - j], src, 64);
                const T b = __shfl(q[j], src, 64);
                q[j] = a;
                q[QW - 1 - j] = b;
            });
        }
        const int s = h[2 + 3 * pi];
        const int steps = h[3 + 3 * pi];
        const T* lg = rot + (size_t)(slot * (NP + 1) + pi) * (N - 1) * 2;
        if (steps > 0) {
            const int me = s + steps;
            if constexpr (RS == 1) {
                if (orient == 0) {
                    static_for_while<N - 1>([&](auto I) {
                        constexpr int p = decltype(I)::value;
                        if (p >= s) F::rot(q[p], q[p + 1], lg[2 * p], lg[2 * p + 1]);
                        return p + 1 < me;
                    });
                } else {
                    static_for_while<N - 1>([&](auto I) {
                        constexpr int p = decltype(I)::value;
                        if (p >= s) F::rot(q[N - 1 - p], q[N - 2 - p], lg[2 * p], lg[2 * p + 1]);
                        return p + 1 < me;
                    });
                }
            } else {
                // Positions kQW .. kQW+QW-2 fall inside part k of the columns,
                // kQW+QW-1 straddles parts k and k+1: the parts run in
                // position order, each under one lane mask (the problem's s
                // and me are uniform over the wavefront; the registers are
                // never mirrored here, see above).
                static_for<RS>([&](auto LQ) {
                    constexpr int lq = decltype(LQ)::value;
                    constexpr int pos0 = lq * QW;
                    const int sl = s - pos0, el = me - pos0;
                    if ((el > 0) & (sl < QW - 1) & (part == lq)) {
                        const T* lgl = lg + 2 * pos0;
                        static_for_while<QW - 1>([&](auto I) {
                            constexpr int p = decltype(I)::value;
                            if (p >= sl) F::rot(q[p], q[p + 1], lgl[2 * p], lgl[2 * p + 1]);
                            return p + 1 < el;
                        });
                    }
                    if constexpr (lq + 1 < RS) {
                        constexpr int ps = pos0 + QW - 1;
                        if ((s <= ps) & (ps < me)) straddle(lq, false, lg[2 * ps], lg[2 * ps + 1]);
                    }
                });
            }
        }
        slot ^= 1;
        STEQR_PHASE_MARK(2);
    }
    __syncthreads();
    STEQR_PHASE_MARK(1);
    // every block is closed, hence un-mirrored, by now (orient ^ fin is
    // 0); a remaining reversal would be folded into the column index
    const bool rev = (orient ^ fin[pi]) != 0;
    // Store through the wavefront's staging tile, GROUP rows at a time: the
    // lanes of those rows write their values unpermuted (contiguous), then
    // the whole wavefront writes the rows (contiguous in HBM) in 16-byte
    // pieces, gathering column c of the sorted order from column inv[c]
    // (the producer's inverse permutation; reversed when a mirror is left).
    // Writing permuted columns straight to HBM touched each line several
    // times (1.6x the algorithmic bytes at order 64).
    static_assert(S::CQ == 1, "one problem per consumer wavefront");
    constexpr int G = S::GROUP;
    constexpr int V = 16 / (int)sizeof(T);
    T* const stg = reinterpret_cast<T*>(
        reinterpret_cast<unsigned char*>(const_cast<int*>(fin)) + S::fin_bytes) +
        (size_t)wave * G * N;
    const int rl = lane % RPW;    // the lane's row among the wavefront's rows
    const int row0 = row - rl;    // the wavefront's first row (uniform)
    if (live) {
        const int* inv = ranks + pi * N;
        T* const qb = gq + prob * (long)n * n;
        static_for<S::ROWS / G>([&](auto GG) {
            constexpr int g = decltype(GG)::value;
            const int rg0 = row0 + g * G;  // first row of the group (uniform)
            if (rg0 < n) {
                const int gl = rl - g * G;
                if ((gl >= 0) & (gl < G)) {
                    static_for<QW>([&](auto J) {
                        constexpr int j = decltype(J)::value;
                        stg[gl * N + c0 + j] = q[j];
                    });
                }
                __builtin_amdgcn_wave_barrier();
                const int rows = n - rg0 < G ? n - rg0 : G;
                const int total = rows * n;
                T* const dst = qb + (long)rg0 * n;
                auto src = [&](int idx) __attribute__((always_inline)) {
                    const int r = idx / n, c = idx - r * n;
                    const int jj = inv[c];
                    return stg[r * N + (rev ? N - 1 - jj : jj)];
                };
                if (((reinterpret_cast<uintptr_t>(dst) & 15) == 0) & ((n % V) == 0)) {
                    // V consecutive elements stay within one row
                    static_for<(G * N + 64 * V - 1) / (64 * V)>([&](auto K) {
                        constexpr int k = decltype(K)::value;
                        const int idx = (k * 64 + lane) * V;
                        if (idx < total) {
                            const int r = idx / n, c = idx - r * n;
                            const T* const sr = stg + r * N;
                            T v[V];
                            static_for<V>([&](auto U) {
                                constexpr int u = decltype(U)::value;
                                const int jj = inv[c + u];
                                v[u] = sr[rev ? N - 1 - jj : jj];
                            });
                            if constexpr (sizeof(T) == 4) {
                                *reinterpret_cast<float4*>(dst + idx) = make_float4(v[0], v[1], v[2], v[3]);
                            } else {
                                *reinterpret_cast<double2*>(dst + idx) = make_double2(v[0], v[1]);
                            }
                        }
                    });
                } else {
                    static_for<(G * N + 63) / 64>([&](auto K) {
                        constexpr int k = decltype(K)::value;
                        const int idx = k * 64 + lane;
                        if (idx < total) dst[idx] = src(idx);
                    });
                }
                __builtin_amdgcn_wave_barrier();
            }
        });
    }
    STEQR_PHASE_MARK(3);
    STEQR_PHASE_STORE(wave, lane);
}

// Wavefronts per SIMD the register allocation must allow: at order 128 in
// float two workgroups of W = 8 consumers and a producer (18 wavefronts)
// share a CU only at five per SIMD.
template <typename T, int N, int W>
constexpr int pc_min_waves() {
    return (N == 128 && sizeof(T) == 4 && W == 8) ? 5 : 1;
}

template <typename T, int N, int W, int P, bool PG, bool WANTQ = true,
          int RS = pc_default_rs<T, N>()>
__global__ void __launch_bounds__((WANTQ ? (W + 1) * 64 : 256), (pc_min_waves<T, N, W>()))
    steqr_pc_kernel(KernelArgs args) {
    using S = SmemPC<T, N, W, P, RS>;
    constexpr int WPP = S::WPP;
    constexpr int CH = 64 / P;
    // problems of one producer wavefront
    constexpr int NP = WANTQ ? S::NP : CH;
    // At order 32 (two problems per consumer) this split measured slower
    // than the LDS-band chunked kernel, so orders 64 and 128 are built.
    static_assert(N == 64 || N == 128 || N == 256 || N == 512,
                  "the producer-consumer kernel is for orders 64, 128, 256 and 512");
    static_assert(!WANTQ || (W % WPP) == 0 || (WPP % W) == 0,
                  "whole problems per workgroup, or whole workgroups per problem");
    static_assert(P >= 2 && (64 % P) == 0 && (N % P) == 0 && 64 / P >= NP, "P lanes per chunk");
    constexpr int K = N / P;  // positions per producer lane
    using M = PosMask<N>;
    using F = Fp<T>;
    enum { ST_OPEN = 0, ST_ITER = 1, ST_DONE = 2 };

    extern __shared__ __align__(16) unsigned char smem_raw[];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    // producer's phase slots: 0 load, 1 settle, 2 chase, 3 epilogue, 4
    // waiting for the consumers, 5 passes, 6 sum of the passes' chase bounds
    STEQR_PHASE_START;
    using SV = SmemPV<T, N, P>;
    unsigned char* const base = WANTQ ? smem_raw : smem_raw + (size_t)wave * SV::bytes_per_wave;
    T* const band = reinterpret_cast<T*>(base);
    T* const rot = reinterpret_cast<T*>(smem_raw + S::band_bytes);
    int* const hdr = reinterpret_cast<int*>(smem_raw + S::band_bytes + S::rot_bytes);
    int* const ranks = WANTQ ? reinterpret_cast<int*>(smem_raw + S::band_bytes + S::rot_bytes +
                                                      S::hdr_bytes)
                             : reinterpret_cast<int*>(base + SV::band_bytes);
    int* const fin = reinterpret_cast<int*>(smem_raw + S::band_bytes + S::rot_bytes +
                                            S::hdr_bytes + S::rank_bytes);

    const T* __restrict__ gd = static_cast<const T*>(args.d);
    const T* __restrict__ ge = static_cast<const T*>(args.e);
    T* __restrict__ glam = static_cast<T*>(args.lam);
    T* __restrict__ gq = static_cast<T*>(args.q);
    const int n = args.n;
    // the first problem of the workgroup (with Q; GPP workgroups share one
    // problem when it needs more consumers than a workgroup holds) or of
    // this wavefront
    const long first = WANTQ ? (long)(blockIdx.x / S::GPP) * NP
                             : ((long)blockIdx.x * (blockDim.x >> 6) + wave) * CH;
    // of the workgroups sharing a problem, the first stores its eigenvalues
    // and status (the others computed the same ones)
    const bool lead_wg = !WANTQ || (blockIdx.x % S::GPP) == 0;

    if constexpr (WANTQ) {
        if (wave < W) {
            consume<T, N, W, P, RS>(args, lane, wave, first, rot, hdr, ranks, fin);
            return;
        }
    }

    // ================================================================ producer
    // The producer's serial chase sets the workgroup's pace and shares its
    // SIMD with consumer wavefronts, which have slack: let the SIMD's
    // instruction arbiter prefer the producer.
    if constexpr (WANTQ) __builtin_amdgcn_s_setprio(3);
    const int chunk = lane / P;
    const int r = lane % P;
    const long prob = first + chunk;
    const bool live = (chunk < NP) & (prob < (long)args.batch);
    const long pb = live ? prob : (long)args.batch - 1;
    T* const sd = band + chunk * S::SLOT;
    T* const se = sd + N;
    int* const srank = ranks + chunk * N;

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
            part |= (se[p] == T(0)) ? bit_at<M>(p) : (M)0;
        });
        zeromask = chunk_or_mask<P>(part);
    }

    int state = live ? ST_OPEN : ST_DONE;
    int l1 = 0, bt = 0, bb = 0, m = 0, s = 0;
    int jtot = 0;
    const int nmaxit = (args.max_sweeps_per_n > 0 ? args.max_sweeps_per_n : 0) * n;
    bool mir = false, failed = false, last = false, pending = false;
    int flip = 0;  // mirrors of Q not yet handed to the consumer (parity)
    int mode = 0;
    T anorm = T(0);
    M zeroed = 0;
    int info = 0;

    // reverse the chunk's band (lane-parallel); Q's columns are the
    // consumer's: count the reversal
    // Each lane swaps whole pairs (p, N-1-p) of d and (p, N-2-p) of e for
    // its positions p = r + kP in the first half, so no value crosses lanes
    // and at most two pairs are held in registers at a time.
    auto mirror_all = [&]() __attribute__((always_inline)) {
        static_for<K / 2>([&](auto KK) {
            constexpr int k = decltype(KK)::value;
            const int p = r + k * P;  // p < N/2
            const T da = sd[p], db = sd[N - 1 - p];
            sd[p] = db;
            sd[N - 1 - p] = da;
            if (p < N / 2 - 1) {
                const T ea = se[p], eb = se[N - 2 - p];
                se[p] = eb;
                se[N - 2 - p] = ea;
            }
        });
        __builtin_amdgcn_wave_barrier();
        flip ^= 1;
    };

    // zero the negligible e's found in the block, undo the scaling (d
    // always, e too when the block failed), undo the mirror
    auto close_block = [&](bool fail) __attribute__((always_inline)) {
        const T un = (mode == 1) ? anorm / F::ssfmax : ((mode == 2) ? anorm / F::ssfmin : T(1));
        static_for<K>([&](auto KK) {
            constexpr int k = decltype(KK)::value;
            const int p = r + k * P;
            T ev = se[p], dv = sd[p];
            ev = bit_test(zeroed, p) ? T(0) : ev;
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

    // open the next block [algo, steqr_cta paragraph; scaling], as in
    // steqr_chunkl.hpp
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
            mir = !(F::abs(sd[hi]) < F::abs(sd[lo]));
            if (mir) mirror_all();
            bt = mir ? N - 1 - hi : lo;
            bb = mir ? N - 1 - lo : hi;
            m = bb;
            zeroed = bt > 0 ? bit_at<M>(bt - 1) : (M)0;
            state = ST_ITER;
        }
    };

    int slot = 0;
    T x = T(0), y = T(0), dcur = T(0);
    STEQR_PHASE_MARK(0);
    while (true) {
        // ------------------------------------------------------------ settle
        if (__any(state == ST_OPEN)) open_blocks();
        const bool iter = state == ST_ITER;
        if (!__any(iter)) break;
        const M neg = scan_negligible<T, N, P, M>(sd, se, r) | zeroed;
        const M rng = bit_range<M>(bt, m - 1);
        const M nb = neg & rng;
        const M clr = rng & ~neg;
        const bool conv = iter & (clr == 0);
        const bool go = iter & (clr != 0);
        const int t = msb((M)(clr | (M)1));
        const M above = nb & bit_range<M>(bt, t - 1);
        const int s2 = above ? msb(above) + 1 : bt;
        const M znew = (nb & bit_range<M>(t + 1, m - 1)) | (above ? bit_at<M>(above ? s2 - 1 : 0) : (M)0);
        zeroed |= conv ? nb : (go ? znew : (M)0);
        const bool jac = go & (t == s2);
        const bool fail = go & !jac & (jtot >= nmaxit);
        const bool sweep = go & !jac & !fail;
        const int jpos = s2;
        m = jac ? s2 - 1 : (go ? t + 1 : m);
        s = go ? s2 : s;
        jtot += sweep ? 1 : 0;
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
                        part |= ((p < n - 1) & (se[p] != T(0))) ? bit_at<M>(p) : (M)0;
                    });
                    info = popc(chunk_or_mask<P>(part));
                    info = info > 0 ? info : 1;
                    // the status is final: store it now rather than keep
                    // it in a register through the remaining passes
                    if (live & lead_wg & (args.info != nullptr) & (r == 0)) args.info[prob] = info;
                }
                state = fail ? ST_DONE : ST_OPEN;
            }
        }
        pending = pending | (conv & last);
        state = (conv & last) ? ST_DONE : state;
        // shift [algo, shift section] and the first running pair; a 2x2
        // block is a one-step chase seeded with its closed-form rotation
        const int mi = sweep ? m : (jac ? jpos + 1 : 1);
        const int si = sweep ? s : (jac ? jpos : 0);
        const T dm = sd[mi], dm1 = sd[mi - 1], em1 = se[mi - 1];
        const T mu = sweep_shift(args.shift_kind != 0, dm, dm1, em1);
        dcur = sd[si];
        x = dcur - mu;
        y = PG ? T(1) : se[si];
        if (__any(jac)) {
            T rt1, rt2, cs, sj;
            sym2x2(dm1, em1, dm, rt1, rt2, cs, sj);
            x = jac ? (PG ? cs * em1 : cs) : x;
            y = jac ? -sj : y;
            zeroed |= jac ? bit_at<M>(jpos) : (M)0;
        }
        const unsigned steps = sweep ? (unsigned)(m - s) : (jac ? 1u : 0u);
        // hand the pass to the consumers: mirror parity, first position,
        // step count (all lanes of a chunk write the same words)
        if constexpr (WANTQ) {
            int* h = hdr + slot * S::HDR;
            if (chunk < NP) {
                h[1 + 3 * chunk] = flip;
                h[2 + 3 * chunk] = s;
                h[3 + 3 * chunk] = (int)steps;
            }
            if (lane == 0) h[0] = PC_CTRL_PASS;
        }
        flip = 0;

        // ------------------------------------------------------------ chase
        STEQR_PHASE_MARK(1);
        STEQR_PHASE_ADD(5, 1);
        T* const lg = rot + (size_t)(slot * (NP + 1) + (chunk < NP ? chunk : NP)) * (N - 1) * 2;
        T d0 = sd[0], e0 = se[0], d1 = sd[1], e1 = se[1];
        T cp = T(1);
        // values only: every wavefront a producer; chase at a raised issue
        // priority, settle at the default one (as in steqr_chunk.hpp)
        if constexpr (!WANTQ) __builtin_amdgcn_s_setprio(1);
        // the chase stops after the last position any chunk of the
        // wavefront steps through, tested after every second position (one
        // scalar branch per two positions; an extra position steps no chunk)
        const int me_w = wave_max_uniform(steps != 0u ? s + (int)steps : 0);
        STEQR_PHASE_ADD(6, me_w);
        static_for_while<N - 1>([&](auto I) {
            constexpr int p = decltype(I)::value;
            T d2 = T(0), e2 = T(0);
            if constexpr (p + 2 < N) {
                d2 = sd[p + 2];
                e2 = se[p + 2];
            }
            if ((unsigned)(p - s) < steps) {
                T c, sn, rr;
                if constexpr (PG) {
                    // PG step [algo, update-scheme paragraph], as in
                    // steqr_chunkl.hpp
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
                    lg[2 * p] = c;
                    lg[2 * p + 1] = sn;
                }
            }
            d0 = d1;
            e0 = e1;
            d1 = d2;
            e1 = e2;
            return (p & 1) == 0 || p + 1 < me_w;
        });
        if (steps != 0u) {
            const int me = s + (int)steps;
            sd[me] = dcur;
            se[me - 1] = x;
        }
        if constexpr (!WANTQ) __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_wave_barrier();
        jtot = (sweep & (mu != mu)) ? nmaxit : jtot;
        STEQR_PHASE_MARK(2);
        if constexpr (WANTQ) __syncthreads();  // the log of this pass is complete
        STEQR_PHASE_MARK(4);
        slot ^= 1;
    }
    STEQR_PHASE_MARK(1);
    if constexpr (WANTQ) {
        // no pass left: tell the consumers (their last pass was the previous slot)
        if (lane == 0) hdr[slot * S::HDR] = PC_CTRL_END;
        __syncthreads();
    }

    // closes of converged last blocks, the final mirror parity and the sort
    if (__any(pending)) {
        if (pending) close_block(false);
    }
    __builtin_amdgcn_wave_barrier();
    if constexpr (WANTQ) {
        if (chunk < NP) fin[chunk] = flip;
    }
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
    // NaN-free path: one pass over the keys serves the lane's K ranks (at
    // 64 and 128 positions per problem; measured faster than a pass per key
    // here, slower in the LDS-band kernel's 2 to 8 keys per lane)
    int rkf[K];
    static_for<K>([&](auto KK) {
        constexpr int kk = decltype(KK)::value;
        myd[kk] = sd[r + kk * P];
        rkf[kk] = 0;
    });
    if (nonan) {
        for (int k = 0; k < n; ++k) {
            const T dk = sd[k];
            static_for<K>([&](auto KK) {
                constexpr int kk = decltype(KK)::value;
                const int j = r + kk * P;
                rkf[kk] += ((dk < myd[kk]) | ((dk == myd[kk]) & (k < j))) ? 1 : 0;
            });
        }
    }
    static_for<K>([&](auto KK) {
        constexpr int kk = decltype(KK)::value;
        const int j = r + kk * P;
        const T dj = sd[j];
        int rk = rkf[kk];
        if (!nonan) {
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
        // the consumers gather column c of the sorted order from column
        // srank[c] (the inverse permutation; ranks of j < n cover 0..n-1)
        if (j < n) srank[myrank[kk]] = j;
    });
    __builtin_amdgcn_wave_barrier();  // srank is complete
    if (live & lead_wg) {
        // addressed from the wavefront's first problem (scalar) and the
        // chunk index, so no 64-bit problem index stays live through the
        // loop; lane r writes sorted places r, r+P, ... (consecutive lanes,
        // consecutive words) from the inverse permutation: a scattered store
        // at the ranks touched each line several times (2.6x the
        // algorithmic bytes for 256 float matrices of order 512 without
        // eigenvectors)
        T* const glw = glam + first * n;
        static_for<K>([&](auto KK) {
            constexpr int kk = decltype(KK)::value;
            const int c = r + kk * P;
            if (c < n) glw[chunk * n + c] = sd[srank[c]];
        });
        if (args.info != nullptr && r == 0 && !failed) (args.info + first)[chunk] = 0;
    }
    if constexpr (WANTQ) __syncthreads();  // ranks and final parity are visible to the consumers
    STEQR_PHASE_MARK(3);
    STEQR_PHASE_STORE(wave, lane);
}

}  // namespace steqr
