// Device building blocks of the chunked steqr solve for CDNA4 (gfx950).
//
// Everything here runs per lane on values the lane holds in registers; no
// cross-lane operation is involved. Citations name the BatchLAS pages:
//   [algo]  the BatchLAS steqr algorithm page (batched symmetric tridiagonal
//           eigensolvers by implicit shifted QR/QL);
//   [cta]   "STEQR: the CTA tridiagonal solver".
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace steqr {

// Compile-time loop: fn(std::integral_constant<int, i>) for i = 0..COUNT-1.
// Register arrays indexed by the constant stay registers from the first
// optimisation pass on (a plain unrolled loop can be folded into a
// run-time-indexed memory access before it is unrolled).
template <typename Fn, int... Is>
__device__ __forceinline__ void static_for_impl(Fn&& fn, std::integer_sequence<int, Is...>) {
    (fn(std::integral_constant<int, Is>{}), ...);
}
template <int COUNT, typename Fn>
__device__ __forceinline__ void static_for(Fn&& fn) {
    if constexpr (COUNT > 0) static_for_impl(fn, std::make_integer_sequence<int, COUNT>{});
}
// As static_for, but stops after the first index whose body returns false
// (meant for wave-uniform conditions: the stop is one scalar branch).
template <typename Fn, int... Is>
__device__ __forceinline__ void static_for_while_impl(Fn&& fn, std::integer_sequence<int, Is...>) {
    (void)(fn(std::integral_constant<int, Is>{}) && ...);
}
template <int COUNT, typename Fn>
__device__ __forceinline__ void static_for_while(Fn&& fn) {
    if constexpr (COUNT > 0) static_for_while_impl(fn, std::make_integer_sequence<int, COUNT>{});
}

// Largest value over the 64 lanes of the wavefront (every lane active), as
// a wave-uniform scalar: bounds a static loop with one scalar branch. DPP
// lane moves within each row of 16 lanes (swap neighbours, swap pairs,
// mirror 8, mirror 16) leave every lane with its row's maximum; the four
// row maxima are read into scalar registers.
__device__ __forceinline__ int wave_max_uniform(int v) {
    int w = __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);
    v = v > w ? v : w;
    w = __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);
    v = v > w ? v : w;
    w = __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);
    v = v > w ? v : w;
    w = __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false);
    v = v > w ? v : w;
    const int r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
    const int r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
    const int a = r0 > r1 ? r0 : r1, b = r2 > r3 ? r2 : r3;
    return a > b ? a : b;
}

// Precision-dependent constants and hardware helpers.
//  eps2    = eps^2 with eps the unit roundoff (2^-24 / 2^-53)  [algo, deflation]
//  safmin  = smallest normal number                            [algo, deflation]
//  ssfmax  = sqrt(1/safmin)/3, ssfmin = sqrt(safmin)/eps^2     [algo, scaling]
//            (LAPACK's definitions; the page names them only)
template <typename T>
struct Fp;

template <>
struct Fp<float> {
    static constexpr float eps2 = 0x1p-48f;
    static constexpr float safmin = 0x1p-126f;
    static constexpr float ssfmax = 0x1p63f / 3.0f;
    static constexpr float ssfmin = 0x1p-15f;
    // v_rsq_f32 is accurate to about 1 ulp: used as is
    __device__ static __forceinline__ float rsq_refined(float t) { return __builtin_amdgcn_rsqf(t); }
    __device__ static __forceinline__ int frexp_exp(float x) { return __builtin_amdgcn_frexp_expf(x); }
    __device__ static __forceinline__ float ldexp(float x, int k) { return __builtin_amdgcn_ldexpf(x, k); }
    __device__ static __forceinline__ float rsq(float x) { return __builtin_amdgcn_rsqf(x); }
    __device__ static __forceinline__ float rcp(float x) { return __builtin_amdgcn_rcpf(x); }
    // true when x is a positive normal number (v_cmp_class, mask bit 8)
    __device__ static __forceinline__ bool pos_normal(float x) { return __builtin_amdgcn_classf(x, 0x100); }
    // true when x is anything but a positive normal number (every other class bit)
    __device__ static __forceinline__ bool not_pos_normal(float x) { return __builtin_amdgcn_classf(x, 0x2ff); }
    __device__ static __forceinline__ float sqrt_fast(float x) { return __builtin_amdgcn_sqrtf(x); }
    __device__ static __forceinline__ float qnan() { return __builtin_nanf(""); }
    __device__ static __forceinline__ float abs(float x) { return __builtin_fabsf(x); }
    __device__ static __forceinline__ float sqrt(float x) { return __builtin_sqrtf(x); }
    __device__ static __forceinline__ float fma(float a, float b, float c) { return __builtin_fmaf(a, b, c); }
    __device__ static __forceinline__ float max(float a, float b) { return __builtin_fmaxf(a, b); }
    __device__ static __forceinline__ float copysign(float a, float b) { return __builtin_copysignf(a, b); }
    // (a, b) <- (fma(c, a, s b), fma(c, b, -s a)) with each result written
    // over its own input register. Inside a lane-masked region the
    // compiler's accumulate-into-temporary form needs a copy back per value.
    __device__ static __forceinline__ void rot(float& a, float& b, float c, float s) {
        const float sa = s * a, sb = s * b;
        asm("v_fma_f32 %0, %1, %0, %2" : "+v"(a) : "v"(c), "v"(sb));
        asm("v_fma_f32 %0, %1, %0, -%2" : "+v"(b) : "v"(c), "v"(sa));
    }
    // dst <- fma(a, b, c) in dst's register (old value of dst unused)
    __device__ static __forceinline__ void fma_over(float& dst, float a, float b, float c) {
        asm("v_fma_f32 %0, %1, %2, %3" : "+v"(dst) : "v"(a), "v"(b), "v"(c));
    }
    // dst <- fma(a, b, -c) in dst's register (old value of dst unused)
    __device__ static __forceinline__ void fma_over_neg(float& dst, float a, float b, float c) {
        asm("v_fma_f32 %0, %1, %2, -%3" : "+v"(dst) : "v"(a), "v"(b), "v"(c));
    }
    // dst <- dst + a b and dst <- dst - a b, in dst's register
    __device__ static __forceinline__ void fma_acc(float& dst, float a, float b) {
        asm("v_fma_f32 %0, %1, %2, %0" : "+v"(dst) : "v"(a), "v"(b));
    }
    __device__ static __forceinline__ void fma_acc_neg(float& dst, float a, float b) {
        asm("v_fma_f32 %0, -%1, %2, %0" : "+v"(dst) : "v"(a), "v"(b));
    }
};

template <>
struct Fp<double> {
    static constexpr double eps2 = 0x1p-106;
    static constexpr double safmin = 0x1p-1022;
    static constexpr double ssfmax = 0x1p511 / 3.0;
    static constexpr double ssfmin = 0x1p-405;
    // 1/sqrt(t) from the v_rsq_f64 seed (relative error below 2^-24, measured
    // on MI355X over 4M inputs with exponents -900..900) and one third-order
    // step: with
    // r = 1 - t y^2, y' = y (1 + r/2 + 3r^2/8) has error O(r^3), below
    // 2^-52 here (two Newton steps cost 8 operations, this one 5)
    __device__ static __forceinline__ double rsq_refined(double t) {
        const double y = __builtin_amdgcn_rsq(t);
        const double r = __builtin_fma(-(t * y), y, 1.0);
        return __builtin_fma(y * r, __builtin_fma(r, 0.375, 0.5), y);
    }
    __device__ static __forceinline__ int frexp_exp(double x) { return __builtin_amdgcn_frexp_exp(x); }
    __device__ static __forceinline__ double ldexp(double x, int k) { return __builtin_amdgcn_ldexp(x, k); }
    __device__ static __forceinline__ double rsq(double x) { return __builtin_amdgcn_rsq(x); }
    __device__ static __forceinline__ bool pos_normal(double x) { return __builtin_amdgcn_class(x, 0x100); }
    __device__ static __forceinline__ bool not_pos_normal(double x) { return __builtin_amdgcn_class(x, 0x2ff); }
    // double reciprocal / square root: hardware seed refined by Newton steps
    __device__ static __forceinline__ double rcp(double x) {
        double y = __builtin_amdgcn_rcp(x);
        y = __builtin_fma(__builtin_fma(-x, y, 1.0), y, y);
        y = __builtin_fma(__builtin_fma(-x, y, 1.0), y, y);
        return y;
    }
    __device__ static __forceinline__ double sqrt_fast(double x) { return __builtin_sqrt(x); }
    __device__ static __forceinline__ double qnan() { return __builtin_nan(""); }
    __device__ static __forceinline__ double abs(double x) { return __builtin_fabs(x); }
    __device__ static __forceinline__ double sqrt(double x) { return __builtin_sqrt(x); }
    __device__ static __forceinline__ double fma(double a, double b, double c) { return __builtin_fma(a, b, c); }
    __device__ static __forceinline__ double max(double a, double b) { return __builtin_fmax(a, b); }
    __device__ static __forceinline__ double copysign(double a, double b) { return __builtin_copysign(a, b); }
    // (a, b) <- (fma(c, a, s b), fma(c, b, -s a)) with each result written
    // over its own input register, as for float: inside a lane-masked region
    // the compiler's form (accumulate into a temporary) costs a 64-bit copy
    // back per value.
    __device__ static __forceinline__ void rot(double& a, double& b, double c, double s) {
        const double sa = s * a, sb = s * b;
        asm("v_fma_f64 %0, %1, %0, %2" : "+v"(a) : "v"(c), "v"(sb));
        asm("v_fma_f64 %0, %1, %0, -%2" : "+v"(b) : "v"(c), "v"(sa));
    }
    // dst <- fma(a, b, c) in dst's register (old value of dst unused)
    __device__ static __forceinline__ void fma_over(double& dst, double a, double b, double c) {
        asm("v_fma_f64 %0, %1, %2, %3" : "+v"(dst) : "v"(a), "v"(b), "v"(c));
    }
    __device__ static __forceinline__ void fma_over_neg(double& dst, double a, double b, double c) {
        asm("v_fma_f64 %0, %1, %2, -%3" : "+v"(dst) : "v"(a), "v"(b), "v"(c));
    }
    __device__ static __forceinline__ void fma_acc(double& dst, double a, double b) {
        asm("v_fma_f64 %0, %1, %2, %0" : "+v"(dst) : "v"(a), "v"(b));
    }
    __device__ static __forceinline__ void fma_acc_neg(double& dst, double a, double b) {
        asm("v_fma_f64 %0, -%1, %2, %0" : "+v"(dst) : "v"(a), "v"(b));
    }
};

// OR over the P consecutive lanes of a chunk (P a power of two, every lane
// of the wavefront active). Up to 16 lanes the partners come from DPP lane
// moves within a row of 16: swap neighbours, swap pairs (quad permutes),
// then mirror 8 and mirror 16 (after the quad steps each quad holds its OR,
// so a mirror pairs every lane with the other half). Beyond 16 lanes a
// ds_bpermute shuffle finishes.
template <int P>
__device__ __forceinline__ unsigned chunk_or_dpp(unsigned v) {
    static_assert(P >= 1 && P <= 64 && (P & (P - 1)) == 0, "P a power of two");
    if constexpr (P >= 2) v |= (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);
    if constexpr (P >= 4) v |= (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);
    if constexpr (P >= 8) v |= (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false);
    if constexpr (P >= 16) v |= (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false);
    if constexpr (P >= 32) v |= (unsigned)__shfl_xor((int)v, 16, 64);
    if constexpr (P >= 64) v |= (unsigned)__shfl_xor((int)v, 32, 64);
    return v;
}

// ---------------------------------------------------------------- bit masks
// Position masks over the off-diagonal index p (bit p <-> e_p).

typedef unsigned __int128 u128;

// Wide position masks (orders 129..512): W 64-bit words, word i holding
// positions 64i .. 64i+63. The operators are the ones the solver's mask
// arithmetic uses; shifts take run-time counts (word index and bit offset
// selected per lane).
template <int W>
struct uwide {
    static constexpr int WORDS = W;
    uint64_t w[W];
    __device__ constexpr uwide() : w{} {}
    __device__ constexpr uwide(uint64_t v) : w{v} {}
    __device__ uwide operator|(const uwide& o) const {
        uwide r;
        for (int i = 0; i < W; ++i) r.w[i] = w[i] | o.w[i];
        return r;
    }
    __device__ uwide operator&(const uwide& o) const {
        uwide r;
        for (int i = 0; i < W; ++i) r.w[i] = w[i] & o.w[i];
        return r;
    }
    __device__ uwide operator~() const {
        uwide r;
        for (int i = 0; i < W; ++i) r.w[i] = ~w[i];
        return r;
    }
    __device__ uwide& operator|=(const uwide& o) { return *this = *this | o; }
    __device__ uwide& operator&=(const uwide& o) { return *this = *this & o; }
    __device__ bool operator==(const uwide& o) const {
        uint64_t d = 0;
        for (int i = 0; i < W; ++i) d |= w[i] ^ o.w[i];
        return d == 0;
    }
    __device__ bool operator!=(const uwide& o) const { return !(*this == o); }
    __device__ explicit operator bool() const {
        uint64_t d = 0;
        for (int i = 0; i < W; ++i) d |= w[i];
        return d != 0;
    }
    __device__ explicit operator unsigned() const { return (unsigned)w[0]; }
    // word j of the value (0 outside 0..W-1)
    __device__ uint64_t word(int j) const {
        uint64_t r = 0;
        for (int i = W - 1; i >= 0; --i) r = j == i ? w[i] : r;
        return r;
    }
    __device__ uwide operator<<(int k) const {
        const int ws = k >> 6, bs = k & 63;
        uwide r;
        for (int i = 0; i < W; ++i) {
            const uint64_t hi = word(i - ws), lo = word(i - ws - 1);
            r.w[i] = (hi << bs) | ((lo >> 1) >> (63 - bs));
        }
        return r;
    }
    __device__ uwide operator>>(int k) const {
        const int ws = k >> 6, bs = k & 63;
        uwide r;
        for (int i = 0; i < W; ++i) {
            const uint64_t lo = word(i + ws), hi = word(i + ws + 1);
            r.w[i] = (lo >> bs) | ((hi << 1) << (63 - bs));
        }
        return r;
    }
};
typedef uwide<4> u256;
typedef uwide<8> u512;

template <int N>
using PosMask = typename std::conditional<
    (N > 256), u512,
    typename std::conditional<
        (N > 128), u256,
        typename std::conditional<(N > 64), u128,
                                  typename std::conditional<(N > 32), uint64_t,
                                                            uint32_t>::type>::type>::type>::type;

// bits [0, k), 0 <= k <= width
template <typename M>
__device__ __forceinline__ M bits_below(int k) {
    if constexpr (sizeof(M) == 4) {
        return (M)((1ull << k) - 1ull);
    } else if constexpr (sizeof(M) == 8) {
        return k >= 64 ? ~(M)0 : (((M)1 << k) - (M)1);
    } else if constexpr (sizeof(M) == 16) {
        return k >= 128 ? ~(M)0 : (((M)1 << k) - (M)1);
    } else {
        M r;
        for (int i = 0; i < M::WORDS; ++i) {
            const int b = k - 64 * i;  // bits of word i below k
            r.w[i] = b >= 64 ? ~0ull : (b <= 0 ? 0ull : ((1ull << b) - 1ull));
        }
        return r;
    }
}

// bits [lo, hi]; empty when hi < lo (lo >= 0)
template <typename M>
__device__ __forceinline__ M bit_range(int lo, int hi) {
    return hi < lo ? (M)0 : (M)(bits_below<M>(hi + 1) & ~bits_below<M>(lo));
}

// index of the highest / lowest set bit (x != 0)
template <typename M>
__device__ __forceinline__ int msb(M x) {
    if constexpr (sizeof(M) == 4) {
        return 31 - __clz((int)x);
    } else if constexpr (sizeof(M) == 8) {
        return 63 - __clzll((long long)x);
    } else if constexpr (sizeof(M) == 16) {
        const uint64_t hi = (uint64_t)(x >> 64), lo = (uint64_t)x;
        return hi ? 127 - __clzll((long long)hi) : 63 - __clzll((long long)lo);
    } else {
        // the highest nonzero word decides
        int r = 0;
        for (int i = 0; i < M::WORDS; ++i)
            r = x.w[i] ? 64 * i + 63 - __clzll((long long)x.w[i]) : r;
        return r;
    }
}
template <typename M>
__device__ __forceinline__ int lsb(M x) {
    if constexpr (sizeof(M) == 4) {
        return __ffs((int)x) - 1;
    } else if constexpr (sizeof(M) == 8) {
        return __ffsll((long long)x) - 1;
    } else if constexpr (sizeof(M) == 16) {
        const uint64_t hi = (uint64_t)(x >> 64), lo = (uint64_t)x;
        return lo ? __ffsll((long long)lo) - 1 : 63 + __ffsll((long long)hi);
    } else {
        // the lowest nonzero word decides
        int r = 0;
        for (int i = M::WORDS - 1; i >= 0; --i)
            r = x.w[i] ? 64 * i + __ffsll((long long)x.w[i]) - 1 : r;
        return r;
    }
}

template <typename M>
__device__ __forceinline__ int popc(M x) {
    if constexpr (sizeof(M) == 4) return __popc((unsigned)x);
    else if constexpr (sizeof(M) == 8) return __popcll((unsigned long long)x);
    else if constexpr (sizeof(M) == 16)
        return __popcll((unsigned long long)x) + __popcll((unsigned long long)(x >> 64));
    else {
        int r = 0;
        for (int i = 0; i < M::WORDS; ++i) r += __popcll(x.w[i]);
        return r;
    }
}

// bit p set (0 <= p < width)
template <typename M>
__device__ __forceinline__ M bit_at(int p) {
    if constexpr (sizeof(M) <= 16) {
        return (M)1 << p;
    } else {
        M r;
        for (int i = 0; i < M::WORDS; ++i) r.w[i] = (p >> 6) == i ? (1ull << (p & 63)) : 0ull;
        return r;
    }
}
// whether bit p is set
template <typename M>
__device__ __forceinline__ bool bit_test(const M& x, int p) {
    if constexpr (sizeof(M) <= 16) {
        return ((x >> p) & 1) != 0;
    } else {
        return ((x.word(p >> 6) >> (p & 63)) & 1ull) != 0;
    }
}

// ---------------------------------------------------------------- arithmetic

// Deflation test [algo, deflation]: e is negligible between d1 and d2 when
// |e|^2 <= eps^2 |d1| |d2| + safmin. NaN never passes.
template <typename T>
__device__ __forceinline__ bool negligible(T e, T d1, T d2) {
    return e * e <= Fp<T>::eps2 * (Fp<T>::abs(d1) * Fp<T>::abs(d2)) + Fp<T>::safmin;
}

// Givens rotation [algo, "G(c,s)" paragraph]: G(c,s) = [[c,-s],[s,c]],
// G^T (f, g)^T = (r, 0)^T with r = sqrt(f^2 + g^2) >= 0 (c takes the sign
// of f). The pages' convention (r with the sign of f, c >= 0) differs by the
// rotation -G, which gives the same similarity and flips the signs of two
// Q columns and of an off-diagonal entry only; the plain one saves the sign
// transfer at every step.
//
// Scaled form (always valid): f and g are first scaled by an exact power of
// two (2^-k with k the exponent of |f| + |g|, which lies within a factor 2
// of max(|f|,|g|)) so that f^2 + g^2 lies in [1/16, 1] and can neither
// overflow nor underflow; the norm is a hardware reciprocal square root
// (refined in double, see rsq_refined) [cta, Givens rotation paragraph]; g = 0 gives
// the identity rotation with r = f, by a final select [cta, Givens rotation
// paragraph]. NaN
// inputs give NaN outputs. |f| + |g| cannot overflow for the block-scaled
// values the solver passes (|f|, |g| stay within a small multiple of ssfmax).
template <typename T>
__device__ __forceinline__ void lartg_scaled(T f, T g, T& c, T& s, T& r) {
    using F = Fp<T>;
    const T mx = F::abs(f) + F::abs(g);
    const int ex = F::frexp_exp(mx);
    const T fs = F::ldexp(f, -ex);
    const T gs = F::ldexp(g, -ex);
    const T t = fs * fs + gs * gs;
    const T y = F::rsq_refined(t);
    const bool gz = (g == T(0));
    c = gz ? T(1) : fs * y;
    s = gz ? T(0) : gs * y;
    r = gz ? f : F::ldexp(t * y, ex);
}

// Givens rotation, fast form: t = f^2 + g^2 directly; whenever t is not a
// positive normal number (overflow, underflow, zero or NaN) the lanes
// concerned take the scaled form above. The test is one ballot and a
// scalar branch the wavefront skips when no active lane needs the scaled
// form (UNIFORM: every lane holds the same (f, g), one lane decides). With
// t normal the unscaled formulas are exact to a few ulps, g = 0 included
// (c = f / |f| = +-1, s = 0, r = |f|: a valid rotation, like the scaled
// form's (1, 0, f)).
template <typename T, bool UNIFORM = false>
__device__ __forceinline__ void lartg(T f, T g, T& c, T& s, T& r) {
    using F = Fp<T>;
    const T t = F::fma(f, f, g * g);
    const T y = F::rsq_refined(t);
    c = f * y;
    s = g * y;
    r = t * y;
    if constexpr (UNIFORM) {
        // every lane holds the same (f, g): the ballot is all or nothing
        if (__builtin_amdgcn_ballot_w64(F::not_pos_normal(t))) lartg_scaled(f, g, c, s, r);
    } else {
        const bool slow = F::not_pos_normal(t);
        if (__builtin_amdgcn_ballot_w64(slow)) {
            T c2, s2, r2;
            lartg_scaled(f, g, c2, s2, r2);
            c = slow ? c2 : c;
            s = slow ? s2 : s;
            r = slow ? r2 : r;
        }
    }
}

// LAPACK-form shift [algo, shift section]: the eigenvalue of the 2x2 block
// [[d2, e1], [e1, d1]] nearest the endpoint d1,
//   g = (d2 - d1)/(2 e1), r = sqrt(g^2 + 1), mu = d1 - e1/(g + copysign(r, g)).
// The shift only steers convergence, so hardware reciprocal and square
// root (about 1 ulp) replace the correctly rounded forms. If g^2 overflows
// (or e1 = 0 makes g infinite), r = inf and mu = d1, which is harmless.
template <typename T>
__device__ __forceinline__ T lapack_shift(T d1, T d2, T e1) {
    using F = Fp<T>;
    const T g = (d2 - d1) * F::rcp(T(2) * e1);
    const T r = F::sqrt_fast(F::fma(g, g, T(1)));
    return d1 - e1 * F::rcp(g + F::copysign(r, g));
}

// EXP step of the chase [algo, similarity paragraph]: the congruence G^T B G
// of the 2x2 block B = [[a, b], [b, dd]] by the rotation (c, s), written with
// c^2 + s^2 = 1 (which the rotation satisfies to rounding):
//   w = s (dd - a) + 2 c b,  a' = a + s w,  dd' = dd - s w,  b' = c w - b,
// the same values as c^2 a + 2cs b + s^2 dd, s^2 a - 2cs b + c^2 dd and
// cs (dd - a) + (c^2 - s^2) b with three multiplications fewer.
template <typename T>
__device__ __forceinline__ T exp_step_w(T c, T s, T a, T b, T dd) {
    const T cb = c * b;
    return Fp<T>::fma(s, dd - a, cb) + cb;
}

// Closed-form shift [algo, shift section]: for the trailing block
// B = [[a, b], [b, c]] (a = d2, b = e1, c = d1 at the converging end),
// lambda+- = (a+c)/2 +- sqrt(((a-c)/2)^2 + b^2); the one nearer c. The block
// is scaled, so the squares cannot overflow.
template <typename T>
__device__ __forceinline__ T closed_shift(T d1, T d2, T e1) {
    using F = Fp<T>;
    const T h = (d2 + d1) * T(0.5), hd = (d2 - d1) * T(0.5);
    const T r = F::sqrt_fast(F::fma(hd, hd, e1 * e1));
    const T lp = h + r, lm = h - r;
    return (F::abs(lp - d1) < F::abs(lm - d1)) ? lp : lm;
}

// The shift of one sweep: the LAPACK form, or the closed form when
// `closed` (a kernel argument, uniform).
template <typename T>
__device__ __forceinline__ T sweep_shift(bool closed, T d1, T d2, T e1) {
    if (closed) return closed_shift(d1, d2, e1);
    return lapack_shift(d1, d2, e1);
}

// Analytic 2x2 solve [algo, 2x2 block paragraph]: for
// B = [[a, b], [b, c]] the symmetric Schur rotation J = [[cs, sn], [-sn, cs]]
// with J^T B J = diag(a - t b, c + t b), tau = (c - a)/(2b),
// t = sign(tau)/(|tau| + sqrt(1 + tau^2)) (sign(0) = +1), cs = 1/sqrt(1+t^2),
// sn = t cs (Golub and Van Loan, symmetric Schur decomposition). b = 0
// gives the identity. Hardware reciprocal / square root as in the shift.
template <typename T>
__device__ __forceinline__ void sym2x2(T a, T b, T c, T& rt1, T& rt2, T& cs, T& sn) {
    using F = Fp<T>;
    const T tau = (c - a) * F::rcp(T(2) * b);
    const T den = F::abs(tau) + F::sqrt_fast(F::fma(tau, tau, T(1)));
    T t = F::copysign(F::rcp(den), tau >= T(0) ? T(1) : T(-1));
    t = (b == T(0)) ? T(0) : t;
    const T y = F::rsq_refined(F::fma(t, t, T(1)));
    cs = y;
    sn = t * y;
    rt1 = a - t * b;
    rt2 = c + t * b;
}

// Initial columns c0 .. c0+W-1 of row `row` of Q [algo, eigenvector
// accumulation]: the identity row without back-transformation; with it, the
// caller's basis Z (qb = the problem's n x n row-major block, in bounds).
// Rows and columns at or beyond n are padding and always start as the
// identity, as do rows of dead problems (ok = false). With n equal to the
// compiled order and a 16-byte aligned block (`vec`) the row is read as
// whole 16-byte pieces (c0 a multiple of 4).
template <typename T, int W>
__device__ __forceinline__ void load_basis_cols(const T* __restrict__ qb, int n, int row, int c0,
                                                bool ok, bool bt, bool vec, T (&q)[W]) {
    const bool in = bt & ok & (row < n);
    if (!in) {
        static_for<W>([&](auto J) {
            constexpr int j = decltype(J)::value;
            q[j] = (row == c0 + j) ? T(1) : T(0);
        });
        return;
    }
    const T* src = qb + (long)row * n + c0;
    if (vec) {
        constexpr int V = 16 / sizeof(T);
        static_for<W / V>([&](auto K) {
            constexpr int k = decltype(K)::value;
            if constexpr (sizeof(T) == 4) {
                const float4 v = *reinterpret_cast<const float4*>(src + k * 4);
                q[k * 4 + 0] = v.x;
                q[k * 4 + 1] = v.y;
                q[k * 4 + 2] = v.z;
                q[k * 4 + 3] = v.w;
            } else {
                const double2 v = *reinterpret_cast<const double2*>(src + k * 2);
                q[k * 2 + 0] = v.x;
                q[k * 2 + 1] = v.y;
            }
        });
    } else {
        static_for<W>([&](auto J) {
            constexpr int j = decltype(J)::value;
            const int jc = (c0 + j < n) ? j : n - 1 - c0;
            const T v = src[jc > 0 ? jc : 0];
            q[j] = (c0 + j < n) ? v : T(0);
        });
    }
}

template <typename T, int N>
__device__ __forceinline__ void load_basis_row(const T* __restrict__ qb, int n, int row, bool ok,
                                               bool bt, bool vec, T (&q)[N]) {
    load_basis_cols<T, N>(qb, n, row, 0, ok, bt, vec, q);
}

}  // namespace steqr
