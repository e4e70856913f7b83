/*
 * CPU oracle for the batched symmetric tridiagonal eigensolver.
 *
 * TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
 * CPU-baseline leg load this library; the GPU library never does. Build:
 *   gcc -O2 -ffp-contract=off -fno-fast-math -fPIC -shared \
 *       -o liboracle_steqr.so steqr_oracle.c -lm
 * The algorithm body lives in steqr_oracle_impl.h (the tridiagonal solve)
 * syev_oracle_impl.h (the dense front end) and stebz_oracle_impl.h (values-
 * only bisection) and is instantiated here for
 * float (REAL = float, every operation in IEEE single precision) and
 * double.
 */
#include <float.h>
#include <math.h>
#include <stdlib.h>

#if defined(__FAST_MATH__) || defined(__FINITE_MATH_ONLY__) && __FINITE_MATH_ONLY__
#error "the oracle must be built without fast-math: NaN tests must hold"
#endif

#define REAL float
#define SFX(name) name##_f32
#define R_EPS (FLT_EPSILON * 0.5f)
#define R_SAFMIN FLT_MIN
#define R_SQRT sqrtf
#define R_FABS fabsf
#define R_HYPOT hypotf
#define R_COPYSIGN copysignf
#include "steqr_oracle_impl.h"
#include "syev_oracle_impl.h"
#include "stebz_oracle_impl.h"
#undef REAL
#undef SFX
#undef R_EPS
#undef R_SAFMIN
#undef R_SQRT
#undef R_FABS
#undef R_HYPOT
#undef R_COPYSIGN

#define REAL double
#define SFX(name) name##_f64
#define R_EPS (DBL_EPSILON * 0.5)
#define R_SAFMIN DBL_MIN
#define R_SQRT sqrt
#define R_FABS fabs
#define R_HYPOT hypot
#define R_COPYSIGN copysign
#include "steqr_oracle_impl.h"
#include "syev_oracle_impl.h"
#include "stebz_oracle_impl.h"

/* Constants as the oracle computes them, for the pins. */
void oracle_constants_f32(float *out5)
{
    out5[0] = c_eps_f32();
    out5[1] = c_safmin_f32();
    out5[2] = c_ssfmax_f32();
    out5[3] = c_ssfmin_f32();
    out5[4] = c_eps2_f32();
}

void oracle_constants_f64(double *out5)
{
    out5[0] = c_eps_f64();
    out5[1] = c_safmin_f64();
    out5[2] = c_ssfmax_f64();
    out5[3] = c_ssfmin_f64();
    out5[4] = c_eps2_f64();
}
