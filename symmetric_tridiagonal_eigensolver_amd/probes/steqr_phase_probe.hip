// Profiling build of four default kernels with their phase timers switched
// on, and dependent-chain latency kernels; not part of libsteqr.so. Built
// and driven by profile_phases.py at the repository root, which checks that
// each kernel here is the one the library's default plan launches for the
// workload it profiles.
#define STEQR_PHASE_TIMERS 1
#include "../csrc/steqr_registry.hpp"

namespace {

using steqr::KernelArgs;
using LaunchFn = steqr::LaunchFn;

// which: 0 chunked <float, 16, 4 lanes, vectors> (16,384 x order 16)
//        1 producer-consumer <double, 64, 11 consumers, 4 lanes> (order 64)
//        2 producer-consumer <double, 128, 8 consumers, 32 lanes> (order 128)
//        3 producer-consumer <float, 128, 10 consumers, 8 lanes, whole rows>
//        4 chunked <float, 16, 2 lanes, values only>
//        5 chunked <double, 32, 1 lane, values only>
//        6 producer-consumer <float, 256, 8 consumers, 64 lanes>
//        7 producer-consumer <double, 256, 8 consumers, 64 lanes> (two
//          workgroups per problem)
//        8 producer-consumer <float, 512, 8 consumers, 64 lanes> (eight
//          workgroups per problem)
//        9 producer-consumer <double, 512, 8 consumers, 64 lanes> (sixteen
//          workgroups per problem)
LaunchFn kernel_of(int which) {
    switch (which) {
        case 0: return &steqr::launch_chunk<float, 16, 4, true, false>;
        case 1: return &steqr::launch_pc<double, 64, 11, 4, false>;
        case 2: return &steqr::launch_pc<double, 128, 8, 32, false>;
        case 3: return &steqr::launch_pc<float, 128, 10, 8, false, 1>;
        case 4: return &steqr::launch_chunk<float, 16, 2, false, false>;
        case 5: return &steqr::launch_chunk<double, 32, 1, false, false>;
        case 6: return &steqr::launch_pc<float, 256, 8, 64, false>;
        case 7: return &steqr::launch_pc<double, 256, 8, 64, false>;
        case 8: return &steqr::launch_pc<float, 512, 8, 64, false>;
        case 9: return &steqr::launch_pc<double, 512, 8, 64, false>;
        default: return nullptr;
    }
}

// One wavefront times `iters` x 16 dependent operations of one kind: 0
// double FMA, 1 double reciprocal square root (the hardware instruction),
// 2 the solver's refined double reciprocal square root, 3 float FMA, 4
// float reciprocal square root (x -> 1/sqrt(x) stays positive and tends to
// 1). cycles[0] is the shader clock counter's advance (s_memtime), cycles[1]
// the constant 100 MHz counter's (s_memrealtime) over the same chain.
template <int KIND>
__global__ void __launch_bounds__(64) latency_kernel(int iters, double seed, double* out,
                                                     unsigned long long* cycles) {
    double x = seed + threadIdx.x * 1e-3;
    float xf = (float)x;
    const double a = 0.999999, b = 1e-7;
    const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
    const unsigned long long t0 = __builtin_readcyclecounter();
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            if constexpr (KIND == 0) x = __builtin_fma(x, a, b);
            if constexpr (KIND == 1) x = __builtin_amdgcn_rsq(x);
            if constexpr (KIND == 2) x = steqr::Fp<double>::rsq_refined(x);
            if constexpr (KIND == 3) xf = __builtin_fmaf(xf, (float)a, (float)b);
            if constexpr (KIND == 4) xf = __builtin_amdgcn_rsqf(xf);
        }
    }
    // the chain's result is needed here, before the second clock read
    asm volatile("" : "+v"(x), "+v"(xf));
    const unsigned long long t1 = __builtin_readcyclecounter();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    out[threadIdx.x] = x + (double)xf;
    if (threadIdx.x == 0) {
        cycles[0] = t1 - t0;
        cycles[1] = r1 - r0;
    }
}

}  // namespace

extern "C" int steqr_phase_launch(int which, const void* d, const void* e, void* lambda, void* Q,
                                  int* info, int n, int batch, int grid, int block,
                                  unsigned long long* phase, hipStream_t stream) {
    const LaunchFn fn = kernel_of(which);
    if (fn == nullptr) return -1;
    if (d == nullptr || e == nullptr || lambda == nullptr || phase == nullptr) return -2;
    if ((which <= 3 || which >= 6) && Q == nullptr) return -2;  // kernels with eigenvectors
    if (n < 1 || batch < 1 || grid < 1 || block < 64 || (block % 64) != 0) return -3;
    KernelArgs a{};
    a.d = d;
    a.e = e;
    a.lam = lambda;
    a.q = Q;
    a.info = info;
    a.n = n;
    a.batch = batch;
    a.max_sweeps_per_n = 30;
    a.do_sort = 1;
    (void)hipGetLastError();
    hipError_t err = hipMemcpyToSymbol(HIP_SYMBOL(steqr::phase_out), &phase, sizeof(phase));
    if (err != hipSuccess) return (int)err;
    err = fn(a, grid, block, stream);
    return err == hipSuccess ? 0 : (int)err;
}

// Hardware seeds of the double reciprocal (kind 0) and reciprocal square
// root (kind 1), one value per thread, for their accuracy against exact
// results computed on the host.
__global__ void __launch_bounds__(256) seed_kernel(int kind, const double* x, double* y, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) y[i] = kind == 0 ? __builtin_amdgcn_rcp(x[i]) : __builtin_amdgcn_rsq(x[i]);
}

extern "C" int steqr_seed_launch(int kind, const double* x, double* y, int n,
                                 hipStream_t stream) {
    if (kind < 0 || kind > 1 || x == nullptr || y == nullptr || n < 1) return -1;
    (void)hipGetLastError();
    hipLaunchKernelGGL(seed_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, kind, x, y, n);
    const hipError_t err = hipGetLastError();
    return err == hipSuccess ? 0 : (int)err;
}

extern "C" int steqr_latency_launch(int kind, int iters, double* out,
                                    unsigned long long* cycles, hipStream_t stream) {
    if (kind < 0 || kind > 4 || iters < 1 || out == nullptr || cycles == nullptr) return -1;
    (void)hipGetLastError();
    switch (kind) {
        case 0: hipLaunchKernelGGL(latency_kernel<0>, dim3(1), dim3(64), 0, stream, iters, 0.75, out, cycles); break;
        case 1: hipLaunchKernelGGL(latency_kernel<1>, dim3(1), dim3(64), 0, stream, iters, 0.75, out, cycles); break;
        case 2: hipLaunchKernelGGL(latency_kernel<2>, dim3(1), dim3(64), 0, stream, iters, 0.75, out, cycles); break;
        case 3: hipLaunchKernelGGL(latency_kernel<3>, dim3(1), dim3(64), 0, stream, iters, 0.75, out, cycles); break;
        default: hipLaunchKernelGGL(latency_kernel<4>, dim3(1), dim3(64), 0, stream, iters, 0.75, out, cycles); break;
    }
    const hipError_t err = hipGetLastError();
    return err == hipSuccess ? 0 : (int)err;
}
