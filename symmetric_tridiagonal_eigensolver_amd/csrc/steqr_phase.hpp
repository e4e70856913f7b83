// Phase timers of the kernels' profiling build. The library is built with
// STEQR_PHASE_TIMERS 0: every STEQR_PHASE_* statement below expands to
// nothing and the kernels' code is exactly that of a source without them.
// The profiling build (probes/steqr_phase_probe.hip, driven by
// profile_phases.py) sets it to 1: each wavefront then adds up the shader
// clock cycles (s_memtime) between consecutive marks per phase slot and
// lane 0 stores the slots to phase_out[wavefront * STEQR_PHASE_SLOTS + slot]:
// 0..6 the kernel's own, 7 and 8 the wavefront's start and end times on the
// constant 100 MHz counter (s_memrealtime, common to the whole GPU).
#pragma once

#ifndef STEQR_PHASE_TIMERS
#define STEQR_PHASE_TIMERS 0
#endif

#if STEQR_PHASE_TIMERS
#include <hip/hip_runtime.h>

namespace steqr {

#define STEQR_PHASE_SLOTS 9

// per-wavefront slots of the current launch (set by the host before it)
static __device__ unsigned long long* phase_out;

struct PhaseClock {
    unsigned long long t0, acc[STEQR_PHASE_SLOTS];
    __device__ __forceinline__ void start() {
        for (int k = 0; k < 7; ++k) acc[k] = 0;
        acc[7] = __builtin_amdgcn_s_memrealtime();
        t0 = __builtin_readcyclecounter();
    }
    // add the cycles since the last mark to slot k
    __device__ __forceinline__ void mark(int k) {
        const unsigned long long t = __builtin_readcyclecounter();
        acc[k] += t - t0;
        t0 = t;
    }
    __device__ __forceinline__ void add(int k, unsigned long long v) { acc[k] += v; }
    __device__ __forceinline__ void store(int wave, int lane) {
        acc[8] = __builtin_amdgcn_s_memrealtime();
        const long w = (long)blockIdx.x * (blockDim.x >> 6) + wave;
        if (phase_out != nullptr && lane == 0)
            for (int k = 0; k < STEQR_PHASE_SLOTS; ++k) phase_out[w * STEQR_PHASE_SLOTS + k] = acc[k];
    }
};

}  // namespace steqr

#define STEQR_PHASE_START ::steqr::PhaseClock phase_clk; phase_clk.start()
#define STEQR_PHASE_MARK(k) phase_clk.mark(k)
#define STEQR_PHASE_ADD(k, v) phase_clk.add(k, v)
#define STEQR_PHASE_STORE(wave, lane) phase_clk.store(wave, lane)
#else
#define STEQR_PHASE_START ((void)0)
#define STEQR_PHASE_MARK(k) ((void)0)
#define STEQR_PHASE_ADD(k, v) ((void)0)
#define STEQR_PHASE_STORE(wave, lane) ((void)0)
#endif
