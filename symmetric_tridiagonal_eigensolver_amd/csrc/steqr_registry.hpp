// Launch registry: one entry per compiled (dtype, padded order, lanes per
// problem, jobz) kernel instantiation. The instantiation units
// (steqr_inst_*.hip) each export a table; steqr_api.hip searches them.
#pragma once

#include <hip/hip_runtime.h>

#include "steqr_chunk.hpp"
#include "steqr_wave.hpp"
#include "steqr_chunkl.hpp"
#include "steqr_pc.hpp"
#include "steqr_bisect.hpp"

namespace steqr {

typedef hipError_t (*LaunchFn)(const KernelArgs& args, int grid, int block, hipStream_t stream);

// Each instantiation unit is compiled twice: once for the EXP form of the
// chase step (STEQR_INST_PG 0) and once for the PG form (STEQR_INST_PG 1,
// the *_pg.hip units), giving one table per unit and scheme.
#ifndef STEQR_INST_PG
#define STEQR_INST_PG 0
#endif

struct Entry {
    int dtype;             // 0 = float, 1 = double
    int N;                 // compile-time (padded) order
    int P;                 // lanes per problem
    int jobz;              // 0 = values, 1 = values and vectors
    int band;              // 1 = band replicated in VGPRs, 2 = band in LDS,
                           // 3 = band in LDS, producer and consumer wavefronts
    int lds_per_wave;      // bytes of LDS each wavefront uses (band 3: each workgroup)
    LaunchFn fn;
    int pc_np = 0;         // band 3: problems per workgroup
    int pc_waves = 0;      // band 3: wavefronts per workgroup (consumers + producer)
    int pc_gpp = 1;        // band 3: workgroups sharing one problem (rows split)
};

template <typename T, int N, int P, bool WANTQ, bool PG, bool DENSE = false>
hipError_t launch_chunk(const KernelArgs& args, int grid, int block, hipStream_t stream) {
    const size_t lds = (size_t)(block / 64) * Smem<T, N, P, WANTQ, DENSE>::bytes_per_wave;
    hipLaunchKernelGGL((steqr_chunk_kernel<T, N, P, WANTQ, PG, DENSE>), dim3(grid), dim3(block),
                       lds, stream, args);
    return hipGetLastError();
}

// Fused dense eigensolver (reduction + solve + back-transformation), chunked
// kernel with the band in registers, EXP form of the step.
#define STEQR_SYEV_ENTRY(DT, T, N, P, Q) \
    { DT, N, P, Q, 1, (int)Smem<T, N, P, (Q) != 0, true>::bytes_per_wave, \
      &launch_chunk<T, N, P, (Q) != 0, false, true> }

// The fused dense solver with the band in LDS (where the replicated band
// would not fit the register file next to the rows of A and Q).
#define STEQR_SYEV_LENTRY(DT, T, N, P, Q) \
    { DT, N, P, Q, 2, (int)SmemL<T, N, P>::bytes_per_wave, \
      &launch_chunkl<T, N, P, (Q) != 0, false, true> }

// One problem per wavefront (P = 64).
template <typename T, int N, bool WANTQ, bool PG>
hipError_t launch_wave(const KernelArgs& args, int grid, int block, hipStream_t stream) {
    const size_t lds = (size_t)(block / 64) * WaveSmem<T, N>::bytes_per_wave;
    hipLaunchKernelGGL((steqr_wave_kernel<T, N, WANTQ, PG>), dim3(grid), dim3(block), lds,
                       stream, args);
    return hipGetLastError();
}

#define STEQR_WAVE_ENTRY(DT, T, N, Q) \
    { DT, N, 64, Q, 2, (int)WaveSmem<T, N>::bytes_per_wave, \
      &launch_wave<T, N, (Q) != 0, STEQR_INST_PG != 0> }

// Chunked, band in LDS.
template <typename T, int N, int P, bool WANTQ, bool PG, bool DENSE = false>
hipError_t launch_chunkl(const KernelArgs& args, int grid, int block, hipStream_t stream) {
    const size_t lds = (size_t)(block / 64) * SmemL<T, N, P>::bytes_per_wave;
    hipLaunchKernelGGL((steqr_chunkl_kernel<T, N, P, WANTQ, PG, DENSE>), dim3(grid), dim3(block),
                       lds, stream, args);
    return hipGetLastError();
}

#define STEQR_LENTRY(DT, T, N, P, Q) \
    { DT, N, P, Q, 2, (int)SmemL<T, N, P>::bytes_per_wave, \
      &launch_chunkl<T, N, P, (Q) != 0, STEQR_INST_PG != 0> }

// Producer-consumer with eigenvectors: W consumer wavefronts (RS lanes per
// row of Q) and one producer per workgroup; the grid and block are given
// by the caller.
template <typename T, int N, int W, int P, bool PG, int RS = pc_default_rs<T, N>()>
hipError_t launch_pc(const KernelArgs& args, int grid, int block, hipStream_t stream) {
    constexpr size_t lds = SmemPC<T, N, W, P, RS>::bytes;
    hipLaunchKernelGGL((steqr_pc_kernel<T, N, W, P, PG, true, RS>), dim3(grid), dim3(block), lds,
                       stream, args);
    return hipGetLastError();
}

// Values only at order 128: the producer's algorithm in every wavefront.
template <typename T, int N, int P, bool PG>
hipError_t launch_pcv(const KernelArgs& args, int grid, int block, hipStream_t stream) {
    const size_t lds = (size_t)(block / 64) * SmemPV<T, N, P>::bytes_per_wave;
    hipLaunchKernelGGL((steqr_pc_kernel<T, N, 0, P, PG, false>), dim3(grid), dim3(block), lds,
                       stream, args);
    return hipGetLastError();
}

#define STEQR_PCV_ENTRY(DT, T, N, P) \
    { DT, N, P, 0, 2, (int)SmemPV<T, N, P>::bytes_per_wave, \
      &launch_pcv<T, N, P, STEQR_INST_PG != 0> }

#define STEQR_PC_ENTRY(DT, T, N, W, P) \
    { DT, N, P, 1, 3, (int)SmemPC<T, N, W, P>::bytes, \
      &launch_pc<T, N, W, P, STEQR_INST_PG != 0>, SmemPC<T, N, W, P>::NP, (W) + 1, \
      SmemPC<T, N, W, P>::GPP }

// The same with RS lanes per row of Q chosen explicitly (order 128 with
// whole rows per lane: RS = 1).
#define STEQR_PCR_ENTRY(DT, T, N, W, P, RS) \
    { DT, N, P, 1, 3, (int)SmemPC<T, N, W, P, RS>::bytes, \
      &launch_pc<T, N, W, P, STEQR_INST_PG != 0, RS>, SmemPC<T, N, W, P, RS>::NP, (W) + 1, \
      SmemPC<T, N, W, P, RS>::GPP }

#define STEQR_ENTRY(DT, T, N, P, Q) \
    { DT, N, P, Q, 1, (int)Smem<T, N, P, (Q) != 0>::bytes_per_wave, \
      &launch_chunk<T, N, P, (Q) != 0, STEQR_INST_PG != 0> }

// Values-only bisection: one lane per eigenvalue index (N / 64 per lane
// from order 128), min(N, 64) lanes per problem; from order 128 also G
// wavefronts of one workgroup per problem (64 G lanes, N / (64 G) indices
// per lane; the workgroup holds whole problems).
template <typename T, int N, int G = 1>
hipError_t launch_bisect(const KernelArgs& args, int grid, int block, hipStream_t stream) {
    const size_t lds = (size_t)(block / 64) * SmemB<T, N>::bytes_per_wave;
    hipLaunchKernelGGL((steqr_bisect_kernel<T, N, G>), dim3(grid), dim3(block), lds, stream, args);
    return hipGetLastError();
}

#define STEQR_BISECT_ENTRY(DT, T, N) \
    { DT, N, (N) < 64 ? (N) : 64, 0, (2 * N * (int)sizeof(T) / 4 <= 128) ? 1 : 2, \
      (int)SmemB<T, N>::bytes_per_wave, &launch_bisect<T, N> }

#define STEQR_BISECT_G_ENTRY(DT, T, N, G) \
    { DT, N, 64 * (G), 0, (2 * N * (int)sizeof(T) / 4 <= 128) ? 1 : 2, \
      (int)SmemB<T, N>::bytes_per_wave, &launch_bisect<T, N, G> }

struct Table {
    const Entry* entries;
    int count;
};

Table table_f32_v();
Table table_f32_n();
Table table_f64_v();
Table table_f64_n();
Table table_wave();
Table table_lds_f32();
Table table_lds_f64();
Table table_pc();
Table table_f32_v_pg();
Table table_f32_n_pg();
Table table_f64_v_pg();
Table table_f64_n_pg();
Table table_wave_pg();
Table table_lds_f32_pg();
Table table_lds_f64_pg();
Table table_pc_pg();
Table table_big();
Table table_big_pg();
Table table_huge();
Table table_huge_pg();
Table table_n512();
Table table_n512_pg();
Table table_syev_f32();
Table table_syev_f64();
Table table_bisect();

// table name for the scheme this unit is compiled for
#if STEQR_INST_PG
#define STEQR_TABLE(name) name##_pg
#else
#define STEQR_TABLE(name) name
#endif

}  // namespace steqr
