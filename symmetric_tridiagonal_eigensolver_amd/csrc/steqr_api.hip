// C ABI of the batched steqr library: argument checks, launch-shape choice
// and dispatch to the compiled kernel instantiations. The declarations and
// the documentation of every entry point are in include/steqr.h.
#include <hip/hip_runtime.h>

#include "../../include/steqr.h"
#include "steqr_registry.hpp"

namespace {

using steqr::Entry;
using steqr::Table;

// Compile-time orders the build provides, smallest first.
constexpr int kOrders[] = {4, 8, 16, 32, 64, 128, 256, 512};

// The compiled order a problem of order n runs at. Orders 9..12 in double
// with eigenvectors have their own instantiation (order 12, 3 rows of Q per
// lane): padded to 16, a block mirrored for its QL direction lands on
// positions 4..15 while unmirrored ones occupy 0..11, so the lockstep pass
// spans both ranges (1.44x the instructions of the lockstep ideal).
int padded_order(int n, int dtype = -1, int jobz = -1) {
    if (n > 8 && n <= 12 && dtype == STEQR_F64 && jobz == STEQR_V) return 12;
    for (int N : kOrders)
        if (n <= N) return N;
    return -1;
}

// Default lanes per problem P, measured on MI355X at the benchmark batches
// (32,768-65,536 matrices). With eigenvectors, fewer lanes per problem
// means more problems per wavefront and less repeated chase arithmetic, at
// the price of R = N/P rows of Q per lane in VGPRs; the best balance is
// four to eight rows per lane while the wavefront still fits two waves per
// SIMD. Values only keep one lane per problem in double and at orders up to
// 8, two at order 16 and four at order 32 in float (measured). At orders
// 33..512 P counts the producer lanes of the producer-consumer kernel (with
// or without its consumers); P = 64 selects one problem per wavefront at
// orders 33..64.
// The smallest of the ascending lane counts cand[0..k) whose launch has at
// least T wavefronts (batch * P / 64), else the largest.
int fill_lanes(long batch, const int* cand, int k, long T) {
    for (int i = 0; i < k; ++i)
        if (batch * cand[i] >= T * 64) return cand[i];
    return cand[k - 1];
}

int default_lanes(int dtype, int N, int jobz, int band, long batch) {
    // orders 256 and 512: one problem per producer wavefront (without
    // eigenvectors 1024 matrices of order 256 took 6.52 ms in float at 64
    // lanes, 6.79 at 32, 6.59 at 16; double 9.48, 9.65, 9.55)
    if (N >= 256) return 64;
    // order 128, producer lanes per problem: float with eigenvectors runs
    // whole rows of Q per lane (5 problems per producer at 8 lanes each);
    // double with eigenvectors measured 1.4% faster at 32 than at 16
    if (N == 128) {
        // float with eigenvectors: whole rows (5 problems per workgroup,
        // one workgroup per CU) unless the batch leaves most CUs idle, then
        // half rows at 32 producer lanes (2 per workgroup): 512 matrices
        // 1.89 against 2.02 ms, 1,024 matrices 3.76 against 2.05
        if (band == 3) return dtype == STEQR_F32 ? (batch <= 512 ? 32 : 8) : 32;
        // values only in float: 8 lanes once they still give 2,048
        // wavefronts (16,384 matrices: 1.96 ms against 2.53 at 16 lanes)
        if (dtype == STEQR_F32 && !jobz) {
            static const int c[] = {8, 16};
            return fill_lanes(batch, c, 2, 2048);
        }
        return 16;
    }
    // producer lanes per problem at order 64 with eigenvectors; in double
    // 4 lanes (11 problems per workgroup) while that still gives 256
    // workgroups, else 16 (3 per workgroup, more CUs busy: 1,024 matrices
    // 0.79 ms against 0.84 at 4 lanes, 256 matrices 0.75 against 0.82)
    if (band == 3) {
        if (dtype == STEQR_F32) return 16;
        return batch >= 256L * 11 ? 4 : 16;
    }
    // order 64 without eigenvectors: the producer's algorithm, 4 to 16
    // problems per wavefront (measured 2.9x (float) and 4x (double) faster
    // than one problem per wavefront), the fewest lanes whose launch has
    // 2,048 wavefronts: 8 at 16,384 matrices; 65,536 matrices 1.18 ms at 4
    // lanes against 1.42 at 8 (float), 2.89 against 3.15 (double); 4,096
    // matrices 0.48 at 16 against 0.51 at 8 (float), 0.69 against 0.74
    if (N == 64 && !jobz && band == 2) {
        static const int c[] = {4, 8, 16};
        return fill_lanes(batch, c, 3, 2048);
    }
    if (N == 64 && !jobz) return 8;
    if (N >= 64) return 64;
    // Orders 8..32 in their default band storage: the lanes per problem
    // follow the batch. Fewer lanes repeat less of the serial chase, more
    // lanes spread a small batch over more SIMDs, so the default is the
    // fewest lanes whose launch still has T wavefronts (all 1,024 SIMDs
    // busy, two wavefronts each where the kernel hides latency with a
    // second one). Each (candidates, T) reproduces the tuned choice at the
    // configurations' batches (65,536 at order 8, 32,768 above) and was
    // swept from 512 to 262,144 matrices on one MI355X, e.g. order 16 in
    // float with eigenvectors: 63.1 us at 16 lanes against 73.0 at 4 on
    // 8,192 matrices, 71.7 at 8 against 76.6 at 4 on 16,384; without
    // eigenvectors 1.00 / 0.56 / 0.40 ns per matrix at one lane against
    // 1.06 / 0.74 / 0.64 at two on 65,536 / 131,072 / 262,144; order 32
    // without eigenvectors 3.62 ns per matrix at two lanes against 4.11 at
    // four on 65,536, 2.05 at one against 3.81 at four on 131,072.
    if (dtype == STEQR_F32) {
        if (jobz && band == 1 && N == 16) {
            static const int c[] = {4, 8, 16};
            return fill_lanes(batch, c, 3, 2048);
        }
        if (jobz && band == 1 && N == 8) {
            static const int c[] = {2, 4, 8};
            return fill_lanes(batch, c, 3, 2048);
        }
        if (jobz && band == 2 && N == 32) {
            static const int c[] = {8, 16};
            return fill_lanes(batch, c, 2, 2048);
        }
        if (!jobz && band == 1 && (N == 16 || N == 32)) {
            static const int c[] = {1, 2, 4};
            return fill_lanes(batch, c, 3, N == 16 ? 1024 : 2048);
        }
    } else {
        if (jobz && band == 2 && N == 16) {
            static const int c[] = {4, 8};
            return fill_lanes(batch, c, 2, 1024);
        }
        if (!jobz && band == 1 && N == 32) {
            static const int c[] = {1, 2};
            return fill_lanes(batch, c, 2, 512);
        }
    }
    if (jobz) {
        if (N == 4 || N == 12) return 4;
        if (N == 8) return dtype == STEQR_F32 ? 2 : 4;
        // double with the band in registers at 4 lanes needs more than
        // 256 registers per lane and is not built: 8 lanes there
        if (N == 16) return (dtype == STEQR_F64 && band == 1) ? 8 : 4;
        if (band == 2) return dtype == STEQR_F32 ? 8 : 16;  // N == 32
        return 16;  // double, band in registers: not built (-10)
    }
    // values only in float with the band in LDS (asked for explicitly): the
    // register kernel's choice at the batch of 32,768
    if (N == 32 && dtype == STEQR_F32) return 4;
    if (N == 16 && dtype == STEQR_F32) return 2;
    return 1;
}

// Lanes per problem of the values-only bisection: min(N, 64) up to order
// 64; from order 128 the fewest of 1, 2 or 4 wavefronts per problem (at most
// N / 64) whose launch has 2,048 wavefronts. The indices' bisections are
// independent, so every choice gives the same bits. Measured: order 512,
// 256 matrices, 1 / 2 / 4 wavefronts: float 2.16 / 1.41 / 1.04 ms, double
// 7.51 / 4.64 / 2.92 ms; 1,024 matrices: float 2.21 / 1.73 / 1.71, double
// 7.58 / 7.08 / 7.12; order 256, 1,024 matrices: float 0.64 / 0.55 / 0.53,
// double 2.27 / 2.01 / 2.04; 4,096 matrices: float 1.60 / 1.68 / 1.69,
// double 6.57 / 7.44 / 6.91; order 128, 8,192 matrices: float 0.82 / 0.88.
int bisect_default_lanes(int dtype, int N, long batch) {
    (void)dtype;
    if (N < 128) return N < 64 ? N : 64;
    int G = 1;
    while (G < 4 && 64 * G < N && batch * G < 2048) G *= 2;
    return 64 * G;
}

const Entry* search(const Table& t, int dtype, int N, int P, int jobz, int band) {
    for (int i = 0; i < t.count; ++i) {
        const Entry& x = t.entries[i];
        if (x.dtype == dtype && x.N == N && x.P == P && x.jobz == jobz && x.band == band) return &x;
    }
    return nullptr;
}

const Entry* find_entry(int dtype, int N, int P, int jobz, int band, int pg) {
    if (N == 512) return search(pg ? steqr::table_n512_pg() : steqr::table_n512(), dtype, N, P, jobz, band);
    if (N == 256) return search(pg ? steqr::table_huge_pg() : steqr::table_huge(), dtype, N, P, jobz, band);
    if (N == 128) return search(pg ? steqr::table_big_pg() : steqr::table_big(), dtype, N, P, jobz, band);
    if (band == 3) return search(pg ? steqr::table_pc_pg() : steqr::table_pc(), dtype, N, P, jobz, band);
    if (N == 64) {
        if (band != 2) return nullptr;
        return search(pg ? steqr::table_wave_pg() : steqr::table_wave(), dtype, N, P, jobz, band);
    }
    Table t;
    if (band == 2) {
        if (dtype == STEQR_F32)
            t = pg ? steqr::table_lds_f32_pg() : steqr::table_lds_f32();
        else
            t = pg ? steqr::table_lds_f64_pg() : steqr::table_lds_f64();
    } else if (dtype == STEQR_F32) {
        if (jobz)
            t = pg ? steqr::table_f32_v_pg() : steqr::table_f32_v();
        else
            t = pg ? steqr::table_f32_n_pg() : steqr::table_f32_n();
    } else {
        if (jobz)
            t = pg ? steqr::table_f64_v_pg() : steqr::table_f64_v();
        else
            t = pg ? steqr::table_f64_n_pg() : steqr::table_f64_n();
    }
    return search(t, dtype, N, P, jobz, band);
}

struct Plan {
    const Entry* entry;
    int N, P, R, waves, grid, band;
};

// Default band storage (measured): above order 32 the producer-consumer
// kernel with eigenvectors (3) and its producer alone without them (2, band
// in LDS); with eigenvectors LDS wherever the registers are better spent on
// rows of Q: order 32, and order 16 in double precision.
int default_band(int dtype, int N, int jobz) {
    if (N >= 64) return jobz ? 3 : 2;
    // (order 12 in double: 82.8 against 136 us for 32,768 matrices)
    if (jobz && (N == 32 || ((N == 16 || N == 12) && dtype == STEQR_F64))) return 2;
    return 1;
}

int plan_launch(int n, int batch, int jobz, int dtype, const steqr_params* prm, Plan* out) {
    if (n < 0 || n > STEQR_MAX_N) return -5;
    if (batch < 0) return -6;
    if (jobz != STEQR_N && jobz != STEQR_V) return -7;
    if (dtype != STEQR_F32 && dtype != STEQR_F64) return -8;
    int waves = 4;
    int P = 0;
    int band = 0;
    int pg = 0;
    if (prm) {
        if (prm->update_scheme != STEQR_EXP && prm->update_scheme != STEQR_PG) return -10;
        if (prm->shift != STEQR_SHIFT_LAPACK && prm->shift != STEQR_SHIFT_CLOSED) return -10;
        pg = prm->update_scheme == STEQR_PG;
        band = prm->band_storage;
        if (band < 0 || band > 3) return -10;
        if (prm->waves_per_block != 0) {
            if (prm->waves_per_block != 1 && prm->waves_per_block != 2 && prm->waves_per_block != 4)
                return -10;
            waves = prm->waves_per_block;
        }
        P = prm->lanes_per_problem;
        // a power of two up to 64; bisection also takes several wavefronts
        // per problem (up to the padded order, checked below)
        const int pmax = prm->method == STEQR_METHOD_BISECT ? 512 : 64;
        if (P < 0 || P > pmax || (P != 0 && (P & (P - 1)) != 0)) return -10;
        if (prm->no_sort != 0 && prm->no_sort != 1) return -10;
        if (prm->back_transform != 0 && prm->back_transform != 1) return -10;
        if (prm->back_transform == 1 && jobz != STEQR_V) return -10;
        if (prm->method != STEQR_METHOD_QR && prm->method != STEQR_METHOD_BISECT) return -10;
    }
    Plan p{};
    p.waves = waves;
    if (n == 0) {
        *out = p;
        return 0;
    }
    const bool bisect = prm && prm->method == STEQR_METHOD_BISECT;
    const int N = bisect ? padded_order(n < 2 ? 2 : n) : padded_order(n < 2 ? 2 : n, dtype, jobz);
    if (N < 0) return -5;  // order not provided by this build
    if (prm && prm->method == STEQR_METHOD_BISECT) {
        // values-only bisection: one lane per eigenvalue index, min(N, 64)
        // lanes of a wavefront per problem; from order 128 also 64 G lanes,
        // G wavefronts of one workgroup per problem
        const int L = N < 64 ? N : 64;
        if (jobz != STEQR_N || prm->update_scheme != 0 || prm->shift != 0 ||
            prm->band_storage != 0 || prm->back_transform != 0)
            return -10;
        const int Pb = P != 0 ? P : bisect_default_lanes(dtype, N, (long)batch);
        if (Pb < L || Pb > (N < 128 ? L : N)) return -10;
        const Entry* ent = search(steqr::table_bisect(), dtype, N, Pb, STEQR_N,
                                  (2 * N * (dtype == STEQR_F32 ? 4 : 8) / 4 <= 128) ? 1 : 2);
        if (!ent) return -10;
        const int G = Pb / L;  // wavefronts per problem
        p.entry = ent;
        p.N = N;
        p.P = Pb;
        p.R = 0;
        p.band = ent->band;
        // several wavefronts per problem: one problem per workgroup (the
        // workgroup size is then G wavefronts, whatever waves_per_block says)
        p.waves = G > 1 ? G : waves;
        const int per_block = G > 1 ? 1 : waves * (64 / L);
        p.grid = batch > 0 ? (int)(((long)batch + per_block - 1) / per_block) : 0;
        *out = p;
        return 0;
    }
    if (band == 0 || (N >= 64 && band == 1)) band = default_band(dtype, N, jobz);
    if (P == 0) P = default_lanes(dtype, N, jobz, band, (long)batch);
    const Entry* ent = find_entry(dtype, N, P, jobz, band, pg);
    if (!ent) return -10;
    int per_block;
    int gpp = 1;  // workgroups per problem (producer-consumer, rows split)
    if (band == 3) {
        // consumer wavefronts (one row of Q per lane) and one producer
        // wavefront per workgroup
        waves = ent->pc_waves;
        per_block = ent->pc_np;
        gpp = ent->pc_gpp;
        p.R = 1;
    } else {
        // keep a workgroup's LDS within 64 KiB
        while (waves > 1 && (long)waves * ent->lds_per_wave > 65536) waves /= 2;
        // a small batch: fewer wavefronts per workgroup, so that the
        // workgroups reach as many of the 256 CUs as there are wavefronts
        // (4,096 matrices of order 4: 9.5 against 10.1 us at 4 per workgroup)
        if (!(prm && prm->waves_per_block != 0)) {
            const long total = ((long)batch * P + 63) / 64;
            while (waves > 1 && (total + waves - 1) / waves < 256) waves /= 2;
        }
        per_block = waves * (64 / P);
        p.R = jobz ? (N + P - 1) / P : 0;
    }
    p.waves = waves;
    p.entry = ent;
    p.N = N;
    p.P = P;
    p.band = band;
    p.grid = batch > 0 ? (int)(((long)batch + per_block - 1) / per_block * gpp) : 0;
    *out = p;
    return 0;
}

}  // namespace

extern "C" int steqr_query(int n, int batch, int jobz, int dtype, const steqr_params* params,
                           int* padded_n, int* lanes_per_problem, int* rows_per_lane,
                           int* waves_per_block, int* workgroups, int* band_storage) {
    Plan p;
    const int rc = plan_launch(n, batch, jobz, dtype, params, &p);
    if (rc != 0) return rc;
    if (padded_n) *padded_n = p.N;
    if (lanes_per_problem) *lanes_per_problem = p.P;
    if (rows_per_lane) *rows_per_lane = p.R;
    if (waves_per_block) *waves_per_block = p.waves;
    if (workgroups) *workgroups = p.grid;
    if (band_storage) *band_storage = p.band;
    return 0;
}

extern "C" int steqr_batched_ex(const void* d, const void* e, void* lambda, void* Q, int n,
                                int batch, int jobz, int dtype, hipStream_t stream, int* info,
                                const steqr_params* params) {
    // arguments in the order of the parameter list: a NULL array is an
    // error only where the call has work to do (n > 0 and batch > 0)
    const bool work = n > 0 && batch > 0;
    if (work && d == nullptr) return -1;
    if (work && n > 1 && e == nullptr) return -2;
    if (work && lambda == nullptr) return -3;
    if (work && jobz == STEQR_V && Q == nullptr) return -4;
    Plan p;
    const int rc = plan_launch(n, batch, jobz, dtype, params, &p);
    if (rc != 0) return rc;
    if (n == 0 || batch == 0) return 0;
    steqr::KernelArgs a{};
    a.d = d;
    a.e = e;
    a.lam = lambda;
    a.q = Q;
    a.info = info;
    a.n = n;
    a.batch = batch;
    const int ms = params ? params->max_sweeps_per_n : 0;
    a.max_sweeps_per_n = ms == 0 ? 30 : (ms < 0 ? 0 : ms);
    a.do_sort = params ? !params->no_sort : 1;
    a.shift_kind = params ? params->shift : 0;
    a.back_transform = params ? params->back_transform : 0;
    // an error left by an earlier, unrelated HIP call is not this launch's
    (void)hipGetLastError();
    const hipError_t err = p.entry->fn(a, p.grid, p.waves * 64, stream);
    return err == hipSuccess ? 0 : (int)err;
}

extern "C" int steqr_batched(const void* d, const void* e, void* lambda, void* Q, int n,
                             int batch, int jobz, int dtype, hipStream_t stream) {
    return steqr_batched_ex(d, e, lambda, Q, n, batch, jobz, dtype, stream, nullptr, nullptr);
}

// ---------------------------------------------------------------- syev

namespace {

// Default lanes per problem of the fused dense kernel (measured on MI355X):
// the lanes hold whole rows of A and Q (N/P rows each), so P keeps A, Q and
// the replicated band within the register file at two wavefronts per SIMD;
// without Q there is room for twice the rows at orders 16 (double) and 32
// (float).
int syev_default_lanes(int dtype, int N, int jobz, long batch) {
    // Below the configurations' batches more lanes per problem spread the
    // batch over more SIMDs: the fewest of the candidates whose launch has
    // T wavefronts (each rule keeps the tuned choice at the configuration's
    // batch). Measured: float order 8 with vectors, 32,768 matrices 32.0 us
    // at 4 lanes against 34.9 at 2; float order 16 with vectors, 16,384
    // matrices 85.0 at 8 against 95.8 at 4; float order 32 values only,
    // 4,096 matrices 201.7 at 16 against 208.4 at 8; double order 16 values
    // only, 4,096 matrices 90.5 at 8 against 96.0 at 4.
    if (dtype == STEQR_F32 && jobz && N == 8) {
        static const int c[] = {2, 4};
        return fill_lanes(batch, c, 2, 2048);
    }
    if (dtype == STEQR_F32 && jobz && N == 16) {
        static const int c[] = {4, 8};
        return fill_lanes(batch, c, 2, 2048);
    }
    if (dtype == STEQR_F32 && !jobz && N == 32) {
        static const int c[] = {8, 16};
        return fill_lanes(batch, c, 2, 2048);
    }
    if (dtype == STEQR_F64 && !jobz && N == 16) {
        static const int c[] = {4, 8};
        return fill_lanes(batch, c, 2, 1024);
    }
    if (N == 4) return 4;
    if (N == 8) return dtype == STEQR_F32 ? 2 : 4;
    // double with vectors at 4 lanes (271 against 351 us at 8) needs more
    // than 256 registers per lane and is not built
    if (N == 16) return (dtype == STEQR_F64 && jobz) ? 8 : 4;
    if (dtype == STEQR_F64) return 32;  // with vectors: the band in LDS
    return jobz ? 16 : 8;
}

int syev_plan(int n, int batch, int jobz, int dtype, const steqr_params* prm, Plan* out) {
    if (n < 0 || n > SYEV_MAX_N) return -4;
    if (dtype == STEQR_F64 && jobz == STEQR_V && n > SYEV_MAX_N_F64_V) return -4;
    if (batch < 0) return -5;
    if (jobz != STEQR_N && jobz != STEQR_V) return -6;
    if (dtype != STEQR_F32 && dtype != STEQR_F64) return -7;
    int waves = 4, P = 0, band = 0;
    if (prm) {
        if (prm->update_scheme != STEQR_EXP) return -10;
        if (prm->shift != STEQR_SHIFT_LAPACK && prm->shift != STEQR_SHIFT_CLOSED) return -10;
        if (prm->back_transform != 0) return -10;
        if (prm->method != STEQR_METHOD_QR) return -10;
        if (prm->band_storage < 0 || prm->band_storage > 2) return -10;
        band = prm->band_storage;
        if (prm->no_sort != 0 && prm->no_sort != 1) return -10;
        if (prm->waves_per_block != 0) {
            if (prm->waves_per_block != 1 && prm->waves_per_block != 2 && prm->waves_per_block != 4)
                return -10;
            waves = prm->waves_per_block;
        }
        P = prm->lanes_per_problem;
        // a power of two up to 64; bisection also takes several wavefronts
        // per problem (up to the padded order, checked below)
        const int pmax = prm->method == STEQR_METHOD_BISECT ? 512 : 64;
        if (P < 0 || P > pmax || (P != 0 && (P & (P - 1)) != 0)) return -10;
    }
    Plan p{};
    p.waves = waves;
    if (n == 0) {
        *out = p;
        return 0;
    }
    const int N = padded_order(n < 2 ? 2 : n);
    if (P == 0) P = syev_default_lanes(dtype, N, jobz, (long)batch);
    const Table t = dtype == STEQR_F32 ? steqr::table_syev_f32() : steqr::table_syev_f64();
    // by default the band in registers where that variant is built, else in
    // LDS; double at order 32 prefers LDS (measured on 16,384 matrices: with
    // vectors 1,432 us there, values only 1,603 us with the band in registers)
    const int first = band != 0 ? band : ((dtype == STEQR_F64 && N == 32) ? 2 : 1);
    const Entry* ent = search(t, dtype, N, P, jobz, first);
    if (!ent && band == 0) ent = search(t, dtype, N, P, jobz, 3 - first);
    if (!ent) return -10;
    while (waves > 1 && (long)waves * ent->lds_per_wave > 65536) waves /= 2;
    p.waves = waves;
    p.entry = ent;
    p.N = N;
    p.P = P;
    p.R = N / P;
    p.band = ent->band;
    const int per_block = waves * (64 / P);
    p.grid = batch > 0 ? (int)(((long)batch + per_block - 1) / per_block) : 0;
    *out = p;
    return 0;
}

}  // namespace

extern "C" int syev_query(int n, int batch, int jobz, int dtype, const steqr_params* params,
                          int* padded_n, int* lanes_per_problem, int* rows_per_lane,
                          int* waves_per_block, int* workgroups, int* band_storage) {
    Plan p;
    const int rc = syev_plan(n, batch, jobz, dtype, params, &p);
    if (rc != 0) return rc;
    if (padded_n) *padded_n = p.N;
    if (lanes_per_problem) *lanes_per_problem = p.P;
    if (rows_per_lane) *rows_per_lane = p.R;
    if (waves_per_block) *waves_per_block = p.waves;
    if (workgroups) *workgroups = p.grid;
    if (band_storage) *band_storage = p.band;
    return 0;
}

extern "C" int syev_batched_ex(const void* A, void* lambda, void* Q, int n, int batch, int jobz,
                               int dtype, hipStream_t stream, int* info,
                               const steqr_params* params) {
    const bool work = n > 0 && batch > 0;
    if (work && A == nullptr) return -1;
    if (work && lambda == nullptr) return -2;
    if (work && jobz == STEQR_V && Q == nullptr) return -3;
    Plan p;
    const int rc = syev_plan(n, batch, jobz, dtype, params, &p);
    if (rc != 0) return rc;
    if (n == 0 || batch == 0) return 0;
    steqr::KernelArgs a{};
    a.a = A;
    a.lam = lambda;
    a.q = Q;
    a.info = info;
    a.n = n;
    a.batch = batch;
    const int ms = params ? params->max_sweeps_per_n : 0;
    a.max_sweeps_per_n = ms == 0 ? 30 : (ms < 0 ? 0 : ms);
    a.do_sort = params ? !params->no_sort : 1;
    a.shift_kind = params ? params->shift : 0;
    a.back_transform = 0;
    (void)hipGetLastError();  // clear an earlier call's error
    const hipError_t err = p.entry->fn(a, p.grid, p.waves * 64, stream);
    return err == hipSuccess ? 0 : (int)err;
}

extern "C" int syev_batched(const void* A, void* lambda, void* Q, int n, int batch, int jobz,
                            int dtype, hipStream_t stream) {
    return syev_batched_ex(A, lambda, Q, n, batch, jobz, dtype, stream, nullptr, nullptr);
}

extern "C" const char* steqr_version(void) { return "steqr-mi355x 0.1.0 gfx950"; }
