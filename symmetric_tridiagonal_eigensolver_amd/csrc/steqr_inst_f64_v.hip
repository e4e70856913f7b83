// Kernel instantiations: float64, eigenvalues and eigenvectors.
#include "steqr_registry.hpp"

namespace steqr {

#define E(N, P) STEQR_ENTRY(1, double, N, P, 1)
static const Entry kEntries[] = {
    E(4, 4), E(4, 2),
    E(8, 8), E(8, 4), E(8, 2),
    E(12, 4),
    E(16, 16), E(16, 8),
    // (16, 4), (32, 16) and (32, 32) need more than 256 registers per lane
    // with the band in registers; the LDS-band kernel serves those lanes
};
#undef E

Table STEQR_TABLE(table_f64_v)() { return {kEntries, (int)(sizeof(kEntries) / sizeof(kEntries[0]))}; }

}  // namespace steqr
