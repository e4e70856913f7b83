// Kernel instantiations: float64, eigenvalues and eigenvectors, band in LDS.
#include "steqr_registry.hpp"

namespace steqr {

#define E(N, P) STEQR_LENTRY(1, double, N, P, 1)
static const Entry kEntries[] = {
    E(12, 4),
    E(16, 8), E(16, 4),
    // (32, 8) needs 256 rows-of-Q registers per lane plus the chase state:
    // register spills, and it produced wrong eigenvectors in one build;
    // not provided
    E(32, 16),
};
#undef E

Table STEQR_TABLE(table_lds_f64)() { return {kEntries, (int)(sizeof(kEntries) / sizeof(kEntries[0]))}; }

}  // namespace steqr
