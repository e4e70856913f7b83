// Kernel instantiations: float32, eigenvalues and eigenvectors, band in LDS.
#include "steqr_registry.hpp"

namespace steqr {

#define E(N, P) STEQR_LENTRY(0, float, N, P, 1)
static const Entry kEntries[] = {
    E(16, 8), E(16, 4), E(16, 2),
    // (32, 4) spills registers (8 rows of Q per lane); not provided
    E(32, 16), E(32, 8),
};
#undef E

Table STEQR_TABLE(table_lds_f32)() { return {kEntries, (int)(sizeof(kEntries) / sizeof(kEntries[0]))}; }

}  // namespace steqr
