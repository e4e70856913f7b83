// Kernel instantiations: float32, eigenvalues and eigenvectors.
#include "steqr_registry.hpp"

namespace steqr {

#define E(N, P) STEQR_ENTRY(0, float, N, P, 1)
static const Entry kEntries[] = {
    E(4, 4), E(4, 2), E(4, 1),
    E(8, 8), E(8, 4), E(8, 2), E(8, 1),
    E(16, 16), E(16, 8), E(16, 4), E(16, 2),
    E(32, 32), E(32, 16),
    // (32, 8) needs more than 256 registers per lane with the band in
    // registers; the LDS-band kernel serves it
};
#undef E

Table STEQR_TABLE(table_f32_v)() { return {kEntries, (int)(sizeof(kEntries) / sizeof(kEntries[0]))}; }

}  // namespace steqr
