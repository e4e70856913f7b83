// Kernel instantiations: float64, eigenvalues and eigenvectors.
#include "steqr_registry.hpp"

namespace steqr {

#define E(N, P) {1, N, P, 1, &launch_chunk<double, N, P, true>}
static const Entry kEntries[] = {
    E(4, 4),   E(4, 2),
    E(8, 8),   E(8, 4),
    E(16, 16), E(16, 8),
    E(32, 32), E(32, 16),
};
#undef E

Table table_f64_v() { return {kEntries, (int)(sizeof(kEntries) / sizeof(kEntries[0]))}; }

}  // namespace steqr
