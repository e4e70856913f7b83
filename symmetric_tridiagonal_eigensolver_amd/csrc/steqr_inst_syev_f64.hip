// Kernel instantiations: fused dense eigensolver, float64.
#include "steqr_registry.hpp"

namespace steqr {

#define E(N, P, Q) STEQR_SYEV_ENTRY(1, double, N, P, Q)
#define EL(N, P, Q) STEQR_SYEV_LENTRY(1, double, N, P, Q)
static const Entry kEntries[] = {
    // with eigenvectors, (16, 4) and every order-32 shape with the band in
    // registers need more than 256 registers per lane (rows of A and Q plus
    // the replicated band): order 32 with eigenvectors keeps the band in LDS
    E(4, 4, 1), E(8, 4, 1), E(16, 8, 1), EL(32, 32, 1),
    E(4, 4, 0), E(8, 4, 0), E(8, 2, 0), E(16, 8, 0), E(16, 4, 0), E(32, 32, 0), EL(32, 32, 0),
};
#undef EL
#undef E

Table table_syev_f64() { return {kEntries, (int)(sizeof(kEntries) / sizeof(kEntries[0]))}; }

}  // namespace steqr
