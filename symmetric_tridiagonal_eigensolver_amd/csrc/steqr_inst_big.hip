// Kernel instantiations: order 128 (orders 65..128), producer and consumer
// wavefronts with eigenvectors (four consumers per problem, two lanes per
// row of Q), producer wavefronts alone for values only.
#include "steqr_registry.hpp"

namespace steqr {

static const Entry kEntries[] = {
    STEQR_PC_ENTRY(0, float, 128, 12, 16),
    STEQR_PC_ENTRY(0, float, 128, 8, 32),
    // whole rows of Q per lane: two consumers per problem, five problems
    STEQR_PCR_ENTRY(0, float, 128, 10, 8, 1),
    STEQR_PC_ENTRY(1, double, 128, 8, 16),
    STEQR_PC_ENTRY(1, double, 128, 8, 32),
    STEQR_PCV_ENTRY(0, float, 128, 8),
    STEQR_PCV_ENTRY(0, float, 128, 16),
    STEQR_PCV_ENTRY(1, double, 128, 8),
    STEQR_PCV_ENTRY(1, double, 128, 16),
};

Table STEQR_TABLE(table_big)() { return {kEntries, (int)(sizeof(kEntries) / sizeof(kEntries[0]))}; }

}  // namespace steqr
