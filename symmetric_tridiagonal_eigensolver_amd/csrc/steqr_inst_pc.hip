// Kernel instantiations: order 64 with eigenvectors, producer and consumer
// wavefronts (W problems per workgroup, P producer lanes per problem).
#include "steqr_registry.hpp"

namespace steqr {

static const Entry kEntries[] = {
    STEQR_PC_ENTRY(0, float, 64, 7, 8),
    STEQR_PC_ENTRY(1, double, 64, 5, 8),
};

Table STEQR_TABLE(table_pc)() { return {kEntries, (int)(sizeof(kEntries) / sizeof(kEntries[0]))}; }

}  // namespace steqr
