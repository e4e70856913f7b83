// Kernel instantiations: order 64 with eigenvectors, producer and consumer
// wavefronts (W problems per workgroup, P producer lanes per problem).
#include "steqr_registry.hpp"

namespace steqr {

static const Entry kEntries[] = {
    // measured: with 64 float rows of Q per consumer several small workgroups
    // per CU (one producer each) win; with double rows the register file
    // holds about 12 problems per CU, best as one workgroup of 11 consumers
    STEQR_PC_ENTRY(0, float, 64, 3, 16),
    STEQR_PC_ENTRY(0, float, 64, 7, 8),
    STEQR_PC_ENTRY(1, double, 64, 11, 4),
    STEQR_PC_ENTRY(1, double, 64, 3, 16),
};

Table STEQR_TABLE(table_pc)() { return {kEntries, (int)(sizeof(kEntries) / sizeof(kEntries[0]))}; }

}  // namespace steqr
