// Kernel instantiations: fused dense eigensolver, float32.
#include "steqr_registry.hpp"

namespace steqr {

#define E(N, P, Q) STEQR_SYEV_ENTRY(0, float, N, P, Q)
static const Entry kEntries[] = {
    E(4, 4, 1), E(8, 2, 1), E(8, 4, 1), E(16, 4, 1), E(16, 8, 1), E(32, 16, 1),
    E(4, 4, 0), E(8, 2, 0), E(8, 1, 0), E(16, 4, 0), E(16, 2, 0), E(32, 16, 0), E(32, 8, 0),
};
#undef E

Table table_syev_f32() { return {kEntries, (int)(sizeof(kEntries) / sizeof(kEntries[0]))}; }

}  // namespace steqr
