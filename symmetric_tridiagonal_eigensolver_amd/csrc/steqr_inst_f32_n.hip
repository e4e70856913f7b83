// Kernel instantiations: float32, eigenvalues only.
#include "steqr_registry.hpp"

namespace steqr {

#define E(N, P) STEQR_ENTRY(0, float, N, P, 0)
static const Entry kEntries[] = {
    E(4, 4), E(4, 1),
    E(8, 8), E(8, 2), E(8, 1),
    E(16, 16), E(16, 4), E(16, 2), E(16, 1),
    E(32, 32), E(32, 4), E(32, 2), E(32, 1),
};
#undef E

Table STEQR_TABLE(table_f32_n)() { return {kEntries, (int)(sizeof(kEntries) / sizeof(kEntries[0]))}; }

}  // namespace steqr
