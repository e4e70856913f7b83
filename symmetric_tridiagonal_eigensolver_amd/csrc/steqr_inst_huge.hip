// Kernel instantiations: order 256 (orders 129..256). With eigenvectors,
// producer and consumer wavefronts: one problem per producer (64 producer
// lanes), eight consumers per workgroup holding 32 rows (float, two lanes
// per row) or 16 rows (double, four lanes per row: two workgroups share a
// problem). Values only: producer wavefronts alone.
#include "steqr_registry.hpp"

namespace steqr {

static const Entry kEntries[] = {
    STEQR_PC_ENTRY(0, float, 256, 8, 64),
    STEQR_PC_ENTRY(1, double, 256, 8, 64),
    STEQR_PCV_ENTRY(0, float, 256, 16),
    STEQR_PCV_ENTRY(0, float, 256, 32),
    STEQR_PCV_ENTRY(0, float, 256, 64),
    STEQR_PCV_ENTRY(1, double, 256, 16),
    STEQR_PCV_ENTRY(1, double, 256, 32),
    STEQR_PCV_ENTRY(1, double, 256, 64),
};

Table STEQR_TABLE(table_huge)() { return {kEntries, (int)(sizeof(kEntries) / sizeof(kEntries[0]))}; }

}  // namespace steqr
