// Kernel instantiations: order 512 (orders 257..512). With eigenvectors,
// producer and consumer wavefronts: one problem per producer (64 producer
// lanes), eight consumers per workgroup holding 8 rows each (float, eight
// lanes per row of 64 columns each: eight workgroups share a problem) or 4
// rows each (double, sixteen lanes per row of 32 columns each: sixteen
// workgroups share a problem). Values only: producer wavefronts alone.
#include "steqr_registry.hpp"

namespace steqr {

static const Entry kEntries[] = {
    STEQR_PC_ENTRY(0, float, 512, 8, 64),
    STEQR_PC_ENTRY(1, double, 512, 8, 64),
    STEQR_PCV_ENTRY(0, float, 512, 64),
    STEQR_PCV_ENTRY(1, double, 512, 64),
};

Table STEQR_TABLE(table_n512)() { return {kEntries, (int)(sizeof(kEntries) / sizeof(kEntries[0]))}; }

}  // namespace steqr
