// Kernel instantiations: values-only bisection, float32 and float64.
#include "steqr_registry.hpp"

namespace steqr {

static const Entry kEntries[] = {
    STEQR_BISECT_ENTRY(0, float, 4), STEQR_BISECT_ENTRY(0, float, 8),
    STEQR_BISECT_ENTRY(0, float, 16), STEQR_BISECT_ENTRY(0, float, 32),
    STEQR_BISECT_ENTRY(0, float, 64), STEQR_BISECT_ENTRY(0, float, 128),
    STEQR_BISECT_ENTRY(0, float, 256), STEQR_BISECT_ENTRY(0, float, 512),
    STEQR_BISECT_ENTRY(1, double, 4), STEQR_BISECT_ENTRY(1, double, 8),
    STEQR_BISECT_ENTRY(1, double, 16), STEQR_BISECT_ENTRY(1, double, 32),
    STEQR_BISECT_ENTRY(1, double, 64), STEQR_BISECT_ENTRY(1, double, 128),
    STEQR_BISECT_ENTRY(1, double, 256), STEQR_BISECT_ENTRY(1, double, 512),
    // several wavefronts per problem (64 G lanes; eight at order 512 spill
    // registers and are not built)
    STEQR_BISECT_G_ENTRY(0, float, 128, 2), STEQR_BISECT_G_ENTRY(0, float, 256, 2),
    STEQR_BISECT_G_ENTRY(0, float, 256, 4), STEQR_BISECT_G_ENTRY(0, float, 512, 2),
    STEQR_BISECT_G_ENTRY(0, float, 512, 4),
    STEQR_BISECT_G_ENTRY(1, double, 128, 2), STEQR_BISECT_G_ENTRY(1, double, 256, 2),
    STEQR_BISECT_G_ENTRY(1, double, 256, 4), STEQR_BISECT_G_ENTRY(1, double, 512, 2),
    STEQR_BISECT_G_ENTRY(1, double, 512, 4),
};

Table table_bisect() { return {kEntries, (int)(sizeof(kEntries) / sizeof(kEntries[0]))}; }

}  // namespace steqr
