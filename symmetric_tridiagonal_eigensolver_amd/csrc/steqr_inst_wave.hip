// Kernel instantiations: one problem per wavefront (orders 33..64).
#include "steqr_registry.hpp"

namespace steqr {

static const Entry kEntries[] = {
    STEQR_WAVE_ENTRY(0, float, 64, 1), STEQR_WAVE_ENTRY(0, float, 64, 0),
    STEQR_WAVE_ENTRY(1, double, 64, 1), STEQR_WAVE_ENTRY(1, double, 64, 0),
};

Table STEQR_TABLE(table_wave)() { return {kEntries, (int)(sizeof(kEntries) / sizeof(kEntries[0]))}; }

}  // namespace steqr
