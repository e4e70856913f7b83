// Kernel instantiations: one problem per wavefront (orders 33..64), and
// for values only the producer's algorithm of the producer-consumer kernel
// with several problems per wavefront (4, 8 or 16 lanes each).
#include "steqr_registry.hpp"

namespace steqr {

static const Entry kEntries[] = {
    STEQR_WAVE_ENTRY(0, float, 64, 1), STEQR_WAVE_ENTRY(0, float, 64, 0),
    // double with eigenvectors (64 rows of Q in 128 registers plus the
    // chase) needs more than 256 registers per lane: not provided
    STEQR_WAVE_ENTRY(1, double, 64, 0),
    STEQR_PCV_ENTRY(0, float, 64, 4), STEQR_PCV_ENTRY(0, float, 64, 8),
    STEQR_PCV_ENTRY(0, float, 64, 16),
    STEQR_PCV_ENTRY(1, double, 64, 4), STEQR_PCV_ENTRY(1, double, 64, 8),
    STEQR_PCV_ENTRY(1, double, 64, 16),
};

Table STEQR_TABLE(table_wave)() { return {kEntries, (int)(sizeof(kEntries) / sizeof(kEntries[0]))}; }

}  // namespace steqr
