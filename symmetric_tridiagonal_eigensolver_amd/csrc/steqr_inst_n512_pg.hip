// Kernel instantiations: as steqr_inst_n512.hip, Parlett-Gray form of the step.
#define STEQR_INST_PG 1
#include "steqr_inst_n512.hip"
