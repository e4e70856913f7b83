// The same instantiations as steqr_inst_pc.hip, with the chase step in the
// PG (Parlett-Gray) form.
#define STEQR_INST_PG 1
#include "steqr_inst_pc.hip"
