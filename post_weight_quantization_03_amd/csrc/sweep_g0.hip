// Instantiations of the column sweep (sweep.h): one grid per row.
#include "sweep.h"

namespace gptq {

template gptq_status launch_sweep_nt<0>(const SweepShape&, hipStream_t, const SweepArgs&, int);

}  // namespace gptq
