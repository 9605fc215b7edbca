// Instantiations of the column sweep (sweep.h): groups of 128.
#include "sweep.h"

namespace gptq {

template gptq_status launch_sweep_nt<128>(const SweepShape&, hipStream_t, const SweepArgs&, int);

}  // namespace gptq
