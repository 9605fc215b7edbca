// Instantiations of the column sweep (sweep.h): groups of 16, 32 and 64, and static groups.
#include "sweep.h"

namespace gptq {

template gptq_status launch_sweep_nt<16>(const SweepShape&, hipStream_t, const SweepArgs&, int);
template gptq_status launch_sweep_nt<32>(const SweepShape&, hipStream_t, const SweepArgs&, int);
template gptq_status launch_sweep_nt<64>(const SweepShape&, hipStream_t, const SweepArgs&, int);

gptq_status launch_sweep_static(const SweepShape& sh, hipStream_t stream, const SweepArgs& a, int blk) {
  if (sh.nt != 256 || sh.lpr != 16 || sh.rpl != 1) return GPTQ_ERR_UNSUPPORTED;
  return launch_sweep<0, 256, 16, true>(sh.grid, stream, a, blk);
}

}  // namespace gptq
