// fa_bwd_wide192.hip -- the recompute-form kernels and the forward for the padded head-dim pairs
// that include 192 (the other dim padded to 128, 192 or 256), e.g. latent attention with a 192-dim
// query/key head and a 128-dim value head. Built like fa_bwd_wide.hip (accumulators may use the
// AGPRs), as a unit of its own so that the two compile in parallel.
#include "fa_bwd_launch.hpp"

namespace fa {

KernelSet wide192_kernel_set(int pq, int pv, bool exact) {
  if (pq == 192) {
    if (pv == 128) return kernel_set<192, 128, false>();
    if (pv == 256) return kernel_set<192, 256, false>();
    return exact ? kernel_set<192, 192, true>() : kernel_set<192, 192, false>();
  }
  return pq == 128 ? kernel_set<128, 192, false>() : kernel_set<256, 192, false>();
}

}  // namespace fa
