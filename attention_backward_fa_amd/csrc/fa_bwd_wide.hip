// fa_bwd_wide.hip -- the recompute-form kernels and the forward for head dims above 128 (padded to
// 256, the other dim padded to at least 128). Built as its own object, without VGPR-form MFMA, so
// that the accumulators of these one-wave-per-SIMD kernels can live in the AGPRs.
#include "fa_bwd_launch.hpp"

namespace fa {

KernelSet wide_kernel_set(int pq, int pv, bool exact) {
  if (pq == 128) return kernel_set<128, 256, false>();
  if (pv == 128) return kernel_set<256, 128, false>();
  return exact ? kernel_set<256, 256, true>() : kernel_set<256, 256, false>();
}

}  // namespace fa
