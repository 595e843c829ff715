// scan_ext.hip -- the scan kernels with the step options and the convolution
// front (instantiations of scan_kernel.h, compiled apart from the plain
// kernels).  The exact hold has kernels of its own: its per-state
// coefficient needs registers that the others would otherwise reserve.
#include "scan_kernel.h"

namespace s6i {

int launch_scan_options(int in_dtype, int mode, const ScanArgs& a, const Plan& p, bool gate, int64_t batch,
                        int64_t segs, hipStream_t st) {
  if (a.zoh) return launch_scan_e<2>(in_dtype, mode, a, p, gate, batch, segs, st);
  return launch_scan_e<1>(in_dtype, mode, a, p, gate, batch, segs, st);
}

}  // namespace s6i
