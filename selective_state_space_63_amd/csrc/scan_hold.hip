// scan_hold.hip -- the scan kernels with the exact zero-order hold (and the
// step bias, softplus and convolution front): instantiations of
// scan_kernel.h.
#include "scan_kernel.h"

namespace s6i {

int launch_scan_hold(int in_dtype, int mode, const ScanArgs& a, const Plan& p, bool gate, int64_t batch,
                     int64_t segs, hipStream_t st) {
  return launch_scan_e<2>(in_dtype, mode, a, p, gate, batch, segs, st);
}

}  // namespace s6i
