// scan_conv.hip -- the scan kernels with the convolution front (and the step
// bias and softplus): instantiations of scan_kernel.h.
#include "scan_kernel.h"

namespace s6i {

int launch_scan_conv(int in_dtype, int mode, const ScanArgs& a, const Plan& p, bool gate, int64_t batch,
                     int64_t segs, hipStream_t st) {
  return launch_scan_e<3>(in_dtype, mode, a, p, gate, batch, segs, st);
}

}  // namespace s6i
