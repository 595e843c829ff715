// scan_ext.hip -- the scan kernels with the step bias and softplus
// (instantiations of scan_kernel.h), and the dispatch among the option
// levels.  The convolution front (scan_conv.hip) and the exact hold
// (scan_hold.hip) have kernels of their own: their per-piece filter and
// per-state coefficient need registers that would otherwise cost these
// kernels their fifth wave per SIMD.
#include "scan_kernel.h"

namespace s6i {

int launch_scan_options(int in_dtype, int mode, const ScanArgs& a, const Plan& p, bool gate, int64_t batch,
                        int64_t segs, hipStream_t st) {
  if (a.zoh) return launch_scan_hold(in_dtype, mode, a, p, gate, batch, segs, st);
  if (a.conv_w) return launch_scan_conv(in_dtype, mode, a, p, gate, batch, segs, st);
  return launch_scan_e<1>(in_dtype, mode, a, p, gate, batch, segs, st);
}

}  // namespace s6i
