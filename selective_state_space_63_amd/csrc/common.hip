// common.hip -- argument checks, errors, version and a fill kernel shared
// by the entry points of libs6.
#include "s6_internal.h"

namespace s6i {

namespace {

// out[i] = v (a fill that a captured graph can hold, unlike a memset node).
__global__ void s6_fill(float* __restrict__ out, float v, int64_t total) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x)
    out[i] = v;
}

}  // namespace

thread_local char g_err[256];

int hip_fail(hipError_t e, const char* what) {
  snprintf(g_err, sizeof(g_err), "HIP error in %s: %s", what, hipGetErrorString(e));
  return S6_ERR_HIP;
}

bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a == 0 || b == 0) { *out = 0; return true; }
  if (a > INT64_MAX / b) return false;
  *out = a * b;
  return true;
}

int check_common(int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate, int in_dtype) {
  if (in_dtype != S6_F32 && in_dtype != S6_BF16) return S6_ERR_DTYPE;
  if (batch < 0 || dim < 0 || seqlen < 0 || dstate < 0) return S6_ERR_SHAPE;
  if (dstate < 1 || dstate > kMaxN) return S6_ERR_UNSUPPORTED;
  int64_t t;
  if (!mul_ok(batch, dim, &t) || !mul_ok(t, seqlen > 0 ? seqlen : 1, &t) || !mul_ok(t, 64, &t))
    return S6_ERR_SHAPE;  // element counts, with headroom for per-state buffers
  if (batch * ((dim + kCW - 1) / kCW) > INT32_MAX) return S6_ERR_SHAPE;  // grid size
  return S6_OK;
}

int cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 256;
  return n;
}

void fill(float* p, float v, int64_t n, hipStream_t st) {
  if (!p || n <= 0) return;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(s6_fill, dim3((unsigned)blocks), dim3(256), 0, st, p, v, n);
}

}  // namespace s6i

using namespace s6i;

extern "C" {

int s6_version(void) { return 20000; }

const char* s6_status_str(int status) {
  switch (status) {
    case S6_OK: return "ok";
    case S6_ERR_NULL: return "a required pointer is NULL";
    case S6_ERR_SHAPE: return "invalid size (negative, or the element count overflows)";
    case S6_ERR_DTYPE: return "in_dtype must be S6_F32 or S6_BF16";
    case S6_ERR_UNSUPPORTED: return "unsupported: dstate outside 1..32, filter width outside 1..4, or an option this entry point lacks";
    case S6_ERR_ALIGN: return "a pointer is not aligned to its element size";
    case S6_ERR_FLAGS: return "unknown option bits in flags";
    case S6_ERR_WORKSPACE:
      return "the call needs a workspace: none given, or smaller than its *_workspace_size (s6_scan_fwd_noalloc: "
             "more than its 16 MiB static scratch)";
    case S6_ERR_HIP: return g_err[0] ? g_err : "HIP error";
    default: return "unknown status";
  }
}

}  // extern "C"
