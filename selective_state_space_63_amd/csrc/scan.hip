// scan.hip -- the fused selective scan (s6_scan_fwd, s6_last_state, their
// _ex forms and s6_conv_scan_fwd): launch planning, the segment carry fold,
// the plain kernels.  The kernel itself is in scan_kernel.h; the kernels with
// the step options and the convolution front are instantiated in
// scan_ext.hip, scan_conv.hip and scan_hold.hip.
#include "scan_kernel.h"

#include <mutex>

namespace s6i {

// Device scratch of s6_scan_fwd_noalloc: every GPU the library runs on holds
// its own copy for the life of the process.  In host code `scratch` is only a
// stand-in for the symbol; its device address comes from hipGetSymbolAddress
// (scratch_ptr), once per device.
constexpr size_t kScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

// Fold segment aggregates into every segment's incoming state:
// H_0 = h0 (or 0); H_{s+1} = exp(A * sum_delta_s) * H_s + S_s.
// hin (S, batch*D*N) receives H_s for s < S; hlast (nullable) gets the state
// after the last of the `nagg` aggregates.  A is (D, N), or (D) with one value
// per channel when a_per_channel is set.
__global__ void s6_fold_carries(const float* __restrict__ A, const float* __restrict__ h0,
                                const float* __restrict__ agg, const float* __restrict__ sumdelta,
                                float* __restrict__ hin, float* __restrict__ hlast, int64_t batch,
                                int64_t D, int64_t N, int64_t S, int64_t nagg, int a_per_channel) {
  const int64_t total = batch * D * N;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int64_t n = i % N;
  const int64_t bd = i / N;
  const int64_t d = bd % D;
  const float A2 = A[a_per_channel ? d : d * N + n] * kLog2e;
  float H = h0 ? h0[i] : 0.0f;
  // Eight segments at a time: their loads are issued before the dependent
  // chain through H (one load latency per eight steps, not per step); the
  // last batch's loads past nagg reread aggregate nagg - 1 and are not used.
  for (int64_t s = 0; s < S; s += 8) {
    float ag[8], sd[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t sj = nagg > 0 ? (s + j < nagg ? s + j : nagg - 1) : 0;
      ag[j] = nagg > 0 ? agg[sj * total + i] : 0.0f;
      sd[j] = nagg > 0 ? sumdelta[sj * batch * D + bd] : 0.0f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (s + j < S && hin) hin[(s + j) * total + i] = H;
      if (s + j < nagg) H = __builtin_fmaf(fast_exp2(A2 * sd[j]), H, ag[j]);
    }
  }
  if (hlast) hlast[i] = H;
}

// Copy h0 (or zeros) to h_last: the empty-sequence case.
__global__ void s6_copy_state(const float* __restrict__ h0, float* __restrict__ hl, int64_t total) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x)
    hl[i] = h0 ? h0[i] : 0.0f;
}

}  // namespace

// Segments: the scan kernel runs five waves per SIMD, i.e. 20 / W workgroups
// per CU (two for W = 8).  When batch * channel blocks fills less than half
// of those slots, L is cut into as many segments as keep the grid within
// one round of slots (each segment at least 4 chunks, and a multiple of 64
// tokens so the kernel's 4-chunk cycles have no phantom chunks).
Plan make_plan(int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate, size_t esz,
               const void* const* ptrs, int nptr) {
  Plan p;
  const int64_t need = (dstate + 3) / 4;
  p.W = need <= 1 ? 1 : need <= 2 ? 2 : need <= 4 ? 4 : 8;
  p.nblk = (dim + kCW - 1) / kCW;
  const int64_t wgs = p.nblk * batch;
  const int64_t slots = (int64_t)cu_count() * (p.W == 8 ? 2 : 20 / p.W);
  int64_t segs = 1;
  if (2 * wgs <= slots) {
    // twice as many segments as the workgroup slots hold at once (two rounds
    // of workgroups): measured faster than one round, 12.1 against 13.1 ms
    // on a million tokens of 1536 channels and 61 against 62.5 us on 2 x
    // 1536 channels x 2048 tokens
    segs = 2 * slots / wgs;
    const int64_t max_segs = (seqlen + 4 * kT - 1) / (4 * kT);
    if (segs > max_segs) segs = max_segs;
    if (segs < 1) segs = 1;
  }
  int64_t seg_len = (seqlen + segs - 1) / segs;
  seg_len = ((seg_len + 4 * kT - 1) / (4 * kT)) * (4 * kT);
  p.segs = (seqlen + seg_len - 1) / seg_len;
  if (p.segs < 1) p.segs = 1;
  p.seg_len = seg_len;
  const int64_t per_vec = 16 / (int64_t)esz;
  bool v = (seqlen % per_vec) == 0;
  for (int i = 0; i < nptr; ++i)
    if (ptrs[i] && !aligned(ptrs[i], 16)) v = false;
  p.vec = v;
  return p;
}

// Offsets (bytes, 256-aligned) of the segmented scan's buffers in the
// workspace: segment end states (nagg, batch, D, N), summed deltas (nagg,
// batch, D) and, for the fused pass, incoming states (S, batch, D, N).
ScanWs scan_ws_layout(bool want_y, const Plan& p, int64_t batch, int64_t dim, int64_t dstate) {
  ScanWs w{0, 0, 0, 0};
  if (p.segs <= 1) return w;
  auto up = [](size_t v) { return (v + 255) & ~(size_t)255; };
  const int64_t nstate = batch * dim * dstate;
  const int64_t nagg = want_y ? p.segs - 1 : p.segs;
  w.agg = 0;
  w.sd = up((size_t)nagg * nstate * sizeof(float));
  w.hin = w.sd + up((size_t)nagg * batch * dim * sizeof(float));
  w.total = w.hin + (want_y ? up((size_t)p.segs * nstate * sizeof(float)) : 0);
  return w;
}

// Kernels with the discretisation options and the convolution front only
// when one is set, so the plain path keeps its own code.
int launch_scan_any(int in_dtype, int mode, const ScanArgs& a, const Plan& p, bool gate, int64_t batch,
                    int64_t segs, hipStream_t st) {
  if (a.softplus || a.zoh || a.dbias || a.conv_w) return launch_scan_options(in_dtype, mode, a, p, gate, batch, segs, st);
  return launch_scan_e<0>(in_dtype, mode, a, p, gate, batch, segs, st);
}

int launch_fold_carries(const float* A, const float* h0, const float* agg, const float* sumdelta, float* hin,
                        float* hlast, int64_t batch, int64_t D, int64_t N, int64_t S, int64_t nagg,
                        hipStream_t st, bool a_per_channel) {
  const int64_t blocks = (batch * D * N + 255) / 256;
  hipLaunchKernelGGL(s6_fold_carries, dim3((unsigned)blocks), dim3(256), 0, st, A, h0, agg, sumdelta, hin, hlast,
                     batch, D, N, S, nagg, a_per_channel ? 1 : 0);
  S6_HIP(hipGetLastError(), "s6_fold_carries launch");
  return S6_OK;
}

int launch_copy_state(const float* src, float* dst, int64_t n, hipStream_t st) {
  if (n <= 0) return S6_OK;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(s6_copy_state, dim3((unsigned)blocks), dim3(256), 0, st, src, dst, n);
  S6_HIP(hipGetLastError(), "s6_copy_state launch");
  return S6_OK;
}

namespace {

// Device address of this device's `scratch`, looked up on the first call on
// each device (with that device current) and kept per device.
int scratch_ptr(void** out) {
  constexpr int kMaxDev = 64;
  static std::mutex mu;
  static void* ptrs[kMaxDev];
  int dev = 0;
  S6_HIP(hipGetDevice(&dev), "hipGetDevice");
  if (dev < 0 || dev >= kMaxDev) {
    snprintf(g_err, sizeof(g_err), "device %d: the static scratch is kept for devices 0..%d", dev, kMaxDev - 1);
    return S6_ERR_HIP;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    S6_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    ptrs[dev] = p;
  }
  *out = ptrs[dev];
  return S6_OK;
}

// The convolution front of s6_conv_scan_fwd: filter (D, width), bias,
// state before token 0; all null for the plain scan.
struct ConvFront {
  const float* w = nullptr;
  const float* bias = nullptr;
  const float* state = nullptr;
  int width = 0;
};

// Shared implementation of s6_scan_fwd(_ex), s6_conv_scan_fwd (want_y) and
// s6_last_state(_ex).
int scan_impl(bool want_y, int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate, int in_dtype,
              const void* x, const void* delta, const float* dbias, int flags, const float* A,
              const void* Bm, const void* Cm, const float* Dskip, const void* z, const float* h0,
              float* y, float* h_last, void* workspace, size_t workspace_bytes, void* stream,
              const ConvFront& cf = ConvFront(), float* ckpt = nullptr, bool static_ws = false) {
  int rc = check_common(batch, dim, seqlen, dstate, in_dtype);
  if (rc) return rc;
  if (flags & ~(S6_DELTA_SOFTPLUS | S6_ZOH_EXACT)) return S6_ERR_FLAGS;
  if (dbias && !aligned(dbias, 4)) return S6_ERR_ALIGN;
  if (cf.w || cf.width) {
    if (cf.width < 1 || cf.width > kMaxConv) return S6_ERR_UNSUPPORTED;
    if (!cf.w) return S6_ERR_NULL;
    const void* cps[] = {cf.w, cf.bias, cf.state};
    for (const void* p : cps)
      if (p && !aligned(p, 4)) return S6_ERR_ALIGN;
  }
  const bool work = batch > 0 && dim > 0 && seqlen > 0;
  if (work && (!x || !delta || !A || !Bm || (want_y && (!Cm || !y)))) return S6_ERR_NULL;
  if (!want_y && !h_last) return S6_ERR_NULL;
  const size_t esz = in_dtype == S6_BF16 ? 2 : 4;
  const void* ins[] = {x, delta, Bm, Cm, z};
  for (const void* p : ins)
    if (p && !aligned(p, esz)) return S6_ERR_ALIGN;
  const void* f32s[] = {A, Dskip, h0, y, h_last, ckpt};
  for (const void* p : f32s)
    if (p && !aligned(p, 4)) return S6_ERR_ALIGN;

  hipStream_t st = static_cast<hipStream_t>(stream);
  if (batch == 0 || dim == 0) return S6_OK;
  const int64_t nstate = batch * dim * dstate;
  if (seqlen == 0) {
    if (h_last) {
      int64_t blocks = (nstate + 255) / 256;
      if (blocks > 65536) blocks = 65536;
      hipLaunchKernelGGL(s6_copy_state, dim3((unsigned)blocks), dim3(256), 0, st, h0, h_last, nstate);
      S6_HIP(hipGetLastError(), "s6_copy_state launch");
    }
    return S6_OK;
  }

  const void* vecptrs[] = {x, delta, Bm, Cm, z, (const void*)y};
  const Plan p = make_plan(batch, dim, seqlen, dstate, esz, vecptrs, 6);
  const bool gate = want_y && z != nullptr;
  const int64_t S = p.segs;
  const ScanWs wl = scan_ws_layout(want_y, p, batch, dim, dstate);
  if (static_ws && wl.total > 0) {
    // the library's own scratch instead of a caller's workspace
    if (wl.total > kScratchBytes) return S6_ERR_WORKSPACE;
    rc = scratch_ptr(&workspace);
    if (rc) return rc;
    workspace_bytes = kScratchBytes;
  }
  if (wl.total > 0 && (!workspace || workspace_bytes < wl.total)) return S6_ERR_WORKSPACE;
  if (wl.total > 0 && !aligned(workspace, 256)) return S6_ERR_ALIGN;

  ScanArgs a;
  memset(&a, 0, sizeof(a));
  a.x = x; a.delta = delta; a.z = gate ? z : nullptr; a.Bm = Bm; a.Cm = want_y ? Cm : nullptr;
  a.A = A; a.Dskip = want_y ? Dskip : nullptr;
  a.softplus = (flags & S6_DELTA_SOFTPLUS) != 0;
  a.zoh = (flags & S6_ZOH_EXACT) != 0;
  a.dbias = dbias;
  a.conv_w = cf.w; a.conv_b = cf.bias; a.conv_state = cf.state; a.conv_k = cf.width;
  a.D = dim; a.L = seqlen; a.N = dstate; a.seg_len = p.seg_len;
  a.ckpt = want_y ? ckpt : nullptr;

  if (S == 1) {
    a.hinit = h0;
    a.hout = h_last;
    a.hout_last_only = 1;
    a.y = y;
    return launch_scan_any(in_dtype, want_y ? kModeY : kModeState, a, p, gate, batch, 1, st);
  }

  // Segmented: the caller's workspace holds the segment end states, summed
  // deltas and incoming states.
  const int64_t nagg = want_y ? S - 1 : S;
  char* wp = static_cast<char*>(workspace);
  float* agg = reinterpret_cast<float*>(wp + wl.agg);
  float* sd = reinterpret_cast<float*>(wp + wl.sd);
  float* hin = reinterpret_cast<float*>(wp + wl.hin);

  // pass 1: end states of the first nagg segments from a zero state
  ScanArgs g = a;
  g.z = nullptr; g.Cm = nullptr; g.Dskip = nullptr; g.ckpt = nullptr;
  g.hinit = nullptr;
  g.hout = agg;
  g.hout_stride = nstate;
  g.sumdelta = sd;
  rc = launch_scan_any(in_dtype, kModeState, g, p, false, batch, nagg, st);
  if (rc == S6_OK) {
    const int64_t blocks = (nstate + 255) / 256;
    hipLaunchKernelGGL(s6_fold_carries, dim3((unsigned)blocks), dim3(256), 0, st, A, h0, agg, sd,
                       want_y ? hin : nullptr, want_y ? nullptr : h_last, batch, dim, dstate, S, nagg, 0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) rc = hip_fail(e, "s6_fold_carries launch");
  }
  // pass 2: the fused scan of every segment from its incoming state
  if (rc == S6_OK && want_y) {
    ScanArgs m = a;
    m.hinit = hin;
    m.hinit_stride = nstate;
    m.hout = h_last;
    m.hout_last_only = 1;
    m.y = y;
    rc = launch_scan_any(in_dtype, kModeY, m, p, gate, batch, S, st);
  }
  return rc;
}

// Workspace of the forward (want_y) or the final-state scan.
int scan_ws_query(bool want_y, int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate, int in_dtype,
                  size_t* bytes) {
  if (!bytes) return S6_ERR_NULL;
  int rc = check_common(batch, dim, seqlen, dstate, in_dtype);
  if (rc) return rc;
  *bytes = 0;
  if (batch == 0 || dim == 0 || seqlen == 0) return S6_OK;
  const Plan p = make_plan(batch, dim, seqlen, dstate, in_dtype == S6_BF16 ? 2 : 4, nullptr, 0);
  *bytes = scan_ws_layout(want_y, p, batch, dim, dstate).total;
  return S6_OK;
}

}  // namespace

}  // namespace s6i

using namespace s6i;

extern "C" {

int s6_scan_fwd(int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate, int in_dtype,
                const void* x, const void* delta, const float* A, const void* Bm, const void* Cm,
                const float* Dskip, const void* z, const float* h0, float* y, float* h_last,
                void* workspace, size_t workspace_bytes, void* stream) {
  return scan_impl(true, batch, dim, seqlen, dstate, in_dtype, x, delta, nullptr, 0, A, Bm, Cm, Dskip,
                   z, h0, y, h_last, workspace, workspace_bytes, stream);
}

int s6_scan_fwd_noalloc(int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate, int in_dtype,
                        const void* x, const void* delta, const float* A, const void* Bm, const void* Cm,
                        const float* Dskip, const void* z, const float* h0, float* y, float* h_last,
                        void* stream) {
  return scan_impl(true, batch, dim, seqlen, dstate, in_dtype, x, delta, nullptr, 0, A, Bm, Cm, Dskip,
                   z, h0, y, h_last, nullptr, 0, stream, ConvFront(), nullptr, true);
}

int s6_scan_fwd_ex(int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate, int in_dtype,
                   const void* x, const void* delta, const float* delta_bias, int flags,
                   const float* A, const void* Bm, const void* Cm, const float* Dskip, const void* z,
                   const float* h0, float* y, float* h_last, void* workspace, size_t workspace_bytes,
                   void* stream) {
  return scan_impl(true, batch, dim, seqlen, dstate, in_dtype, x, delta, delta_bias, flags, A, Bm, Cm,
                   Dskip, z, h0, y, h_last, workspace, workspace_bytes, stream);
}

int s6_conv_scan_fwd(int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate, int in_dtype,
                     const void* x, const float* conv_w, const float* conv_bias, int conv_width,
                     const float* conv_state, const void* delta, const float* delta_bias, int flags,
                     const float* A, const void* Bm, const void* Cm, const float* Dskip, const void* z,
                     const float* h0, float* y, float* h_last, void* workspace, size_t workspace_bytes,
                     void* stream) {
  ConvFront cf;
  cf.w = conv_w;
  cf.bias = conv_bias;
  cf.state = conv_state;
  cf.width = conv_width;
  if (!conv_w && conv_width == 0) return S6_ERR_NULL;
  return scan_impl(true, batch, dim, seqlen, dstate, in_dtype, x, delta, delta_bias, flags, A, Bm, Cm,
                   Dskip, z, h0, y, h_last, workspace, workspace_bytes, stream, cf);
}

int s6_scan_fwd_ckpt(int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate, int in_dtype,
                     const void* x, const void* delta, const float* delta_bias, int flags,
                     const float* A, const void* Bm, const void* Cm, const float* Dskip, const void* z,
                     const float* h0, float* y, float* h_last, float* ckpt, void* workspace,
                     size_t workspace_bytes, void* stream) {
  if (!ckpt && batch > 0 && dim > 0 && seqlen > 0) return S6_ERR_NULL;
  return scan_impl(true, batch, dim, seqlen, dstate, in_dtype, x, delta, delta_bias, flags, A, Bm, Cm,
                   Dskip, z, h0, y, h_last, workspace, workspace_bytes, stream, ConvFront(), ckpt);
}

int s6_last_state(int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate, int in_dtype,
                  const void* x, const void* delta, const float* A, const void* Bm,
                  const float* h0, float* h_last, void* workspace, size_t workspace_bytes, void* stream) {
  return scan_impl(false, batch, dim, seqlen, dstate, in_dtype, x, delta, nullptr, 0, A, Bm, nullptr,
                   nullptr, nullptr, h0, nullptr, h_last, workspace, workspace_bytes, stream);
}

int s6_last_state_ex(int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate, int in_dtype,
                     const void* x, const void* delta, const float* delta_bias, int flags,
                     const float* A, const void* Bm, const float* h0, float* h_last, void* workspace,
                     size_t workspace_bytes, void* stream) {
  return scan_impl(false, batch, dim, seqlen, dstate, in_dtype, x, delta, delta_bias, flags, A, Bm,
                   nullptr, nullptr, nullptr, h0, nullptr, h_last, workspace, workspace_bytes, stream);
}

int s6_scan_fwd_workspace_size(int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate, int in_dtype,
                               size_t* bytes) {
  return scan_ws_query(true, batch, dim, seqlen, dstate, in_dtype, bytes);
}

int s6_last_state_workspace_size(int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate, int in_dtype,
                                 size_t* bytes) {
  return scan_ws_query(false, batch, dim, seqlen, dstate, in_dtype, bytes);
}

}  // extern "C"
