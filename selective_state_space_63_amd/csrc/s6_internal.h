// s6_internal.h -- shared internals of libs6 (not installed; the C ABI is
// include/s6.h): constants and device helpers of every kernel, the scan's
// argument block and launch entry points used by the backward, and the host
// helpers for argument checks and errors.
//
// What is computed: see include/s6.h, which cites the pages ("【LLM】Mamba和
// State Space Models详解" §2.2-§2.4 and §3.2-§3.4).  Per (batch, channel,
// state):  h = exp(delta*A) * h + delta*B*x ;  y = (sum_n C*h + D*x) * SiLU(z)
//
// Files: scan_kernel.h (the fused scan kernel), scan.hip (its plain
// instantiations, final-state scan, segments and carries, entry points),
// scan_ext.hip, scan_conv.hip, scan_hold.hip (option kernels: step bias
// and softplus; convolution front; exact hold), step.hip (decode step), bwd.hip
// (gradients), common.hip (checks, errors, version).
#ifndef S6_INTERNAL_H_
#define S6_INTERNAL_H_

#include <hip/hip_runtime.h>

#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <type_traits>
#include <utility>

#include "s6.h"

namespace s6i {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kCW = 32;            // channels per workgroup
constexpr int kT = 16;             // tokens per chunk
constexpr int kP = kT;             // LDS tile pitch in floats (channel-major [c][t], swizzled)
constexpr int kMaxN = 32;          // largest dstate supported
constexpr int kMaxConv = 4;        // widest filter of the convolution front
constexpr int kCkpt = 64;          // tokens per checkpoint block (S6_CKPT_TOKENS)

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

// Pointer into global memory.  Loads through it are global_load_*: a
// generic pointer picked among several could become a flat load, which also
// counts against the LDS wait counter and would stall LDS waits on prefetches.
template <typename T>
using gptr = const T __attribute__((address_space(1)))*;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));  // raw 16-byte piece

__device__ __forceinline__ float fast_exp2(float v) { return __builtin_amdgcn_exp2f(v); }
__device__ __forceinline__ float fast_rcp(float v) { return __builtin_amdgcn_rcpf(v); }

// SiLU(z) = z / (1 + e^-z) = z * rcp(1 + 2^(-z*log2 e))
__device__ __forceinline__ float silu(float z) { return z * fast_rcp(1.0f + fast_exp2(-z * kLog2e)); }

// softplus(v) = ln(1 + e^v) = max(v, 0) + ln(1 + w) with w = e^-|v| in (0, 1].
// ln(1 + w) is taken as w ln(u) / (u - 1) with u = 1 + w as rounded (Kahan's
// log1p): the rounding of u cancels between the two factors, so small w keep
// full relative accuracy.  u == 1 (w below 2^-24) gives w itself.
__device__ __forceinline__ float softplus_f(float v) {
  const float w = fast_exp2(-fabsf(v) * kLog2e);
  const float u = 1.0f + w;
  const float l = w * (__builtin_amdgcn_logf(u) * kLn2) * fast_rcp(u - 1.0f);
  return fmaxf(v, 0.0f) + (u == 1.0f ? w : l);
}

// Exact zero-order-hold input coefficient (e^(delta A) - 1) / A, the integral
// of e^(s A) over s in [0, delta], given arg = delta A log2(e) and e = 2^arg
// as computed for the state transition.  Taken as delta (e - 1) / ln(e) from
// the rounded e itself (Kahan's expm1), so the coefficient keeps full relative
// accuracy as delta A -> 0; e == 1 gives the limit delta.  Below 2^-64,
// e - 1 = -1 in fp32 and log2(e) is taken as arg (no underflow to 0).
__device__ __forceinline__ float zoh_coef(float dl, float arg, float e) {
  const float lg = arg < -64.0f ? arg : __builtin_amdgcn_logf(e);
  const float c = (e - 1.0f) * (dl * kLog2e) * fast_rcp(lg);
  return e == 1.0f ? dl : c;
}

// Value of lane J of this lane's 16-lane row (DPP row_newbcast).  Used as an
// operand of a multiply, the compiler folds it into v_mul_f32_dpp.
template <int J>
__device__ __forceinline__ float row_bcast(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x150 + J,
                                                               0xf, 0xf, true));
}

// Offset (floats) of the 4-token group `grp` of channel row c in a
// channel-major tile of pitch kT = 16.  The group index is XORed with
// ((c >> 2) & 3) ^ ((c >> 1) & 1), a swizzle that leaves no bank conflicts
// on gfx950 in either direction (measured with SQ_LDS_BANK_CONFLICT on
// each access pattern alone): 16-byte reads there take 16 lanes per cycle
// over 64 banks, so one group of 16 consecutive channels must cover all 64
// banks; 16-byte writes take 8 lanes over 32 banks, and the staging writes
// two groups of each of 4 consecutive rows at once.
__device__ __forceinline__ int tsw(int c, int grp) {
  return c * kP + ((grp ^ ((c >> 2) & 3) ^ ((c >> 1) & 1)) << 2);
}

// Value of lane CTRL's DPP source (a DPP control code: quad permutation, row
// rotation, row mirror, ...) in this lane; lanes whose source is outside the
// row read 0.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}

// ------------------------------------------------------------ scan entry --
enum { kModeY = 0, kModeState = 1 };

struct ScanArgs {
  const void* x;
  const void* delta;
  const void* z;          // gate input (kModeY with GATE only)
  const void* Bm;         // (batch, N, L)
  const void* Cm;         // (batch, N, L), kModeY only
  const float* A;         // (D, N)
  const float* Dskip;     // (D) or null
  const float* hinit;     // initial states or null (zero)
  float* y;               // kModeY output
  float* hout;            // final states or null
  float* sumdelta;        // kModeState without ckpt: per-segment sum of delta (S, batch, D) or null
  const float* dbias;     // (D) bias of the softplus step, or null (zero)
  int softplus;           // step = softplus(delta + dbias[d])  (option kernels only; the
                          // bias alone is added without it)
  int zoh;                // exact zero-order-hold input coefficient (option kernels only)
  const float* conv_w;    // (D, conv_k) causal filter of the convolution front, or null
                          // (option kernels only; x is then SiLU(conv_b + filter * x))
  const float* conv_b;    // (D) its bias, or null (zero)
  const float* conv_state;  // (batch, D, conv_k - 1) inputs before token 0, oldest first,
                            // or null (zero)
  int conv_k;             // filter width, 1..kMaxConv
  int64_t D, L, N;
  int64_t seg_len;        // tokens per segment (multiple of 4 kT); segment = blockIdx.z
  int64_t hinit_stride;   // elements between segments in hinit (0: same for all)
  int64_t hout_stride;    // elements between segments in hout
  int64_t hout_last_only; // 1: only the last segment writes hout (at offset 0)
  float* ckpt;            // kModeY: the state entering every kCkpt-token block,
                          // (ceil(L / kCkpt), batch, D, N); kModeState (one
                          // segment): the state entering every 2^ckpt_log2
                          // tokens, (ceil(L / 2^ckpt_log2), batch, D, N); or null
  int ckpt_log2;          // kModeState with ckpt: 4 (every kT-token chunk) or 6 (every kCkpt tokens)
};

struct Plan {
  int W;              // waves per workgroup (power of two, 4*W >= dstate)
  int64_t nblk;       // channel blocks per batch row
  int64_t segs;       // segments along L
  int64_t seg_len;    // tokens per segment, multiple of 4 kT
  bool vec;           // 16-byte staging and 8-byte stores
};

// Compute units of the current device (256 on MI355X; 256 when no device
// can be queried).
int cu_count();

// Launch plan of a scan: waves per workgroup, channel blocks, segments, and
// whether the 16-byte load path applies (every pointer in ptrs aligned).
Plan make_plan(int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate, size_t esz,
               const void* const* ptrs, int nptr);

// Byte offsets of a segmented scan's buffers in the caller's workspace, and
// its size (all zero when the plan has one segment).
struct ScanWs {
  size_t agg;    // segment end states from a zero state (nagg, batch, D, N)
  size_t sd;     // summed delta of those segments (nagg, batch, D)
  size_t hin;    // state entering every segment (S, batch, D, N), fused pass only
  size_t total;
};
ScanWs scan_ws_layout(bool want_y, const Plan& p, int64_t batch, int64_t dim, int64_t dstate);

// One launch of the scan kernel (mode kModeY or kModeState) over `segs`
// segments; the option kernels when a.softplus, a.zoh, a.dbias or a.conv_w
// is set.
int launch_scan_any(int in_dtype, int mode, const ScanArgs& a, const Plan& p, bool gate, int64_t batch,
                    int64_t segs, hipStream_t st);

// The option kernels: step bias, softplus, exact hold, convolution front
// (dispatch in scan_ext.hip).  Three levels, each compiled in a file of its
// own: the step bias and softplus (scan_ext.hip), those and the convolution
// front (scan_conv.hip), all of them and the exact hold (scan_hold.hip).
int launch_scan_options(int in_dtype, int mode, const ScanArgs& a, const Plan& p, bool gate, int64_t batch,
                        int64_t segs, hipStream_t st);
int launch_scan_conv(int in_dtype, int mode, const ScanArgs& a, const Plan& p, bool gate, int64_t batch,
                     int64_t segs, hipStream_t st);
int launch_scan_hold(int in_dtype, int mode, const ScanArgs& a, const Plan& p, bool gate, int64_t batch,
                     int64_t segs, hipStream_t st);

// The carry fold over segments: hin[s] (nullable) receives the state entering
// segment s, hlast (nullable) the state after the last of `nagg` aggregates.
int launch_fold_carries(const float* A, const float* h0, const float* agg, const float* sumdelta, float* hin,
                        float* hlast, int64_t batch, int64_t D, int64_t N, int64_t S, int64_t nagg,
                        hipStream_t st, bool a_per_channel = false);

// dst[i] = src ? src[i] : 0 for i < n.
int launch_copy_state(const float* src, float* dst, int64_t n, hipStream_t st);

// ------------------------------------------------------------ host helpers --
extern thread_local char g_err[256];

// Records the HIP error for s6_status_str and returns S6_ERR_HIP.
int hip_fail(hipError_t e, const char* what);

#define S6_HIP(call, what)                           \
  do {                                               \
    hipError_t e_ = (call);                          \
    if (e_ != hipSuccess) return hip_fail(e_, what); \
  } while (0)

bool mul_ok(int64_t a, int64_t b, int64_t* out);
inline bool aligned(const void* p, size_t al) { return ((uintptr_t)p % al) == 0; }

// Checks shared by every entry point (dtype, sizes, dstate, grid limits).
int check_common(int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate, int in_dtype);

// out[i] = v for i < n by a kernel (a captured graph can hold it).
void fill(float* p, float v, int64_t n, hipStream_t st);

}  // namespace s6i

#endif  // S6_INTERNAL_H_
