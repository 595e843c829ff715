// libs6 -- selective SSM scan (S6) for AMD MI355X (gfx950): kernels and C ABI.
//
// What is computed: see include/s6.h, which cites the pages ("【LLM】Mamba和
// State Space Models详解" §2.2-§2.4 and §3.2-§3.4).  This file only
// restates the recurrence per (batch, channel, state):
//     h = exp(delta*A) * h + delta*B*x ;  y = (sum_n C*h + D*x) * SiLU(z)
//
// Design (gfx950, wave64):
//  * The path is bound by the exponential (v_exp_f32 issues from the same
//    VALU port as FMA at a quarter of its rate) and by HBM streaming, not by
//    a dense contraction, so no MFMA is used.
//  * Workgroup = 64 channels of one batch row x G waves; lane = channel,
//    wave w = states [4w, 4w+4).  B and C of a token are then the same for
//    the whole wave and are read with scalar loads into SGPRs from a packed
//    fp32 copy [batch][L][G][B0..B3 C0..C3] made by s6_pack_bc.  A, the
//    state h and the per-lane partial output stay in VGPRs; the
//    (batch, D, L, N) state is never written anywhere.
//  * x, delta, z are staged per chunk of kT tokens into LDS with coalesced
//    row loads (token-major tiles, padded pitch), read there by every wave.
//  * Each wave writes its partial sum over its 4 states per token into LDS;
//    after the chunk every wave finalises a 1/G share of the tokens (sum of
//    G partials, skip term, gate) into the x tile, which is then stored to y
//    with coalesced row writes.
//  * Few long rows (too few workgroups to fill 256 CUs) are cut into
//    segments along L: pass 1 computes every segment's end state from zero
//    and its summed delta, a tiny pass folds them into each segment's
//    incoming state (associativity of the (a, b) pairs), and pass 2 runs the
//    fused scan of every segment from its incoming state.
//  * Decode: one lane per 4 states of a channel, h streamed in place with
//    16-byte accesses, partial outputs reduced across the channel's lanes.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "s6.h"

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kCh = 64;            // channels per workgroup (one per lane)
constexpr int kNS = 4;             // states per lane
constexpr int kT = 16;             // tokens per chunk
constexpr int kPitch = kCh + 1;    // LDS tile pitch in floats (token-major [t][c])
constexpr int kMaxN = 32;          // largest dstate supported
constexpr int kMaxG = kMaxN / kNS; // waves per workgroup at most

typedef const float __attribute__((address_space(4)))* const_f32_p;

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

__device__ __forceinline__ float fast_exp2(float v) { return __builtin_amdgcn_exp2f(v); }
__device__ __forceinline__ float fast_rcp(float v) { return __builtin_amdgcn_rcpf(v); }

// SiLU(z) = z / (1 + e^-z) = z * rcp(1 + 2^(-z*log2 e))
__device__ __forceinline__ float silu(float z) { return z * fast_rcp(1.0f + fast_exp2(-z * kLog2e)); }

// ----------------------------------------------------------------- packing --
// B, C (batch, N, L) -> fp32 [batch][L][G][8] with slot j < 4 = B[4g + j],
// slot 4 + j = C[4g + j]; states beyond N are zero.
template <typename In>
__global__ void s6_pack_bc(const In* __restrict__ Bm, const In* __restrict__ Cm,
                           float* __restrict__ out, int64_t batch, int64_t L, int64_t N, int64_t G) {
  const int64_t total = batch * L * G * 8;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t slot = i & 7;
    const int64_t g = (i >> 3) % G;
    const int64_t t = (i / (8 * G)) % L;
    const int64_t b = i / (8 * G * L);
    const int64_t n = g * kNS + (slot & 3);
    float v = 0.0f;
    if (n < N) {
      const In* src = (slot < 4) ? Bm : Cm;
      v = to_f32(src[(b * N + n) * L + t]);
    }
    out[i] = v;
  }
}

// -------------------------------------------------------------------- scan --
enum { kModeY = 0, kModeState = 1 };

struct ScanArgs {
  const void* x;
  const void* delta;
  const void* z;          // gate input (kModeY with GATE only)
  const float* A;         // (D, N)
  const float* Dskip;     // (D) or null
  const float* bc;        // packed B/C
  const float* hinit;     // initial states or null (zero)
  float* y;               // kModeY output
  float* hout;            // final states or null
  float* sumdelta;        // kModeState: per-segment sum of delta (S, batch, D) or null
  int64_t D, L, N, G;
  int64_t seg_len;        // tokens per segment (multiple of kT); segment = blockIdx.z
  int64_t hinit_stride;   // elements between segments in hinit (0: same for all)
  int64_t hout_stride;    // elements between segments in hout
  int64_t hout_last_only; // 1: only the last segment writes hout (at offset 0)
};

// Load one chunk of a (rows, L) tensor into a token-major LDS tile.
// VEC = elements per 16-byte vector (1 = element loads).
template <typename In, int VEC>
__device__ __forceinline__ void stage_tile(float* __restrict__ tile, const In* __restrict__ src,
                                           int64_t row0, int64_t rows_valid, int64_t L, int64_t t0,
                                           int64_t tend, int tid, int nthr) {
  constexpr int kVecs = kT / VEC;  // vectors per row per chunk
  for (int i = tid; i < kCh * kVecs; i += nthr) {
    const int c = i / kVecs;
    const int v = i - c * kVecs;
    const int64_t t = t0 + v * VEC;
    const bool ok = (c < rows_valid) && (t < tend);
    if constexpr (VEC == 1) {
      float val = ok ? to_f32(src[(row0 + c) * L + t]) : 0.0f;
      tile[v * kPitch + c] = val;
    } else {
      uint4 raw = make_uint4(0u, 0u, 0u, 0u);
      if (ok) raw = *reinterpret_cast<const uint4*>(src + (row0 + c) * L + t);
      const In* e = reinterpret_cast<const In*>(&raw);
#pragma unroll
      for (int k = 0; k < VEC; ++k) tile[(v * VEC + k) * kPitch + c] = to_f32(e[k]);
    }
  }
}

template <typename In, int VEC, bool GATE, int MODE>
__global__ void __launch_bounds__(kCh * kMaxG) s6_scan_kernel(ScanArgs a) {
  extern __shared__ float lds[];
  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  const int lane = tid & (kCh - 1);
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = (int)a.G;
  const int64_t D = a.D, L = a.L, N = a.N;
  const int64_t nblk = (a.D + kCh - 1) / kCh;
  const int64_t b = blockIdx.x / nblk;
  const int64_t d0 = (int64_t)(blockIdx.x % nblk) * kCh;
  const int64_t d = d0 + lane;
  const bool chv = d < D;
  const int64_t rows_valid = D - d0;
  const int64_t seg = blockIdx.z;
  const int64_t tb = seg * a.seg_len;
  const int64_t te = (tb + a.seg_len < L) ? tb + a.seg_len : L;
  const int64_t row0 = b * D + d0;

  constexpr int kTiles = (MODE == kModeY) ? (GATE ? 3 : 2) : 2;
  float* tx = lds;
  float* tdl = lds + kT * kPitch;
  float* tz = lds + 2 * kT * kPitch;
  float* part = lds + kTiles * kT * kPitch;

  const In* xp = static_cast<const In*>(a.x);
  const In* dp = static_cast<const In*>(a.delta);
  const In* zp = static_cast<const In*>(a.z);

  float A2[kNS], h[kNS];
#pragma unroll
  for (int j = 0; j < kNS; ++j) {
    const int64_t n = (int64_t)w * kNS + j;
    const bool sv = chv && n < N;
    A2[j] = sv ? a.A[d * N + n] * kLog2e : 0.0f;
    h[j] = (sv && a.hinit) ? a.hinit[seg * a.hinit_stride + (b * D + d) * N + n] : 0.0f;
  }
  const float dsk = (MODE == kModeY && a.Dskip && chv) ? a.Dskip[d] : 0.0f;
  double dsum = 0.0;

  for (int64_t t0 = tb; t0 < te; t0 += kT) {
    const int nt = (int)((te - t0) < kT ? (te - t0) : kT);
    __syncthreads();  // previous chunk fully consumed
    stage_tile<In, VEC>(tx, xp, row0, rows_valid, L, t0, te, tid, nthr);
    stage_tile<In, VEC>(tdl, dp, row0, rows_valid, L, t0, te, tid, nthr);
    if constexpr (MODE == kModeY && GATE) stage_tile<In, VEC>(tz, zp, row0, rows_valid, L, t0, te, tid, nthr);
    __syncthreads();

    const float* bcrow = a.bc + ((b * L + t0) * G + w) * 8;
    float csum = 0.0f;
    for (int t = 0; t < nt; ++t) {
      const float dt = tdl[t * kPitch + lane];
      const float xt = tx[t * kPitch + lane];
      const float u = dt * xt;
      const_f32_p q = (const_f32_p)(bcrow + (int64_t)t * G * 8);
      float yp = 0.0f;
#pragma unroll
      for (int j = 0; j < kNS; ++j) {
        const float e = fast_exp2(dt * A2[j]);
        h[j] = __builtin_fmaf(e, h[j], u * q[j]);
        if constexpr (MODE == kModeY) yp = __builtin_fmaf(q[kNS + j], h[j], yp);
      }
      if constexpr (MODE == kModeY) part[(w * kT + t) * kCh + lane] = yp;
      else csum += dt;
    }
    if constexpr (MODE == kModeState) dsum += (double)csum;

    if constexpr (MODE == kModeY) {
      __syncthreads();
      for (int t = w; t < nt; t += G) {
        float ys = 0.0f;
        for (int g = 0; g < G; ++g) ys += part[(g * kT + t) * kCh + lane];
        ys = __builtin_fmaf(dsk, tx[t * kPitch + lane], ys);
        if constexpr (GATE) ys *= silu(tz[t * kPitch + lane]);
        tx[t * kPitch + lane] = ys;  // y replaces x in the tile
      }
      __syncthreads();
      // coalesced store of the y tile: rows of nt fp32 values
      constexpr int kVY = (VEC == 1) ? 1 : 4;
      constexpr int kVecs = kT / kVY;
      for (int i = tid; i < kCh * kVecs; i += nthr) {
        const int c = i / kVecs;
        const int v = i - c * kVecs;
        const int64_t t = t0 + v * kVY;
        if (c < rows_valid && t < te) {
          float* dst = a.y + (row0 + c) * L + t;
          if constexpr (kVY == 1) {
            *dst = tx[v * kPitch + c];
          } else {
            float4 o;
            o.x = tx[(v * 4 + 0) * kPitch + c];
            o.y = tx[(v * 4 + 1) * kPitch + c];
            o.z = tx[(v * 4 + 2) * kPitch + c];
            o.w = tx[(v * 4 + 3) * kPitch + c];
            *reinterpret_cast<float4*>(dst) = o;
          }
        }
      }
    }
  }

  const bool write_h = a.hout && (!a.hout_last_only || seg == (int64_t)gridDim.z - 1);
  if (write_h && chv) {
    const int64_t off = a.hout_last_only ? 0 : seg * a.hout_stride;
#pragma unroll
    for (int j = 0; j < kNS; ++j) {
      const int64_t n = (int64_t)w * kNS + j;
      if (n < N) a.hout[off + (b * D + d) * N + n] = h[j];
    }
  }
  if constexpr (MODE == kModeState) {
    if (a.sumdelta && chv && w == 0) a.sumdelta[seg * (int64_t)(gridDim.x / nblk) * D + b * D + d] = (float)dsum;
  }
}

// Fold segment aggregates into every segment's incoming state:
// H_0 = h0 (or 0); H_{s+1} = exp(A * sum_delta_s) * H_s + S_s.
// hin (S, batch*D*N) receives H_s for s < S; hlast (nullable) gets H_S when
// `nagg` == S aggregates are present.
__global__ void s6_fold_carries(const float* __restrict__ A, const float* __restrict__ h0,
                                const float* __restrict__ agg, const float* __restrict__ sumdelta,
                                float* __restrict__ hin, float* __restrict__ hlast, int64_t batch,
                                int64_t D, int64_t N, int64_t S, int64_t nagg) {
  const int64_t total = batch * D * N;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int64_t n = i % N;
  const int64_t bd = i / N;
  const int64_t d = bd % D;
  const float A2 = A[d * N + n] * kLog2e;
  float H = h0 ? h0[i] : 0.0f;
  for (int64_t s = 0; s < S; ++s) {
    if (hin) hin[s * total + i] = H;
    if (s < nagg) {
      const float P = fast_exp2(A2 * sumdelta[s * batch * D + bd]);
      H = __builtin_fmaf(P, H, agg[s * total + i]);
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

// ------------------------------------------------------------------ decode --
struct StepArgs {
  float* h;
  const void* x;
  const void* delta;
  const void* z;
  const float* A;
  const void* Bm;
  const void* Cm;
  const float* Dskip;
  float* y;
  int64_t batch, D, N;
};

// P lanes per channel, 4 states per lane.  V4: 16-byte state accesses
// (N % 4 == 0 and h 16-byte aligned).
template <typename In, bool GATE, int P, bool V4>
__global__ void __launch_bounds__(256) s6_step_kernel(StepArgs a) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t ch = gid / P;
  const int q = (int)(gid % P);
  const int64_t pairs = a.batch * a.D;
  const bool valid = ch < pairs;
  const int64_t N = a.N;
  const int64_t b = valid ? ch / a.D : 0;
  const int64_t d = valid ? ch % a.D : 0;
  const In* xp = static_cast<const In*>(a.x);
  const In* dp = static_cast<const In*>(a.delta);
  const In* zp = static_cast<const In*>(a.z);
  const In* Bp = static_cast<const In*>(a.Bm);
  const In* Cp = static_cast<const In*>(a.Cm);

  float hv[4] = {0.f, 0.f, 0.f, 0.f};
  float yp = 0.0f;
  float xt = 0.0f;
  if (valid) {
    const float dt = to_f32(dp[ch]);
    xt = to_f32(xp[ch]);
    const float u = dt * xt;
    float* hrow = a.h + ch * N;
    const int64_t n0 = (int64_t)q * 4;
    if constexpr (V4) {
      if (n0 < N) {
        const float4 v = *reinterpret_cast<const float4*>(hrow + n0);
        hv[0] = v.x; hv[1] = v.y; hv[2] = v.z; hv[3] = v.w;
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (n0 + j < N) hv[j] = hrow[n0 + j];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t n = n0 + j;
      if (n < N) {
        const float e = fast_exp2(dt * (a.A[d * N + n] * kLog2e));
        hv[j] = __builtin_fmaf(e, hv[j], u * to_f32(Bp[b * N + n]));
        yp = __builtin_fmaf(to_f32(Cp[b * N + n]), hv[j], yp);
      }
    }
    if constexpr (V4) {
      if (n0 < N) *reinterpret_cast<float4*>(hrow + n0) = make_float4(hv[0], hv[1], hv[2], hv[3]);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (n0 + j < N) hrow[n0 + j] = hv[j];
    }
  }
  // reduce the P partial outputs of a channel (P consecutive lanes)
#pragma unroll
  for (int off = P / 2; off > 0; off >>= 1) yp += __shfl_xor(yp, off, P);
  if (valid && q == 0) {
    float yv = yp;
    if (a.Dskip) yv = __builtin_fmaf(a.Dskip[d], xt, yv);
    if constexpr (GATE) yv *= silu(to_f32(zp[ch]));
    a.y[ch] = yv;
  }
}

// ------------------------------------------------------------------- host --
thread_local char g_err[256];

int hip_fail(hipError_t e, const char* what) {
  snprintf(g_err, sizeof(g_err), "HIP error in %s: %s", what, hipGetErrorString(e));
  return S6_ERR_HIP;
}

#define S6_HIP(call, what)                       \
  do {                                           \
    hipError_t e_ = (call);                      \
    if (e_ != hipSuccess) return hip_fail(e_, what); \
  } while (0)

bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a == 0 || b == 0) { *out = 0; return true; }
  if (a > INT64_MAX / b) return false;
  *out = a * b;
  return true;
}

bool aligned(const void* p, size_t al) { return ((uintptr_t)p % al) == 0; }

int check_common(int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate, int in_dtype) {
  if (in_dtype != S6_F32 && in_dtype != S6_BF16) return S6_ERR_DTYPE;
  if (batch < 0 || dim < 0 || seqlen < 0 || dstate < 0) return S6_ERR_SHAPE;
  if (dstate < 1 || dstate > kMaxN) return S6_ERR_UNSUPPORTED;
  int64_t t;
  if (!mul_ok(batch, dim, &t) || !mul_ok(t, seqlen > 0 ? seqlen : 1, &t) ||
      !mul_ok(t, 64, &t))  // headroom for packed and per-state buffers
    return S6_ERR_SHAPE;
  int64_t u;
  if (!mul_ok(batch, seqlen > 0 ? seqlen : 1, &u) || !mul_ok(u, 8 * kMaxG, &u)) return S6_ERR_SHAPE;
  if (batch * ((dim + kCh - 1) / kCh) > INT32_MAX) return S6_ERR_SHAPE;  // grid size
  return S6_OK;
}

struct Plan {
  int64_t G, nblk, segs, seg_len;
  int vec;
};

// Segments: enough workgroups to give every CU about three; a segment holds
// at least 4 chunks.
Plan make_plan(int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate, size_t esz,
               const void* const* ptrs, int nptr) {
  Plan p;
  p.G = (dstate + kNS - 1) / kNS;
  p.nblk = (dim + kCh - 1) / kCh;
  const int64_t wgs = p.nblk * batch;
  const int64_t target = 768;
  int64_t segs = 1;
  if (wgs < 512) {
    segs = (target + wgs - 1) / wgs;
    const int64_t max_segs = (seqlen + 4 * kT - 1) / (4 * kT);
    if (segs > max_segs) segs = max_segs;
    if (segs < 1) segs = 1;
  }
  int64_t seg_len = (seqlen + segs - 1) / segs;
  seg_len = ((seg_len + kT - 1) / kT) * kT;
  if (seg_len < kT) seg_len = kT;
  p.segs = (seqlen + seg_len - 1) / seg_len;
  if (p.segs < 1) p.segs = 1;
  p.seg_len = seg_len;
  const int64_t per_vec = 16 / (int64_t)esz;
  bool v = (seqlen % per_vec) == 0;
  for (int i = 0; i < nptr; ++i)
    if (ptrs[i] && !aligned(ptrs[i], 16)) v = false;
  p.vec = v ? 1 : 0;
  return p;
}

template <typename In>
int launch_pack(const void* Bm, const void* Cm, float* out, int64_t batch, int64_t L, int64_t N,
                int64_t G, hipStream_t st) {
  const int64_t total = batch * L * G * 8;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL((s6_pack_bc<In>), dim3((unsigned)blocks), dim3(256), 0, st,
                     static_cast<const In*>(Bm), static_cast<const In*>(Cm), out, batch, L, N, G);
  S6_HIP(hipGetLastError(), "s6_pack_bc launch");
  return S6_OK;
}

template <typename In, int VEC, bool GATE, int MODE>
int launch_scan_t(const ScanArgs& a, int64_t batch, int64_t nblk, int64_t segs, hipStream_t st) {
  const int tiles = (MODE == kModeY) ? (GATE ? 3 : 2) : 2;
  size_t lds = (size_t)tiles * kT * kPitch * sizeof(float);
  if (MODE == kModeY) lds += (size_t)a.G * kT * kCh * sizeof(float);
  dim3 grid((unsigned)(nblk * batch), 1u, (unsigned)segs);
  hipLaunchKernelGGL((s6_scan_kernel<In, VEC, GATE, MODE>), grid, dim3((unsigned)(a.G * kCh)), lds, st, a);
  S6_HIP(hipGetLastError(), "s6_scan_kernel launch");
  return S6_OK;
}

template <typename In, int MODE>
int launch_scan(const ScanArgs& a, bool vec, bool gate, int64_t batch, int64_t nblk, int64_t segs,
                hipStream_t st) {
  constexpr int kV = 16 / sizeof(In);
  if constexpr (MODE == kModeY) {
    if (vec && gate) return launch_scan_t<In, kV, true, MODE>(a, batch, nblk, segs, st);
    if (vec) return launch_scan_t<In, kV, false, MODE>(a, batch, nblk, segs, st);
    if (gate) return launch_scan_t<In, 1, true, MODE>(a, batch, nblk, segs, st);
    return launch_scan_t<In, 1, false, MODE>(a, batch, nblk, segs, st);
  } else {
    if (vec) return launch_scan_t<In, kV, false, MODE>(a, batch, nblk, segs, st);
    return launch_scan_t<In, 1, false, MODE>(a, batch, nblk, segs, st);
  }
}

int launch_scan_any(int in_dtype, int mode, const ScanArgs& a, bool vec, bool gate, int64_t batch,
                    int64_t nblk, int64_t segs, hipStream_t st) {
  if (in_dtype == S6_BF16) {
    return mode == kModeY ? launch_scan<uint16_t, kModeY>(a, vec, gate, batch, nblk, segs, st)
                          : launch_scan<uint16_t, kModeState>(a, vec, gate, batch, nblk, segs, st);
  }
  return mode == kModeY ? launch_scan<float, kModeY>(a, vec, gate, batch, nblk, segs, st)
                        : launch_scan<float, kModeState>(a, vec, gate, batch, nblk, segs, st);
}

// Shared implementation of s6_scan_fwd (want_y) and s6_last_state.
int scan_impl(bool want_y, int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate, int in_dtype,
              const void* x, const void* delta, const float* A, const void* Bm, const void* Cm,
              const float* Dskip, const void* z, const float* h0, float* y, float* h_last,
              void* stream) {
  int rc = check_common(batch, dim, seqlen, dstate, in_dtype);
  if (rc) return rc;
  const bool work = batch > 0 && dim > 0 && seqlen > 0;
  if (work && (!x || !delta || !A || !Bm || (want_y && (!Cm || !y)))) return S6_ERR_NULL;
  if (!want_y && !h_last) return S6_ERR_NULL;
  const size_t esz = in_dtype == S6_BF16 ? 2 : 4;
  const void* ins[] = {x, delta, Bm, Cm, z};
  for (const void* p : ins)
    if (p && !aligned(p, esz)) return S6_ERR_ALIGN;
  const void* f32s[] = {A, Dskip, h0, y, h_last};
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

  const void* vecptrs[] = {x, delta, z, (const void*)y};
  Plan p = make_plan(batch, dim, seqlen, dstate, esz, vecptrs, want_y ? 4 : 2);
  const bool gate = want_y && z != nullptr;
  const int64_t S = p.segs;

  // workspace: packed B/C, then (segmented) aggregates, sums of delta, carries
  const size_t bc_bytes = (size_t)batch * seqlen * p.G * 8 * sizeof(float);
  const int64_t nagg = want_y ? S - 1 : S;
  const size_t agg_bytes = (S > 1) ? (size_t)nagg * nstate * sizeof(float) : 0;
  const size_t sd_bytes = (S > 1) ? (size_t)nagg * batch * dim * sizeof(float) : 0;
  const size_t hin_bytes = (S > 1 && want_y) ? (size_t)S * nstate * sizeof(float) : 0;
  auto up = [](size_t v) { return (v + 255) & ~(size_t)255; };
  const size_t ws_bytes = up(bc_bytes) + up(agg_bytes) + up(sd_bytes) + up(hin_bytes);
  void* ws = nullptr;
  S6_HIP(hipMallocAsync(&ws, ws_bytes, st), "hipMallocAsync(workspace)");
  char* wp = static_cast<char*>(ws);
  float* bc = reinterpret_cast<float*>(wp);
  float* agg = reinterpret_cast<float*>(wp + up(bc_bytes));
  float* sd = reinterpret_cast<float*>(wp + up(bc_bytes) + up(agg_bytes));
  float* hin = reinterpret_cast<float*>(wp + up(bc_bytes) + up(agg_bytes) + up(sd_bytes));

  rc = (in_dtype == S6_BF16)
           ? launch_pack<uint16_t>(Bm, want_y ? Cm : Bm, bc, batch, seqlen, dstate, p.G, st)
           : launch_pack<float>(Bm, want_y ? Cm : Bm, bc, batch, seqlen, dstate, p.G, st);

  ScanArgs a;
  memset(&a, 0, sizeof(a));
  a.x = x; a.delta = delta; a.z = z; a.A = A; a.Dskip = Dskip; a.bc = bc;
  a.D = dim; a.L = seqlen; a.N = dstate; a.G = p.G; a.seg_len = p.seg_len;

  if (rc == S6_OK && S > 1) {
    // pass 1: aggregates of the first nagg segments, from a zero state
    ScanArgs g = a;
    g.hinit = nullptr;
    g.hout = agg;
    g.hout_stride = nstate;
    g.sumdelta = sd;
    rc = launch_scan_any(in_dtype, kModeState, g, p.vec, false, batch, p.nblk, nagg, st);
    if (rc == S6_OK) {
      const int64_t blocks = (nstate + 255) / 256;
      hipLaunchKernelGGL(s6_fold_carries, dim3((unsigned)blocks), dim3(256), 0, st, A, h0, agg, sd,
                         want_y ? hin : nullptr, want_y ? nullptr : h_last, batch, dim, dstate, S, nagg);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) rc = hip_fail(e, "s6_fold_carries launch");
    }
  }
  if (rc == S6_OK && (want_y || S == 1)) {
    ScanArgs m = a;
    if (S > 1) {
      m.hinit = hin;
      m.hinit_stride = nstate;
    } else {
      m.hinit = h0;
    }
    m.hout = h_last;
    m.hout_last_only = 1;
    m.y = y;
    rc = launch_scan_any(in_dtype, want_y ? kModeY : kModeState, m, p.vec, gate, batch, p.nblk, S, st);
  }
  hipError_t e = hipFreeAsync(ws, st);
  if (rc == S6_OK && e != hipSuccess) rc = hip_fail(e, "hipFreeAsync(workspace)");
  return rc;
}

template <typename In, bool GATE, int P>
int launch_step_t(const StepArgs& a, bool v4, hipStream_t st) {
  const int64_t threads = a.batch * a.D * P;
  const int64_t blocks = (threads + 255) / 256;
  if (v4)
    hipLaunchKernelGGL((s6_step_kernel<In, GATE, P, true>), dim3((unsigned)blocks), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((s6_step_kernel<In, GATE, P, false>), dim3((unsigned)blocks), dim3(256), 0, st, a);
  S6_HIP(hipGetLastError(), "s6_step_kernel launch");
  return S6_OK;
}

template <typename In, bool GATE>
int launch_step_g(const StepArgs& a, bool v4, hipStream_t st) {
  const int64_t lanes = (a.N + 3) / 4;
  if (lanes <= 1) return launch_step_t<In, GATE, 1>(a, v4, st);
  if (lanes <= 2) return launch_step_t<In, GATE, 2>(a, v4, st);
  if (lanes <= 4) return launch_step_t<In, GATE, 4>(a, v4, st);
  return launch_step_t<In, GATE, 8>(a, v4, st);
}

}  // namespace

extern "C" {

int s6_version(void) { return 10000; }

const char* s6_status_str(int status) {
  switch (status) {
    case S6_OK: return "ok";
    case S6_ERR_NULL: return "a required pointer is NULL";
    case S6_ERR_SHAPE: return "invalid size (negative, or the element count overflows)";
    case S6_ERR_DTYPE: return "in_dtype must be S6_F32 or S6_BF16";
    case S6_ERR_UNSUPPORTED: return "dstate must be between 1 and 32";
    case S6_ERR_ALIGN: return "a pointer is not aligned to its element size";
    case S6_ERR_HIP: return g_err[0] ? g_err : "HIP error";
    default: return "unknown status";
  }
}

int s6_scan_fwd(int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate, int in_dtype,
                const void* x, const void* delta, const float* A, const void* Bm, const void* Cm,
                const float* Dskip, const void* z, const float* h0, float* y, float* h_last,
                void* stream) {
  return scan_impl(true, batch, dim, seqlen, dstate, in_dtype, x, delta, A, Bm, Cm, Dskip, z, h0, y,
                   h_last, stream);
}

int s6_last_state(int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate, int in_dtype,
                  const void* x, const void* delta, const float* A, const void* Bm,
                  const float* h0, float* h_last, void* stream) {
  return scan_impl(false, batch, dim, seqlen, dstate, in_dtype, x, delta, A, Bm, nullptr, nullptr,
                   nullptr, h0, nullptr, h_last, stream);
}

int s6_state_update(int64_t batch, int64_t dim, int64_t dstate, int in_dtype, float* h,
                    const void* x, const void* delta, const float* A, const void* Bm,
                    const void* Cm, const float* Dskip, const void* z, float* y, void* stream) {
  int rc = check_common(batch, dim, 1, dstate, in_dtype);
  if (rc) return rc;
  if (batch == 0 || dim == 0) return S6_OK;
  if (!h || !x || !delta || !A || !Bm || !Cm || !y) return S6_ERR_NULL;
  const size_t esz = in_dtype == S6_BF16 ? 2 : 4;
  const void* ins[] = {x, delta, Bm, Cm, z};
  for (const void* p : ins)
    if (p && !aligned(p, esz)) return S6_ERR_ALIGN;
  const void* f32s[] = {h, A, Dskip, y};
  for (const void* p : f32s)
    if (p && !aligned(p, 4)) return S6_ERR_ALIGN;
  StepArgs a;
  a.h = h; a.x = x; a.delta = delta; a.z = z; a.A = A; a.Bm = Bm; a.Cm = Cm; a.Dskip = Dskip; a.y = y;
  a.batch = batch; a.D = dim; a.N = dstate;
  const bool v4 = (dstate % 4 == 0) && aligned(h, 16);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (in_dtype == S6_BF16)
    return z ? launch_step_g<uint16_t, true>(a, v4, st) : launch_step_g<uint16_t, false>(a, v4, st);
  return z ? launch_step_g<float, true>(a, v4, st) : launch_step_g<float, false>(a, v4, st);
}

}  // extern "C"
