// step.hip -- the single-token decode step (s6_state_update and its _ex
// form): h is read, advanced by one token and written back in place.
//
// Layout: 4 states per lane (P = dstate / 4 adjacent lanes per channel,
// partial outputs added with DPP quad permutations), 4 batch rows per lane
// with all their loads issued first; h, A, B, C read and h written with
// 8/16-byte accesses that are contiguous across the lanes of a wave.  The
// step is HBM-bound (or Infinity-Cache-bound when the state fits there).
// s6_conv_state_update also runs the convolution front on the token: the
// filter over the kept inputs and the new one, then SiLU, and shifts the
// kept inputs by one.
#include "s6_internal.h"

namespace s6i {

namespace {

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
  const float* dbias;  // (D) step bias or null
  int softplus;        // step = softplus(delta + dbias[d])
  int zoh;             // exact zero-order-hold input coefficient
  const float* conv_w; // (D, conv_k) filter of the convolution front, or null
  const float* conv_b; // (D) its bias, or null
  float* conv_state;   // (batch, D, conv_k - 1) last inputs, oldest first; in/out
  int conv_k;
  int64_t batch, D, N;
};

// Value of lane g of this lane's quad (DPP quad broadcast; g is a constant
// once the caller's loop is unrolled).
__device__ __forceinline__ float quad_bcast(float v, int g) {
  switch (g) {
    case 0: return dpp_f<0x00>(v);
    case 1: return dpp_f<0x55>(v);
    case 2: return dpp_f<0xAA>(v);
    default: return dpp_f<0xFF>(v);
  }
}

// P lanes per channel, SPL states per lane (lane q: states q*SPL ...), G
// batch rows per lane (the same channel d of rows b0 .. b0+G-1, so the row of
// A is read once).  All G rows' loads are issued before any arithmetic.
// VEC: N == P * SPL and every row of h, A, B and C starts aligned, so h and A
// are read with 16-byte loads (h written back the same way) and B, C with
// 16- or 8-byte loads.  The step's B and C rows are the same for every
// channel of a batch row and stay in cache; h is streamed once in and once
// out.
template <typename In, bool GATE, int P, int SPL, bool VEC, int G, bool EXT>
__global__ void __launch_bounds__(256) s6_step_kernel(StepArgs a) {
  static_assert(!VEC || (SPL * sizeof(In)) % 8 == 0, "8- or 16-byte pieces of B and C");
  static_assert(P == 1 || P == 2 || P == 4, "lanes per channel");
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t idx = gid / P;  // (batch group, channel)
  const int q = (int)(gid % P);
  const int64_t D = a.D, N = a.N;
  const int64_t groups = (a.batch + G - 1) / G;
  const bool valid = idx < groups * D;
  const int64_t d = valid ? idx % D : 0;
  const int64_t b0 = valid ? (idx / D) * G : 0;
  const In* xp = static_cast<const In*>(a.x);
  const In* dp = static_cast<const In*>(a.delta);
  const In* zp = static_cast<const In*>(a.z);
  const In* Bp = static_cast<const In*>(a.Bm);
  const In* Cp = static_cast<const In*>(a.Cm);
  const int64_t n0 = (int64_t)q * SPL;
  using Piece = typename std::conditional<(SPL * sizeof(In)) % 16 == 0, u32x4, uint2>::type;
  constexpr int PER = (int)(sizeof(Piece) / sizeof(In));  // B/C elements per load
  constexpr int NP = VEC ? SPL / PER : 1;

  // the channel's row of A, scaled to base 2
  float A2[SPL];
  const float* arow = a.A + d * N + n0;
  if constexpr (VEC) {
#pragma unroll
    for (int j = 0; j < SPL; j += 4) {
      const float4 aa = *reinterpret_cast<const float4*>(arow + j);
      A2[j] = aa.x * kLog2e; A2[j + 1] = aa.y * kLog2e; A2[j + 2] = aa.z * kLog2e; A2[j + 3] = aa.w * kLog2e;
    }
  } else {
#pragma unroll
    for (int j = 0; j < SPL; ++j) A2[j] = (valid && n0 + j < N) ? arow[j] * kLog2e : 0.0f;
  }
  const float dsk = (a.Dskip && valid) ? a.Dskip[d] : 0.0f;
  const float dbias = (EXT && a.dbias && valid) ? a.dbias[d] : 0.0f;

  // With as many rows as lanes per channel (P = G = 4), lane q loads row
  // b0 + q's x, delta (and z) and the quad shares them by DPP broadcasts: one
  // 2-byte load per tensor instead of four, which matters when the step's
  // inputs come cold from HBM.
  constexpr bool QS = P == 4 && G == 4;
  float xq = 0.0f, dq = 0.0f, zq = 0.0f;
  if constexpr (QS) {
    const int64_t bq = b0 + q;
    const int64_t chq = (valid && bq < a.batch) ? bq * D + d : 0;
    dq = to_f32(dp[chq]);
    xq = to_f32(xp[chq]);
    if constexpr (GATE) zq = to_f32(zp[chq]);
  }

  // loads of all G rows
  bool vb[G];
  float hv[G][SPL], dt[G], xt[G];
  Piece bp[G][NP], cp[G][NP];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int64_t b = b0 + g;
    vb[g] = valid && b < a.batch;
    const int64_t ch = vb[g] ? b * D + d : 0;  // invalid rows read row 0 and store nothing
    const int64_t bb = vb[g] ? b : 0;
    if constexpr (QS) {
      dt[g] = quad_bcast(dq, g);
      xt[g] = quad_bcast(xq, g);
    } else {
      dt[g] = to_f32(dp[ch]);
      xt[g] = to_f32(xp[ch]);
    }
    const float* hrow = a.h + ch * N + n0;
    if constexpr (VEC) {
#pragma unroll
      for (int j = 0; j < SPL; j += 4) {
        const float4 hh = *reinterpret_cast<const float4*>(hrow + j);
        hv[g][j] = hh.x; hv[g][j + 1] = hh.y; hv[g][j + 2] = hh.z; hv[g][j + 3] = hh.w;
      }
#pragma unroll
      for (int k = 0; k < NP; ++k) {
        bp[g][k] = *reinterpret_cast<const Piece*>(Bp + bb * N + n0 + k * PER);
        cp[g][k] = *reinterpret_cast<const Piece*>(Cp + bb * N + n0 + k * PER);
      }
    } else {
#pragma unroll
      for (int j = 0; j < SPL; ++j) hv[g][j] = (vb[g] && n0 + j < N) ? hrow[j] : 0.0f;
    }
  }

#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int64_t b = b0 + g;
    const int64_t ch = vb[g] ? b * D + d : 0;
    const int64_t bb = vb[g] ? b : 0;
    float Bv[SPL], Cv[SPL];
    if constexpr (VEC) {
#pragma unroll
      for (int k = 0; k < NP; ++k) {
        const In* be = reinterpret_cast<const In*>(&bp[g][k]);
        const In* ce = reinterpret_cast<const In*>(&cp[g][k]);
#pragma unroll
        for (int m = 0; m < PER; ++m) {
          Bv[k * PER + m] = to_f32(be[m]);
          Cv[k * PER + m] = to_f32(ce[m]);
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < SPL; ++j) {
        const bool sv = vb[g] && n0 + j < N;
        Bv[j] = sv ? to_f32(Bp[bb * N + n0 + j]) : 0.0f;
        Cv[j] = sv ? to_f32(Cp[bb * N + n0 + j]) : 0.0f;
      }
    }
    // convolution front: the filter over the kept inputs and this token's,
    // then SiLU; the first lane of the channel shifts the kept inputs (every
    // lane's loads of them complete before, as the filter consumes them)
    if (EXT && a.conv_w) {
      const int K = a.conv_k;
      const float* cw = a.conv_w + d * K;
      float* cs = a.conv_state + ch * (K - 1);
      float keep[kMaxConv];
      float acc = (a.conv_b && valid) ? a.conv_b[d] : 0.0f;
      for (int k = 0; k < K - 1; ++k) {
        keep[k] = cs[k];
        acc = __builtin_fmaf(cw[k], keep[k], acc);
      }
      acc = __builtin_fmaf(cw[K - 1], xt[g], acc);
      if (vb[g] && q == 0 && K > 1) {
        for (int k = 0; k + 1 < K - 1; ++k) cs[k] = keep[k + 1];
        cs[K - 2] = xt[g];
      }
      xt[g] = silu(acc);
    }
    // the step: delta, plus the channel's bias, through softplus if asked
    float dl = dt[g];
    if (EXT && a.dbias) dl += dbias;
    if (EXT && a.softplus) dl = softplus_f(dl);
    float yp = 0.0f;
    if (EXT && a.zoh) {
#pragma unroll
      for (int j = 0; j < SPL; ++j) {
        const float arg = dl * A2[j];
        const float e = fast_exp2(arg);
        hv[g][j] = __builtin_fmaf(e, hv[g][j], (zoh_coef(dl, arg, e) * xt[g]) * Bv[j]);
        yp = __builtin_fmaf(Cv[j], hv[g][j], yp);
      }
    } else {
      const float u = dl * xt[g];
#pragma unroll
      for (int j = 0; j < SPL; ++j) {
        const float e = fast_exp2(dl * A2[j]);
        hv[g][j] = __builtin_fmaf(e, hv[g][j], u * Bv[j]);
        yp = __builtin_fmaf(Cv[j], hv[g][j], yp);
      }
    }
    float* hrow = a.h + ch * N + n0;
    if (vb[g]) {
      if constexpr (VEC) {
#pragma unroll
        for (int j = 0; j < SPL; j += 4)
          *reinterpret_cast<float4*>(hrow + j) = make_float4(hv[g][j], hv[g][j + 1], hv[g][j + 2], hv[g][j + 3]);
      } else {
#pragma unroll
        for (int j = 0; j < SPL; ++j)
          if (n0 + j < N) hrow[j] = hv[g][j];
      }
    }
    // the P partial outputs of a channel sit in P consecutive lanes (P <= 4):
    // add them with DPP quad permutations (lane ^ 1, then lane ^ 2)
    if constexpr (P >= 2)
      yp += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, yp), 0xB1, 0xf, 0xf, false));
    if constexpr (P >= 4)
      yp += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, yp), 0x4E, 0xf, 0xf, false));
    const float zg = (GATE && QS) ? quad_bcast(zq, g) : 0.0f;
    if (vb[g] && q == 0) {
      float yv = __builtin_fmaf(dsk, xt[g], yp);
      if constexpr (GATE) yv *= silu(QS ? zg : to_f32(zp[ch]));
      a.y[ch] = yv;
    }
  }
}

template <typename In, bool GATE, int P, int SPL, int G, bool EXT>
int launch_step_t(const StepArgs& a, bool vec, hipStream_t st) {
  const int64_t threads = ((a.batch + G - 1) / G) * a.D * P;
  const int64_t blocks = (threads + 255) / 256;
  if constexpr ((SPL * sizeof(In)) % 8 == 0) {
    if (vec) {
      hipLaunchKernelGGL((s6_step_kernel<In, GATE, P, SPL, true, G, EXT>), dim3((unsigned)blocks), dim3(256), 0, st, a);
      S6_HIP(hipGetLastError(), "s6_step_kernel launch");
      return S6_OK;
    }
  }
  hipLaunchKernelGGL((s6_step_kernel<In, GATE, P, SPL, false, G, EXT>), dim3((unsigned)blocks), dim3(256), 0, st, a);
  S6_HIP(hipGetLastError(), "s6_step_kernel launch");
  return S6_OK;
}

// Four batch rows per lane when that still leaves many lanes, else one.
// Kernels with the step options only when an option is set.
template <typename In, bool GATE, int P, int SPL, int G>
int launch_step_e(const StepArgs& a, bool vec, hipStream_t st) {
  if (a.dbias || a.softplus || a.zoh || a.conv_w) return launch_step_t<In, GATE, P, SPL, G, true>(a, vec, st);
  return launch_step_t<In, GATE, P, SPL, G, false>(a, vec, st);
}

template <typename In, bool GATE, int P, int SPL>
int launch_step_b(const StepArgs& a, bool vec, hipStream_t st) {
  if (a.batch >= 4 && a.batch * a.D * P >= 4 * 65536) return launch_step_e<In, GATE, P, SPL, 4>(a, vec, st);
  return launch_step_e<In, GATE, P, SPL, 1>(a, vec, st);
}

// Lanes per channel: 4 states per lane (P = 1, 2, 4 for dstate <= 4, 8,
// 16), so the lanes of a wave read h and A in one contiguous run; 8 states
// per lane over 4 lanes for 17..32.
template <typename In, bool GATE>
int launch_step_g(const StepArgs& a, hipStream_t st) {
  const int64_t N = a.N;
  const size_t esz = sizeof(In);
  auto vec_ok = [&](int64_t P, int64_t SPL) {
    const int64_t piece = (SPL * (int64_t)esz) % 16 == 0 ? 16 : 8;  // bytes of a B/C load
    return N == P * SPL && aligned(a.h, 16) && aligned(a.A, 16) && aligned(a.Bm, piece) &&
           aligned(a.Cm, piece) && (N * (int64_t)esz) % piece == 0 && (SPL * (int64_t)esz) % 8 == 0;
  };
  if (N <= 4) return launch_step_b<In, GATE, 1, 4>(a, vec_ok(1, 4), st);
  if (N <= 8) return launch_step_b<In, GATE, 2, 4>(a, vec_ok(2, 4), st);
  if (N <= 16) return launch_step_b<In, GATE, 4, 4>(a, vec_ok(4, 4), st);
  return launch_step_b<In, GATE, 4, 8>(a, vec_ok(4, 8), st);
}

}  // namespace

}  // namespace s6i

using namespace s6i;

namespace {

int state_update_impl(int64_t batch, int64_t dim, int64_t dstate, int in_dtype, float* h,
                      const void* x, const void* delta, const float* delta_bias, int flags,
                      const float* A, const void* Bm, const void* Cm, const float* Dskip,
                      const void* z, float* y, void* stream, const float* conv_w = nullptr,
                      const float* conv_b = nullptr, float* conv_state = nullptr, int conv_k = 0) {
  int rc = check_common(batch, dim, 1, dstate, in_dtype);
  if (rc) return rc;
  if (flags & ~(S6_DELTA_SOFTPLUS | S6_ZOH_EXACT)) return S6_ERR_FLAGS;
  if (conv_w || conv_k) {
    if (conv_k < 1 || conv_k > kMaxConv) return S6_ERR_UNSUPPORTED;
    if (!conv_w || (conv_k > 1 && !conv_state)) return S6_ERR_NULL;
    const void* cps[] = {conv_w, conv_b, conv_state};
    for (const void* p : cps)
      if (p && !aligned(p, 4)) return S6_ERR_ALIGN;
  }
  // one thread per (batch, channel, 4 states) at most: the grid must fit
  if (batch * dim > (int64_t)INT32_MAX * 256 / 8) return S6_ERR_SHAPE;
  if (batch == 0 || dim == 0) return S6_OK;
  if (!h || !x || !delta || !A || !Bm || !Cm || !y) return S6_ERR_NULL;
  const size_t esz = in_dtype == S6_BF16 ? 2 : 4;
  const void* ins[] = {x, delta, Bm, Cm, z};
  for (const void* p : ins)
    if (p && !aligned(p, esz)) return S6_ERR_ALIGN;
  const void* f32s[] = {h, A, Dskip, y, delta_bias};
  for (const void* p : f32s)
    if (p && !aligned(p, 4)) return S6_ERR_ALIGN;
  StepArgs a;
  a.h = h; a.x = x; a.delta = delta; a.z = z; a.A = A; a.Bm = Bm; a.Cm = Cm; a.Dskip = Dskip; a.y = y;
  a.dbias = delta_bias;
  a.softplus = (flags & S6_DELTA_SOFTPLUS) != 0;
  a.zoh = (flags & S6_ZOH_EXACT) != 0;
  a.conv_w = conv_w; a.conv_b = conv_b; a.conv_state = conv_state; a.conv_k = conv_k;
  a.batch = batch; a.D = dim; a.N = dstate;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (in_dtype == S6_BF16)
    return z ? launch_step_g<uint16_t, true>(a, st) : launch_step_g<uint16_t, false>(a, st);
  return z ? launch_step_g<float, true>(a, st) : launch_step_g<float, false>(a, st);
}

}  // namespace

extern "C" {

int s6_state_update_ex(int64_t batch, int64_t dim, int64_t dstate, int in_dtype, float* h,
                       const void* x, const void* delta, const float* delta_bias, int flags,
                       const float* A, const void* Bm, const void* Cm, const float* Dskip,
                       const void* z, float* y, void* stream) {
  return state_update_impl(batch, dim, dstate, in_dtype, h, x, delta, delta_bias, flags, A, Bm, Cm, Dskip,
                           z, y, stream);
}

int s6_conv_state_update(int64_t batch, int64_t dim, int64_t dstate, int in_dtype, float* h,
                         float* conv_state, const void* x, const float* conv_w, const float* conv_bias,
                         int conv_width, const void* delta, const float* delta_bias, int flags,
                         const float* A, const void* Bm, const void* Cm, const float* Dskip,
                         const void* z, float* y, void* stream) {
  if (!conv_w && conv_width == 0) return S6_ERR_NULL;
  return state_update_impl(batch, dim, dstate, in_dtype, h, x, delta, delta_bias, flags, A, Bm, Cm, Dskip,
                           z, y, stream, conv_w, conv_bias, conv_state, conv_width);
}

int s6_state_update(int64_t batch, int64_t dim, int64_t dstate, int in_dtype, float* h,
                    const void* x, const void* delta, const float* A, const void* Bm,
                    const void* Cm, const float* Dskip, const void* z, float* y, void* stream) {
  return s6_state_update_ex(batch, dim, dstate, in_dtype, h, x, delta, nullptr, 0, A, Bm, Cm, Dskip, z,
                            y, stream);
}

}  // extern "C"
