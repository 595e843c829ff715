// bwd.hip -- gradients of the scan (s6_scan_bwd and its _ex form) with the
// states recomputed.
#include "s6_internal.h"

namespace s6i {

namespace {

// Reverse-mode gradients of the scan for the loss <dy, y> + <dh_last, h_last>
// (plain step).  The states are recomputed, never stored per token.  A first
// pass gives the state entering every segment of kBwdSeg tokens (one
// sequential state-only scan when its workgroups fill the GPU, else the
// segments scanned side by side from zero and folded, the kernels of a
// segmented forward scan) or, from the sequential scan for the exact hold and
// the convolution front, the state entering every 16-token chunk; this kernel then walks
// the segments of a (batch row, 16-channel block) from the last to the first.
// Per segment it stages the inputs in LDS, loads or recomputes the states at
// the four chunk starts, and per 16-token chunk (last first) recomputes the
// chunk's states and transitions in registers and runs the adjoint
// lambda_t = dyc_t C_t + a_{t+1} lambda_{t+1} backwards through it.
//
// Lane l of wave w: channel c = 4w + (l >> 4) of the block, states
// (l & 15) * SPL + j.  Sums over states (for dx, ddelta and the pre-gate
// output) are taken across the 16 lanes of a row with a DPP butterfly that
// leaves token l's sums in lane l; sums
// over channels (dB, dC) across the 4 rows of a wave with permlane swaps,
// across the 4 waves in LDS, and across channel blocks by a second kernel
// from per-block partials (a fixed order: results are bitwise repeatable).
constexpr int kBwdSeg = 64;    // tokens per recomputation segment
// Pitch (floats) of the staged [row][token] tiles.  With a pitch of 64 the
// 16 states of a channel (float4 reads of B and C, one row each) and the 4
// channels of a wave would all fall on the same LDS banks; 4 more floats put
// consecutive rows 4 banks apart, so 16 lanes' 16-byte reads cover all 64.
constexpr int kBwdPitch = kBwdSeg + 4;

// Waves per workgroup (4 channels each).  With one state per lane the
// kernels take 103-128 VGPRs (four waves per SIMD), with two (N > 16) about
// 180 (two waves per SIMD).  Several 4-wave workgroups per CU, whose barriers
// fall at different times, run faster than fewer 8-wave ones.
#ifndef S6_BWD_WAVES
#define S6_BWD_WAVES 4
#endif
template <int SPL>
constexpr int bwd_waves() { return S6_BWD_WAVES; }

template <int SPL>
constexpr size_t bwd_lds_bytes(bool sp) {
  // tiles x, delta, dyc, dy SiLU'(z), then delta * x (plain) or dstep/dv (SP)
  return sizeof(float) * ((size_t)5 * (4 * bwd_waves<SPL>()) * kBwdPitch + (size_t)2 * 16 * SPL * kBwdPitch +
                          (size_t)bwd_waves<SPL>() * 2 * 16 * 16 * SPL);
}

// Step of a stored delta value under the step options (SP kernels): v =
// delta + bias, then softplus(v) if asked; *js receives dstep/dv.
__device__ __forceinline__ float bwd_step(float raw, float bias, bool softplus, float* js) {
  const float v = raw + bias;
  if (!softplus) {
    *js = 1.0f;
    return v;
  }
  *js = fast_rcp(1.0f + fast_exp2(-v * kLog2e));
  return softplus_f(v);
}

// Input factor of one state's input term under the exact hold: c x with the
// hold's coefficient c (zoh_coef) from the transition e = 2^arg the caller
// computed; x is the token's input.
__device__ __forceinline__ float zoh_input(float dl, float x, float arg, float e) { return zoh_coef(dl, arg, e) * x; }

// dc/dA of the hold's coefficient c = (e^u - 1) / A, u = dl A (e = e^u):
// (u e^u - (e^u - 1)) / A^2 = dl^2 q(u) with q(u) = sum_{k>=0} (k+1) u^k /
// (k+2)!.  The difference cancels for small |u|, so below |u| = 1/2 the
// series is summed (8 terms: the next is below 1e-8 relative); q(0) = 1/2.
__device__ __forceinline__ float zoh_dcoef_da(float dl, float u, float e) {
  float qs = 1.0f / 45360;
  qs = __builtin_fmaf(qs, u, 1.0f / 5760);
  qs = __builtin_fmaf(qs, u, 1.0f / 840);
  qs = __builtin_fmaf(qs, u, 1.0f / 144);
  qs = __builtin_fmaf(qs, u, 1.0f / 30);
  qs = __builtin_fmaf(qs, u, 1.0f / 8);
  qs = __builtin_fmaf(qs, u, 1.0f / 3);
  qs = __builtin_fmaf(qs, u, 0.5f);
  const float qd = __builtin_fmaf(u, e, 1.0f - e) * fast_rcp(u * u);
  return dl * dl * (fabsf(u) < 0.5f ? qs : qd);
}

struct BwdArgs {
  const void* x;
  const void* delta;
  const void* z;          // null: no gate
  const void* Bm;
  const void* Cm;
  const float* A;
  const float* Dskip;     // nullable
  const float* dy;        // (batch, D, L)
  const float* dh_last;   // nullable
  const float* hin;       // (S, batch*D*N): state entering each segment
  float* dx;              // (batch, D, L)
  float* ddelta;          // (batch, D, L)
  float* dz;              // (batch, D, L), gate only
  float* dA_part;         // (G, batch, D, N): sums over the tokens of one batch row and part
  float* dD_part;         // (G, batch, D)
  float* dB_part;         // (nblk, batch, N, L)
  float* dC_part;         // (nblk, batch, N, L)
  float* dh0;             // nullable (batch, D, N)
  const float* mu_in;     // (G, batch*D*N): adjoint carry entering each part from the right, or
                          // null (one part: the carry is dh_last)
  float* carry_M;         // (G, batch*D*N): carry leaving each part from a zero carry-in
  float* carry_SD;        // (G, batch*D): summed delta of each part
  const float* dbias;     // SP kernels: (D) step bias or null
  int softplus;           // SP kernels: step = softplus(delta + dbias)
  int zoh;                // exact zero-order-hold input coefficient (OPT 2 kernels)
  const float* conv_w;    // SP kernels: the convolution front (as in ScanArgs), or null
  const float* conv_b;
  const float* conv_state;
  int conv_k;
  float* ddbias_part;     // SP kernels: (G, batch, D) gradient of the bias, or null
  int64_t batch, D, L, N, nseg;
  int64_t seg_per_part;   // segments per part (the sequence is cut into G parts, blockIdx.y)
};

// Sums over the 16 lanes of a row of 16 per-token values, leaving token l's
// sum in lane l of the row: a butterfly over the lane partners l^8 (row
// rotation by 8), l^7 (half-row mirror), l^2 and l^1 (quad permutations).  At
// each step a lane keeps the half of its values whose token index has the
// lane's bit (8, 4, 2, 1), and adds its partner's copy of that half; the
// partner shares the bits already used, so both hold the same tokens.
//
// Lane bits 3 and 2 are bank bits (a bank is 4 lanes of a row), so the first
// two steps need no selects: out[j] = hi[j] + partner's hi[j] is written in
// every lane, then lo[j] + partner's lo[j] over it in the banks whose bit is
// 0 (a DPP add with a bank mask leaves the other banks' value in place).
// The sums are the same additions as with selects, bit for bit.
#define S6_BANKED_PAIR_SUMS4(CTRL, BANKS)                                                        \
  asm("s_nop 1\n\t"                                                                            \
      "v_add_f32_dpp %0, %4, %4 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                       \
      "v_add_f32_dpp %1, %5, %5 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                       \
      "v_add_f32_dpp %2, %6, %6 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                       \
      "v_add_f32_dpp %3, %7, %7 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                       \
      "v_add_f32_dpp %0, %8, %8 " CTRL " row_mask:0xf bank_mask:" BANKS "\n\t"                 \
      "v_add_f32_dpp %1, %9, %9 " CTRL " row_mask:0xf bank_mask:" BANKS "\n\t"                 \
      "v_add_f32_dpp %2, %10, %10 " CTRL " row_mask:0xf bank_mask:" BANKS "\n\t"               \
      "v_add_f32_dpp %3, %11, %11 " CTRL " row_mask:0xf bank_mask:" BANKS                        \
      : "=&v"(out[0]), "=&v"(out[1]), "=&v"(out[2]), "=&v"(out[3])                              \
      : "v"(hi[0]), "v"(hi[1]), "v"(hi[2]), "v"(hi[3]), "v"(lo[0]), "v"(lo[1]), "v"(lo[2]), "v"(lo[3]))
// partner l^8 (row rotation by 8); bit 3 is clear in banks 0 and 1
__device__ __forceinline__ void pair_sums4_l8(const float* lo, const float* hi, float* out) {
  S6_BANKED_PAIR_SUMS4("row_ror:8", "0x3");
}
// partner l^7 (half-row mirror); bit 2 is clear in banks 0 and 2
__device__ __forceinline__ void pair_sums4_l7(const float* lo, const float* hi, float* out) {
  S6_BANKED_PAIR_SUMS4("row_half_mirror", "0x5");
}
#undef S6_BANKED_PAIR_SUMS4
__device__ __forceinline__ float row_reduce_scatter16(const float (&v)[16], int nl) {
  const bool b1 = nl & 2, b0 = nl & 1;
  float a8[8], a4[4], a2[2];
  pair_sums4_l8(v, v + 8, a8);
  pair_sums4_l8(v + 4, v + 12, a8 + 4);
  pair_sums4_l7(a8, a8 + 4, a4);
#pragma unroll
  for (int j = 0; j < 2; ++j) a2[j] = (b1 ? a4[j + 2] : a4[j]) + dpp_f<0x4E>(b1 ? a4[j] : a4[j + 2]);
  return (b0 ? a2[1] : a2[0]) + dpp_f<0xB1>(b0 ? a2[0] : a2[1]);
}

// Sums over the 4 rows (channels) of a wave for 4 tokens at once: v[k] is
// this lane's value of token k; the result in row r is the 4-row sum of
// token row_tok(r) = 0, 2, 1, 3 (v_permlane32_swap pairs rows 0,1 with 2,3
// for two tokens, v_permlane16_swap then rows 0 with 1 and 2 with 3).
__device__ __forceinline__ int row_tok(int r) { return ((r & 1) << 1) | (r >> 1); }
__device__ __forceinline__ float rows_sum4(const float (&v)[4]) {
  const auto p = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, v[0]),
                                                  __builtin_bit_cast(unsigned, v[1]), false, false);
  const auto q = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, v[2]),
                                                  __builtin_bit_cast(unsigned, v[3]), false, false);
  const float w01 = __builtin_bit_cast(float, (unsigned)p[0]) + __builtin_bit_cast(float, (unsigned)p[1]);
  const float w23 = __builtin_bit_cast(float, (unsigned)q[0]) + __builtin_bit_cast(float, (unsigned)q[1]);
  const auto s = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, w01),
                                                  __builtin_bit_cast(unsigned, w23), false, false);
  return __builtin_bit_cast(float, (unsigned)s[0]) + __builtin_bit_cast(float, (unsigned)s[1]);
}

// SP: the step bias / softplus options (the gradient of the stored delta
// gets the factor dstep/dv; the bias gradient is summed per channel).
// OPT: 0 plain; 1 step bias / softplus; 3 those and the convolution front;
// 2 bias / softplus and the exact hold, whose
// input coefficient c = (e^{delta A} - 1) / A replaces delta in the input
// term: dx and dB take c, the input part of ddelta takes dc/ddelta = e^{delta
// A}, and dA gains lambda B x dc/dA.
// The exact-hold and convolution levels would take about 140 VGPRs (three
// waves per SIMD); held to 128 they spill a dozen values to scratch and run
// 4-6% faster with the fourth wave.
//
// H16 (exact-hold and convolution levels): a.hin holds the state entering
// every 16-token chunk (from a state-only pass that wrote one per chunk), so
// the four chunk-start states of a segment are loaded instead of recomputed
// from the segment's first state.
template <typename In, bool GATE, int SPL, int OPT, bool H16>
__global__ void __launch_bounds__(64 * bwd_waves<SPL>())
    __attribute__((amdgpu_waves_per_eu((OPT >= 2 && SPL == 1) ? 4 : 1))) s6_bwd_kernel(BwdArgs a) {
  static_assert(!H16 || OPT >= 2, "per-chunk states: exact-hold and convolution levels only");
  constexpr bool SP = OPT >= 1;
  constexpr bool ZOH = OPT == 2;
  constexpr bool CONV = OPT == 3;  // the convolution front (its own kernels: it costs registers)
  constexpr int WB = bwd_waves<SPL>();
  constexpr int NTHR = 64 * WB;
  constexpr int CW = 4 * WB;         // channels per workgroup
  constexpr int NS = 16 * SPL;       // state slots per channel
  constexpr int KS = kBwdSeg;
  constexpr int KP = kBwdPitch;  // LDS row pitch: rows 4 banks apart
  extern __shared__ float4 lds4[];
  float* lds = reinterpret_cast<float*>(lds4);
  float* sx = lds;                   // [CW][KS] x
  float* sdl = sx + CW * KP;         // [CW][KP] delta
  float* sdyc = sdl + CW * KP;       // [CW][KP] dy * SiLU(z)
  float* sq = sdyc + CW * KP;        // [CW][KP] dy * SiLU'(z)
  float* su = sq + CW * KP;          // [CW][KP] plain: delta * x; SP: dstep/dv
  float* sB = su + CW * KP;          // [NS][KP]
  float* sC = sB + NS * KP;          // [NS][KP]
  float* red = sC + NS * KP;         // [waves][2][16][NS]
  float* sjs = su;                   // SP: the fifth tile holds dstep/dv (delta * x is formed on use)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int row = lane >> 4;
  const int nl = lane & 15;
  const int c = 4 * w + row;
  const int64_t D = a.D, L = a.L, N = a.N;
  const int64_t nblk = (D + CW - 1) / CW;
  // Without parts, each of the 8 XCDs (workgroups are dispatched to them in
  // turn, each has its own L2) takes a contiguous run of (row, block), so
  // the workgroups that stage the same B and C share one L2.
  uint32_t wgx = blockIdx.x;
  if (gridDim.y == 1) {
    const uint32_t nx = gridDim.x, q = nx / 8, rem = nx % 8, xcd = wgx % 8;
    wgx = xcd * q + (xcd < rem ? xcd : rem) + wgx / 8;
  }
  const int64_t blk = wgx % nblk;
  const int64_t b = wgx / nblk;
  const int64_t d0 = blk * CW;
  const int64_t rows_valid = D - d0 < CW ? D - d0 : CW;
  const int64_t d = d0 + c;
  const bool chv = c < rows_valid;
  const In* xp = static_cast<const In*>(a.x);
  const In* dp = static_cast<const In*>(a.delta);
  const In* zp = static_cast<const In*>(a.z);
  const In* Bp = static_cast<const In*>(a.Bm);
  const In* Cp = static_cast<const In*>(a.Cm);
  const float dsk = (a.Dskip && chv) ? a.Dskip[d] : 0.0f;

  // this workgroup's part of the sequence: segments [s_begin, s_end)
  const int64_t part = blockIdx.y;
  const int64_t nstate = a.batch * D * N;
  const int64_t s_begin = part * a.seg_per_part;
  const int64_t s_end = s_begin + a.seg_per_part < a.nseg ? s_begin + a.seg_per_part : a.nseg;

  float A2[SPL], An[SPL], mu[SPL], dA[SPL];
  bool sv[SPL];
#pragma unroll
  for (int j = 0; j < SPL; ++j) {
    const int64_t n = (int64_t)nl * SPL + j;
    sv[j] = chv && n < N;
    An[j] = sv[j] ? a.A[d * N + n] : 0.0f;
    A2[j] = An[j] * kLog2e;
    // a_{t+1} lambda_{t+1} entering the part's last token
    mu[j] = !sv[j] ? 0.0f
            : a.mu_in ? a.mu_in[part * nstate + (b * D + d) * N + n]
            : a.dh_last ? a.dh_last[(b * D + d) * N + n] : 0.0f;
    dA[j] = 0.0f;
  }
  float dD = 0.0f, dbias = 0.0f;

  // delta * x of 4 tokens of this lane's channel from LDS (formed from delta
  // and x in SP kernels, whose fifth tile holds dstep/dv instead; x itself
  // in the exact-hold kernels)
  auto load_u4 = [&](int t, const float4& dl4) {
    if constexpr (ZOH) {
      return *reinterpret_cast<const float4*>(sx + c * KP + t);  // x: the coefficient is per state
    } else if constexpr (SP) {
      const float4 x4 = *reinterpret_cast<const float4*>(sx + c * KP + t);
      return make_float4(dl4.x * x4.x, dl4.y * x4.y, dl4.z * x4.z, dl4.w * x4.w);
    } else {
      return *reinterpret_cast<const float4*>(su + c * KP + t);
    }
  };

  for (int64_t s = s_end - 1; s >= s_begin; --s) {
    const int64_t tb = s * KS;
    const int64_t tl = L - tb < KS ? L - tb : KS;  // valid tokens of the segment
    // the state entering the segment: loaded before the staging, so that its
    // latency is not exposed after the barrier, where registers allow (the
    // kernels held to 128 VGPRs load it after the staging)
    float hseg[SPL];
    auto load_hseg = [&]() {
#pragma unroll
      for (int j = 0; j < SPL; ++j) {
        const int64_t n = (int64_t)nl * SPL + j;
        hseg[j] = sv[j] ? a.hin[s * a.batch * D * N + (b * D + d) * N + n] : 0.0f;
      }
    };
    // states at the four chunk starts of the segment (chunks past the end of
    // the sequence: 0, their tokens are staged as delta = 0 and change nothing)
    float hc[4][SPL];
    auto load_hc16 = [&]() {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int64_t q = s * (KS / 16) + k;
#pragma unroll
        for (int j = 0; j < SPL; ++j) {
          const int64_t n = (int64_t)nl * SPL + j;
          hc[k][j] = (sv[j] && q * 16 < L) ? a.hin[q * nstate + (b * D + d) * N + n] : 0.0f;
        }
      }
    };
    // (the kernels held to 128 VGPRs load them after the staging)
    if constexpr (OPT < 2) load_hseg();
    __syncthreads();  // the previous segment's reads of the staged inputs are done
    for (int i = tid; i < CW * KS; i += NTHR) {
      const int cc = i / KS, t = i % KS;
      const bool ok = cc < rows_valid && t < tl;
      const int64_t off = (b * D + d0 + (cc < rows_valid ? cc : 0)) * L + tb + (t < tl ? t : 0);
      float xv = 0.0f, dl = 0.0f, dyc = 0.0f, q = 0.0f, js = 0.0f;
      if (ok) {
        xv = to_f32(xp[off]);
        dl = to_f32(dp[off]);
        if constexpr (SP) dl = bwd_step(dl, a.dbias ? a.dbias[d0 + cc] : 0.0f, a.softplus, &js);
        const float g = a.dy[off];
        if constexpr (GATE) {
          const float zz = to_f32(zp[off]);
          const float sg = fast_rcp(1.0f + fast_exp2(-zz * kLog2e));
          dyc = g * (zz * sg);
          q = g * (sg * (1.0f + zz * (1.0f - sg)));
        } else {
          dyc = g;
        }
      }
      const int li = cc * KP + t;
      sx[li] = xv;
      sdl[li] = dl;
      sdyc[li] = dyc;
      sq[li] = q;
      if constexpr (SP) sjs[li] = js;
      else su[li] = dl * xv;
    }
    for (int i = tid; i < NS * KS; i += NTHR) {
      const int n = i / KS, t = i % KS;
      const bool ok = n < N && t < tl;
      const int64_t off = (b * N + (n < N ? n : 0)) * L + tb + (t < tl ? t : 0);
      sB[n * KP + t] = ok ? to_f32(Bp[off]) : 0.0f;
      sC[n * KP + t] = ok ? to_f32(Cp[off]) : 0.0f;
    }
    if constexpr (CONV) {
      // the raw inputs of the kMaxConv - 1 tokens before the segment (from
      // the previous segment, or the front's state before token 0) go to the
      // row's padding slots KS .. KS + kMaxConv - 2, loaded with the rest
      static_assert(KP - KS >= kMaxConv - 1, "halo fits the row padding");
      if (tid < CW * (kMaxConv - 1)) {
        const int hc = tid / (kMaxConv - 1), hj = tid % (kMaxConv - 1);
        const int64_t sg = tb - (kMaxConv - 1) + hj;
        const int K = a.conv_k;
        float v = 0.0f;
        if (hc < rows_valid) {
          const int64_t rw = b * D + d0 + hc;
          if (sg >= 0) v = to_f32(xp[rw * L + sg]);
          else if (sg >= -(int64_t)(K - 1) && a.conv_state) v = a.conv_state[rw * (K - 1) + (K - 1) + sg];
        }
        sx[hc * KP + KS + hj] = v;
      }
    }
    __syncthreads();
    if constexpr (CONV) {
      // The convolution front's output x' replaces the staged x, as the
      // forward computes it: 4 consecutive tokens of one channel per thread
      // from the 3 + 4 raw inputs around them (the 3 before the segment from
      // the row's padding slots), read before any thread overwrites its tokens.
      static_assert(CW * KS == 4 * NTHR, "one group of 4 tokens per thread");
      const int fcc = tid / (KS / 4), ft4 = (tid % (KS / 4)) * 4;
      const int K = a.conv_k;
      float xin[4 + kMaxConv - 1];  // raw inputs at ft4 - (kMaxConv - 1) .. ft4 + 3
#pragma unroll
      for (int i = 0; i < 4 + kMaxConv - 1; ++i) {
        const int t = ft4 - (kMaxConv - 1) + i;
        xin[i] = sx[fcc * KP + (t >= 0 ? t : KS + (kMaxConv - 1) + t)];
      }
      __syncthreads();  // every raw input is read
      float xo[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      if (fcc < rows_valid) {
        const int64_t ch = d0 + fcc;
        float wk[kMaxConv];
#pragma unroll
        for (int k = 0; k < kMaxConv; ++k) wk[k] = k < K ? a.conv_w[ch * K + k] : 0.0f;
        const float cbias = a.conv_b ? a.conv_b[ch] : 0.0f;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (ft4 + u < tl) {
            float acc = cbias;
#pragma unroll
            for (int j = 0; j < kMaxConv; ++j)
              if (j < K) acc = __builtin_fmaf(wk[K - 1 - j], xin[(kMaxConv - 1) + u - j], acc);
            xo[u] = silu(acc);
          }
        }
      }
      *reinterpret_cast<float4*>(sx + fcc * KP + ft4) = make_float4(xo[0], xo[1], xo[2], xo[3]);
      __syncthreads();
    }

    if constexpr (H16 && OPT >= 2) load_hc16();
    // states at the four chunk starts, recomputed from the segment's first
    if constexpr (!H16) {
      if constexpr (OPT >= 2) load_hseg();
      float h[SPL];
#pragma unroll
      for (int j = 0; j < SPL; ++j) h[j] = hseg[j];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
#pragma unroll
        for (int j = 0; j < SPL; ++j) hc[k][j] = h[j];
        if (k == 3) break;  // the state after the last chunk is not needed
        for (int g = 0; g < 4; ++g) {
          // one group of 4 tokens at a time: the compiler would otherwise
          // hoist every LDS read of the segment and run out of registers
          __builtin_amdgcn_sched_barrier(0);
          const int t = 16 * k + 4 * g;
          const float4 dl4 = *reinterpret_cast<const float4*>(sdl + c * KP + t);
          const float4 u4 = load_u4(t, dl4);
          const float dl[4] = {dl4.x, dl4.y, dl4.z, dl4.w};
          const float u[4] = {u4.x, u4.y, u4.z, u4.w};
#pragma unroll
          for (int j = 0; j < SPL; ++j) {
            const float4 b4 = *reinterpret_cast<const float4*>(sB + (nl * SPL + j) * KP + t);
            const float Bv[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float arg = dl[i] * A2[j];
              const float e = fast_exp2(arg);
              const float in = ZOH ? zoh_input(dl[i], u[i], arg, e) : u[i];
              h[j] = __builtin_fmaf(e, h[j], in * Bv[i]);
            }
          }
        }
      }
    }

    for (int k = 3; k >= 0; --k) {
      // the chunk's transitions ea and states: hist[j][i] = h before token i
      float ea[SPL][16], hist[SPL][17];
#pragma unroll
      for (int j = 0; j < SPL; ++j) hist[j][0] = hc[k][j];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        __builtin_amdgcn_sched_barrier(0);
        const int t = 16 * k + 4 * g;
        const float4 dl4 = *reinterpret_cast<const float4*>(sdl + c * KP + t);
        const float4 u4 = load_u4(t, dl4);
        const float dl[4] = {dl4.x, dl4.y, dl4.z, dl4.w};
        const float u[4] = {u4.x, u4.y, u4.z, u4.w};
#pragma unroll
        for (int j = 0; j < SPL; ++j) {
          const float4 b4 = *reinterpret_cast<const float4*>(sB + (nl * SPL + j) * KP + t);
          const float Bv[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float arg = dl[i] * A2[j];
            ea[j][4 * g + i] = fast_exp2(arg);
            const float in = ZOH ? zoh_input(dl[i], u[i], arg, ea[j][4 * g + i]) : u[i];
            hist[j][4 * g + i + 1] = __builtin_fmaf(ea[j][4 * g + i], hist[j][4 * g + i], in * Bv[i]);
          }
        }
      }
      // adjoint, last token first; lane nl keeps the row sums of token nl
      float s1[16], s2[16], s3[16];  // this lane's terms of the state sums, per token
#pragma unroll
      for (int g4 = 3; g4 >= 0; --g4) {
        __builtin_amdgcn_sched_barrier(0);
        const int t4 = 16 * k + 4 * g4;
        const float4 dl4 = *reinterpret_cast<const float4*>(sdl + c * KP + t4);
        const float4 u4 = load_u4(t4, dl4);
        const float4 y4 = *reinterpret_cast<const float4*>(sdyc + c * KP + t4);
        const float dlv[4] = {dl4.x, dl4.y, dl4.z, dl4.w};
        const float uv[4] = {u4.x, u4.y, u4.z, u4.w};
        const float dycv[4] = {y4.x, y4.y, y4.z, y4.w};
        float Bv[SPL][4], Cv[SPL][4];
#pragma unroll
        for (int j = 0; j < SPL; ++j) {
          const float4 b4 = *reinterpret_cast<const float4*>(sB + (nl * SPL + j) * KP + t4);
          const float4 c4 = *reinterpret_cast<const float4*>(sC + (nl * SPL + j) * KP + t4);
          Bv[j][0] = b4.x; Bv[j][1] = b4.y; Bv[j][2] = b4.z; Bv[j][3] = b4.w;
          Cv[j][0] = c4.x; Cv[j][1] = c4.y; Cv[j][2] = c4.z; Cv[j][3] = c4.w;
        }
        float pb[SPL][4], pc[SPL][4];
#pragma unroll
        for (int ii = 3; ii >= 0; --ii) {
          const int i = 4 * g4 + ii;
          const float dl = dlv[ii], uu = uv[ii], dyc = dycv[ii];
          s1[i] = 0.0f;
          s2[i] = 0.0f;
          s3[i] = 0.0f;
#pragma unroll
          for (int j = 0; j < SPL; ++j) {
            const float lam = __builtin_fmaf(dyc, Cv[j][ii], mu[j]);
            mu[j] = ea[j][i] * lam;
            const float r = lam * (ea[j][i] * hist[j][i]);
            s3[i] = __builtin_fmaf(Cv[j][ii], hist[j][i + 1], s3[i]);
            pc[j][ii] = dyc * hist[j][i + 1];
            if constexpr (ZOH) {
              // uu is x here: dx sums lambda c B, ddelta lambda (A a h + a B x),
              // dA lambda (delta a h + B x dc/dA), dB lambda c x
              const float arg = dl * A2[j];
              const float cf = zoh_coef(dl, arg, ea[j][i]);
              const float lb = lam * Bv[j][ii];
              s1[i] = __builtin_fmaf(lb, cf, s1[i]);
              s2[i] = __builtin_fmaf(An[j], r, s2[i]);
              s2[i] = __builtin_fmaf(lb * ea[j][i], uu, s2[i]);
              dA[j] = __builtin_fmaf(dl, r, dA[j]);
              dA[j] = __builtin_fmaf(lb * uu, zoh_dcoef_da(dl, arg * kLn2, ea[j][i]), dA[j]);
              pb[j][ii] = (lam * cf) * uu;
            } else {
              s1[i] = __builtin_fmaf(lam, Bv[j][ii], s1[i]);
              s2[i] = __builtin_fmaf(An[j], r, s2[i]);
              dA[j] = __builtin_fmaf(dl, r, dA[j]);
              pb[j][ii] = lam * uu;
            }
          }
        }
        // the running sums are updated here (left alone, the compiler defers
        // them to the end of the chunk and keeps all their operands live)
#pragma unroll
        for (int j = 0; j < SPL; ++j) asm volatile("" : "+v"(dA[j]), "+v"(mu[j]));
        // channel sums of the 4 tokens over the wave's rows, then to LDS
#pragma unroll
        for (int j = 0; j < SPL; ++j) {
          const int tok = 4 * g4 + row_tok(row);
          red[((w * 2 + 0) * 16 + tok) * NS + nl * SPL + j] = rows_sum4(pb[j]);
          red[((w * 2 + 1) * 16 + tok) * NS + nl * SPL + j] = rows_sum4(pc[j]);
        }
      }
      // sums over the row's states: lane nl gets those of token nl
      const float k1 = row_reduce_scatter16(s1, nl);
      const float k2 = row_reduce_scatter16(s2, nl);
      const float k3 = GATE ? row_reduce_scatter16(s3, nl) : 0.0f;
      // outputs of token nl of the chunk for this lane's channel
      {
        const int t = 16 * k + nl;
        const int64_t tt = tb + t;
        if (chv && tt < L) {
          const float dl = sdl[c * KP + t];
          const float xv = sx[c * KP + t];
          const float dyc = sdyc[c * KP + t];
          const int64_t off = (b * D + d) * L + tt;
          dD = __builtin_fmaf(dyc, xv, dD);  // lane nl: the tokens nl mod 16
          // (the exact hold's sums already carry the coefficient and x)
          a.dx[off] = __builtin_fmaf(dyc, dsk, ZOH ? k1 : dl * k1);
          float gd = ZOH ? k2 : __builtin_fmaf(xv, k1, k2);
          if constexpr (SP) {
            gd *= sjs[c * KP + t];
            dbias += gd;
          }
          a.ddelta[off] = gd;
          if (GATE && a.dz) a.dz[off] = __builtin_fmaf(dsk, xv, k3) * sq[c * KP + t];
        }
      }
      __syncthreads();  // every wave's channel sums of the chunk are in LDS
      for (int e = tid; e < 2 * 16 * NS; e += NTHR) {
        const int kind = e / (16 * NS);
        const int tok = (e / NS) % 16;
        const int n = e % NS;
        float sum = 0.0f;
#pragma unroll
        for (int ww = 0; ww < WB; ++ww) sum += red[((ww * 2 + kind) * 16 + tok) * NS + n];
        const int64_t tt = tb + 16 * k + tok;
        if (n < N && tt < L) {
          float* dst = kind ? a.dC_part : a.dB_part;
          dst[((blk * a.batch + b) * N + n) * L + tt] = sum;
        }
      }
      __syncthreads();  // red is free again
    }
  }
  // the channel's dD: lane nl summed the tokens it wrote
  dD += dpp_f<0x128>(dD);
  dD += dpp_f<0x124>(dD);
  dD += dpp_f<0x122>(dD);
  dD += dpp_f<0x121>(dD);
  if (chv) {
#pragma unroll
    for (int j = 0; j < SPL; ++j) {
      const int64_t n = (int64_t)nl * SPL + j;
      if (n < N) {
        a.dA_part[part * nstate + (b * D + d) * N + n] = dA[j];
        if (a.dh0 && part == 0) a.dh0[(b * D + d) * N + n] = mu[j];
      }
    }
    if (nl == 0) a.dD_part[part * a.batch * D + b * D + d] = dD;
  }
  if constexpr (SP) {
    // the channel's bias gradient: lane nl summed the tokens it wrote
    dbias += dpp_f<0x128>(dbias);
    dbias += dpp_f<0x124>(dbias);
    dbias += dpp_f<0x122>(dbias);
    dbias += dpp_f<0x121>(dbias);
    if (chv && nl == 0 && a.ddbias_part) a.ddbias_part[part * a.batch * D + b * D + d] = dbias;
  }
}

// Adjoint carries of the parts of a long sequence: for part g = blockIdx.y + 1
// (the first part's carry is never needed), the carry a_t lambda_t that
// leaves its first token when zero enters its last one, mu <- a_t (dyc_t C_t
// + mu) from the last token back, and the part's summed delta (compensated),
// from which exp(A sum delta) carries the right neighbour's carry through.
template <typename In, bool GATE, int SPL, bool SP>
__global__ void __launch_bounds__(64 * bwd_waves<SPL>()) s6_bwd_carry_kernel(BwdArgs a) {
  constexpr int WB = bwd_waves<SPL>();
  constexpr int NTHR = 64 * WB;
  constexpr int CW = 4 * WB;
  constexpr int NS = 16 * SPL;
  constexpr int KS = kBwdSeg;
  constexpr int KP = kBwdPitch;  // LDS row pitch: rows 4 banks apart
  extern __shared__ float4 lds4[];
  float* sdl = reinterpret_cast<float*>(lds4);  // [CW][KP]
  float* sdyc = sdl + CW * KP;                  // [CW][KP]
  float* sC = sdyc + CW * KP;                   // [NS][KP]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int nl = lane & 15;
  const int c = 4 * (tid >> 6) + (lane >> 4);
  const int64_t D = a.D, L = a.L, N = a.N;
  const int64_t nblk = (D + CW - 1) / CW;
  const int64_t b = blockIdx.x / nblk;
  const int64_t d0 = (blockIdx.x % nblk) * CW;
  const int64_t rows_valid = D - d0 < CW ? D - d0 : CW;
  const int64_t d = d0 + c;
  const bool chv = c < rows_valid;
  const int64_t part = blockIdx.y + 1;
  const int64_t nstate = a.batch * D * N;
  const int64_t s_begin = part * a.seg_per_part;
  const int64_t s_end = s_begin + a.seg_per_part < a.nseg ? s_begin + a.seg_per_part : a.nseg;
  const In* dp = static_cast<const In*>(a.delta);
  const In* zp = static_cast<const In*>(a.z);
  const In* Cp = static_cast<const In*>(a.Cm);

  float A2[SPL], mu[SPL];
#pragma unroll
  for (int j = 0; j < SPL; ++j) {
    const int64_t n = (int64_t)nl * SPL + j;
    A2[j] = (chv && n < N) ? a.A[d * N + n] * kLog2e : 0.0f;
    mu[j] = 0.0f;
  }
  float dsum = 0.0f, dcomp = 0.0f;
  for (int64_t s = s_end - 1; s >= s_begin; --s) {
    const int64_t tb = s * KS;
    const int64_t tl = L - tb < KS ? L - tb : KS;
    __syncthreads();
    for (int i = tid; i < CW * KS; i += NTHR) {
      const int cc = i / KS, t = i % KS;
      const bool ok = cc < rows_valid && t < tl;
      const int64_t off = (b * D + d0 + (cc < rows_valid ? cc : 0)) * L + tb + (t < tl ? t : 0);
      float dl = 0.0f, dyc = 0.0f;
      if (ok) {
        dl = to_f32(dp[off]);
        if constexpr (SP) {
          float js;
          dl = bwd_step(dl, a.dbias ? a.dbias[d0 + cc] : 0.0f, a.softplus, &js);
        }
        dyc = a.dy[off];
        if constexpr (GATE) {
          const float zz = to_f32(zp[off]);
          dyc *= zz * fast_rcp(1.0f + fast_exp2(-zz * kLog2e));
        }
      }
      sdl[cc * KP + t] = dl;
      sdyc[cc * KP + t] = dyc;
    }
    for (int i = tid; i < NS * KS; i += NTHR) {
      const int n = i / KS, t = i % KS;
      const bool ok = n < N && t < tl;
      sC[n * KP + t] = ok ? to_f32(Cp[(b * N + (n < N ? n : 0)) * L + tb + (t < tl ? t : 0)]) : 0.0f;
    }
    __syncthreads();
    float cs = 0.0f;
    for (int t = KS - 1; t >= 0; --t) {
      const float dlt = sdl[c * KP + t];
      const float dyct = sdyc[c * KP + t];
#pragma unroll
      for (int j = 0; j < SPL; ++j)
        mu[j] = fast_exp2(dlt * A2[j]) * __builtin_fmaf(dyct, sC[(nl * SPL + j) * KP + t], mu[j]);
      cs += dlt;
    }
    const float tsum = dsum + cs;
    dcomp += (fabsf(dsum) >= fabsf(cs)) ? (dsum - tsum) + cs : (cs - tsum) + dsum;
    dsum = tsum;
  }
  if (chv) {
#pragma unroll
    for (int j = 0; j < SPL; ++j) {
      const int64_t n = (int64_t)nl * SPL + j;
      if (n < N) a.carry_M[part * nstate + (b * D + d) * N + n] = mu[j];
    }
    if (nl == 0) a.carry_SD[part * a.batch * D + b * D + d] = dsum + dcomp;
  }
}

// Carries entering each part from the right: mu_in[G-1] = dh_last (or 0),
// mu_in[g-1] = carry_M[g] + exp(A * carry_SD[g]) * mu_in[g].
__global__ void s6_bwd_fold(const float* __restrict__ A, const float* __restrict__ dh_last,
                            const float* __restrict__ M, const float* __restrict__ SD, float* __restrict__ mu_in,
                            int64_t batch, int64_t D, int64_t N, int64_t G) {
  const int64_t total = batch * D * N;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int64_t n = i % N;
  const int64_t bd = i / N;
  const float A2 = A[(bd % D) * N + n] * kLog2e;
  float mu = dh_last ? dh_last[i] : 0.0f;
  mu_in[(G - 1) * total + i] = mu;
  for (int64_t g = G - 1; g >= 1; --g) {
    mu = __builtin_fmaf(fast_exp2(A2 * SD[g * batch * D + bd]), mu, M[g * total + i]);
    mu_in[(g - 1) * total + i] = mu;
  }
}

// dB and dC (blockIdx.y = 0, 1): sums of the per-block partials over the
// channel blocks.  Eight running sums (blocks k = 8m + j go to sum j), added
// at the end in a fixed order: the loads of eight blocks are in flight at
// once, and the result does not depend on the launch shape.
__global__ void s6_bwd_reduce_bc(const float* __restrict__ part_b, const float* __restrict__ part_c,
                                 float* __restrict__ out_b, float* __restrict__ out_c, int64_t nblk,
                                 int64_t total) {
  const float* part = blockIdx.y ? part_c : part_b;
  float* out = blockIdx.y ? out_c : out_b;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    float sm[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) sm[j] = 0.0f;
    int64_t k = 0;
    for (; k + 8 <= nblk; k += 8) {
#pragma unroll
      for (int j = 0; j < 8; ++j) sm[j] += part[(k + j) * total + i];
    }
#pragma unroll
    for (int j = 0; j < 7; ++j)
      if (k + j < nblk) sm[j] += part[(k + j) * total + i];
    out[i] = ((sm[0] + sm[1]) + (sm[2] + sm[3])) + ((sm[4] + sm[5]) + (sm[6] + sm[7]));
  }
}

// The same sums four adjacent elements at a time (16-byte loads; total a
// multiple of 4, every pointer 16-byte aligned): each element is added in
// the same order as above, so the results are the same bit for bit.
__global__ void s6_bwd_reduce_bc4(const float4* __restrict__ part_b, const float4* __restrict__ part_c,
                                  float4* __restrict__ out_b, float4* __restrict__ out_c, int64_t nblk,
                                  int64_t total4) {
  const float4* part = blockIdx.y ? part_c : part_b;
  float4* out = blockIdx.y ? out_c : out_b;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total4;
       i += (int64_t)gridDim.x * blockDim.x) {
    float4 sm[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) sm[j] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    auto add = [](float4& a, const float4& v) { a.x += v.x; a.y += v.y; a.z += v.z; a.w += v.w; };
    int64_t k = 0;
    for (; k + 8 <= nblk; k += 8) {
      float4 v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = part[(k + j) * total4 + i];
#pragma unroll
      for (int j = 0; j < 8; ++j) add(sm[j], v[j]);
    }
#pragma unroll
    for (int j = 0; j < 7; ++j)
      if (k + j < nblk) add(sm[j], part[(k + j) * total4 + i]);
    auto tree = [&](float s0, float s1, float s2, float s3, float s4, float s5, float s6, float s7) {
      return ((s0 + s1) + (s2 + s3)) + ((s4 + s5) + (s6 + s7));
    };
    out[i] = make_float4(tree(sm[0].x, sm[1].x, sm[2].x, sm[3].x, sm[4].x, sm[5].x, sm[6].x, sm[7].x),
                         tree(sm[0].y, sm[1].y, sm[2].y, sm[3].y, sm[4].y, sm[5].y, sm[6].y, sm[7].y),
                         tree(sm[0].z, sm[1].z, sm[2].z, sm[3].z, sm[4].z, sm[5].z, sm[6].z, sm[7].z),
                         tree(sm[0].w, sm[1].w, sm[2].w, sm[3].w, sm[4].w, sm[5].w, sm[6].w, sm[7].w));
  }
}

// dA (D, N) and dD (D): sums over batch rows, in order.
__global__ void s6_bwd_reduce_rows(const float* __restrict__ dA_part, const float* __restrict__ dD_part,
                                   const float* __restrict__ db_part, float* __restrict__ dA,
                                   float* __restrict__ dD, float* __restrict__ db, int64_t batch, int64_t D,
                                   int64_t N) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < D * N) {
    float s = 0.0f;
    for (int64_t b = 0; b < batch; ++b) s += dA_part[b * D * N + i];
    dA[i] = s;
  }
  if (dD && i < D) {
    float s = 0.0f;
    for (int64_t b = 0; b < batch; ++b) s += dD_part[b * D + i];
    dD[i] = s;
  }
  if (db && i < D) {
    float s = 0.0f;
    for (int64_t b = 0; b < batch; ++b) s += db_part[b * D + i];
    db[i] = s;
  }
}

// Backward through the convolution front.  dxo: the gradient with respect
// to its output x' (the adjoint kernel's dx when the scan ran on x').  A
// block of 256 threads covers 2048 tokens of one (batch, channel) row
// (blockIdx.x = row * nlb + block); thread tid takes tokens tid, tid + 256,
// ... of the block, so every load is contiguous across the threads.  Each
// thread recomputes the filter's output xc and dxc = dxo * SiLU'(xc) for its
// tokens into LDS (the first K - 1 threads also the tokens just past the
// block), then writes dx_s = sum_k w_k dxc_{s+K-1-k}; the block sums
// dxc_t x_{t-K+1+k} (filter) and dxc_t (bias) in a fixed order (DPP sums
// over the 16 lanes of a row, then the 16 row sums one after another) into
// part[(b * nlb + block) * D + ch][k]; the row's first block also writes the
// state's gradient (the same sum for s < 0).
constexpr int kConvTok = 8;  // tokens per thread
template <typename In>
__global__ void __launch_bounds__(256) s6_conv_bwd_kernel(const In* __restrict__ xp, const float* __restrict__ cw,
                                                          const float* __restrict__ cb,
                                                          const float* __restrict__ cstate, int K,
                                                          const float* __restrict__ dxo, float* __restrict__ dx,
                                                          float* __restrict__ dstate, float* __restrict__ part,
                                                          int64_t batch, int64_t D, int64_t L, int64_t nlb) {
  constexpr int TB = 256 * kConvTok;  // tokens per block
  constexpr int H = kMaxConv - 1;       // halo
  __shared__ float sdxc[TB + H];
  __shared__ float sxin[TB + 2 * H];    // inputs at tb0 - H .. tb0 + TB + H - 1
  __shared__ float red[16 * (kMaxConv + 1)];
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x / nlb;
  const int64_t lb = blockIdx.x % nlb;
  const int64_t ch = row % D;
  const int64_t b = row / D;
  const int64_t tb0 = lb * TB;
  float wk[kMaxConv];
#pragma unroll
  for (int k = 0; k < kMaxConv; ++k) wk[k] = k < K ? cw[ch * K + k] : 0.0f;
  const float bias = cb ? cb[ch] : 0.0f;
  for (int i = tid; i < TB + 2 * H; i += 256) {
    const int64_t sg = tb0 - H + i;
    float v = 0.0f;
    if (sg >= 0 && sg < L) v = to_f32(xp[row * L + sg]);
    else if (sg < 0 && sg >= -(int64_t)(K - 1) && cstate) v = cstate[row * (K - 1) + (K - 1) + sg];
    sxin[i] = v;
  }
  __syncthreads();
  auto x_at = [&](int64_t s) -> float { return sxin[s - tb0 + H]; };
  // dxc of token t (0 past the end); xs[j] receives the input j tokens back
  auto dxc_at = [&](int64_t t, float (&xs)[kMaxConv]) -> float {
#pragma unroll
    for (int j = 0; j < kMaxConv; ++j) xs[j] = 0.0f;
    if (t >= L) return 0.0f;
    float acc = bias;
#pragma unroll
    for (int j = 0; j < kMaxConv; ++j) {
      if (j < K) {
        xs[j] = x_at(t - j);
        acc = __builtin_fmaf(wk[K - 1 - j], xs[j], acc);
      }
    }
    const float sg = fast_rcp(1.0f + fast_exp2(-acc * kLog2e));
    return dxo[row * L + t] * (sg * __builtin_fmaf(acc, 1.0f - sg, 1.0f));
  };
  float pk[kMaxConv + 1];
#pragma unroll
  for (int k = 0; k <= kMaxConv; ++k) pk[k] = 0.0f;
#pragma unroll
  for (int i = 0; i < kConvTok; ++i) {
    float xs[kMaxConv];
    const float v = dxc_at(tb0 + i * 256 + tid, xs);
    sdxc[i * 256 + tid] = v;
    pk[kMaxConv] += v;
    // tap k reads the input K - 1 - k tokens back
#pragma unroll
    for (int k = 0; k < kMaxConv; ++k)
      if (k < K) pk[k] = __builtin_fmaf(v, xs[K - 1 - k], pk[k]);
  }
  if (tid < K - 1) {
    float xs[kMaxConv];
    sdxc[TB + tid] = dxc_at(tb0 + TB + tid, xs);
  }
  __syncthreads();
  // input gradients: token s feeds outputs s + K - 1 - k through tap k
#pragma unroll
  for (int i = 0; i < kConvTok; ++i) {
    const int li = i * 256 + tid;
    const int64_t s = tb0 + li;
    if (s < L) {
      float g = 0.0f;
#pragma unroll
      for (int k = 0; k < kMaxConv; ++k)
        if (k < K) g = __builtin_fmaf(wk[k], sdxc[li + K - 1 - k], g);
      dx[row * L + s] = g;
    }
  }
  if (dstate && lb == 0 && tid == 0) {
    for (int s = -(K - 1); s < 0; ++s) {
      float g = 0.0f;
      for (int k = 0; k < K; ++k) {
        const int t = s + K - 1 - k;
        if (t >= 0) g = __builtin_fmaf(wk[k], sdxc[t], g);
      }
      dstate[row * (K - 1) + (K - 1) + s] = g;
    }
  }
  // Sums over the 16 lanes of each row (DPP: partners l^1, l^2, the half-row
  // mirror, rotation by 8), then the 16 row sums of the block in order.
#pragma unroll
  for (int k = 0; k <= kMaxConv; ++k) {
    float v = pk[k];
    v += dpp_f<0xB1>(v);
    v += dpp_f<0x4E>(v);
    v += dpp_f<0x141>(v);
    v += dpp_f<0x128>(v);
    if ((tid & 15) == 0) red[k * 16 + (tid >> 4)] = v;
  }
  __syncthreads();
  if (tid <= kMaxConv && (tid < K || tid == kMaxConv)) {
    float acc = 0.0f;
    for (int r = 0; r < 16; ++r) acc += red[tid * 16 + r];
    part[((b * nlb + lb) * D + ch) * (kMaxConv + 1) + tid] = acc;
  }
}

// The filter's and bias's gradients: sums of the per-block partials over
// batch rows and blocks, in order.
__global__ void s6_conv_bwd_reduce(const float* __restrict__ part, float* __restrict__ dw, float* __restrict__ db,
                                   int K, int64_t rows_blocks, int64_t D) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // (channel, tap or bias)
  if (i >= D * (kMaxConv + 1)) return;
  const int64_t ch = i / (kMaxConv + 1);
  const int k = (int)(i % (kMaxConv + 1));
  if (k >= K && k != kMaxConv) return;
  float sum = 0.0f;
  for (int64_t r = 0; r < rows_blocks; ++r) sum += part[(r * D + ch) * (kMaxConv + 1) + k];
  if (k == kMaxConv) {
    if (db) db[ch] = sum;
  } else {
    dw[ch * K + k] = sum;
  }
}

// carry: the part-carry kernel (parts 1 .. G-1) instead of the main kernel.
template <typename In, bool GATE, int SPL, int OPT, bool H16>
int launch_bwd_t(const BwdArgs& a, int64_t parts, bool carry, hipStream_t st) {
  constexpr int CW = 4 * bwd_waves<SPL>();
  const int64_t nblk = (a.D + CW - 1) / CW;
  const dim3 block(64 * bwd_waves<SPL>());
  if (carry) {
    const size_t lds = sizeof(float) * ((size_t)2 * CW * kBwdPitch + (size_t)16 * SPL * kBwdPitch);
    hipLaunchKernelGGL((s6_bwd_carry_kernel<In, GATE, SPL, (OPT >= 1)>),
                       dim3((unsigned)(nblk * a.batch), (unsigned)(parts - 1)), block, lds, st, a);
    S6_HIP(hipGetLastError(), "s6_bwd_carry_kernel launch");
  } else {
    hipLaunchKernelGGL((s6_bwd_kernel<In, GATE, SPL, OPT, H16>), dim3((unsigned)(nblk * a.batch), (unsigned)parts), block,
                       bwd_lds_bytes<SPL>(OPT >= 1), st, a);
    S6_HIP(hipGetLastError(), "s6_bwd_kernel launch");
  }
  return S6_OK;
}

template <typename In, int SPL, int OPT, bool H16 = false>
int launch_bwd_g(const BwdArgs& a, bool gate, int64_t parts, bool carry, hipStream_t st) {
  return gate ? launch_bwd_t<In, true, SPL, OPT, H16>(a, parts, carry, st)
              : launch_bwd_t<In, false, SPL, OPT, H16>(a, parts, carry, st);
}

// h16: a.hin holds the state entering every chunk (one part): the exact
// hold and the convolution front only (the other levels start from one
// state per 64-token segment).
template <typename In, int SPL>
int launch_bwd_h16(const BwdArgs& a, bool gate, int opt, hipStream_t st) {
  switch (opt) {
    case 2: return launch_bwd_g<In, SPL, 2, true>(a, gate, 1, false, st);
    case 3: return launch_bwd_g<In, SPL, 3, true>(a, gate, 1, false, st);
    default: return S6_ERR_UNSUPPORTED;
  }
}

template <typename In>
int launch_bwd(const BwdArgs& a, bool gate, int64_t parts, bool carry, bool h16, hipStream_t st) {
  const int opt = a.conv_w ? 3 : a.zoh ? 2 : (a.dbias || a.softplus || a.ddbias_part) ? 1 : 0;
  if (h16) {
    if (parts != 1 || carry) return S6_ERR_UNSUPPORTED;
    return a.N <= 16 ? launch_bwd_h16<In, 1>(a, gate, opt, st) : launch_bwd_h16<In, 2>(a, gate, opt, st);
  }
  if (a.N <= 16) {
    if (opt == 3) return launch_bwd_g<In, 1, 3>(a, gate, parts, carry, st);
    if (opt == 2) return launch_bwd_g<In, 1, 2>(a, gate, parts, carry, st);
    return opt ? launch_bwd_g<In, 1, 1>(a, gate, parts, carry, st) : launch_bwd_g<In, 1, 0>(a, gate, parts, carry, st);
  }
  if (opt == 3) return launch_bwd_g<In, 2, 3>(a, gate, parts, carry, st);
  if (opt == 2) return launch_bwd_g<In, 2, 2>(a, gate, parts, carry, st);
  return opt ? launch_bwd_g<In, 2, 1>(a, gate, parts, carry, st) : launch_bwd_g<In, 2, 0>(a, gate, parts, carry, st);
}

int bwd_channels_per_block(int64_t dstate) { return dstate <= 16 ? 4 * bwd_waves<1>() : 4 * bwd_waves<2>(); }

// The backward's launch geometry and the byte offsets (256-aligned) of its
// buffers in the caller's workspace.
struct BwdWs {
  int64_t S, nblkb, G, spp, nlb;  // segments, channel blocks, parts, segments per part, front blocks
  bool h16;                       // the states come from one sequential state-only pass (every 16 or 64 tokens)
  size_t agg, sd, hin;            // checkpoint pass: segment end states, summed deltas, incoming states
  size_t hin16;                   // h16: the state entering every 16- or 64-token block (over agg, sd, hin)
  size_t dap, ddp, dbp;           // per (part, row) partials of dA, dD and the bias gradient
  size_t dBp, dCp;                // per channel-block partials of dB and dC
  size_t cM, muin, cSD;           // parts: adjoint carries and summed deltas
  size_t dxo, cpart;              // convolution front: gradient of x', filter/bias partials
  size_t total;                   // 0: the grid limits are exceeded
};

BwdWs bwd_ws_layout(int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate, bool ckpt, bool conv) {
  BwdWs w;
  memset(&w, 0, sizeof(w));
  w.S = (seqlen + kBwdSeg - 1) / kBwdSeg;
  const int64_t nagg = w.S - 1;
  const int64_t cw = bwd_channels_per_block(dstate);
  w.nblkb = (dim + cw - 1) / cw;
  if (w.nblkb * batch > INT32_MAX) return w;  // grid size
  // Parts: when the (row, channel block) workgroups fill less than half of
  // the workgroup slots (few long rows), the sequence is cut into parts run
  // side by side; the adjoint carry entering each part from the right comes
  // from a carry pass and a fold.  The parts fill the slots twice (two rounds
  // of workgroups; on a million tokens of 1536 channels 55.0 ms against
  // 59.4-59.9 ms for one round, three rounds no faster).
  int64_t G = 1;
  {
    const int64_t wgs = w.nblkb * batch;
    const int64_t slots = (int64_t)cu_count() * (dstate <= 16 ? 4 : 3);
    if (2 * wgs <= slots) G = 2 * slots / wgs < w.S ? 2 * slots / wgs : w.S;
    if (G < 1) G = 1;
  }
  w.spp = (w.S + G - 1) / G;
  w.G = (w.S + w.spp - 1) / w.spp;
  w.nlb = (seqlen + 256 * kConvTok - 1) / (256 * kConvTok);
  if (conv && (double)batch * dim * w.nlb > (double)INT32_MAX) return w;
  const int64_t nstate = batch * dim * dstate;
  auto up = [](size_t v) { return (v + 255) & ~(size_t)255; };
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += up(bytes);
    return o;
  };
  // Without checkpoints and with one part, when the sequential state-only
  // scan has enough workgroups to fill the GPU on its own (the forward's
  // plan keeps one segment), that scan writes the state entering every
  // 64-token segment, or every 16-token chunk for the exact hold and the
  // convolution front (the region is sized for the chunks: the size query
  // takes no options).  Otherwise 64-token segments are scanned side by side
  // and folded.  The layouts share the region.
  if (!ckpt && G == 1) {
    const void* none[] = {nullptr};
    w.h16 = make_plan(batch, dim, seqlen, dstate, 4, none, 1).segs == 1;
  }
  const size_t seg_bytes = ckpt ? 0
                                : up((size_t)(nagg > 0 ? nagg : 0) * nstate * sizeof(float)) +
                                      up((size_t)(nagg > 0 ? nagg : 0) * batch * dim * sizeof(float)) +
                                      up((size_t)w.S * nstate * sizeof(float));
  const size_t h16_bytes = w.h16 ? up((size_t)((seqlen + 15) / 16) * nstate * sizeof(float)) : 0;
  const size_t base = take(seg_bytes > h16_bytes ? seg_bytes : h16_bytes);
  w.agg = base;
  w.sd = w.agg + up((size_t)(nagg > 0 ? nagg : 0) * nstate * sizeof(float));
  w.hin = w.sd + up((size_t)(nagg > 0 ? nagg : 0) * batch * dim * sizeof(float));
  w.hin16 = base;
  w.dap = take((size_t)w.G * nstate * sizeof(float));
  w.ddp = take((size_t)w.G * batch * dim * sizeof(float));
  w.dbp = take((size_t)w.G * batch * dim * sizeof(float));
  w.dBp = take((size_t)w.nblkb * batch * dstate * seqlen * sizeof(float));
  w.dCp = take((size_t)w.nblkb * batch * dstate * seqlen * sizeof(float));
  w.cM = take(w.G > 1 ? (size_t)w.G * nstate * sizeof(float) : 0);
  w.muin = take(w.G > 1 ? (size_t)w.G * nstate * sizeof(float) : 0);
  w.cSD = take(w.G > 1 ? (size_t)w.G * batch * dim * sizeof(float) : 0);
  w.dxo = take(conv ? (size_t)batch * dim * seqlen * sizeof(float) : 0);
  w.cpart = take(conv ? (size_t)batch * w.nlb * dim * (kMaxConv + 1) * sizeof(float) : 0);
  w.total = off;
  return w;
}

}  // namespace

}  // namespace s6i

using namespace s6i;

namespace {

// The convolution front of s6_conv_scan_bwd and its gradient outputs.
struct ConvGrad {
  const float* w = nullptr;
  const float* bias = nullptr;
  const float* state = nullptr;
  int width = 0;
  float* dw = nullptr;
  float* dbias = nullptr;
  float* dstate = nullptr;
};

// s6_scan_bwd_ex, and s6_scan_bwd_ckpt when ckpt (the states entering every
// kCkpt-token block, from s6_scan_fwd_ckpt) is given: the checkpoint pass is
// then skipped; s6_conv_scan_bwd with a convolution front (cg.w).
int scan_bwd_impl(int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate, int in_dtype,
                  const void* x, const void* delta, const float* delta_bias, int flags, const float* A,
                  const void* Bm, const void* Cm, const float* Dskip, const void* z, const float* h0,
                  const float* dy, const float* dh_last, float* dx, float* ddelta, float* dA, float* dBm,
                  float* dCm, float* dDskip, float* dz, float* dh0, float* ddelta_bias, const float* ckpt,
                  void* workspace, size_t workspace_bytes, void* stream, const ConvGrad& cg = ConvGrad()) {
  static_assert(kBwdSeg == kCkpt, "backward segments are the checkpoint blocks");
  const bool conv = cg.w != nullptr || cg.width != 0;
  int rc = check_common(batch, dim, seqlen, dstate, in_dtype);
  if (rc) return rc;
  if (flags & ~(S6_DELTA_SOFTPLUS | S6_ZOH_EXACT)) return S6_ERR_FLAGS;
  const bool softplus = (flags & S6_DELTA_SOFTPLUS) != 0;
  const bool zoh = (flags & S6_ZOH_EXACT) != 0;
  const bool work = batch > 0 && dim > 0 && seqlen > 0;
  if (conv) {
    if (cg.width < 1 || cg.width > kMaxConv) return S6_ERR_UNSUPPORTED;
    if (zoh) return S6_ERR_UNSUPPORTED;  // the front's kernels have no exact hold
    if (!cg.w || (dim > 0 && !cg.dw)) return S6_ERR_NULL;
    const void* cps[] = {cg.w, cg.bias, cg.state, cg.dw, cg.dbias, cg.dstate};
    for (const void* p : cps)
      if (p && !aligned(p, 4)) return S6_ERR_ALIGN;
  }
  if (dim > 0 && !dA) return S6_ERR_NULL;
  if (work && (!x || !delta || !A || !Bm || !Cm || !dy || !dx || !ddelta || !dBm || !dCm))
    return S6_ERR_NULL;
  const size_t esz = in_dtype == S6_BF16 ? 2 : 4;
  const void* ins[] = {x, delta, Bm, Cm, z};
  for (const void* p : ins)
    if (p && !aligned(p, esz)) return S6_ERR_ALIGN;
  const void* f32s[] = {A, Dskip, h0, dy, dh_last, dx, ddelta, dA, dBm, dCm, dDskip, dz, dh0, delta_bias,
                        ddelta_bias, ckpt};
  for (const void* p : f32s)
    if (p && !aligned(p, 4)) return S6_ERR_ALIGN;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (dim == 0) return S6_OK;
  const int64_t nstate = batch * dim * dstate;
  if (!work) {
    // no tokens or no rows: the parameter gradients are zero and dh0 = dh_last
    fill(dA, 0.0f, dim * dstate, st);
    fill(dDskip, 0.0f, dim, st);
    fill(ddelta_bias, 0.0f, dim, st);
    if (conv) {
      fill(cg.dw, 0.0f, dim * cg.width, st);
      fill(cg.dbias, 0.0f, dim, st);
      fill(cg.dstate, 0.0f, batch * dim * (cg.width - 1), st);
    }
    S6_HIP(hipGetLastError(), "s6_scan_bwd fill");
    return dh0 ? launch_copy_state(dh_last, dh0, nstate, st) : S6_OK;
  }

  const BwdWs w = bwd_ws_layout(batch, dim, seqlen, dstate, ckpt != nullptr, conv);
  if (w.total == 0) return S6_ERR_SHAPE;  // grid limits
  if (!workspace || workspace_bytes < w.total) return S6_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return S6_ERR_ALIGN;
  const int64_t S = w.S, nagg = S - 1, nblkb = w.nblkb, G = w.G, spp = w.spp, nlb = w.nlb;
  const bool h16 = w.h16;
  // The sequential state-only scan stores the state entering every 16-token
  // chunk for the exact hold and the convolution front, whose adjoint
  // kernels would spend more recomputing the chunk starts (4.00 against
  // 3.81 ms, 2.82 against 2.73 ms on the 3B layer), and the state entering
  // every 64-token block otherwise, from which the adjoint kernel recomputes
  // the chunk starts (1.873-1.882 against 1.935-1.936 ms: a quarter of the
  // states written; bit-identical gradients).  The region is sized for the
  // former.
  const bool chunk16 = zoh || conv;
  char* wp = static_cast<char*>(workspace);
  float* agg = reinterpret_cast<float*>(wp + w.agg);
  float* sd = reinterpret_cast<float*>(wp + w.sd);
  float* hin16 = reinterpret_cast<float*>(wp + w.hin16);
  const float* hin = ckpt ? ckpt : h16 ? hin16 : reinterpret_cast<float*>(wp + w.hin);
  float* dap = reinterpret_cast<float*>(wp + w.dap);
  float* ddp = reinterpret_cast<float*>(wp + w.ddp);
  float* dbp = reinterpret_cast<float*>(wp + w.dbp);  // bias gradient per part and row
  float* dBp = reinterpret_cast<float*>(wp + w.dBp);
  float* dcp = reinterpret_cast<float*>(wp + w.dCp);
  float* cM = reinterpret_cast<float*>(wp + w.cM);
  float* muin = reinterpret_cast<float*>(wp + w.muin);
  float* cSD = reinterpret_cast<float*>(wp + w.cSD);
  float* dxo = conv ? reinterpret_cast<float*>(wp + w.dxo) : nullptr;
  float* cpart = reinterpret_cast<float*>(wp + w.cpart);

  // the state entering every segment (or chunk): one sequential state-only scan from h0
  if (h16) {
    const void* vecptrs[] = {x, delta, Bm};
    Plan p = make_plan(batch, dim, seqlen, dstate, esz, vecptrs, 3);
    if (p.segs != 1) return S6_ERR_UNSUPPORTED;  // the layout's plan kept one segment
    ScanArgs g;
    memset(&g, 0, sizeof(g));
    g.x = x; g.delta = delta; g.Bm = Bm; g.A = A;
    g.hinit = h0; g.hinit_stride = 0; g.ckpt = hin16; g.ckpt_log2 = chunk16 ? 4 : 6;
    g.dbias = delta_bias; g.softplus = softplus; g.zoh = zoh;
    g.conv_w = cg.w; g.conv_b = cg.bias; g.conv_state = cg.state; g.conv_k = cg.width;
    g.D = dim; g.L = seqlen; g.N = dstate; g.seg_len = p.seg_len;
    rc = launch_scan_any(in_dtype, kModeState, g, p, false, batch, 1, st);
  }
  // pass 1: end state (from zero) and summed delta of every segment but the last
  if (nagg > 0 && !ckpt && !h16) {
    const void* vecptrs[] = {x, delta, Bm};
    Plan p = make_plan(batch, dim, seqlen, dstate, esz, vecptrs, 3);
    ScanArgs g;
    memset(&g, 0, sizeof(g));
    g.x = x; g.delta = delta; g.Bm = Bm; g.A = A;
    g.hout = agg; g.hout_stride = nstate; g.sumdelta = sd;
    g.dbias = delta_bias; g.softplus = softplus; g.zoh = zoh;
    g.conv_w = cg.w; g.conv_b = cg.bias; g.conv_state = cg.state; g.conv_k = cg.width;
    g.D = dim; g.L = seqlen; g.N = dstate; g.seg_len = kBwdSeg;
    rc = launch_scan_any(in_dtype, kModeState, g, p, false, batch, nagg, st);
  }
  // the state entering every segment
  if (rc == S6_OK && !ckpt && !h16) {
    rc = launch_fold_carries(A, h0, agg, sd, const_cast<float*>(hin), nullptr, batch, dim, dstate, S, nagg, st);
  }
  if (rc == S6_OK) {
    BwdArgs b;
    memset(&b, 0, sizeof(b));
    b.x = x; b.delta = delta; b.z = z; b.Bm = Bm; b.Cm = Cm; b.A = A; b.Dskip = Dskip;
    b.dy = dy; b.dh_last = dh_last; b.hin = hin;
    b.dx = conv ? dxo : dx; b.ddelta = ddelta; b.dz = dz; b.dA_part = dap; b.dD_part = ddp;
    b.conv_w = cg.w; b.conv_b = cg.bias; b.conv_state = cg.state; b.conv_k = cg.width;
    b.dB_part = dBp; b.dC_part = dcp; b.dh0 = dh0;
    b.dbias = delta_bias; b.softplus = softplus; b.zoh = zoh; b.ddbias_part = ddelta_bias ? dbp : nullptr;
    b.batch = batch; b.D = dim; b.L = seqlen; b.N = dstate; b.nseg = S; b.seg_per_part = spp;
    const bool gate = z != nullptr;
    if (G > 1) {
      b.carry_M = cM;
      b.carry_SD = cSD;
      rc = in_dtype == S6_BF16 ? launch_bwd<uint16_t>(b, gate, G, true, false, st)
                               : launch_bwd<float>(b, gate, G, true, false, st);
      if (rc == S6_OK) {
        hipLaunchKernelGGL(s6_bwd_fold, dim3((unsigned)((nstate + 255) / 256)), dim3(256), 0, st, A, dh_last, cM, cSD,
                           muin, batch, dim, dstate, G);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) rc = hip_fail(e, "s6_bwd_fold launch");
      }
      b.mu_in = muin;
    }
    if (rc == S6_OK)
      rc = in_dtype == S6_BF16 ? launch_bwd<uint16_t>(b, gate, G, false, h16 && chunk16, st)
                               : launch_bwd<float>(b, gate, G, false, h16 && chunk16, st);
  }
  if (rc == S6_OK) {
    const int64_t tot = batch * dstate * seqlen;
    const void* bcp[] = {dBp, dcp, dBm, dCm};
    bool v4 = tot % 4 == 0;
    for (const void* q : bcp) v4 = v4 && aligned(q, 16);
    if (v4) {
      int64_t blocks = (tot / 4 + 255) / 256;
      if (blocks > 65536) blocks = 65536;
      hipLaunchKernelGGL(s6_bwd_reduce_bc4, dim3((unsigned)blocks, 2u), dim3(256), 0, st,
                         reinterpret_cast<const float4*>(dBp), reinterpret_cast<const float4*>(dcp),
                         reinterpret_cast<float4*>(dBm), reinterpret_cast<float4*>(dCm), nblkb, tot / 4);
    } else {
      int64_t blocks = (tot + 255) / 256;
      if (blocks > 65536) blocks = 65536;
      hipLaunchKernelGGL(s6_bwd_reduce_bc, dim3((unsigned)blocks, 2u), dim3(256), 0, st, dBp, dcp, dBm, dCm,
                         nblkb, tot);
    }
    const int64_t rows = dim * dstate;
    hipLaunchKernelGGL(s6_bwd_reduce_rows, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, st, dap, ddp, dbp,
                       dA, dDskip, ddelta_bias, G * batch, dim, dstate);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) rc = hip_fail(e, "s6_bwd reduction launch");
  }
  if (rc == S6_OK && conv) {
    const dim3 grid((unsigned)(batch * dim * nlb));
    if (in_dtype == S6_BF16)
      hipLaunchKernelGGL(s6_conv_bwd_kernel<uint16_t>, grid, dim3(256), 0, st, static_cast<const uint16_t*>(x), cg.w,
                         cg.bias, cg.state, cg.width, dxo, dx, cg.dstate, cpart, batch, dim, seqlen, nlb);
    else
      hipLaunchKernelGGL(s6_conv_bwd_kernel<float>, grid, dim3(256), 0, st, static_cast<const float*>(x), cg.w,
                         cg.bias, cg.state, cg.width, dxo, dx, cg.dstate, cpart, batch, dim, seqlen, nlb);
    const int64_t n = dim * (kMaxConv + 1);
    hipLaunchKernelGGL(s6_conv_bwd_reduce, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, cpart, cg.dw,
                       cg.dbias, cg.width, batch * nlb, dim);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) rc = hip_fail(e, "s6_conv_bwd launch");
  }
  return rc;
}

}  // namespace

extern "C" {

int s6_scan_bwd_ex(int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate, int in_dtype,
                   const void* x, const void* delta, const float* delta_bias, int flags, const float* A,
                   const void* Bm, const void* Cm, const float* Dskip, const void* z, const float* h0,
                   const float* dy, const float* dh_last, float* dx, float* ddelta, float* dA, float* dBm,
                   float* dCm, float* dDskip, float* dz, float* dh0, float* ddelta_bias, void* workspace,
                   size_t workspace_bytes, void* stream) {
  return scan_bwd_impl(batch, dim, seqlen, dstate, in_dtype, x, delta, delta_bias, flags, A, Bm, Cm, Dskip, z, h0,
                       dy, dh_last, dx, ddelta, dA, dBm, dCm, dDskip, dz, dh0, ddelta_bias, nullptr, workspace,
                       workspace_bytes, stream);
}

int s6_scan_bwd_ckpt(int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate, int in_dtype,
                     const void* x, const void* delta, const float* delta_bias, int flags, const float* A,
                     const void* Bm, const void* Cm, const float* Dskip, const void* z, const float* ckpt,
                     const float* dy, const float* dh_last, float* dx, float* ddelta, float* dA, float* dBm,
                     float* dCm, float* dDskip, float* dz, float* dh0, float* ddelta_bias, void* workspace,
                     size_t workspace_bytes, void* stream) {
  if (!ckpt && batch > 0 && dim > 0 && seqlen > 0) return S6_ERR_NULL;
  return scan_bwd_impl(batch, dim, seqlen, dstate, in_dtype, x, delta, delta_bias, flags, A, Bm, Cm, Dskip, z,
                       nullptr, dy, dh_last, dx, ddelta, dA, dBm, dCm, dDskip, dz, dh0, ddelta_bias, ckpt, workspace,
                       workspace_bytes, stream);
}

int s6_conv_scan_bwd(int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate, int in_dtype,
                     const void* x, const float* conv_w, const float* conv_bias, int conv_width,
                     const float* conv_state, const void* delta, const float* delta_bias, int flags,
                     const float* A, const void* Bm, const void* Cm, const float* Dskip, const void* z,
                     const float* h0, const float* dy, const float* dh_last, float* dx, float* ddelta,
                     float* dA, float* dBm, float* dCm, float* dDskip, float* dz, float* dh0,
                     float* ddelta_bias, float* dconv_w, float* dconv_bias, float* dconv_state, void* workspace,
                     size_t workspace_bytes, void* stream) {
  if (!conv_w && conv_width == 0) return S6_ERR_NULL;
  ConvGrad cg;
  cg.w = conv_w;
  cg.bias = conv_bias;
  cg.state = conv_state;
  cg.width = conv_width;
  cg.dw = dconv_w;
  cg.dbias = dconv_bias;
  cg.dstate = dconv_state;
  return scan_bwd_impl(batch, dim, seqlen, dstate, in_dtype, x, delta, delta_bias, flags, A, Bm, Cm, Dskip, z, h0,
                       dy, dh_last, dx, ddelta, dA, dBm, dCm, dDskip, dz, dh0, ddelta_bias, nullptr, workspace,
                       workspace_bytes, stream, cg);
}

int s6_scan_bwd(int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate, int in_dtype,
                const void* x, const void* delta, const float* A, const void* Bm, const void* Cm,
                const float* Dskip, const void* z, const float* h0, const float* dy,
                const float* dh_last, float* dx, float* ddelta, float* dA, float* dBm, float* dCm,
                float* dDskip, float* dz, float* dh0, void* workspace, size_t workspace_bytes, void* stream) {
  return s6_scan_bwd_ex(batch, dim, seqlen, dstate, in_dtype, x, delta, nullptr, 0, A, Bm, Cm, Dskip, z, h0, dy,
                        dh_last, dx, ddelta, dA, dBm, dCm, dDskip, dz, dh0, nullptr, workspace, workspace_bytes,
                        stream);
}

int s6_scan_bwd_workspace_size(int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate, int in_dtype,
                               int conv_width, int from_ckpt, size_t* bytes) {
  if (!bytes) return S6_ERR_NULL;
  int rc = check_common(batch, dim, seqlen, dstate, in_dtype);
  if (rc) return rc;
  if (conv_width < 0 || conv_width > kMaxConv) return S6_ERR_UNSUPPORTED;
  *bytes = 0;
  if (batch == 0 || dim == 0 || seqlen == 0) return S6_OK;
  const BwdWs w = bwd_ws_layout(batch, dim, seqlen, dstate, from_ckpt != 0, conv_width > 0);
  if (w.total == 0) return S6_ERR_SHAPE;
  *bytes = w.total;
  return S6_OK;
}

}  // extern "C"
