// ssd.hip -- the selective scan with one A value per channel (A[d, n] = a_d
// for every state n), in chunked matrix form on the matrix cores:
// s6_ssd_scan_fwd.
//
// What is computed is the recurrence of s6_scan_fwd with that A (the pages'
// guide, "【LLM】Mamba和State Space Models详解" §2.3-§2.4 and §3.2); the
// paper-list page's Mamba-2 abstract (state space duality) notes that such
// a scan is a structured semiseparable matrix and computes it with matrix
// products.  Within a chunk of 16 tokens starting after state H_in:
//
//   y_t   = sum_{s<=t} (C_t . B_s) e^{a (c_t - c_s)} Delta_s x_s
//           + e^{a c_t} C_t . H_in + D x_t,        then the gate SiLU(z_t)
//   H_out = e^{a c_16} H_in + sum_s B_s e^{a (c_16 - c_s)} Delta_s x_s
//
// with c_t = Delta_0 + ... + Delta_t (inclusive, within the chunk).  The Gram
// matrix G[t, s] = C_t . B_s is the same for every channel of a batch row;
// the decays separate around the chunk's midpoint r = c_16 / 2 as
// e^{a (c_t - c_s)} = P_t Q_s with P_t = e^{a (c_t - r)}, Q_s = e^{-a (c_s - r)},
// so with V_s = Delta_s x_s Q_s (per channel):
//
//   y   = P o ( tril(G) V + C (e^{a r} H_in) ) + D x
//   H'  = e^{a c_16} H_in + e^{a (c_16 - r)} B^T V
//
// four 16 x 16 x 16 products per chunk and channel tile (G, tril(G) V, C H,
// B^T V) and two exponentials per token and channel (P and Q), where the
// scan of s6_scan_fwd needs one per token, channel and state.  P and Q lie in
// [e^{-R/2}, e^{R/2}] with R = |a| c_16; when R exceeds kRangeLog2 (in log2
// units) for a channel of the tile, the tile's chunk is computed without the
// separation (per-pair decays for the intra-chunk part, decays to the chunk's
// ends for the rest), so no factor leaves fp32's range.
//
// Layout on the wave: a wave owns 16 channels of one batch row and walks the
// sequence in 16-token chunks with its 16 x 16 state tile (states x channels)
// in 4 VGPRs per lane.  Lane l = 16 g + c: for the per-(token, channel)
// values it holds channel c, tokens 4g .. 4g+3 (the natural row-major layout
// of x, delta, z and y, and the layout of a 16 x 16 x 16 MFMA's B operand
// and result); B and C are loaded the same way (state c, tokens 4g .. 4g+3)
// and turned token-major by an MFMA with the identity.  Operands in fp32
// (V, G, the state) enter bf16 MFMAs as a sum of two bf16 parts (hi + lo,
// three products, relative error below 2^-16); with fp32 inputs the products
// run on fp32 MFMAs instead.
#include "s6_internal.h"

namespace s6i {

namespace {

typedef short bf16x4 __attribute__((ext_vector_type(4)));  // 4 bf16 bit patterns (an MFMA operand)
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kQ = 16;                 // tokens per chunk
constexpr int kTile = 16;              // channels per wave
constexpr int kPF = 4;                 // chunks in flight (ring of staged loads)
// Largest |a| c_16 (log2 units) for the separated decays: P, Q, e^{a r} stay
// within 2^-80 .. 2^80 of the data, far from fp32's limits.
constexpr float kRangeLog2 = 160.0f;

// Two floats as packed bf16 (round to nearest even: v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf_lo(uint32_t p) { return __uint_as_float(p << 16); }
__device__ __forceinline__ float bf_hi(uint32_t p) { return __uint_as_float(p & 0xffff0000u); }

// An MFMA operand of four fp32 values per lane, as bf16 parts (hi, lo) or
// as the fp32 values themselves.
struct Opnd {
  bf16x4 hi, lo;
  float f[4];
};

template <bool F32>
__device__ __forceinline__ void split(const float v[4], Opnd& o) {
  if constexpr (F32) {
    for (int j = 0; j < 4; ++j) o.f[j] = v[j];
  } else {
    const uint32_t h01 = pack_bf16(v[0], v[1]), h23 = pack_bf16(v[2], v[3]);
    const uint32_t l01 = pack_bf16(v[0] - bf_lo(h01), v[1] - bf_hi(h01));
    const uint32_t l23 = pack_bf16(v[2] - bf_lo(h23), v[3] - bf_hi(h23));
    o.hi = __builtin_bit_cast(bf16x4, (uint64_t)h01 | ((uint64_t)h23 << 32));
    o.lo = __builtin_bit_cast(bf16x4, (uint64_t)l01 | ((uint64_t)l23 << 32));
  }
}

// Values that are exact in bf16 (inputs, transposed inputs): one part.
template <bool F32>
__device__ __forceinline__ void exact(const float v[4], Opnd& o) {
  if constexpr (F32) {
    for (int j = 0; j < 4; ++j) o.f[j] = v[j];
  } else {
    const uint32_t h01 = pack_bf16(v[0], v[1]), h23 = pack_bf16(v[2], v[3]);
    o.hi = __builtin_bit_cast(bf16x4, (uint64_t)h01 | ((uint64_t)h23 << 32));
  }
}

__device__ __forceinline__ f32x4 mma_bf(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// D += A B (16 x 16 x 16).  Lane 16 g + c holds A[c][4g + j] and B[4g + j][c]
// (j = 0..3); D's lane holds D[4g + r][c] (r = 0..3).  EA / EB: the operand
// is exact in one bf16 part; otherwise its lo part enters too (the lo x lo
// product is left out).
template <bool F32, bool EA, bool EB>
__device__ __forceinline__ f32x4 mma(const Opnd& a, const Opnd& b, f32x4 d) {
  if constexpr (F32) {
    for (int j = 0; j < 4; ++j) d = __builtin_amdgcn_mfma_f32_16x16x4f32(a.f[j], b.f[j], d, 0, 0, 0);
  } else {
    d = mma_bf(a.hi, b.hi, d);
    if constexpr (!EB) d = mma_bf(a.hi, b.lo, d);
    if constexpr (!EA) d = mma_bf(a.lo, b.hi, d);
  }
  return d;
}

// Raw inputs of one chunk for one lane: 4 tokens of x, delta, z of channel
// c and 4 tokens of B and C of state c.
template <typename In>
struct Raw {
  In x[4], dl[4], z[4], b[4], c[4];
};

struct SsdArgs {
  const void* x;
  const void* delta;
  const void* z;       // nullable
  const void* Bm;
  const void* Cm;
  const float* A;      // (D)
  const float* Dskip;  // nullable
  const float* h0;     // nullable
  float* y;
  float* h_last;       // nullable
  int64_t D, L, N;
};

template <typename In, bool VEC>
__device__ __forceinline__ void load4(const In* __restrict__ row, int64_t t, int64_t L, In out[4]) {
  if constexpr (VEC) {
    // L % 4 == 0 and rows aligned: a lane's 4 tokens are all in or all out;
    // out-of-range groups read the row's last group (masked by the caller).
    const int64_t tc = t < L ? t : L - 4;
    if constexpr (sizeof(In) == 2) {
      const uint2 v = *reinterpret_cast<const uint2*>(row + tc);
      out[0] = (In)(v.x & 0xffff); out[1] = (In)(v.x >> 16);
      out[2] = (In)(v.y & 0xffff); out[3] = (In)(v.y >> 16);
    } else {
      const float4 v = *reinterpret_cast<const float4*>(row + tc);
      out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
    }
  } else {
    for (int j = 0; j < 4; ++j) {
      const int64_t tj = t + j < L ? t + j : L - 1;
      out[j] = row[tj];
    }
  }
}

template <typename In, bool GATE, bool VEC>
__global__ void __launch_bounds__(64) s6_ssd_kernel(SsdArgs a, int64_t batch) {
  constexpr bool kF32 = std::is_same<In, float>::value;
  __shared__ float lds[3 * kQ * kTile];  // the exact path's G, cumulative steps and inputs

  const int lane = threadIdx.x;
  const int g = lane >> 4, c = lane & 15;
  const int64_t b = blockIdx.x % batch;              // batch rows spread over the XCDs
  const int64_t d0 = (blockIdx.x / batch) * kTile;
  const int64_t D = a.D, L = a.L, N = a.N;
  const bool dval = d0 + c < D;
  const int64_t dc = dval ? d0 + c : D - 1;          // clamped channel of this lane
  const bool nval = c < N;
  const int64_t nc = nval ? c : N - 1;               // clamped state of this lane

  const In* xr = static_cast<const In*>(a.x) + (b * D + dc) * L;
  const In* dr = static_cast<const In*>(a.delta) + (b * D + dc) * L;
  const In* zr = GATE ? static_cast<const In*>(a.z) + (b * D + dc) * L : nullptr;
  const In* br = static_cast<const In*>(a.Bm) + (b * N + nc) * L;
  const In* cr = static_cast<const In*>(a.Cm) + (b * N + nc) * L;
  const float a2 = a.A[dc] * kLog2e;                  // a log2(e) <= 0
  const float dsk = a.Dskip ? a.Dskip[dc] : 0.0f;

  // identity (B operand): lane (g, c) holds I[4g + j][c]
  Opnd ident;
  {
    float v[4];
    for (int j = 0; j < 4; ++j) v[j] = (4 * g + j == c) ? 1.0f : 0.0f;
    exact<kF32>(v, ident);
  }
  // state tile: lane (g, c) holds H[n = 4g + r][d = c]
  f32x4 H;
  for (int r = 0; r < 4; ++r) {
    const int n = 4 * g + r;
    H[r] = (a.h0 && dval && n < N) ? a.h0[(b * D + d0 + c) * N + n] : 0.0f;
  }

  const int64_t nch = (L + kQ - 1) / kQ;
  Raw<In> ring[kPF];
  auto issue = [&](Raw<In>& rw, int64_t k) {
    const int64_t t = k * kQ + 4 * g;
    load4<In, VEC>(xr, t, L, rw.x);
    load4<In, VEC>(dr, t, L, rw.dl);
    if constexpr (GATE) load4<In, VEC>(zr, t, L, rw.z);
    load4<In, VEC>(br, t, L, rw.b);
    load4<In, VEC>(cr, t, L, rw.c);
  };
  for (int i = 0; i < kPF; ++i) issue(ring[i], i);

  auto chunk = [&](const Raw<In>& rw, int64_t k) {
    const int64_t t0 = k * kQ + 4 * g;
    float xv[4], dv[4], bv[4], cv[4];
    for (int j = 0; j < 4; ++j) {
      const bool ok = t0 + j < L;
      xv[j] = (ok && dval) ? to_f32(rw.x[j]) : 0.0f;
      dv[j] = (ok && dval) ? to_f32(rw.dl[j]) : 0.0f;
      bv[j] = (ok && nval) ? to_f32(rw.b[j]) : 0.0f;
      cv[j] = (ok && nval) ? to_f32(rw.c[j]) : 0.0f;
    }
    // cumulative step within the chunk: the lane's 4 tokens, then the
    // groups before it (lanes c, c+16, c+32, c+48 hold the 4 groups)
    float p[4];
    p[0] = dv[0];
    p[1] = p[0] + dv[1];
    p[2] = p[1] + dv[2];
    p[3] = p[2] + dv[3];
    const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(p[3]), __float_as_uint(p[3]), false, false);
    const float lo16 = __uint_as_float((unsigned)s16[0]), hi16 = __uint_as_float((unsigned)s16[1]);
    const float pair = lo16 + hi16;
    const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(pair), __float_as_uint(pair), false, false);
    const float lo32 = __uint_as_float((unsigned)s32[0]), hi32 = __uint_as_float((unsigned)s32[1]);
    const float total = lo32 + hi32;
    const float ex = ((g & 1) ? lo16 : 0.0f) + ((g & 2) ? lo32 : 0.0f);
    float cs[4];
    for (int j = 0; j < 4; ++j) cs[j] = ex + p[j];

    // B and C token-major: lane (g, c) holds X[n = 4g + j][t = c]
    Opnd bn, cn;
    exact<kF32>(bv, bn);
    exact<kF32>(cv, cn);
    const f32x4 z4 = {0.0f, 0.0f, 0.0f, 0.0f};
    const f32x4 btf = mma<kF32, true, true>(bn, ident, z4);
    const f32x4 ctf = mma<kF32, true, true>(cn, ident, z4);
    Opnd bt, ct;
    {
      float v[4] = {btf[0], btf[1], btf[2], btf[3]};
      exact<kF32>(v, bt);
      float w[4] = {ctf[0], ctf[1], ctf[2], ctf[3]};
      exact<kF32>(w, ct);
    }
    // G^T = Bmat Cmat^T: lane (g, c) gets G[t = c][s = 4g + r], the A
    // operand of tril(G) V; entries with s > t are dropped
    const f32x4 gt = mma<kF32, true, true>(bt, ct, z4);
    float gv[4];
    for (int r = 0; r < 4; ++r) gv[r] = (4 * g + r <= c) ? gt[r] : 0.0f;

    float v[4];
    for (int j = 0; j < 4; ++j) v[j] = dv[j] * xv[j];
    const float rng = fabsf(a2) * total;  // |a| c_16 in log2 units
    float P[4];
    f32x4 Y;
    const bool wide = __builtin_amdgcn_ballot_w64(rng > kRangeLog2) != 0;
    if (!wide) {
      const float half = 0.5f * total;
      float V[4];
      for (int j = 0; j < 4; ++j) {
        const float u = a2 * (cs[j] - half);
        P[j] = fast_exp2(u);
        V[j] = v[j] * fast_exp2(-u);
      }
      const float kr = fast_exp2(a2 * half);  // e^{a r} = e^{a (c_16 - r)}
      Opnd Vo, Go, Ho;
      split<kF32>(V, Vo);
      split<kF32>(gv, Go);
      float hs[4] = {H[0] * kr, H[1] * kr, H[2] * kr, H[3] * kr};
      split<kF32>(hs, Ho);
      Y = mma<kF32, false, false>(Go, Vo, z4);
      Y = mma<kF32, true, false>(ct, Ho, Y);
      const f32x4 S = mma<kF32, true, false>(bn, Vo, z4);
      const float dec = fast_exp2(a2 * total);
      for (int r = 0; r < 4; ++r) H[r] = __builtin_fmaf(dec, H[r], kr * S[r]);
    } else {
      // decays to the chunk's ends (each <= 1) and per-pair decays within it
      float W[4];
      for (int j = 0; j < 4; ++j) {
        P[j] = fast_exp2(a2 * cs[j]);
        W[j] = v[j] * fast_exp2(a2 * (total - cs[j]));
      }
      Opnd Wo, Ho;
      split<kF32>(W, Wo);
      float hs[4] = {H[0], H[1], H[2], H[3]};
      split<kF32>(hs, Ho);
      const f32x4 Yo = mma<kF32, true, false>(ct, Ho, z4);
      const f32x4 S = mma<kF32, true, false>(bn, Wo, z4);
      const float dec = fast_exp2(a2 * total);
      for (int r = 0; r < 4; ++r) H[r] = __builtin_fmaf(dec, H[r], S[r]);
      float* sg = lds;                 // [t][s]
      float* sc = lds + kQ * kTile;    // [channel][token] cumulative step
      float* sv = sc + kQ * kTile;     // [channel][token] delta x
      __syncthreads();
      for (int r = 0; r < 4; ++r) sg[c * kQ + 4 * g + r] = gv[r];
      for (int j = 0; j < 4; ++j) {
        sc[c * kQ + 4 * g + j] = cs[j];
        sv[c * kQ + 4 * g + j] = v[j];
      }
      __syncthreads();
      for (int r = 0; r < 4; ++r) {
        const int t = 4 * g + r;
        float acc = 0.0f;
        for (int s = 0; s <= t; ++s)
          acc = __builtin_fmaf(sg[t * kQ + s] * fast_exp2(a2 * (sc[c * kQ + t] - sc[c * kQ + s])), sv[c * kQ + s],
                               acc);
        Y[r] = __builtin_fmaf(P[r], Yo[r], acc);
        P[r] = 1.0f;
      }
    }
    // output: y_t = P_t Y_t + D x_t, gated; lane (g, c) holds tokens 4g + r of channel c
    float yo[4];
    for (int r = 0; r < 4; ++r) {
      float yy = __builtin_fmaf(P[r], Y[r], dsk * xv[r]);
      if constexpr (GATE) yy *= silu(to_f32(rw.z[r]));
      yo[r] = yy;
    }
    if (dval && t0 < L) {
      float* yp = a.y + (b * D + d0 + c) * L + t0;
      if constexpr (VEC) {
        *reinterpret_cast<float4*>(yp) = make_float4(yo[0], yo[1], yo[2], yo[3]);
      } else {
        for (int r = 0; r < 4; ++r)
          if (t0 + r < L) yp[r] = yo[r];
      }
    }
  };

  // Whole cycles of kPF chunks; chunks past the end are masked (zero step
  // and input: the state passes through unchanged) and store nothing.
  for (int64_t k = 0; k < nch; k += kPF) {
#pragma unroll
    for (int i = 0; i < kPF; ++i) {
      chunk(ring[i], k + i);
      issue(ring[i], k + i + kPF);
    }
  }
  if (a.h_last && dval) {
    for (int r = 0; r < 4; ++r) {
      const int n = 4 * g + r;
      if (n < N) a.h_last[(b * D + d0 + c) * N + n] = H[r];
    }
  }
}

template <typename In, bool GATE>
int launch_ssd_t(const SsdArgs& a, int64_t batch, bool vec, hipStream_t st) {
  const int64_t tiles = (a.D + kTile - 1) / kTile;
  const dim3 grid((unsigned)(tiles * batch));
  if (vec)
    hipLaunchKernelGGL((s6_ssd_kernel<In, GATE, true>), grid, dim3(64), 0, st, a, batch);
  else
    hipLaunchKernelGGL((s6_ssd_kernel<In, GATE, false>), grid, dim3(64), 0, st, a, batch);
  S6_HIP(hipGetLastError(), "s6_ssd_kernel launch");
  return S6_OK;
}

}  // namespace

}  // namespace s6i

using namespace s6i;

extern "C" {

int s6_ssd_scan_fwd_workspace_size(int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate, int in_dtype,
                                   size_t* bytes) {
  if (!bytes) return S6_ERR_NULL;
  int rc = check_common(batch, dim, seqlen, dstate, in_dtype);
  if (rc) return rc;
  if (dstate > 16) return S6_ERR_UNSUPPORTED;
  *bytes = 0;
  return S6_OK;
}

int s6_ssd_scan_fwd(int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate, int in_dtype, const void* x,
                    const void* delta, const float* A, const void* Bm, const void* Cm, const float* Dskip,
                    const void* z, const float* h0, float* y, float* h_last, void* workspace,
                    size_t workspace_bytes, void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  int rc = check_common(batch, dim, seqlen, dstate, in_dtype);
  if (rc) return rc;
  if (dstate > 16) return S6_ERR_UNSUPPORTED;
  const bool work = batch > 0 && dim > 0 && seqlen > 0;
  if (work && (!x || !delta || !A || !Bm || !Cm || !y)) return S6_ERR_NULL;
  const size_t esz = in_dtype == S6_BF16 ? 2 : 4;
  const void* ins[] = {x, delta, Bm, Cm, z};
  for (const void* p : ins)
    if (p && !aligned(p, esz)) return S6_ERR_ALIGN;
  const void* f32s[] = {A, Dskip, h0, y, h_last};
  for (const void* p : f32s)
    if (p && !aligned(p, 4)) return S6_ERR_ALIGN;
  if (batch * ((dim + 15) / 16) > INT32_MAX) return S6_ERR_SHAPE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (batch == 0 || dim == 0) return S6_OK;
  if (seqlen == 0) return h_last ? launch_copy_state(h0, h_last, batch * dim * dstate, st) : S6_OK;
  // 4-token vector path: every row starts on a 4-token boundary and every
  // base pointer is aligned to 4 tokens (and y to 16 bytes).
  bool vec = seqlen % 4 == 0 && aligned(y, 16);
  for (const void* p : ins)
    if (p && !aligned(p, 4 * esz)) vec = false;
  SsdArgs a;
  a.x = x; a.delta = delta; a.z = z; a.Bm = Bm; a.Cm = Cm; a.A = A; a.Dskip = Dskip; a.h0 = h0; a.y = y;
  a.h_last = h_last; a.D = dim; a.L = seqlen; a.N = dstate;
  if (in_dtype == S6_BF16)
    return z ? launch_ssd_t<uint16_t, true>(a, batch, vec, st) : launch_ssd_t<uint16_t, false>(a, batch, vec, st);
  return z ? launch_ssd_t<float, true>(a, batch, vec, st) : launch_ssd_t<float, false>(a, batch, vec, st);
}

}  // extern "C"
