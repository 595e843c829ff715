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
// and turned token-major by an MFMA with the identity.  Products whose
// operands are exact in bf16 (the transposes and the Gram matrix of bf16 B
// and C) run on the bf16 matrix cores; the three with an fp32 operand (V, the
// state) on the fp32 matrix cores, so no operand is rounded below fp32.
#include "s6_internal.h"

namespace s6i {

namespace {

typedef short bf16x4 __attribute__((ext_vector_type(4)));  // 4 bf16 bit patterns (an MFMA operand)
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kQ = 16;                 // tokens per chunk
constexpr int kTile = 16;              // channels per wave
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

// Four tokens of one row as loaded: packed bf16 (uint2) or fp32 (float4).
template <typename In>
struct Four;
template <>
struct Four<uint16_t> {
  uint2 v;
  __device__ __forceinline__ void unpack(float f[4]) const {
    f[0] = bf_lo(v.x); f[1] = bf_hi(v.x); f[2] = bf_lo(v.y); f[3] = bf_hi(v.y);
  }
  __device__ __forceinline__ void pack(const float f[4]) { v.x = pack_bf16(f[0], f[1]); v.y = pack_bf16(f[2], f[3]); }
  __device__ __forceinline__ void keep_if(bool k) { v.x = k ? v.x : 0u; v.y = k ? v.y : 0u; }
};
template <>
struct Four<float> {
  float4 v;
  __device__ __forceinline__ void unpack(float f[4]) const { f[0] = v.x; f[1] = v.y; f[2] = v.z; f[3] = v.w; }
  __device__ __forceinline__ void pack(const float f[4]) { v = make_float4(f[0], f[1], f[2], f[3]); }
  __device__ __forceinline__ void keep_if(bool k) {
    v.x = k ? v.x : 0.0f; v.y = k ? v.y : 0.0f; v.z = k ? v.z : 0.0f; v.w = k ? v.w : 0.0f;
  }
};

// Four tokens of one row at byte offset `off` from a wave-uniform base (the
// tile's first row): one 8- or 16-byte load (VEC: L % 4 == 0, rows aligned;
// groups past the end read the row's last group, masked by the caller), or
// four clamped element loads.
template <typename In, bool VEC>
__device__ __forceinline__ Four<In> load4(const char* __restrict__ base, uint32_t row_off, int64_t t, int64_t L) {
  Four<In> o;
  if constexpr (VEC) {
    const uint32_t tc = (uint32_t)(t < L ? t : L - 4);
    const char* p = base + row_off + tc * (uint32_t)sizeof(In);
    if constexpr (sizeof(In) == 2)
      o.v = *reinterpret_cast<const uint2*>(p);
    else
      o.v = *reinterpret_cast<const float4*>(p);
  } else {
    In e[4];
    for (int j = 0; j < 4; ++j) {
      const uint32_t tj = (uint32_t)(t + j < L ? t + j : L - 1);
      e[j] = *reinterpret_cast<const In*>(base + row_off + tj * (uint32_t)sizeof(In));
    }
    if constexpr (sizeof(In) == 2)
      o.v = make_uint2((uint32_t)e[0] | ((uint32_t)e[1] << 16), (uint32_t)e[2] | ((uint32_t)e[3] << 16));
    else
      o.v = make_float4(e[0], e[1], e[2], e[3]);
  }
  return o;
}

// D += A B on the fp32 matrix cores (16 x 16 x 16 as four 16 x 16 x 4
// products).  Lane 16 g + c holds A[c][4g + j] and B[4g + j][c] in a[j],
// b[j]; D's lane holds D[4g + r][c] in d[r].
__device__ __forceinline__ f32x4 mma_f32(const float a[4], const float b[4], f32x4 d) {
  for (int j = 0; j < 4; ++j) d = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], d, 0, 0, 0);
  return d;
}

// The same product with both operands exact in bf16 (inputs, transposed
// inputs): one bf16 matrix-core instruction, or fp32 products for fp32 data.
template <typename In>
__device__ __forceinline__ f32x4 mma_in(const Four<In>& a, const Four<In>& b, f32x4 d) {
  if constexpr (sizeof(In) == 2) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4, a.v), __builtin_bit_cast(bf16x4, b.v),
                                                      d, 0, 0, 0);
  } else {
    float fa[4], fb[4];
    a.unpack(fa);
    b.unpack(fb);
    return mma_f32(fa, fb, d);
  }
}

// An fp32 operand as the sum of two bf16 parts: hi = bf16(v), lo = bf16(v -
// hi) (v - hi is exact in fp32); hi + lo is within 2^-17 |v| of v.  A product
// with an exact bf16 operand then takes two bf16 matrix-core instructions,
// a product of two split operands three (the lo x lo term, below 2^-32 of
// the product, is left out).
__device__ __forceinline__ void split_bf16(const float v[4], Four<uint16_t>& hi, Four<uint16_t>& lo) {
  hi.pack(v);
  float h[4], r[4];
  hi.unpack(h);
  for (int j = 0; j < 4; ++j) r[j] = v[j] - h[j];
  lo.pack(r);
}

// Raw inputs of one chunk for one lane: 4 tokens of x, delta, z of channel
// c and 4 tokens of B and C of state c.
template <typename In>
struct Raw {
  Four<In> x, dl, z, b, c;
};

// A chunk's results that do not depend on the state entering it.
template <typename In>
struct Front {
  f32x4 Yd;      // tril(G) V
  f32x4 S;       // B^T V
  float P[4];    // e^{a (c_t - r)} of the lane's 4 tokens
  float ct[4];   // C token-major: lane (g, c) holds C[n = 4g + j][t = c] (A operand of C H)
  Four<In> ctp;  // the same packed (exact: C's own values)
  float xv[4];   // x of the lane's 4 tokens (skip term)
  Four<In> z;    // gate input
  float kr;      // e^{a r} = e^{a (c_16 - r)}
  float dec;     // e^{a c_16}
  bool wide;     // a channel of the tile has |a| c_16 > kRangeLog2 (wave-uniform)
};

// Cumulative step of a chunk: lane (g, c) holds tokens 4g .. 4g+3 of channel
// c in dv; cs receives the inclusive cumulative step of those tokens within
// the chunk and total the chunk's sum (lanes c, c+16, c+32, c+48 hold the
// chunk's 4 groups).
__device__ __forceinline__ void chunk_cumsum(const float dv[4], int g, float cs[4], float& total) {
  float q[4];
  q[0] = dv[0];
  q[1] = q[0] + dv[1];
  q[2] = q[1] + dv[2];
  q[3] = q[2] + dv[3];
  const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(q[3]), __float_as_uint(q[3]), false, false);
  const float lo16 = __uint_as_float((unsigned)s16[0]), hi16 = __uint_as_float((unsigned)s16[1]);
  const float pair = lo16 + hi16;
  const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(pair), __float_as_uint(pair), false, false);
  const float lo32 = __uint_as_float((unsigned)s32[0]), hi32 = __uint_as_float((unsigned)s32[1]);
  total = lo32 + hi32;
  const float ex = ((g & 1) ? lo16 : 0.0f) + ((g & 2) ? lo32 : 0.0f);
  for (int j = 0; j < 4; ++j) cs[j] = ex + q[j];
}

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
  // Segments along L (blockIdx.y), seg_len tokens each (a multiple of 32):
  // the state entering segment s is hin[s] ((S, batch, D, N)), or h0 when
  // hin is null (one segment).  State-only pass: agg[s] receives segment s's
  // end state from a zero state, sumdelta[s] (S, batch, D) its summed step.
  int64_t seg_len;
  const float* hin;
  float* agg;
  float* sumdelta;
};

// Staging of 2-chunk groups through LDS (STG): per input one or two 16-byte
// loads per lane cover the group's 32 tokens of the tile's 16 rows in runs of
// 64 (bf16) or 128 (fp32) contiguous bytes, written to LDS and read back per
// chunk in the MFMA layout; the group's y (16 rows x 32 fp32) is collected in
// LDS and written as whole 128-byte lines.
//
// Bank conflicts (gfx950, as measured: 16-byte reads take 16 lanes per cycle
// over 64 banks; 16-byte writes 8 lanes, 8-byte accesses 16 lanes, over 32):
// * bf16 inputs: rows of 64 bytes, the 8-byte slot s (tokens 4s .. 4s+3) of
//   row c stored at slot s ^ ((c >> 1) & 7), each loaded 16-byte piece
//   written as its two 8-byte halves.  The chunk reads (8 bytes of 16
//   consecutive rows per cycle) and the half writes (4 rows x 4 pieces)
//   then meet every bank once.  No padding gives both: 16-byte aligned rows
//   leave 8-byte reads of 16 rows at most 8 distinct bank pairs.
// * fp32 inputs: rows padded to 36 floats.
// * y: rows of 32 floats, the 16-byte piece p of row c stored at p ^ (c & 7),
//   so that the writes of 8 channels and the reads of two rows each cover
//   the banks once.
constexpr int kGT = 2 * kQ;                    // tokens per staged group
template <typename In>
struct Stg {
  static constexpr int kPitch = sizeof(In) == 2 ? 32 : 36;  // input row pitch (elements)
  static constexpr int kLoads = sizeof(In) / 2;             // 16-byte loads per lane per input
  static constexpr int kIn = 16 * kPitch;                   // elements per input tile
};
constexpr int kYPitch = 32;                    // y row pitch (floats)
// element offset of the 4 bf16 tokens in slot s of staged row c
__device__ __forceinline__ int stg_slot(int c, int s) { return c * 32 + 4 * (s ^ ((c >> 1) & 7)); }
// float offset of the 16-byte piece p of y row c
__device__ __forceinline__ int y_piece(int c, int p) { return c * kYPitch + 4 * (p ^ (c & 7)); }

template <typename In, bool GATE, bool VEC, bool STG>
__global__ void __launch_bounds__(64, 3) s6_ssd_kernel(SsdArgs a, int64_t batch) {
  __shared__ float lds[3 * kQ * kTile];  // the unseparated path's G, cumulative steps and inputs
  __shared__ __align__(16) In sin[STG ? 5 * Stg<In>::kIn : 1];  // staged inputs: x, delta, z, B, C
  __shared__ __align__(16) float sy[STG ? 16 * kYPitch : 1];     // staged y of a group

  const int lane = threadIdx.x;
  const int g = lane >> 4, c = lane & 15;
  const int64_t b = blockIdx.x % batch;              // batch rows spread over the XCDs
  const int64_t d0 = (blockIdx.x / batch) * kTile;
  const int64_t D = a.D, L = a.L, N = a.N;
  const bool dval = d0 + c < D;
  const int cl = dval ? c : (int)(D - 1 - d0);       // clamped channel within the tile (never stored)
  const bool nval = c < N;
  const int nc = nval ? c : (int)N - 1;              // clamped state (its B and C rows are zeroed)

  // wave-uniform bases of the tile's rows and 32-bit lane offsets
  constexpr uint32_t esz = sizeof(In);
  const char* xb = static_cast<const char*>(a.x) + (b * D + d0) * L * esz;
  const char* db = static_cast<const char*>(a.delta) + (b * D + d0) * L * esz;
  const char* zb = GATE ? static_cast<const char*>(a.z) + (b * D + d0) * L * esz : nullptr;
  const char* bb = static_cast<const char*>(a.Bm) + b * N * L * esz;
  const char* cb = static_cast<const char*>(a.Cm) + b * N * L * esz;
  float* yb = a.y + (b * D + d0) * L;
  const uint32_t xo = (uint32_t)cl * (uint32_t)L * esz;
  const uint32_t no = (uint32_t)nc * (uint32_t)L * esz;
  const uint32_t yo4 = (uint32_t)c * (uint32_t)L;
  const float a2 = a.A[d0 + cl] * kLog2e;             // a log2(e)
  const float dsk = a.Dskip ? a.Dskip[d0 + cl] : 0.0f;

  // identity (B operand): lane (g, c) holds I[4g + j][c]; lower-triangle mask
  // of G (A layout: lane (g, c) holds G[t = c][s = 4g + j], kept for s <= t)
  Four<In> ident;
  float tri[4];
  {
    float v[4];
    for (int j = 0; j < 4; ++j) {
      v[j] = (4 * g + j == c) ? 1.0f : 0.0f;
      tri[j] = (4 * g + j <= c) ? 1.0f : 0.0f;
    }
    ident.pack(v);
  }
  // this wave's segment of the sequence: tokens [tb, te)
  const int64_t seg = blockIdx.y;
  const int64_t tb = seg * a.seg_len;
  const int64_t te = tb + a.seg_len < L ? tb + a.seg_len : L;
  // state tile: lane (g, c) holds H[n = 4g + r][d = c]
  float H[4];
  {
    const float* h_in = a.hin ? a.hin + seg * batch * D * N : a.h0;
    for (int r = 0; r < 4; ++r) {
      const int n = 4 * g + r;
      H[r] = (h_in && dval && n < N) ? h_in[(b * D + d0 + c) * N + n] : 0.0f;
    }
  }

  auto issue = [&](Raw<In>& rw, int64_t k) {
    const int64_t t = k * kQ + 4 * g;
    rw.x = load4<In, VEC>(xb, xo, t, L);
    rw.dl = load4<In, VEC>(db, xo, t, L);
    if constexpr (GATE) rw.z = load4<In, VEC>(zb, xo, t, L);
    rw.b = load4<In, VEC>(bb, no, t, L);
    rw.c = load4<In, VEC>(cb, no, t, L);
  };

  // Inputs of chunk k as values; mask: tokens past the end get a zero step,
  // input, B and C (the state then passes through unchanged).  B and C rows
  // of states >= N are zero.  Returns the cumulative step within the chunk
  // (inclusive) in cs and its total.
  auto prep = [&](Raw<In>& rw, int64_t k, bool mask, float xv[4], float dv[4], float cs[4], float& total) {
    rw.x.unpack(xv);
    rw.dl.unpack(dv);
    rw.b.keep_if(nval);
    rw.c.keep_if(nval);
    if (mask) {
      const int64_t t0 = k * kQ + 4 * g;
      float bv[4], cv[4];
      rw.b.unpack(bv);
      rw.c.unpack(cv);
      for (int j = 0; j < 4; ++j) {
        const bool ok = t0 + j < L;
        xv[j] = ok ? xv[j] : 0.0f;
        dv[j] = ok ? dv[j] : 0.0f;
        bv[j] = ok ? bv[j] : 0.0f;
        cv[j] = ok ? cv[j] : 0.0f;
      }
      rw.b.pack(bv);
      rw.c.pack(cv);
    }
    chunk_cumsum(dv, g, cs, total);
  };

  // B and C token-major (an MFMA with the identity) and G^T = Bmat Cmat^T:
  // lane (g, c) gets G[t = c][s = 4g + r], the A operand of tril(G) V.
  auto gram = [&](const Raw<In>& rw, float ct[4], float gm[4], Four<In>& ctp) {
    const f32x4 z4 = {0.0f, 0.0f, 0.0f, 0.0f};
    const f32x4 btf = mma_in<In>(rw.b, ident, z4);
    const f32x4 ctf = mma_in<In>(rw.c, ident, z4);
    Four<In> bt;
    float bv[4] = {btf[0], btf[1], btf[2], btf[3]};
    for (int j = 0; j < 4; ++j) ct[j] = ctf[j];
    bt.pack(bv);
    ctp.pack(ct);
    const f32x4 gt = mma_in<In>(bt, ctp, z4);
    for (int j = 0; j < 4; ++j) gm[j] = gt[j] * tri[j];
  };

  // Everything of chunk k that does not depend on the state entering it,
  // with the decays separated around the chunk's midpoint (the values are
  // meaningless when f.wide; the chunk is then recomputed by `exact`).
  auto front = [&](Raw<In>& rw, int64_t k, bool mask) {
    Front<In> f;
    float dv[4], cs[4], total;
    prep(rw, k, mask, f.xv, dv, cs, total);
    f.wide = __builtin_amdgcn_ballot_w64(!(fabsf(a2) * total <= kRangeLog2)) != 0;
    const float ah = a2 * (0.5f * total);
    float V[4];
    for (int j = 0; j < 4; ++j) {
      const float u = __builtin_fmaf(a2, cs[j], -ah);  // a (c_t - r) in log2 units
      f.P[j] = fast_exp2(u);
      V[j] = (dv[j] * f.xv[j]) * fast_exp2(-u);
    }
    f.kr = fast_exp2(ah);
    f.dec = fast_exp2(a2 * total);
    float gm[4];
    gram(rw, f.ct, gm, f.ctp);
    const f32x4 z4 = {0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (sizeof(In) == 2) {
      // bf16 matrix cores with V and tril(G) split into two bf16 parts; B
      // is its own bf16 values
      Four<In> vh, vl, gh, gl;
      split_bf16(V, vh, vl);
      split_bf16(gm, gh, gl);
      f.Yd = mma_in<In>(gh, vh, z4);  // tril(G) V
      f.Yd = mma_in<In>(gh, vl, f.Yd);
      f.Yd = mma_in<In>(gl, vh, f.Yd);
      f.S = mma_in<In>(rw.b, vh, z4);  // B^T V
      f.S = mma_in<In>(rw.b, vl, f.S);
    } else {
      float bn[4];
      rw.b.unpack(bn);
      f.Yd = mma_f32(gm, V, z4);   // tril(G) V
      f.S = mma_f32(bn, V, z4);    // B^T V
    }
    f.z = rw.z;
    return f;
  };

  // slot >= 0: chunk `slot` of a staged group, y goes to the LDS staging.
  auto output = [&](const Four<In>& zr, const float P[4], const f32x4& Y, const float xv[4], int64_t k, bool mask,
                    int slot) {
    const int64_t t0 = k * kQ + 4 * g;
    float zv[4];
    if constexpr (GATE) zr.unpack(zv);
    float yo[4];
    for (int r = 0; r < 4; ++r) {
      float yy = __builtin_fmaf(P[r], Y[r], dsk * xv[r]);
      if constexpr (GATE) yy *= silu(zv[r]);
      yo[r] = yy;
    }
    if (STG && slot >= 0) {
      *reinterpret_cast<float4*>(sy + y_piece(c, slot * 4 + g)) = make_float4(yo[0], yo[1], yo[2], yo[3]);
      return;
    }
    if (dval && (!mask || t0 < L)) {
      float* yp = yb + yo4 + (uint32_t)t0;
      if constexpr (VEC) {
        *reinterpret_cast<float4*>(yp) = make_float4(yo[0], yo[1], yo[2], yo[3]);
      } else {
        for (int r = 0; r < 4; ++r)
          if (t0 + r < L) yp[r] = yo[r];
      }
    }
  };

  // The state-dependent rest of a chunk: C (e^{a r} H) joins tril(G) V, the
  // state advances, the output is written.
  auto back = [&](const Front<In>& f, int64_t k, bool mask, int slot) {
    float hs[4];
    for (int r = 0; r < 4; ++r) hs[r] = H[r] * f.kr;
    f32x4 Y;
    if constexpr (sizeof(In) == 2) {
      Four<In> hh, hl;
      split_bf16(hs, hh, hl);
      Y = mma_in<In>(f.ctp, hh, f.Yd);
      Y = mma_in<In>(f.ctp, hl, Y);
    } else {
      Y = mma_f32(f.ct, hs, f.Yd);
    }
    for (int r = 0; r < 4; ++r) H[r] = __builtin_fmaf(f.dec, H[r], f.kr * f.S[r]);
    output(f.z, f.P, Y, f.xv, k, mask, slot);
  };

  // Chunk k without the separation (reloads its inputs): decays to the
  // chunk's ends (each <= 1) for the carried state and its update, per-pair
  // decays within the chunk.
  auto exact = [&](int64_t k, bool mask, int slot) {
    Raw<In> rw;
    issue(rw, k);
    float xv[4], dv[4], cs[4], total;
    prep(rw, k, mask, xv, dv, cs, total);
    float P[4], W[4], v[4];
    for (int j = 0; j < 4; ++j) {
      v[j] = dv[j] * xv[j];
      P[j] = fast_exp2(a2 * cs[j]);
      W[j] = v[j] * fast_exp2(a2 * (total - cs[j]));
    }
    float ct[4], gm[4], bn[4];
    Four<In> ctp;
    gram(rw, ct, gm, ctp);
    rw.b.unpack(bn);
    const f32x4 z4 = {0.0f, 0.0f, 0.0f, 0.0f};
    const f32x4 Yo = mma_f32(ct, H, z4);
    const f32x4 S = mma_f32(bn, W, z4);
    const float dec = fast_exp2(a2 * total);
    for (int r = 0; r < 4; ++r) H[r] = __builtin_fmaf(dec, H[r], S[r]);
    float* sg = lds;                 // [t][s]
    float* sc = lds + kQ * kTile;    // [channel][token] cumulative step
    float* sv = sc + kQ * kTile;     // [channel][token] step times input
    __syncthreads();
    for (int r = 0; r < 4; ++r) sg[c * kQ + 4 * g + r] = gm[r];
    for (int j = 0; j < 4; ++j) {
      sc[c * kQ + 4 * g + j] = cs[j];
      sv[c * kQ + 4 * g + j] = v[j];
    }
    __syncthreads();
    f32x4 Y;
    float one[4];
    for (int r = 0; r < 4; ++r) {
      const int t = 4 * g + r;
      float acc = 0.0f;
      for (int s = 0; s <= t; ++s)
        acc = __builtin_fmaf(sg[t * kQ + s] * fast_exp2(a2 * (sc[c * kQ + t] - sc[c * kQ + s])), sv[c * kQ + s], acc);
      Y[r] = __builtin_fmaf(P[r], Yo[r], acc);
      one[r] = 1.0f;
    }
    output(rw.z, one, Y, xv, k, mask, slot);
  };

  // One chunk's back half; a chunk flagged wide is recomputed exactly from
  // the state it entered with (the fast results are discarded).
  auto finish = [&](const Front<In>& f, int64_t k, bool mask, int slot = -1) {
    const float h0[4] = {H[0], H[1], H[2], H[3]};
    back(f, k, mask, slot);
    if (f.wide) {
      for (int r = 0; r < 4; ++r) H[r] = h0[r];
      exact(k, mask, slot);
    }
  };

  const int64_t nch = (te + kQ - 1) / kQ;  // chunks [tb / kQ, nch) of this segment
  int64_t k = tb / kQ;
  if constexpr (STG) {
    // Whole 32-token groups through the LDS staging; the next group's loads
    // are in flight while a group is computed.
    constexpr int NL = Stg<In>::kLoads;
    constexpr int RPL = 16 / NL;                 // rows covered by one load instruction
    constexpr int LPR = 64 / RPL;                // lanes per row
    constexpr int EPP = 16 / (int)sizeof(In);    // elements per 16-byte piece
    const int prow = lane / LPR, ppc = lane % LPR;  // this lane's row (within a load) and piece
    u32x4 stage[5][NL];
    const char* bases[5] = {xb, db, GATE ? zb : xb, bb, cb};
    auto stage_rows = [&](int q, int in) {       // tile row this lane loads for load q of input in
      const int r = prow + q * RPL;
      if (in >= 3) return (uint32_t)(r < N ? r : N - 1);
      return (uint32_t)(d0 + r < D ? r : (int)(D - 1 - d0));
    };
    auto load_group = [&](int64_t G) {
      for (int in = 0; in < 5; ++in) {
        if (!GATE && in == 2) continue;
        for (int q = 0; q < NL; ++q) {
          const uint32_t off = stage_rows(q, in) * (uint32_t)L * esz + (uint32_t)(G * kGT + ppc * EPP) * esz;
          stage[in][q] = *reinterpret_cast<const u32x4*>(bases[in] + off);
        }
      }
    };
    const int64_t g0 = tb / kGT, ngrp = te / kGT;  // whole groups of the segment
    if (ngrp > g0) load_group(g0);
    for (int64_t G = g0; G < ngrp; ++G) {
      __syncthreads();  // the previous group's reads of the staging are done
      for (int in = 0; in < 5; ++in) {
        if (!GATE && in == 2) continue;
        for (int q = 0; q < NL; ++q) {
          const int row = prow + q * RPL;
          if constexpr (sizeof(In) == 2) {
            In* t = sin + in * Stg<In>::kIn;
            *reinterpret_cast<uint2*>(t + stg_slot(row, 2 * ppc)) = make_uint2(stage[in][q].x, stage[in][q].y);
            *reinterpret_cast<uint2*>(t + stg_slot(row, 2 * ppc + 1)) = make_uint2(stage[in][q].z, stage[in][q].w);
          } else {
            *reinterpret_cast<u32x4*>(sin + in * Stg<In>::kIn + row * Stg<In>::kPitch + ppc * EPP) = stage[in][q];
          }
        }
      }
      if (G + 1 < ngrp) load_group(G + 1);
      __syncthreads();
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        // the lane's 4 tokens of chunk j: row c (channel or state), tokens 16 j + 4 g ..
        Raw<In> rw;
        const int eo = sizeof(In) == 2 ? stg_slot(c, 4 * j + g) : c * Stg<In>::kPitch + j * kQ + 4 * g;
        Four<In>* dst[5] = {&rw.x, &rw.dl, &rw.z, &rw.b, &rw.c};
        for (int in = 0; in < 5; ++in) {
          if (!GATE && in == 2) continue;
          const In* src = sin + in * Stg<In>::kIn + eo;
          if constexpr (sizeof(In) == 2)
            dst[in]->v = *reinterpret_cast<const uint2*>(src);
          else
            dst[in]->v = *reinterpret_cast<const float4*>(src);
        }
        const Front<In> f = front(rw, G * 2 + j, false);
        finish(f, G * 2 + j, false, j);
      }
      __syncthreads();
      // y of the group: 16 rows x 32 tokens, 8 lanes x 16 bytes per row
      for (int h = 0; h < 2; ++h) {
        const int r = (lane >> 3) + 8 * h, pc = lane & 7;
        if (d0 + r < D)
          *reinterpret_cast<float4*>(yb + (uint32_t)r * (uint32_t)L + (uint32_t)(G * kGT + pc * 4)) =
              *reinterpret_cast<const float4*>(sy + y_piece(r, pc));
      }
    }
    k = ngrp > g0 ? ngrp * 2 : k;
  }
  // Chunks not covered by the staging (all of them without it; otherwise the
  // last one or two), directly from global memory; tokens past the end masked.
  for (; k < nch; ++k) {
    Raw<In> rw;
    issue(rw, k);
    const Front<In> f = front(rw, k, true);
    finish(f, k, true);
  }
  if (a.h_last && dval && seg == (int64_t)gridDim.y - 1) {
    for (int r = 0; r < 4; ++r) {
      const int n = 4 * g + r;
      if (n < N) a.h_last[(b * D + d0 + c) * N + n] = H[r];
    }
  }
}

// State-only pass of a segmented scan (segments 0 .. gridDim.y - 1, every one
// whole: seg_len tokens): the segment's end state from a zero state,
// H' = e^{a c_16} H + B^T W per chunk with W_s = Delta_s x_s e^{a (c_16 - c_s)}
// (each decay <= 1 for a <= 0, so no range split is needed), and its summed
// step (compensated).  Same lane layout as s6_ssd_kernel.  Two register sets
// of kPB chunks' loads alternate, so a set's loads are issued kPB to 2 kPB
// chunks ahead of their use (loads past the segment reread its last chunk and
// are not used).
template <typename In, bool VEC>
__global__ void __launch_bounds__(64) s6_ssd_state_kernel(SsdArgs a, int64_t batch) {
  const int lane = threadIdx.x;
  const int g = lane >> 4, c = lane & 15;
  const int64_t b = blockIdx.x % batch;
  const int64_t d0 = (blockIdx.x / batch) * kTile;
  const int64_t D = a.D, L = a.L, N = a.N;
  const bool dval = d0 + c < D;
  const int cl = dval ? c : (int)(D - 1 - d0);
  const bool nval = c < N;
  const int nc = nval ? c : (int)N - 1;
  constexpr uint32_t esz = sizeof(In);
  const char* xb = static_cast<const char*>(a.x) + (b * D + d0) * L * esz;
  const char* db = static_cast<const char*>(a.delta) + (b * D + d0) * L * esz;
  const char* bb = static_cast<const char*>(a.Bm) + b * N * L * esz;
  const uint32_t xo = (uint32_t)cl * (uint32_t)L * esz;
  const uint32_t no = (uint32_t)nc * (uint32_t)L * esz;
  const float a2 = a.A[d0 + cl] * kLog2e;
  const int64_t seg = blockIdx.y;
  const int64_t kb = seg * a.seg_len / kQ, ke = (seg + 1) * a.seg_len / kQ;
  float H[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  float dsum = 0.0f, dcomp = 0.0f;
  constexpr int kPB = 4;  // chunks per register set
  Four<In> px[2][kPB], pd[2][kPB], pb[2][kPB];
  auto issue = [&](auto setc, int64_t k0) {
    constexpr int SET = decltype(setc)::value;
#pragma unroll
    for (int i = 0; i < kPB; ++i) {
      const int64_t k = k0 + i < ke ? k0 + i : ke - 1;
      const int64_t t = k * kQ + 4 * g;
      px[SET][i] = load4<In, VEC>(xb, xo, t, L);
      pd[SET][i] = load4<In, VEC>(db, xo, t, L);
      pb[SET][i] = load4<In, VEC>(bb, no, t, L);
    }
  };
  auto compute = [&](auto setc, int64_t k0) {
    constexpr int SET = decltype(setc)::value;
#pragma unroll
    for (int i = 0; i < kPB; ++i) {
      if (k0 + i >= ke) break;  // uniform
      float xv[4], dv[4], bn[4];
      px[SET][i].unpack(xv);
      pd[SET][i].unpack(dv);
      pb[SET][i].keep_if(nval);
      pb[SET][i].unpack(bn);
      float cs[4], total;
      chunk_cumsum(dv, g, cs, total);
      float W[4];
      for (int j = 0; j < 4; ++j) W[j] = (dv[j] * xv[j]) * fast_exp2(a2 * (total - cs[j]));
      const f32x4 z4 = {0.0f, 0.0f, 0.0f, 0.0f};
      // B^T W: lane (g, c) gets states 4g + r of channel c
      f32x4 S;
      if constexpr (sizeof(In) == 2) {
        Four<In> wh, wl;
        split_bf16(W, wh, wl);
        S = mma_in<In>(pb[SET][i], wh, z4);
        S = mma_in<In>(pb[SET][i], wl, S);
      } else {
        S = mma_f32(bn, W, z4);
      }
      const float dec = fast_exp2(a2 * total);
      for (int r = 0; r < 4; ++r) H[r] = __builtin_fmaf(dec, H[r], S[r]);
      const float t = dsum + total;
      dcomp += (fabsf(dsum) >= fabsf(total)) ? (dsum - t) + total : (total - t) + dsum;
      dsum = t;
    }
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  issue(S0{}, kb);
  issue(S1{}, kb + kPB);
  for (int64_t k0 = kb; k0 < ke; k0 += 2 * kPB) {
    compute(S0{}, k0);
    issue(S0{}, k0 + 2 * kPB);
    compute(S1{}, k0 + kPB);
    issue(S1{}, k0 + 3 * kPB);
  }
  if (dval) {
    const int64_t nstate = batch * D * N;
    for (int r = 0; r < 4; ++r) {
      const int n = 4 * g + r;
      if (n < N) a.agg[seg * nstate + (b * D + d0 + c) * N + n] = H[r];
    }
    if (g == 0) a.sumdelta[seg * batch * D + b * D + d0 + c] = dsum + dcomp;
  }
}

// Segments along L for few long rows: when the batch x tile waves fill less
// than half of the wave slots (3 per SIMD), the sequence is cut into
// segments of whole 32-token groups, as many as fill the slots twice; their
// carries go to the caller's workspace: end states from zero and summed
// steps (S - 1 of each), incoming states (S).
struct SsdPlan {
  int64_t S, seg_len;
  size_t agg, sd, hin, total;
};
SsdPlan ssd_plan(int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate) {
  SsdPlan p{1, seqlen, 0, 0, 0, 0};
  const int64_t waves = batch * ((dim + kTile - 1) / kTile);
  const int64_t slots = (int64_t)cu_count() * 4 * 3;
  if (waves > 0 && 2 * waves <= slots) {
    int64_t S = 2 * slots / waves;
    const int64_t max_s = (seqlen + kGT - 1) / kGT;
    if (S > max_s) S = max_s;
    if (S > 1) {
      const int64_t sl = ((seqlen + S - 1) / S + kGT - 1) / kGT * kGT;
      p.seg_len = sl;
      p.S = (seqlen + sl - 1) / sl;
    }
  }
  if (p.S > 1) {
    auto up = [](size_t v) { return (v + 255) & ~(size_t)255; };
    const size_t nstate = (size_t)batch * dim * dstate;
    p.agg = 0;
    p.sd = up((size_t)(p.S - 1) * nstate * sizeof(float));
    p.hin = p.sd + up((size_t)(p.S - 1) * batch * dim * sizeof(float));
    p.total = p.hin + up((size_t)p.S * nstate * sizeof(float));
  }
  return p;
}

template <typename In>
int launch_ssd_state(const SsdArgs& a, int64_t batch, bool vec, int64_t segs, hipStream_t st) {
  const int64_t tiles = (a.D + kTile - 1) / kTile;
  const dim3 grid((unsigned)(tiles * batch), (unsigned)segs);
  if (vec)
    hipLaunchKernelGGL((s6_ssd_state_kernel<In, true>), grid, dim3(64), 0, st, a, batch);
  else
    hipLaunchKernelGGL((s6_ssd_state_kernel<In, false>), grid, dim3(64), 0, st, a, batch);
  S6_HIP(hipGetLastError(), "s6_ssd_state_kernel launch");
  return S6_OK;
}

template <typename In, bool GATE>
int launch_ssd_t(const SsdArgs& a, int64_t batch, int64_t segs, bool vec, bool stg, hipStream_t st) {
  const int64_t tiles = (a.D + kTile - 1) / kTile;
  const dim3 grid((unsigned)(tiles * batch), (unsigned)segs);
  if (stg)
    hipLaunchKernelGGL((s6_ssd_kernel<In, GATE, true, true>), grid, dim3(64), 0, st, a, batch);
  else if (vec)
    hipLaunchKernelGGL((s6_ssd_kernel<In, GATE, true, false>), grid, dim3(64), 0, st, a, batch);
  else
    hipLaunchKernelGGL((s6_ssd_kernel<In, GATE, false, false>), grid, dim3(64), 0, st, a, batch);
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
  if (batch == 0 || dim == 0 || seqlen == 0) return S6_OK;
  *bytes = ssd_plan(batch, dim, seqlen, dstate).total;
  return S6_OK;
}

int s6_ssd_scan_fwd(int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate, int in_dtype, const void* x,
                    const void* delta, const float* A, const void* Bm, const void* Cm, const float* Dskip,
                    const void* z, const float* h0, float* y, float* h_last, void* workspace,
                    size_t workspace_bytes, void* stream) {
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
  // LDS staging of 32-token groups: every row starts 16-byte aligned
  bool stg = vec && (seqlen * (int64_t)esz) % 16 == 0;
  for (const void* p : ins)
    if (p && !aligned(p, 16)) stg = false;
  const SsdPlan pl = ssd_plan(batch, dim, seqlen, dstate);
  if (pl.total > 0 && (!workspace || workspace_bytes < pl.total)) return S6_ERR_WORKSPACE;
  if (pl.total > 0 && !aligned(workspace, 256)) return S6_ERR_ALIGN;
  SsdArgs a;
  memset(&a, 0, sizeof(a));
  a.x = x; a.delta = delta; a.z = z; a.Bm = Bm; a.Cm = Cm; a.A = A; a.Dskip = Dskip; a.h0 = h0; a.y = y;
  a.h_last = h_last; a.D = dim; a.L = seqlen; a.N = dstate; a.seg_len = pl.seg_len;
  const bool bf = in_dtype == S6_BF16;
  if (pl.S > 1) {
    // pass 1: end states (from zero) and summed steps of all segments but the
    // last; the fold gives every segment's incoming state
    char* wp = static_cast<char*>(workspace);
    SsdArgs g = a;
    g.agg = reinterpret_cast<float*>(wp + pl.agg);
    g.sumdelta = reinterpret_cast<float*>(wp + pl.sd);
    float* hin = reinterpret_cast<float*>(wp + pl.hin);
    rc = bf ? launch_ssd_state<uint16_t>(g, batch, vec, pl.S - 1, st) : launch_ssd_state<float>(g, batch, vec, pl.S - 1, st);
    if (rc == S6_OK)
      rc = launch_fold_carries(A, h0, g.agg, g.sumdelta, hin, nullptr, batch, dim, dstate, pl.S, pl.S - 1, st, true);
    if (rc) return rc;
    a.hin = hin;
  }
  if (bf)
    return z ? launch_ssd_t<uint16_t, true>(a, batch, pl.S, vec, stg, st)
             : launch_ssd_t<uint16_t, false>(a, batch, pl.S, vec, stg, st);
  return z ? launch_ssd_t<float, true>(a, batch, pl.S, vec, stg, st) : launch_ssd_t<float, false>(a, batch, pl.S, vec, stg, st);
}

}  // extern "C"
