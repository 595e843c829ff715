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
//    wave w = states [4w, 4w+4).  A, the state h and the per-lane partial
//    output stay in VGPRs; the (batch, D, L, N) state is never written.
//  * B and C of a token are the same for all 64 channels of a wave.  For 4
//    tokens x 4 states they sit in one VGPR per tensor, replicated in each
//    16-lane row (lane x of a row holds token x/4, state x%4), and every use
//    reads them through a DPP row_newbcast operand folded into the multiply:
//    no LDS traffic and no extra instruction.  They are loaded from the bf16
//    or fp32 inputs one chunk ahead.
//  * x, delta, z are staged per chunk of kT tokens into double-buffered,
//    channel-major LDS tiles with coalesced row loads issued one chunk ahead;
//    the token loop reads its lane's 16 deltas and x values in bulk, so it
//    contains no memory waits.  Tokens past the end of the sequence are
//    staged as delta = 0, which leaves the state unchanged, so every chunk
//    runs the full unrolled loop.
//  * Each wave writes its partial sum over its 4 states per token into LDS;
//    after the chunk the G waves finalise the 64 x kT outputs (sum of G
//    partials, skip term, gate), each lane 4 consecutive tokens of one
//    channel, stored as 16-byte writes.  Two barriers per chunk.
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

#include <type_traits>
#include <utility>

#include "s6.h"

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kCW = 32;            // channels per workgroup
constexpr int kT = 16;             // tokens per chunk
constexpr int kP = kT;             // LDS tile pitch in floats (channel-major [c][t], swizzled)
constexpr int kMaxN = 32;          // largest dstate supported

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

// Value of lane J of this lane's 16-lane row (DPP row_newbcast).  Used as an
// operand of a multiply, the compiler folds it into v_mul_f32_dpp.
template <int J>
__device__ __forceinline__ float row_bcast(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x150 + J,
                                                               0xf, 0xf, true));
}

// Offset (floats) of the 4-token group `grp` of channel row c in a
// channel-major tile of pitch kT = 16.  The group index is XORed with
// (c >> 1) & 3 so that 16-byte reads of one group by 8 consecutive lanes
// fall on 8 distinct 4-bank groups (no padding needed).
__device__ __forceinline__ int tsw(int c, int grp) { return c * kP + ((grp ^ ((c >> 1) & 3)) << 2); }

// -------------------------------------------------------------------- scan --
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
  float* sumdelta;        // kModeState: per-segment sum of delta (S, batch, D) or null
  int64_t D, L, N;
  int64_t seg_len;        // tokens per segment (multiple of kT); segment = blockIdx.z
  int64_t hinit_stride;   // elements between segments in hinit (0: same for all)
  int64_t hout_stride;    // elements between segments in hout
  int64_t hout_last_only; // 1: only the last segment writes hout (at offset 0)
};

// One chunk of a (rows, L) tensor for the kCW channels of a workgroup: kCW
// rows x kT tokens, cut into pieces of VEC elements (16 bytes, or single
// elements when VEC == 1).
template <typename In, int VEC>
struct Stage {
  static constexpr int kPieces = kCW * (kT / VEC);
  using Raw = typename std::conditional<VEC == 1, In, u32x4>::type;

  __device__ __forceinline__ static bool valid(int p, int64_t rows_valid, int64_t t0, int64_t tend) {
    const int c = p / (kT / VEC);
    const int v = p - c * (kT / VEC);
    return c < rows_valid && t0 + v * VEC < tend;
  }

  // Unconditional load (a piece outside the tensor reads element 0 instead,
  // and is replaced by zeros in store()): a conditional load would make the
  // compiler wait for it at once and defeat the prefetch.
  __device__ __forceinline__ static Raw load(gptr<In> src, int p, int64_t row0, int64_t rows_valid,
                                             int64_t L, int64_t t0, int64_t tend) {
    const int c = p / (kT / VEC);
    const int v = p - c * (kT / VEC);
    const int64_t idx = valid(p, rows_valid, t0, tend) ? (row0 + c) * L + t0 + v * VEC : 0;
    if constexpr (VEC == 1) return src[idx];
    else return *reinterpret_cast<gptr<u32x4>>(src + idx);
  }

  // Same layout, values kept in the input type (the gate tile).
  __device__ __forceinline__ static void store_raw(In* __restrict__ tile, int p, const Raw& r, bool ok) {
    const int c = p / (kT / VEC);
    const int v = p - c * (kT / VEC);
    if constexpr (VEC == 1) {
      tile[tsw(c, v >> 2) + (v & 3)] = ok ? r : In(0);
    } else {
      const In* e = reinterpret_cast<const In*>(&r);
#pragma unroll
      for (int k = 0; k < VEC; k += 4) {
        In* dst = tile + tsw(c, (v * VEC + k) >> 2);
#pragma unroll
        for (int m = 0; m < 4; ++m) dst[m] = ok ? e[k + m] : In(0);
      }
    }
  }

  __device__ __forceinline__ static void store(float* __restrict__ tile, int p, const Raw& r, bool ok) {
    const int c = p / (kT / VEC);
    const int v = p - c * (kT / VEC);
    if constexpr (VEC == 1) {
      tile[tsw(c, v >> 2) + (v & 3)] = ok ? to_f32(r) : 0.0f;
    } else {
      const In* e = reinterpret_cast<const In*>(&r);
#pragma unroll
      for (int k = 0; k < VEC; k += 4)
        *reinterpret_cast<float4*>(tile + tsw(c, (v * VEC + k) >> 2)) =
            ok ? make_float4(to_f32(e[k]), to_f32(e[k + 1]), to_f32(e[k + 2]), to_f32(e[k + 3]))
               : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
};

// B and C of one chunk: per tensor 4*W state rows (states beyond N are zero)
// of kT tokens, cut into VEC-element pieces.  In LDS they are laid out as
// the DPP operands want them: for token group g (4 tokens), wave w and row
// parity r (state pair 4w + 2r, 4w + 2r + 1), 16 slots: B of token k, state
// pair member j at slot 2k + j, C at slot 8 + 2k + j.
template <typename In, int VEC, int W>
struct StageBC {
  static constexpr int kPiecesT = 4 * W * (kT / VEC);  // per tensor
  static constexpr int kPieces = 2 * kPiecesT;
  static constexpr int kFloats = (kT / 4) * W * 2 * 16;  // LDS floats per chunk
  using Raw = typename std::conditional<VEC == 1, In, u32x4>::type;

  __device__ __forceinline__ static bool valid(int p, int64_t N, int64_t t0, int64_t tend) {
    const int q = p % kPiecesT;
    const int n = q / (kT / VEC);
    const int v = q - n * (kT / VEC);
    return n < N && t0 + v * VEC < tend;
  }

  __device__ __forceinline__ static Raw load(gptr<In> Bm, gptr<In> Cm, int p, int64_t b, int64_t N,
                                             int64_t L, int64_t t0, int64_t tend) {
    const int q = p % kPiecesT;
    const int n = q / (kT / VEC);
    const int v = q - n * (kT / VEC);
    gptr<In> M = (p < kPiecesT) ? Bm : Cm;
    const int64_t idx = valid(p, N, t0, tend) ? (b * N + n) * L + t0 + v * VEC : 0;
    if constexpr (VEC == 1) return M[idx];
    else return *reinterpret_cast<gptr<u32x4>>(M + idx);
  }

  // LDS position of slot x of (group g, wave w, row parity r).  The slot is
  // XORed with a (g, w)-dependent mask so that the scattered writes of one
  // instruction fall on distinct banks; readers apply the same mask, so
  // lane x still receives slot x.
  __device__ __forceinline__ static int pos(int g, int w, int r, int x) {
    return ((g * W + w) * 2 + r) * 16 + (x ^ (((w & 3) << 2) ^ (((g >> 1) & 1) << 1)));
  }
  __device__ __forceinline__ static int slot(int tens, int n, int j) {
    const int g = j >> 2, k = j & 3;
    const int w = n >> 2, r = (n >> 1) & 1, m = n & 1;
    return pos(g, w, r, tens * 8 + 2 * k + m);
  }

  __device__ __forceinline__ static void store(float* __restrict__ bcs, int p, const Raw& r, bool ok) {
    const int tens = p / kPiecesT;
    const int q = p % kPiecesT;
    const int n = q / (kT / VEC);
    const int v = q - n * (kT / VEC);
    if constexpr (VEC == 1) {
      bcs[slot(tens, n, v)] = ok ? to_f32(r) : 0.0f;
    } else {
      const In* e = reinterpret_cast<const In*>(&r);
#pragma unroll
      for (int k = 0; k < VEC; ++k) bcs[slot(tens, n, v * VEC + k)] = ok ? to_f32(e[k]) : 0.0f;
    }
  }
};

// Product of v with lane J of this lane's 16-lane row (v_mul_f32_dpp).
template <int J>
__device__ __forceinline__ float mul_bc(float bc, float v) { return row_bcast<J>(bc) * v; }

// Value of lane (l ^ 16) -- the other state pair of the same channel -- via
// the LDS crossbar (ds_swizzle, bit mode, xor mask 16).
__device__ __forceinline__ float swap_rows(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));
}

// One group of 4 tokens for this lane's 2 states.  dl/xv: the lane's deltas
// and inputs; bc: the row's B/C operand register.  All exponentials are
// issued first, then the input terms, the state chains and the output terms,
// so every result is consumed well after it is produced.  On return
// ys[0], ys[1] hold the channel's output sums over this wave's 4 states for
// tokens 2*0 + r and 2*1 + r of the group (r = row parity), i.e. the two
// state pairs of the channel are added across rows.
template <int MODE>
__device__ __forceinline__ void token_group(const float* dl, const float* xv, const float (&A2)[2],
                                            float (&h)[2], float bc, bool odd_row, float (&ys)[2]) {
  float e[4][2], bx[4][2], u[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    e[t][0] = fast_exp2(dl[t] * A2[0]);
    e[t][1] = fast_exp2(dl[t] * A2[1]);
  }
#pragma unroll
  for (int t = 0; t < 4; ++t) u[t] = dl[t] * xv[t];
  bx[0][0] = mul_bc<0>(bc, u[0]); bx[0][1] = mul_bc<1>(bc, u[0]);
  bx[1][0] = mul_bc<2>(bc, u[1]); bx[1][1] = mul_bc<3>(bc, u[1]);
  bx[2][0] = mul_bc<4>(bc, u[2]); bx[2][1] = mul_bc<5>(bc, u[2]);
  bx[3][0] = mul_bc<6>(bc, u[3]); bx[3][1] = mul_bc<7>(bc, u[3]);
  float hs[4][2];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    h[0] = __builtin_fmaf(e[t][0], h[0], bx[t][0]);
    h[1] = __builtin_fmaf(e[t][1], h[1], bx[t][1]);
    hs[t][0] = h[0];
    hs[t][1] = h[1];
  }
  if constexpr (MODE == kModeY) {
    float p[4];
    p[0] = mul_bc<8>(bc, hs[0][0]) + mul_bc<9>(bc, hs[0][1]);
    p[1] = mul_bc<10>(bc, hs[1][0]) + mul_bc<11>(bc, hs[1][1]);
    p[2] = mul_bc<12>(bc, hs[2][0]) + mul_bc<13>(bc, hs[2][1]);
    p[3] = mul_bc<14>(bc, hs[3][0]) + mul_bc<15>(bc, hs[3][1]);
    // token pairs (0,1) and (2,3): even rows keep the first, odd rows the second
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const float send = odd_row ? p[2 * q] : p[2 * q + 1];
      const float keep = odd_row ? p[2 * q + 1] : p[2 * q];
      ys[q] = keep + swap_rows(send);
    }
  }
}

// Workgroup = kCW channels of one batch row x W waves.  Lane l of wave w:
// channel cl = (l >> 5) * 16 + (l & 15), states 4w + 2r and 4w + 2r + 1 with
// r = (l >> 4) & 1 (the row parity).  The lane also finalises TPL = kT/(2W)
// consecutive tokens of its own channel (lane group 2w + r); it takes their
// x and z from the tiles into registers before the chunk's barrier, so one
// barrier per chunk suffices (tiles and partial outputs are double-buffered).
template <typename In, int VEC, bool GATE, int MODE, int W>
__global__ void __launch_bounds__(64 * W) s6_scan_kernel(ScanArgs a) {
  constexpr int NTHR = 64 * W;
  constexpr int NTS = (MODE == kModeY && GATE) ? 3 : 2;  // staged tensors: x, delta (, z)
  using S = Stage<In, VEC>;
  using SB = StageBC<In, VEC, W>;
  constexpr int TILE = kCW * kP;                  // floats per tensor tile
  constexpr int PART = 2 * kCW * (kT / 2);        // partial floats per wave
  constexpr int TPL = (kT / (2 * W)) > 0 ? kT / (2 * W) : 1;  // finalised tokens per lane
  constexpr int LG = kT / TPL;                    // lane groups that finalise

  extern __shared__ float4 lds4[];
  float* lds = reinterpret_cast<float*>(lds4);
  float* tiles = lds;                                         // [2][2][kCW][kP] x, delta, swizzled
  In* ztile = reinterpret_cast<In*>(tiles + 2 * 2 * TILE);    // [2][kCW][kP] gate input, input type
  constexpr int ZFL = (MODE == kModeY && GATE) ? (2 * TILE * (int)sizeof(In) + 15) / 16 * 4 : 0;
  float* part = tiles + 2 * 2 * TILE + ZFL;                   // [2][W][2][kCW][8]
  float* bcs = part + (MODE == kModeY ? 2 * W * PART : 0);    // [2][SB::kFloats]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = (lane >> 4) & 1;
  const int cl = ((lane >> 5) << 4) | (lane & 15);          // channel within the block
  const int lg = 2 * w + r;                                  // finalize lane group
  const bool fin = lg < LG;
  const int64_t D = a.D, L = a.L, N = a.N;
  const int64_t nblk = (D + kCW - 1) / kCW;
  const int64_t b = blockIdx.x / nblk;
  const int64_t d0 = (int64_t)(blockIdx.x % nblk) * kCW;
  const int64_t d = d0 + cl;
  const bool chv = d < D;
  const int64_t rows_valid = D - d0;
  const int64_t seg = blockIdx.z;
  const int64_t tb = seg * a.seg_len;
  const int64_t te = (tb + a.seg_len < L) ? tb + a.seg_len : L;
  const int64_t row0 = b * D + d0;
  const int64_t nchunks = (te - tb + kT - 1) / kT;

  gptr<In> src[3] = {(gptr<In>)a.x, (gptr<In>)a.delta, (gptr<In>)a.z};
  gptr<In> Bp = (gptr<In>)a.Bm;
  gptr<In> Cp = (gptr<In>)(MODE == kModeY ? a.Cm : a.Bm);

  float A2[2], h[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int64_t n = (int64_t)w * 4 + 2 * r + j;
    const bool sv = chv && n < N;
    A2[j] = sv ? a.A[d * N + n] * kLog2e : 0.0f;
    h[j] = (sv && a.hinit) ? a.hinit[seg * a.hinit_stride + (b * D + d) * N + n] : 0.0f;
  }
  const float dsk = (MODE == kModeY && a.Dskip && chv) ? a.Dskip[d] : 0.0f;
  double dsum = 0.0;
  // Let the loads above (A, h0, D) complete here: otherwise their pending
  // state reaches the loop header and the first use of h inside the loop
  // would wait for every outstanding load, prefetches included.
  __builtin_amdgcn_s_waitcnt(0);

  // Staging: one flat list of pieces -- NTS tile tensors of TP pieces each,
  // then the B/C pieces.  Loads are unconditional (invalid pieces read
  // element 0); only the LDS writes depend on the piece.
  constexpr int TP = S::kPieces;
  constexpr int TOTAL = NTS * TP + SB::kPieces;
  constexpr int SLOTS = (TOTAL + NTHR - 1) / NTHR;
  // Two register sets of loads in flight: chunk j goes to set j % 2, is
  // issued two chunks ahead and written to LDS one chunk ahead of its use.
  typename S::Raw preA[SLOTS], preB[SLOTS];

  auto issue_chunk = [&](int64_t t0, typename S::Raw (&pre)[SLOTS]) {
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) {
      const int p = tid + s * NTHR;
      if (p < NTS * TP) {
        const int k = p / TP;
        pre[s] = S::load(src[k], p - k * TP, row0, rows_valid, L, t0, te);
      } else {
        const int q = p - NTS * TP;
        pre[s] = SB::load(Bp, Cp, q < SB::kPieces ? q : 0, b, N, L, t0, te);
      }
    }
  };
  auto write_chunk = [&](int buf, int64_t t0, typename S::Raw (&pre)[SLOTS]) {
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) {
      const int p = tid + s * NTHR;
      if (p < NTS * TP) {
        const int k = p / TP;
        const int q = p - k * TP;
        if (k < 2) S::store(tiles + (buf * 2 + k) * TILE, q, pre[s], S::valid(q, rows_valid, t0, te));
        else S::store_raw(ztile + buf * TILE, q, pre[s], S::valid(q, rows_valid, t0, te));
      } else if (p < TOTAL) {
        const int q = p - NTS * TP;
        SB::store(bcs + buf * SB::kFloats, q, pre[s], SB::valid(q, N, t0, te));
      }
    }
  };

  if (nchunks > 0) {
    issue_chunk(tb, preA);
    write_chunk(0, tb, preA);
    issue_chunk(tb + kT, preB);
    issue_chunk(tb + 2 * kT, preA);
  }
  __syncthreads();

  // One chunk; `nxt` holds the loads of chunk k+1 and receives chunk k+3.
  auto chunk = [&](int64_t k, typename S::Raw (&nxt)[SLOTS]) {
    const int64_t t0 = tb + k * kT;
    const int buf = (int)(k & 1);
    const float* tx = tiles + (buf * 2 + 0) * TILE;
    const float* tdl = tiles + (buf * 2 + 1) * TILE;

    // this lane's kT deltas and inputs
    float dl[kT], xv[kT];
#pragma unroll
    for (int i = 0; i < kT; i += 4) {
      const float4 dv = *reinterpret_cast<const float4*>(tdl + tsw(cl, i >> 2));
      const float4 xx = *reinterpret_cast<const float4*>(tx + tsw(cl, i >> 2));
      dl[i] = dv.x; dl[i + 1] = dv.y; dl[i + 2] = dv.z; dl[i + 3] = dv.w;
      xv[i] = xx.x; xv[i + 1] = xx.y; xv[i + 2] = xx.z; xv[i + 3] = xx.w;
    }

    // x and z of the tokens this lane finalises (the tiles are overwritten
    // before this chunk's finalisation can run)
    float xfin[TPL], zfin[TPL];
#pragma unroll
    for (int i = 0; i < TPL; ++i) {
      const int t = (fin ? lg * TPL : 0) + i;
      xfin[i] = tx[tsw(cl, t >> 2) + (t & 3)];
      zfin[i] = (MODE == kModeY && GATE) ? to_f32(ztile[buf * TILE + tsw(cl, t >> 2) + (t & 3)]) : 0.0f;
    }

    float ysum[kT / 2];
#pragma unroll
    for (int g = 0; g < kT / 4; ++g) {
      const float bc = bcs[buf * SB::kFloats + SB::pos(g, w, r, lane & 15)];
      float ys[2];
      token_group<MODE>(dl + 4 * g, xv + 4 * g, A2, h, bc, r != 0, ys);
      ysum[2 * g] = ys[0];
      ysum[2 * g + 1] = ys[1];
    }
    float* pbuf = part + buf * (W * PART);
    if constexpr (MODE == kModeY) {
      // ysum[i] is this wave's sum for token 2i + r: part[buf][w][r][cl][i]
      float* pp = pbuf + w * PART + (r * kCW + cl) * (kT / 2);
      *reinterpret_cast<float4*>(pp) = make_float4(ysum[0], ysum[1], ysum[2], ysum[3]);
      *reinterpret_cast<float4*>(pp + 4) = make_float4(ysum[4], ysum[5], ysum[6], ysum[7]);
    }
    if constexpr (MODE == kModeState) {
      float cs = 0.0f;
#pragma unroll
      for (int i = 0; i < kT; ++i) cs += dl[i];
      dsum += (double)cs;
    }

    // Stage chunk k+1 into the other tile buffer (read last before the
    // previous barrier; its loads were issued one chunk ago).
    write_chunk(buf ^ 1, t0 + kT, nxt);
    __syncthreads();  // partial outputs of chunk k and the tiles of chunk k+1 are complete
    issue_chunk(t0 + 3 * kT, nxt);

    if constexpr (MODE == kModeY) {
      if (fin) {
        float yo[TPL];
#pragma unroll
        for (int i = 0; i < TPL; ++i) {
          const int t = lg * TPL + i;  // token within the chunk
          float acc = 0.0f;
#pragma unroll
          for (int ww = 0; ww < W; ++ww) acc += pbuf[ww * PART + ((t & 1) * kCW + cl) * (kT / 2) + (t >> 1)];
          acc = __builtin_fmaf(dsk, xfin[i], acc);
          if constexpr (GATE) acc *= silu(zfin[i]);
          yo[i] = acc;
        }
        const int64_t t = t0 + lg * TPL;
        if (chv) {
          float* dst = a.y + (b * D + d) * L + t;
          if constexpr (VEC > 1 && TPL % 2 == 0) {
#pragma unroll
            for (int i = 0; i < TPL; i += 2)
              if (t + i < te) *reinterpret_cast<float2*>(dst + i) = make_float2(yo[i], yo[i + 1]);
          } else {
#pragma unroll
            for (int i = 0; i < TPL; ++i)
              if (t + i < te) dst[i] = yo[i];
          }
        }
      }
    }
   };
  for (int64_t k = 0; k < nchunks; k += 2) {
    chunk(k, preB);
    if (k + 1 < nchunks) chunk(k + 1, preA);
  }

  const bool write_h = a.hout && (!a.hout_last_only || seg == (int64_t)gridDim.z - 1);
  if (write_h && chv) {
    const int64_t off = a.hout_last_only ? 0 : seg * a.hout_stride;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t n = (int64_t)w * 4 + 2 * r + j;
      if (n < N) a.hout[off + (b * D + d) * N + n] = h[j];
    }
  }
  if constexpr (MODE == kModeState) {
    if (a.sumdelta && chv && w == 0 && r == 0)
      a.sumdelta[seg * (int64_t)(gridDim.x / nblk) * D + b * D + d] = (float)dsum;
  }
}

// Fold segment aggregates into every segment's incoming state:
// H_0 = h0 (or 0); H_{s+1} = exp(A * sum_delta_s) * H_s + S_s.
// hin (S, batch*D*N) receives H_s for s < S; hlast (nullable) gets the state
// after the last of the `nagg` aggregates.
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

#define S6_HIP(call, what)                           \
  do {                                               \
    hipError_t e_ = (call);                          \
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
  if (!mul_ok(batch, dim, &t) || !mul_ok(t, seqlen > 0 ? seqlen : 1, &t) || !mul_ok(t, 64, &t))
    return S6_ERR_SHAPE;  // element counts, with headroom for per-state buffers
  if (batch * ((dim + kCW - 1) / kCW) > INT32_MAX) return S6_ERR_SHAPE;  // grid size
  return S6_OK;
}

struct Plan {
  int W;              // waves per workgroup (power of two, 4*W >= dstate)
  int64_t nblk;       // channel blocks per batch row
  int64_t segs;       // segments along L
  int64_t seg_len;    // tokens per segment, multiple of kT
  bool vec;           // 16-byte staging and 8-byte stores
};

// Segments: when batch * channel blocks gives fewer than 640 workgroups
// (2.5 per CU), cut L so that there are about 1280 (five per CU), each
// segment holding at least 4 chunks.
Plan make_plan(int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate, size_t esz,
               const void* const* ptrs, int nptr) {
  Plan p;
  const int64_t need = (dstate + 3) / 4;
  p.W = need <= 1 ? 1 : need <= 2 ? 2 : need <= 4 ? 4 : 8;
  p.nblk = (dim + kCW - 1) / kCW;
  const int64_t wgs = p.nblk * batch;
  int64_t segs = 1;
  if (wgs < 640) {
    segs = (1280 + wgs - 1) / wgs;
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
  p.vec = v;
  return p;
}

template <typename In, int VEC, bool GATE, int MODE, int W>
int launch_scan_t(const ScanArgs& a, int64_t batch, int64_t nblk, int64_t segs, hipStream_t st) {
  size_t lds = (size_t)2 * 2 * kCW * kP * sizeof(float);                       // x, delta tiles
  if (MODE == kModeY && GATE) lds += ((size_t)2 * kCW * kP * sizeof(In) + 15) / 16 * 16;  // gate tile
  if (MODE == kModeY) lds += (size_t)2 * W * 2 * kCW * (kT / 2) * sizeof(float);  // partials
  lds += (size_t)2 * StageBC<In, VEC, W>::kFloats * sizeof(float);              // B/C
  dim3 grid((unsigned)(nblk * batch), 1u, (unsigned)segs);
  hipLaunchKernelGGL((s6_scan_kernel<In, VEC, GATE, MODE, W>), grid, dim3(64 * W), lds, st, a);
  S6_HIP(hipGetLastError(), "s6_scan_kernel launch");
  return S6_OK;
}

template <typename In, int MODE, int W>
int launch_scan_w(const ScanArgs& a, bool vec, bool gate, int64_t batch, int64_t nblk, int64_t segs,
                  hipStream_t st) {
  constexpr int kV = 16 / sizeof(In);
  if constexpr (MODE == kModeY) {
    if (vec && gate) return launch_scan_t<In, kV, true, MODE, W>(a, batch, nblk, segs, st);
    if (vec) return launch_scan_t<In, kV, false, MODE, W>(a, batch, nblk, segs, st);
    if (gate) return launch_scan_t<In, 1, true, MODE, W>(a, batch, nblk, segs, st);
    return launch_scan_t<In, 1, false, MODE, W>(a, batch, nblk, segs, st);
  } else {
    if (vec) return launch_scan_t<In, kV, false, MODE, W>(a, batch, nblk, segs, st);
    return launch_scan_t<In, 1, false, MODE, W>(a, batch, nblk, segs, st);
  }
}

template <typename In, int MODE>
int launch_scan(const ScanArgs& a, int W, bool vec, bool gate, int64_t batch, int64_t nblk, int64_t segs,
                hipStream_t st) {
  switch (W) {
    case 1: return launch_scan_w<In, MODE, 1>(a, vec, gate, batch, nblk, segs, st);
    case 2: return launch_scan_w<In, MODE, 2>(a, vec, gate, batch, nblk, segs, st);
    case 4: return launch_scan_w<In, MODE, 4>(a, vec, gate, batch, nblk, segs, st);
    default: return launch_scan_w<In, MODE, 8>(a, vec, gate, batch, nblk, segs, st);
  }
}

int launch_scan_any(int in_dtype, int mode, const ScanArgs& a, const Plan& p, bool gate, int64_t batch,
                    int64_t segs, hipStream_t st) {
  if (in_dtype == S6_BF16) {
    return mode == kModeY ? launch_scan<uint16_t, kModeY>(a, p.W, p.vec, gate, batch, p.nblk, segs, st)
                          : launch_scan<uint16_t, kModeState>(a, p.W, p.vec, gate, batch, p.nblk, segs, st);
  }
  return mode == kModeY ? launch_scan<float, kModeY>(a, p.W, p.vec, gate, batch, p.nblk, segs, st)
                        : launch_scan<float, kModeState>(a, p.W, p.vec, gate, batch, p.nblk, segs, st);
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
  const Plan p = make_plan(batch, dim, seqlen, dstate, esz, vecptrs, want_y ? 4 : 2);
  const bool gate = want_y && z != nullptr;
  const int64_t S = p.segs;

  ScanArgs a;
  memset(&a, 0, sizeof(a));
  a.x = x; a.delta = delta; a.z = gate ? z : nullptr; a.Bm = Bm; a.Cm = want_y ? Cm : nullptr;
  a.A = A; a.Dskip = want_y ? Dskip : nullptr;
  a.D = dim; a.L = seqlen; a.N = dstate; a.seg_len = p.seg_len;

  if (S == 1) {
    a.hinit = h0;
    a.hout = h_last;
    a.hout_last_only = 1;
    a.y = y;
    return launch_scan_any(in_dtype, want_y ? kModeY : kModeState, a, p, gate, batch, 1, st);
  }

  // Segmented: workspace for segment end states, summed deltas and carries.
  const int64_t nagg = want_y ? S - 1 : S;
  auto up = [](size_t v) { return (v + 255) & ~(size_t)255; };
  const size_t agg_bytes = (size_t)nagg * nstate * sizeof(float);
  const size_t sd_bytes = (size_t)nagg * batch * dim * sizeof(float);
  const size_t hin_bytes = want_y ? (size_t)S * nstate * sizeof(float) : 0;
  void* ws = nullptr;
  S6_HIP(hipMallocAsync(&ws, up(agg_bytes) + up(sd_bytes) + up(hin_bytes), st), "hipMallocAsync(workspace)");
  char* wp = static_cast<char*>(ws);
  float* agg = reinterpret_cast<float*>(wp);
  float* sd = reinterpret_cast<float*>(wp + up(agg_bytes));
  float* hin = reinterpret_cast<float*>(wp + up(agg_bytes) + up(sd_bytes));

  // pass 1: end states of the first nagg segments from a zero state
  ScanArgs g = a;
  g.z = nullptr; g.Cm = nullptr; g.Dskip = nullptr;
  g.hinit = nullptr;
  g.hout = agg;
  g.hout_stride = nstate;
  g.sumdelta = sd;
  rc = launch_scan_any(in_dtype, kModeState, g, p, false, batch, nagg, st);
  if (rc == S6_OK) {
    const int64_t blocks = (nstate + 255) / 256;
    hipLaunchKernelGGL(s6_fold_carries, dim3((unsigned)blocks), dim3(256), 0, st, A, h0, agg, sd,
                       want_y ? hin : nullptr, want_y ? nullptr : h_last, batch, dim, dstate, S, nagg);
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
