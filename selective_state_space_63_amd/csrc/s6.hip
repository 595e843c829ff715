// libs6 -- selective SSM scan (S6) for AMD MI355X (gfx950): kernels and C ABI.
//
// What is computed: see include/s6.h, which cites the pages ("【LLM】Mamba和
// State Space Models详解" §2.2-§2.4 and §3.2-§3.4).  This file only
// restates the recurrence per (batch, channel, state):
//     h = exp(delta*A) * h + delta*B*x ;  y = (sum_n C*h + D*x) * SiLU(z)
//
// Design (gfx950, wave64):
//  * The scan is bound by VALU issue: per (token, channel, state) it needs an
//    exponential (v_exp_f32, two issue slots) and four multiply/FMA slots,
//    and packed fp32 math is not used.  There is no dense contraction, so no
//    MFMA.  Everything below serves to keep the VALU busy with little else.
//  * Workgroup = 32 channels of one batch row x W waves (W = 4 for N = 16).
//    Lane l of wave w: channel (l >> 5) * 16 + (l & 15), states 4w + 2r and
//    4w + 2r + 1 with r = (l >> 4) & 1.  For the 3B layer that is exactly 5
//    waves per SIMD on 256 CUs.  A and the state stay in VGPRs; the
//    (batch, D, L, N) state is never written.
//  * B and C differ per state pair, i.e. per 16-lane row.  For a group of 4
//    tokens a row keeps them in one VGPR (lane 4m + k: B of pair member m,
//    token k; lane 8 + 4m + k: C), read through DPP row_newbcast operands of
//    v_mul_f32_dpp / v_fmac_f32_dpp: no extra instruction per use.
//  * The two state pairs of a channel sit in rows 2i and 2i + 1; one
//    v_permlane16_swap plus an add combines their output terms for two
//    tokens at once.  The W waves add theirs through LDS.
//  * Inputs are staged per 16-token chunk: threads load 16-byte pieces of
//    x, delta, z, B and C two 32-token windows ahead into registers (so each
//    row is read in 64-byte runs), convert them to fp32 into double-buffered
//    LDS tiles one chunk ahead (x, delta in a channel-major XOR-swizzled
//    layout; B/C in the DPP layout), and each lane reads its channel's values
//    per group of 4 tokens.  One barrier per chunk; after it, every lane
//    finalises 2 tokens of one channel (sum of the W partial outputs, skip
//    term, SiLU gate) and adjacent lanes store 64-byte runs of y.
//  * Chunks past the end of a sequence are staged as delta = 0 (the state
//    stays exactly unchanged) and store nothing, so the loop body has no
//    conditional memory operations.
//  * Few long rows (too few workgroups to fill the GPU) are cut into
//    segments along L: pass 1 computes every segment's end state from zero
//    and its summed delta, a tiny pass folds them into each segment's
//    incoming state (associativity of the (a, b) pairs), and pass 2 runs the
//    fused scan of every segment from its incoming state.
//  * Decode: 4 states per lane (P = dstate / 4 adjacent lanes per channel,
//    partial outputs added with DPP quad permutations), 4 batch rows per
//    lane with all their loads issued first; h, A, B, C read and h written
//    with 8/16-byte accesses that are contiguous across the lanes of a wave.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <type_traits>
#include <utility>

#include "s6.h"

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
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
  const float* dbias;     // (D) bias of the softplus step, or null (zero)
  int softplus;           // step = softplus(delta + dbias[d])  (option kernels only; the
                          // bias alone is added without it)
  int zoh;                // exact zero-order-hold input coefficient (option kernels only)
  int64_t D, L, N;
  int64_t seg_len;        // tokens per segment (multiple of 4 kT); segment = blockIdx.z
  int64_t hinit_stride;   // elements between segments in hinit (0: same for all)
  int64_t hout_stride;    // elements between segments in hout
  int64_t hout_last_only; // 1: only the last segment writes hout (at offset 0)
};

// One chunk of kT tokens of the kCW channel rows of x, delta (and z) and of
// the 4W state rows of B (and C), cut into pieces of VEC elements (16 bytes;
// single elements when VEC == 1).  Piece order: tensor, row, piece within
// the row, so adjacent threads take adjacent pieces of a row.  A load window
// is WIN consecutive chunks: a thread loads the same piece of each of them
// back to back, so together they cover runs of WIN * 16 tokens of a row.
template <typename In, int VEC, int W, int NTS, int NBC>
struct ChunkPieces {
  static constexpr int PPC = kT / VEC;            // pieces per row
  static constexpr int kTens = NTS * kCW * PPC;   // x, delta (, z) pieces
  static constexpr int kRowsBC = 4 * W;           // state rows per B/C tensor
  static constexpr int kTotal = kTens + NBC * kRowsBC * PPC;
  using Raw = typename std::conditional<VEC == 1, In, u32x4>::type;
};

// B and C of one chunk in LDS, laid out as the DPP operands want them: for
// token group g (4 tokens), wave w and row parity r (state pair 4w + 2r,
// 4w + 2r + 1), a block of 16 slots read by the 16 lanes of the row: B of
// pair member m, token k at slot 4m + k; C at slot 8 + 4m + k.  The four
// 4-slot quarters of a block are permuted by XOR with f(g, w) so that the
// 16-byte writes of one instruction spread over the banks; readers apply
// the same permutation, so lane x of a row still receives slot x.  States
// beyond N stay zero.
template <int W>
struct BCLayout {
  static constexpr int kFloats = (kT / 4) * W * 2 * 16;  // floats per chunk
  __device__ __forceinline__ static int quarter(int g, int w, int q) { return q ^ (((g >> 1) ^ w) & 3); }
  __device__ __forceinline__ static int pos(int g, int w, int r, int x) {
    return ((g * W + w) * 2 + r) * 16 + (quarter(g, w, x >> 2) << 2) + (x & 3);
  }
  // first of the 4 slots of token group g for tensor tens (0 = B, 1 = C), state n
  __device__ __forceinline__ static int group_pos(int tens, int n, int g) {
    const int w = n >> 2, r = (n >> 1) & 1, m = n & 1;
    return ((g * W + w) * 2 + r) * 16 + (quarter(g, w, tens * 2 + m) << 2);
  }
};

// The row-broadcast products of a token group, written out as DPP
// instructions (lane J of the 16-lane row of bc as the first operand): the
// compiler folds such broadcasts only sometimes, and never into a
// multiply-add with a tied accumulator.  The leading s_nop gives the two wait
// states a DPP read needs after a VALU write of its source register.
//
// Input terms: bx[t][m] = bc[lane 4m + t] * u[t].
__device__ __forceinline__ void bcast_inputs(float bc, const float (&u)[4], float (&bx)[4][2]) {
  asm("s_nop 1\n\t"
      "v_mul_f32_dpp %0, %8, %9 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %1, %8, %9 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %2, %8, %10 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %3, %8, %10 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %4, %8, %11 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %5, %8, %11 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %6, %8, %12 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %7, %8, %12 row_newbcast:7 row_mask:0xf bank_mask:0xf"
      : "=&v"(bx[0][0]), "=&v"(bx[0][1]), "=&v"(bx[1][0]), "=&v"(bx[1][1]), "=&v"(bx[2][0]),
        "=&v"(bx[2][1]), "=&v"(bx[3][0]), "=&v"(bx[3][1])
      : "v"(bc), "v"(u[0]), "v"(u[1]), "v"(u[2]), "v"(u[3]));
}

// Input terms with a coefficient per state: bx[t][m] = bc[lane 4m + t] * v[t][m].
__device__ __forceinline__ void bcast_inputs2(float bc, const float (&v)[4][2], float (&bx)[4][2]) {
  asm("s_nop 1\n\t"
      "v_mul_f32_dpp %0, %8, %9 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %1, %8, %10 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %2, %8, %11 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %3, %8, %12 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %4, %8, %13 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %5, %8, %14 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %6, %8, %15 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %7, %8, %16 row_newbcast:7 row_mask:0xf bank_mask:0xf"
      : "=&v"(bx[0][0]), "=&v"(bx[0][1]), "=&v"(bx[1][0]), "=&v"(bx[1][1]), "=&v"(bx[2][0]),
        "=&v"(bx[2][1]), "=&v"(bx[3][0]), "=&v"(bx[3][1])
      : "v"(bc), "v"(v[0][0]), "v"(v[0][1]), "v"(v[1][0]), "v"(v[1][1]), "v"(v[2][0]), "v"(v[2][1]),
        "v"(v[3][0]), "v"(v[3][1]));
}

// Output terms: p[t] = bc[lane 8 + t] * hs[t][0] + bc[lane 12 + t] * hs[t][1].
__device__ __forceinline__ void bcast_outputs(float bc, const float (&hs)[4][2], float (&p)[4]) {
  asm("s_nop 1\n\t"
      "v_mul_f32_dpp %0, %4, %5 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %1, %4, %7 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %2, %4, %9 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %3, %4, %11 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %0, %4, %6 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %1, %4, %8 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %2, %4, %10 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %3, %4, %12 row_newbcast:15 row_mask:0xf bank_mask:0xf"
      : "=&v"(p[0]), "=&v"(p[1]), "=&v"(p[2]), "=&v"(p[3])
      : "v"(bc), "v"(hs[0][0]), "v"(hs[0][1]), "v"(hs[1][0]), "v"(hs[1][1]), "v"(hs[2][0]),
        "v"(hs[2][1]), "v"(hs[3][0]), "v"(hs[3][1]));
}

// Adds the output terms of the two state pairs of a channel (rows 2i and
// 2i+1 of the wave, same lane within the row) for two tokens at once:
// v_permlane16_swap exchanges the odd rows of its first operand with the
// even rows of its second, so with the even token's value in the first and
// the odd token's in the second, the sum of the two results holds the even
// token in even rows and the odd token in odd rows.
__device__ __forceinline__ float pair_rows(float even_tok, float odd_tok) {
  const auto s = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, even_tok),
                                                  __builtin_bit_cast(unsigned, odd_tok), false, false);
  return __builtin_bit_cast(float, (unsigned)s[0]) + __builtin_bit_cast(float, (unsigned)s[1]);
}

// One group of 4 tokens for this lane's 2 states.  dl/xv: the lane's deltas
// and inputs; bc: the row's B/C operand register (lane 4m + k: B of pair
// member m for token k, lane 8 + 4m + k: C).  All exponentials are
// issued first, then the input terms, the state chains and the output terms,
// so every result is consumed well after it is produced.  On return
// ys[0], ys[1] hold the channel's output sums over this wave's 4 states for
// tokens 2*0 + r and 2*1 + r of the group (r = row parity), i.e. the two
// state pairs of the channel are added across rows.  EXT kernels take the
// exact zero-order-hold input coefficient when `zoh` is set.
template <int MODE, bool EXT>
__device__ __forceinline__ void token_group(const float* dl, const float* xv, const float (&A2)[2],
                                            float (&h)[2], float bc, bool zoh, float (&ys)[2]) {
  float e[4][2], bx[4][2], arg[4][2];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    arg[t][0] = dl[t] * A2[0];
    arg[t][1] = dl[t] * A2[1];
    e[t][0] = fast_exp2(arg[t][0]);
    e[t][1] = fast_exp2(arg[t][1]);
  }
  if (EXT && zoh) {
    float v[4][2];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      v[t][0] = zoh_coef(dl[t], arg[t][0], e[t][0]) * xv[t];
      v[t][1] = zoh_coef(dl[t], arg[t][1], e[t][1]) * xv[t];
    }
    bcast_inputs2(bc, v, bx);
  } else {
    float u[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) u[t] = dl[t] * xv[t];
    bcast_inputs(bc, u, bx);
  }
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
    bcast_outputs(bc, hs, p);
    // token pairs (0,1) and (2,3): even rows get the first, odd rows the second
    ys[0] = pair_rows(p[0], p[1]);
    ys[1] = pair_rows(p[2], p[3]);
  }
}

// Workgroup = kCW channels of one batch row x W waves.  Lane l of wave w:
// channel cl = (l >> 5) * 16 + (l & 15), states 4w + 2r and 4w + 2r + 1 with
// r = (l >> 4) & 1 (the row parity).  Per chunk of kT tokens the lane reads
// its channel's deltas and inputs from LDS, runs the recurrence for its two
// states and writes the wave's partial outputs to LDS; after the chunk's
// single barrier every lane finalises TPL consecutive tokens of one channel
// (sum of the W partials, skip term, gate) and stores them.
//
// Staging: loads of window j (WIN chunks) go to register set j % 2 two
// windows ahead; chunk k + 1 is converted into the other LDS buffer during
// chunk k, before the barrier.  Only the last, partial chunk of a sequence
// is written with per-piece masking (delta = 0 past the end keeps the
// state), and only a window that would cross the end of the rows clamps its
// piece addresses.
//
// EXT kernels also take the step bias and discretisation options of ScanArgs:
// the bias and softplus are applied to delta while it is staged (once per
// element), the exact hold in the token groups, and the
// kind of piece each wave stages rotates with the workgroup index so that
// this extra work falls on every SIMD alike.
template <typename In, int VEC, bool GATE, int MODE, int W, int WIN, bool EXT>
__global__ void __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(W == 4 ? (EXT ? 4 : 5) : 1)))
s6_scan_kernel(ScanArgs a) {
  constexpr int NTHR = 64 * W;
  constexpr int NTS = (MODE == kModeY && GATE) ? 3 : 2;  // staged tensors: x, delta (, z)
  constexpr int NBC = MODE == kModeY ? 2 : 1;             // B (, C)
  using CP = ChunkPieces<In, VEC, W, NTS, NBC>;
  using Raw = typename CP::Raw;
  using BCL = BCLayout<W>;
  constexpr int WT = WIN * kT;                    // tokens per load window
  constexpr int SLOTS = (CP::kTotal + NTHR - 1) / NTHR;
  constexpr int TILE = kCW * kP;                  // floats per tensor tile
  constexpr int PART = 2 * kCW * (kT / 2);        // partial floats per wave
  // Finalisation: lane tid owns TPL consecutive tokens of channel fc; the
  // LPR lanes of a channel are adjacent, so one store instruction writes
  // whole 64-byte runs of y rows.
  constexpr int TPL = kT * kCW / NTHR;            // finalised tokens per lane
  constexpr int LPR = kT / TPL;                   // lanes per channel
  static_assert(TPL >= 1 && kT % TPL == 0, "finalisation layout");

  extern __shared__ float4 lds4[];
  float* lds = reinterpret_cast<float*>(lds4);
  float* tiles = lds;                                         // [2][2][kCW][kP] x, delta, swizzled
  In* ztile = reinterpret_cast<In*>(tiles + 2 * 2 * TILE);    // [2][kCW][kP] gate input, input type
  constexpr int ZFL = (MODE == kModeY && GATE) ? (2 * TILE * (int)sizeof(In) + 15) / 16 * 4 : 0;
  float* part = tiles + 2 * 2 * TILE + ZFL;                   // [2][W][2][kCW][8]
  float* bcs = part + (MODE == kModeY ? 2 * W * PART : 0);    // [2][BCL::kFloats]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = (lane >> 4) & 1;
  const int cl = ((lane >> 5) << 4) | (lane & 15);          // channel within the block
  const int fc = tid / LPR;                                   // finalised channel within the block
  const int ft = (tid % LPR) * TPL;                          // its first token within a chunk
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
  const int64_t nwin = (te - tb + WT - 1) / WT;
  const int64_t lastw = tb + (nwin > 0 ? nwin - 1 : 0) * WT;  // start of the last window
  const bool part_chunk = ((te - tb) % kT) != 0;               // last chunk only partly valid
  const int64_t nplain = nchunks - (part_chunk ? 1 : 0);        // chunks staged without masking

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
  const bool fchv = d0 + fc < D;
  const float dsk = (MODE == kModeY && a.Dskip && fchv) ? a.Dskip[d0 + fc] : 0.0f;
  // Sum of delta over the segment (state mode), compensated (Neumaier):
  // dsum + dcomp.  (A double accumulator here costs dozens of registers.)
  float dsum = 0.0f, dcomp = 0.0f;

  // This thread's pieces: slot s holds piece tid + s * NTHR of every chunk.
  // Rows past the end of the block read the last valid row (their channels
  // are never stored); B/C state rows >= N read state N-1 and are not
  // written, so their LDS slots stay zero.
  gptr<In> sptr[SLOTS];  // piece at token 0
  int scol[SLOTS];       // first token of the piece within a chunk
  int srow[SLOTS];       // row within its tensor (channel or state)
  int skind[SLOTS];      // 0..NTS-1: x, delta, z; NTS + m: B (m = 0) or C (m = 1); -1: idle
  float sbias[SLOTS];    // EXT: softplus bias of the piece's channel
  const bool softplus = EXT && a.softplus;
  const bool dstep = EXT && (a.softplus || a.dbias);  // delta is rewritten while staged
  const bool zoh = EXT && a.zoh;
  const int rot = EXT ? (int)(blockIdx.x % W) * 64 : 0;
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) {
    int p = ((tid + rot) & (NTHR - 1)) + s * NTHR;
    sbias[s] = 0.0f;
    const bool idle = p >= CP::kTotal;
    if (idle) p = 0;  // idle slot: loads piece 0, never writes
    if (p < CP::kTens) {
      const int k = p / (kCW * CP::PPC);
      const int q = p - k * (kCW * CP::PPC);
      const int row = q / CP::PPC;
      const int64_t rowc = row < rows_valid ? row : rows_valid - 1;
      skind[s] = k;
      srow[s] = row;
      scol[s] = (q - row * CP::PPC) * VEC;
      sptr[s] = src[k] + (row0 + rowc) * L + scol[s];
      if (EXT && k == 1 && a.dbias) sbias[s] = a.dbias[d0 + rowc];
    } else {
      const int q = p - CP::kTens;
      const int m = q / (CP::kRowsBC * CP::PPC);
      const int q2 = q - m * (CP::kRowsBC * CP::PPC);
      const int n = q2 / CP::PPC;
      const int64_t nc = n < N ? n : N - 1;
      skind[s] = NTS + m;
      srow[s] = n;
      scol[s] = (q2 - n * CP::PPC) * VEC;
      sptr[s] = (m ? Cp : Bp) + (b * N + nc) * L + scol[s];
    }
    if (idle) skind[s] = -1;
  }

  // B/C slots of states >= N are never written: clear both buffers once.
  if (N < 4 * W) {
    for (int i = tid; i < 2 * BCL::kFloats; i += NTHR) bcs[i] = 0.0f;
    __syncthreads();
  }
  // Let the loads above (A, h0, D) complete here: otherwise their pending
  // state reaches the loop header and the first use of h inside the loop
  // would wait for every outstanding load, prefetches included.
  __builtin_amdgcn_s_waitcnt(0);

  Raw pre[2][WIN][SLOTS];  // two windows in flight

  // Loads of the window starting at token t0w (clamped to the segment's last
  // window: prefetches past the end repeat it and are never used).
  auto issue = [&](int64_t t0w, Raw (&dst)[WIN][SLOTS]) {
    t0w = t0w < lastw ? t0w : lastw;
    if (t0w + WT <= L) {
#pragma unroll
      for (int hh = 0; hh < WIN; ++hh)
#pragma unroll
        for (int s = 0; s < SLOTS; ++s)
          dst[hh][s] = *reinterpret_cast<gptr<Raw>>(sptr[s] + (t0w + hh * kT));
    } else {
#pragma unroll
      for (int hh = 0; hh < WIN; ++hh)
#pragma unroll
        for (int s = 0; s < SLOTS; ++s) {
          // past the end of the row: reread its last piece (masked when staged)
          int64_t tp = t0w + hh * kT;
          const int64_t lim = L - VEC - scol[s];
          tp = tp < lim ? tp : lim;
          dst[hh][s] = *reinterpret_cast<gptr<Raw>>(sptr[s] + tp);
        }
    }
  };

  // Convert the pieces of chunk c (in `src_`) into LDS buffer `buf`.  MASK:
  // zero the tokens at or past te (only the last chunk can need it).
  auto stage = [&](int buf, int64_t c, const Raw (&src_)[SLOTS], auto maskc) {
    constexpr bool MASK = decltype(maskc)::value;
    const int64_t t0c = tb + c * kT;
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) {
      const int col = scol[s];
      if (skind[s] < 0) continue;
      const bool ok = !MASK || t0c + col < te;
      const In* e = reinterpret_cast<const In*>(&src_[s]);
      if (dstep && skind[s] == 1) {
        // step = delta + bias, then softplus if asked; masked tokens stay 0
        float* tile = tiles + (buf * 2 + 1) * TILE;
        float v[VEC];
#pragma unroll
        for (int k = 0; k < VEC; ++k) v[k] = to_f32(e[k]) + sbias[s];
        if (softplus) {
#pragma unroll
          for (int k = 0; k < VEC; ++k) v[k] = softplus_f(v[k]);
        }
        if constexpr (VEC == 1) {
          tile[tsw(srow[s], col >> 2) + (col & 3)] = ok ? v[0] : 0.0f;
        } else {
#pragma unroll
          for (int k = 0; k < VEC; k += 4)
            *reinterpret_cast<float4*>(tile + tsw(srow[s], (col + k) >> 2)) =
                ok ? make_float4(v[k], v[k + 1], v[k + 2], v[k + 3]) : make_float4(0.f, 0.f, 0.f, 0.f);
        }
      } else if (skind[s] < 2) {
        float* tile = tiles + (buf * 2 + skind[s]) * TILE;
        if constexpr (VEC == 1) {
          tile[tsw(srow[s], col >> 2) + (col & 3)] = ok ? to_f32(e[0]) : 0.0f;
        } else {
#pragma unroll
          for (int k = 0; k < VEC; k += 4)
            *reinterpret_cast<float4*>(tile + tsw(srow[s], (col + k) >> 2)) =
                ok ? make_float4(to_f32(e[k]), to_f32(e[k + 1]), to_f32(e[k + 2]), to_f32(e[k + 3]))
                   : make_float4(0.f, 0.f, 0.f, 0.f);
        }
      } else if (skind[s] < NTS) {
        In* zt = ztile + buf * TILE;
        if constexpr (VEC == 1) {
          zt[tsw(srow[s], col >> 2) + (col & 3)] = ok ? e[0] : In(0);
        } else if constexpr (sizeof(In) == 2) {
          // groups of 4 elements stay contiguous (8 bytes) in the swizzled tile
          const u32x4 v = src_[s];
          *reinterpret_cast<uint2*>(zt + tsw(srow[s], col >> 2)) = ok ? make_uint2(v.x, v.y) : make_uint2(0u, 0u);
          *reinterpret_cast<uint2*>(zt + tsw(srow[s], (col + 4) >> 2)) = ok ? make_uint2(v.z, v.w) : make_uint2(0u, 0u);
        } else {
          const u32x4 zero = {0u, 0u, 0u, 0u};
          *reinterpret_cast<u32x4*>(zt + tsw(srow[s], col >> 2)) = ok ? src_[s] : zero;
        }
      } else if (srow[s] < N) {
        float* bt = bcs + buf * BCL::kFloats;
        const int m = skind[s] - NTS;
        if constexpr (VEC == 1) {
          bt[BCL::group_pos(m, srow[s], col >> 2) + (col & 3)] = ok ? to_f32(e[0]) : 0.0f;
        } else {
#pragma unroll
          for (int k = 0; k < VEC; k += 4)
            *reinterpret_cast<float4*>(bt + BCL::group_pos(m, srow[s], (col + k) >> 2)) =
                ok ? make_float4(to_f32(e[k]), to_f32(e[k + 1]), to_f32(e[k + 2]), to_f32(e[k + 3]))
                   : make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
    }
  };

  if (nchunks > 0) {
    issue(tb, pre[0]);
    issue(tb + WT, pre[1]);
    if (nplain == 0) stage(0, 0, pre[0][0], std::true_type{});
    else stage(0, 0, pre[0][0], std::false_type{});
    if constexpr (WIN == 1) issue(tb + 2 * WT, pre[0]);  // window 0 is fully staged: refill its set
  }
  __syncthreads();

  // Chunk k at position P = k % (2 WIN) of the two-window cycle.
  // The loop runs whole cycles of 2 WIN chunks: chunks past the end of the
  // segment are staged fully masked (delta = 0 leaves the state exactly
  // unchanged) and store nothing.  So the loop body has no conditional loads,
  // which would make the compiler's wait placement conservative across the
  // loop back edge.
  auto chunk = [&](int64_t k, auto pos) {
    constexpr int P = decltype(pos)::value;
    // keep the scheduler from interleaving consecutive chunks (it raises the
    // register pressure past five waves per SIMD)
    __builtin_amdgcn_sched_barrier(0);
    constexpr int NP = (P + 1) % (2 * WIN);  // position of chunk k + 1
    constexpr int SET = NP / WIN, HALF = NP % WIN;
    const int64_t t0 = tb + k * kT;
    const int buf = (int)(k & 1);
    const float* tx = tiles + (buf * 2 + 0) * TILE;
    const float* tdl = tiles + (buf * 2 + 1) * TILE;


    // x and z of the tokens this lane finalises (buffer `buf` is restaged
    // before this chunk's finalisation can run in every wave)
    float xfin[TPL], zfin[TPL];
#pragma unroll
    for (int i = 0; i < TPL; ++i) {
      const int t = ft + i;
      xfin[i] = tx[tsw(fc, t >> 2) + (t & 3)];
      zfin[i] = (MODE == kModeY && GATE) ? to_f32(ztile[buf * TILE + tsw(fc, t >> 2) + (t & 3)]) : 0.0f;
    }

    // the lane's deltas and inputs, one group of 4 tokens at a time
    float ysum[kT / 2];
    float cs = 0.0f;
#pragma unroll
    for (int g = 0; g < kT / 4; ++g) {
      const float4 dv = *reinterpret_cast<const float4*>(tdl + tsw(cl, g));
      const float4 xx = *reinterpret_cast<const float4*>(tx + tsw(cl, g));
      const float dl[4] = {dv.x, dv.y, dv.z, dv.w};
      const float xv[4] = {xx.x, xx.y, xx.z, xx.w};
      const float bc = bcs[buf * BCL::kFloats + BCL::pos(g, w, r, lane & 15)];
      float ys[2];
      token_group<MODE, EXT>(dl, xv, A2, h, bc, zoh, ys);
      ysum[2 * g] = ys[0];
      ysum[2 * g + 1] = ys[1];
      if constexpr (MODE == kModeState) cs += (dl[0] + dl[1]) + (dl[2] + dl[3]);
    }
    // The chunk's state updates (and delta sum) complete here.  (Without
    // output terms nothing else ties them to the chunk, and the compiler would
    // sink them past the barriers, keeping every chunk's inputs live at once.)
    asm volatile("" : "+v"(h[0]), "+v"(h[1]), "+v"(cs));
    float* pbuf = part + buf * (W * PART);
    if constexpr (MODE == kModeY) {
      // ysum[i] is this wave's sum for token 2i + r: part[buf][w][r][cl][i]
      float* pp = pbuf + w * PART + (r * kCW + cl) * (kT / 2);
      *reinterpret_cast<float4*>(pp) = make_float4(ysum[0], ysum[1], ysum[2], ysum[3]);
      *reinterpret_cast<float4*>(pp + 4) = make_float4(ysum[4], ysum[5], ysum[6], ysum[7]);
    }
    if constexpr (MODE == kModeState) {
      const float t = dsum + cs;
      dcomp += (fabsf(dsum) >= fabsf(cs)) ? (dsum - t) + cs : (cs - t) + dsum;
      dsum = t;
    }

    // Stage chunk k + 1 into the other buffer (read last before the previous
    // barrier).  The register set it came from is free once its window's
    // last chunk is staged: refill it with the window two ahead.
    if (k + 1 < nplain) stage(buf ^ 1, k + 1, pre[SET][HALF], std::false_type{});
    else stage(buf ^ 1, k + 1, pre[SET][HALF], std::true_type{});
    __syncthreads();  // partial outputs of chunk k and the tiles of chunk k + 1 are complete
    if constexpr (HALF == WIN - 1) issue(tb + ((k + 1) / WIN + 2) * WT, pre[SET]);

    if constexpr (MODE == kModeY) {
      float yo[TPL];
#pragma unroll
      for (int i = 0; i < TPL; ++i) {
        const int t = ft + i;  // token within the chunk
        float acc = 0.0f;
#pragma unroll
        for (int ww = 0; ww < W; ++ww) acc += pbuf[ww * PART + ((t & 1) * kCW + fc) * (kT / 2) + (t >> 1)];
        acc = __builtin_fmaf(dsk, xfin[i], acc);
        if constexpr (GATE) acc *= silu(zfin[i]);
        yo[i] = acc;
      }
      const int64_t t = t0 + ft;
      if (fchv) {
        float* dst = a.y + (row0 + fc) * L + t;
        // Vector path: L is a multiple of 8 (4 for fp32 input) and y is
        // 16-byte aligned, so runs of 2 (or 4) tokens are all valid or all
        // past the end, and aligned.
        if constexpr (VEC > 1 && TPL % 4 == 0) {
#pragma unroll
          for (int i = 0; i < TPL; i += 4)
            if (t + i < te) *reinterpret_cast<float4*>(dst + i) = make_float4(yo[i], yo[i + 1], yo[i + 2], yo[i + 3]);
        } else if constexpr (VEC > 1 && TPL % 2 == 0) {
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
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  for (int64_t k = 0; k < nchunks; k += 2 * WIN) {
    chunk(k, I0{});
    chunk(k + 1, I1{});
    if constexpr (WIN == 2) {
      chunk(k + 2, I2{});
      chunk(k + 3, I3{});
    }
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
      a.sumdelta[seg * (int64_t)(gridDim.x / nblk) * D + b * D + d] = dsum + dcomp;
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
  const float* dbias;  // (D) step bias or null
  int softplus;        // step = softplus(delta + dbias[d])
  int zoh;             // exact zero-order-hold input coefficient
  int64_t batch, D, N;
};

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
    dt[g] = to_f32(dp[ch]);
    xt[g] = to_f32(xp[ch]);
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
    if (vb[g] && q == 0) {
      float yv = __builtin_fmaf(dsk, xt[g], yp);
      if constexpr (GATE) yv *= silu(to_f32(zp[ch]));
      a.y[ch] = yv;
    }
  }
}

// ---------------------------------------------------------------- backward --
// Reverse-mode gradients of the scan for the loss <dy, y> + <dh_last, h_last>
// (plain step).  The states are recomputed, never stored per token: a
// state-only pass and the carry fold give the state entering every segment of
// kBwdSeg tokens (the same kernels as a segmented forward scan); this kernel
// then walks the segments of a (batch row, 16-channel block) from the last to
// the first.  Per segment it stages the inputs in LDS, recomputes the states
// at the four chunk starts, and per 16-token chunk (last first) recomputes
// the chunk's states and transitions in registers and runs the adjoint
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

// Waves per workgroup (4 channels each).  The kernel needs 150-190 VGPRs,
// i.e. two waves per SIMD: two 4-wave workgroups per CU, whose barriers fall
// at different times, run faster than one 8-wave workgroup.
template <int SPL>
constexpr int bwd_waves() { return 4; }

template <int SPL>
constexpr size_t bwd_lds_bytes(bool sp) {
  return sizeof(float) * ((size_t)(sp ? 5 : 4) * (4 * bwd_waves<SPL>()) * kBwdPitch + (size_t)2 * 16 * SPL * kBwdPitch +
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
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float row_reduce_scatter16(const float (&v)[16], int nl) {
  const bool b3 = nl & 8, b2 = nl & 4, b1 = nl & 2, b0 = nl & 1;
  float a8[8], a4[4], a2[2];
#pragma unroll
  for (int j = 0; j < 8; ++j) a8[j] = (b3 ? v[j + 8] : v[j]) + dpp_f<0x128>(b3 ? v[j] : v[j + 8]);
#pragma unroll
  for (int j = 0; j < 4; ++j) a4[j] = (b2 ? a8[j + 4] : a8[j]) + dpp_f<0x141>(b2 ? a8[j] : a8[j + 4]);
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
template <typename In, bool GATE, int SPL, bool SP>
__global__ void __launch_bounds__(64 * bwd_waves<SPL>()) s6_bwd_kernel(BwdArgs a) {
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
  float* sB = sq + CW * KP;          // [NS][KP]
  float* sC = sB + NS * KP;          // [NS][KP]
  float* red = sC + NS * KP;         // [waves][2][16][NS]
  float* sjs = red + WB * 2 * 16 * NS;  // SP: [CW][KP] dstep/dv

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int row = lane >> 4;
  const int nl = lane & 15;
  const int c = 4 * w + row;
  const int64_t D = a.D, L = a.L, N = a.N;
  const int64_t nblk = (D + CW - 1) / CW;
  const int64_t blk = blockIdx.x % nblk;
  const int64_t b = blockIdx.x / nblk;
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

  for (int64_t s = s_end - 1; s >= s_begin; --s) {
    const int64_t tb = s * KS;
    const int64_t tl = L - tb < KS ? L - tb : KS;  // valid tokens of the segment
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
    }
    for (int i = tid; i < NS * KS; i += NTHR) {
      const int n = i / KS, t = i % KS;
      const bool ok = n < N && t < tl;
      const int64_t off = (b * N + (n < N ? n : 0)) * L + tb + (t < tl ? t : 0);
      sB[n * KP + t] = ok ? to_f32(Bp[off]) : 0.0f;
      sC[n * KP + t] = ok ? to_f32(Cp[off]) : 0.0f;
    }
    __syncthreads();

    // states at the four chunk starts of the segment
    float hc[4][SPL];
    {
      float h[SPL];
#pragma unroll
      for (int j = 0; j < SPL; ++j) {
        const int64_t n = (int64_t)nl * SPL + j;
        h[j] = sv[j] ? a.hin[s * a.batch * D * N + (b * D + d) * N + n] : 0.0f;
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
#pragma unroll
        for (int j = 0; j < SPL; ++j) hc[k][j] = h[j];
        for (int g = 0; g < 4; ++g) {
          // one group of 4 tokens at a time: the compiler would otherwise
          // hoist every LDS read of the segment and run out of registers
          __builtin_amdgcn_sched_barrier(0);
          const int t = 16 * k + 4 * g;
          const float4 dl4 = *reinterpret_cast<const float4*>(sdl + c * KP + t);
          const float4 x4 = *reinterpret_cast<const float4*>(sx + c * KP + t);
          const float dl[4] = {dl4.x, dl4.y, dl4.z, dl4.w};
          const float u[4] = {dl4.x * x4.x, dl4.y * x4.y, dl4.z * x4.z, dl4.w * x4.w};
#pragma unroll
          for (int j = 0; j < SPL; ++j) {
            const float4 b4 = *reinterpret_cast<const float4*>(sB + (nl * SPL + j) * KP + t);
            const float Bv[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) h[j] = __builtin_fmaf(fast_exp2(dl[i] * A2[j]), h[j], u[i] * Bv[i]);
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
        const float4 x4 = *reinterpret_cast<const float4*>(sx + c * KP + t);
        const float dl[4] = {dl4.x, dl4.y, dl4.z, dl4.w};
        const float u[4] = {dl4.x * x4.x, dl4.y * x4.y, dl4.z * x4.z, dl4.w * x4.w};
#pragma unroll
        for (int j = 0; j < SPL; ++j) {
          const float4 b4 = *reinterpret_cast<const float4*>(sB + (nl * SPL + j) * KP + t);
          const float Bv[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            ea[j][4 * g + i] = fast_exp2(dl[i] * A2[j]);
            hist[j][4 * g + i + 1] = __builtin_fmaf(ea[j][4 * g + i], hist[j][4 * g + i], u[i] * Bv[i]);
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
        const float4 x4 = *reinterpret_cast<const float4*>(sx + c * KP + t4);
        const float4 y4 = *reinterpret_cast<const float4*>(sdyc + c * KP + t4);
        const float dlv[4] = {dl4.x, dl4.y, dl4.z, dl4.w};
        const float xvv[4] = {x4.x, x4.y, x4.z, x4.w};
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
          const float dl = dlv[ii], xv = xvv[ii], dyc = dycv[ii];
          s1[i] = 0.0f;
          s2[i] = 0.0f;
          s3[i] = 0.0f;
#pragma unroll
          for (int j = 0; j < SPL; ++j) {
            const float lam = __builtin_fmaf(dyc, Cv[j][ii], mu[j]);
            mu[j] = ea[j][i] * lam;
            const float r = lam * (ea[j][i] * hist[j][i]);
            s1[i] = __builtin_fmaf(lam, Bv[j][ii], s1[i]);
            s2[i] = __builtin_fmaf(An[j], r, s2[i]);
            s3[i] = __builtin_fmaf(Cv[j][ii], hist[j][i + 1], s3[i]);
            dA[j] = __builtin_fmaf(dl, r, dA[j]);
            pb[j][ii] = lam * (dl * xv);
            pc[j][ii] = dyc * hist[j][i + 1];
          }
          dD = __builtin_fmaf(dyc, xv, dD);
        }
        // the running sums are updated here (left alone, the compiler defers
        // them to the end of the chunk and keeps all their operands live)
#pragma unroll
        for (int j = 0; j < SPL; ++j) asm volatile("" : "+v"(dA[j]), "+v"(mu[j]));
        asm volatile("" : "+v"(dD));
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
          a.dx[off] = __builtin_fmaf(dyc, dsk, dl * k1);
          float gd = __builtin_fmaf(xv, k1, k2);
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

// dB and dC: sums of the per-block partials over the channel blocks.  Four
// running sums (blocks k = 4m + j go to sum j), added at the end in a fixed
// order: the loads of four blocks are in flight at once, and the result does
// not depend on the launch shape.
__global__ void s6_bwd_reduce_bc(const float* __restrict__ part, float* __restrict__ out, int64_t nblk,
                                 int64_t total) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f, s3 = 0.0f;
    int64_t k = 0;
    for (; k + 4 <= nblk; k += 4) {
      s0 += part[k * total + i];
      s1 += part[(k + 1) * total + i];
      s2 += part[(k + 2) * total + i];
      s3 += part[(k + 3) * total + i];
    }
    if (k < nblk) s0 += part[k * total + i];
    if (k + 1 < nblk) s1 += part[(k + 1) * total + i];
    if (k + 2 < nblk) s2 += part[(k + 2) * total + i];
    out[i] = (s0 + s1) + (s2 + s3);
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

// out[i] = v (a fill that a captured graph can hold, unlike a memset node).
__global__ void s6_fill(float* __restrict__ out, float v, int64_t total) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x)
    out[i] = v;
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
  int64_t seg_len;    // tokens per segment, multiple of 4 kT
  bool vec;           // 16-byte staging and 8-byte stores
};

// Compute units of the current device (cached; 256 on MI355X).
int cu_count() {
  static int cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] <= 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

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
    segs = slots / wgs;
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

template <typename In, int VEC, bool GATE, int MODE, int W, bool EXT>
int launch_scan_t(const ScanArgs& a, int64_t batch, int64_t nblk, int64_t segs, hipStream_t st) {
  // 64-byte row runs per load: two chunks per window for bf16 vectors with
  // enough threads to hold them, one chunk otherwise.
  constexpr int WIN = (sizeof(In) == 2 && VEC > 1 && W >= 4) ? 2 : 1;
  size_t lds = (size_t)2 * 2 * kCW * kP * sizeof(float);                       // x, delta tiles
  if (MODE == kModeY && GATE) lds += ((size_t)2 * kCW * kP * sizeof(In) + 15) / 16 * 16;  // gate tile
  if (MODE == kModeY) lds += (size_t)2 * W * 2 * kCW * (kT / 2) * sizeof(float);  // partials
  lds += (size_t)2 * BCLayout<W>::kFloats * sizeof(float);                     // B/C
  dim3 grid((unsigned)(nblk * batch), 1u, (unsigned)segs);
  hipLaunchKernelGGL((s6_scan_kernel<In, VEC, GATE, MODE, W, WIN, EXT>), grid, dim3(64 * W), lds, st, a);
  S6_HIP(hipGetLastError(), "s6_scan_kernel launch");
  return S6_OK;
}

template <typename In, int MODE, int W, bool EXT>
int launch_scan_w(const ScanArgs& a, bool vec, bool gate, int64_t batch, int64_t nblk, int64_t segs,
                  hipStream_t st) {
  constexpr int kV = 16 / sizeof(In);
  if constexpr (MODE == kModeY) {
    if (vec && gate) return launch_scan_t<In, kV, true, MODE, W, EXT>(a, batch, nblk, segs, st);
    if (vec) return launch_scan_t<In, kV, false, MODE, W, EXT>(a, batch, nblk, segs, st);
    if (gate) return launch_scan_t<In, 1, true, MODE, W, EXT>(a, batch, nblk, segs, st);
    return launch_scan_t<In, 1, false, MODE, W, EXT>(a, batch, nblk, segs, st);
  } else {
    if (vec) return launch_scan_t<In, kV, false, MODE, W, EXT>(a, batch, nblk, segs, st);
    return launch_scan_t<In, 1, false, MODE, W, EXT>(a, batch, nblk, segs, st);
  }
}

template <typename In, int MODE, bool EXT>
int launch_scan(const ScanArgs& a, int W, bool vec, bool gate, int64_t batch, int64_t nblk, int64_t segs,
                hipStream_t st) {
  switch (W) {
    case 1: return launch_scan_w<In, MODE, 1, EXT>(a, vec, gate, batch, nblk, segs, st);
    case 2: return launch_scan_w<In, MODE, 2, EXT>(a, vec, gate, batch, nblk, segs, st);
    case 4: return launch_scan_w<In, MODE, 4, EXT>(a, vec, gate, batch, nblk, segs, st);
    default: return launch_scan_w<In, MODE, 8, EXT>(a, vec, gate, batch, nblk, segs, st);
  }
}

template <bool EXT>
int launch_scan_e(int in_dtype, int mode, const ScanArgs& a, const Plan& p, bool gate, int64_t batch,
                  int64_t segs, hipStream_t st) {
  if (in_dtype == S6_BF16) {
    return mode == kModeY ? launch_scan<uint16_t, kModeY, EXT>(a, p.W, p.vec, gate, batch, p.nblk, segs, st)
                          : launch_scan<uint16_t, kModeState, EXT>(a, p.W, p.vec, gate, batch, p.nblk, segs, st);
  }
  return mode == kModeY ? launch_scan<float, kModeY, EXT>(a, p.W, p.vec, gate, batch, p.nblk, segs, st)
                        : launch_scan<float, kModeState, EXT>(a, p.W, p.vec, gate, batch, p.nblk, segs, st);
}

// Kernels with the discretisation options only when an option is set, so
// the plain path keeps its own code.
int launch_scan_any(int in_dtype, int mode, const ScanArgs& a, const Plan& p, bool gate, int64_t batch,
                    int64_t segs, hipStream_t st) {
  if (a.softplus || a.zoh || a.dbias) return launch_scan_e<true>(in_dtype, mode, a, p, gate, batch, segs, st);
  return launch_scan_e<false>(in_dtype, mode, a, p, gate, batch, segs, st);
}

// Shared implementation of s6_scan_fwd(_ex) (want_y) and s6_last_state(_ex).
int scan_impl(bool want_y, int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate, int in_dtype,
              const void* x, const void* delta, const float* dbias, int flags, const float* A,
              const void* Bm, const void* Cm, const float* Dskip, const void* z, const float* h0,
              float* y, float* h_last, void* stream) {
  int rc = check_common(batch, dim, seqlen, dstate, in_dtype);
  if (rc) return rc;
  if (flags & ~(S6_DELTA_SOFTPLUS | S6_ZOH_EXACT)) return S6_ERR_FLAGS;
  if (dbias && !aligned(dbias, 4)) return S6_ERR_ALIGN;
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

  const void* vecptrs[] = {x, delta, Bm, Cm, z, (const void*)y};
  const Plan p = make_plan(batch, dim, seqlen, dstate, esz, vecptrs, 6);
  const bool gate = want_y && z != nullptr;
  const int64_t S = p.segs;

  ScanArgs a;
  memset(&a, 0, sizeof(a));
  a.x = x; a.delta = delta; a.z = gate ? z : nullptr; a.Bm = Bm; a.Cm = want_y ? Cm : nullptr;
  a.A = A; a.Dskip = want_y ? Dskip : nullptr;
  a.softplus = (flags & S6_DELTA_SOFTPLUS) != 0;
  a.zoh = (flags & S6_ZOH_EXACT) != 0;
  a.dbias = dbias;
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
  if (a.dbias || a.softplus || a.zoh) return launch_step_t<In, GATE, P, SPL, G, true>(a, vec, st);
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

// carry: the part-carry kernel (parts 1 .. G-1) instead of the main kernel.
template <typename In, bool GATE, int SPL, bool SP>
int launch_bwd_t(const BwdArgs& a, int64_t parts, bool carry, hipStream_t st) {
  constexpr int CW = 4 * bwd_waves<SPL>();
  const int64_t nblk = (a.D + CW - 1) / CW;
  const dim3 block(64 * bwd_waves<SPL>());
  if (carry) {
    const size_t lds = sizeof(float) * ((size_t)2 * CW * kBwdPitch + (size_t)16 * SPL * kBwdPitch);
    hipLaunchKernelGGL((s6_bwd_carry_kernel<In, GATE, SPL, SP>),
                       dim3((unsigned)(nblk * a.batch), (unsigned)(parts - 1)), block, lds, st, a);
    S6_HIP(hipGetLastError(), "s6_bwd_carry_kernel launch");
  } else {
    hipLaunchKernelGGL((s6_bwd_kernel<In, GATE, SPL, SP>), dim3((unsigned)(nblk * a.batch), (unsigned)parts), block,
                       bwd_lds_bytes<SPL>(SP), st, a);
    S6_HIP(hipGetLastError(), "s6_bwd_kernel launch");
  }
  return S6_OK;
}

template <typename In, int SPL, bool SP>
int launch_bwd_g(const BwdArgs& a, bool gate, int64_t parts, bool carry, hipStream_t st) {
  return gate ? launch_bwd_t<In, true, SPL, SP>(a, parts, carry, st)
              : launch_bwd_t<In, false, SPL, SP>(a, parts, carry, st);
}

template <typename In>
int launch_bwd(const BwdArgs& a, bool gate, int64_t parts, bool carry, hipStream_t st) {
  const bool sp = a.dbias || a.softplus || a.ddbias_part;
  if (a.N <= 16)
    return sp ? launch_bwd_g<In, 1, true>(a, gate, parts, carry, st) : launch_bwd_g<In, 1, false>(a, gate, parts, carry, st);
  return sp ? launch_bwd_g<In, 2, true>(a, gate, parts, carry, st) : launch_bwd_g<In, 2, false>(a, gate, parts, carry, st);
}

int bwd_channels_per_block(int64_t dstate) { return dstate <= 16 ? 4 * bwd_waves<1>() : 4 * bwd_waves<2>(); }

void fill(float* p, float v, int64_t n, hipStream_t st) {
  if (!p || n <= 0) return;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(s6_fill, dim3((unsigned)blocks), dim3(256), 0, st, p, v, n);
}

}  // namespace

extern "C" {

int s6_version(void) { return 10100; }

const char* s6_status_str(int status) {
  switch (status) {
    case S6_OK: return "ok";
    case S6_ERR_NULL: return "a required pointer is NULL";
    case S6_ERR_SHAPE: return "invalid size (negative, or the element count overflows)";
    case S6_ERR_DTYPE: return "in_dtype must be S6_F32 or S6_BF16";
    case S6_ERR_UNSUPPORTED: return "dstate must be between 1 and 32";
    case S6_ERR_ALIGN: return "a pointer is not aligned to its element size";
    case S6_ERR_FLAGS: return "unknown option bits in flags";
    case S6_ERR_HIP: return g_err[0] ? g_err : "HIP error";
    default: return "unknown status";
  }
}

int s6_scan_fwd(int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate, int in_dtype,
                const void* x, const void* delta, const float* A, const void* Bm, const void* Cm,
                const float* Dskip, const void* z, const float* h0, float* y, float* h_last,
                void* stream) {
  return scan_impl(true, batch, dim, seqlen, dstate, in_dtype, x, delta, nullptr, 0, A, Bm, Cm, Dskip,
                   z, h0, y, h_last, stream);
}

int s6_scan_fwd_ex(int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate, int in_dtype,
                   const void* x, const void* delta, const float* delta_bias, int flags,
                   const float* A, const void* Bm, const void* Cm, const float* Dskip, const void* z,
                   const float* h0, float* y, float* h_last, void* stream) {
  return scan_impl(true, batch, dim, seqlen, dstate, in_dtype, x, delta, delta_bias, flags, A, Bm, Cm,
                   Dskip, z, h0, y, h_last, stream);
}

int s6_last_state(int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate, int in_dtype,
                  const void* x, const void* delta, const float* A, const void* Bm,
                  const float* h0, float* h_last, void* stream) {
  return scan_impl(false, batch, dim, seqlen, dstate, in_dtype, x, delta, nullptr, 0, A, Bm, nullptr,
                   nullptr, nullptr, h0, nullptr, h_last, stream);
}

int s6_last_state_ex(int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate, int in_dtype,
                     const void* x, const void* delta, const float* delta_bias, int flags,
                     const float* A, const void* Bm, const float* h0, float* h_last, void* stream) {
  return scan_impl(false, batch, dim, seqlen, dstate, in_dtype, x, delta, delta_bias, flags, A, Bm,
                   nullptr, nullptr, nullptr, h0, nullptr, h_last, stream);
}

int s6_state_update_ex(int64_t batch, int64_t dim, int64_t dstate, int in_dtype, float* h,
                       const void* x, const void* delta, const float* delta_bias, int flags,
                       const float* A, const void* Bm, const void* Cm, const float* Dskip,
                       const void* z, float* y, void* stream) {
  int rc = check_common(batch, dim, 1, dstate, in_dtype);
  if (rc) return rc;
  if (flags & ~(S6_DELTA_SOFTPLUS | S6_ZOH_EXACT)) return S6_ERR_FLAGS;
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
  a.batch = batch; a.D = dim; a.N = dstate;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (in_dtype == S6_BF16)
    return z ? launch_step_g<uint16_t, true>(a, st) : launch_step_g<uint16_t, false>(a, st);
  return z ? launch_step_g<float, true>(a, st) : launch_step_g<float, false>(a, st);
}

int s6_state_update(int64_t batch, int64_t dim, int64_t dstate, int in_dtype, float* h,
                    const void* x, const void* delta, const float* A, const void* Bm,
                    const void* Cm, const float* Dskip, const void* z, float* y, void* stream) {
  return s6_state_update_ex(batch, dim, dstate, in_dtype, h, x, delta, nullptr, 0, A, Bm, Cm, Dskip, z,
                            y, stream);
}

int s6_scan_bwd_ex(int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate, int in_dtype,
                   const void* x, const void* delta, const float* delta_bias, int flags, const float* A,
                   const void* Bm, const void* Cm, const float* Dskip, const void* z, const float* h0,
                   const float* dy, const float* dh_last, float* dx, float* ddelta, float* dA, float* dBm,
                   float* dCm, float* dDskip, float* dz, float* dh0, float* ddelta_bias, void* stream) {
  int rc = check_common(batch, dim, seqlen, dstate, in_dtype);
  if (rc) return rc;
  if (flags & ~(S6_DELTA_SOFTPLUS | S6_ZOH_EXACT)) return S6_ERR_FLAGS;
  if (flags & S6_ZOH_EXACT) return S6_ERR_UNSUPPORTED;
  const bool softplus = (flags & S6_DELTA_SOFTPLUS) != 0;
  const bool work = batch > 0 && dim > 0 && seqlen > 0;
  if (dim > 0 && !dA) return S6_ERR_NULL;
  if (work && (!x || !delta || !A || !Bm || !Cm || !dy || !dx || !ddelta || !dBm || !dCm))
    return S6_ERR_NULL;
  const size_t esz = in_dtype == S6_BF16 ? 2 : 4;
  const void* ins[] = {x, delta, Bm, Cm, z};
  for (const void* p : ins)
    if (p && !aligned(p, esz)) return S6_ERR_ALIGN;
  const void* f32s[] = {A, Dskip, h0, dy, dh_last, dx, ddelta, dA, dBm, dCm, dDskip, dz, dh0, delta_bias,
                        ddelta_bias};
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
    if (dh0 && nstate > 0) {
      int64_t blocks = (nstate + 255) / 256;
      if (blocks > 65536) blocks = 65536;
      hipLaunchKernelGGL(s6_copy_state, dim3((unsigned)blocks), dim3(256), 0, st, dh_last, dh0, nstate);
    }
    S6_HIP(hipGetLastError(), "s6_scan_bwd fill");
    return S6_OK;
  }

  // workspace: segment states (pass 1, fold), per-row and per-block partials
  const int64_t S = (seqlen + kBwdSeg - 1) / kBwdSeg;
  const int64_t nagg = S - 1;
  const int64_t cw = bwd_channels_per_block(dstate);
  const int64_t nblkb = (dim + cw - 1) / cw;
  // Parts: when the (row, channel block) workgroups fill less than half of
  // the workgroup slots (few long rows), the sequence is cut into parts run
  // side by side; the adjoint carry entering each part from the right comes
  // from a carry pass and a fold.
  int64_t G = 1;
  {
    const int64_t wgs = nblkb * batch;
    const int64_t slots = (int64_t)cu_count() * (dstate <= 16 ? 4 : 3);
    if (2 * wgs <= slots) G = slots / wgs < S ? slots / wgs : S;
    if (G < 1) G = 1;
  }
  const int64_t spp = (S + G - 1) / G;  // segments per part
  G = (S + spp - 1) / spp;
  auto up = [](size_t v) { return (v + 255) & ~(size_t)255; };
  const size_t agg_b = (size_t)(nagg > 0 ? nagg : 0) * nstate * sizeof(float);
  const size_t sd_b = (size_t)(nagg > 0 ? nagg : 0) * batch * dim * sizeof(float);
  const size_t hin_b = (size_t)S * nstate * sizeof(float);
  const size_t dap_b = (size_t)G * nstate * sizeof(float);
  const size_t ddp_b = (size_t)G * batch * dim * sizeof(float);
  const size_t bc_b = (size_t)nblkb * batch * dstate * seqlen * sizeof(float);
  const size_t mu_b = G > 1 ? (size_t)G * nstate * sizeof(float) : 0;     // carries: M and mu_in
  const size_t csd_b = G > 1 ? (size_t)G * batch * dim * sizeof(float) : 0;
  const size_t total = up(agg_b) + up(sd_b) + up(hin_b) + up(dap_b) + 2 * up(ddp_b) + 2 * up(bc_b) + 2 * up(mu_b) +
                       up(csd_b);
  void* ws = nullptr;
  S6_HIP(hipMallocAsync(&ws, total, st), "hipMallocAsync(backward workspace)");
  char* wp = static_cast<char*>(ws);
  float* agg = reinterpret_cast<float*>(wp);
  wp += up(agg_b);
  float* sd = reinterpret_cast<float*>(wp);
  wp += up(sd_b);
  float* hin = reinterpret_cast<float*>(wp);
  wp += up(hin_b);
  float* dap = reinterpret_cast<float*>(wp);
  wp += up(dap_b);
  float* ddp = reinterpret_cast<float*>(wp);
  wp += up(ddp_b);
  float* dbp = reinterpret_cast<float*>(wp);  // bias gradient per part and row
  wp += up(ddp_b);
  float* dBp = reinterpret_cast<float*>(wp);
  wp += up(bc_b);
  float* dcp = reinterpret_cast<float*>(wp);
  wp += up(bc_b);
  float* cM = reinterpret_cast<float*>(wp);
  wp += up(mu_b);
  float* muin = reinterpret_cast<float*>(wp);
  wp += up(mu_b);
  float* cSD = reinterpret_cast<float*>(wp);

  // pass 1: end state (from zero) and summed delta of every segment but the last
  if (nagg > 0) {
    const void* vecptrs[] = {x, delta, Bm};
    Plan p = make_plan(batch, dim, seqlen, dstate, esz, vecptrs, 3);
    ScanArgs g;
    memset(&g, 0, sizeof(g));
    g.x = x; g.delta = delta; g.Bm = Bm; g.A = A;
    g.hout = agg; g.hout_stride = nstate; g.sumdelta = sd;
    g.dbias = delta_bias; g.softplus = softplus;
    g.D = dim; g.L = seqlen; g.N = dstate; g.seg_len = kBwdSeg;
    rc = launch_scan_any(in_dtype, kModeState, g, p, false, batch, nagg, st);
  }
  // the state entering every segment
  if (rc == S6_OK) {
    const int64_t blocks = (nstate + 255) / 256;
    hipLaunchKernelGGL(s6_fold_carries, dim3((unsigned)blocks), dim3(256), 0, st, A, h0, agg, sd, hin,
                       nullptr, batch, dim, dstate, S, nagg);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) rc = hip_fail(e, "s6_fold_carries launch");
  }
  if (rc == S6_OK) {
    BwdArgs b;
    memset(&b, 0, sizeof(b));
    b.x = x; b.delta = delta; b.z = z; b.Bm = Bm; b.Cm = Cm; b.A = A; b.Dskip = Dskip;
    b.dy = dy; b.dh_last = dh_last; b.hin = hin;
    b.dx = dx; b.ddelta = ddelta; b.dz = dz; b.dA_part = dap; b.dD_part = ddp;
    b.dB_part = dBp; b.dC_part = dcp; b.dh0 = dh0;
    b.dbias = delta_bias; b.softplus = softplus; b.ddbias_part = ddelta_bias ? dbp : nullptr;
    b.batch = batch; b.D = dim; b.L = seqlen; b.N = dstate; b.nseg = S; b.seg_per_part = spp;
    const bool gate = z != nullptr;
    if (G > 1) {
      b.carry_M = cM;
      b.carry_SD = cSD;
      rc = in_dtype == S6_BF16 ? launch_bwd<uint16_t>(b, gate, G, true, st) : launch_bwd<float>(b, gate, G, true, st);
      if (rc == S6_OK) {
        hipLaunchKernelGGL(s6_bwd_fold, dim3((unsigned)((nstate + 255) / 256)), dim3(256), 0, st, A, dh_last, cM, cSD,
                           muin, batch, dim, dstate, G);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) rc = hip_fail(e, "s6_bwd_fold launch");
      }
      b.mu_in = muin;
    }
    if (rc == S6_OK)
      rc = in_dtype == S6_BF16 ? launch_bwd<uint16_t>(b, gate, G, false, st) : launch_bwd<float>(b, gate, G, false, st);
  }
  if (rc == S6_OK) {
    const int64_t tot = batch * dstate * seqlen;
    int64_t blocks = (tot + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(s6_bwd_reduce_bc, dim3((unsigned)blocks), dim3(256), 0, st, dBp, dBm, nblkb, tot);
    hipLaunchKernelGGL(s6_bwd_reduce_bc, dim3((unsigned)blocks), dim3(256), 0, st, dcp, dCm, nblkb, tot);
    const int64_t rows = dim * dstate;
    hipLaunchKernelGGL(s6_bwd_reduce_rows, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, st, dap, ddp, dbp,
                       dA, dDskip, ddelta_bias, G * batch, dim, dstate);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) rc = hip_fail(e, "s6_bwd reduction launch");
  }
  hipError_t e = hipFreeAsync(ws, st);
  if (rc == S6_OK && e != hipSuccess) rc = hip_fail(e, "hipFreeAsync(backward workspace)");
  return rc;
}

int s6_scan_bwd(int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate, int in_dtype,
                const void* x, const void* delta, const float* A, const void* Bm, const void* Cm,
                const float* Dskip, const void* z, const float* h0, const float* dy,
                const float* dh_last, float* dx, float* ddelta, float* dA, float* dBm, float* dCm,
                float* dDskip, float* dz, float* dh0, void* stream) {
  return s6_scan_bwd_ex(batch, dim, seqlen, dstate, in_dtype, x, delta, nullptr, 0, A, Bm, Cm, Dskip, z, h0, dy,
                        dh_last, dx, ddelta, dA, dBm, dCm, dDskip, dz, dh0, nullptr, stream);
}

}  // extern "C"
