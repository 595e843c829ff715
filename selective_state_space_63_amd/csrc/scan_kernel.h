// scan_kernel.h -- the fused selective-scan kernel template and its launch
// helpers, shared by scan.hip (plain kernels and the host side) and
// scan_ext.hip, scan_conv.hip, scan_hold.hip (the kernels with the step
// options and the convolution front).  Internal to libs6.
//
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
//  * The convolution front (option kernels): the threads that stage x
//    pieces replace them by SiLU(bias + causal filter * x) before writing
//    the tile, so the scan, the skip term and the state-only passes all see
//    the filtered input and it never goes to memory.  The three inputs
//    before a piece come from the neighbouring lane's piece (DPP), or from
//    the previous chunk's last piece, which its lane keeps in registers.
//  * Few long rows (too few workgroups to fill the GPU) are cut into
//    segments along L: pass 1 computes every segment's end state from zero
//    and its summed delta, a tiny pass folds them into each segment's
//    incoming state (associativity of the (a, b) pairs), and pass 2 runs the
//    fused scan of every segment from its incoming state.
#ifndef S6_SCAN_KERNEL_H_
#define S6_SCAN_KERNEL_H_

#include "s6_internal.h"

namespace s6i {

namespace {

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
// 4-slot quarters of a block are permuted by XOR with f(g, w), readers
// applying the same permutation, so lane x of a row still receives slot x.
// A staging write covers groups g and g + 2 of one state (16-byte writes
// take 8 lanes per cycle over 32 banks on gfx950: two pair members x two
// groups x two row parities must fill the 32 banks), so bit 1 of f flips
// between g and g + 2.  States beyond N stay zero.
template <int W>
struct BCLayout {
  static constexpr int kFloats = (kT / 4) * W * 2 * 16;  // floats per chunk
  __device__ __forceinline__ static int quarter(int g, int w, int q) { return q ^ (((g >> 1) & 1) << 1) ^ (w & 3); }
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
// EXT kernels also take the step bias and discretisation options of ScanArgs
// (EXT 1: bias and softplus; 3: and the convolution front; 2: and the exact
// hold): the bias and softplus are applied to delta while it is staged (once
// per element), the convolution front to x the same way, the exact hold in
// the token groups, and the kind of piece each wave stages rotates with the
// workgroup index so that this extra work falls on every SIMD alike.
template <typename In, int VEC, bool GATE, int MODE, int W, int WIN, int EXT, bool CK>
__global__ void __launch_bounds__(64 * W)
    __attribute__((amdgpu_waves_per_eu(W == 4 ? ((EXT == 0 || (EXT == 1 && VEC > 1 && !CK)) ? 5 : 4) : 1)))
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
  // Workgroup -> (segment, batch row, channel block).  The dispatcher
  // hands workgroups to the 8 XCDs in turn (linear id i to XCD i mod 8) and
  // each XCD has its own L2.  Without segments the ids are remapped to give
  // every XCD a contiguous run of the (row, block) order (a bijection for
  // any count): the workgroups of one batch row, which read the same B and
  // C, then share one L2 (3B layer: one batch row per XCD; 0.9% faster).
  // Segmented grids keep the plain order: the same remap over (segment,
  // block) made the million-token scan 1.5% slower.
  uint32_t wgx = blockIdx.x, wgz = blockIdx.z;
  if (gridDim.z == 1) {
    const uint32_t nx = gridDim.x;
    const uint32_t q = nx / 8, rem = nx % 8, xcd = wgx % 8;
    wgx = xcd * q + (xcd < rem ? xcd : rem) + wgx / 8;
  }
  const int64_t b = wgx / nblk;
  const int64_t d0 = (int64_t)(wgx % nblk) * kCW;
  const int64_t d = d0 + cl;
  const bool chv = d < D;
  const int64_t rows_valid = D - d0;
  const int64_t seg = wgz;
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
  // Checkpoints (fused pass): the state entering every kCkpt-token block of
  // this segment, the first one being the segment's incoming state.
  // (The offsets are rebuilt from the thread index here, inside the rarely
  // taken branch: values kept from outside would hold registers through the
  // whole chunk loop.)
  // (The state-only kernels write the states the backward's adjoint kernel
  // starts from: every kCkpt tokens, or every chunk when a.ckpt_log2 is 4.)
  const int ck_shift = MODE == kModeState ? a.ckpt_log2 : 6;  // log2 of kT or kCkpt
  static_assert(kT == 16 && kCkpt == 64, "checkpoint strides");
  // uniform: elements per checkpoint and this block's first one (a division
  // here, not inside the chunk loop)
  const int64_t ck_nst = (int64_t)(gridDim.x / nblk) * D * N;
  const int64_t ck_off = (b * D + d0) * N;
  auto write_ckpt = [&](int64_t tok) {
    float* base = a.ckpt + (tok >> ck_shift) * ck_nst + ck_off;  // uniform
    const int ln = (int)threadIdx.x & 63;
    const int c = ((ln >> 5) << 4) | (ln & 15);
    const int n0 = ((int)threadIdx.x >> 6) * 4 + 2 * ((ln >> 4) & 1);
    if (c < rows_valid) {
      if ((N & 1) == 0 && n0 + 1 < N) {  // both states, 8-byte aligned
        *reinterpret_cast<float2*>(base + c * N + n0) = make_float2(h[0], h[1]);
      } else {
        if (n0 < N) base[c * N + n0] = h[0];
        if (n0 + 1 < N) base[c * N + n0 + 1] = h[1];
      }
    }
  };
  // The plain and step-bias kernels write checkpoints only in their CK
  // instantiations (the write in the chunk loop costs registers); the
  // exact-hold and convolution y kernels check a.ckpt.
  constexpr bool kCk = CK || (MODE == kModeY && EXT >= 2);
  if (kCk && a.ckpt && tb < te) write_ckpt(tb);
  // Sum of delta over the segment (state mode), compensated (Neumaier):
  // dsum + dcomp.  (A double accumulator here costs dozens of registers.)
  // The checkpoint-writing state kernels (one segment) write no sum.
  constexpr bool kSum = MODE == kModeState && !CK;
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
  const bool zoh = EXT == 2 && a.zoh;
  const int rot = EXT ? (int)(wgx % W) * 64 : 0;
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

  // Convolution front: per slot the filter taps newest first (cwr[j] weighs
  // the input j tokens back; taps past the width are 0), the bias, and the
  // inputs carried over from the previous chunk: elements VEC-3 .. VEC-1 of
  // this lane's piece (only the last piece of a row passes them on), or the
  // single element (VEC == 1).  Before the segment's first chunk they are
  // the inputs before it: x itself, or conv_state / 0 before token 0.
  const bool conv = EXT >= 2 && a.conv_w != nullptr;
  constexpr int NCAR = VEC == 1 ? 1 : 3;
  float cwr[SLOTS][kMaxConv], cbias[SLOTS], carry[SLOTS][NCAR];
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) {
#pragma unroll
    for (int j = 0; j < kMaxConv; ++j) cwr[s][j] = 0.0f;
    cbias[s] = 0.0f;
#pragma unroll
    for (int j = 0; j < NCAR; ++j) carry[s][j] = 0.0f;
    if (conv && skind[s] == 0) {
      const int K = a.conv_k;
      const int64_t rowc = srow[s] < rows_valid ? srow[s] : rows_valid - 1;
      const int64_t ch = d0 + rowc;
      for (int j = 0; j < K; ++j) cwr[s][j] = a.conv_w[ch * K + (K - 1 - j)];
      if (a.conv_b) cbias[s] = a.conv_b[ch];
#pragma unroll
      for (int j = 0; j < NCAR; ++j) {
        const int64_t u = tb - kT + scol[s] + (VEC == 1 ? 0 : VEC - 3 + j);  // token of the carried input
        if (u >= 0) {
          carry[s][j] = to_f32(sptr[s][u - scol[s]]);
        } else if (a.conv_state && u >= -(int64_t)(K - 1)) {
          carry[s][j] = a.conv_state[(b * D + ch) * (K - 1) + (K - 1) + u];
        }
      }
    }
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
      const In* e = reinterpret_cast<const In*>(&src_[s]);
      // Convolution front (all lanes take part in the exchange; x lanes use it).
      float xf[VEC];
      if (conv) {
        float cur[VEC], prev[3];  // prev[i]: the input 3 - i tokens before the piece
#pragma unroll
        for (int k = 0; k < VEC; ++k) cur[k] = to_f32(e[k]);
        if constexpr (VEC == 1) {
          // the 16 pieces of a row are the 16 lanes of a DPP row: lane q
          // reads lane q - i (rotating; lanes 16 - i .. 15 send the previous
          // chunk's element)
          const int q = lane & 15;
          prev[2] = dpp_f<0x121>(q >= 15 ? carry[s][0] : cur[0]);
          prev[1] = dpp_f<0x122>(q >= 14 ? carry[s][0] : cur[0]);
          prev[0] = dpp_f<0x123>(q >= 13 ? carry[s][0] : cur[0]);
          carry[s][0] = cur[0];
        } else {
          // the PPC pieces of a row sit in PPC adjacent lanes; piece q reads
          // piece q - 1, the first piece the last one (which sends the
          // previous chunk's inputs)
          static_assert(CP::PPC == 2 || CP::PPC == 4, "pieces per row");
          constexpr int CTRL = CP::PPC == 2 ? 0xB1 : 0x93;  // quad_perm [1,0,3,2] / [3,0,1,2]
          const bool lastp = col == (CP::PPC - 1) * VEC;
#pragma unroll
          for (int j = 0; j < 3; ++j) {
            prev[j] = dpp_f<CTRL>(lastp ? carry[s][j] : cur[VEC - 3 + j]);
            carry[s][j] = cur[VEC - 3 + j];
          }
        }
        if (skind[s] == 0) {
#pragma unroll
          for (int k = 0; k < VEC; ++k) {
            float acc = cbias[s];
#pragma unroll
            for (int j = 0; j < kMaxConv; ++j) {
              const float v = k - j >= 0 ? cur[k - j] : prev[3 + k - j];
              acc = __builtin_fmaf(cwr[s][j], v, acc);
            }
            xf[k] = silu(acc);
          }
        }
      }
      if (skind[s] < 0) continue;
      const bool ok = !MASK || t0c + col < te;
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
      } else if (conv && skind[s] == 0) {
        float* tile = tiles + buf * 2 * TILE;
        if constexpr (VEC == 1) {
          tile[tsw(srow[s], col >> 2) + (col & 3)] = ok ? xf[0] : 0.0f;
        } else {
#pragma unroll
          for (int k = 0; k < VEC; k += 4)
            *reinterpret_cast<float4*>(tile + tsw(srow[s], (col + k) >> 2)) =
                ok ? make_float4(xf[k], xf[k + 1], xf[k + 2], xf[k + 3]) : make_float4(0.f, 0.f, 0.f, 0.f);
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
      token_group<MODE, EXT == 2>(dl, xv, A2, h, bc, zoh, ys);
      ysum[2 * g] = ys[0];
      ysum[2 * g + 1] = ys[1];
      if constexpr (kSum) cs += (dl[0] + dl[1]) + (dl[2] + dl[3]);
    }
    // The chunk's state updates (and delta sum) complete here.  (Without
    // output terms nothing else ties them to the chunk, and the compiler would
    // sink them past the barriers, keeping every chunk's inputs live at once.)
    asm volatile("" : "+v"(h[0]), "+v"(h[1]), "+v"(cs));
    if constexpr (kCk && MODE == kModeY) {
      // A block ends with this chunk: segments start at multiples of kCkpt
      // tokens, so with 4-chunk cycles only the cycle's last chunk can end one.
      if constexpr (2 * WIN != 4 || P == 3) {
        const int64_t tn = t0 + kT;  // tokens done after this chunk
        if (a.ckpt && (tn & (kCkpt - 1)) == 0 && tn < te) write_ckpt(tn);
      }
    }
    float* pbuf = part + buf * (W * PART);
    if constexpr (MODE == kModeY) {
      // ysum[i] is this wave's sum for token 2i + r: part[buf][w][r][cl][i],
      // the two halves of the row swapped for channels with bit 2 set (so
      // the 16-byte writes of 8 consecutive channels meet no bank twice)
      float* pp = pbuf + w * PART + (r * kCW + cl) * (kT / 2);
      const int sw = cl & 4;
      *reinterpret_cast<float4*>(pp + sw) = make_float4(ysum[0], ysum[1], ysum[2], ysum[3]);
      *reinterpret_cast<float4*>(pp + (sw ^ 4)) = make_float4(ysum[4], ysum[5], ysum[6], ysum[7]);
    }
    if constexpr (kSum) {
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
    if constexpr (kCk && MODE == kModeState) {
      // the state after chunk k when a stride ends with it, stored after the
      // window's loads are issued (as the y kernels store y)
      const int64_t tn = t0 + kT;
      if (a.ckpt && (tn & ((1 << ck_shift) - 1)) == 0 && tn < te) write_ckpt(tn);
    }

    if constexpr (MODE == kModeY) {
      float yo[TPL];
#pragma unroll
      for (int i = 0; i < TPL; ++i) {
        const int t = ft + i;  // token within the chunk
        float acc = 0.0f;
#pragma unroll
        for (int ww = 0; ww < W; ++ww) acc += pbuf[ww * PART + ((t & 1) * kCW + fc) * (kT / 2) + ((t >> 1) ^ (fc & 4))];
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
  if constexpr (kSum) {
    if (a.sumdelta && chv && w == 0 && r == 0)
      a.sumdelta[seg * (int64_t)(gridDim.x / nblk) * D + b * D + d] = dsum + dcomp;
  }
}

template <typename In, int VEC, bool GATE, int MODE, int W, int EXT, bool CK>
int launch_scan_t(const ScanArgs& a, int64_t batch, int64_t nblk, int64_t segs, hipStream_t st) {
  // 64-byte row runs per load: two chunks per window for bf16 vectors with
  // enough threads to hold them, one chunk otherwise.
  constexpr int WIN = (sizeof(In) == 2 && VEC > 1 && W >= 4) ? 2 : 1;
  size_t lds = (size_t)2 * 2 * kCW * kP * sizeof(float);                       // x, delta tiles
  if (MODE == kModeY && GATE) lds += ((size_t)2 * kCW * kP * sizeof(In) + 15) / 16 * 16;  // gate tile
  if (MODE == kModeY) lds += (size_t)2 * W * 2 * kCW * (kT / 2) * sizeof(float);  // partials
  lds += (size_t)2 * BCLayout<W>::kFloats * sizeof(float);                     // B/C
  dim3 grid((unsigned)(nblk * batch), 1u, (unsigned)segs);
  hipLaunchKernelGGL((s6_scan_kernel<In, VEC, GATE, MODE, W, WIN, EXT, CK>), grid, dim3(64 * W), lds, st, a);
  S6_HIP(hipGetLastError(), "s6_scan_kernel launch");
  return S6_OK;
}

// The checkpoint-writing instantiation when a.ckpt is set: of the plain and
// step-bias y kernels and of every state-only kernel (the convolution and
// exact-hold y kernels write them whenever it is set).
template <typename In, int VEC, bool GATE, int MODE, int W, int EXT>
int launch_scan_c(const ScanArgs& a, int64_t batch, int64_t nblk, int64_t segs, hipStream_t st) {
  if constexpr (EXT <= 1 || MODE == kModeState) {
    if (a.ckpt) return launch_scan_t<In, VEC, GATE, MODE, W, EXT, true>(a, batch, nblk, segs, st);
  }
  return launch_scan_t<In, VEC, GATE, MODE, W, EXT, false>(a, batch, nblk, segs, st);
}

template <typename In, int MODE, int W, int EXT>
int launch_scan_w(const ScanArgs& a, bool vec, bool gate, int64_t batch, int64_t nblk, int64_t segs,
                  hipStream_t st) {
  constexpr int kV = 16 / sizeof(In);
  if constexpr (MODE == kModeY) {
    if (vec && gate) return launch_scan_c<In, kV, true, MODE, W, EXT>(a, batch, nblk, segs, st);
    if (vec) return launch_scan_c<In, kV, false, MODE, W, EXT>(a, batch, nblk, segs, st);
    if (gate) return launch_scan_c<In, 1, true, MODE, W, EXT>(a, batch, nblk, segs, st);
    return launch_scan_c<In, 1, false, MODE, W, EXT>(a, batch, nblk, segs, st);
  } else {
    if (vec) return launch_scan_c<In, kV, false, MODE, W, EXT>(a, batch, nblk, segs, st);
    return launch_scan_c<In, 1, false, MODE, W, EXT>(a, batch, nblk, segs, st);
  }
}

template <typename In, int MODE, int EXT>
int launch_scan(const ScanArgs& a, int W, bool vec, bool gate, int64_t batch, int64_t nblk, int64_t segs,
                hipStream_t st) {
  switch (W) {
    case 1: return launch_scan_w<In, MODE, 1, EXT>(a, vec, gate, batch, nblk, segs, st);
    case 2: return launch_scan_w<In, MODE, 2, EXT>(a, vec, gate, batch, nblk, segs, st);
    case 4: return launch_scan_w<In, MODE, 4, EXT>(a, vec, gate, batch, nblk, segs, st);
    default: return launch_scan_w<In, MODE, 8, EXT>(a, vec, gate, batch, nblk, segs, st);
  }
}

// EXT: 0 the plain kernels; 1 the step bias and softplus (few enough
// registers for five waves per SIMD); 3 those and the convolution front; 2
// all of them and the exact hold.  Each level costs registers.
template <int EXT>
int launch_scan_e(int in_dtype, int mode, const ScanArgs& a, const Plan& p, bool gate, int64_t batch,
                  int64_t segs, hipStream_t st) {
  if (in_dtype == S6_BF16) {
    return mode == kModeY ? launch_scan<uint16_t, kModeY, EXT>(a, p.W, p.vec, gate, batch, p.nblk, segs, st)
                          : launch_scan<uint16_t, kModeState, EXT>(a, p.W, p.vec, gate, batch, p.nblk, segs, st);
  }
  return mode == kModeY ? launch_scan<float, kModeY, EXT>(a, p.W, p.vec, gate, batch, p.nblk, segs, st)
                        : launch_scan<float, kModeState, EXT>(a, p.W, p.vec, gate, batch, p.nblk, segs, st);
}

}  // namespace

}  // namespace s6i

#endif  // S6_SCAN_KERNEL_H_
