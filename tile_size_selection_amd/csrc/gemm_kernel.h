// Multi-level tiled GEMM for gfx950:  C[b] = A[b] x B[b], fp16/bf16 inputs,
// fp32 accumulation.
//
// The hierarchy is the one of the "Tiling（分块）" page's multi-level tiling
// section, mapped onto CDNA4:
//   block  : a BM x BN tile of C per workgroup; A (BM x BK) and B (BK x BN)
//            slices staged HBM -> LDS once per K step and reused by every wave
//   wave   : the block splits into WM x WN waves, each owning a
//            (BM/WM) x (BN/WN) sub-tile held in accumulation registers
//   MFMA   : v_mfma_f32_32x32x16 or v_mfma_f32_16x16x32 on LDS fragments
//
// Memory-hierarchy techniques of the same page, in their gfx950 form:
//   * staging with a multi-stage pipeline: `stages` LDS buffers in a ring;
//     the next stages-1 K tiles are in flight while one tile is computed.
//     The copy is a direct HBM->LDS buffer load (buffer_load_dwordx4 ... lds)
//     that bypasses registers, the analogue of the page's asynchronous copy,
//     so several tiles are in flight without holding registers.  In the GEMM
//     loop the copies are spread between the MFMAs and the next tile's
//     fragments are read before the barrier that frees a stage (see the loop);
//   * coalescing: each load instruction moves 64 lanes x 16 B = 1 KiB of whole
//     rows;
//   * bank-conflict-free LDS: 16-byte chunks are XOR-swizzled per row (the
//     page's row-xor-column remapping) for 64 banks of 4 bytes;
//   * B is row-major K x N: its fragments are read with the gfx950 LDS
//     transpose read (ds_read_b64_tr_b16) instead of being transposed on the
//     way in.
// Ragged edges: a 16-byte chunk outside the operand is given an offset past
// the buffer's range, so the hardware range check writes zeros into LDS; the
// epilogue masks rows >= M and columns >= N.
//
// The same kernel computes a convolution as an implicit GEMM (CONV = true).
// A is the weight matrix Cout x (kh*kw*Cp) with K ordered (r, s, ci), each
// tap's channels padded to Cp (a multiple of BK); it is loaded like the
// GEMM's A, the columns of a K tile taken from the tap cursor.  B is the
// im2col matrix of one output tile (images x output rows x output columns),
// stored in LDS transposed (pixels x K, laid out like A) and copied
// HBM -> LDS from a channel-last input, 16 bytes (8 channels of one input
// pixel) per lane.  The operands are either the caller's channel-last
// tensors (NHWC input, OHWI weights) or copies of NCHW / OIHW ones made by
// conv_layout.h.  The batch index of the GEMM is the tile.  Each block
// derives its input rows and columns and the sub-operator pads from the
// Tiling page's H/W tiling formulas; chunks that fall in a pad, outside the
// slice or past the channels read as zero.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

#include "../../include/tss.h"

namespace tss {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) i16x8 lds_i16x8;

struct KernelArgs {
  const void *A;  // GEMM: A[batch][M][K].       conv: weights w[Cout][kh][kw][Cs]
  const void *B;  // GEMM: B[batch][K][N].       conv: input x[Nb][H][W][Cs] (channel-last)
  void *C;        // GEMM: C[batch][M][N].       conv: output y[Nb][Cout][OH][OW]
  int32_t M, N, K;  // conv: M = Cout, K = kh*kw*Cp, N = pixels of a full tile; lda = kh*kw*Cs
  int32_t tiles_m, tiles_n;
  int32_t group_m;    // tile rows per group of the L2-friendly tile order
  int32_t out_dtype;  // TSS_F32 / TSS_F16 / TSS_BF16
  int64_t batch_stride_a, batch_stride_b;  // GEMM only, elements
  // C: GEMM, elements between the outputs of consecutive (batch, K range)
  // pairs; conv, elements between the outputs of consecutive K ranges
  int64_t batch_stride_c;
  // Split K: the block's z index (batch entry or conv tile) is split into
  // `splits` K ranges of k_split elements (a multiple of BK; the last range
  // holds the rest), each computed by its own blocks into its own output
  // slice (fp32 partial sums, added up by splitk_reduce_kernel).
  // splits == 1, k_split == K: the plain GEMM.  lda: A's row stride.
  int32_t splits, k_split, lda;
  // convolution geometry (CONV only).  The output is cut into tiles of
  // tile_n images x tile_oh rows x tile_ow columns; the GEMM batch index is
  // the tile, (image group * n_ht + row tile) * n_wt + column tile.
  int32_t Nb, Cin, H, W, kh, kw, sh, sw, ph, pw, dh, dw, OH, OW, tile_oh;
  int32_t Cp;  // K per tap: Cin rounded up to a multiple of BK (a K tile is one tap)
  int32_t Cs;  // channels per pixel in memory: B's pixel stride and A's stride per tap (Cp or Cin)
  int32_t tile_ow, tile_n, n_ht, n_wt;
  int32_t y_nhwc;  // output y[Nb][OH][OW][Cout] (channel-last) instead of y[Nb][Cout][OH][OW]
};

// ---- small device helpers --------------------------------------------------

constexpr uint32_t kOOB = 0x80000000u;  // voffset beyond any accepted buffer range

// GEMM main loop: MFMA rows of a tile's last step issued before the barrier
// that frees a stage (measured at 4096^3 and 8192^3: 2 rows ahead of 0 and 1).
constexpr int kBarrierRows = 2;

// s_waitcnt vmcnt(n) lgkmcnt(0) (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] |
// lgkmcnt[11:8] | vmcnt[5:4] in bits [15:14]): at most n copies of this wave
// still in flight, and its LDS accesses done.
template <int N>
__device__ __forceinline__ void wait_vmcnt_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14));
}

// Workgroup barrier without the release/acquire fence of __syncthreads (which
// would wait for every outstanding HBM->LDS copy, prefetches included).  The
// memory clobber keeps the compiler from moving LDS accesses across it; the
// needed waits are issued explicitly.
__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Buffer resource for the HBM -> LDS copy below: base, no stride, `range`
// bytes (accesses at or past it read as zero), the gfx950 default format word.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 buffer_rsrc(const void *base, uint32_t range) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r[0] = int(uint32_t(a));
  r[1] = int(uint32_t(a >> 32) & 0xffffu);
  r[2] = int(range);
  r[3] = 0x00020000;
  return r;
}

// Direct HBM -> LDS copy of 16 bytes per lane (buffer_load_dwordx4 ... lds):
// lane i's 16 bytes at byte offset voff + soff land at dst + 16*i.  Issued as
// inline assembly because the compiler, unable to tell which stage a later
// LDS read touches, would otherwise make every LDS read wait for every copy
// in flight (vmcnt(0)), which serializes the multi-stage ring.  The kernel
// orders the copies itself with explicit s_waitcnt vmcnt + s_barrier pairs.
// M0 holds the LDS address; one wait state separates its write from the load
// that reads it.  soff is wave-uniform (an SGPR): the K advance of a tile, so
// the per-lane voff stays fixed over the K loop and costs no vector ALU work.
// Callers keep voff + soff below 2^32 and give out-of-range lanes a voff at
// or past the range on its own, so the result does not depend on whether the
// hardware's range check includes soff.
// NT: the non-temporal cache policy (the convolution's input copies: see the
// B copy plan).
template <bool NT = false>
__device__ __forceinline__ void copy_to_lds16(i32x4 rs, uint32_t voff, uint32_t soff, const lds_void *dst) {
  const uint32_t m0 = uint32_t(reinterpret_cast<uintptr_t>(dst));
  if constexpr (NT)
    asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen nt lds" ::"v"(voff), "s"(rs),
                 "s"(soff), "s"(m0)
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(voff), "s"(rs),
                 "s"(soff), "s"(m0)
                 : "memory", "m0");
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x40);  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

template <typename T>
struct Mfma;

template <>
struct Mfma<_Float16> {
  static __device__ __forceinline__ f32x16 m32(i16x8 a, i16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 m16(i16x8 a, i16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
};

template <>
struct Mfma<__bf16> {
  static __device__ __forceinline__ f32x16 m32(i16x8 a, i16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 m16(i16x8 a, i16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};

template <int MF>
struct AccType;
template <>
struct AccType<32> { using type = f32x16; static constexpr int n = 16; };
template <>
struct AccType<16> { using type = f32x4; static constexpr int n = 4; };

// ---- compile-time tile geometry ----------------------------------------------

template <int BM_, int BN_, int BK_, int ST_, int NW_, int MF_>
struct Geometry {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, ST = ST_, NW = NW_, MF = MF_;
  static constexpr int THREADS = NW * 64;
  static constexpr int WM = NW == 1 ? 1 : NW == 2 ? 1 : NW == 4 ? 2 : NW == 8 ? 2 : 4;
  static constexpr int WN = NW / WM;
  static constexpr int WTM = BM / WM, WTN = BN / WN;   // wave sub-tile
  static constexpr int FK = MF == 32 ? 16 : 32;        // K per MFMA
  static constexpr int TM = WTM / MF, TN = WTN / MF;   // MFMA tiles per wave
  static constexpr int KSUB = BK / FK;                 // MFMA K steps per stage
  static constexpr int CA = BK / 8;                    // 16-byte chunks per A row
  static constexpr int CB = BN / 8;                    // 16-byte chunks per B row
  static constexpr int A_BYTES = BM * BK * 2, B_BYTES = BK * BN * 2;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  static constexpr int A_LOADS = A_BYTES / 1024 / NW;  // 1 KiB wave loads per wave per stage
  static constexpr int B_LOADS = B_BYTES / 1024 / NW;
  static constexpr int LPW = A_LOADS + B_LOADS;
  static_assert(WTM % MF == 0 && WTN % MF == 0, "wave tile must hold whole MFMA tiles");
  static_assert(BK % FK == 0, "BK must hold whole MFMA K steps");
  static_assert(A_BYTES % (1024 * NW) == 0 && B_BYTES % (1024 * NW) == 0, "whole wave loads");
  static_assert(CA >= 2 && CA <= 16 && CB >= 8, "swizzle assumes 2..16 chunks per A row, >= 8 per B row");
  static_assert(ST >= 2 && ST <= 4, "2..4 pipeline stages");
  static_assert((ST - 2) * LPW < 64, "outstanding loads must fit the 6-bit vmcnt");
  // GEMM with a 2-stage ring: a third A buffer, when the LDS holds it without
  // costing a resident block, lets the A refill start a K step earlier (A3).
  static constexpr int LDS_PER_CU = 163840;
  static constexpr int occ(int bytes) { return LDS_PER_CU / bytes < 2048 / THREADS ? LDS_PER_CU / bytes : 2048 / THREADS; }
  static constexpr bool A3 = ST == 2 && KSUB >= 2 && 3 * A_BYTES + 2 * B_BYTES <= LDS_PER_CU &&
                             occ(3 * A_BYTES + 2 * B_BYTES) == occ(2 * STAGE_BYTES);
  static constexpr int lds_bytes(bool conv) { return (!conv && A3) ? 3 * A_BYTES + 2 * B_BYTES : ST * STAGE_BYTES; }

  // A rows (K-contiguous, BK*2 bytes): chunk c of row r lives at chunk
  // c ^ swz_a(r).  16 consecutive rows read at one logical chunk land in 16
  // distinct 16-byte bank groups of the 256-byte bank space.
  static __device__ __forceinline__ int swz_a(int r) { return (r / (16 / CA)) % CA; }
  // B rows (N-contiguous, BN*2 bytes): a transpose read touches 4 consecutive
  // rows (k % 4 == 0) in each 16-lane group, rows 8 apart across groups; the
  // swizzle spreads those rows over distinct 64-byte quarters and 32-byte
  // halves of the bank space.
  static __device__ __forceinline__ int swz_b(int k) {
    int q = CB >= 16 ? 4 * (k % 4) : 4 * ((k / 2) % 2);
    return q ^ (2 * ((k / 8) % 2));
  }

  // Fragment addresses, bytes within an operand slot.
  // K-contiguous rows (A; the conv's transposed B): a lane reads row
  // row0 + lane % MF, logical chunk q*(FK/8) + lane/MF of MFMA K step q; the
  // swizzle depends only on lane % MF, so MFMA tile i adds i*MF rows as an
  // immediate.
  static __device__ __forceinline__ uint32_t frag_k_rows(int row0, int lane, int q, bool swizzle = true) {
    const int r = lane % MF;
    const int lc = q * (FK / 8) + lane / MF;
    return uint32_t((row0 + r) * BK * 2 + ((swizzle ? lc ^ swz_a(r) : lc) * 16));
  }
  // N-contiguous rows (the GEMM's B), read by the transpose read (4 k-rows x
  // 16 columns per 16-lane group): source lane s = lane % 16 points at row
  // kbase + s/4, columns col0 + 4*(s%4) .. +3; K step q adds q*FK rows.
  static __device__ __forceinline__ uint32_t frag_n_rows(int col0, int lane, bool swizzle = true) {
    const int g = lane / 16, s = lane % 16;
    const int krow = MF == 32 ? (g / 2) * 8 + s / 4 : g * 8 + s / 4;
    const int n = col0 + (MF == 32 ? (g % 2) * 16 + 4 * (s % 4) : 4 * (s % 4));
    const int lc = n / 8;
    return uint32_t(krow * BN * 2 + ((swizzle ? lc ^ swz_b(krow) : lc) * 16) + (n % 8) * 2);
  }
};

// Convert and store one wave's accumulators (row-major C, masked edges).
template <typename O>
__device__ __forceinline__ O convert_out(float v) {
  if constexpr (__is_same(O, float)) return v;
  else if constexpr (__is_same(O, _Float16)) return (_Float16)v;
  else return __builtin_bit_cast(__bf16, f32_to_bf16_rne(v));
}

// Accumulator layout (B fragment as the MFMA row operand): register e of
// MFMA tile (i, j) holds C[row][col] with
//   row = wave row base + i*MF + lane % MF
//   col = wave col base + j*MF + c4(e, lane) + e % 4,
//   c4  = (e/4)*8 + (lane/32)*4 for 32x32 tiles, (lane/16)*4 for 16x16 tiles,
// so every group of 4 registers is 4 consecutive columns of one row.
template <int MF>
__device__ __forceinline__ int acc_col4(int e4, int lane) {
  return MF == 32 ? e4 * 8 + (lane / 32) * 4 : (lane / 16) * 4;
}

template <typename O>
struct Vec4 {
  typedef O type __attribute__((ext_vector_type(4)));
};

// Epilogue staged through LDS: each wave converts one MFMA row of its
// sub-tile (MF rows x WTN columns) into a private LDS area, then stores it
// with 16-byte, row-contiguous global writes.  The row pitch is padded by
// 16 bytes so the 4-column writes of 32 consecutive rows hit distinct banks.
template <typename G, typename O>
struct LdsEpilogue {
  static constexpr int PITCH = G::WTN * int(sizeof(O)) + 16;
  static constexpr int WAVE_BYTES = G::MF * PITCH;
  static constexpr bool fits = G::NW * WAVE_BYTES <= G::ST * G::STAGE_BYTES;
};

template <typename G, typename O, typename Acc>
__device__ __forceinline__ void store_tile(const Acc (&acc)[G::TM][G::TN], O *C, char *smem, int m0, int n0,
                                           int wave, int wr, int wc, int lane, int M, int N) {
  constexpr int MF = G::MF;
  constexpr int NACC = AccType<MF>::n;
  using V4 = typename Vec4<O>::type;
  if constexpr (LdsEpilogue<G, O>::fits) {
    using E = LdsEpilogue<G, O>;
    char *area = smem + wave * E::WAVE_BYTES;
    constexpr int ELEMS16 = 16 / int(sizeof(O));        // elements per 16-byte chunk
    constexpr int CPR = G::WTN / ELEMS16;                // chunks per row
    constexpr int CHUNKS = MF * CPR;
    block_barrier();  // every wave is done with the last stage's fragments
#pragma unroll
    for (int i = 0; i < G::TM; ++i) {
#pragma unroll
      for (int j = 0; j < G::TN; ++j)
#pragma unroll
        for (int e4 = 0; e4 < NACC / 4; ++e4) {
          V4 v;
          v[0] = convert_out<O>(acc[i][j][e4 * 4 + 0]);
          v[1] = convert_out<O>(acc[i][j][e4 * 4 + 1]);
          v[2] = convert_out<O>(acc[i][j][e4 * 4 + 2]);
          v[3] = convert_out<O>(acc[i][j][e4 * 4 + 3]);
          const int col = j * MF + acc_col4<MF>(e4, lane);
          *(__attribute__((address_space(3))) V4 *)(area + (lane % MF) * E::PITCH + col * int(sizeof(O))) = v;
        }
#pragma unroll
      for (int c = 0; c < (CHUNKS + 63) / 64; ++c) {
        const int chunk = c * 64 + lane;
        if (CHUNKS % 64 && chunk >= CHUNKS) break;
        const int r = chunk / CPR, cc = chunk % CPR;
        const i16x8 v = *(const lds_i16x8 *)(area + r * E::PITCH + cc * 16);
        const int row = m0 + wr * G::WTM + i * MF + r;
        const int col = n0 + wc * G::WTN + cc * ELEMS16;
        // streaming store: the tile is written once and not read again here
        if (row < M && col < N) __builtin_nontemporal_store(v, (i16x8 *)(C + int64_t(row) * N + col));
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < G::TM; ++i) {
      const int row = m0 + wr * G::WTM + i * MF + lane % MF;
      if (row >= M) continue;
#pragma unroll
      for (int j = 0; j < G::TN; ++j)
#pragma unroll
        for (int e4 = 0; e4 < NACC / 4; ++e4) {
          const int col = n0 + wc * G::WTN + j * MF + acc_col4<MF>(e4, lane);
          if (col >= N) continue;  // N % 4 == 0: the 4 columns are all in or all out
          V4 v;
          v[0] = convert_out<O>(acc[i][j][e4 * 4 + 0]);
          v[1] = convert_out<O>(acc[i][j][e4 * 4 + 1]);
          v[2] = convert_out<O>(acc[i][j][e4 * 4 + 2]);
          v[3] = convert_out<O>(acc[i][j][e4 * 4 + 3]);
          *(V4 *)(C + int64_t(row) * N + col) = v;
        }
    }
  }
}

// Convolution epilogue: row = output channel, column = pixel of the tile
// (image nb0 + n_l, output row o0 + oh_l, output column q0 + ow_l); y is
// NCHW, or NHWC with p.y_nhwc.  The pixels a lane holds do not depend on the
// MFMA row, so each is decoded once: the first of every group of 4
// consecutive columns by division, the next three by stepping (ow_l, oh_l,
// n) forward.  NCHW: a lane's 4 consecutive columns are 4 consecutive y
// elements unless they straddle two images; where they are (and the channel
// plane keeps them aligned) they go out as one vector store.  NHWC: the 16
// (or 32) lanes of an MFMA column hold consecutive channels of one pixel, so
// each store instruction writes runs of consecutive channels.
template <typename G, typename O, typename Acc>
__device__ __forceinline__ void store_conv(const Acc (&acc)[G::TM][G::TN], O *y, const KernelArgs &p, int m0, int n0,
                                           int wr, int wc, int lane, int nb0, int o0, int rows_t, int q0, int cols_t,
                                           int npix) {
  constexpr int MF = G::MF;
  constexpr int NACC = AccType<MF>::n;
  using V4 = typename Vec4<O>::type;
  const int plane = rows_t * cols_t;
  const int64_t chan = int64_t(p.OH) * p.OW;
  const bool nhwc = p.y_nhwc != 0;
  const int64_t pix_mul = nhwc ? p.M : 1, co_mul = nhwc ? 1 : chan;  // y strides of a pixel and a channel
  int64_t off[G::TN][NACC];  // y offset of the pixel at channel 0, or -1 past the last pixel
  bool run[G::TN][NACC / 4];  // the group of 4 is one aligned vector in every channel
#pragma unroll
  for (int j = 0; j < G::TN; ++j)
#pragma unroll
    for (int e4 = 0; e4 < NACC / 4; ++e4) {
      int pix = n0 + wc * G::WTN + j * MF + acc_col4<MF>(e4, lane);
      int n = pix / plane;
      const int rem = pix - n * plane;
      int oh = rem / cols_t;
      int ow = rem - oh * cols_t;
      n += nb0;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        off[j][e4 * 4 + d] =
            pix < npix ? (int64_t(n) * p.M * chan + (int64_t(o0 + oh) * p.OW + q0 + ow) * pix_mul) : int64_t(-1);
        ++pix;
        if (++ow == cols_t) {
          ow = 0;
          if (++oh == rows_t) {
            oh = 0;
            ++n;
          }
        }
      }
      const int64_t o = off[j][e4 * 4];
      run[j][e4] = !nhwc && chan % 4 == 0 && o >= 0 && o % 4 == 0 && off[j][e4 * 4 + 3] == o + 3;
    }
#pragma unroll
  for (int i = 0; i < G::TM; ++i) {
    const int co = m0 + wr * G::WTM + i * MF + lane % MF;
    if (co >= p.M) continue;
#pragma unroll
    for (int j = 0; j < G::TN; ++j)
#pragma unroll
      for (int e4 = 0; e4 < NACC / 4; ++e4) {
        if (run[j][e4]) {
          V4 v;
#pragma unroll
          for (int d = 0; d < 4; ++d) v[d] = convert_out<O>(acc[i][j][e4 * 4 + d]);
          *(V4 *)(y + off[j][e4 * 4] + int64_t(co) * chan) = v;
        } else {
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            const int e = e4 * 4 + d;
            if (off[j][e] >= 0) y[off[j][e] + int64_t(co) * co_mul] = convert_out<O>(acc[i][j][e]);
          }
        }
      }
  }
}

// ---- the kernel ----------------------------------------------------------------

template <typename G, typename T, bool CONV>
__global__ __launch_bounds__(G::THREADS) void tiled_gemm_kernel(KernelArgs p) {
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  using Acc = typename AccType<G::MF>::type;
  constexpr int MF = G::MF;
  constexpr int S = G::ST;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wr = wave / G::WN, wc = wave % G::WN;

  // -- block -> tile.  Workgroups are dealt to the 8 XCDs round-robin; remap
  // so that each XCD gets a contiguous run of tiles, ordered in groups of
  // group_m tile rows so that the run shares A and B panels in its L2.
  const int nblk = gridDim.x, bid = blockIdx.x;
  const int xcd = bid & 7, local = bid >> 3;
  const int per = nblk >> 3, extra = nblk & 7;
  const int t = xcd < extra ? xcd * (per + 1) + local : extra * (per + 1) + (xcd - extra) * per + local;
  const int tiles_mn = p.tiles_m * p.tiles_n;
  const int bzs = t / tiles_mn;  // (batch entry or conv tile) * splits + K range
  const int tt = t - bzs * tiles_mn;
  const int split = bzs % p.splits, bz = bzs / p.splits;
  const int span = p.group_m * p.tiles_n;
  const int first_m = (tt / span) * p.group_m;
  const int gm = min(p.tiles_m - first_m, p.group_m);
  const int in_g = tt - (tt / span) * span;
  const int tm = first_m + in_g % gm, tn = in_g / gm;
  const int m0 = tm * G::BM, n0 = tn * G::BN;
  const int M = p.M;
  // this block's K range [kbeg, kbeg + K) (K == 0 for a range past the end)
  const int kbeg = split * p.k_split;
  const int K = max(0, min(p.k_split, p.K - kbeg));
  const int lda = p.lda;

  // -- convolution: this block's tile (images, output rows, output
  // columns), its input slice and the sub-operator pads.  Rows and columns
  // each follow the H/W tiling formulas; images split with no halo.
  int N = p.N;
  int o0 = 0, rows_t = 0, in_start = 0, pt_sub = 0, rows_in = 0;
  int q0 = 0, cols_t = 0, w_start = 0, pl_sub = 0, cols_in = 0, nb0 = 0;
  if constexpr (CONV) {
    const int wt = bz % p.n_wt, hz = bz / p.n_wt;
    const int ht = hz % p.n_ht, ng = hz / p.n_ht;
    o0 = ht * p.tile_oh;
    const int o1 = min(o0 + p.tile_oh, p.OH);
    rows_t = o1 - o0;
    q0 = wt * p.tile_ow;
    const int q1 = min(q0 + p.tile_ow, p.OW);
    cols_t = q1 - q0;
    nb0 = ng * p.tile_n;
    N = min(p.tile_n, p.Nb - nb0) * rows_t * cols_t;  // pixels of this tile
    if (n0 >= N) return;                                  // ragged last tile: whole block idle
    in_start = max(0, o0 * p.sh - p.ph);                                // (1)
    const int in_end = (o1 - 1) * p.sh - p.ph + (p.kh - 1) * p.dh + 1;  // (2), exclusive
    pt_sub = max(0, p.ph - o0 * p.sh);                                  // (3)
    // slice rows; (4) pads the rest.  A tile whose windows all lie in the
    // padding has an empty slice (the formulas give min(in_end, H) <= in_start)
    rows_in = max(0, min(in_end, p.H) - in_start);
    w_start = max(0, q0 * p.sw - p.pw);
    const int w_end = (q1 - 1) * p.sw - p.pw + (p.kw - 1) * p.dw + 1;
    pl_sub = max(0, p.pw - q0 * p.sw);
    cols_in = max(0, min(w_end, p.W) - w_start);
  }

  // GEMM: rows [m0, M), columns [kbeg, kbeg + K) of each (rows past the last
  // one read as zero).  conv: rows [m0, M) whole; a K tile's columns come
  // from the tap cursor (below)
  const T *Ab = reinterpret_cast<const T *>(p.A) + (CONV ? 0 : int64_t(bz) * p.batch_stride_a) + int64_t(m0) * lda +
                (CONV ? 0 : kbeg);
  const int a_rows = min(G::BM, M - m0);
  const uint32_t a_range =
      (a_rows > 0 && K > 0) ? (CONV ? uint32_t(a_rows) * uint32_t(lda) * 2u
                                    : (uint32_t(a_rows - 1) * uint32_t(lda) + uint32_t(K)) * 2u)
                            : 0u;
  const i32x4 rsA4 = buffer_rsrc(Ab, a_range);
  i32x4 rsB4;
  if constexpr (CONV) {
    // the channel-last input x[Nb][H][W][Cs]
    rsB4 = buffer_rsrc(p.B, uint32_t(p.Nb) * uint32_t(p.H) * uint32_t(p.W) * uint32_t(p.Cs) * 2u);
  } else {
    const T *Bb = reinterpret_cast<const T *>(p.B) + int64_t(bz) * p.batch_stride_b + int64_t(kbeg) * N + n0;
    // elements [n0, K*N); with K == 0 the range is empty (otherwise n0 < N <= K*N)
    rsB4 = buffer_rsrc(Bb, K > 0 ? (uint32_t(K) * uint32_t(N) - uint32_t(n0)) * 2u : 0u);
  }

  // -- A copy plan: wave load j of a stage covers LDS chunks (j*NW+wave)*64 + lane
  uint32_t a_off[G::A_LOADS];
  int a_kc[G::A_LOADS];  // first K element of the lane's chunk within the stage
#pragma unroll
  for (int j = 0; j < G::A_LOADS; ++j) {
    int pchunk = (j * G::NW + wave) * 64 + lane;
    int r = pchunk / G::CA, pc = pchunk % G::CA;
    int lc = pc ^ G::swz_a(r);
    a_off[j] = uint32_t(r) * uint32_t(lda) * 2u + uint32_t(lc) * 16u;
    a_kc[j] = lc * 8;
  }
  // -- B copy plan.
  // GEMM: B is K x N, N-contiguous; chunk (k, lc) of the stage holds columns
  // 8lc .. 8lc+7 of row k.
  // conv: B is the im2col matrix, stored transposed (pixels x K, K-contiguous,
  // laid out and swizzled like A); K runs over (r, s, ci) of the channel-last
  // input, so a 16-byte chunk is 8 consecutive channels of one input pixel.
  // These copies use the non-temporal policy: the input's lines then do not
  // stay in L2 after the GEMM, and an NCHW call's layout pass, which rewrites
  // the channel-last copy the previous call read, runs faster (measured on the
  // 8x256x56x56 workload: 28.7 -> 27.7 us per NCHW call; the channel-last call,
  // 18.1 us, unchanged; the sc1 and sc0 sc1 policies change neither).
  // Per lane: the byte offset of its pixel's window corner (channel 0), the
  // corner's slice row and slice column, and the chunk's first K element.
  uint32_t b_off[G::B_LOADS];
  int b_k[G::B_LOADS];
  int b_row[CONV ? G::B_LOADS : 1], b_col[CONV ? G::B_LOADS : 1];
#pragma unroll
  for (int j = 0; j < G::B_LOADS; ++j) {
    const int pchunk = (j * G::NW + wave) * 64 + lane;
    if constexpr (!CONV) {
      int k = pchunk / G::CB, pc = pchunk % G::CB;
      int lc = pc ^ G::swz_b(k);
      bool col_ok = n0 + lc * 8 < N;
      b_off[j] = col_ok ? uint32_t(k) * uint32_t(N) * 2u + uint32_t(lc) * 16u : kOOB;
      b_k[j] = col_ok ? k : (1 << 30);
    } else {
      const int r = pchunk / G::CA, pc = pchunk % G::CA;
      const int lc = pc ^ G::swz_a(r);
      const int pix = n0 + r;
      const int plane = rows_t * cols_t;
      const int n = pix / plane, rem = pix - n * plane;
      const int oh_l = rem / cols_t, ow_l = rem - oh_l * cols_t;
      const int sr = oh_l * p.sh;                 // padded-slice row of the window's top tap
      const int sc = ow_l * p.sw;                 // padded-slice column of its left tap
      const int ih = in_start - pt_sub + sr;      // its input row (= (o0 + oh_l)*sh - ph)
      const int iw = w_start - pl_sub + sc;       // its input column (= (q0 + ow_l)*sw - pw)
      // may wrap below zero for a pad corner; used only where the chunk is valid
      b_off[j] = uint32_t((((nb0 + n) * p.H + ih) * p.W + iw) * p.Cs + lc * 8) * 2u;
      b_k[j] = lc * 8;
      b_row[j] = pix < N ? sr - pt_sub : (1 << 30);  // slice rows [pt', pt' + rows_in) hold data
      b_col[j] = sc - pl_sub;                        // slice columns [pl', pl' + cols_in) likewise
    }
  }

  const int nk = (K + G::BK - 1) / G::BK;
  const int nfull = K / G::BK;  // K tiles that lie inside K

  // conv: the refill cursor.  K tiles are copied in order 0, 1, 2, ...; Cp is
  // a multiple of BK, so each tile is one tap (r, s) and channels ci0 ..
  // ci0+BK-1 of it, and the cursor steps to the next tile with scalar adds
  // once a tile's copies are issued.  Channels at or past Cin (Cp > Cs = Cin:
  // operands read in place) are not in memory and read as zero.
  int cur_ci = 0, cur_s = 0, cur_r = 0;
  if constexpr (CONV) {
    // a K range starts at a whole K tile: tap kbeg / Cp, channel kbeg % Cp
    const int tap = kbeg / p.Cp;
    cur_ci = kbeg - tap * p.Cp;
    cur_s = tap % p.kw;
    cur_r = tap / p.kw;
  }
  auto cursor_next = [&]() __attribute__((always_inline)) {
    if constexpr (CONV) {
      cur_ci += G::BK;
      if (cur_ci == p.Cp) {
        cur_ci = 0;
        if (++cur_s == p.kw) {
          cur_s = 0;
          ++cur_r;
        }
      }
    }
  };
  // conv, the K tile at the cursor (starting at k0): byte offset of the copy
  // of B chunk j, or kOOB where the chunk lies in a pad, outside the tile's
  // slice, past the last pixel, past the channels or past K
  auto conv_b_off = [&](int k0, int j) __attribute__((always_inline)) -> uint32_t {
    const int dr = cur_r * p.dh, ds = cur_s * p.dw;
    const bool ok = k0 + b_k[j] < K && cur_ci + b_k[j] < p.Cin && uint32_t(b_row[j] + dr) < uint32_t(rows_in) &&
                    uint32_t(b_col[j] + ds) < uint32_t(cols_in);
    return ok ? b_off[j] + uint32_t(((dr * p.W + ds) * p.Cs + cur_ci) * 2) : kOOB;
  };
  // conv, the K tile at the cursor: the A row offset of its first column
  // (tap (cur_r, cur_s), channel cur_ci; rows hold kh*kw*Cs elements), and
  // whether A chunk j holds channels (and lies before K)
  auto conv_a_soff = [&]() __attribute__((always_inline)) -> uint32_t {
    return uint32_t(((cur_r * p.kw + cur_s) * p.Cs + cur_ci) * 2);
  };
  auto conv_a_ok = [&](int k0, int j) __attribute__((always_inline)) -> bool {
    return k0 + a_kc[j] < K && cur_ci + a_kc[j] < p.Cin;
  };
  // LDS slots.  The plain ring: stage s holds A at s*STAGE_BYTES and B right
  // after it.  The A3 ring (GEMM, 2 stages): three A slots, then two B slots.
  constexpr bool A3 = !CONV && G::A3;
  auto a_slot = [&](int s) __attribute__((always_inline)) -> char * {
    return smem + (A3 ? s * G::A_BYTES : s * G::STAGE_BYTES);
  };
  auto b_slot = [&](int s) __attribute__((always_inline)) -> char * {
    return smem + (A3 ? 3 * G::A_BYTES + s * G::B_BYTES : s * G::STAGE_BYTES + G::A_BYTES);
  };
  // Copy j (0 .. LPW-1) of full K tile kt, A copies (j < A_LOADS) into A slot
  // sa, B copies into B slot sb.  A (and the GEMM's B) advance through the
  // scalar offset: the per-lane offsets stay fixed over the K loop.
  auto issue_one = [&](int kt, int sa, int sb, int j) __attribute__((always_inline)) {
    const int k0 = kt * G::BK;
    if (j < G::A_LOADS) {
      lds_void *dst = (lds_void *)(a_slot(sa) + (j * G::NW + wave) * 1024);
      if constexpr (CONV) copy_to_lds16(rsA4, conv_a_ok(k0, j) ? a_off[j] : kOOB, conv_a_soff(), dst);
      else copy_to_lds16(rsA4, a_off[j], uint32_t(k0) * 2u, dst);
    } else {
      const int jb = j - G::A_LOADS;
      lds_void *dst = (lds_void *)(b_slot(sb) + (jb * G::NW + wave) * 1024);
      if constexpr (CONV) copy_to_lds16<true>(rsB4, conv_b_off(k0, jb), 0u, dst);
      else copy_to_lds16(rsB4, b_off[jb], uint32_t(k0) * uint32_t(N) * 2u, dst);
    }
  };
  // Copy j of any K tile ckt: a full tile as above; the ragged last tile
  // masks the chunks at or past K per lane; a tile past the end reads zeros.
  auto copy = [&](int ckt, int sa, int sb, int j) __attribute__((always_inline)) {
    if (ckt < nfull) {
      issue_one(ckt, sa, sb, j);
    } else {
      const int k0 = ckt * G::BK;
      if (j < G::A_LOADS) {
        lds_void *dst = (lds_void *)(a_slot(sa) + (j * G::NW + wave) * 1024);
        if constexpr (CONV) {
          copy_to_lds16(rsA4, conv_a_ok(k0, j) ? a_off[j] : kOOB, conv_a_soff(), dst);
        } else {
          const uint32_t off = (k0 + a_kc[j] < K) ? a_off[j] + uint32_t(k0) * 2u : kOOB;
          copy_to_lds16(rsA4, off, 0u, dst);
        }
      } else {
        const int jb = j - G::A_LOADS;
        lds_void *dst = (lds_void *)(b_slot(sb) + (jb * G::NW + wave) * 1024);
        if constexpr (CONV) {
          copy_to_lds16<true>(rsB4, conv_b_off(k0, jb), 0u, dst);
        } else {
          const uint32_t off = (k0 + b_k[jb] < K) ? b_off[jb] + uint32_t(k0) * uint32_t(N) * 2u : kOOB;
          copy_to_lds16(rsB4, off, 0u, dst);
        }
      }
    }
  };

  // -- per-lane fragment addresses (bytes within an A or B slot)
  // A: one address per MFMA K step (MFMA tile i adds i*MF rows).
  // B, GEMM: one address per MFMA tile (K step q adds q*FK rows).
  // B, conv (pixel rows, K-contiguous): read like A, one address per K step.
  uint32_t fa[G::KSUB];
#pragma unroll
  for (int q = 0; q < G::KSUB; ++q) fa[q] = G::frag_k_rows(wr * G::WTM, lane, q);
  constexpr int NFB = CONV ? G::KSUB : G::TN;
  uint32_t fb[NFB];
  if constexpr (CONV) {
#pragma unroll
    for (int q = 0; q < G::KSUB; ++q) fb[q] = G::frag_k_rows(wc * G::WTN, lane, q);
  } else {
#pragma unroll
    for (int nt = 0; nt < G::TN; ++nt) fb[nt] = G::frag_n_rows(wc * G::WTN + nt * MF, lane);
  }

  Acc acc[G::TM][G::TN];
#pragma unroll
  for (int i = 0; i < G::TM; ++i)
#pragma unroll
    for (int j = 0; j < G::TN; ++j) acc[i][j] = Acc{};

  int kt = 0;
  int ca = 0, cb = 0;  // A and B slots of the tile being computed

  // The copies read buffer descriptors that may have just been written by a
  // vector instruction (v_readfirstlane); five wait states cover that hazard
  // once, before the first copy.
  asm volatile("s_nop 4" ::: "memory");
  {
    // The K loop.  Changes to a plain ring (barrier, burst of copies, fragment
    // reads, MFMAs), all against stalls of the matrix pipe:
    //  * fragment reads cross the barrier: the last MFMA step of tile kt runs
    //    on fragments already in registers while the first step's fragments
    //    of tile kt+1 are read, and the barrier sits inside that last step,
    //    after its first MFMA rows, so the pipe has work while the waves meet;
    //  * the refill copies are spread over MFMA rows (a copy occupies the
    //    CU's load path for about as long as four MFMAs; issued as a burst,
    //    they block the in-order issue of every wave in front of its MFMAs).
    //    The plain ring refills the stage freed at the barrier during the
    //    last step.  The A3 ring (a 2-stage GEMM ring with a third A buffer)
    //    refills A during the first step, into the A slot freed a tile
    //    earlier, and B during the last step, so the copies of a tile are
    //    spread over all of it;
    //  * every tile refills: refills past the last K tile copy zeros into
    //    slots nobody reads again, so the waits are the same for every tile
    //    and one loop body serves the whole K loop.
    // A fragments are single-buffered (slot i is refilled right after the
    // last MFMA that reads it); B fragments are double-buffered, every MFMA
    // row of a step reads all of them.  The steps alternate B buffers and
    // every tile starts on buffer 0.
    i16x8 fa_[G::TM], fb_[2][G::TN];
    auto read_a = [&](const char *sta, int q, int i) __attribute__((always_inline)) {
      fa_[i] = *(const lds_i16x8 *)(sta + fa[q] + i * MF * G::BK * 2);
    };
    auto read_b = [&](const char *stb, int q, int pb, int j) __attribute__((always_inline)) {
      if constexpr (CONV) {
        fb_[pb][j] = *(const lds_i16x8 *)(stb + fb[q] + j * MF * G::BK * 2);
      } else {
        const char *bp = stb + fb[j] + q * G::FK * G::BN * 2;
        i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(bp));
        i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(bp + 4 * G::BN * 2));
        fb_[pb][j] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
    };
    constexpr int BREADS = CONV ? 1 : 2;  // LDS reads per B fragment
    // outstanding copies at the barrier once the next tile has landed: the
    // plain ring's S-2 younger tiles; the A3 ring's A refill of this tile
    constexpr int WAIT_VM = A3 ? G::A_LOADS : (S - 2) * G::LPW;
    // copy selections: which copies of a tile a step issues, and whether the
    // tile is a full K tile (copied without a per-copy test)
    enum { kNone = 0, kAll = 1, kA = 2, kB = 3 };
    // One MFMA step on (fa_, fb_[PB]).  NEXT: the fragments of step nq of the
    // slots at (nsa, nsb) are read into (fa_, fb_[1-PB]) meanwhile, each A
    // fragment right after its last MFMA row, the B fragments spread over the
    // rows.  CP = 2*part + full: the selected copies of K tile ckt into A slot
    // csa / B slot csb are spread over the rows.  BAR >= 0: the step starts
    // with BAR MFMA rows, then the wait and barrier that make the next tile
    // readable and free the slots computed; the reads and copies fill the
    // rows from there on, while the MFMAs already issued keep the matrix
    // pipe busy through the barrier.
    auto step = [&](auto pb_c, auto next_c, auto cp_c, auto bar_c, const char *nsa, const char *nsb, int nq, int ckt,
                    int csa, int csb) __attribute__((always_inline)) {
      constexpr int PB = decltype(pb_c)::value;
      constexpr bool NEXT = decltype(next_c)::value;
      constexpr int PART = decltype(cp_c)::value / 2;
      constexpr bool FULL = decltype(cp_c)::value % 2 == 1;
      constexpr int NC = PART == kAll ? G::LPW : PART == kA ? G::A_LOADS : PART == kB ? G::B_LOADS : 0;
      constexpr int J0 = PART == kB ? G::A_LOADS : 0;
      constexpr int BAR = decltype(bar_c)::value;
      constexpr int R0 = BAR > 0 ? BAR : 0;     // first row that may read or copy
      constexpr int NR = G::TM - R0;            // rows that read and copy
      auto row = [&](auto i_c) __attribute__((always_inline)) {
        constexpr int i = decltype(i_c)::value;
        if constexpr (i == BAR) {
          __builtin_amdgcn_sched_barrier(0);
          wait_vmcnt_lgkm0<WAIT_VM>();  // the next tile has landed (this wave's copies)
          block_barrier();              // ... every wave's; the slots computed are free
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int j = 0; j < G::TN; ++j) {
          if constexpr (MF == 32) acc[i][j] = Mfma<T>::m32(fb_[PB][j], fa_[i], acc[i][j]);
          else acc[i][j] = Mfma<T>::m16(fb_[PB][j], fa_[i], acc[i][j]);
        }
        if constexpr (i >= R0) {
          constexpr int r = i - R0;
          constexpr int a0 = r == 0 ? 0 : i, a1 = i + 1;                     // A fragments refilled here
          constexpr int b0 = r * G::TN / NR, b1 = (r + 1) * G::TN / NR;     // B fragments read here
          if constexpr (NEXT) {
#pragma unroll
            for (int j = b0; j < b1; ++j) read_b(nsb, nq, 1 - PB, j);
#pragma unroll
            for (int a = a0; a < a1; ++a) read_a(nsa, nq, a);
            // the row's MFMAs with its LDS reads in between, one read after each MFMA
            constexpr int NRD = BREADS * (b1 - b0) + (a1 - a0);
            [&]<int... U>(std::integer_sequence<int, U...>) __attribute__((always_inline)) {
              ((__builtin_amdgcn_sched_group_barrier(0x008, 1, 0),
                (U < NRD ? __builtin_amdgcn_sched_group_barrier(0x100, 1, 0) : (void)0)),
               ...);
            }(std::make_integer_sequence<int, G::TN>{});
            if constexpr (NRD > G::TN) __builtin_amdgcn_sched_group_barrier(0x100, NRD - G::TN, 0);
          }
          if constexpr (NC > 0) {
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int c = r * NC / NR; c < (r + 1) * NC / NR; ++c) {
              if constexpr (FULL) issue_one(ckt, csa, csb, J0 + c);
              else copy(ckt, csa, csb, J0 + c);
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        } else {
          __builtin_amdgcn_sched_group_barrier(0x008, G::TN, 0);
        }
      };
      [&]<int... I>(std::integer_sequence<int, I...>) __attribute__((always_inline)) {
        (row(std::integral_constant<int, I>{}), ...);
      }(std::make_integer_sequence<int, G::TM>{});
    };
    using F = std::false_type;
    using Tr = std::true_type;
    using NoBar = std::integral_constant<int, -1>;
    using BarRow = std::integral_constant<int, (kBarrierRows < G::TM ? kBarrierRows : G::TM - 1)>;
    using NoCopy = std::integral_constant<int, 0>;
    // One tile.  MODE 2: its refill is a full K tile; 1: any tile (ragged or
    // past the end); 0: the last tile, no refill and no read-ahead.
    auto tile = [&](auto mode_c) __attribute__((always_inline)) {
      constexpr int MODE = decltype(mode_c)::value;
      constexpr int FULL = MODE == 2 ? 1 : 0;
      const char *sta = a_slot(ca), *stb = b_slot(cb);
      // the A3 ring's A refill (tile kt+2, into the A slot computed a tile ago)
      // rides the first step; the plain ring refills everything in the last
      const int ra = ca == 0 ? 2 : ca - 1;
      using FirstCopy = std::integral_constant<int, (A3 && MODE != 0) ? 2 * kA + FULL : 0>;
      // steps 0 .. KSUB-2, each reading the next step's fragments from this tile's slots
      [&]<int... Q>(std::integer_sequence<int, Q...>) __attribute__((always_inline)) {
        (step(std::integral_constant<int, Q & 1>{}, Tr{},
              std::integral_constant<int, Q == 0 ? FirstCopy::value : 0>{}, NoBar{}, sta, stb, Q + 1, kt + 2, ra,
              0),
         ...);
      }(std::make_integer_sequence<int, G::KSUB - 1>{});
      using PLast = std::integral_constant<int, (G::KSUB - 1) & 1>;
      if constexpr (MODE != 0) {
        const int na = A3 ? (ca == 2 ? 0 : ca + 1) : (ca + 1 == S ? 0 : ca + 1);
        const int nb = A3 ? 1 - cb : na;
        using LastCopy = std::integral_constant<int, 2 * (A3 ? kB : kAll) + FULL>;
        step(PLast{}, Tr{}, LastCopy{}, BarRow{}, a_slot(na), b_slot(nb), 0, A3 ? kt + 2 : kt + S, ca, cb);
        cursor_next();
        if constexpr (PLast::value == 0) {
          // odd number of steps: the next tile's first B fragments were read
          // into buffer 1; move them so that every tile starts on buffer 0
#pragma unroll
          for (int j = 0; j < G::TN; ++j) fb_[0][j] = fb_[1][j];
        }
        ca = na;
        cb = nb;
        ++kt;
      } else {
        step(PLast{}, F{}, NoCopy{}, NoBar{}, sta, stb, 0, 0, 0, 0);
      }
    };

    // prologue: tiles 0 .. S-1 in flight (the A3 ring: tiles 0 and 1), tile
    // 0's first fragments read
#pragma unroll
    for (int s = 0; s < S; ++s) {
#pragma unroll
      for (int j = 0; j < G::LPW; ++j) copy(s, s, s, j);
      cursor_next();
    }
    wait_vmcnt_lgkm0<(S - 1) * G::LPW>();
    block_barrier();
    if (nk > 0) {
#pragma unroll
      for (int i = 0; i < G::TM; ++i) read_a(a_slot(0), 0, i);
#pragma unroll
      for (int j = 0; j < G::TN; ++j) read_b(b_slot(0), 0, 0, j);
    }
    // steady state: the refill is a full K tile; then the tiles whose refill
    // is the ragged tile or past the end; then the last tile
    constexpr int AHEAD = A3 ? 2 : S;  // the refill of tile kt is tile kt + AHEAD
    while (kt + AHEAD < nfull) tile(std::integral_constant<int, 2>{});
    while (kt + 1 < nk) tile(std::integral_constant<int, 1>{});
    if (kt < nk) tile(std::integral_constant<int, 0>{});
    // the refills past the end are still landing in LDS, which the epilogue reuses
    wait_vmcnt_lgkm0<0>();
  }

  // -- epilogue
  if constexpr (!CONV) {
    const int64_t cbase = (int64_t(bz) * p.splits + split) * p.batch_stride_c;
    if (p.out_dtype == TSS_F32)
      store_tile<G, float>(acc, reinterpret_cast<float *>(p.C) + cbase, smem, m0, n0, wave, wr, wc, lane, M, N);
    else if (p.out_dtype == TSS_F16)
      store_tile<G, _Float16>(acc, reinterpret_cast<_Float16 *>(p.C) + cbase, smem, m0, n0, wave, wr, wc, lane, M, N);
    else
      store_tile<G, __bf16>(acc, reinterpret_cast<__bf16 *>(p.C) + cbase, smem, m0, n0, wave, wr, wc, lane, M, N);
  } else {
    if (p.out_dtype == TSS_F32)
      store_conv<G, float>(acc, reinterpret_cast<float *>(p.C) + int64_t(split) * p.batch_stride_c, p, m0, n0, wr, wc,
                           lane, nb0, o0, rows_t, q0, cols_t, N);
    else if (p.out_dtype == TSS_F16)
      store_conv<G, _Float16>(acc, reinterpret_cast<_Float16 *>(p.C), p, m0, n0, wr, wc, lane, nb0, o0, rows_t, q0, cols_t,
                                N);
    else
      store_conv<G, __bf16>(acc, reinterpret_cast<__bf16 *>(p.C), p, m0, n0, wr, wc, lane, nb0, o0, rows_t, q0, cols_t,
                                N);
  }
}

}  // namespace tss
