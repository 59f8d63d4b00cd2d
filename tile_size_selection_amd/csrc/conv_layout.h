// Operand layout for the convolution's implicit GEMM.
//
// The implicit GEMM runs K over (r, s, ci): a 16-byte chunk of a B row is then
// 8 consecutive channels of one input pixel, which a direct HBM -> LDS copy
// moves in one piece, and both MFMA operands are read from LDS K-contiguous.
// One launch rewrites both operands in that order (16-bit elements, so one
// kernel serves fp16 and bf16):
//   xc[n][h][w][c]  = c < C ? x[n][c][h][w]  : 0     (c < Cp)
//   wr[o][r][s][c]  = c < C ? w[o][c][r][s]  : 0     (c < Cp)
// Cp is C rounded up to a multiple of the tile's K step (16, 32 or 64): every
// pixel's channel vector is 16-byte aligned and a K tile is one tap.  Blocks [0, Cout) reorder the weights, one output channel
// each: its C*kh*kw elements are contiguous in w and in wr, so both sides are
// coalesced and the reorder happens in LDS (dispatched first, their load
// latency overlaps the transpose).  Blocks [Cout, Cout + x_blocks) transpose
// 64-channel x 64-pixel tiles of one image through LDS: 16-byte loads along
// the pixels, and 8 consecutive lanes store one pixel's 64 channels as a
// whole 128-byte line.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tss {

struct LayoutArgs {
  const uint16_t *x;  // [N][C][HW]
  uint16_t *xc;       // [N][HW][Cp]
  const uint16_t *w;  // [Cout][C][KHW]
  uint16_t *wr;       // [Cout][KHW][Cp]
  int32_t N, C, HW, Cp, Cout, KHW;
  int32_t c_tiles, p_tiles;
};

constexpr int kLayoutThreads = 256;
// elements of one output channel's weights a block reorders through LDS
constexpr int kLayoutWeightElems = 8192;

typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

__global__ __launch_bounds__(kLayoutThreads) void conv_layout_kernel(LayoutArgs a) {
  constexpr int T = 64;         // channels and pixels per tile
  // LDS row pitch in elements: 33 words, so the 8 channel rows one wave's
  // stores read (8 apart) start in distinct banks
  constexpr int PITCH = T + 2;
  __shared__ __attribute__((aligned(16))) uint16_t lds[T * PITCH > kLayoutWeightElems ? T * PITCH
                                                                                       : kLayoutWeightElems];
  const int tid = threadIdx.x;
  if (int(blockIdx.x) >= a.Cout) {
    const int bid = blockIdx.x - a.Cout;
    uint16_t *tile = lds;
    const int pt = bid % a.p_tiles;
    const int ct = (bid / a.p_tiles) % a.c_tiles;
    const int n = bid / (a.p_tiles * a.c_tiles);
    const int c0 = ct * T, p0 = pt * T;
    const uint16_t *xn = a.x + int64_t(n) * a.C * a.HW;
    // load: rows of 64 pixels of 64 channels (coalesced along the pixels)
    if (a.HW % 8 == 0) {
      // 16-byte chunks: chunk q = (channel q/8, pixels 8*(q%8) .. +7), written
      // to LDS as four 4-byte words (rows are 4-byte aligned)
      for (int q = tid; q < T * T / 8; q += kLayoutThreads) {
        const int cl = q / 8, pl = (q % 8) * 8;
        const int c = c0 + cl, pix = p0 + pl;
        u16x8 v = {};
        if (c < a.C && pix < a.HW) v = *(const u16x8 *)(xn + int64_t(c) * a.HW + pix);
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        const u32x4 d = __builtin_bit_cast(u32x4, v);
        uint32_t *row = reinterpret_cast<uint32_t *>(tile + cl * PITCH + pl);
#pragma unroll
        for (int e = 0; e < 4; ++e) row[e] = d[e];
      }
    } else {
      for (int q = tid; q < T * T; q += kLayoutThreads) {
        const int cl = q / T, pl = q % T;
        const int c = c0 + cl, pix = p0 + pl;
        tile[cl * PITCH + pl] = (c < a.C && pix < a.HW) ? xn[int64_t(c) * a.HW + pix] : uint16_t(0);
      }
    }
    __syncthreads();
    // store: chunk q = (pixel q/8, channels 8*(q%8) .. +7); 8 consecutive
    // lanes write one pixel's 128-byte channel line
    uint16_t *xcn = a.xc + int64_t(n) * a.HW * a.Cp;
    for (int q = tid; q < T * T / 8; q += kLayoutThreads) {
      const int pl = q / 8, cl = (q % 8) * 8;
      const int pix = p0 + pl, c = c0 + cl;
      if (pix >= a.HW || c >= a.Cp) continue;
      u16x8 v;
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = tile[(cl + e) * PITCH + pl];
      *(u16x8 *)(xcn + int64_t(pix) * a.Cp + c) = v;
    }
  } else {
    // one output channel o: w[o] is C x KHW, wr[o] is KHW x Cp
    const int64_t o = blockIdx.x;
    const int row = a.C * a.KHW;
    const uint16_t *wo = a.w + o * row;
    uint16_t *wro = a.wr + o * int64_t(a.KHW) * a.Cp;
    const int chunks = a.KHW * (a.Cp / 8);
    if (a.KHW * 8 > kLayoutWeightElems) {
      // windows of more than 1024 taps: 8 strided loads per output chunk
      for (int q = tid; q < chunks; q += kLayoutThreads) {
        const int rs = q / (a.Cp / 8), cc = (q % (a.Cp / 8)) * 8;
        u16x8 v;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = cc + e < a.C ? wo[int64_t(cc + e) * a.KHW + rs] : uint16_t(0);
        *(u16x8 *)(wro + int64_t(rs) * a.Cp + cc) = v;
      }
      return;
    }
    // channel slices of the row that fit in LDS (one slice for C*KHW <= 8192)
    const int cs = kLayoutWeightElems / a.KHW / 8 * 8 < a.Cp ? kLayoutWeightElems / a.KHW / 8 * 8 : a.Cp;
    for (int cb = 0; cb < a.Cp; cb += cs) {
      const int cn = cs < a.Cp - cb ? cs : a.Cp - cb;  // channels of this slice
      __syncthreads();
      for (int i = tid; i < cn * a.KHW; i += kLayoutThreads) {
        const int c = cb + i / a.KHW;
        lds[i] = c < a.C ? wo[int64_t(cb) * a.KHW + i] : uint16_t(0);
      }
      __syncthreads();
      for (int q = tid; q < chunks; q += kLayoutThreads) {
        const int rs = q / (a.Cp / 8), cc = (q % (a.Cp / 8)) * 8;
        if (cc < cb || cc >= cb + cn) continue;
        u16x8 v;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = lds[(cc - cb + e) * a.KHW + rs];
        *(u16x8 *)(wro + int64_t(rs) * a.Cp + cc) = v;
      }
    }
  }
}

}  // namespace tss
