// Pieces shared by the base GEMMs (bf16 and MXFP8 main steps): the
// k-contiguous LDS swizzle, the XCD-aware tile order and the epilogue.
#pragma once

#include "device_common.hpp"
#include "kernels.hpp"

namespace mlora {

// Chunk c (16 bytes) of row r of a k-contiguous 128-byte-row LDS unit sits at
// position c ^ kx8(r).
__device__ __forceinline__ int kx8(int r) { return (r >> 1) & 7; }

// Output tile of workgroup blockIdx.x.  Workgroup b runs on XCD b mod 8;
// each XCD takes a contiguous run of logical tiles, and logical tiles go
// down groups of four row tiles before moving along N, so the 32 tiles an
// XCD runs together (4 x 8) share operand rows and columns in its L2.  On
// the 70B-shaped projections groups of 4 ran the four base GEMMs of a step
// 3-4.5% faster than groups of 8 (1, 2, 3, 6, 16 and 32 were slower still);
// on a 4096x4096 layer 4 and 8 are within noise.  With split-K the logical
// index also names the K part.
struct TileCoord {
  int sp, TT, tm, tn;
};
template <bool SPLIT>
__device__ __forceinline__ TileCoord tile_coord(const GemmArgs& g) {
  const int G = gridDim.x, bid = blockIdx.x;
  const int xcd = bid & 7, q = bid >> 3, per = G >> 3, rem = G & 7;
  const int L0 = xcd * per + min(xcd, rem) + q;
  const int nM = g.n_mtiles, nN = g.n_ntiles;
  const int TT = nM * nN;
  const int sp = SPLIT ? L0 / TT : 0;
  const int L = L0 - sp * TT;
  constexpr int GM = 4;
  const int grpm = L / (GM * nN);
  const int fm = grpm * GM;
  const int gm = min(GM, nM - fm);
  const int within = L - grpm * GM * nN;
  return TileCoord{sp, TT, fm + within % gm, within / gm};
}

// Epilogue of both GEMM kernels; the ring is free (every wave is past its
// last read and no copy is in flight).  SPLIT: the fp32 partial tile of K
// part sp (rows past the tile are written too, finite values from clamped
// rows, and never read).  Otherwise the tile is staged in LDS as bf16
// [256][256]: 512-byte rows of 32 16-byte granules, granule c of row m at
// c ^ (m & 31), so the 32 rows a fragment writes and the 32 granules a row
// read takes both spread evenly over the banks; each wave then stores 64
// rows, two 512-byte rows per instruction.  acc[fi][fj][4gg+e] holds
// C[m = wrow + 32fi + l32][n = wcol + 32fj + 8gg + 4half + e].
template <bool PERM, bool SPLIT>
__device__ __forceinline__ void gemm_store(const GemmArgs& g, const f32x16 (&acc)[4][4], char* ct,
                                           const TileCoord& tc, int row0, int mrows, int n0, int w,
                                           int lane) {
  constexpr int FI = 4, FJ = 4;
  const int half = lane >> 5, l32 = lane & 31;
  const int wrow = 128 * (w >> 1), wcol = 128 * (w & 1);
  if constexpr (SPLIT) {
    float* pt = g.part + (int64_t)(tc.sp * tc.TT + tc.tm * g.n_ntiles + tc.tn) * 65536;
#pragma unroll
    for (int fi = 0; fi < FI; ++fi) {
      const int m = wrow + 32 * fi + l32;
#pragma unroll
      for (int fj = 0; fj < FJ; ++fj)
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
          const int nn = wcol + 32 * fj + 8 * gg + 4 * half;
          const f32x4 v = {acc[fi][fj][4 * gg], acc[fi][fj][4 * gg + 1], acc[fi][fj][4 * gg + 2],
                           acc[fi][fj][4 * gg + 3]};
          *reinterpret_cast<f32x4*>(pt + m * 256 + nn) = v;
        }
    }
    return;
  }
#pragma unroll
  for (int fi = 0; fi < FI; ++fi) {
    const int m = wrow + 32 * fi + l32;
#pragma unroll
    for (int fj = 0; fj < FJ; ++fj) {
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        const int c = (wcol >> 3) + 4 * fj + gg;
        u32x2 pk;
        pk[0] = pack_bf16x2(acc[fi][fj][4 * gg + 0], acc[fi][fj][4 * gg + 1]);
        pk[1] = pack_bf16x2(acc[fi][fj][4 * gg + 2], acc[fi][fj][4 * gg + 3]);
        *reinterpret_cast<u32x2*>(ct + m * 512 + 16 * (c ^ (m & 31)) + 8 * half) = pk;
      }
    }
  }
  __syncthreads();
  const int gc = lane & 31;
#pragma unroll 4
  for (int it = 0; it < 32; ++it) {
    const int m = 64 * w + 2 * it + half;
    const u32x4 v = *reinterpret_cast<const u32x4*>(ct + m * 512 + 16 * (gc ^ (m & 31)));
    const int n = n0 + 8 * gc;
    if (m < mrows && n < g.N) {
      const int cr = PERM ? ldg_i32(g.t.perm + row0 + m) : row0 + m;
      *reinterpret_cast<u32x4*>(g.C + (int64_t)cr * g.ldc + n) = v;
    }
  }
}

}  // namespace mlora
