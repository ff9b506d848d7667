// bf16 kernels of the packed multi-LoRA layer for gfx950 (CDNA4).
//
// All products run on v_mfma_f32_32x32x16_bf16 with fp32 accumulation.  The
// step structure follows the PLoRA page (PLoRA: Efficient Concurrent LoRA
// Training for Large Language Models, §9.2): adapters are concatenated, work
// is tiled along tokens and hidden dimensions and never along the rank; the
// shrink splits the input dimension, the expand the output dimension; the
// backward has the four cases (dB, gradient into B's input, dA, gradient into
// A's input).  Rank-padded tiles with one code path per padded rank follow the
// tLoRA page's per-rank low-rank tiles (tLoRA: Efficient Multi-LoRA Training
// with Elastic Shared Super-Models, abstract).
#include "device_common.hpp"
#include "kernels.hpp"

#include <type_traits>

namespace mlora {


// ---------------------------------------------------------------------------
// Rank-padded concatenations of the adapters, rebuilt per call (A_i and B_i
// change every training step):
//   A_cat^T [rpad_total][d_in]: row roff(j)+c holds column c of A_j
//   A_cat   [d_in][rpad_total]: column roff(j)+c holds column c of A_j
//   B_cat^T [d_out][rpad_total]: column roff(j)+c holds row c of B_j
// with zeros for r_j <= c < r_pad(j).  Either A output may be NULL.  One
// workgroup per (64-row slab, adapter j): a slab of A_j ([64][r_j]) is one
// contiguous, 128-byte-aligned block, and a slab of B_j ([r_j][64]) is r_j
// 128-byte rows, so both arrive with 16-byte loads into LDS and leave
// transposed or padded from there.
// ---------------------------------------------------------------------------
// Slab k0 .. k0+63 of A for every adapter (blockIdx.y strides over them).
__device__ __forceinline__ void prep_a_slab(u32x4* tile4, int64_t k0, const DevTables& t, int32_t n,
                                            int64_t d_in, int64_t rtot, const void* const* A,
                                            uint16_t* acat_t, uint16_t* acat) {
  const uint16_t* tile = reinterpret_cast<const uint16_t*>(tile4);   // [64][r] bf16, r <= 256
  for (int32_t j = blockIdx.y; j < n; j += gridDim.y) {
    const int r = ldc(t.ranks + j), rp = ldc(t.rpad + j), ro = ldc(t.roff + j);
    const u32x4* src = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(ldc(A + j)) + k0 * r);
    const int nv = 8 * r;                          // 16-byte vectors in the slab
    for (int i = threadIdx.x; i < nv; i += 256) tile4[i] = src[i];
    __syncthreads();
    if (acat_t) {
      // eight consecutive k of one column c per thread: one 16-byte store
      uint16_t* dst = acat_t + (int64_t)ro * d_in + k0;
      for (int i = threadIdx.x; i < rp * 8; i += 256) {
        const int c = i >> 3, kb = (i & 7) * 8;
        uint32_t wv[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t lo = c < r ? tile[(kb + 2 * q) * r + c] : 0u;
          const uint32_t hi = c < r ? tile[(kb + 2 * q + 1) * r + c] : 0u;
          wv[q] = lo | (hi << 16);
        }
        *reinterpret_cast<u32x4*>(dst + (int64_t)c * d_in + kb) = u32x4{wv[0], wv[1], wv[2], wv[3]};
      }
    }
    if (acat) {
      for (int i = threadIdx.x; i < 64 * rp; i += 256) {
        const int k = i / rp, c = i - k * rp;
        acat[(k0 + k) * rtot + ro + c] = c < r ? tile[k * r + c] : (uint16_t)0;
      }
    }
    __syncthreads();
  }
}

// Slab n0 .. n0+63 of the output columns of B for every adapter.
__device__ __forceinline__ void prep_b_slab(u32x4* tile4, int64_t n0, const DevTables& t, int32_t n,
                                            int64_t rtot, const void* const* B, uint16_t* bcat_t) {
  const uint16_t* tile = reinterpret_cast<const uint16_t*>(tile4);   // [r][64] bf16, r <= 256
  for (int32_t j = blockIdx.y; j < n; j += gridDim.y) {
    // pair j's projection owns output columns [c0, c0 + w): other slabs skip it
    const int pq = j % t.nproj;
    const int64_t c0 = ldc(t.pcol + pq), w = ldc(t.pcol + pq + 1) - c0;
    if (n0 < c0 || n0 >= c0 + w) continue;
    const int r = ldc(t.ranks + j), rp = ldc(t.rpad + j), ro = ldc(t.roff + j);
    const uint16_t* Bj = static_cast<const uint16_t*>(ldc(B + j));
    for (int i = threadIdx.x; i < 8 * r; i += 256) {
      const int c = i >> 3, q = i & 7;
      tile4[i] = *reinterpret_cast<const u32x4*>(Bj + (int64_t)c * w + (n0 - c0) + 8 * q);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < 64 * rp; i += 256) {
      const int nn = i / rp, c = i - nn * rp;
      bcat_t[(n0 + nn) * rtot + ro + c] = c < r ? tile[c * 64 + nn] : (uint16_t)0;
    }
    __syncthreads();
  }
}

// One launch for whichever concatenations a call needs: blocks x < d_in/64
// take A slabs, the rest (when bcat_t is set) B slabs.
__global__ __launch_bounds__(256) void k_prep(DevTables t, int32_t n, int64_t d_in, int64_t d_out,
                                              int64_t rtot, const void* const* A, uint16_t* acat_t,
                                              uint16_t* acat, const void* const* B, uint16_t* bcat_t) {
  __shared__ u32x4 tile4[2048];                  // 32 KiB: [64][r] or [r][64] bf16, r <= 256
  const int64_t na = (acat_t || acat) ? d_in / 64 : 0;
  if ((int64_t)blockIdx.x < na)
    prep_a_slab(tile4, (int64_t)blockIdx.x * 64, t, n, d_in, rtot, A, acat_t, acat);
  else
    prep_b_slab(tile4, ((int64_t)blockIdx.x - na) * 64, t, n, rtot, B, bcat_t);
}

void launch_prep(const DevTables& t, int32_t n, int64_t d_in, int64_t d_out, int64_t rtot,
                 const void* const* A, uint16_t* acat_t, uint16_t* acat, const void* const* B,
                 uint16_t* bcat_t, hipStream_t s) {
  const int64_t na = (acat_t || acat) ? d_in / 64 : 0, nb = bcat_t ? d_out / 64 : 0;
  if (na + nb == 0) return;
  dim3 grid((unsigned)(na + nb), (unsigned)(n < 65535 ? n : 65535));
  hipLaunchKernelGGL(k_prep, grid, dim3(256), 0, s, t, n, d_in, d_out, rtot, A, acat_t, acat, B, bcat_t);
}

void launch_prep_a(const DevTables& t, int32_t n, int64_t d_in, int64_t rtot, const void* const* A,
                   uint16_t* acat_t, uint16_t* acat, hipStream_t s) {
  launch_prep(t, n, d_in, 0, rtot, A, acat_t, acat, nullptr, nullptr, s);
}

void launch_prep_b(const DevTables& t, int32_t n, int64_t d_out, int64_t rtot,
                   const void* const* B, uint16_t* bcat_t, hipStream_t s) {
  launch_prep(t, n, 0, d_out, rtot, nullptr, nullptr, nullptr, B, bcat_t, s);
}

// ---------------------------------------------------------------------------
// Skinny products over one nano-batch (rows of one adapter):
//   out[row][c] = s_j * sum_k P[row][k] * Q_j[c][k],  c < RP = r_pad(j)
// MODE 0: shrink (P = X, Q = rows of A_cat^T, all RP rows present);
// MODE 1: dZ (P = dY, Q = B_j, rows >= r_j read as zeros).
//
// One workgroup of four waves per nano-batch, in blocks of up to 128 rows.
// A block of R row fragments of 32 rows (R = 1, 2 or 4 by the block's
// rows) gives fragment f to waves f, f + R, ..; those 4/R waves split the
// 16-deep k-steps of every stage between them and their partial sums are
// added through LDS in wave order at the end.  Both operands are
// k-contiguous rows; each 64-deep stage of the block's 32 R P-rows and the RP
// Q-rows is copied straight into LDS, 128 contiguous bytes per row, chunk c of
// row r at c ^ ((r >> 1) & 7) (the base GEMM's conflict-free layout), and
// fragments are read from there.  The Q rows of a stage are read from L2 once
// per block and shared by all its row fragments, so larger blocks put more of
// the ring's bytes into the streamed operand P.  A ring of NS stages keeps
// NS - 1 stages of copies in flight.  One launch covers every padded-rank
// bucket of a stream group: each workgroup switches on its adapter's r_pad
// and its block's row count.
//
// Projections sharing the input (plans over (adapter, projection) pairs):
// an adapter's projections are cut, in order, into groups whose padded
// ranks sum to at most 256, and the shrink of a group's first pair computes
// every pair of the group at once (FUSED), so X is read once per group:
// A_cat^T holds the pairs of an adapter in consecutive rows, the rows past
// the group's sum read as zero, and column c goes to the pair whose rows it
// falls in, scaled by that pair's s.  The nano-batches of the group's other
// pairs then have nothing to do.
// ---------------------------------------------------------------------------
constexpr int kSkinnyRows = 1280;               // 128-byte LDS rows: 160 KiB

template <int RP, int R>
struct SkinnyCfg {
  static constexpr int ROWS = 32 * R + RP;                  // LDS rows per stage
  static constexpr int NS0 = kSkinnyRows / ROWS;
  static constexpr int NS = NS0 > 16 ? 16 : NS0;            // ring stages
  static constexpr int LPS = ROWS / 32;                     // copies per wave per stage
  static_assert(NS >= 3, "ring too short");
  static_assert((NS - 2) * LPS <= 63, "vmcnt takes 0..63");
  static_assert(4 * 16 * 64 * 4 <= NS * ROWS * 128, "reduction area exceeds ring");
};

__device__ __forceinline__ int skx(int r) { return (r >> 1) & 7; }

// The pair that column block c0 (a multiple of 32) of a fused shrink belongs
// to, among pairs j0 .. j0 + np - 1, and c0's column within that pair.
struct FusedCol {
  int j, c;
};
__device__ __forceinline__ FusedCol fused_col(const DevTables& t, int j0, int np, int c0) {
  int off = 0;
  for (int q = 0; q < np - 1; ++q) {
    const int rp = ldc(t.rpad + j0 + q);
    if (c0 < off + rp) return FusedCol{j0 + q, c0 - off};
    off += rp;
  }
  return FusedCol{j0 + np - 1, c0 - off};
}

template <int RP, int R, int MODE, bool PERM, bool FUSED>
__device__ __forceinline__ void skinny_block(const DevTables& t, int j, int row0, int nrows,
                                             const uint16_t* P, int64_t K, int64_t ldp,
                                             const uint16_t* acat_t, const void* const* Bptr,
                                             const float* scales, uint16_t* out, u32x4* ring, int rlim,
                                             int fnp) {
  using C = SkinnyCfg<RP, R>;
  constexpr int F = RP / 32, NS = C::NS, LPS = C::LPS, SK = 4 / R;
  const int64_t oj = ldc(t.seg0 + j);
  const int rj = ldc(t.ranks + j);
  const uint16_t* Q = MODE == 0 ? acat_t + (int64_t)ldc(t.roff + j) * K
                                : static_cast<const uint16_t*>(ldc(Bptr + j));

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: the copies' LDS base
  const int half = lane >> 5, l32 = lane & 31;
  const int rf = w % R, kg = w / R;          // this wave's row fragment and k-step group
  const int nst = (int)(K >> 6);             // 64-deep stages (K is a multiple of 64)
  const uint32_t ring_lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(MLORA_LDS void*)ring);

  // Copy q of this wave fills stage rows 8 m .. 8 m + 7, m = w + 4 q: lane i
  // -> row 8 m + i / 8 at position i % 8, holding the row's chunk
  // (i % 8) ^ skx(row).  P rows past the block read its last row (never
  // stored); Q rows past the rank read the zero page (no advance).
  const uint16_t* src[LPS];
  bool adv[LPS];
#pragma unroll
  for (int q = 0; q < LPS; ++q) {
    const int row = 8 * (w + 4 * q) + (lane >> 3);
    const int ch = (lane & 7) ^ skx(row);
    if (row < 32 * R) {
      const int pr = row0 + min(row, nrows - 1);
      src[q] = P + (int64_t)(PERM ? ldg_i32(t.perm + pr) : pr) * ldp + 8 * ch;
      adv[q] = true;
    } else {
      const int c = row - 32 * R;
      adv[q] = MODE == 0 ? (!FUSED || c < rlim) : c < rj;
      src[q] = adv[q] ? Q + (int64_t)c * K + 8 * ch : t.zero + 8 * (lane & 7);
    }
  }
  // Stages past the end repeat the last one into slots never read, so every
  // wave issues the same number of copies per stage.
  auto issue = [&](int stage) {
    const int sc = min(stage, nst - 1);
    const uint32_t slot = ring_lds + 16u * (uint32_t)((stage % NS) * C::ROWS * 8);
#pragma unroll
    for (int q = 0; q < LPS; ++q)
      dma16_at(adv[q] ? src[q] + 64 * (int64_t)sc : src[q], slot + 1024u * (uint32_t)(w + 4 * q));
  };

  f32x16 acc[F];
#pragma unroll
  for (int f = 0; f < F; ++f)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[f][e] = 0.f;

#pragma unroll
  for (int i = 0; i < NS - 1; ++i) issue(i);
  for (int st = 0; st < nst; ++st) {
    wait_vm_barrier<(NS - 2) * LPS>();
    issue(st + NS - 1);
    const u32x4* slot = ring + (st % NS) * C::ROWS * 8;
#pragma unroll
    for (int kk = 0; kk < 4 / SK; ++kk) {
      const int ks = kg + SK * kk;           // 16-deep k-step of the stage
      const int c = 2 * ks + half;
      const int prow = 32 * rf + l32;
      const u32x4 pa = slot[prow * 8 + (c ^ skx(prow))];
#pragma unroll
      for (int f = 0; f < F; ++f) {
        const int qrow = 32 * R + 32 * f + l32;
        const u32x4 qa = slot[qrow * 8 + (c ^ skx(qrow))];
        acc[f] = mfma32(qa, pa, acc[f]);
      }
    }
  }
  // drain the trailing copies before the ring is reused for the reduction
  wait_vm_barrier<0>();

  // acc[f][4g+e] = D[c = 32f + 8g + 4 half + e][row = 32 rf + l32]
  // Where column block f (32 columns) of the result goes: pair, its Z'
  // slab, row stride (the pair's r_pad), first column and scale.
  struct Dst {
    uint16_t* base;
    int ld, c;
    float s;
  };
  auto dst = [&](int f) -> Dst {
    if constexpr (FUSED) {
      const FusedCol fc = fused_col(t, j, fnp, 32 * f);
      return Dst{out + ldc(t.zoff + fc.j), ldc(t.rpad + fc.j), fc.c, ldc(scales + fc.j)};
    }
    return Dst{out + ldc(t.zoff + j), RP, 32 * f, ldc(scales + j)};
  };
  if constexpr (R == 4) {
#pragma unroll
    for (int f = 0; f < F; ++f) {
      const int row = 32 * rf + l32;
      if (FUSED && 32 * f >= rlim) continue;
      const Dst d = dst(f);
      if (row < nrows) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int c = d.c + 8 * g + 4 * half;
          u32x2 pk;
          pk[0] = pack_bf16x2(d.s * acc[f][4 * g + 0], d.s * acc[f][4 * g + 1]);
          pk[1] = pack_bf16x2(d.s * acc[f][4 * g + 2], d.s * acc[f][4 * g + 3]);
          *reinterpret_cast<u32x2*>(d.base + (int64_t)(row0 + row - oj) * d.ld + c) = pk;
        }
      }
    }
  } else {
    // The 4/R waves of each fragment are added in wave order: thread tid
    // takes fragment fr = tid / (256 / R), lane l of it, and the R groups
    // g = gq R .. gq R + R - 1 of four elements each.
    float* red = reinterpret_cast<float*>(ring);
    const int fr = tid / (256 / R), l = tid & 63, gq = (tid % (256 / R)) >> 6;
#pragma unroll
    for (int f = 0; f < F; ++f) {
      if (FUSED && 32 * f >= rlim) continue;
      const Dst d = dst(f);
#pragma unroll
      for (int e = 0; e < 16; ++e) red[(w * 16 + e) * 64 + lane] = acc[f][e];
      __syncthreads();
      const int row = 32 * fr + (l & 31);
#pragma unroll
      for (int gg = 0; gg < R; ++gg) {
        const int g = gq * R + gg;
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float sum = 0.f;
#pragma unroll
          for (int k2 = 0; k2 < SK; ++k2) sum += red[((fr + R * k2) * 16 + 4 * g + i) * 64 + l];
          v[i] = sum;
        }
        if (row < nrows) {
          const int c = d.c + 8 * g + 4 * (l >> 5);
          u32x2 pk;
          pk[0] = pack_bf16x2(d.s * v[0], d.s * v[1]);
          pk[1] = pack_bf16x2(d.s * v[2], d.s * v[3]);
          *reinterpret_cast<u32x2*>(d.base + (int64_t)(row0 + row - oj) * d.ld + c) = pk;
        }
      }
      __syncthreads();
    }
  }
}

template <int RP, int MODE, bool PERM, bool FUSED>
__device__ __forceinline__ void skinny_item(const DevTables& t, int j, int row0, int nrows, const uint16_t* P,
                                            int64_t K, int64_t ldp, const uint16_t* acat_t,
                                            const void* const* Bptr, const float* scales, uint16_t* out,
                                            u32x4* ring, int rlim, int fnp) {
  // blocks of up to 128 rows; each block's copies are drained before the next
  for (int b0 = 0; b0 < nrows; b0 += 128) {
    const int nb = min(128, nrows - b0);
    if (nb <= 32)
      skinny_block<RP, 1, MODE, PERM, FUSED>(t, j, row0 + b0, nb, P, K, ldp, acat_t, Bptr, scales, out, ring, rlim, fnp);
    else if (nb <= 64)
      skinny_block<RP, 2, MODE, PERM, FUSED>(t, j, row0 + b0, nb, P, K, ldp, acat_t, Bptr, scales, out, ring, rlim, fnp);
    else
      skinny_block<RP, 4, MODE, PERM, FUSED>(t, j, row0 + b0, nb, P, K, ldp, acat_t, Bptr, scales, out, ring, rlim, fnp);
    __syncthreads();
  }
}

template <int MODE, bool PERM>
__global__ __launch_bounds__(256) void k_skinny(DevTables t, int32_t nano_begin, const uint16_t* P,
                                                int64_t K, const uint16_t* acat_t,
                                                const void* const* Bptr, const float* scales,
                                                uint16_t* out) {
  __shared__ u32x4 ring[kSkinnyRows * 8];
  const int nb = nano_begin + blockIdx.x;
  const int j = ldc(t.nano + 3 * nb), row0 = ldc(t.nano + 3 * nb + 1), nrows = ldc(t.nano + 3 * nb + 2);
  if (MODE == 0 && t.nproj > 1) {
    // Shrink over a group of an adapter's projections (consecutive, padded
    // ranks summing to at most 256, cut greedily from the first): the
    // group's first pair computes all of them (X read once per group).
    const int np = t.nproj, j0 = j - j % np, qj = j % np;
    int gs = 0, rs = 0;
    for (int q = 0; q <= qj; ++q) {
      const int rp = ldc(t.rpad + j0 + q);
      if (rs + rp > 256) {
        gs = q;
        rs = 0;
      }
      rs += rp;
    }
    int ge = qj + 1;
    while (ge < np && rs + ldc(t.rpad + j0 + ge) <= 256) rs += ldc(t.rpad + j0 + ge++);
    if (ge - gs > 1) {
      if (qj != gs) return;
      const int jg = j0 + gs, gn = ge - gs;
      if (rs <= 64) skinny_item<64, 0, PERM, true>(t, jg, row0, nrows, P, K, K, acat_t, Bptr, scales, out, ring, rs, gn);
      else if (rs <= 128) skinny_item<128, 0, PERM, true>(t, jg, row0, nrows, P, K, K, acat_t, Bptr, scales, out, ring, rs, gn);
      else skinny_item<256, 0, PERM, true>(t, jg, row0, nrows, P, K, K, acat_t, Bptr, scales, out, ring, rs, gn);
      return;
    }
  }
  // dZ of pair j reads its projection's columns of dY: K = the projection's
  // width, rows K0 = the full row length apart
  int64_t Kj = K;
  const uint16_t* Pj = P;
  if (MODE == 1) {
    const int pq = j % t.nproj;
    const int64_t c0 = ldc(t.pcol + pq);
    Kj = ldc(t.pcol + pq + 1) - c0;
    Pj = P + c0;
  }
  switch (ldc(t.rpad + j)) {
    case 32: skinny_item<32, MODE, PERM, false>(t, j, row0, nrows, Pj, Kj, K, acat_t, Bptr, scales, out, ring, 32, 1); break;
    case 64: skinny_item<64, MODE, PERM, false>(t, j, row0, nrows, Pj, Kj, K, acat_t, Bptr, scales, out, ring, 64, 1); break;
    case 128: skinny_item<128, MODE, PERM, false>(t, j, row0, nrows, Pj, Kj, K, acat_t, Bptr, scales, out, ring, 128, 1); break;
    default: skinny_item<256, MODE, PERM, false>(t, j, row0, nrows, Pj, Kj, K, acat_t, Bptr, scales, out, ring, 256, 1); break;
  }
}

void launch_skinny(int mode, const DevTables& t, int32_t nano_begin, int32_t nano_count,
                   const uint16_t* P, int64_t K, const uint16_t* acat_t, const void* const* Bptr,
                   const float* scales, uint16_t* out, hipStream_t s) {
  if (nano_count <= 0) return;
  dim3 grid((unsigned)nano_count), block(256);
#define MLORA_SKINNY(M, PM) \
  hipLaunchKernelGGL((k_skinny<M, PM>), grid, block, 0, s, t, nano_begin, P, K, acat_t, Bptr, scales, out)
  if (mode == 0) {
    if (t.perm) MLORA_SKINNY(0, true); else MLORA_SKINNY(0, false);
  } else {
    if (t.perm) MLORA_SKINNY(1, true); else MLORA_SKINNY(1, false);
  }
#undef MLORA_SKINNY
}

// ---------------------------------------------------------------------------
// Token reductions over one chunk (<= KC rows of one adapter) and one block of
// 128 columns of the wide operand:
//   dB item: part[c][n] = sum_t R[t][c] Wd[t][n]  (R = Z', Wd = dY)
//   dA item: part[d][c] = sum_t Wd[t][d] R[t][c]  (R = dZ, Wd = X)
// One launch per padded-rank bucket holds the dB items of the bucket's chunks
// followed by their dA items.  This register-staged form serves plans whose
// rows come in the caller's order: each thread gathers its rows through the
// permutation table (k_token_reduce_dma below serves grouped rows).  Both
// operands are token-major, so each 8x8
// block is transposed in registers on its way into k-contiguous, swizzled LDS
// tiles (double buffered, one barrier per 64-token step).  The global loads
// run two steps ahead in two register stages up to r_pad 64 (one above, to
// keep the registers of two waves per SIMD); every load is issued, at a clamped
// address, and rows past the chunk or columns past the operand are zeroed
// after it, so the compiler's wait counts stay exact.
// ---------------------------------------------------------------------------
struct TokenReduceArgs {
  DevTables t;
  int32_t chunk_begin, n_chunks;
  const uint16_t* dY;       // first column of the chunks' projection
  int64_t ld_dy;            // row stride of dY (all projections' columns)
  const uint16_t* Z;
  float* partB;
  int64_t d_out;            // the projection's width
  const uint16_t* X;
  const uint16_t* dZ;
  float* partA;
  int64_t d_in;
  // Grouped rows: an adapter with a single chunk writes its dA_j / dB_j
  // (fp32, rank r_j unpadded) directly, and the partial sums skip it.
  void* const* dA;
  void* const* dB;
  int32_t direct;
};

template <int RP, int MODE, bool PERM>
__device__ __forceinline__ void token_reduce_body(const TokenReduceArgs& a, int ch, int col0,
                                                  u32x4 (*sbig)[128 * 8], u32x4 (*srk)[RP * 8]) {
  constexpr int F = RP / 32;
  constexpr int NBLK = 128 + RP;                 // 8x8 blocks per 64-token step
  constexpr int PER = (NBLK + 255) / 256;        // blocks per thread
  const uint16_t* big = MODE == 0 ? a.dY : a.X;
  const int64_t big_ld = MODE == 0 ? a.ld_dy : a.d_in;   // row stride
  const int64_t big_n = MODE == 0 ? a.d_out : a.d_in;    // columns, partial row length
  const uint16_t* rk = MODE == 0 ? a.Z : a.dZ;
  float* part = MODE == 0 ? a.partB : a.partA;
  const int j = ldc(a.t.chunks + 3 * ch), r0 = ldc(a.t.chunks + 3 * ch + 1), nr = ldc(a.t.chunks + 3 * ch + 2);
  const int64_t cp = ldc(a.t.cpref + ch);
  const uint16_t* rbase = rk + ldc(a.t.zoff + j) + (int64_t)(r0 - ldc(a.t.seg0 + j)) * RP;
  const uint16_t* bbase = big + (int64_t)r0 * big_ld;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;

  // Block b of a step: b < 128 -> 8 tokens x 8 columns of the wide operand
  // (column block mb = b % 16, token block kb = b / 16), else of the rank
  // operand (mb = (b-128) % (RP/8), kb = (b-128) / (RP/8)).
  // Threads past the last block (256*PER > NBLK) duplicate block b - NBLK:
  // same loads, same values to the same LDS slots, and no branch around the
  // loads (which would make the compiler drain every load in flight).
  // PERM: the wide operand's row is the caller's row of grouped row r0 + tc.
  // Those row indexes are loaded two steps ahead (two register sets, by step
  // parity), so a step's data loads never wait on its index loads.
  int ix[PERM ? 2 : 1][PER][8];
  auto fetch_idx = [&](int step) {
    if constexpr (PERM) {
#pragma unroll
      for (int p = 0; p < PER; ++p) {
        const int b = tid + 256 * p < NBLK ? tid + 256 * p : tid + 256 * p - NBLK;
        const int kb = b < 128 ? b / 16 : 0;
#pragma unroll
        for (int i = 0; i < 8; ++i)
          ix[step & 1][p][i] = ldg_i32(a.t.perm + r0 + min(step * 64 + 8 * kb + i, nr - 1)) - r0;
      }
    }
  };
  auto load = [&](int step, u32x4 (&stage)[PER][8]) {
    const int t0 = step * 64;
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int b = tid + 256 * p < NBLK ? tid + 256 * p : tid + 256 * p - NBLK;
      {
        const bool isbig = b < 128;
        const int bb = isbig ? b : b - 128;
        const int MB = isbig ? 16 : RP / 8;
        const int mb = bb % MB, kb = bb / MB;
        const int64_t col = isbig ? min((int64_t)(col0 + 8 * mb), big_n - 8) : 8 * mb;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int tc = min(t0 + 8 * kb + i, nr - 1);
          const int64_t br = PERM ? (int64_t)ix[step & 1][p][i] : tc;
          stage[p][i] = isbig ? ld16(bbase + br * big_ld + col) : ld16(rbase + (int64_t)tc * RP + col);
        }
      }
    }
    fetch_idx(step + 2);
  };
  fetch_idx(0);
  fetch_idx(1);
  // Rows past the chunk and columns past the operand are zeroed here, when
  // the stage is consumed, not when it is loaded.
  auto store = [&](int buf, int step, u32x4 (&stage)[PER][8]) {
    const int t0 = step * 64;
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int b = tid + 256 * p < NBLK ? tid + 256 * p : tid + 256 * p - NBLK;
      {
        const bool isbig = b < 128;
        const int bb = isbig ? b : b - 128;
        const int MB = isbig ? 16 : RP / 8;
        const int mb = bb % MB, kb = bb / MB;
        const bool colok = !isbig || (col0 + 8 * mb < big_n);
#pragma unroll
        for (int i = 0; i < 8; ++i)
          stage[p][i] = (t0 + 8 * kb + i < nr && colok) ? stage[p][i] : zero4();
        u32x4 tr[8];
        transpose8x8(stage[p], tr);
        u32x4* dst = isbig ? sbig[buf] : srk[buf];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) dst[swz(8 * mb + jj, kb)] = tr[jj];
      }
    }
  };

  f32x16 acc[F];
#pragma unroll
  for (int f = 0; f < F; ++f)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[f][e] = 0.f;
  auto compute = [&](int buf) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const u32x4 bf = sbig[buf][swz(32 * w + l32, 2 * ks + half)];
#pragma unroll
      for (int f = 0; f < F; ++f) {
        const u32x4 rf = srk[buf][swz(32 * f + l32, 2 * ks + half)];
        if (MODE == 0)
          acc[f] = mfma32(bf, rf, acc[f]);  // D[n][c]
        else
          acc[f] = mfma32(rf, bf, acc[f]);  // D[c][d]
      }
    }
  };

  const int steps = (nr + 63) / 64;
  if constexpr (RP <= 64) {
    // Two register stages S0/S1.  Invariant at the loop top: LDS buffer 0
    // holds step st, S1 holds (or is receiving) step st+1.
    u32x4 S0[PER][8], S1[PER][8];
    load(0, S0);
    if (steps > 1) load(1, S1);
    store(0, 0, S0);
    __syncthreads();
    int st = 0;
    for (; st + 3 < steps; st += 2) {
      load(st + 2, S0);
      compute(0);
      store(1, st + 1, S1);
      __syncthreads();
      load(st + 3, S1);
      compute(1);
      store(0, st + 2, S0);
      __syncthreads();
    }
    // at most three steps remain: st, st+1, st+2
    if (st + 2 < steps) load(st + 2, S0);
    compute(0);
    if (st + 1 < steps) store(1, st + 1, S1);
    __syncthreads();
    if (st + 1 < steps) compute(1);
    if (st + 2 < steps) store(0, st + 2, S0);
    __syncthreads();
    if (st + 2 < steps) compute(0);
  } else {
    u32x4 S0[PER][8];
    load(0, S0);
    store(0, 0, S0);
    __syncthreads();
    for (int st = 0; st < steps; ++st) {
      const int buf = st & 1;
      if (st + 1 < steps) load(st + 1, S0);
      compute(buf);
      if (st + 1 < steps) store(buf ^ 1, st + 1, S0);
      __syncthreads();
    }
  }

#pragma unroll
  for (int f = 0; f < F; ++f) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      f32x4 v;
      v[0] = acc[f][4 * g + 0];
      v[1] = acc[f][4 * g + 1];
      v[2] = acc[f][4 * g + 2];
      v[3] = acc[f][4 * g + 3];
      if (MODE == 0) {
        // lane holds c = 32f + l32, n = col0 + 32w + 8g + 4half + e
        const int c = 32 * f + l32;
        const int n = col0 + 32 * w + 8 * g + 4 * half;
        if (n < big_n)
          *reinterpret_cast<f32x4*>(part + ldc(a.t.cboff + ch) + (int64_t)c * big_n + n) = v;
      } else {
        // lane holds d = col0 + 32w + l32, c = 32f + 8g + 4half + e
        const int d = col0 + 32 * w + l32;
        const int c = 32 * f + 8 * g + 4 * half;
        if (d < big_n)
          *reinterpret_cast<f32x4*>(part + cp * big_n + (int64_t)d * RP + c) = v;
      }
    }
  }
}

template <int RP, bool PERM>
__global__ __launch_bounds__(256) void k_token_reduce(TokenReduceArgs a) {
  __shared__ u32x4 sbig[2][128 * 8];
  __shared__ u32x4 srk[2][RP * 8];
  const int nbb_b = (int)((a.d_out + 127) / 128);
  const int nbb_a = (int)((a.d_in + 127) / 128);
  const int b = blockIdx.x, nb_b = a.n_chunks * nbb_b;
  if (b < nb_b)
    token_reduce_body<RP, 0, PERM>(a, a.chunk_begin + b / nbb_b, (b % nbb_b) * 128, sbig, srk);
  else
    token_reduce_body<RP, 1, PERM>(a, a.chunk_begin + (b - nb_b) / nbb_a, ((b - nb_b) % nbb_a) * 128, sbig, srk);
}

// ---------------------------------------------------------------------------
// The same token reductions with both operands copied straight into LDS
// (plans whose rows are already grouped by adapter).  One (chunk, WN-column
// block) per workgroup.  Each KS-token stage holds the wide operand's
// KS x WN block and the rank operand's KS x r_pad block, both with the
// token axis along LDS rows as they lie in memory; the MFMA fragments, which take eight consecutive tokens per lane,
// are read with the transposing ds_read_b64_tr_b16, so no register staging
// and no transposes.  NS stages form a ring: while one is reduced, the next
// NS - 1 are in flight.  Copies of rows past the chunk (and of columns past
// the operand) read the zero page, so every stage issues the same number of
// copies and one vmcnt bound fits every wait.
//
// LDS rows: a k-row (token) of CH 16-byte chunks; chunk c of k-row kr sits
// at c ^ trsw<CH>(kr).  A transposing read group (32 lanes) covers four
// consecutive k-rows (a multiple of 4 first) and four consecutive chunks (a
// multiple of 4 first), i.e. 16 chunks that must fall in distinct 16-byte
// bank groups (chunk index mod 16 of the tile): 16 or more chunks per row:
// XOR bits 2-3 with the k-row's low bits; 8 per row (two rows per bank
// line): XOR bit 2 with bit 1 of the k-row; 4 per row: already distinct.
// ---------------------------------------------------------------------------
template <int CH>
__device__ __forceinline__ int trsw(int kr) {
  return CH >= 16 ? ((kr & 3) << 2) : (CH == 8 ? (((kr >> 1) & 1) << 2) : 0);
}

// Operand fragment of a 32x32x16 MFMA from a token-major tile: lane l gets
// tokens kb + 8 (l/32) + 0..7 of column cb + l%32.  ds_read_b64_tr_b16 hands
// lane i of a 16-lane group element (i % 4) of the 8 bytes addressed by group
// lane 4e + i/4, so group lane s addresses k-row kb' + s/4, columns
// cb' + 4 (s%4); two reads cover the eight tokens.
template <int CH>
__device__ __forceinline__ u32x4 read_tok(const MLORA_LDS char* tile, int cb, int kb, int lane) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  const int g = lane >> 4, s = lane & 15;
  const int n = cb + 16 * (g & 1) + 4 * (s & 3);
  const int k = kb + 8 * (g >> 1) + (s >> 2);
  u32x4 out;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int kr = k + 4 * h;
    const int byte = (kr * CH + ((n >> 3) ^ trsw<CH>(kr))) * 16 + 2 * (n & 7);
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLORA_LDS s16x4*)(tile + byte));
    const u32x2 u = __builtin_bit_cast(u32x2, v);
    out[2 * h] = u[0];
    out[2 * h + 1] = u[1];
  }
  return out;
}

// Shape per padded rank: WN wide columns per workgroup, KS tokens per
// stage, WA x WB waves along the wide block and the rank, NS ring stages,
// WGS workgroups per CU (160 KiB of LDS).  Measured on the 70B-shaped MLP
// pair (isolated launches, one projection): 256-wide blocks in 32-token
// stages took the r_pad 256 bucket from 693 to 500-530 us and r_pad 64/128
// down 5%; at r_pad 32 they gain 2.5% there but lose 15% on a 4096x4096
// layer, whose few chunks then fill fewer CUs.
template <int RP>
struct TrShape;
template <> struct TrShape<32> { static constexpr int WN = 128, KS = 64, WA = 4, NS = 4, WGS = 2; };
template <> struct TrShape<64> { static constexpr int WN = 256, KS = 32, WA = 2, NS = 4, WGS = 1; };
template <> struct TrShape<128> { static constexpr int WN = 256, KS = 32, WA = 2, NS = 6, WGS = 1; };
template <> struct TrShape<256> { static constexpr int WN = 256, KS = 32, WA = 2, NS = 4, WGS = 1; };

template <int RP>
struct TrCfg : TrShape<RP> {
  using S = TrShape<RP>;
  static constexpr int CHW = S::WN / 8;           // 16-byte chunks per wide k-row
  static constexpr int CHR = RP / 8;              //   and per rank k-row
  static constexpr int WB = 4 / S::WA;
  static constexpr int FW = S::WN / S::WA / 32;   // wide fragments per wave
  static constexpr int FR = RP / WB / 32;         // rank fragments per wave
  static constexpr int WIDE = S::KS * S::WN * 2;  // bytes of a stage's wide block
  static constexpr int RANK = S::KS * RP * 2;     //   and rank block
  static constexpr int STAGE = WIDE + RANK;
  static constexpr int CWW = WIDE / 4096;         // 1 KiB copies per wave per stage: wide
  static constexpr int CWR = RANK / 4096;         //   and rank
  static constexpr int CW = CWW + CWR;
  static_assert(WIDE % 4096 == 0 && RANK % 4096 == 0 && FW >= 1 && FR >= 1, "shape");
  static_assert(S::NS * STAGE * S::WGS <= 160 * 1024, "LDS");
  static_assert((S::NS - 2) * CW <= 63, "vmcnt");
};

template <int RP, int MODE>
__device__ __forceinline__ void token_reduce_dma_body(const TokenReduceArgs& a, int ch, int col0,
                                                      const MLORA_LDS char* lds, uint32_t ring_lds) {
  using C = TrCfg<RP>;
  constexpr int KS = C::KS, NS = C::NS;
  const uint16_t* big = MODE == 0 ? a.dY : a.X;
  const int64_t big_ld = MODE == 0 ? a.ld_dy : a.d_in;   // row stride
  const int64_t big_n = MODE == 0 ? a.d_out : a.d_in;    // columns, partial row length
  const uint16_t* rk = MODE == 0 ? a.Z : a.dZ;
  float* part = MODE == 0 ? a.partB : a.partA;
  const int j = ldc(a.t.chunks + 3 * ch), r0 = ldc(a.t.chunks + 3 * ch + 1), nr = ldc(a.t.chunks + 3 * ch + 2);
  const int64_t cp = ldc(a.t.cpref + ch);
  const uint16_t* rbase = rk + ldc(a.t.zoff + j) + (int64_t)(r0 - ldc(a.t.seg0 + j)) * RP;
  const uint16_t* wbase = big + (int64_t)r0 * big_ld;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, l32 = lane & 31;

  // Copy i of wave w fills LDS chunks 64 (CW* w + i) + lane of its block:
  // chunk q is k-row q / CH at position q % CH, which holds the row's chunk
  // (q % CH) ^ trsw<CH>(k-row).
  int wkr[C::CWW], wcol[C::CWW], rkr[C::CWR], roff[C::CWR];
#pragma unroll
  for (int i = 0; i < C::CWW; ++i) {
    const int q = 64 * (C::CWW * w + i) + lane;
    wkr[i] = q / C::CHW;
    wcol[i] = col0 + 8 * ((q % C::CHW) ^ trsw<C::CHW>(wkr[i]));
  }
#pragma unroll
  for (int i = 0; i < C::CWR; ++i) {
    const int q = 64 * (C::CWR * w + i) + lane;
    rkr[i] = q / C::CHR;
    roff[i] = rkr[i] * RP + 8 * ((q % C::CHR) ^ trsw<C::CHR>(rkr[i]));
  }
  auto issue = [&](int st, int slot) {
    const int t0 = KS * st;
    const uint32_t base = ring_lds + (uint32_t)(slot * C::STAGE);
#pragma unroll
    for (int i = 0; i < C::CWW; ++i) {
      const int t = t0 + wkr[i];
      const void* src = (wcol[i] < big_n && t < nr) ? (const void*)(wbase + (int64_t)t * big_ld + wcol[i])
                                                    : (const void*)a.t.zero;
      dma16_at(src, base + 1024u * (uint32_t)(C::CWW * w + i));
    }
#pragma unroll
    for (int i = 0; i < C::CWR; ++i) {
      const void* src = t0 + rkr[i] < nr ? (const void*)(rbase + (int64_t)t0 * RP + roff[i]) : (const void*)a.t.zero;
      dma16_at(src, base + (uint32_t)C::WIDE + 1024u * (uint32_t)(C::CWR * w + i));
    }
  };

  const int wa = w % C::WA, wb = w / C::WA;
  f32x16 acc[C::FW][C::FR];
#pragma unroll
  for (int x = 0; x < C::FW; ++x)
#pragma unroll
    for (int y = 0; y < C::FR; ++y)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[x][y][e] = 0.f;
  auto compute = [&](int slot) {
    const MLORA_LDS char* wt = lds + slot * C::STAGE;
    const MLORA_LDS char* rt = wt + C::WIDE;
#pragma unroll
    for (int ks = 0; ks < KS / 16; ++ks) {
      u32x4 fw[C::FW], fr[C::FR];
#pragma unroll
      for (int x = 0; x < C::FW; ++x) fw[x] = read_tok<C::CHW>(wt, 32 * (C::FW * wa + x), 16 * ks, lane);
#pragma unroll
      for (int y = 0; y < C::FR; ++y) fr[y] = read_tok<C::CHR>(rt, 32 * (C::FR * wb + y), 16 * ks, lane);
#pragma unroll
      for (int x = 0; x < C::FW; ++x)
#pragma unroll
        for (int y = 0; y < C::FR; ++y)
          acc[x][y] = MODE == 0 ? mfma32(fw[x], fr[y], acc[x][y])    // D[n][c]
                                : mfma32(fr[y], fw[x], acc[x][y]);   // D[c][d]
    }
  };

  const int steps = (nr + KS - 1) / KS;
#pragma unroll
  for (int st = 0; st < NS - 1; ++st) issue(st, st);
  for (int st = 0; st < steps; ++st) {
    // This wave's reads of the slot refilled below (step st-1's) are done;
    // once its copies of stage st have landed, meet the other waves.
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    wait_vm_barrier<(NS - 2) * C::CW>();
    issue(st + NS - 1, (st + NS - 1) % NS);
    compute(st % NS);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // zero-page copies past the last stage

  // A single-chunk adapter's sum is its gradient: written straight to dB_j
  // [r_j][big_n] or dA_j [d_in][r_j] (columns c < r_j), not to the partials.
  const bool direct = a.direct && ldc(a.t.ch_count + j) == 1;
  const int rj = ldc(a.t.ranks + j);
  float* const grad = direct ? static_cast<float*>(ldc((MODE == 0 ? a.dB : a.dA) + j)) : nullptr;
#pragma unroll
  for (int x = 0; x < C::FW; ++x) {
#pragma unroll
    for (int y = 0; y < C::FR; ++y) {
      const int nb = col0 + 32 * (C::FW * wa + x), cb = 32 * (C::FR * wb + y);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 v;
        v[0] = acc[x][y][4 * g + 0];
        v[1] = acc[x][y][4 * g + 1];
        v[2] = acc[x][y][4 * g + 2];
        v[3] = acc[x][y][4 * g + 3];
        if (MODE == 0) {
          // D[n][c]: lane holds c = cb + l32, n = nb + 8g + 4half + e
          const int c = cb + l32;
          const int n = nb + 8 * g + 4 * half;
          if (n < big_n) {
            if (!direct)
              *reinterpret_cast<f32x4*>(part + ldc(a.t.cboff + ch) + (int64_t)c * big_n + n) = v;
            else if (c < rj) {
              f32x4* gp = reinterpret_cast<f32x4*>(grad + (int64_t)c * big_n + n);
              *gp = a.t.accumulate ? *gp + v : v;
            }
          }
        } else {
          // D[c][d]: lane holds d = nb + l32, c = cb + 8g + 4half + e
          const int d = nb + l32;
          const int c = cb + 8 * g + 4 * half;
          if (d < big_n) {
            if (!direct) {
              *reinterpret_cast<f32x4*>(part + cp * big_n + (int64_t)d * RP + c) = v;
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (c + e < rj) {
                  float* gp = grad + (int64_t)d * rj + c + e;
                  *gp = a.t.accumulate ? *gp + v[e] : v[e];
                }
            }
          }
        }
      }
    }
  }
}

// Workgroup b runs on XCD b % 8; item b' gives XCD x the contiguous items
// [x q + min(x, r), ...) of total = 8 q + r, so the column blocks of one
// chunk, which share its rank operand, meet in one XCD's L2.
__device__ __forceinline__ int xcd_item(int b, int total) {
  const int x = b & 7, q = total >> 3, r = total & 7;
  return x * q + min(x, r) + (b >> 3);
}

template <int RP>
__global__ __launch_bounds__(256, TrCfg<RP>::WGS) void k_token_reduce_dma(TokenReduceArgs a) {
  __shared__ u32x4 ring[TrCfg<RP>::NS * TrCfg<RP>::STAGE / 16];
  const MLORA_LDS char* lds = (const MLORA_LDS char*)(MLORA_LDS void*)&ring[0];
  const uint32_t ring_lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(MLORA_LDS void*)&ring[0]);
  constexpr int WN = TrCfg<RP>::WN;
  const int nbb_b = (int)((a.d_out + WN - 1) / WN);
  const int nbb_a = (int)((a.d_in + WN - 1) / WN);
  const int nb_b = a.n_chunks * nbb_b;
  const int b = xcd_item(blockIdx.x, a.n_chunks * (nbb_b + nbb_a));
  if (b < nb_b)
    token_reduce_dma_body<RP, 0>(a, a.chunk_begin + b / nbb_b, (b % nbb_b) * WN, lds, ring_lds);
  else
    token_reduce_dma_body<RP, 1>(a, a.chunk_begin + (b - nb_b) / nbb_a, ((b - nb_b) % nbb_a) * WN, lds,
                                 ring_lds);
}

// Rows in the caller's order (a permutation table) go through the register
// path, which gathers them; grouped rows through the direct-to-LDS path.
template <int RP>
static void launch_token_reduce_rp(const TokenReduceArgs& a, hipStream_t s) {
  const int wn = a.t.perm ? 128 : TrCfg<RP>::WN;
  const int nbb = (int)((a.d_out + wn - 1) / wn + (a.d_in + wn - 1) / wn);
  const dim3 grid((unsigned)(a.n_chunks * nbb)), block(256);
  if (a.t.perm) hipLaunchKernelGGL((k_token_reduce<RP, true>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((k_token_reduce_dma<RP>), grid, block, 0, s, a);
}

void launch_token_reduce(int rp, const DevTables& t, int32_t chunk_begin, int32_t chunk_count,
                         const uint16_t* dY, int64_t ld_dy, const uint16_t* Z, float* partB,
                         int64_t d_out, const uint16_t* X, const uint16_t* dZ, float* partA,
                         int64_t d_in, void* const* dA, void* const* dB, hipStream_t s) {
  if (chunk_count <= 0) return;
  const TokenReduceArgs a{t, chunk_begin, chunk_count, dY, ld_dy, Z, partB, d_out, X, dZ, partA, d_in,
                          dA, dB, t.perm ? 0 : 1};
  switch (rp) {
    case 32: launch_token_reduce_rp<32>(a, s); break;
    case 64: launch_token_reduce_rp<64>(a, s); break;
    case 128: launch_token_reduce_rp<128>(a, s); break;
    default: launch_token_reduce_rp<256>(a, s); break;
  }
}

// ---------------------------------------------------------------------------
// Fixed-order sum of chunk partials: dA_j[d][c] and dB_j[c][n] for c < r_j.
// grid.y walks adapters; each thread owns four consecutive partial columns
// (c of one d for dA, n of one c for dB) and adds the adapter's chunks in
// chunk order, so results do not depend on the launch shape.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_reduce_partials(DevTables t, int32_t a_begin, int32_t a_end,
                                                         int64_t d_in, int64_t d_out,
                                                         const float* partA, const float* partB,
                                                         void* const* dA, void* const* dB) {
  for (int32_t j = a_begin + blockIdx.y; j < a_end; j += gridDim.y) {
    const int r = ldc(t.ranks + j), rp = ldc(t.rpad + j);
    const int first = ldc(t.ch_first + j), cnt = ldc(t.ch_count + j);
    if (cnt == 1 && !t.perm) continue;   // written by the token reduction itself
    const int pq = j % t.nproj;
    const int64_t w = ldc(t.pcol + pq + 1) - ldc(t.pcol + pq);   // dB_j is [r][w]
    const int64_t na4 = d_in * (rp / 4), nb4 = (int64_t)r * (w / 4);
    float* gA = static_cast<float*>(ldc(dA + j));
    float* gB = static_cast<float*>(ldc(dB + j));
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < na4 + nb4;
         i += (int64_t)gridDim.x * 256) {
      f32x4 sum = {0.f, 0.f, 0.f, 0.f};
      if (i < na4) {
        const int64_t d = i / (rp / 4);
        const int c0 = 4 * (int)(i - d * (rp / 4));
        if (c0 >= r) continue;
        for (int k = 0; k < cnt; ++k)
          sum += *reinterpret_cast<const f32x4*>(partA + (int64_t)ldc(t.cpref + first + k) * d_in + d * rp + c0);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (c0 + e < r) gA[d * r + c0 + e] = t.accumulate ? gA[d * r + c0 + e] + sum[e] : sum[e];
      } else {
        const int64_t q = 4 * (i - na4);
        for (int k = 0; k < cnt; ++k)
          sum += *reinterpret_cast<const f32x4*>(partB + ldc(t.cboff + first + k) + q);
        if (t.accumulate) sum += *reinterpret_cast<const f32x4*>(gB + q);
        *reinterpret_cast<f32x4*>(gB + q) = sum;
      }
    }
  }
}

void launch_reduce_partials(const DevTables& t, int32_t a_begin, int32_t a_end, int64_t d_in,
                            int64_t d_out, const float* partA, const float* partB,
                            void* const* dA, void* const* dB, int32_t max_rank, hipStream_t s) {
  const int32_t na = a_end - a_begin;
  if (na <= 0) return;
  const int64_t max_rp = max_rank <= 32 ? 32 : (max_rank <= 64 ? 64 : (max_rank <= 128 ? 128 : 256));
  const int64_t per = (d_in * max_rp + (int64_t)max_rank * d_out) / 4;
  int64_t bx = (per + 255) / 256;
  if (bx > 1024) bx = 1024;
  dim3 grid((unsigned)bx, (unsigned)(na < 65535 ? na : 65535));
  hipLaunchKernelGGL(k_reduce_partials, grid, dim3(256), 0, s, t, a_begin, a_end, d_in, d_out,
                     partA, partB, dA, dB);
}

}  // namespace mlora
