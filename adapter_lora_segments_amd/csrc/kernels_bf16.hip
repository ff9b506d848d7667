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

namespace mlora {

// ---------------------------------------------------------------------------
// A_cat^T: row roff(j)+c, c < r_pad(j), holds column c of A_j (zero past r_j).
// One workgroup per (64-row slab of A_j, adapter j).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_prep_acat_t(DevTables t, int32_t n, int64_t d_in,
                                                     const void* const* A, uint16_t* acat_t) {
  __shared__ uint16_t tile[64][258];
  const int64_t k0 = (int64_t)blockIdx.x * 64;
  for (int32_t j = blockIdx.y; j < n; j += gridDim.y) {
    const int r = t.ranks[j], rp = t.rpad[j];
    const uint16_t* Aj = static_cast<const uint16_t*>(A[j]);
    for (int i = threadIdx.x; i < 64 * r; i += 256) {
      const int k = i / r, c = i - k * r;
      tile[k][c] = Aj[k0 * r + i];
    }
    __syncthreads();
    uint16_t* dst = acat_t + (int64_t)t.roff[j] * d_in + k0;
    for (int i = threadIdx.x; i < 64 * rp; i += 256) {
      const int c = i >> 6, k = i & 63;
      dst[(int64_t)c * d_in + k] = c < r ? tile[k][c] : (uint16_t)0;
    }
    __syncthreads();
  }
}

void launch_prep_acat_t(const DevTables& t, int32_t n, int64_t d_in, const void* const* A,
                        uint16_t* acat_t, hipStream_t s) {
  dim3 grid((unsigned)(d_in / 64), (unsigned)(n < 65535 ? n : 65535));
  hipLaunchKernelGGL(k_prep_acat_t, grid, dim3(256), 0, s, t, n, d_in, A, acat_t);
}

// ---------------------------------------------------------------------------
// Skinny products over one nano-batch (<= nano_rows rows of one adapter):
//   out[row][c] = s_j * sum_k P[row][k] * Q_j[c][k],  c < RP = r_pad(j)
// Both operands are k-contiguous, so MFMA fragments load straight from
// global memory (16 bytes per lane).  The four waves split K into quarters
// and their accumulators are summed through LDS.  MODE 0: shrink (Q = rows
// of A_cat^T, all RP rows present); MODE 1: dZ (Q = B_j, rows >= r_j are 0).
// ---------------------------------------------------------------------------
template <int RP, int MODE>
__global__ __launch_bounds__(256) void k_skinny(DevTables t, int32_t nano_begin, const uint16_t* P,
                                                int64_t K, const uint16_t* acat_t,
                                                const void* const* Bptr, const float* scales,
                                                uint16_t* out) {
  constexpr int F = RP / 32;
  constexpr int U = F <= 2 ? 8 : (F == 4 ? 4 : 2);
  __shared__ float red[4][16 * 64];

  const int nb = nano_begin + blockIdx.x;
  const int j = t.nano[3 * nb], row0 = t.nano[3 * nb + 1], nrows = t.nano[3 * nb + 2];
  const float s = scales[j];
  const int64_t oj = t.offsets[j];
  const int64_t zo = t.zoff[j];
  const int rj = t.ranks[j];
  const uint16_t* Q = MODE == 0 ? acat_t + (int64_t)t.roff[j] * K : static_cast<const uint16_t*>(Bptr[j]);

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t kq = K / 4, kbeg = w * kq;
  const int half = lane >> 5, l32 = lane & 31;

  const uint16_t* qp[F];
  bool qv[F];
#pragma unroll
  for (int f = 0; f < F; ++f) {
    const int c = 32 * f + l32;
    qv[f] = MODE == 0 || c < rj;
    qp[f] = Q + (int64_t)(qv[f] ? c : 0) * K + kbeg + 8 * half;
  }

  for (int rf = 0; rf * 32 < nrows; ++rf) {
    const int prow = row0 + 32 * rf + min(l32, nrows - 32 * rf - 1);
    const uint16_t* pp = P + (int64_t)prow * K + kbeg + 8 * half;
    f32x16 acc[F];
#pragma unroll
    for (int f = 0; f < F; ++f)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[f][e] = 0.f;

    int64_t k = 0;
    for (; k + 16 * U <= kq; k += 16 * U) {
      u32x4 pa[U], qa[U][F];
#pragma unroll
      for (int u = 0; u < U; ++u) pa[u] = ld16(pp + k + 16 * u);
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int f = 0; f < F; ++f) qa[u][f] = qv[f] ? ld16(qp[f] + k + 16 * u) : zero4();
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int f = 0; f < F; ++f) acc[f] = mfma32(qa[u][f], pa[u], acc[f]);
    }
    for (; k < kq; k += 16) {
      const u32x4 pa = ld16(pp + k);
#pragma unroll
      for (int f = 0; f < F; ++f) {
        const u32x4 qa = qv[f] ? ld16(qp[f] + k) : zero4();
        acc[f] = mfma32(qa, pa, acc[f]);
      }
    }

    // acc[f][4g+e] = D[c = 32f + 8g + 4*half + e][row = l32]
#pragma unroll
    for (int f = 0; f < F; ++f) {
#pragma unroll
      for (int e = 0; e < 16; ++e) red[w][e * 64 + lane] = acc[f][e];
      __syncthreads();
      {
        const int l = tid & 63, g = tid >> 6;
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int e = 4 * g + i;
          v[i] = red[0][e * 64 + l] + red[1][e * 64 + l] + red[2][e * 64 + l] + red[3][e * 64 + l];
        }
        const int row = 32 * rf + (l & 31);
        if (row < nrows) {
          const int c = 32 * f + 8 * g + 4 * (l >> 5);
          u32x2 pk;
          pk[0] = pack_bf16x2(s * v[0], s * v[1]);
          pk[1] = pack_bf16x2(s * v[2], s * v[3]);
          *reinterpret_cast<u32x2*>(out + zo + (int64_t)(row0 + row - oj) * RP + c) = pk;
        }
      }
      __syncthreads();
    }
  }
}

template <int MODE>
static void skinny_dispatch(int rp, const DevTables& t, int32_t nb0, int32_t cnt, const uint16_t* P,
                            int64_t K, const uint16_t* acat_t, const void* const* Bptr,
                            const float* scales, uint16_t* out, hipStream_t s) {
  dim3 grid((unsigned)cnt), block(256);
  switch (rp) {
    case 32: hipLaunchKernelGGL((k_skinny<32, MODE>), grid, block, 0, s, t, nb0, P, K, acat_t, Bptr, scales, out); break;
    case 64: hipLaunchKernelGGL((k_skinny<64, MODE>), grid, block, 0, s, t, nb0, P, K, acat_t, Bptr, scales, out); break;
    case 128: hipLaunchKernelGGL((k_skinny<128, MODE>), grid, block, 0, s, t, nb0, P, K, acat_t, Bptr, scales, out); break;
    default: hipLaunchKernelGGL((k_skinny<256, MODE>), grid, block, 0, s, t, nb0, P, K, acat_t, Bptr, scales, out); break;
  }
}

// One launch per padded-rank bucket: the caller passes a nano range whose
// adapters share r_pad (the plan orders nano-batches by r_pad inside a group).
void launch_skinny(int mode, const DevTables& t, int32_t nano_begin, int32_t nano_count,
                   const uint16_t* P, int64_t K, const uint16_t* acat_t, const void* const* Bptr,
                   const float* scales, uint16_t* out, hipStream_t s) {
  // The bucket's padded rank is passed in the high bits of `mode`.
  const int rp = mode >> 8;
  if (nano_count <= 0) return;
  if ((mode & 0xff) == 0)
    skinny_dispatch<0>(rp, t, nano_begin, nano_count, P, K, acat_t, Bptr, scales, out, s);
  else
    skinny_dispatch<1>(rp, t, nano_begin, nano_count, P, K, acat_t, Bptr, scales, out, s);
}

// ---------------------------------------------------------------------------
// Token reductions over one chunk (<= KC rows of one adapter) and one block of
// 128 columns of the wide operand:
//   MODE 0 (dB): part[c][n] = sum_t R[t][c] Wd[t][n]  (R = Z', Wd = dY)
//   MODE 1 (dA): part[d][c] = sum_t Wd[t][d] R[t][c]  (R = dZ, Wd = X)
// Both operands are token-major, so each 8x8 block is transposed in
// registers on its way into k-contiguous, swizzled LDS tiles (double
// buffered, one barrier per 64-token step).  Rows past the chunk are zero.
// ---------------------------------------------------------------------------
template <int RP, int MODE>
__global__ __launch_bounds__(256) void k_token_reduce(DevTables t, int32_t chunk_begin, int32_t nbb,
                                                      const uint16_t* big, int64_t big_ld,
                                                      const uint16_t* rk, float* part) {
  constexpr int F = RP / 32;
  constexpr int NBLK = 128 + RP;                 // 8x8 blocks per 64-token step
  constexpr int PER = (NBLK + 255) / 256;        // blocks per thread
  __shared__ u32x4 sbig[2][128 * 8];
  __shared__ u32x4 srk[2][RP * 8];

  const int ch = chunk_begin + blockIdx.x / nbb;
  const int col0 = (blockIdx.x % nbb) * 128;
  const int j = t.chunks[3 * ch], r0 = t.chunks[3 * ch + 1], nr = t.chunks[3 * ch + 2];
  const int64_t cp = t.cpref[ch];
  const uint16_t* rbase = rk + t.zoff[j] + (int64_t)(r0 - t.offsets[j]) * RP;
  const uint16_t* bbase = big + (int64_t)r0 * big_ld;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;

  u32x4 stage[PER][8];

  auto load = [&](int step) {
    const int t0 = step * 64;
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int b = tid + 256 * p;
      if (b < NBLK) {
        const bool isbig = b < 128;
        const int bb = isbig ? b : b - 128;
        const int MB = isbig ? 16 : RP / 8;
        const int mb = bb % MB, kb = bb / MB;
        const bool colok = !isbig || (col0 + 8 * mb < big_ld);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int tk = t0 + 8 * kb + i;
          if (tk < nr && colok) {
            stage[p][i] = isbig ? ld16(bbase + (int64_t)tk * big_ld + col0 + 8 * mb)
                                : ld16(rbase + (int64_t)tk * RP + 8 * mb);
          } else {
            stage[p][i] = zero4();
          }
        }
      }
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int b = tid + 256 * p;
      if (b < NBLK) {
        const bool isbig = b < 128;
        const int bb = isbig ? b : b - 128;
        const int MB = isbig ? 16 : RP / 8;
        const int mb = bb % MB, kb = bb / MB;
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

  const int steps = (nr + 63) / 64;
  load(0);
  store(0);
  __syncthreads();
  for (int st = 0; st < steps; ++st) {
    const int buf = st & 1;
    if (st + 1 < steps) load(st + 1);
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
    if (st + 1 < steps) store(buf ^ 1);
    __syncthreads();
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
        if (n < big_ld)
          *reinterpret_cast<f32x4*>(part + cp * big_ld + (int64_t)c * big_ld + n) = v;
      } else {
        // lane holds d = col0 + 32w + l32, c = 32f + 8g + 4half + e
        const int d = col0 + 32 * w + l32;
        const int c = 32 * f + 8 * g + 4 * half;
        if (d < big_ld)
          *reinterpret_cast<f32x4*>(part + cp * big_ld + (int64_t)d * RP + c) = v;
      }
    }
  }
}

template <int MODE>
static void token_reduce_dispatch(int rp, const DevTables& t, int32_t c0, int32_t cnt,
                                  const uint16_t* big, int64_t big_ld, const uint16_t* rk,
                                  float* part, hipStream_t s) {
  const int nbb = (int)((big_ld + 127) / 128);
  dim3 grid((unsigned)(cnt * nbb)), block(256);
  switch (rp) {
    case 32: hipLaunchKernelGGL((k_token_reduce<32, MODE>), grid, block, 0, s, t, c0, nbb, big, big_ld, rk, part); break;
    case 64: hipLaunchKernelGGL((k_token_reduce<64, MODE>), grid, block, 0, s, t, c0, nbb, big, big_ld, rk, part); break;
    case 128: hipLaunchKernelGGL((k_token_reduce<128, MODE>), grid, block, 0, s, t, c0, nbb, big, big_ld, rk, part); break;
    default: hipLaunchKernelGGL((k_token_reduce<256, MODE>), grid, block, 0, s, t, c0, nbb, big, big_ld, rk, part); break;
  }
}

void launch_token_reduce(int mode, const DevTables& t, int32_t chunk_begin, int32_t chunk_count,
                         const uint16_t* big, int64_t big_ld, const uint16_t* rk, float* part,
                         hipStream_t s) {
  const int rp = mode >> 8;
  if (chunk_count <= 0) return;
  if ((mode & 0xff) == 0)
    token_reduce_dispatch<0>(rp, t, chunk_begin, chunk_count, big, big_ld, rk, part, s);
  else
    token_reduce_dispatch<1>(rp, t, chunk_begin, chunk_count, big, big_ld, rk, part, s);
}

// ---------------------------------------------------------------------------
// Fixed-order sum of chunk partials: dA_j[d][c] and dB_j[c][n] for c < r_j.
// grid.y walks adapters; each thread owns one output element.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_reduce_partials(DevTables t, int32_t a_begin, int32_t a_end,
                                                         int64_t d_in, int64_t d_out,
                                                         const float* partA, const float* partB,
                                                         void* const* dA, void* const* dB) {
  for (int32_t j = a_begin + blockIdx.y; j < a_end; j += gridDim.y) {
    const int r = t.ranks[j], rp = t.rpad[j];
    const int first = t.ch_first[j], cnt = t.ch_count[j];
    const int64_t na = d_in * r, nbv = (int64_t)r * d_out;
    float* gA = static_cast<float*>(dA[j]);
    float* gB = static_cast<float*>(dB[j]);
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < na + nbv;
         i += (int64_t)gridDim.x * 256) {
      float sum = 0.f;
      if (i < na) {
        const int64_t d = i / r;
        const int c = (int)(i - d * r);
        for (int k = 0; k < cnt; ++k)
          sum += partA[(int64_t)t.cpref[first + k] * d_in + d * rp + c];
        gA[i] = sum;
      } else {
        const int64_t q = i - na;
        for (int k = 0; k < cnt; ++k) sum += partB[(int64_t)t.cpref[first + k] * d_out + q];
        gB[q] = sum;
      }
    }
  }
}

void launch_reduce_partials(const DevTables& t, int32_t a_begin, int32_t a_end, int64_t d_in,
                            int64_t d_out, const float* partA, const float* partB,
                            void* const* dA, void* const* dB, int32_t max_rank, hipStream_t s) {
  const int32_t na = a_end - a_begin;
  if (na <= 0) return;
  int64_t per = (d_in + d_out) * (int64_t)max_rank;
  int64_t bx = (per + 255) / 256;
  if (bx > 1024) bx = 1024;
  dim3 grid((unsigned)bx, (unsigned)(na < 65535 ? na : 65535));
  hipLaunchKernelGGL(k_reduce_partials, grid, dim3(256), 0, s, t, a_begin, a_end, d_in, d_out,
                     partA, partB, dA, dB);
}

// ---------------------------------------------------------------------------
// Base GEMM with the LoRA term as extra K-steps (the expand of the forward,
// PLoRA §9.2 Case 4's dZ.A^T in the backward).  256x256 tile per workgroup,
// four waves of 128x128, 64-deep K-steps through double-buffered swizzled
// LDS (128 KiB), one barrier per step.  Extension step e of a row tile loads
// rows [lo,hi) of E_j (other rows zero) and k-rows [k0, k0+64) of EB_j
// (rows >= r_j zero).  Output written as bf16.
// ---------------------------------------------------------------------------
template <bool FWD, bool MAIN_B_KC>
__global__ __launch_bounds__(256, 1) void k_gemm(GemmArgs g) {
  __shared__ u32x4 lds[2][2][256 * 8];

  // XCD-aware order: workgroup b runs on XCD b % 8; give each XCD a
  // contiguous range of logical tiles, grouped 8 row tiles at a time.
  const int G = gridDim.x, bid = blockIdx.x;
  const int xcd = bid & 7, q = bid >> 3, per = G >> 3, rem = G & 7;
  const int L = xcd * per + min(xcd, rem) + q;
  const int nM = g.n_mtiles, nN = g.n_ntiles;
  constexpr int GM = 8;
  const int grp = L / (GM * nN);
  const int fm = grp * GM;
  const int gm = min(GM, nM - fm);
  const int within = L - grp * GM * nN;
  const int tm = fm + within % gm, tn = within / gm;

  const int tix = g.tile_begin + tm;
  const int row0 = g.t.tiles[2 * tix], mrows = g.t.tiles[2 * tix + 1];
  const int e0 = g.t.ext_start[tix], e1 = g.t.ext_start[tix + 1];
  const int n0 = tn * 256;
  const int nk = g.K / 64;
  const int nsteps = nk + (e1 - e0);

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int wm = w >> 1, wn = w & 1;
  const int lrow = tid >> 3, lch = tid & 7;      // k-contiguous loader: row, chunk
  const int tmb = tid & 31, tkb = tid >> 5;      // transposing loader: 8x8 block

  u32x4 ra[8], rb[8];
  bool b_transposed = false;  // how rb must be written for the staged step

  auto load = [&](int step) {
    if (step < nk) {
      const int k0 = step * 64;
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        const int r = lrow + 32 * p;
        const int grow = row0 + min(r, mrows - 1);
        ra[p] = ld16(g.A + (int64_t)grow * g.lda + k0 + 8 * lch);
      }
      if (MAIN_B_KC) {
#pragma unroll
        for (int p = 0; p < 8; ++p) {
          const int gn = min(n0 + lrow + 32 * p, g.N - 1);
          rb[p] = ld16(g.B + (int64_t)gn * g.ldb + k0 + 8 * lch);
        }
        b_transposed = false;
      } else {
        const int col = min(n0 + 8 * tmb, g.N - 8);
#pragma unroll
        for (int i = 0; i < 8; ++i) rb[i] = ld16(g.B + (int64_t)(k0 + 8 * tkb + i) * g.ldb + col);
        b_transposed = true;
      }
    } else {
      const int e = e0 + step - nk;
      const int j = g.t.ext[4 * e], lo = g.t.ext[4 * e + 1], hi = g.t.ext[4 * e + 2];
      const int k0 = g.t.ext[4 * e + 3];
      const int rp = g.t.rpad[j], rj = g.t.ranks[j];
      const int64_t oj = g.t.offsets[j];
      const uint16_t* zb = g.ebuf + g.t.zoff[j];
      const int kk = k0 + 8 * lch;
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        const int grow = row0 + lrow + 32 * p;
        ra[p] = (grow >= lo && grow < hi && kk < rp) ? ld16(zb + (grow - oj) * rp + kk) : zero4();
      }
      const uint16_t* eb = static_cast<const uint16_t*>(g.eb[j]);
      if (FWD) {
        // EB_j = B_j [r_j][N], n contiguous: transposing loader
        const int col = min(n0 + 8 * tmb, g.N - 8);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int k = k0 + 8 * tkb + i;
          rb[i] = k < rj ? ld16(eb + (int64_t)k * g.N + col) : zero4();
        }
        b_transposed = true;
      } else {
        // EB_j(k, n) = A_j[n][k], k contiguous with row stride r_j
#pragma unroll
        for (int p = 0; p < 8; ++p) {
          const int gn = min(n0 + lrow + 32 * p, g.N - 1);
          const uint16_t* src = eb + (int64_t)gn * rj;
          if ((rj & 7) == 0) {
            rb[p] = kk < rj ? ld16(src + kk) : zero4();
          } else {
            uint32_t v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = (kk + i < rj) ? (uint32_t)src[kk + i] : 0u;
            rb[p] = u32x4{v[0] | (v[1] << 16), v[2] | (v[3] << 16), v[4] | (v[5] << 16),
                          v[6] | (v[7] << 16)};
          }
        }
        b_transposed = false;
      }
    }
  };

  auto store = [&](int buf) {
#pragma unroll
    for (int p = 0; p < 8; ++p) lds[buf][0][swz(lrow + 32 * p, lch)] = ra[p];
    if (b_transposed) {
      u32x4 tr[8];
      transpose8x8(rb, tr);
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) lds[buf][1][swz(8 * tmb + jj, tkb)] = tr[jj];
    } else {
#pragma unroll
      for (int p = 0; p < 8; ++p) lds[buf][1][swz(lrow + 32 * p, lch)] = rb[p];
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.f;

  load(0);
  store(0);
  __syncthreads();
  for (int st = 0; st < nsteps; ++st) {
    const int buf = st & 1;
    if (st + 1 < nsteps) load(st + 1);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      u32x4 af[4], bfr[4];
#pragma unroll
      for (int fi = 0; fi < 4; ++fi) af[fi] = lds[buf][0][swz(128 * wm + 32 * fi + l32, 2 * ks + half)];
#pragma unroll
      for (int fj = 0; fj < 4; ++fj) bfr[fj] = lds[buf][1][swz(128 * wn + 32 * fj + l32, 2 * ks + half)];
#pragma unroll
      for (int fi = 0; fi < 4; ++fi)
#pragma unroll
        for (int fj = 0; fj < 4; ++fj) acc[fi][fj] = mfma32(bfr[fj], af[fi], acc[fi][fj]);
    }
    if (st + 1 < nsteps) store(buf ^ 1);
    __syncthreads();
  }

  // acc[fi][fj][4gg+e] = C[m = 128wm + 32fi + l32][n = 128wn + 32fj + 8gg + 4half + e]
#pragma unroll
  for (int fi = 0; fi < 4; ++fi) {
    const int m = 128 * wm + 32 * fi + l32;
    if (m < mrows) {
      uint16_t* crow = g.C + (int64_t)(row0 + m) * g.ldc;
#pragma unroll
      for (int fj = 0; fj < 4; ++fj) {
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
          const int n = n0 + 128 * wn + 32 * fj + 8 * gg + 4 * half;
          if (n < g.N) {
            u32x2 pk;
            pk[0] = pack_bf16x2(acc[fi][fj][4 * gg + 0], acc[fi][fj][4 * gg + 1]);
            pk[1] = pack_bf16x2(acc[fi][fj][4 * gg + 2], acc[fi][fj][4 * gg + 3]);
            *reinterpret_cast<u32x2*>(crow + n) = pk;
          }
        }
      }
    }
  }
}

void launch_gemm(bool fwd, bool main_b_kcontig, const GemmArgs& g, hipStream_t s) {
  const int total = g.n_mtiles * g.n_ntiles;
  if (total <= 0) return;
  dim3 grid((unsigned)total), block(256);
  if (fwd) {
    if (main_b_kcontig) hipLaunchKernelGGL((k_gemm<true, true>), grid, block, 0, s, g);
    else hipLaunchKernelGGL((k_gemm<true, false>), grid, block, 0, s, g);
  } else {
    if (main_b_kcontig) hipLaunchKernelGGL((k_gemm<false, true>), grid, block, 0, s, g);
    else hipLaunchKernelGGL((k_gemm<false, false>), grid, block, 0, s, g);
  }
}

}  // namespace mlora
