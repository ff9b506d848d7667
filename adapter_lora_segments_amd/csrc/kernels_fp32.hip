// fp32 kernels of the packed multi-LoRA layer (vector ALU, fp32 throughout,
// no reduced-precision step).  Rows are grouped by adapter; with a plan from
// per-token ids, X, dY, Y and dX rows are read and written at the caller's
// row through the plan's permutation.  Same steps as the bf16 path (PLoRA: Efficient
// Concurrent LoRA Training for Large Language Models, §2.1 and §9.2); each
// row finds its adapter by binary search over the segment offsets, and each
// weight gradient is one thread's sum over its adapter's rows in row order.
// With several projections sharing the input, pair v = i * nproj + q of
// adapter i and projection q owns output columns [pcol[q], pcol[q+1]).
#include "device_common.hpp"
#include "kernels.hpp"

namespace mlora {

// Caller's row of grouped row `row` (plans from per-token ids), else `row`.
__device__ __forceinline__ int64_t caller_row(const DevTables& t, int64_t row) {
  return t.perm ? (int64_t)t.perm[row] : row;
}

// Adapter owning `row`: the largest i with offsets[i] <= row (empty
// segments before it are skipped because their end equals their start).
__device__ __forceinline__ int adapter_of(const int64_t* off, int n, int64_t row) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (off[mid] <= row) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// Z'[row][c] = s_j sum_k X[row][k] A_j[k][c]; zero for r_j <= c < r_pad(j).
// blockIdx.y is the projection.
__global__ __launch_bounds__(256) void k_f32_shrink(DevTables t, int32_t n, int64_t d_in,
                                                    const float* X, const void* const* A,
                                                    const float* scales, float* Z) {
  const int64_t row = blockIdx.x;
  const int i = adapter_of(t.offsets, n, row);
  const int j = i * t.nproj + blockIdx.y;
  const int c = threadIdx.x;
  const int r = t.ranks[j], rp = t.rpad[j];
  if (c >= rp) return;
  float acc = 0.f;
  if (c < r) {
    const float* Aj = static_cast<const float*>(A[j]);
    const float* x = X + caller_row(t, row) * d_in;
    for (int64_t k = 0; k < d_in; ++k) acc = fmaf(x[k], Aj[k * r + c], acc);
    acc *= scales[j];
  }
  Z[t.zoff[j] + (row - t.offsets[i]) * rp + c] = acc;
}

// dZ[row][c] = s_j sum_o dY[row][c_q + o] B_j[c][o] over projection q's
// width (blockIdx.y = q; rows of dY are d_out long).
__global__ __launch_bounds__(256) void k_f32_dz(DevTables t, int32_t n, int64_t d_out,
                                                const float* dY, const void* const* B,
                                                const float* scales, float* dZ) {
  const int64_t row = blockIdx.x;
  const int i = adapter_of(t.offsets, n, row);
  const int q = blockIdx.y, j = i * t.nproj + q;
  const int64_t c0 = t.pcol[q], w = t.pcol[q + 1] - c0;
  const int c = threadIdx.x;
  const int r = t.ranks[j], rp = t.rpad[j];
  if (c >= rp) return;
  float acc = 0.f;
  if (c < r) {
    const float* Bj = static_cast<const float*>(B[j]) + (int64_t)c * w;
    const float* g = dY + caller_row(t, row) * d_out + c0;
    for (int64_t o = 0; o < w; ++o) acc = fmaf(g[o], Bj[o], acc);
    acc *= scales[j];
  }
  dZ[t.zoff[j] + (row - t.offsets[i]) * rp + c] = acc;
}

// C = Aop Bop + per-row LoRA term.  64x64 tile, 16x16 threads, 4x4 outputs
// each, 16-deep K-steps through LDS.
template <bool FWD, bool B_KC>
__global__ __launch_bounds__(256) void k_f32_gemm(DevTables t, int32_t n, int64_t T,
                                                  const float* A, int64_t lda, const float* B,
                                                  int64_t ldb, float* C, int64_t ldc, int32_t K,
                                                  int32_t N, const float* E,
                                                  const void* const* eb) {
  __shared__ float As[16][65];
  __shared__ float Bs[16][65];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int64_t m0 = (int64_t)blockIdx.y * 64;
  const int n0 = blockIdx.x * 64;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += 16) {
    for (int i = threadIdx.x; i < 1024; i += 256) {
      const int r = i >> 4, kk = i & 15;
      int64_t row = m0 + r;
      if (row >= T) row = T - 1;
      As[kk][r] = A[caller_row(t, row) * lda + k0 + kk];
      const int nn = i >> 4, k2 = i & 15;
      if (B_KC) {
        Bs[k2][nn] = B[(int64_t)(n0 + nn) * ldb + k0 + k2];
      } else {
        const int kr = i >> 6, nc = i & 63;
        Bs[kr][nc] = B[(int64_t)(k0 + kr) * ldb + n0 + nc];
      }
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty + 16 * i];
#pragma unroll
      for (int i = 0; i < 4; ++i) b[i] = Bs[kk][tx + 16 * i];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[i][q] = fmaf(a[i], b[q], acc[i][q]);
    }
    __syncthreads();
  }
  // Forward: the 64-column tile lies in one projection, whose pair adds its
  // expand; dX: every projection's pair adds dZ A^T.
  const int NP = t.nproj;
  int pq = 0;
  while (FWD && pq + 1 < NP && t.pcol[pq + 1] <= n0) ++pq;
  const int64_t pc0 = t.pcol[pq], pw = t.pcol[pq + 1] - pc0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t row = m0 + ty + 16 * i;
    if (row >= T) continue;
    const int ad = adapter_of(t.offsets, n, row);
    for (int qq = FWD ? pq : 0; qq < (FWD ? pq + 1 : NP); ++qq) {
      const int j = ad * NP + qq;
      const int r = t.ranks[j], rp = t.rpad[j];
      const float* e = E + t.zoff[j] + (row - t.offsets[ad]) * rp;
      const float* w = static_cast<const float*>(eb[j]);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = n0 + tx + 16 * q;
        float v = acc[i][q];
        for (int c = 0; c < r; ++c) {
          const float ebv = FWD ? w[(int64_t)c * pw + (col - pc0)] : w[(int64_t)col * r + c];
          v = fmaf(e[c], ebv, v);
        }
        acc[i][q] = v;
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) C[caller_row(t, row) * ldc + n0 + tx + 16 * q] = acc[i][q];
  }
}

// dB_j[c][o] = sum_{rows of j} Z'[t][c] dY[t][c_q + o] over pairs j (n of
// them), o below the width of j's projection q; rows of dY are d_out long.
__global__ __launch_bounds__(256) void k_f32_db(DevTables t, int32_t n, int64_t d_out,
                                                const float* Z, const float* dY,
                                                void* const* dB) {
  for (int32_t j = blockIdx.y; j < n; j += gridDim.y) {
    const int r = t.ranks[j], rp = t.rpad[j];
    const int q = j % t.nproj, ad = j / t.nproj;
    const int64_t c0 = t.pcol[q], w = t.pcol[q + 1] - c0;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (int64_t)r * w) continue;
    const int c = (int)(idx / w);
    const int64_t o = idx - (int64_t)c * w;
    const int64_t a = t.offsets[ad], b = t.offsets[ad + 1];
    const float* z = Z + t.zoff[j] + c;
    float acc = 0.f;
    for (int64_t row = a; row < b; ++row)
      acc = fmaf(z[(row - a) * rp], dY[caller_row(t, row) * d_out + c0 + o], acc);
    float* gp = static_cast<float*>(dB[j]) + idx;
    *gp = t.accumulate ? *gp + acc : acc;
  }
}

// dA_j[d][c] = sum_{rows of j} X[t][d] dZ[t][c]
__global__ __launch_bounds__(256) void k_f32_da(DevTables t, int32_t n, int64_t d_in,
                                                const float* X, const float* dZ,
                                                void* const* dA) {
  for (int32_t j = blockIdx.y; j < n; j += gridDim.y) {
    const int r = t.ranks[j], rp = t.rpad[j];
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= d_in * r) continue;
    const int64_t d = idx / r;
    const int c = (int)(idx - d * r);
    const int ad = j / t.nproj;
    const int64_t a = t.offsets[ad], b = t.offsets[ad + 1];
    const float* g = dZ + t.zoff[j] + c;
    float acc = 0.f;
    for (int64_t row = a; row < b; ++row)
      acc = fmaf(X[caller_row(t, row) * d_in + d], g[(row - a) * rp], acc);
    float* gp = static_cast<float*>(dA[j]) + idx;
    *gp = t.accumulate ? *gp + acc : acc;
  }
}

void launch_f32_shrink(const DevTables& t, int32_t n, int64_t T, int64_t d_in, const float* X,
                       const void* const* A, const float* scales, float* Z, hipStream_t s) {
  if (T <= 0) return;
  hipLaunchKernelGGL(k_f32_shrink, dim3((unsigned)T, (unsigned)t.nproj), dim3(256), 0, s, t, n, d_in, X, A,
                     scales, Z);
}

void launch_f32_dz(const DevTables& t, int32_t n, int64_t T, int64_t d_out, const float* dY,
                   const void* const* B, const float* scales, float* dZ, hipStream_t s) {
  if (T <= 0) return;
  hipLaunchKernelGGL(k_f32_dz, dim3((unsigned)T, (unsigned)t.nproj), dim3(256), 0, s, t, n, d_out, dY, B,
                     scales, dZ);
}

void launch_f32_gemm(bool fwd, bool kc, const DevTables& t, int32_t n, int64_t T, const float* A,
                     int64_t lda, const float* B, int64_t ldb, float* C, int64_t ldc, int32_t K,
                     int32_t N, const float* E, const void* const* eb, hipStream_t s) {
  if (T <= 0) return;
  dim3 grid((unsigned)(N / 64), (unsigned)((T + 63) / 64));
  if (fwd) {
    if (kc) hipLaunchKernelGGL((k_f32_gemm<true, true>), grid, dim3(256), 0, s, t, n, T, A, lda, B, ldb, C, ldc, K, N, E, eb);
    else hipLaunchKernelGGL((k_f32_gemm<true, false>), grid, dim3(256), 0, s, t, n, T, A, lda, B, ldb, C, ldc, K, N, E, eb);
  } else {
    if (kc) hipLaunchKernelGGL((k_f32_gemm<false, true>), grid, dim3(256), 0, s, t, n, T, A, lda, B, ldb, C, ldc, K, N, E, eb);
    else hipLaunchKernelGGL((k_f32_gemm<false, false>), grid, dim3(256), 0, s, t, n, T, A, lda, B, ldb, C, ldc, K, N, E, eb);
  }
}

void launch_f32_db(const DevTables& t, int32_t n, int64_t d_out, const float* Z, const float* dY,
                   void* const* dB, int32_t max_rank, hipStream_t s) {
  dim3 grid((unsigned)(((int64_t)max_rank * d_out + 255) / 256), (unsigned)(n < 65535 ? n : 65535));
  hipLaunchKernelGGL(k_f32_db, grid, dim3(256), 0, s, t, n, d_out, Z, dY, dB);
}

void launch_f32_da(const DevTables& t, int32_t n, int64_t d_in, const float* X, const float* dZ,
                   void* const* dA, int32_t max_rank, hipStream_t s) {
  dim3 grid((unsigned)((d_in * max_rank + 255) / 256), (unsigned)(n < 65535 ? n : 65535));
  hipLaunchKernelGGL(k_f32_da, grid, dim3(256), 0, s, t, n, d_in, X, dZ, dA);
}

}  // namespace mlora
