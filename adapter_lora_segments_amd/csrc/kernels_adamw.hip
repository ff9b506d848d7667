// Per-adapter AdamW step for gfx950: one pass over every adapter's fp32
// weights, gradients and moments.
//
// Every packed adapter owns its weights and optimizer state (PLoRA: Efficient
// Concurrent LoRA Training for Large Language Models, §2.4) and its own
// hyperparameters (§2.2, §11.1); AdamW keeps a momentum and a velocity beside
// each weight (§8).  The update is elementwise and reads 16 and writes 12
// bytes per weight (14 with the bf16 copy), so it is bound by HBM bandwidth:
// the kernel streams 16-byte vectors with non-temporal loads and stores
// (every byte is touched once, so none of it is worth keeping in the caches),
// issues all of a thread's loads before the arithmetic, and takes its work
// items from a plan table of fixed-size pieces, so tensors of any rank share
// one launch.
#include "device_common.hpp"
#include "kernels.hpp"

namespace mlora {

namespace {

constexpr int kThreads = 256;
constexpr int kVecPerThread = kOptBlockElems / (4 * kThreads);

__device__ __forceinline__ f32x4 ld_stream(const float* q) {
  return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(q));
}
__device__ __forceinline__ void st_stream(float* q, const f32x4& x) {
  __builtin_nontemporal_store(x, reinterpret_cast<f32x4*>(q));
}

}  // namespace

// Square sum of work item blockIdx.x's gradient elements, 0 for an adapter
// that is not stepped or does not clip.  Fixed order: each thread sums its
// elements in sequence, then a tree over the workgroup.
__global__ __launch_bounds__(kThreads) void k_grad_sq(AdamwArgs a) {
  __shared__ float red[kThreads];
  const int tsr = ldc(a.t.oblk + 2 * blockIdx.x);
  const int piece = ldc(a.t.oblk + 2 * blockIdx.x + 1);
  const int i = tsr >> 1;
  const bool isB = tsr & 1;
  const mlora_adamw_hparams* hp = a.hp + i;
  float acc = 0.f;
  if (ldc(&hp->step) > 0 && ldc(&hp->max_grad_norm) > 0.f) {
    const int pq = i % a.t.nproj;
    const int64_t width = (int64_t)ldc(a.t.pcol + pq + 1) - ldc(a.t.pcol + pq);
    const int64_t numel = (int64_t)ldc(a.t.ranks + i) * (isB ? width : a.d_in);
    const int64_t base = (int64_t)piece * kOptBlockElems + 4 * threadIdx.x;
    const float* g = ldc((isB ? a.dB : a.dA) + i);
#pragma unroll
    for (int u = 0; u < kVecPerThread; ++u) {
      const int64_t e = base + (int64_t)u * 4 * kThreads;
      if (e < numel) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(g + e);
        acc = fmaf(x[0], x[0], acc);
        acc = fmaf(x[1], x[1], acc);
        acc = fmaf(x[2], x[2], acc);
        acc = fmaf(x[3], x[3], acc);
      }
    }
  }
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int h = kThreads / 2; h > 0; h >>= 1) {
    if ((int)threadIdx.x < h) red[threadIdx.x] += red[threadIdx.x + h];
    __syncthreads();
  }
  if (threadIdx.x == 0) a.gsq[blockIdx.x] = red[0];
}

// Clip factor of each pair: the square sums of its work items added in item
// order (thread-strided, then a tree), min(1, max_grad_norm / (norm + 1e-6)),
// or 1 without clipping.
__global__ __launch_bounds__(kThreads) void k_clip_coef(AdamwArgs a, int32_t nv) {
  __shared__ float red[kThreads];
  for (int32_t v = blockIdx.x; v < nv; v += gridDim.x) {
    const int b0 = ldc(a.t.oblk_first + v), b1 = ldc(a.t.oblk_first + v + 1);
    float acc = 0.f;
    for (int b = b0 + (int)threadIdx.x; b < b1; b += kThreads) acc += a.gsq[b];
    red[threadIdx.x] = acc;
    __syncthreads();
    for (int h = kThreads / 2; h > 0; h >>= 1) {
      if ((int)threadIdx.x < h) red[threadIdx.x] += red[threadIdx.x + h];
      __syncthreads();
    }
    if (threadIdx.x == 0) {
      const float mx = ldc(&a.hp[v].max_grad_norm);
      a.coef[v] = mx > 0.f ? fminf(1.0f, mx / (sqrtf(red[0]) + 1e-6f)) : 1.0f;
    }
    __syncthreads();
  }
}

template <bool COPY>
__global__ __launch_bounds__(kThreads) void k_adamw(AdamwArgs a) {
  const int tsr = ldc(a.t.oblk + 2 * blockIdx.x);
  const int piece = ldc(a.t.oblk + 2 * blockIdx.x + 1);
  const int i = tsr >> 1;
  const bool isB = tsr & 1;
  const mlora_adamw_hparams* hp = a.hp + i;
  const int32_t step = ldc(&hp->step);
  if (step <= 0) return;  // whole workgroup: the adapter is not stepped
  const float lr = ldc(&hp->lr), beta1 = ldc(&hp->beta1), beta2 = ldc(&hp->beta2);
  const float eps = ldc(&hp->eps), wd = ldc(&hp->weight_decay);
  const float clip = a.coef ? a.coef[i] : 1.0f;   // per-adapter gradient clip factor

  const int pq = i % a.t.nproj;   // B_i spans its projection's width
  const int64_t width = (int64_t)ldc(a.t.pcol + pq + 1) - ldc(a.t.pcol + pq);
  const int64_t numel = (int64_t)ldc(a.t.ranks + i) * (isB ? width : a.d_in);
  const int64_t base = (int64_t)piece * kOptBlockElems + 4 * threadIdx.x;
  float* p = ldc((isB ? a.B : a.A) + i);
  const float* g = ldc((isB ? a.dB : a.dA) + i);
  float* m = ldc((isB ? a.mB : a.mA) + i);
  float* v = ldc((isB ? a.vB : a.vA) + i);

  // Bias corrections 1 - beta^t as -expm1(t log beta): no cancellation for
  // betas near 1; a beta of 0 gives exactly 1.
  const float t = (float)step;
  const float bc1 = -expm1f(t * logf(beta1));
  const float bc2 = -expm1f(t * logf(beta2));
  const float step_size = lr / bc1;
  const float inv_sqrt_bc2 = 1.0f / sqrtf(bc2);
  const float decay = 1.0f - lr * wd;
  const float omb1 = 1.0f - beta1, omb2 = 1.0f - beta2;

  f32x4 P[kVecPerThread], G[kVecPerThread], M[kVecPerThread], V[kVecPerThread];
#pragma unroll
  for (int u = 0; u < kVecPerThread; ++u) {
    const int64_t e = base + (int64_t)u * 4 * kThreads;
    if (e < numel) {  // numel is a multiple of 64: a vector is wholly in or out
      P[u] = ld_stream(p + e);
      G[u] = ld_stream(g + e);
      M[u] = ld_stream(m + e);
      V[u] = ld_stream(v + e);
    }
  }
#pragma unroll
  for (int u = 0; u < kVecPerThread; ++u) {
    const int64_t e = base + (int64_t)u * 4 * kThreads;
    if (e >= numel) continue;
    f32x4 pn, mn, vn;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float gc = G[u][c] * clip;
      const float mc = fmaf(beta1, M[u][c], omb1 * gc);
      const float vc = fmaf(beta2, V[u][c], omb2 * (gc * gc));
      const float den = sqrtf(vc) * inv_sqrt_bc2 + eps;
      pn[c] = P[u][c] * decay - step_size * (mc / den);
      mn[c] = mc;
      vn[c] = vc;
    }
    st_stream(p + e, pn);
    st_stream(m + e, mn);
    st_stream(v + e, vn);
    if constexpr (COPY) {
      uint16_t* w = ldc((isB ? a.B_copy : a.A_copy) + i);
      __builtin_nontemporal_store(u32x2{pack_bf16x2(pn[0], pn[1]), pack_bf16x2(pn[2], pn[3])},
                                  reinterpret_cast<u32x2*>(w + e));
    }
  }
}

void launch_grad_norm(const AdamwArgs& a, int64_t n_blocks, int32_t nv, hipStream_t s) {
  if (n_blocks > 0) hipLaunchKernelGGL(k_grad_sq, dim3((unsigned)n_blocks), dim3(kThreads), 0, s, a);
  if (nv > 0)
    hipLaunchKernelGGL(k_clip_coef, dim3((unsigned)(nv < 65535 ? nv : 65535)), dim3(kThreads), 0, s, a, nv);
}

void launch_adamw(const AdamwArgs& a, int64_t n_blocks, hipStream_t s) {
  if (n_blocks <= 0) return;
  const dim3 grid((unsigned)n_blocks), block(kThreads);
  if (a.A_copy)
    hipLaunchKernelGGL(k_adamw<true>, grid, block, 0, s, a);
  else
    hipLaunchKernelGGL(k_adamw<false>, grid, block, 0, s, a);
}

}  // namespace mlora
