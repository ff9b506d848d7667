// Ceiling probes (include/mlora_probes.h): a pure-MFMA loop in the base
// GEMM's instruction pattern, streaming copy / read kernels, and the paths
// from L2 into LDS.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mlora_probes.h"
#include "device_common.hpp"

namespace {

using mlora::f32x16;
using mlora::u32x4;

// Sixteen independent accumulators per wave, as a 128x128 GEMM wave tile
// holds (4 A fragments x 4 B fragments); every MFMA reads a fragment pair,
// so the loop issues back to back with no dependency shorter than 16 MFMAs.
__global__ __launch_bounds__(256, 1) void k_mfma_loop(const u32x4* ops, int64_t iters, float* out) {
  const int lane = threadIdx.x & 63;
  u32x4 a[4], b[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    a[f] = ops[f * 64 + lane];
    b[f] = ops[(4 + f) * 64 + lane];
  }
  f32x16 acc[16];
#pragma unroll
  for (int q = 0; q < 16; ++q)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[q][e] = 0.f;
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[q] = mlora::mfma32(b[q & 3], a[q >> 2], acc[q]);
  }
  float s = 0.f;
#pragma unroll
  for (int q = 0; q < 16; ++q)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[q][e];
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

// Four 16-byte vectors in flight per thread per iteration.
__global__ __launch_bounds__(256) void k_copy(const u32x4* src, u32x4* dst, int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 v0 = src[i], v1 = src[i + stride], v2 = src[i + 2 * stride], v3 = src[i + 3 * stride];
    dst[i] = v0;
    dst[i + stride] = v1;
    dst[i + 2 * stride] = v2;
    dst[i + 3 * stride] = v3;
  }
  for (; i < n16; i += stride) dst[i] = src[i];
}

__global__ __launch_bounds__(256) void k_read(const u32x4* src, int64_t n16, float* out) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 v0 = src[i], v1 = src[i + stride], v2 = src[i + 2 * stride], v3 = src[i + 3 * stride];
    acc ^= v0[0] ^ v1[1] ^ v2[2] ^ v3[3] ^ v0[3] ^ v1[2] ^ v2[1] ^ v3[0];
  }
  for (; i < n16; i += stride) acc ^= src[i][0] ^ src[i][3];
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = (float)acc;
}

// The same loop on the MXFP8 instruction of the quantized base's forward
// (v_mfma_scale_f32_32x32x64_f8f6f4, E4M3 x E4M3, unit scales): 131072
// flops per instruction.
typedef int i32x8 __attribute__((ext_vector_type(8)));
__global__ __launch_bounds__(256, 1) void k_mfma8_loop(const u32x4* ops, int64_t iters, float* out) {
  const int lane = threadIdx.x & 63;
  i32x8 a[4], b[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    const u32x4 p0 = ops[f * 64 + lane], p1 = ops[(4 + f) * 64 + lane];
    a[f] = __builtin_bit_cast(i32x8, __builtin_shufflevector(p0, p1, 0, 1, 2, 3, 4, 5, 6, 7));
    b[f] = __builtin_bit_cast(i32x8, __builtin_shufflevector(p1, p0, 0, 1, 2, 3, 4, 5, 6, 7));
  }
  f32x16 acc[16];
#pragma unroll
  for (int q = 0; q < 16; ++q)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[q][e] = 0.f;
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int q = 0; q < 16; ++q)
      acc[q] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b[q & 3], a[q >> 2], acc[q], 0, 0, 0, 127, 0, 127);
  }
  float s = 0.f;
#pragma unroll
  for (int q = 0; q < 16; ++q)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[q][e];
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

constexpr int kStreamBlocks = 2048;

// Three ways to move L2-resident operand blocks into LDS, the base GEMM's
// copy path and its alternatives.  Every workgroup (160 KiB of LDS, so one
// per CU) streams its own 64 KiB slab `iters` times, each wave sixteen
// 1 KiB pieces per pass:
//   L2L_DIRECT: global_load_lds_dwordx4 (the GEMM's copies), sixteen of the
//     wave's loads in flight;
//   L2L_STAGED: global_load_dwordx4 into registers one pass ahead, then
//     ds_write_b128;
//   L2L_VGPR: the same loads into registers only.
// The slab of workgroup b is src[b * 4096 .. b * 4096 + 4096] (16-byte
// vectors; the staged and register paths read one vector past it on odd
// passes, so src holds n_wg + 1 slabs).
constexpr int kL2lVec = 4096;                  // 16-byte vectors per slab

__device__ __forceinline__ uint32_t l2l_slot(int64_t it, int w, int i) {
  return (uint32_t)((((int)(it & 1)) * 64 + w * 16 + i) % 160);
}

__global__ __launch_bounds__(256, 1) void k_l2l_direct(const u32x4* src, int64_t iters, uint32_t* out) {
  __shared__ u32x4 lds[10240];
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const u32x4* slab = src + (int64_t)blockIdx.x * kL2lVec;
  const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(MLORA_LDS void*)lds);
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 16; ++i) mlora::dma16_at(slab + (w * 16 + i) * 64 + lane, base + 1024u * l2l_slot(it, w, i));
    asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = lds[threadIdx.x][0];
}

template <bool STORE>
__global__ __launch_bounds__(256, 1) void k_l2l_vgpr(const u32x4* src, int64_t iters, uint32_t* out) {
  __shared__ u32x4 lds[10240];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const u32x4* slab = src + (int64_t)blockIdx.x * kL2lVec;
  u32x4 v[16], sink = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = __builtin_nontemporal_load(slab + (w * 16 + i) * 64 + lane);
  for (int64_t it = 1; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (STORE) lds[l2l_slot(it, w, i) * 64 + lane] = v[i];
      else sink ^= v[i];
      v[i] = __builtin_nontemporal_load(slab + (w * 16 + i) * 64 + lane + (it & 1));
    }
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) sink ^= v[i];
  lds[4096 + threadIdx.x] = sink;
  __syncthreads();
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = lds[threadIdx.x][0] ^ lds[4096 + threadIdx.x][1];
}

}  // namespace

extern "C" {

int mlora_probe_mfma(int64_t n_wg, int64_t iters, const void* operands, float* out, void* stream) {
  if (n_wg < 1 || n_wg > (1 << 20) || iters < 1 || iters > (1 << 24) || !operands || !out ||
      (reinterpret_cast<uintptr_t>(operands) & 15u))
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(k_mfma_loop, dim3((unsigned)n_wg), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(operands), iters, out);
  return (int)hipGetLastError();
}

int mlora_probe_mfma8(int64_t n_wg, int64_t iters, const void* operands, float* out, void* stream) {
  if (n_wg < 1 || n_wg > (1 << 20) || iters < 1 || iters > (1 << 24) || !operands || !out ||
      (reinterpret_cast<uintptr_t>(operands) & 15u))
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(k_mfma8_loop, dim3((unsigned)n_wg), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(operands), iters, out);
  return (int)hipGetLastError();
}

int mlora_probe_copy(const void* src, void* dst, int64_t bytes, void* stream) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(src), b = reinterpret_cast<uintptr_t>(dst);
  if (!src || !dst || bytes <= 0 || (bytes & 15) || (a & 15u) || (b & 15u) ||
      (a < b + (uintptr_t)bytes && b < a + (uintptr_t)bytes))
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(k_copy, dim3(kStreamBlocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), bytes / 16);
  return (int)hipGetLastError();
}

int mlora_probe_read(const void* src, int64_t bytes, float* out, void* stream) {
  if (!src || !out || bytes <= 0 || (bytes & 15) || (reinterpret_cast<uintptr_t>(src) & 15u))
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(k_read, dim3(kStreamBlocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(src), bytes / 16, out);
  return (int)hipGetLastError();
}

int mlora_probe_l2_to_lds(int path, int64_t n_wg, int64_t iters, const void* src, uint32_t* out,
                          void* stream) {
  if (path < 0 || path > 2 || n_wg < 1 || n_wg > 4096 || iters < 2 || iters > (1 << 20) || !src || !out ||
      (reinterpret_cast<uintptr_t>(src) & 15u))
    return (int)hipErrorInvalidValue;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const u32x4* v = static_cast<const u32x4*>(src);
  if (path == MLORA_L2L_DIRECT) hipLaunchKernelGGL(k_l2l_direct, dim3((unsigned)n_wg), dim3(256), 0, s, v, iters, out);
  else if (path == MLORA_L2L_STAGED) hipLaunchKernelGGL(k_l2l_vgpr<true>, dim3((unsigned)n_wg), dim3(256), 0, s, v, iters, out);
  else hipLaunchKernelGGL(k_l2l_vgpr<false>, dim3((unsigned)n_wg), dim3(256), 0, s, v, iters, out);
  return (int)hipGetLastError();
}

}  // extern "C"
