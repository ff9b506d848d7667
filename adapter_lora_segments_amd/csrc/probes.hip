// Ceiling probes (include/mlora_probes.h): a pure-MFMA loop in the base
// GEMM's instruction pattern, and streaming copy / read kernels.
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

}  // extern "C"
