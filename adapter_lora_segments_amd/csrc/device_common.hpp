// Device helpers shared by the gfx950 kernels: bf16 bit handling, the
// MFMA wrappers, and the swizzled LDS tile layout.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mlora {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

// Two fp32 values -> packed bf16 pair (lo in the low half), rounded to
// nearest, ties to even, by gfx950's v_cvt_pk_bf16_f32; NaN stays NaN.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// D[i][j] += sum_k a[i][k] b[k][j] on a 32x32x16 bf16 tile.  Lane l supplies
// row/column l%32 and eight consecutive k values starting at 8*(l/32); the
// accumulator holds D[8g + 4(l/32) + e][l%32] in element 4g+e.
__device__ __forceinline__ f32x16 mfma32(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// LDS tile: rows of 64 bf16 (eight 16-byte chunks).  Chunk c of row r lives
// at chunk position c ^ ((r ^ (r >> 3)) & 7): eight consecutive rows read at
// one chunk, and eight rows 8 apart written at one chunk, both land in eight
// distinct 16-byte bank groups.
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * 8 + (chunk ^ ((row ^ (row >> 3)) & 7));
}

// Transpose an 8x8 block of 16-bit values.  in[i] holds row i (8 values,
// value j in half j&1 of word j>>1); out[j] receives column j.
__device__ __forceinline__ void transpose8x8(const u32x4 (&in)[8], u32x4 (&out)[8]) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {     // word p of the input rows: columns 2p, 2p+1
#pragma unroll
    for (int q = 0; q < 4; ++q) {   // word q of the output: rows 2q, 2q+1
      const uint32_t lo = in[2 * q][p], hi = in[2 * q + 1][p];
      out[2 * p][q] = (lo & 0xffffu) | (hi << 16);
      out[2 * p + 1][q] = (lo >> 16) | (hi & 0xffff0000u);
    }
  }
}

__device__ __forceinline__ u32x4 ld16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ u32x4 zero4() { return u32x4{0u, 0u, 0u, 0u}; }

// Per-lane load of a plan table entry (e.g. the row permutation).
__device__ __forceinline__ int ldg_i32(const int32_t* p) { return *p; }

// Load of a value that no kernel writes while it runs (plan tables, pointer
// arrays) through the constant address space, so a wave-uniform address
// becomes a scalar load: it then waits on lgkmcnt, not on the vector-memory
// counter that tracks the direct-to-LDS pipeline.
template <class T>
__device__ __forceinline__ T ldc(const T* p) {
  return *(const __attribute__((address_space(4))) T*)p;
}

#define MLORA_LDS __attribute__((address_space(3)))

// 16 bytes per lane from global memory straight into LDS: the wave's 64 lanes
// fill the 1 KiB block at LDS byte address `lds` (wave-uniform) in lane order
// (lane i at byte 16 i), with global_load_lds_dwordx4, whose LDS base is M0.
// Inline assembly, not the compiler builtin: with the builtin the compiler
// waits for every copy in flight (vmcnt(0)) before each transposing LDS read
// (ds_read_b64_tr_b16), which would serialize the copy pipeline; the kernels'
// own vmcnt waits and barriers order the ring.  M0 is saved to a scratch
// SGPR and restored inside the statement, so the compiler's use of M0 is
// untouched (M0 is read when the load issues).  The "memory" clobber keeps
// LDS reads from being cached or moved across the copy.
__device__ __forceinline__ void dma16_at(const void* src, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(src)
      : "memory");
}

// 4 bytes per lane straight into LDS (global_load_lds_dword): the wave's 64
// lanes fill the 256-byte block at LDS byte address `lds` (wave-uniform) in
// lane order.  Same M0 handling as dma16_at.
__device__ __forceinline__ void dma4_at(const void* src, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %2, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(src)
      : "memory");
}

// The same copy into the 1 KiB block at `blk`.
__device__ __forceinline__ void dma16(const void* src, u32x4* blk) {
  dma16_at(src, __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(MLORA_LDS void*)blk));
}

// Wait until at most N direct-to-LDS loads of this wave are in flight, then
// meet the other waves.  A bare s_barrier (no fence): the loads still in
// flight target other ring stages and must not be drained here.
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  static_assert(N >= 0 && N <= 63, "vmcnt takes 0..63");
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" :: "n"(N) : "memory");
}

}  // namespace mlora
