// Decode of an MXFP8 or MXFP4 frozen base weight into bf16 for gfx950.
//
// The PLoRA page (PLoRA: Efficient Concurrent LoRA Training for Large
// Language Models, §5, §11.3) trains adapters over a frozen base that
// QLoRA-style methods keep in a low precision: the base is only read.  Here
// it is held in the OCP microscaling format MXFP8 (E4M3 elements, one E8M0
// power-of-two scale per 32 consecutive inputs of an output column) and
// decoded per call into the bf16 weight the GEMMs read: element x scale,
// rounded to nearest even.  Reads 1 + 1/32 bytes and writes 2 bytes per
// weight: HBM-bound, 16-byte vector loads and stores.  The 4-bit base of
// QLoRA (§11.3) is held as MXFP4: E2M1 elements (S.EE.M, bias 1: 0, 0.5, 1,
// 1.5, 2, 3, 4, 6), two to a byte along the layout's rows with the even
// element in the low four bits, and the same E8M0 block scales; it reads
// 0.5 + 1/32 bytes per weight.
#include "device_common.hpp"
#include "kernels.hpp"

namespace mlora {

namespace {

// Value of E4M3 code c times 2^sexp in fp32: the element is exact in fp32
// (at most four significant bits); the scaling rounds to nearest even only
// below fp32's normal range.  S.1111.111 is NaN, and so is a NaN scale.
__device__ __forceinline__ float mx_value(uint32_t c, uint32_t x) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  float v = e ? ldexpf((float)(8u + m), (int)e - 10) : ldexpf((float)m, -9);
  v = ldexpf(v, (int)x - 127);
  v = (c & 0x80u) ? -v : v;
  return ((c & 0x7Fu) == 0x7Fu || x == 255u) ? __builtin_nanf("") : v;
}

// Value of E2M1 code c (low four bits) times 2^(x - 127) in fp32: exact
// (two significant bits) except past fp32's range, which gives infinity; a
// NaN scale gives NaN.
__device__ __forceinline__ float mx4_value(uint32_t c, uint32_t x) {
  const uint32_t e = (c >> 1) & 3u, m = c & 1u;
  float v = e ? ldexpf((float)(2u + m), (int)e - 2) : 0.5f * (float)m;
  v = ldexpf(v, (int)x - 127);
  v = (c & 8u) ? -v : v;
  return x == 255u ? __builtin_nanf("") : v;
}

// 32 E2M1 codes (one 16-byte vector, element 2j in the low nibble of byte
// j) -> 32 bf16 (four 16-byte vectors); scale code per element from `xs`.
template <class XS>
__device__ __forceinline__ void decode32_e2m1(const u32x4 cw, XS xs, u32x4 (&out)[4]) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {          // word w of the codes: elements 8w .. 8w+7
    uint32_t o[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {        // byte b: elements 8w+2b (low nibble), 8w+2b+1
      const uint32_t byte = (cw[w] >> (8 * b)) & 0xFFu;
      const int i = 8 * w + 2 * b;
      o[b] = pack_bf16x2(mx4_value(byte & 15u, xs(i)), mx4_value(byte >> 4, xs(i + 1)));
    }
    out[w] = u32x4{o[0], o[1], o[2], o[3]};
  }
}

// 16 codes (one 16-byte vector) -> 16 bf16 (two 16-byte vectors); scale
// exponent code per element from `xs`.
template <class XS>
__device__ __forceinline__ void decode16(const u32x4 cw, XS xs, u32x4& lo, u32x4& hi) {
  uint32_t out[8];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int i = 4 * w + 2 * h;
      const uint32_t c0 = (cw[w] >> (16 * h)) & 0xFFu, c1 = (cw[w] >> (16 * h + 8)) & 0xFFu;
      out[2 * w + h] = pack_bf16x2(mx_value(c0, xs(i)), mx_value(c1, xs(i + 1)));
    }
  }
  lo = u32x4{out[0], out[1], out[2], out[3]};
  hi = u32x4{out[4], out[5], out[6], out[7]};
}

}  // namespace

// W0 as [d_in][d_out]: a workgroup takes one 32-row scale block kb and 512
// columns; the 512 scale codes of the block go through LDS, then each thread
// decodes 16 columns of four rows.
__global__ __launch_bounds__(256) void k_dequant_mx_kn(const uint8_t* codes, const uint8_t* scales,
                                                       int64_t d_in, int64_t d_out, uint16_t* out) {
  __shared__ uint8_t sx[512];
  const int64_t kb = blockIdx.y, n0 = (int64_t)blockIdx.x * 512;
  const int64_t nkb = d_in / 32;
  const int c16 = 16 * (threadIdx.x & 31);
  const int64_t n = n0 + c16;
  // The four rows' codes are in flight (at a clamped column past d_out)
  // while the block's scale codes are staged in LDS.
  const int64_t nc = min(n, d_out - 16);
  u32x4 cw[4];
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int64_t k = kb * 32 + (threadIdx.x >> 5) + 8 * it;
    cw[it] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(codes + k * d_out + nc));
  }
  for (int j = threadIdx.x; j < 512; j += 256)
    sx[j] = n0 + j < d_out ? scales[(n0 + j) * nkb + kb] : (uint8_t)127;
  __syncthreads();
  if (n >= d_out) return;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int64_t k = kb * 32 + (threadIdx.x >> 5) + 8 * it;
    u32x4 lo, hi;
    decode16(cw[it], [&](int i) { return (uint32_t)sx[c16 + i]; }, lo, hi);
    u32x4* dst = reinterpret_cast<u32x4*>(out + k * d_out + n);
    dst[0] = lo;
    dst[1] = hi;
  }
}

// W0 as [d_out][d_in]: a thread takes one scale block, 32 consecutive codes
// of a row.
__global__ __launch_bounds__(256) void k_dequant_mx_nk(const uint8_t* codes, const uint8_t* scales,
                                                       int64_t d_in, int64_t d_out, uint16_t* out) {
  const int64_t nkb = d_in / 32;
  const int64_t item = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (item >= d_out * nkb) return;
  const uint32_t x = scales[item];
  const int64_t off = item * 32;  // row n = item / nkb, columns 32 (item % nkb) ..
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const u32x4 cw = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(codes + off + 16 * h));
    u32x4 lo, hi;
    decode16(cw, [&](int) { return x; }, lo, hi);
    u32x4* dst = reinterpret_cast<u32x4*>(out + off + 16 * h);
    dst[0] = lo;
    dst[1] = hi;
  }
}

// MXFP4, W0 as [d_in][d_out] (codes [d_in][d_out / 2]): a workgroup takes
// one 32-row scale block kb and 512 columns; the block's 512 scale codes go
// through LDS, then each thread decodes 16 columns (8 code bytes) of four
// rows.
__global__ __launch_bounds__(256) void k_dequant_mx4_kn(const uint8_t* codes, const uint8_t* scales,
                                                        int64_t d_in, int64_t d_out, uint16_t* out) {
  __shared__ uint8_t sx[512];
  const int64_t kb = blockIdx.y, n0 = (int64_t)blockIdx.x * 512;
  const int64_t nkb = d_in / 32;
  const int c16 = 16 * (threadIdx.x & 31);
  const int64_t n = n0 + c16;
  // Codes of the four rows in flight (at a clamped column past d_out) while
  // the block's scale codes are staged in LDS.
  const int64_t nc = min(n, d_out - 16);
  u32x2 cw[4];
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int64_t k = kb * 32 + (threadIdx.x >> 5) + 8 * it;
    cw[it] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(codes + k * (d_out / 2) + nc / 2));
  }
  for (int j = threadIdx.x; j < 512; j += 256)
    sx[j] = n0 + j < d_out ? scales[(n0 + j) * nkb + kb] : (uint8_t)127;
  __syncthreads();
  if (n >= d_out) return;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int64_t k = kb * 32 + (threadIdx.x >> 5) + 8 * it;
    u32x4 v[4];
    decode32_e2m1(u32x4{cw[it][0], cw[it][1], 0u, 0u}, [&](int i) { return (uint32_t)sx[c16 + (i & 15)]; }, v);
    u32x4* dst = reinterpret_cast<u32x4*>(out + k * d_out + n);
    dst[0] = v[0];
    dst[1] = v[1];
  }
}

// MXFP4, W0 as [d_out][d_in] (codes [d_out][d_in / 2]): a thread takes one
// scale block, 32 consecutive inputs of a row in 16 code bytes.
__global__ __launch_bounds__(256) void k_dequant_mx4_nk(const uint8_t* codes, const uint8_t* scales,
                                                        int64_t d_in, int64_t d_out, uint16_t* out) {
  const int64_t nkb = d_in / 32;
  const int64_t item = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (item >= d_out * nkb) return;
  const uint32_t x = scales[item];
  const u32x4 cw = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(codes + item * 16));
  u32x4 v[4];
  decode32_e2m1(cw, [&](int) { return x; }, v);
  u32x4* dst = reinterpret_cast<u32x4*>(out + item * 32);   // row item / nkb, inputs 32 (item % nkb) ..
#pragma unroll
  for (int q = 0; q < 4; ++q) dst[q] = v[q];
}

// Transpose of a base weight (run once: the base is frozen).  A 64x64 tile
// per workgroup goes through LDS, padded one element per row so the
// transposed reads spread over the banks; reads and writes are row-major
// and coalesced.
template <class T>
__global__ __launch_bounds__(256) void k_transpose(const T* in, T* out, int64_t rows, int64_t cols) {
  __shared__ T tile[64][65];
  const int64_t r0 = (int64_t)blockIdx.y * 64, c0 = (int64_t)blockIdx.x * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < 64; i += 4) tile[i][tx] = in[(r0 + i) * cols + c0 + tx];
  __syncthreads();
  for (int i = ty; i < 64; i += 4) out[(c0 + i) * rows + r0 + tx] = tile[tx][i];
}

void launch_transpose(const void* in, void* out, int64_t rows, int64_t cols, int esz, hipStream_t s) {
  const dim3 grid((unsigned)(cols / 64), (unsigned)(rows / 64));
  if (esz == 4)
    hipLaunchKernelGGL(k_transpose<float>, grid, dim3(256), 0, s, static_cast<const float*>(in),
                       static_cast<float*>(out), rows, cols);
  else
    hipLaunchKernelGGL(k_transpose<uint16_t>, grid, dim3(256), 0, s, static_cast<const uint16_t*>(in),
                       static_cast<uint16_t*>(out), rows, cols);
}

void launch_dequant_mx4(bool nk, const uint8_t* codes, const uint8_t* scales, int64_t d_in,
                        int64_t d_out, uint16_t* out, hipStream_t s) {
  if (nk) {
    const int64_t items = d_out * (d_in / 32);
    hipLaunchKernelGGL(k_dequant_mx4_nk, dim3((unsigned)((items + 255) / 256)), dim3(256), 0, s, codes,
                       scales, d_in, d_out, out);
  } else {
    hipLaunchKernelGGL(k_dequant_mx4_kn, dim3((unsigned)((d_out + 511) / 512), (unsigned)(d_in / 32)),
                       dim3(256), 0, s, codes, scales, d_in, d_out, out);
  }
}

void launch_dequant_mx(bool nk, const uint8_t* codes, const uint8_t* scales, int64_t d_in,
                       int64_t d_out, uint16_t* out, hipStream_t s) {
  if (nk) {
    const int64_t items = d_out * (d_in / 32);
    hipLaunchKernelGGL(k_dequant_mx_nk, dim3((unsigned)((items + 255) / 256)), dim3(256), 0, s, codes,
                       scales, d_in, d_out, out);
  } else {
    hipLaunchKernelGGL(k_dequant_mx_kn, dim3((unsigned)((d_out + 511) / 512), (unsigned)(d_in / 32)),
                       dim3(256), 0, s, codes, scales, d_in, d_out, out);
  }
}

}  // namespace mlora
