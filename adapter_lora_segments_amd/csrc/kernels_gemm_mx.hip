// The frozen base's product on gfx950's MXFP8 matrix cores: activations
// quantized to MXFP8 (E4M3 elements, one E8M0 scale per 32 inputs along
// d_in, the OCP microscaling conversion), then Y = Q(X) W0 + Z' B with the
// base W0 held as MXFP8 codes [d_out][d_in] (k-contiguous) and its scales
// [d_out][d_in / 32], on v_mfma_scale_f32_32x32x64_f8f6f4.  The LoRA expand
// stays bf16: extra K-steps on v_mfma_f32_32x32x16_bf16 into the same
// accumulators (the expand splits the output dimension, PLoRA: Efficient
// Concurrent LoRA Training for Large Language Models, §9.2; the quantized
// base follows the page's QLoRA setting, §5 and §11.3).
#include "device_common.hpp"
#include "gemm_common.hpp"
#include "kernels.hpp"

namespace mlora {

typedef int i32x8 __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------------------
// Activations to MXFP8.  One thread per block of 32 consecutive inputs of a
// row: the block's largest magnitude gives the shared exponent
// floor(log2 amax) - 8 (8 is E4M3's largest exponent), clamped to
// [-127, 127] (-127 for a block of zeros); each element x 2^-exponent
// (exact: a power-of-two scaling) is rounded to the nearest E4M3 value,
// ties to even, and magnitudes from 448 up saturate to 448.  All decisions
// are taken on the bf16 bits and on exactly scaled fp32 values.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t e4m3_of(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fabsf(v);
  uint32_t code;
  if (a >= 448.f) {
    code = 0x7Eu;
  } else if (a < 0.015625f) {                         // below 2^-6: subnormal steps of 2^-9
    code = (uint32_t)rintf(a * 512.f);                // 8 gives 0x08, the smallest normal
  } else {
    int e = (int)((__float_as_uint(a) >> 23) & 0xFF) - 127;   // floor(log2 a), a normal fp32
    uint32_t n = (uint32_t)rintf(ldexpf(a, 3 - e));   // 8 .. 16 eighths
    if (n == 16u) {
      ++e;
      n = 8u;
    }
    code = ((uint32_t)(e + 7) << 3) | (n - 8u);
  }
  return sign | code;
}

__global__ __launch_bounds__(256) void k_quant_act_mx8(const uint16_t* X, int64_t T, int64_t K, uint8_t* codes,
                                                       uint8_t* scales) {
  const int64_t nb = K / 32;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= T * nb) return;
  const int64_t row = idx / nb, b = idx - row * nb;
  const u32x4* src = reinterpret_cast<const u32x4*>(X + row * K + 32 * b);
  u32x4 v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = src[i];
  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      amax = max(amax, v[i][j] & 0x7FFFu);
      amax = max(amax, (v[i][j] >> 16) & 0x7FFFu);
    }
  int shared = -127;
  if (amax != 0u) {
    const int ex = (int)(amax >> 7);
    const int fl = ex > 0 ? ex - 127 : -133 + (31 - __clz((int)(amax & 0x7Fu)));
    shared = min(127, max(-127, fl - 8));
  }
  scales[idx] = (uint8_t)(shared + 127);
  // input word j of vector i holds elements k = 8 i + 2 j (low half) and
  // k + 1; their codes go to bytes k % 4, k % 4 + 1 of output word k / 4
  uint32_t words[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t wv = v[i][j];
      const uint32_t lo = e4m3_of(ldexpf(__uint_as_float(wv << 16), -shared));
      const uint32_t hi = e4m3_of(ldexpf(__uint_as_float(wv & 0xFFFF0000u), -shared));
      words[2 * i + (j >> 1)] |= (lo | (hi << 8)) << (16 * (j & 1));
    }
  const u32x4 out[2] = {u32x4{words[0], words[1], words[2], words[3]}, u32x4{words[4], words[5], words[6], words[7]}};
  u32x4* dst = reinterpret_cast<u32x4*>(codes + row * K + 32 * b);
  dst[0] = out[0];
  dst[1] = out[1];
}

void launch_quant_act_mx8(const uint16_t* X, int64_t T, int64_t K, uint8_t* codes, uint8_t* scales,
                          hipStream_t s) {
  const int64_t n = T * (K / 32);
  if (n <= 0) return;
  hipLaunchKernelGGL(k_quant_act_mx8, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, X, T, K, codes, scales);
}

// ---------------------------------------------------------------------------
// Forward base GEMM on MXFP8 operands with the LoRA expand as bf16 extension
// steps.  256x256 output tile per workgroup of four waves (2x2, 128x128 of
// fp32 accumulators each), as the bf16 kernel.  A main step covers 128 of
// K: a 256-row unit of X codes and one of W0 codes, 128 bytes per row (the
// bf16 kernel's unit shape, so the same swizzle: chunk c of row r at
// c ^ kx8(r)), plus each operand's 256 scale words (4 bytes: the row's four
// 32-blocks of the step).  Two buffers of units and scale words: step s+1
// is copied while step s is computed.  An extension step is 64 bf16 deep:
// two entries of the plan's list (adapter j, rows [lo, hi), k0), as in the
// bf16 kernel.  The scale MFMA takes 64 of K: lane l = r + 32 h holds row r's
// 16-value pieces h of both 32-blocks of the slice (chunk 4 sl + h, then
// 4 sl + 2 + h) and supplies the scale of block h.
// B4: W0 as MXFP4 (E2M1 codes, two a byte along K, [N][K / 2]) on the same
// instruction with an FP4 first operand.  A main step's W0 unit is then 256
// rows of 64 bytes (chunk c of row r at c ^ ((r >> 2) & 3), which spreads a
// read group's rows over the banks), copied four per wave; measured with a
// structured probe, an FP4 operand's lane r + 32 h holds row r's whole
// 32-block h of the 64-K slice (16 bytes, the low nibble first), one 16-byte
// read, and supplies block h's scale as in the FP8 case.
// ---------------------------------------------------------------------------
template <bool PERM, bool B4>
__global__ __launch_bounds__(256, 1) void k_gemm_mx8(GemmMxArgs m) {
  const GemmArgs& g = m.g;
  constexpr int FI = 4, FJ = 4, CPW = 8;
  __shared__ u32x4 ring[4][2048];                // buffer b: X unit at 2b, W0 unit at 2b + 1
  __shared__ uint32_t scl[2][2][256];            // [buffer][operand][row]

  const TileCoord tc = tile_coord<false>(g);
  const int tm = tc.tm, tn = tc.tn;
  const int tix = g.tile_begin + tm;
  const int row0 = ldc(g.t.tiles + 2 * tix), mrows = ldc(g.t.tiles + 2 * tix + 1);
  const int n0 = tn * 256;
  const int NP = g.t.nproj;
  int pq = 0;
  while (pq + 1 < NP && ldc(g.t.pcol + pq + 1) <= n0) ++pq;
  const int e0 = ldc(g.t.ext_start + tix * NP + pq);
  const int e1 = ldc(g.t.ext_start + tix * NP + pq + 1);
  const int nk = g.K / 128;                      // main steps
  const int nsteps = nk + (e1 - e0 + 1) / 2;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, l32 = lane & 31;
  const int wrow = 128 * (w >> 1), wcol = 128 * (w & 1);
  const int64_t kb32 = g.K / 32;                 // scale words per row are 4-byte groups of these

  // Copy i of a unit: tile row 64 w + 8 i + lane / 8 into LDS position
  // lane % 8, which holds the row's chunk (lane % 8) ^ kx8(row).
  // B4: copy i (< 4) of a W0 unit: rows 64 w + 16 i + lane / 4, LDS position
  // lane % 4 holding chunk (lane % 4) ^ ((row >> 2) & 3).
  int crow[CPW], cch[CPW];
  const uint8_t* aq[CPW];
  const uint8_t* bq[CPW];
  const int64_t kbq = B4 ? g.K / 2 : g.K;        // W0 code bytes per row
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    crow[i] = 64 * w + 8 * i + (lane >> 3);
    cch[i] = (lane & 7) ^ kx8(crow[i]);
    const int ar = row0 + min(crow[i], mrows - 1);
    aq[i] = m.Aq + (int64_t)(PERM ? ldg_i32(g.t.perm + ar) : ar) * g.K + 16 * cch[i];
    if (B4) {
      const int br = 64 * w + 16 * (i & 3) + (lane >> 2);
      bq[i] = m.Bq + (int64_t)min(n0 + br, g.N - 1) * kbq + 16 * ((lane & 3) ^ ((br >> 2) & 3));
    } else {
      bq[i] = m.Bq + (int64_t)min(n0 + crow[i], g.N - 1) * kbq + 16 * cch[i];
    }
  }
  // scale words: lane -> row 64 w + lane of the tile
  const int sr = row0 + min(64 * w + lane, mrows - 1);
  const uint8_t* asc = m.Asc + (int64_t)(PERM ? ldg_i32(g.t.perm + sr) : sr) * kb32;
  const uint8_t* bsc = m.Bsc + (int64_t)min(n0 + 64 * w + lane, g.N - 1) * kb32;

  const uint32_t ring_lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(MLORA_LDS void*)&ring[0][0]);
  const uint32_t scl_lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(MLORA_LDS void*)&scl[0][0][0]);

  // Copies of step st into buffer b.
  auto issue = [&](int st, int b) {
    const uint32_t ua = ring_lds + 16u * (uint32_t)((2 * b) * 2048 + 512 * w);
    const uint32_t ub = ring_lds + 16u * (uint32_t)((2 * b + 1) * 2048 + 512 * w);
    if (st < nk) {
#pragma unroll
      for (int i = 0; i < CPW; ++i) dma16_at(aq[i] + 128 * (int64_t)st, ua + 1024u * i);
      if (B4) {
        const uint32_t ub4 = ring_lds + 16u * (uint32_t)((2 * b + 1) * 2048 + 256 * w);
#pragma unroll
        for (int i = 0; i < 4; ++i) dma16_at(bq[i] + 64 * (int64_t)st, ub4 + 1024u * i);
      } else {
#pragma unroll
        for (int i = 0; i < CPW; ++i) dma16_at(bq[i] + 128 * (int64_t)st, ub + 1024u * i);
      }
      dma4_at(asc + 4 * st, scl_lds + 4u * (uint32_t)((b * 2 + 0) * 256 + 64 * w));
      dma4_at(bsc + 4 * st, scl_lds + 4u * (uint32_t)((b * 2 + 1) * 256 + 64 * w));
      return;
    }
    // extension step: entries e0 + 2 t + h fill chunks 4 h .. 4 h + 3 (32 of K each)
    const int t = st - nk;
    int lo[2], hi[2], k0[2], rp[2];
    int64_t oj[2], ro[2];
    bool on[2];
    const uint16_t* zb[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int e = e0 + 2 * t + h;
      on[h] = e < e1;
      lo[h] = hi[h] = k0[h] = rp[h] = 0;
      oj[h] = ro[h] = 0;
      zb[h] = g.t.zero;
      if (on[h]) {
        const int j = ldc(g.t.ext + 4 * e);
        lo[h] = ldc(g.t.ext + 4 * e + 1);
        hi[h] = ldc(g.t.ext + 4 * e + 2);
        k0[h] = ldc(g.t.ext + 4 * e + 3);
        rp[h] = ldc(g.t.rpad + j);
        oj[h] = ldc(g.t.seg0 + j);
        ro[h] = ldc(g.t.roff + j);
        zb[h] = g.ebuf + ldc(g.t.zoff + j);
      }
    }
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      const int h = cch[i] >> 2, kk = 8 * (cch[i] & 3);
      const int grow = row0 + crow[i];
      const bool onh = h ? on[1] : on[0];
      const int l = h ? lo[1] : lo[0], hh = h ? hi[1] : hi[0];
      const uint16_t* sa = onh && grow >= l && grow < hh
                               ? (h ? zb[1] : zb[0]) + (int64_t)(grow - (h ? oj[1] : oj[0])) * (h ? rp[1] : rp[0]) +
                                     (h ? k0[1] : k0[0]) + kk
                               : g.t.zero;
      const uint16_t* sb = onh ? g.ext_k + (int64_t)min(n0 + crow[i], g.N - 1) * g.rtot + (h ? ro[1] : ro[0]) +
                                     (h ? k0[1] : k0[0]) + kk
                               : g.t.zero;
      dma16_at(sa, ua + 1024u * i);
      dma16_at(sb, ub + 1024u * i);
    }
  };

  f32x16 acc[FI][FJ];
#pragma unroll
  for (int a = 0; a < FI; ++a)
#pragma unroll
    for (int b = 0; b < FJ; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.f;

  // 32 bytes of row r for the scale MFMA of slice sl: chunk 4 sl + half
  // (this lane's piece of the slice's first 32-block), then 4 sl + 2 + half
  // (its piece of the second)
  auto frag8 = [&](const u32x4* unit, int r, int sl) -> i32x8 {
    const u32x4 p0 = unit[r * 8 + ((4 * sl + half) ^ kx8(r))];
    const u32x4 p1 = unit[r * 8 + ((4 * sl + 2 + half) ^ kx8(r))];
    return __builtin_bit_cast(i32x8, __builtin_shufflevector(p0, p1, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  // W0 fragment of slice sl: FP8 as above; FP4 (B4) 16 bytes of row r, chunk
  // 2 sl + half, in the first four dwords.
  auto fragb = [&](const u32x4* unit, int r, int sl) -> i32x8 {
    if constexpr (B4) {
      const u32x4 p = unit[r * 4 + ((2 * sl + half) ^ ((r >> 2) & 3))];
      return __builtin_bit_cast(i32x8, __builtin_shufflevector(p, zero4(), 0, 1, 2, 3, 4, 5, 6, 7));
    } else {
      return frag8(unit, r, sl);
    }
  };
  constexpr int FMT_B = B4 ? 4 : 0;              // first operand: E2M1 (4) or E4M3 (0)

  issue(0, 0);
  int st = 0;
  // main steps: MXFP8 x MXFP8, 128 of K each
  for (; st < nk; ++st) {
    const int b = st & 1;
    // step st has landed, and every wave is done with the other buffer
    wait_vm_barrier<0>();
    if (st + 1 < nsteps) issue(st + 1, b ^ 1);
    const u32x4* ua = ring[2 * b];
    const u32x4* ub = ring[2 * b + 1];
    int sa[FI], sb[FJ];
#pragma unroll
    for (int f = 0; f < FI; ++f) sa[f] = (int)(scl[b][0][wrow + 32 * f + l32] >> (8 * half));
#pragma unroll
    for (int f = 0; f < FJ; ++f) sb[f] = (int)(scl[b][1][wcol + 32 * f + l32] >> (8 * half));
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) {
      i32x8 fa[FI];
#pragma unroll
      for (int f = 0; f < FI; ++f) fa[f] = frag8(ua, wrow + 32 * f + l32, sl);
      i32x8 fbc = fragb(ub, wcol + l32, sl);
#pragma unroll
      for (int fj = 0; fj < FJ; ++fj) {
        const i32x8 fbn = fj + 1 < FJ ? fragb(ub, wcol + 32 * (fj + 1) + l32, sl) : fbc;
#pragma unroll
        for (int fi = 0; fi < FI; ++fi) {
          if (sl == 0)
            acc[fi][fj] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fbc, fa[fi], acc[fi][fj], FMT_B, 0, 0,
                                                                          sb[fj], 0, sa[fi]);
          else
            acc[fi][fj] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fbc, fa[fi], acc[fi][fj], FMT_B, 0, 2,
                                                                          sb[fj], 2, sa[fi]);
        }
        fbc = fbn;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // extension steps: the bf16 LoRA expand, 64 of K each
  for (; st < nsteps; ++st) {
    const int b = st & 1;
    wait_vm_barrier<0>();
    if (st + 1 < nsteps) issue(st + 1, b ^ 1);
    const u32x4* ua = ring[2 * b];
    const u32x4* ub = ring[2 * b + 1];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int c = 2 * ks + half;
      u32x4 ra[FI];
#pragma unroll
      for (int f = 0; f < FI; ++f) {
        const int r = wrow + 32 * f + l32;
        ra[f] = ua[r * 8 + (c ^ kx8(r))];
      }
#pragma unroll
      for (int fj = 0; fj < FJ; ++fj) {
        const int r = wcol + 32 * fj + l32;
        const u32x4 rb = ub[r * 8 + (c ^ kx8(r))];
#pragma unroll
        for (int fi = 0; fi < FI; ++fi) acc[fi][fj] = mfma32(rb, ra[fi], acc[fi][fj]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  __syncthreads();
  gemm_store<PERM, false>(g, acc, reinterpret_cast<char*>(&ring[0][0]), tc, row0, mrows, n0, w, lane);
}

void launch_gemm_mx8(const GemmMxArgs& m, hipStream_t s) {
  const int total = m.g.n_mtiles * m.g.n_ntiles;
  if (total <= 0) return;
  dim3 grid((unsigned)total), block(256);
  if (m.b4) {
    if (m.g.t.perm) hipLaunchKernelGGL((k_gemm_mx8<true, true>), grid, block, 0, s, m);
    else hipLaunchKernelGGL((k_gemm_mx8<false, true>), grid, block, 0, s, m);
  } else {
    if (m.g.t.perm) hipLaunchKernelGGL((k_gemm_mx8<true, false>), grid, block, 0, s, m);
    else hipLaunchKernelGGL((k_gemm_mx8<false, false>), grid, block, 0, s, m);
  }
}

}  // namespace mlora
