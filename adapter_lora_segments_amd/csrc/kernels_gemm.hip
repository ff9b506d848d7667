// Base GEMM of the packed multi-LoRA layer for gfx950 (CDNA4): Y = X W0 with
// the LoRA expand Z' B as extra K-steps on the same accumulators (PLoRA:
// Efficient Concurrent LoRA Training for Large Language Models, §9.2: the
// expand splits the output dimension; the backward's Case 4 dZ A^T joins the
// dX GEMM the same way), bf16 operands on v_mfma_f32_32x32x16_bf16 with fp32
// accumulation.
#include "device_common.hpp"
#include "gemm_common.hpp"
#include "kernels.hpp"

#include <type_traits>

namespace mlora {

// ---------------------------------------------------------------------------
// Base GEMM with the LoRA term as extra K-steps (the expand of the forward,
// PLoRA §9.2 Case 4's dZ.A^T in the backward).  256x256 tile per workgroup of
// four waves; 64-deep K-steps copied straight from global memory into an LDS
// ring; output written as bf16, staged through LDS so every store writes
// whole 512-byte rows.
//
// LDS has 64 banks of 4 bytes.  Measured on gfx950 (read timings of many
// layouts): a 16-byte read is served in 16-lane groups that never mix the
// two half-waves and split each half-wave by the parity of lane-index bits 2
// and 4; an 8-byte transposing read in 32-lane groups.  The layouts of one
// operand of one step (32 KiB each) give every group distinct banks:
//  k-contiguous: 256 rows of 128 bytes (eight 16-byte chunks); chunk c of
//    row r sits at c ^ ((r >> 1) & 7).  In each 16-lane read group the eight
//    even rows, and the eight odd ones, take eight distinct positions, and
//    even and odd rows fill the two halves of a 256-byte bank line;
//  n-contiguous: 64 k-rows of 512 bytes (thirty-two chunks); chunk c of
//    k-row kr sits at c ^ nx(kr), nx the XOR of 4, 8 and 9 over bits 0, 1
//    and 3 of kr, so the k-rows and chunks of one transposing read group are
//    distinct.
__device__ __forceinline__ int nx(int kr) {
  return ((kr & 1) ? 4 : 0) ^ ((kr & 2) ? 8 : 0) ^ ((kr & 8) ? 9 : 0);
}
__device__ __forceinline__ int npos(int kr, int c) { return kr * 32 + (c ^ nx(kr)); }

// B fragment of a 32x32x16 MFMA from an n-contiguous tile: lane l needs
// B[k = kb + 8 (l/32) + 0..7][n = nb + l%32].  ds_read_b64_tr_b16 hands lane i
// of a 16-lane group element (i % 4) of the 8 bytes addressed by group lane
// 4e + i/4, so group lane s addresses k-row kb' + s/4, columns n' + 4 (s%4).
__device__ __forceinline__ u32x4 read_b_tr(const u32x4* tile, int nb, int kb, int lane) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  const int g = lane >> 4, s = lane & 15;
  const int n = nb + 16 * (g & 1) + 4 * (s & 3);
  const int k = kb + 8 * (g >> 1) + (s >> 2);
  u32x4 out;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int kr = k + 4 * h;
    const int byte = npos(kr, n >> 3) * 16 + 2 * (n & 7);
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (MLORA_LDS s16x4*)((MLORA_LDS char*)(MLORA_LDS void*)tile + byte));
    const u32x2 u = __builtin_bit_cast(u32x2, v);
    out[2 * h] = u[0];
    out[2 * h + 1] = u[1];
  }
  return out;
}

// 16 bytes per lane into LDS from a wave-uniform base plus a 32-bit lane
// offset (global_load_lds_dwordx4 with a scalar base): the base lives in
// SGPRs, so advancing it costs scalar adds only.  M0 as in dma16_at.
__device__ __forceinline__ uint64_t uniform64(const void* p) {
  const uint64_t b = reinterpret_cast<uint64_t>(p);
  // readfirstlane returns int: widen through uint32_t, never sign-extend
  return (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b) |
         ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32);
}
__device__ __forceinline__ void dma16_sv(uint64_t sbase, uint32_t voff, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %3\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(voff), "s"(sbase)
      : "memory");
}

// Four waves, one per SIMD, share the tile, two along M and two along N;
// each wave owns 128x128 accumulators (256 registers), so every 16-byte
// fragment read from LDS feeds four MFMAs.
//
// Steps are 64 deep so that a copy of a k-contiguous operand reads whole
// 128-byte lines (32-deep steps read half a line per row and cross the L2
// twice per line).  The 160 KiB ring holds five units of 32 KiB, one operand
// of one step each: unit u = 2 step + operand, in slot u mod 5.  While step
// s is read, step s+1 and the A unit of step s+2 are in flight.
//
// A step is two 32-deep sub-steps: the main K-steps first, then the tile's
// LoRA extension steps from the plan's list (adapter, rows, k0): sub-step e
// loads rows [lo,hi) of E_j (other rows zero) and k-rows [k0, k0+32) of
// EB_j (rows >= r_j zero).  Chunk c of a k-contiguous row belongs to
// sub-step 2s + c/4, k-row kr of an n-contiguous unit to sub-step 2s +
// kr/32; past the last sub-step copies read the zero page.
//
// Four 16-deep slices per step with fragments double buffered in
// registers; one memory instruction follows each MFMA.  Step s:
//   slices 0-1: read the next slice's fragments; copy unit 2s+4 (A of step
//     s+2) into the slot freed at the previous step's barrier;
//   slice 2: read slice 3's fragments; then wait until this wave's copies
//     of step s+1 have landed (only unit 2s+4's eight may be in flight) and
//     its reads are done, and meet the other waves: step s+1 is complete in
//     LDS and nobody reads step s's units any more;
//   slice 3: read step s+1's first slice; copy unit 2s+5 (B of step s+2)
//     into the slot of step s's A unit.
// Steps whose refills are main K-steps run a branch-free loop; the ones
// that refill LoRA steps look their sources up in the plan's tables; the
// last two, whose refills would lie past the last sub-step, copy nothing
// and wait for every copy in flight at their barrier (else every barrier
// waits for the same count: only the eight copies of unit 2s+4 in flight).
template <bool FWD, bool MAIN_B_KC, bool PERM, bool SPLIT>
__global__ __launch_bounds__(256, 1) void k_gemm(GemmArgs g) {
  constexpr int NU = 5;                    // ring units of 32 KiB
  constexpr int FI = 4, FJ = 4;            // 32x32 fragments per wave along M, N
  constexpr int CPW = 8;                   // copies per wave per unit (8 rows x 128 B each)
  __shared__ u32x4 ring[NU][2048];

  const TileCoord tc = tile_coord<SPLIT>(g);
  const int sp = tc.sp, tm = tc.tm, tn = tc.tn;
  const int tix = g.tile_begin + tm;
  const int row0 = ldc(g.t.tiles + 2 * tix), mrows = ldc(g.t.tiles + 2 * tix + 1);
  const int n0 = tn * 256;
  const int NP = g.t.nproj;
  int pq = 0;
  while (FWD && pq + 1 < NP && ldc(g.t.pcol + pq + 1) <= n0) ++pq;
  const int e0 = ldc(g.t.ext_start + tix * NP + (FWD ? pq : 0));
  const int e1 = !SPLIT || sp == g.ksplit - 1 ? ldc(g.t.ext_start + tix * NP + (FWD ? pq + 1 : NP)) : e0;
  const int pc0 = ldc(g.t.pcol + pq), pw = ldc(g.t.pcol + pq + 1) - pc0;  // forward: B_j is [r_j][pw]
  const int kb = SPLIT ? sp * g.kper : 0;         // first main 32-deep sub-step of this part
  const int nk = SPLIT ? min(g.K / 32 - kb, g.kper) : g.K / 32;
  const int nsub = nk + (e1 - e0);
  const int nsteps = (nsub + 1) >> 1;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, l32 = lane & 31;
  const int wrow = 128 * (w >> 1), wcol = 128 * (w & 1);

  // Copy i of a k-contiguous unit: tile row 64w + 8i + lane/8 into LDS
  // position lane%8, which holds the row's chunk c = (lane%8) ^ kx8(row).
  // Copy i of an n-contiguous unit: k-row 16w + 2i + lane/32 into LDS
  // position lane%32, which holds the k-row's chunk (lane%32) ^ nx(k-row).
  // Main K-steps read a wave-uniform base (the tile's first row or column at
  // the step's k) plus a fixed 32-bit lane offset (bytes), so a step only
  // advances scalar bases; with rows through the permutation table the A
  // copies keep one full pointer each.
  int crow[CPW], cch[CPW], nkr[CPW], nch[CPW];
  uint32_t aoff[CPW], boff[CPW];
  const uint16_t* aptr[CPW];
  const char* const baseA = reinterpret_cast<const char*>(g.A + (int64_t)row0 * g.lda + 32 * kb);
  const char* const baseB = reinterpret_cast<const char*>(
      MAIN_B_KC ? g.B + (int64_t)n0 * g.ldb + 32 * kb : g.B + (int64_t)(32 * kb) * g.ldb + n0);
  const int64_t strideB = MAIN_B_KC ? 128 : (int64_t)128 * g.ldb;   // bytes per 64-deep step
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    crow[i] = 64 * w + 8 * i + (lane >> 3);
    cch[i] = (lane & 7) ^ kx8(crow[i]);
    nkr[i] = 16 * w + 2 * i + (lane >> 5);
    nch[i] = (lane & 31) ^ nx(nkr[i]);
    const int ar = min(crow[i], mrows - 1);
    if constexpr (PERM)
      aptr[i] = g.A + (int64_t)ldg_i32(g.t.perm + row0 + ar) * g.lda + 32 * kb + 8 * cch[i];
    else
      aoff[i] = (uint32_t)(((int64_t)ar * g.lda + 8 * cch[i]) * 2);
    boff[i] = MAIN_B_KC ? (uint32_t)(((int64_t)(min(n0 + crow[i], g.N - 1) - n0) * g.ldb + 8 * cch[i]) * 2)
                        : (uint32_t)(((int64_t)nkr[i] * g.ldb + (min(n0 + 8 * nch[i], g.N - 8) - n0)) * 2);
  }
  // Copy i of main K-step t, operand op: its source as a pointer.
  auto main_src = [&](int t, int op, int i) -> const uint16_t* {
    if (op) return reinterpret_cast<const uint16_t*>(baseB + t * strideB + boff[i]);
    if constexpr (PERM) return aptr[i] + 64 * t;
    return reinterpret_cast<const uint16_t*>(baseA + (int64_t)t * 128 + aoff[i]);
  };

  // Sources of unit u's copies: main sub-steps at the operand's pointer plus
  // 64 k per step; extension sub-steps from the plan's list (rows outside the
  // entry's rows, and B rows past the rank, read as zero); the rest zero.
  auto unit_sources = [&](int u, const uint16_t* (&src)[CPW]) {
    const int t = u >> 1, op = u & 1;
    int kind[2], lo[2], hi[2], k0[2], rp[2], rk[2];
    int64_t oj[2], ro[2];
    const uint16_t* zb[2];
    const uint16_t* ebj[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int sub = 2 * t + h;
      kind[h] = sub < nk ? 0 : (sub < nsub ? 1 : 2);
      lo[h] = hi[h] = k0[h] = rp[h] = rk[h] = 0;
      oj[h] = ro[h] = 0;
      zb[h] = ebj[h] = g.t.zero;
      if (kind[h] == 1) {
        const int e = e0 + sub - nk;
        const int j = ldc(g.t.ext + 4 * e);
        if (FWD && !MAIN_B_KC) {
          rk[h] = ldc(g.t.ranks + j);
          ebj[h] = static_cast<const uint16_t*>(ldc(g.eb + j));
        }
        lo[h] = ldc(g.t.ext + 4 * e + 1);
        hi[h] = ldc(g.t.ext + 4 * e + 2);
        k0[h] = ldc(g.t.ext + 4 * e + 3);
        rp[h] = ldc(g.t.rpad + j);
        oj[h] = ldc(g.t.seg0 + j);
        ro[h] = ldc(g.t.roff + j);
        zb[h] = g.ebuf + ldc(g.t.zoff + j);
      }
    }
    if (op == 1 && !MAIN_B_KC) {
      // n-contiguous B: k-row nkr of the step is row nkr % 32 of sub-step
      // 2t + nkr / 32
#pragma unroll
      for (int i = 0; i < CPW; ++i) {
        const int h = nkr[i] >> 5, kr = nkr[i] & 31;
        const int kd = h ? kind[1] : kind[0];
        const int col = min(n0 + 8 * nch[i], g.N - 8);
        const int k = (h ? k0[1] : k0[0]) + kr;
        const uint16_t* ext;
        if (FWD) {
          ext = k < (h ? rk[1] : rk[0]) ? (h ? ebj[1] : ebj[0]) + (int64_t)k * pw + (col - pc0) : g.t.zero;
        } else {
          ext = g.ext_n + ((h ? ro[1] : ro[0]) + k) * g.N + col;
        }
        src[i] = kd == 0 ? main_src(t, 1, i) : (kd == 1 ? ext : g.t.zero);
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      const int h = cch[i] >> 2, kk = 8 * (cch[i] & 3);
      const int kd = h ? kind[1] : kind[0];
      const uint16_t* main = main_src(t, op, i);
      const uint16_t* ext;
      if (op == 0) {
        const int grow = row0 + crow[i];
        const int l = h ? lo[1] : lo[0], hh = h ? hi[1] : hi[0];
        ext = (grow >= l && grow < hh)
                  ? (h ? zb[1] : zb[0]) + (int64_t)(grow - (h ? oj[1] : oj[0])) * (h ? rp[1] : rp[0]) +
                        (h ? k0[1] : k0[0]) + kk
                  : g.t.zero;
      } else {
        ext = g.ext_k + (int64_t)min(n0 + crow[i], g.N - 1) * g.rtot + (h ? ro[1] : ro[0]) +
              (h ? k0[1] : k0[0]) + kk;
      }
      src[i] = kd == 0 ? main : (kd == 1 ? ext : g.t.zero);
    }
  };
  const uint32_t ring_lds = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(MLORA_LDS void*)&ring[0][0]);
  auto copy = [&](const uint16_t* src, int u, int i) {
    dma16_at(src, ring_lds + 16u * (uint32_t)((u % NU) * 2048 + 512 * w + 64 * i));
  };
  // Copy i of unit u, a main K-step.
  // Copy i of unit u, a main K-step; sbase: the operand's uniform base at
  // the unit's step (made once per unit).
  auto copy_main = [&](int u, int i, uint64_t sbase) {
    const uint32_t lds = ring_lds + 16u * (uint32_t)((u % NU) * 2048 + 512 * w + 64 * i);
    if (u & 1) dma16_sv(sbase, boff[i], lds);
    else if constexpr (PERM) dma16_at(aptr[i] + 64 * (u >> 1), lds);
    else dma16_sv(sbase, aoff[i], lds);
  };

  f32x16 acc[FI][FJ];
#pragma unroll
  for (int a = 0; a < FI; ++a)
#pragma unroll
    for (int b = 0; b < FJ; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.f;

  u32x4 fa[2][FI], fb[2][FJ];
  // LDS byte offsets of this lane's fragment reads, split into a lane part
  // and immediates.  k-contiguous: row wrow + 32 r + l32 (r: +4096 bytes),
  // chunk (2 ks + half) ^ kx8(l32), one lane part per ks.  n-contiguous
  // (transposing reads): one lane part per fragment fj, with ks (+8192) and
  // the second half of the k-rows (+2048) as immediates (nx depends only on
  // k-row bits 0, 1 and 3, which the lane fixes).
  const MLORA_LDS char* const lds0 = (const MLORA_LDS char*)(MLORA_LDS void*)&ring[0][0];
  uint32_t alane[4], blane[4];
  {
    const int kxl = kx8(l32);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      alane[ks] = (uint32_t)(((wrow + l32) * 8 + ((2 * ks + half) ^ kxl)) * 16);
      if (MAIN_B_KC) blane[ks] = (uint32_t)(((wcol + l32) * 8 + ((2 * ks + half) ^ kxl)) * 16);
    }
    if (!MAIN_B_KC) {
      const int gq = lane >> 4, sq = lane & 15;
      const int kq = 8 * (gq >> 1) + (sq >> 2);
#pragma unroll
      for (int fj = 0; fj < FJ; ++fj) {
        const int n = wcol + 32 * fj + 16 * (gq & 1) + 4 * (sq & 3);
        blane[fj] = (uint32_t)(npos(kq, n >> 3) * 16 + 2 * (n & 7));
      }
    }
  }
  // Per-step read bases: a lane part plus the step's ring slot, made once
  // per step (the empty asm keeps the compiler from folding the slot into
  // every read's address), so each read is a base plus an immediate.
  struct Bases {
    uint32_t a[4], b[4];   // A per ks; B per ks (k-contiguous) or per fragment (n-contiguous)
  };
  auto step_bases = [&](int s, Bases& bs, int ks0, int ks1) {
    const uint32_t sa = (uint32_t)((2 * s) % NU) * 32768u, sb = (uint32_t)((2 * s + 1) % NU) * 32768u;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (ks < ks0 || ks > ks1) continue;
      bs.a[ks] = alane[ks] + sa;
      asm volatile("" : "+v"(bs.a[ks]));
      if (MAIN_B_KC) {
        bs.b[ks] = blane[ks] + sb;
        asm volatile("" : "+v"(bs.b[ks]));
      }
    }
    if (!MAIN_B_KC) {
#pragma unroll
      for (int fj = 0; fj < FJ; ++fj) {
        bs.b[fj] = blane[fj] + sb;
        asm volatile("" : "+v"(bs.b[fj]));
      }
    }
  };
  // Fragment read r (0..7) of slice ks (A fragments first) from bases bs.
  auto read_frag = [&](const Bases& bs, int ks, u32x4 (&ra)[FI], u32x4 (&rb)[FJ], int r) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    if (r < FI) {
      ra[r] = *(const MLORA_LDS u32x4*)(lds0 + bs.a[ks] + 4096 * r);
    } else if (MAIN_B_KC) {
      rb[r - FI] = *(const MLORA_LDS u32x4*)(lds0 + bs.b[ks] + 4096 * (r - FI));
    } else {
      const MLORA_LDS char* p = lds0 + bs.b[r - FI] + 8192 * ks;
      const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLORA_LDS s16x4*)p);
      const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLORA_LDS s16x4*)(p + 2048));
      const u32x2 u0 = __builtin_bit_cast(u32x2, v0), u1 = __builtin_bit_cast(u32x2, v1);
      rb[r - FI] = u32x4{u0[0], u0[1], u1[0], u1[1]};
    }
  };
  auto mma = [&](const u32x4 (&ra)[FI], const u32x4 (&rb)[FJ], int qq) {
    const int fi = qq >> 2, fj = qq & 3;
    acc[fi][fj] = mfma32(rb[fj], ra[fi], acc[fi][fj]);
  };

  // Fragment reads of a slice, issued over the MFMA slots of the slice
  // before.  k-contiguous B: in the order the first MFMAs need them (A0 with
  // B0..B3 for the first four, then A1, A2, A3), two per slot in the first
  // four slots, so no MFMA waits for a read issued less than about fifteen
  // MFMAs earlier.  n-contiguous B (two transposing reads per fragment): one
  // fragment per slot in the first eight, A fragments first.
  constexpr int kOrder[FI + FJ] = {0, FI, FI + 1, FI + 2, FI + 3, 1, 2, 3};
  auto reads_at = [&](int qq, const Bases& bs, int ks, u32x4 (&ra)[FI], u32x4 (&rb)[FJ]) {
    if (MAIN_B_KC) {
      if (qq < 4) {
        read_frag(bs, ks, ra, rb, kOrder[2 * qq]);
        read_frag(bs, ks, ra, rb, kOrder[2 * qq + 1]);
      }
    } else if (qq < FI + FJ) {
      read_frag(bs, ks, ra, rb, qq);
    }
  };
  // First MFMA slot of a slice that carries a copy.
  constexpr int C0 = MAIN_B_KC ? 4 : 8;
  // Step kinds (the units a step refills are 2s+4 and 2s+5, those of step
  // s+2): 0, both are main K-steps (scalar bases, no lookups); 1, they look
  // their sources up (LoRA steps, or a mix); 2, step s+2 does not exist:
  // no copies, and the barrier waits for every copy in flight.
  auto step_block = [&](int s, auto kind_tag) {
    constexpr int KIND = decltype(kind_tag)::value;
    constexpr bool MAIN = KIND == 0, LOOKUP = KIND == 1, COPY = KIND != 2;
    const uint16_t* sa[CPW];
    if (LOOKUP) unit_sources(2 * s + 4, sa);
    Bases cur;
    step_bases(s, cur, 1, 3);
    const uint64_t cbA = MAIN && !PERM ? uniform64(baseA + (int64_t)(s + 2) * 128) : 0;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int qq = 0; qq < 16; ++qq) {
      mma(fa[0], fb[0], qq);
      reads_at(qq, cur, 1, fa[1], fb[1]);
      if (COPY && qq >= C0 && qq < C0 + 4) {
        if (MAIN) copy_main(2 * s + 4, qq - C0, cbA);
        else copy(sa[qq - C0], 2 * s + 4, qq - C0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int qq = 0; qq < 16; ++qq) {
      mma(fa[1], fb[1], qq);
      reads_at(qq, cur, 2, fa[0], fb[0]);
      if (COPY && qq >= C0 && qq < C0 + 4) {
        if (MAIN) copy_main(2 * s + 4, qq - C0 + 4, cbA);
        else copy(sa[qq - C0 + 4], 2 * s + 4, qq - C0 + 4);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int qq = 0; qq < 16; ++qq) {
      mma(fa[0], fb[0], qq);
      reads_at(qq, cur, 3, fa[1], fb[1]);
      __builtin_amdgcn_sched_barrier(0);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    wait_vm_barrier<COPY ? CPW : 0>();
    const uint16_t* sb[CPW];
    if (LOOKUP) unit_sources(2 * s + 5, sb);
    Bases nxt;
    step_bases(s + 1, nxt, 0, 0);
    const uint64_t cbB = MAIN ? uniform64(baseB + (int64_t)(s + 2) * strideB) : 0;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int qq = 0; qq < 16; ++qq) {
      mma(fa[1], fb[1], qq);
      reads_at(qq, nxt, 0, fa[0], fb[0]);
      if (COPY && qq >= C0 && qq < C0 + 8) {
        if (MAIN) copy_main(2 * s + 5, qq - C0, cbB);
        else copy(sb[qq - C0], 2 * s + 5, qq - C0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Prologue: units 0-3 (steps 0 and 1); step 0's first slice is read once
  // every wave's copies of step 0 have landed.
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const uint16_t* src[CPW];
    unit_sources(u, src);
#pragma unroll
    for (int i = 0; i < CPW; ++i) copy(src[i], u, i);
  }
  wait_vm_barrier<2 * CPW>();
  {
    Bases b0;
    step_bases(0, b0, 0, 0);
#pragma unroll
    for (int r = 0; r < FI + FJ; ++r) read_frag(b0, 0, fa[0], fb[0], r);
  }

  int s = 0;
  for (; 2 * s + 6 <= nk; ++s) step_block(s, std::integral_constant<int, 0>());
  for (; s < nsteps - 2; ++s) step_block(s, std::integral_constant<int, 1>());
  for (; s < nsteps; ++s) step_block(s, std::integral_constant<int, 2>());
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  __syncthreads();
  gemm_store<PERM, SPLIT>(g, acc, reinterpret_cast<char*>(&ring[0][0]), tc, row0, mrows, n0, w, lane);
}

// Sum of the K parts of split-K tiles, in part order, rounded to bf16 and
// stored at the caller's rows.  One workgroup per 32 rows of a tile, eight
// columns per thread.
template <bool PERM>
__global__ __launch_bounds__(256) void k_splitk_reduce(GemmArgs g) {
  const int TT = g.n_mtiles * g.n_ntiles;
  const int tile = blockIdx.x >> 3, chunk = blockIdx.x & 7;
  const int tm = tile / g.n_ntiles, tn = tile - tm * g.n_ntiles;
  const int tix = g.tile_begin + tm;
  const int row0 = ldc(g.t.tiles + 2 * tix), mrows = ldc(g.t.tiles + 2 * tix + 1);
  const int c8 = 8 * (threadIdx.x & 31);
  const int n = tn * 256 + c8;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int m = 32 * chunk + 8 * it + (threadIdx.x >> 5);
    if (m >= mrows || n >= g.N) continue;
    f32x4 lo = {0.f, 0.f, 0.f, 0.f}, hi = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < g.ksplit; ++s) {
      const float* pt = g.part + (int64_t)(s * TT + tile) * 65536 + m * 256 + c8;
      lo += *reinterpret_cast<const f32x4*>(pt);
      hi += *reinterpret_cast<const f32x4*>(pt + 4);
    }
    const u32x4 v = {pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3]), pack_bf16x2(hi[0], hi[1]),
                     pack_bf16x2(hi[2], hi[3])};
    const int cr = PERM ? ldg_i32(g.t.perm + row0 + m) : row0 + m;
    *reinterpret_cast<u32x4*>(g.C + (int64_t)cr * g.ldc + n) = v;
  }
}

void launch_gemm(bool fwd, bool main_b_kcontig, const GemmArgs& g, hipStream_t s) {
  const int total = g.n_mtiles * g.n_ntiles;
  if (total <= 0) return;
  dim3 grid((unsigned)(total * g.ksplit)), block(256);
#define MLORA_GEMM2(F, KC, SP)                                                              \
  if (g.t.perm) hipLaunchKernelGGL((k_gemm<F, KC, true, SP>), grid, block, 0, s, g);        \
  else hipLaunchKernelGGL((k_gemm<F, KC, false, SP>), grid, block, 0, s, g);
#define MLORA_GEMM(F, KC)                                                                  \
  if (g.ksplit > 1) { MLORA_GEMM2(F, KC, true) } else { MLORA_GEMM2(F, KC, false) }
  if (fwd) {
    if (main_b_kcontig) { MLORA_GEMM(true, true) } else { MLORA_GEMM(true, false) }
  } else {
    if (main_b_kcontig) { MLORA_GEMM(false, true) } else { MLORA_GEMM(false, false) }
  }
#undef MLORA_GEMM
#undef MLORA_GEMM2
  if (g.ksplit > 1) {
    const dim3 rgrid((unsigned)(total * 8));
    if (g.t.perm) hipLaunchKernelGGL(k_splitk_reduce<true>, rgrid, block, 0, s, g);
    else hipLaunchKernelGGL(k_splitk_reduce<false>, rgrid, block, 0, s, g);
  }
}

}  // namespace mlora
