// Launch interface of the device kernels (host side).  Every launcher checks
// nothing itself: the C interface validates shapes and sizes before calling.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mlora.h"

namespace mlora {

// Device copies of the plan tables (pointers into the workspace).
struct DevTables {
  const int64_t* offsets;   // [n+1]
  const int64_t* zoff;      // [n]
  const int32_t* ranks;     // [n]
  const int32_t* rpad;      // [n]
  const int32_t* roff;      // [n]
  const int32_t* ch_first;  // [n]
  const int32_t* ch_count;  // [n]
  const int32_t* nano;      // [n_nano][3]
  const int32_t* chunks;    // [n_chunks][3]
  const int32_t* cpref;     // [n_chunks]
  const int32_t* tiles;     // [n_tiles][2]
  const int32_t* ext_start; // [n_tiles+1]
  const int32_t* ext;       // [n_ext][4]
  const uint16_t* zero;     // 256 zero bytes
  const int32_t* perm;      // [T] grouped row -> caller row, or NULL (rows already grouped)
  const int32_t* oblk;      // [n_oblk][2] optimizer work items (tensor, piece)
  const int32_t* oblk_first;  // [nv+1] first optimizer work item of each pair
  // Several projections sharing the input: "adapter" j in the tables above
  // is the pair (j / nproj, j % nproj); projection q owns output columns
  // [pcol[q], pcol[q+1]).
  const int64_t* seg0;      // [nv] first row of pair j's adapter
  const int32_t* pcol;      // [nproj+1]
  const int64_t* cboff;     // [n_chunks] element offset of a chunk's dB partial
  int32_t nproj;
  int32_t accumulate;       // 1: the backward adds to dA_i, dB_i; 0: it overwrites them
};

// ---------------- bf16 path (MFMA) ----------------

// Rank-padded concatenations (zero for r_j <= c < r_pad(j)):
//   A_cat^T [rtot][d_in] (row roff(j)+c = column c of A_j), A_cat [d_in][rtot],
//   B_cat^T [d_out][rtot] (column roff(j)+c = row c of B_j).  NULL skips an output.
void launch_prep_a(const DevTables& t, int32_t n, int64_t d_in, int64_t rtot, const void* const* A,
                   uint16_t* acat_t, uint16_t* acat, hipStream_t s);
void launch_prep_b(const DevTables& t, int32_t n, int64_t d_out, int64_t rtot,
                   const void* const* B, uint16_t* bcat_t, hipStream_t s);
// Both in one launch; any output NULL is skipped.
void launch_prep(const DevTables& t, int32_t n, int64_t d_in, int64_t d_out, int64_t rtot,
                 const void* const* A, uint16_t* acat_t, uint16_t* acat, const void* const* B,
                 uint16_t* bcat_t, hipStream_t s);

// Skinny products over nano-batches [nano_begin, nano_begin + nano_count) of
// any padded ranks: out rows of adapter j (r_pad(j) columns)
//   mode 0 (shrink): Z'[t][c] = s_j sum_k X[t][k] A_cat^T[roff_j + c][k]
//   mode 1 (dZ)    : dZ[t][c] = s_j sum_k dY[t][c_j + k] B_j[c][k] over the
//                    width of j's projection (first column c_j); K is then
//                    the row length of dY
void launch_skinny(int mode, const DevTables& t, int32_t nano_begin, int32_t nano_count,
                   const uint16_t* P, int64_t K, const uint16_t* acat_t, const void* const* Bptr,
                   const float* scales, uint16_t* out, hipStream_t s);

// Token reductions over the chunks [chunk_begin, chunk_begin + chunk_count)
// of one padded-rank bucket (r_pad = rp) and one projection, both in one
// launch; partial sums in fp32:
//   dB: partB[cboff + c*d_out + n] = sum_t Z'[t][c] dY[t][n]   (n < d_out)
//   dA: partA[cpref][d][c] = sum_t X[t][d] dZ[t][c]            (d < d_in)
// dY points at the projection's first column, rows ld_dy apart; d_out is the
// projection's width.  With rows grouped by adapter (no permutation table),
// an adapter with a single chunk writes its fp32 dA_j [d_in][r_j] and dB_j
// [r_j][d_out] (pointer arrays dA, dB) directly instead of a partial.
void launch_token_reduce(int rp, const DevTables& t, int32_t chunk_begin, int32_t chunk_count,
                         const uint16_t* dY, int64_t ld_dy, const uint16_t* Z, float* partB,
                         int64_t d_out, const uint16_t* X, const uint16_t* dZ, float* partA,
                         int64_t d_in, void* const* dA, void* const* dB, hipStream_t s);

// Fixed-order sum of the chunk partials into the caller's dA_j / dB_j
// (adapters [a_begin, a_end)); adapters without rows get zeros; with rows
// grouped by adapter, single-chunk adapters are skipped (the token
// reductions wrote them).
void launch_reduce_partials(const DevTables& t, int32_t a_begin, int32_t a_end, int64_t d_in,
                            int64_t d_out, const float* partA, const float* partB,
                            void* const* dA, void* const* dB, int32_t max_rank, hipStream_t s);

// C[row][n] = sum_k Aop[row][k] Bop[k][n] over K, then the extension steps of
// each row tile: rows of adapter j times E_j (Z' or dZ) against EB_j, read in
// the same layout as the main B operand:
//   fwd: Aop = X, Bop = W0, E = Z', EB_j = B_j: n-contiguous from B_j itself,
//        k-contiguous from B_cat^T
//   dx : Aop = dY, Bop = W0^T, E = dZ, EB_j = A_j^T: n-contiguous from rows
//        roff_j.. of A_cat^T, k-contiguous from A_cat
struct GemmArgs {
  const uint16_t* A;
  int64_t lda;
  const uint16_t* B;
  int64_t ldb;
  uint16_t* C;
  int64_t ldc;
  int32_t K, N;
  int32_t tile_begin, n_mtiles, n_ntiles;
  const uint16_t* ebuf;     // Z' (fwd) or dZ (dx), plan layout
  const void* const* eb;    // fwd, n-contiguous: B_j pointers
  const uint16_t* ext_n;    // dx, n-contiguous: A_cat^T [rtot][N]
  const uint16_t* ext_k;    // k-contiguous: [N][rtot] (B_cat^T fwd, A_cat dx)
  int64_t rtot;             // sum of padded ranks
  // Split-K: ksplit > 1 runs ksplit workgroups per output tile, part s
  // taking main K-steps [s*kper, (s+1)*kper) (the last part also the
  // extension steps), each writing a 256x256 fp32 partial tile to
  // part[(s * n_mtiles*n_ntiles + tile)]; a second kernel adds the parts in
  // order and stores C.
  int32_t ksplit, kper;
  float* part;
  DevTables t;
};
// Forward GEMM over microscaled operands (kernels_gemm_mx.hip): g as for
// launch_gemm(true, true, ...) without split-K; the main operands are X's
// E4M3 codes [rows][K] with scales [rows][K / 32] (rows in the caller's
// order) and W0's codes [N][K] (b4: E2M1, [N][K / 2], two a byte, the even
// element low) with scales [N][K / 32]; K a multiple of 128.
struct GemmMxArgs {
  GemmArgs g;
  const uint8_t* Aq;
  const uint8_t* Asc;
  const uint8_t* Bq;
  const uint8_t* Bsc;
  int32_t b4;
};
void launch_gemm_mx8(const GemmMxArgs& m, hipStream_t s);
// Activations [T][K] (bf16, rows dense) to MXFP8 codes [T][K] and scales [T][K / 32].
void launch_quant_act_mx8(const uint16_t* X, int64_t T, int64_t K, uint8_t* codes, uint8_t* scales,
                          hipStream_t s);

// main_b_kcontig: Bop element (k, n) at B[n*ldb + k] (else at B[k*ldb + n]).
void launch_gemm(bool fwd, bool main_b_kcontig, const GemmArgs& g, hipStream_t s);

// out[c][r] = in[r][c], rows x cols elements of `esz` bytes (2 or 4); rows
// and cols multiples of 64.
void launch_transpose(const void* in, void* out, int64_t rows, int64_t cols, int esz, hipStream_t s);

// MXFP8 base weight -> bf16, same layout: codes [d_in][d_out] (nk: [d_out]
// [d_in]) E4M3, scales [d_out][d_in / 32] E8M0; out = element x scale,
// nearest-even bf16.
void launch_dequant_mx(bool nk, const uint8_t* codes, const uint8_t* scales, int64_t d_in,
                       int64_t d_out, uint16_t* out, hipStream_t s);
// MXFP4 base weight -> bf16: codes [d_in][d_out / 2] (nk: [d_out][d_in / 2])
// E2M1, two per byte along the row (even element low), scales as above.
void launch_dequant_mx4(bool nk, const uint8_t* codes, const uint8_t* scales, int64_t d_in,
                        int64_t d_out, uint16_t* out, hipStream_t s);

// ---------------- fp32 path (vector ALU) ----------------
void launch_f32_shrink(const DevTables& t, int32_t n, int64_t T, int64_t d_in, const float* X,
                       const void* const* A, const float* scales, float* Z, hipStream_t s);
void launch_f32_dz(const DevTables& t, int32_t n, int64_t T, int64_t d_out, const float* dY,
                   const void* const* B, const float* scales, float* dZ, hipStream_t s);
// fwd: Y = X W0 + Z' B; dx: dX = dY W0^T + dZ A^T.
void launch_f32_gemm(bool fwd, bool main_b_kcontig, const DevTables& t, int32_t n, int64_t T,
                     const float* A, int64_t lda, const float* B, int64_t ldb, float* C,
                     int64_t ldc, int32_t K, int32_t N, const float* E, const void* const* eb,
                     hipStream_t s);
void launch_f32_db(const DevTables& t, int32_t n, int64_t d_out, const float* Z, const float* dY,
                   void* const* dB, int32_t max_rank, hipStream_t s);
void launch_f32_da(const DevTables& t, int32_t n, int64_t d_in, const float* X, const float* dZ,
                   void* const* dA, int32_t max_rank, hipStream_t s);

// ---------------- optimizer step ----------------

constexpr int kOptBlockElems = 2048;  // elements per optimizer work item (the plan's piece size)

// One AdamW update of every adapter's fp32 A_i and B_i with its own
// hyperparameters (work items [0, n_blocks) of the plan's optimizer table);
// A_copy/B_copy (bf16, or NULL arrays) receive the updated values rounded to
// nearest even.
struct AdamwArgs {
  DevTables t;
  const mlora_adamw_hparams* hp;  // [n]
  int64_t d_in, d_out;
  float* const* A;
  float* const* B;
  const float* const* dA;
  const float* const* dB;
  float* const* mA;
  float* const* vA;
  float* const* mB;
  float* const* vB;
  uint16_t* const* A_copy;
  uint16_t* const* B_copy;
  float* gsq;        // [n_blocks] partial square sums of the gradients (clipping)
  float* coef;       // [nv] clip factor per pair, or NULL (no clipping)
};
// The update; with a.coef set, each pair's gradients are scaled by its clip
// factor first.
// ---------------- static scratch of the allocation-free forward ----------------
// A file-scope device array (scratch.hip) of this many bytes per GPU, held
// until the process ends.
constexpr size_t kNoallocScratchBytes = size_t(64) << 20;
// Device address of the current device's copy (looked up with
// hipGetSymbolAddress once per device, then cached); *dev receives the
// device index.  hipErrorInvalidDevice for an index beyond the cache.
hipError_t noalloc_scratch(void** out, int* dev);

void launch_adamw(const AdamwArgs& a, int64_t n_blocks, hipStream_t s);
// Clip factors into a.coef: per work item the gradients' square sum (into
// a.gsq), then per pair the sum of its items in order (two launches).
void launch_grad_norm(const AdamwArgs& a, int64_t n_blocks, int32_t nv, hipStream_t s);

}  // namespace mlora
