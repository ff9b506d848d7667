// Host plan: the integer tables that drive every kernel of the packed
// multi-LoRA layer.  Pure C++17, no HIP call, so it is testable without a GPU.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>
#include <vector>

#include "../../include/mlora.h"

namespace mlora {

constexpr int kKStep = 32;       // K extent of one extension step
constexpr int kMinRankPad = 32;  // smallest padded rank (one MFMA tile edge)
constexpr int kOptBlock = 2048;  // elements per work item of the optimizer step
constexpr int64_t kMaxOptBlocks = int64_t(1) << 27;  // larger layers get no optimizer table

struct Opts {
  int32_t nano_rows = 0;   // 0: chosen from the rows a launch covers (auto_nano_rows)
  int32_t gemm_rows = 256;
  int32_t n_streams = 1;
  int32_t chunk_min = 256;
  int32_t chunk_max = 2048;
  int32_t chunk_per_rank = 8;
  int32_t w0_layout = MLORA_W0_KN;
  int32_t w0_format = MLORA_W0_BF16;
  int32_t act_format = MLORA_ACT_BF16;
  int32_t wg_overlap = MLORA_WG_AUTO;
  int32_t grad_accumulate = 0;
};

// Several projections that share one input (nproj > 1) split the output
// columns: projection q owns [pcol[q], pcol[q+1]).  Every (adapter i,
// projection q) pair is planned as its own unit v = i*nproj + q over adapter
// i's rows; tables indexed "per adapter" below have one entry per pair.  A
// single projection is nproj = 1 and v = i.
struct PlanTables {
  int32_t n = 0;
  int32_t nproj = 1;
  int64_t T = 0, d_in = 0, d_out = 0;
  int32_t dtype = MLORA_BF16;
  Opts opts;
  int32_t n_groups = 0;
  int64_t z_elems = 0, rpad_total = 0, partial_rows = 0, partial_b_elems = 0;

  std::vector<int64_t> offsets, zoff;
  std::vector<int32_t> ranks, rpad, roff, groups;
  std::vector<int32_t> nano, nano_start;           // nano: [n_nano][3]
  std::vector<int32_t> chunks, chunk_start, cpref; // chunks: [n_chunks][3]
  std::vector<int32_t> ch_first, ch_count;
  std::vector<int32_t> tiles, tile_start;          // tiles: [n_tiles][2]
  std::vector<int32_t> ext, ext_start;             // ext: [n_ext][4]
  std::vector<int32_t> pcol;   // [nproj+1] first output column of each projection
  std::vector<int64_t> seg0;   // [nv] first row of the pair's adapter
  std::vector<int64_t> cboff;  // [n_chunks] element offset of the chunk's dB partial
  std::vector<int32_t> ksplit;    // [S'][2] K-split of each group's forward and dX GEMM
  std::vector<int64_t> kpart_off; // [S'+1] each group's fp32 partial tiles (elements)
  std::vector<int32_t> perm;  // [T] grouped row -> caller row (plans from ids; empty otherwise)
  std::vector<int32_t> oblk;  // [n_oblk][2] optimizer work items (tensor 2i: A_i, 2i+1: B_i; piece)
  bool oblk_ok = true;        // false: the layer is too large for the optimizer table
  std::vector<int32_t> oblk_first;  // [nv+1] first optimizer work item of each pair

  int64_t n_nano() const { return (int64_t)nano.size() / 3; }
  int64_t n_chunks() const { return (int64_t)chunks.size() / 3; }
  int64_t n_tiles() const { return (int64_t)tiles.size() / 2; }
  int64_t n_ext() const { return (int64_t)ext.size() / 4; }
  int64_t n_oblk() const { return (int64_t)oblk.size() / 2; }
  int32_t nv() const { return n * nproj; }
};

// Validates and fills `out`.  On error returns the status and a message.
mlora_status build_plan(int32_t n, const int64_t* seg_offsets, const int32_t* ranks, int64_t d_in,
                        int64_t d_out, int32_t dtype, const mlora_plan_opts* opts, PlanTables& out,
                        std::string& err);

// Several projections sharing one input: widths [P], ranks [n][P].
mlora_status build_plan_multi(int32_t n, const int64_t* seg_offsets, int32_t P, const int64_t* widths,
                              const int32_t* ranks, int64_t d_in, int32_t dtype, const mlora_plan_opts* opts,
                              PlanTables& out, std::string& err);

// Rows in the caller's order with per-token adapter ids, several projections.
mlora_status build_plan_multi_from_ids(int32_t n, int64_t T, const int32_t* token_adapter, int32_t nproj,
                                       const int64_t* widths, const int32_t* ranks, int64_t d_in,
                                       int32_t dtype, const mlora_plan_opts* opts, PlanTables& out,
                                       std::string& err);

// The same for rows in the caller's order with per-token adapter ids: a
// stable counting sort by id gives the segments and the permutation.
mlora_status build_plan_from_ids(int32_t n, int64_t T, const int32_t* token_adapter,
                                 const int32_t* ranks, int64_t d_in, int64_t d_out, int32_t dtype,
                                 const mlora_plan_opts* opts, PlanTables& out, std::string& err);

// Byte layout of the device copy of the tables and of the workspace.
struct DeviceLayout {
  // offsets (bytes) of each table inside the table blob
  size_t offsets, zoff, ranks, rpad, roff, ch_first, ch_count, nano, chunks, cpref, tiles,
      ext_start, ext, zero, perm, oblk, oblk_first, seg0, pcol, cboff;
  size_t table_bytes;
  // offsets (bytes) of the work buffers inside the workspace
  size_t acat_t, acat, bcat_t, dz, kpart, w0deq, xq, gnorm, part_a, part_b;
  size_t workspace_bytes;
};

DeviceLayout device_layout(const PlanTables& p);

// Default rows per nano-batch (rule 5 of the plan): 128 when T * n_proj >=
// 65536, 64 when >= 32768, else 32.
int32_t auto_nano_rows(int64_t T, int32_t nproj);

// K-split factor of a bf16 GEMM launch (rule 9 of the plan).
int32_t split_k(int64_t tiles, int64_t nk);
std::vector<uint8_t> table_blob(const PlanTables& p, const DeviceLayout& L);

}  // namespace mlora
