// Host plan builder.  The rule is stated in include/mlora.h (mlora_plan); it
// is this library's own: the tLoRA page (tLoRA: Efficient Multi-LoRA Training
// with Elastic Shared Super-Models, abstract) asks for rank-aware nano-batches
// and per-rank low-rank tiles without fixing them, and the PLoRA page (§9.2)
// asks that work be tiled along tokens and hidden dimensions, never the rank.
#include "plan.hpp"

#include <algorithm>
#include <cstring>

namespace mlora {

namespace {

int32_t pad_rank(int32_t r) {
  int32_t p = 1;
  while (p < r) p <<= 1;
  return std::max(p, kMinRankPad);
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace

// Rule 9: a bf16 GEMM launch of `tiles` 256x256 output tiles and `nk` K
// units of 32 (the GEMM takes them two per step) splits K into S parts when
// it would fill under half the chip: S x tiles stays within one round of 256
// CUs, each part keeps at least 8 units, S <= 16, and the parts are
// ceil(nk / S) units each (S recomputed so none is empty).
int32_t auto_nano_rows(int64_t T, int32_t nproj) {
  const int64_t rows = T * nproj;
  return rows >= 65536 ? 128 : (rows >= 32768 ? 64 : 32);
}

int32_t split_k(int64_t tiles, int64_t nk) {
  if (tiles <= 0 || tiles >= 128 || nk < 16) return 1;
  int64_t sp = std::min<int64_t>({256 / tiles, nk / 8, 16});
  if (sp < 2) return 1;
  const int64_t kper = (nk + sp - 1) / sp;
  return (int32_t)((nk + kper - 1) / kper);
}

mlora_status build_plan_multi(int32_t n, const int64_t* seg_offsets, int32_t P, const int64_t* widths,
                              const int32_t* ranks, int64_t d_in, int32_t dtype, const mlora_plan_opts* opts,
                              PlanTables& P_out, std::string& err) {
  if (!seg_offsets || !ranks || !widths) {
    err = "seg_offsets, ranks and the projection widths must be non-NULL";
    return MLORA_ERR_INVALID_ARG;
  }
  if (P < 1 || P > MLORA_MAX_PROJECTIONS) {
    err = "n_proj must be in [1, " + std::to_string(MLORA_MAX_PROJECTIONS) + "], got " + std::to_string(P);
    return MLORA_ERR_INVALID_ARG;
  }
  if (n < 1 || (int64_t)n * P > MLORA_MAX_ADAPTERS) {
    err = "n must be >= 1 and n * n_proj at most " + std::to_string(MLORA_MAX_ADAPTERS) + ", got n = " +
          std::to_string(n);
    return MLORA_ERR_INVALID_ARG;
  }
  if (dtype != MLORA_FP32 && dtype != MLORA_BF16) {
    err = "unknown dtype " + std::to_string(dtype);
    return MLORA_ERR_INVALID_ARG;
  }
  int64_t d_out = 0;
  for (int32_t q = 0; q < P; ++q) {
    if (widths[q] <= 0) {
      err = "d_in and every output width must be positive";
      return MLORA_ERR_INVALID_ARG;
    }
    // bounded before the sum, so no width can overflow it
    if (widths[q] > (1 << 20)) {
      err = "every output width must be at most 2^20 (width " + std::to_string(q) + " is " +
            std::to_string(widths[q]) + ")";
      return MLORA_ERR_UNSUPPORTED;
    }
    d_out += widths[q];
  }
  if (d_in <= 0) {
    err = "d_in and d_out must be positive";
    return MLORA_ERR_INVALID_ARG;
  }
  if (d_in % 64 != 0 || d_out % 64 != 0 || d_in > (1 << 20) || d_out > (1 << 20)) {
    err = "d_in and d_out must be multiples of 64 and at most 2^20 (got " + std::to_string(d_in) +
          ", " + std::to_string(d_out) + ")";
    return MLORA_ERR_UNSUPPORTED;
  }
  // Projections split the output columns; a GEMM column tile (256 wide in
  // bf16, 64 in fp32) must lie inside one projection.
  const int64_t col_tile = dtype == MLORA_BF16 ? 256 : 64;
  if (P > 1)
    for (int32_t q = 0; q < P; ++q)
      if (widths[q] % col_tile != 0) {
        err = "with several projections every output width must be a multiple of " +
              std::to_string(col_tile) + " (width " + std::to_string(q) + " is " +
              std::to_string(widths[q]) + ")";
        return MLORA_ERR_UNSUPPORTED;
      }
  if (seg_offsets[0] != 0) {
    err = "seg_offsets[0] must be 0";
    return MLORA_ERR_INVALID_ARG;
  }
  for (int32_t i = 0; i < n; ++i) {
    if (seg_offsets[i + 1] < seg_offsets[i]) {
      err = "seg_offsets must be non-decreasing (index " + std::to_string(i + 1) + ")";
      return MLORA_ERR_INVALID_ARG;
    }
  }
  const int64_t T = seg_offsets[n];
  if (T >= (int64_t(1) << 31) - 1) {
    err = "total rows must be below 2^31 - 1";
    return MLORA_ERR_UNSUPPORTED;
  }
  const int32_t nv = n * P;
  for (int32_t v = 0; v < nv; ++v) {
    const std::string who = P == 1 ? "adapter " + std::to_string(v)
                                   : "adapter " + std::to_string(v / P) + ", projection " + std::to_string(v % P);
    if (ranks[v] < 1) {
      err = "rank of " + who + " must be >= 1";
      return MLORA_ERR_INVALID_ARG;
    }
    if (ranks[v] > MLORA_MAX_RANK) {
      err = "rank of " + who + " exceeds " + std::to_string(MLORA_MAX_RANK);
      return MLORA_ERR_UNSUPPORTED;
    }
  }
  Opts o;
  if (opts) {
    if (opts->nano_rows) o.nano_rows = opts->nano_rows;
    if (opts->gemm_rows) o.gemm_rows = opts->gemm_rows;
    if (opts->n_streams) o.n_streams = opts->n_streams;
    if (opts->chunk_min) o.chunk_min = opts->chunk_min;
    if (opts->chunk_max) o.chunk_max = opts->chunk_max;
    if (opts->chunk_per_rank) o.chunk_per_rank = opts->chunk_per_rank;
    o.w0_layout = opts->w0_layout;
    o.w0_format = opts->w0_format;
    o.act_format = opts->act_format;
    o.wg_overlap = opts->wg_overlap;
    o.grad_accumulate = opts->grad_accumulate;
  }
  if (o.nano_rows != 0 && (o.nano_rows < 16 || o.nano_rows > 256 || o.nano_rows % 16 != 0)) {
    err = "nano_rows must be a multiple of 16 in [16, 256]";
    return MLORA_ERR_INVALID_ARG;
  }
  if (o.gemm_rows < 32 || o.gemm_rows > 1024 || o.gemm_rows % 32 != 0) {
    err = "gemm_rows must be a multiple of 32 in [32, 1024]";
    return MLORA_ERR_INVALID_ARG;
  }
  if (dtype == MLORA_BF16 && o.gemm_rows != 256) {
    err = "bf16 plans use 256-row GEMM tiles (gemm_rows must be 0 or 256)";
    return MLORA_ERR_UNSUPPORTED;
  }
  if (dtype == MLORA_BF16 && o.nano_rows % 32 != 0) {
    err = "bf16 plans need nano_rows to be a multiple of 32";
    return MLORA_ERR_UNSUPPORTED;
  }
  if (o.nano_rows == 0) o.nano_rows = auto_nano_rows(T, P);

  if (o.n_streams < 1 || o.n_streams > MLORA_MAX_STREAMS) {
    err = "n_streams must be in [1, " + std::to_string(MLORA_MAX_STREAMS) + "]";
    return MLORA_ERR_INVALID_ARG;
  }
  if (o.chunk_min < 16 || o.chunk_max < o.chunk_min || o.chunk_max > (1 << 20) ||
      o.chunk_per_rank < 0 || o.chunk_per_rank > 4096) {
    err = "chunk_min/chunk_max/chunk_per_rank out of range";
    return MLORA_ERR_INVALID_ARG;
  }
  if (o.w0_layout != MLORA_W0_KN && o.w0_layout != MLORA_W0_NK && o.w0_layout != MLORA_W0_BOTH) {
    err = "w0_layout must be MLORA_W0_KN, MLORA_W0_NK or MLORA_W0_BOTH";
    return MLORA_ERR_INVALID_ARG;
  }
  if (o.w0_format != MLORA_W0_BF16 && o.w0_format != MLORA_W0_MXFP8 && o.w0_format != MLORA_W0_MXFP4) {
    err = "w0_format must be MLORA_W0_BF16, MLORA_W0_MXFP8 or MLORA_W0_MXFP4";
    return MLORA_ERR_INVALID_ARG;
  }
  if (o.w0_format != MLORA_W0_BF16 && o.w0_layout == MLORA_W0_BOTH) {
    err = "a microscaled base is held in one layout (MLORA_W0_BOTH needs a bf16/fp32 W0)";
    return MLORA_ERR_UNSUPPORTED;
  }
  if (o.w0_format != MLORA_W0_BF16 && dtype != MLORA_BF16) {
    err = "a microscaled (MXFP8/MXFP4) base weight needs a bf16 plan";
    return MLORA_ERR_UNSUPPORTED;
  }
  if (o.grad_accumulate != 0 && o.grad_accumulate != 1) {
    err = "grad_accumulate must be 0 or 1";
    return MLORA_ERR_INVALID_ARG;
  }
  if (o.wg_overlap != MLORA_WG_AUTO && o.wg_overlap != MLORA_WG_SIDE && o.wg_overlap != MLORA_WG_AFTER) {
    err = "wg_overlap must be MLORA_WG_AUTO, MLORA_WG_SIDE or MLORA_WG_AFTER";
    return MLORA_ERR_INVALID_ARG;
  }
  if (o.act_format != MLORA_ACT_BF16 && o.act_format != MLORA_ACT_MXFP8) {
    err = "act_format must be MLORA_ACT_BF16 or MLORA_ACT_MXFP8";
    return MLORA_ERR_INVALID_ARG;
  }
  if (o.act_format == MLORA_ACT_MXFP8 &&
      (o.w0_format == MLORA_W0_BF16 || o.w0_layout != MLORA_W0_NK || d_in % 128 != 0)) {
    err = "MXFP8 activations need an MXFP8 or MXFP4 base held as [d_out][d_in] (w0_layout NK) and d_in a multiple of 128";
    return MLORA_ERR_UNSUPPORTED;
  }

  PlanTables p;
  p.n = n;
  p.nproj = P;
  p.T = T;
  p.d_in = d_in;
  p.d_out = d_out;
  p.dtype = dtype;
  p.opts = o;
  p.offsets.assign(seg_offsets, seg_offsets + n + 1);
  p.ranks.assign(ranks, ranks + nv);
  p.pcol.assign(P + 1, 0);
  for (int32_t q = 0; q < P; ++q) p.pcol[q + 1] = p.pcol[q] + (int32_t)widths[q];
  auto width_of = [&](int32_t v) { return (int64_t)p.pcol[v % P + 1] - p.pcol[v % P]; };

  // 1-2: padded ranks, Z' offsets, rank offsets, first row of each
  // (adapter, projection) pair v = i*P + p
  p.rpad.resize(nv);
  p.zoff.resize(nv);
  p.roff.resize(nv);
  p.seg0.resize(nv);
  int64_t z = 0, rr = 0;
  for (int32_t v = 0; v < nv; ++v) {
    const int32_t i = v / P;
    p.rpad[v] = pad_rank(ranks[v]);
    p.zoff[v] = z;
    p.roff[v] = (int32_t)rr;
    p.seg0[v] = seg_offsets[i];
    z += (seg_offsets[i + 1] - seg_offsets[i]) * p.rpad[v];
    rr += p.rpad[v];
  }
  p.z_elems = z;
  p.rpad_total = rr;

  // 3: stream groups of consecutive adapters split near equal row counts
  const int32_t S = std::min<int32_t>(o.n_streams, n);
  p.n_groups = S;
  p.groups.assign(S + 1, 0);
  p.groups[S] = n;
  for (int32_t s = 1; s < S; ++s) {
    const int64_t target = (s * T + S - 1) / S;
    int32_t a = n;
    for (int32_t j = 0; j < n; ++j) {
      if (seg_offsets[j] >= target) {
        a = j;
        break;
      }
    }
    p.groups[s] = std::max(p.groups[s - 1], a);
  }

  // 4-6: bucket-ordered walk (padded rank descending, then projection, then
  // adapter) producing nano-batches and reduction chunks
  p.ch_first.assign(nv, 0);
  p.ch_count.assign(nv, 0);
  int64_t cp = 0, cb = 0;
  std::vector<int32_t> order;
  for (int32_t s = 0; s < S; ++s) {
    p.nano_start.push_back((int32_t)p.n_nano());
    p.chunk_start.push_back((int32_t)p.n_chunks());
    order.clear();
    for (int32_t v = p.groups[s] * P; v < p.groups[s + 1] * P; ++v) order.push_back(v);
    std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) {
      if (p.rpad[a] != p.rpad[b]) return p.rpad[a] > p.rpad[b];
      if (a % P != b % P) return a % P < b % P;
      return a < b;
    });
    for (int32_t v : order) {
      const int64_t lo = seg_offsets[v / P], hi = seg_offsets[v / P + 1];
      for (int64_t r0 = lo; r0 < hi; r0 += o.nano_rows) {
        p.nano.push_back(v);
        p.nano.push_back((int32_t)r0);
        p.nano.push_back((int32_t)std::min<int64_t>(o.nano_rows, hi - r0));
      }
      const int64_t kc = std::min<int64_t>(
          o.chunk_max, std::max<int64_t>(o.chunk_min, (int64_t)o.chunk_per_rank * p.rpad[v]));
      p.ch_first[v] = (int32_t)p.n_chunks();
      for (int64_t r0 = lo; r0 < hi; r0 += kc) {
        p.chunks.push_back(v);
        p.chunks.push_back((int32_t)r0);
        p.chunks.push_back((int32_t)std::min<int64_t>(kc, hi - r0));
        p.cpref.push_back((int32_t)cp);
        p.cboff.push_back(cb);
        cp += p.rpad[v];
        cb += p.rpad[v] * width_of(v);
        p.ch_count[v] += 1;
      }
    }
  }
  p.nano_start.push_back((int32_t)p.n_nano());
  p.chunk_start.push_back((int32_t)p.n_chunks());
  p.partial_rows = cp;
  p.partial_b_elems = cb;

  // 7: GEMM row tiles of BM rows from row 0; group s's GEMMs take tiles
  // [a_s, a_s+1), each boundary the largest multiple of G tiles that still
  // ends at or before the group's first row (so a group's GEMM holds rows of
  // its own and earlier groups only, whose shrink or dZ has run).  G = 16
  // when every group can average two such units: a launch then covers whole
  // rounds of 256 output tiles for any output width that is a multiple of
  // 4096, with no partial row tile at a group boundary.  Each tile lists its
  // extension steps per projection (the forward's column tiles take their
  // own projection's list, the dX GEMM takes all of them).
  const int64_t BM = o.gemm_rows;
  const int64_t ntile = (T + BM - 1) / BM;
  const int64_t G = ntile >= 32 * (int64_t)S ? 16 : 1;
  std::vector<int64_t> bound(S + 1, 0);
  bound[S] = ntile;
  for (int32_t s = 1; s < S; ++s)
    bound[s] = std::max(bound[s - 1], seg_offsets[p.groups[s]] / BM / G * G);
  int32_t first = 0;  // first adapter that can still meet a tile
  for (int32_t s = 0; s < S; ++s) {
    p.tile_start.push_back((int32_t)p.n_tiles());
    for (int64_t tt = bound[s]; tt < bound[s + 1]; ++tt) {
      const int64_t t0 = tt * BM, rows = std::min<int64_t>(BM, T - t0);
      while (first < n && seg_offsets[first + 1] <= t0) ++first;
      for (int32_t q = 0; q < P; ++q) {
        p.ext_start.push_back((int32_t)p.n_ext());
        for (int32_t j = first; j < n && seg_offsets[j] < t0 + rows; ++j) {
          const int64_t lo = std::max<int64_t>(seg_offsets[j], t0);
          const int64_t hi = std::min<int64_t>(seg_offsets[j + 1], t0 + rows);
          if (lo >= hi) continue;
          const int32_t v = j * P + q;
          for (int32_t k0 = 0; k0 < p.rpad[v]; k0 += kKStep) {
            p.ext.push_back(v);
            p.ext.push_back((int32_t)lo);
            p.ext.push_back((int32_t)hi);
            p.ext.push_back(k0);
          }
        }
      }
      p.tiles.push_back((int32_t)t0);
      p.tiles.push_back((int32_t)rows);
    }
  }
  p.tile_start.push_back((int32_t)p.n_tiles());
  p.ext_start.push_back((int32_t)p.n_ext());

  // 9: split-K of each group's forward and dX GEMM (bf16), and each group's
  // region of fp32 partial tiles (groups run concurrently; a group's two
  // GEMMs never do)
  p.ksplit.assign(2 * S, 1);
  p.kpart_off.assign(S + 1, 0);
  for (int32_t s = 0; s < S; ++s) {
    const int64_t nm = p.tile_start[s + 1] - p.tile_start[s];
    const int64_t tf = nm * ((d_out + 255) / 256), td = nm * ((d_in + 255) / 256);
    if (dtype == MLORA_BF16) {
      p.ksplit[2 * s] = split_k(tf, d_in / kKStep);
      p.ksplit[2 * s + 1] = split_k(td, d_out / kKStep);
    }
    const int64_t need = std::max(p.ksplit[2 * s] > 1 ? p.ksplit[2 * s] * tf : 0,
                                  p.ksplit[2 * s + 1] > 1 ? p.ksplit[2 * s + 1] * td : 0);
    p.kpart_off[s + 1] = p.kpart_off[s] + need * 65536;
  }

  // 8: optimizer work items, A_v then B_v of every pair in pieces of
  // kOptBlock elements
  int64_t nob = 0;
  for (int32_t v = 0; v < nv; ++v)
    nob += (d_in * ranks[v] + kOptBlock - 1) / kOptBlock + (ranks[v] * width_of(v) + kOptBlock - 1) / kOptBlock;
  p.oblk_ok = nob <= kMaxOptBlocks;
  if (p.oblk_ok) {
    p.oblk.reserve((size_t)(2 * nob));
    p.oblk_first.reserve((size_t)nv + 1);
    for (int32_t v = 0; v < nv; ++v) {
      p.oblk_first.push_back((int32_t)p.n_oblk());
      const int64_t numel[2] = {d_in * ranks[v], ranks[v] * width_of(v)};
      for (int w = 0; w < 2; ++w)
        for (int64_t q = 0; q * kOptBlock < numel[w]; ++q) {
          p.oblk.push_back(2 * v + w);
          p.oblk.push_back((int32_t)q);
        }
    }
    p.oblk_first.push_back((int32_t)p.n_oblk());
  }

  P_out = std::move(p);
  return MLORA_OK;
}

mlora_status build_plan(int32_t n, const int64_t* seg_offsets, const int32_t* ranks, int64_t d_in,
                        int64_t d_out, int32_t dtype, const mlora_plan_opts* opts, PlanTables& P,
                        std::string& err) {
  return build_plan_multi(n, seg_offsets, 1, &d_out, ranks, d_in, dtype, opts, P, err);
}

mlora_status build_plan_multi_from_ids(int32_t n, int64_t T, const int32_t* token_adapter, int32_t nproj,
                                       const int64_t* widths, const int32_t* ranks, int64_t d_in,
                                       int32_t dtype, const mlora_plan_opts* opts, PlanTables& P,
                                       std::string& err) {
  if (n < 1 || n > MLORA_MAX_ADAPTERS) {
    err = "n must be in [1, " + std::to_string(MLORA_MAX_ADAPTERS) + "], got " + std::to_string(n);
    return MLORA_ERR_INVALID_ARG;
  }
  if (T < 0) {
    err = "T must be >= 0";
    return MLORA_ERR_INVALID_ARG;
  }
  if (T > 0 && !token_adapter) {
    err = "token_adapter must be non-NULL";
    return MLORA_ERR_INVALID_ARG;
  }
  if (T >= (int64_t(1) << 31) - 1) {
    err = "total rows must be below 2^31 - 1";
    return MLORA_ERR_UNSUPPORTED;
  }
  // stable counting sort: counts, exclusive prefix sums, placement in row order
  std::vector<int64_t> off(n + 1, 0);
  for (int64_t t = 0; t < T; ++t) {
    const int32_t a = token_adapter[t];
    if (a < 0 || a >= n) {
      err = "token_adapter[" + std::to_string(t) + "] = " + std::to_string(a) + " is not in [0, n)";
      return MLORA_ERR_INVALID_ARG;
    }
    off[a + 1] += 1;
  }
  for (int32_t a = 0; a < n; ++a) off[a + 1] += off[a];
  std::vector<int32_t> perm((size_t)T);
  std::vector<int64_t> next(off.begin(), off.end() - 1);
  for (int64_t t = 0; t < T; ++t) perm[(size_t)next[token_adapter[t]]++] = (int32_t)t;
  mlora_status st = build_plan_multi(n, off.data(), nproj, widths, ranks, d_in, dtype, opts, P, err);
  if (st != MLORA_OK) return st;
  P.perm = std::move(perm);
  return MLORA_OK;
}

mlora_status build_plan_from_ids(int32_t n, int64_t T, const int32_t* token_adapter,
                                 const int32_t* ranks, int64_t d_in, int64_t d_out, int32_t dtype,
                                 const mlora_plan_opts* opts, PlanTables& P, std::string& err) {
  return build_plan_multi_from_ids(n, T, token_adapter, 1, &d_out, ranks, d_in, dtype, opts, P, err);
}

DeviceLayout device_layout(const PlanTables& p) {
  DeviceLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off = align_up(off + std::max<size_t>(bytes, 1), 256);
    return at;
  };
  const size_t n = (size_t)p.n, nv = (size_t)p.nv();
  L.offsets = take(8 * (n + 1));
  L.zoff = take(8 * nv);
  L.ranks = take(4 * nv);
  L.rpad = take(4 * nv);
  L.roff = take(4 * nv);
  L.ch_first = take(4 * nv);
  L.ch_count = take(4 * nv);
  L.nano = take(4 * p.nano.size());
  L.chunks = take(4 * p.chunks.size());
  L.cpref = take(4 * p.cpref.size());
  L.tiles = take(4 * p.tiles.size());
  L.ext_start = take(4 * p.ext_start.size());
  L.ext = take(4 * p.ext.size());
  L.perm = take(4 * p.perm.size());
  L.oblk = take(4 * p.oblk.size());
  L.oblk_first = take(4 * p.oblk_first.size());
  L.seg0 = take(8 * p.seg0.size());
  L.pcol = take(4 * p.pcol.size());
  L.cboff = take(8 * p.cboff.size());
  L.zero = take(256);  // a zero page: loads of rows that must read as zero point here
  L.table_bytes = off;
  const size_t esz = p.dtype == MLORA_BF16 ? 2 : 4;
  if (p.dtype == MLORA_BF16) {
    L.acat_t = take((size_t)p.rpad_total * (size_t)p.d_in * esz);
    L.acat = take((size_t)p.rpad_total * (size_t)p.d_in * esz);
    L.bcat_t = take((size_t)p.rpad_total * (size_t)p.d_out * esz);
  } else {
    L.acat_t = L.acat = L.bcat_t = off;
  }
  L.dz = take((size_t)p.z_elems * esz);
  L.kpart = take((size_t)p.kpart_off.back() * 4);
  L.w0deq = take(p.opts.w0_format != MLORA_W0_BF16 ? (size_t)p.d_in * (size_t)p.d_out * 2 : 0);
  // MXFP8 activations: E4M3 codes [T][d_in], then E8M0 scales [T][d_in / 32]
  L.xq = take(p.opts.act_format == MLORA_ACT_MXFP8 ? (size_t)p.T * (size_t)p.d_in * 33 / 32 : 0);
  // gradient clipping: one partial square sum per optimizer work item, then
  // one clip factor per pair
  L.gnorm = take(4 * ((size_t)p.n_oblk() + (size_t)p.nv()));
  if (p.dtype == MLORA_BF16) {
    L.part_a = take((size_t)p.partial_rows * (size_t)p.d_in * 4);
    L.part_b = take((size_t)p.partial_b_elems * 4);
  } else {
    L.part_a = L.part_b = off;
  }
  L.workspace_bytes = off;
  return L;
}

std::vector<uint8_t> table_blob(const PlanTables& p, const DeviceLayout& L) {
  std::vector<uint8_t> b(L.table_bytes, 0);
  auto put = [&](size_t at, const void* src, size_t bytes) {
    if (bytes) std::memcpy(b.data() + at, src, bytes);
  };
  put(L.offsets, p.offsets.data(), 8 * p.offsets.size());
  put(L.zoff, p.zoff.data(), 8 * p.zoff.size());
  put(L.ranks, p.ranks.data(), 4 * p.ranks.size());
  put(L.rpad, p.rpad.data(), 4 * p.rpad.size());
  put(L.roff, p.roff.data(), 4 * p.roff.size());
  put(L.ch_first, p.ch_first.data(), 4 * p.ch_first.size());
  put(L.ch_count, p.ch_count.data(), 4 * p.ch_count.size());
  put(L.nano, p.nano.data(), 4 * p.nano.size());
  put(L.chunks, p.chunks.data(), 4 * p.chunks.size());
  put(L.cpref, p.cpref.data(), 4 * p.cpref.size());
  put(L.tiles, p.tiles.data(), 4 * p.tiles.size());
  put(L.ext_start, p.ext_start.data(), 4 * p.ext_start.size());
  put(L.ext, p.ext.data(), 4 * p.ext.size());
  put(L.perm, p.perm.data(), 4 * p.perm.size());
  put(L.oblk, p.oblk.data(), 4 * p.oblk.size());
  put(L.oblk_first, p.oblk_first.data(), 4 * p.oblk_first.size());
  put(L.seg0, p.seg0.data(), 8 * p.seg0.size());
  put(L.pcol, p.pcol.data(), 4 * p.pcol.size());
  put(L.cboff, p.cboff.data(), 8 * p.cboff.size());
  return b;
}

}  // namespace mlora
