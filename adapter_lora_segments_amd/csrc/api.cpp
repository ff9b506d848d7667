// C interface (include/mlora.h): argument checks, the plan object, launch
// orchestration over adapter groups and streams, and per-kernel timing.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "../../include/mlora.h"
#include "kernels.hpp"
#include "plan.hpp"

static_assert(mlora::kOptBlockElems == mlora::kOptBlock, "optimizer piece size differs");

namespace {

thread_local std::string g_err;

mlora_status fail(mlora_status s, const std::string& msg) {
  g_err = msg;
  return s;
}

struct Range {
  int32_t begin, count, rp, proj;
};

}  // namespace

struct mlora_plan_s {
  mlora::PlanTables P;
  mlora::DeviceLayout L;
  std::vector<uint8_t> blob;
  void* uploaded_ws = nullptr;
  std::vector<std::vector<Range>> chunk_b;  // per group: one chunk range per padded rank
  std::vector<int32_t> group_max_rank;
  int32_t max_rank = 1;
  // One stream group: the backward's weight gradients run beside the dX GEMM
  // on the side stream (wg_overlap resolved), else after it.
  bool wg_side = true;
  // The side stream: with one stream group, the backward's weight-gradient
  // branch (beside the dX GEMM); with several, every group's HBM-bound LoRA
  // work (shrink; dZ and the weight gradients), one group ahead of the base
  // GEMMs on the caller's stream.  Created on first use.  Events: fork_ev
  // (caller -> side), group_ev[g] (side -> caller: group g's shrink or dZ is
  // done), done_ev (side -> caller: the weight gradients are done).
  hipStream_t side = nullptr;
  hipEvent_t fork_ev = nullptr, done_ev = nullptr;
  std::vector<hipEvent_t> group_ev;
  // profiling
  uint32_t prof = 0;  // bit k: bracket launches of kernel kind k
  struct Rec {
    int kind;
    hipEvent_t a, b;
  };
  std::vector<Rec> recs;
  std::vector<hipEvent_t> pool;
};

namespace {

// Runs of consecutive items (chunks) with the same padded rank and projection.
std::vector<Range> bucket_ranges(const std::vector<int32_t>& items, int stride, int32_t begin,
                                 int32_t end, const std::vector<int32_t>& rpad, int32_t nproj) {
  std::vector<Range> out;
  for (int32_t i = begin; i < end; ++i) {
    const int32_t v = items[(size_t)stride * i];
    const int32_t rp = rpad[v], q = v % nproj;
    if (out.empty() || out.back().rp != rp || out.back().proj != q) out.push_back({i, 0, rp, q});
    out.back().count++;
  }
  return out;
}

mlora::DevTables dev_tables(const mlora_plan_s* p, void* ws) {
  const uint8_t* b = static_cast<const uint8_t*>(ws);
  const auto& L = p->L;
  mlora::DevTables t;
  t.offsets = reinterpret_cast<const int64_t*>(b + L.offsets);
  t.zoff = reinterpret_cast<const int64_t*>(b + L.zoff);
  t.ranks = reinterpret_cast<const int32_t*>(b + L.ranks);
  t.rpad = reinterpret_cast<const int32_t*>(b + L.rpad);
  t.roff = reinterpret_cast<const int32_t*>(b + L.roff);
  t.ch_first = reinterpret_cast<const int32_t*>(b + L.ch_first);
  t.ch_count = reinterpret_cast<const int32_t*>(b + L.ch_count);
  t.nano = reinterpret_cast<const int32_t*>(b + L.nano);
  t.chunks = reinterpret_cast<const int32_t*>(b + L.chunks);
  t.cpref = reinterpret_cast<const int32_t*>(b + L.cpref);
  t.tiles = reinterpret_cast<const int32_t*>(b + L.tiles);
  t.ext_start = reinterpret_cast<const int32_t*>(b + L.ext_start);
  t.ext = reinterpret_cast<const int32_t*>(b + L.ext);
  t.zero = reinterpret_cast<const uint16_t*>(b + L.zero);
  t.perm = p->P.perm.empty() ? nullptr : reinterpret_cast<const int32_t*>(b + L.perm);
  t.oblk = reinterpret_cast<const int32_t*>(b + L.oblk);
  t.oblk_first = reinterpret_cast<const int32_t*>(b + L.oblk_first);
  t.seg0 = reinterpret_cast<const int64_t*>(b + L.seg0);
  t.pcol = reinterpret_cast<const int32_t*>(b + L.pcol);
  t.cboff = reinterpret_cast<const int64_t*>(b + L.cboff);
  t.nproj = p->P.nproj;
  t.accumulate = p->P.opts.grad_accumulate;
  return t;
}

mlora_status hip_fail(hipError_t e, const char* what) {
  return fail(MLORA_ERR_HIP, std::string(what) + ": " + hipGetErrorName(e) + " (" +
                                 hipGetErrorString(e) + ")");
}

// Brackets one launch with events when profiling is on.
template <class F>
mlora_status timed(mlora_plan_s* p, int kind, hipStream_t s, F&& launch) {
  hipEvent_t a = nullptr, b = nullptr;
  const bool on = (p->prof >> kind) & 1u;
  if (on) {
    for (hipEvent_t* e : {&a, &b}) {
      if (!p->pool.empty()) {
        *e = p->pool.back();
        p->pool.pop_back();
      } else {
        hipError_t err = hipEventCreate(e);
        if (err != hipSuccess) return hip_fail(err, "hipEventCreate");
      }
    }
    hipError_t err = hipEventRecord(a, s);
    if (err != hipSuccess) return hip_fail(err, "hipEventRecord");
  }
  launch();
  hipError_t err = hipGetLastError();
  if (on) {
    hipError_t e2 = hipEventRecord(b, s);
    p->recs.push_back({kind, a, b});
    if (err == hipSuccess && e2 != hipSuccess) return hip_fail(e2, "hipEventRecord");
  }
  if (err != hipSuccess) return hip_fail(err, "kernel launch");
  return MLORA_OK;
}

// Events that only order the internal streams on this device: no timing and
// no system-scope fence (the host never inspects them; the producing
// kernel's completion makes its results visible to the device).
constexpr unsigned kOrderEvent = hipEventDisableTiming | hipEventDisableSystemFence;

mlora_status ensure_side(mlora_plan_s* p) {
  if (!p->side) {
    hipError_t e = hipStreamCreateWithFlags(&p->side, hipStreamNonBlocking);
    if (e != hipSuccess) {
      p->side = nullptr;
      return hip_fail(e, "hipStreamCreateWithFlags");
    }
  }
  for (hipEvent_t* ev : {&p->fork_ev, &p->done_ev})
    if (!*ev) {
      hipError_t e = hipEventCreateWithFlags(ev, kOrderEvent);
      if (e != hipSuccess) {
        *ev = nullptr;
        return hip_fail(e, "hipEventCreateWithFlags");
      }
    }
  while ((int)p->group_ev.size() < p->P.n_groups) {
    hipEvent_t ev;
    hipError_t e = hipEventCreateWithFlags(&ev, kOrderEvent);
    if (e != hipSuccess) return hip_fail(e, "hipEventCreateWithFlags");
    p->group_ev.push_back(ev);
  }
  return MLORA_OK;
}

// The side stream starts after everything enqueued on the caller's stream so far.
mlora_status fork_side(mlora_plan_s* p, hipStream_t cs) {
  mlora_status st = ensure_side(p);
  if (st != MLORA_OK) return st;
  hipError_t e = hipEventRecord(p->fork_ev, cs);
  if (e == hipSuccess) e = hipStreamWaitEvent(p->side, p->fork_ev, 0);
  return e == hipSuccess ? MLORA_OK : hip_fail(e, "fork of the side stream");
}

// The caller's stream waits for what the side stream has done so far; ev is
// recorded on the side stream.
mlora_status wait_side(mlora_plan_s* p, hipEvent_t ev, hipStream_t cs) {
  hipError_t e = hipEventRecord(ev, p->side);
  if (e == hipSuccess) e = hipStreamWaitEvent(cs, ev, 0);
  return e == hipSuccess ? MLORA_OK : hip_fail(e, "join of the side stream");
}

bool aligned16(const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15u) == 0; }

// A graph capture of a plan with several stream groups once ended in a fault
// of the runtime, under an earlier arrangement of the internal streams (one
// stream per group, forked twice per step, each forking a weight-gradient
// stream of its own).  Its cause was not shown, so such plans stay refused
// on a capturing stream; one group captures and replays exactly.
mlora_status check_capture(const mlora_plan_s* p, hipStream_t cs) {
  if (p->P.n_groups <= 1) return MLORA_OK;
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  hipError_t e = hipStreamIsCapturing(cs, &cap);
  if (e != hipSuccess) return hip_fail(e, "hipStreamIsCapturing");
  if (cap != hipStreamCaptureStatusNone)
    return fail(MLORA_ERR_UNSUPPORTED,
                "plans with several stream groups are not supported under graph capture; use n_streams = 1");
  return MLORA_OK;
}

mlora_status check_ws(const mlora_plan_s* p, void* ws, size_t ws_bytes) {
  if (!ws) return fail(MLORA_ERR_INVALID_ARG, "workspace is NULL");
  if (ws_bytes < p->L.workspace_bytes)
    return fail(MLORA_ERR_WORKSPACE, "workspace has " + std::to_string(ws_bytes) + " bytes, plan needs " +
                                         std::to_string(p->L.workspace_bytes));
  if (ws != p->uploaded_ws)
    return fail(MLORA_ERR_WORKSPACE, "plan tables were not uploaded to this workspace (mlora_plan_upload)");
  return MLORA_OK;
}

}  // namespace

// Decode of an MXFP8 or MXFP4 base (codes, then the E8M0 scales) into the
// workspace's bf16 copy, in the base's layout.
mlora_status decode_base(mlora_plan_s* p, const void* W0, uint16_t* w0deq, bool nk, hipStream_t cs) {
  const auto& P = p->P;
  const uint8_t* codes = static_cast<const uint8_t*>(W0);
  const bool fp4 = P.opts.w0_format == MLORA_W0_MXFP4;
  const int64_t code_bytes = fp4 ? P.d_in * P.d_out / 2 : P.d_in * P.d_out;
  return timed(p, MLORA_K_DEQUANT, cs, [&] {
    if (fp4) mlora::launch_dequant_mx4(nk, codes, codes + code_bytes, P.d_in, P.d_out, w0deq, cs);
    else mlora::launch_dequant_mx(nk, codes, codes + code_bytes, P.d_in, P.d_out, w0deq, cs);
  });
}

extern "C" {

const char* mlora_version(void) { return "mlora 0.1 gfx950"; }

const char* mlora_status_string(mlora_status s) {
  switch (s) {
    case MLORA_OK: return "MLORA_OK";
    case MLORA_ERR_INVALID_ARG: return "MLORA_ERR_INVALID_ARG";
    case MLORA_ERR_UNSUPPORTED: return "MLORA_ERR_UNSUPPORTED";
    case MLORA_ERR_HIP: return "MLORA_ERR_HIP";
    case MLORA_ERR_WORKSPACE: return "MLORA_ERR_WORKSPACE";
    case MLORA_ERR_NOMEM: return "MLORA_ERR_NOMEM";
  }
  return "MLORA_ERR_UNKNOWN";
}

const char* mlora_last_error(void) { return g_err.c_str(); }

namespace {

mlora_status finish_plan(mlora::PlanTables&& P, mlora_plan_t* out) {
  auto* p = new mlora_plan_s();
  p->P = std::move(P);
  p->L = mlora::device_layout(p->P);
  p->blob = mlora::table_blob(p->P, p->L);
  const int S = p->P.n_groups;
  p->chunk_b.resize(S);
  p->group_max_rank.assign(S, 1);
  for (int g = 0; g < S; ++g) {
    p->chunk_b[g] = bucket_ranges(p->P.chunks, 3, p->P.chunk_start[g], p->P.chunk_start[g + 1], p->P.rpad,
                                  p->P.nproj);
    for (int32_t v = p->P.groups[g] * p->P.nproj; v < p->P.groups[g + 1] * p->P.nproj; ++v)
      p->group_max_rank[g] = std::max(p->group_max_rank[g], p->P.ranks[v]);
    p->max_rank = std::max(p->max_rank, p->group_max_rank[g]);
  }
  // Where the weight gradients run (the fp32 path runs everything on the
  // caller's stream): by wg_overlap, AUTO choosing the side stream while the
  // dX GEMMs of all groups together have at most 16 rounds of 256 output
  // tiles.
  const auto& Q = p->P;
  const int64_t dx_tiles = (int64_t)(Q.tile_start[S] - Q.tile_start[0]) * ((Q.d_in + 255) / 256);
  if (Q.dtype != MLORA_BF16) p->wg_side = false;
  else if (Q.opts.wg_overlap == MLORA_WG_SIDE) p->wg_side = true;
  else if (Q.opts.wg_overlap == MLORA_WG_AFTER) p->wg_side = false;
  else p->wg_side = dx_tiles <= 16 * 256;
  *out = p;
  return MLORA_OK;
}

}  // namespace

mlora_status mlora_plan(int32_t n, const int64_t* seg_offsets, const int32_t* ranks, int64_t d_in,
                        int64_t d_out, mlora_dtype dtype, const mlora_plan_opts* opts,
                        mlora_plan_t* out) {
  if (!out) return fail(MLORA_ERR_INVALID_ARG, "out is NULL");
  try {
    mlora::PlanTables P;
    std::string err;
    mlora_status st = mlora::build_plan(n, seg_offsets, ranks, d_in, d_out, (int32_t)dtype, opts, P, err);
    if (st != MLORA_OK) return fail(st, err);
    return finish_plan(std::move(P), out);
  } catch (const std::bad_alloc&) {
    return fail(MLORA_ERR_NOMEM, "host allocation failed while building the plan");
  }
}

mlora_status mlora_plan_from_ids(int32_t n, int64_t T, const int32_t* token_adapter,
                                 const int32_t* ranks, int64_t d_in, int64_t d_out, mlora_dtype dtype,
                                 const mlora_plan_opts* opts, mlora_plan_t* out) {
  if (!out) return fail(MLORA_ERR_INVALID_ARG, "out is NULL");
  try {
    mlora::PlanTables P;
    std::string err;
    mlora_status st = mlora::build_plan_from_ids(n, T, token_adapter, ranks, d_in, d_out,
                                                 (int32_t)dtype, opts, P, err);
    if (st != MLORA_OK) return fail(st, err);
    return finish_plan(std::move(P), out);
  } catch (const std::bad_alloc&) {
    return fail(MLORA_ERR_NOMEM, "host allocation failed while building the plan");
  }
}

mlora_status mlora_plan_multi(int32_t n, const int64_t* seg_offsets, int32_t n_proj, const int64_t* widths,
                              const int32_t* ranks, int64_t d_in, mlora_dtype dtype,
                              const mlora_plan_opts* opts, mlora_plan_t* out) {
  if (!out) return fail(MLORA_ERR_INVALID_ARG, "out is NULL");
  try {
    mlora::PlanTables P;
    std::string err;
    mlora_status st = mlora::build_plan_multi(n, seg_offsets, n_proj, widths, ranks, d_in, (int32_t)dtype,
                                               opts, P, err);
    if (st != MLORA_OK) return fail(st, err);
    return finish_plan(std::move(P), out);
  } catch (const std::bad_alloc&) {
    return fail(MLORA_ERR_NOMEM, "host allocation failed while building the plan");
  }
}

mlora_status mlora_plan_multi_from_ids(int32_t n, int64_t T, const int32_t* token_adapter, int32_t n_proj,
                                       const int64_t* widths, const int32_t* ranks, int64_t d_in,
                                       mlora_dtype dtype, const mlora_plan_opts* opts, mlora_plan_t* out) {
  if (!out) return fail(MLORA_ERR_INVALID_ARG, "out is NULL");
  try {
    mlora::PlanTables P;
    std::string err;
    mlora_status st = mlora::build_plan_multi_from_ids(n, T, token_adapter, n_proj, widths, ranks, d_in,
                                                       (int32_t)dtype, opts, P, err);
    if (st != MLORA_OK) return fail(st, err);
    return finish_plan(std::move(P), out);
  } catch (const std::bad_alloc&) {
    return fail(MLORA_ERR_NOMEM, "host allocation failed while building the plan");
  }
}

void mlora_plan_destroy(mlora_plan_t p) {
  if (!p) return;
  // Teardown is best effort: errors here have no caller to report to.
  if (p->side) (void)hipStreamDestroy(p->side);
  for (hipEvent_t e : {p->fork_ev, p->done_ev})
    if (e) (void)hipEventDestroy(e);
  for (hipEvent_t e : p->group_ev) (void)hipEventDestroy(e);
  for (auto& r : p->recs) {
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
  for (hipEvent_t e : p->pool) (void)hipEventDestroy(e);
  delete p;
}

mlora_status mlora_plan_get_info(mlora_plan_t p, mlora_plan_info* info) {
  if (!p || !info) return fail(MLORA_ERR_INVALID_ARG, "plan and info must be non-NULL");
  const auto& P = p->P;
  mlora_plan_info i{};
  i.T = P.T;
  i.n = P.n;
  i.d_in = P.d_in;
  i.d_out = P.d_out;
  i.dtype = P.dtype;
  i.n_groups = P.n_groups;
  i.z_elems = P.z_elems;
  i.z_bytes = P.z_elems * (P.dtype == MLORA_BF16 ? 2 : 4);
  i.workspace_bytes = (int64_t)p->L.workspace_bytes;
  i.table_bytes = (int64_t)p->L.table_bytes;
  i.rpad_total = P.rpad_total;
  i.partial_rows = P.partial_rows;
  i.n_nano = P.n_nano();
  i.n_chunks = P.n_chunks();
  i.n_tiles = P.n_tiles();
  i.n_ext = P.n_ext();
  i.n_opt_blocks = P.n_oblk();
  i.n_proj = P.nproj;
  i.dz_offset = (int64_t)p->L.dz;
  i.act_offset = P.opts.act_format == MLORA_ACT_MXFP8 ? (int64_t)p->L.xq : -1;
  i.wg_side = p->wg_side ? 1 : 0;
  *info = i;
  return MLORA_OK;
}

mlora_status mlora_plan_export(mlora_plan_t p, int32_t table, void* dst, size_t* bytes_inout) {
  if (!p || !bytes_inout) return fail(MLORA_ERR_INVALID_ARG, "plan and bytes_inout must be non-NULL");
  const auto& P = p->P;
  const void* src = nullptr;
  size_t bytes = 0;
  auto v32 = [&](const std::vector<int32_t>& v) { src = v.data(); bytes = 4 * v.size(); };
  auto v64 = [&](const std::vector<int64_t>& v) { src = v.data(); bytes = 8 * v.size(); };
  switch (table) {
    case MLORA_TAB_RPAD: v32(P.rpad); break;
    case MLORA_TAB_ZOFF: v64(P.zoff); break;
    case MLORA_TAB_ROFF: v32(P.roff); break;
    case MLORA_TAB_GROUPS: v32(P.groups); break;
    case MLORA_TAB_NANO: v32(P.nano); break;
    case MLORA_TAB_NANO_START: v32(P.nano_start); break;
    case MLORA_TAB_CHUNKS: v32(P.chunks); break;
    case MLORA_TAB_CHUNK_START: v32(P.chunk_start); break;
    case MLORA_TAB_CHUNK_RPREF: v32(P.cpref); break;
    case MLORA_TAB_ADAPTER_CHUNK_FIRST: v32(P.ch_first); break;
    case MLORA_TAB_ADAPTER_CHUNK_COUNT: v32(P.ch_count); break;
    case MLORA_TAB_TILES: v32(P.tiles); break;
    case MLORA_TAB_TILE_START: v32(P.tile_start); break;
    case MLORA_TAB_EXT: v32(P.ext); break;
    case MLORA_TAB_TILE_EXT_START: v32(P.ext_start); break;
    case MLORA_TAB_OFFSETS: v64(P.offsets); break;
    case MLORA_TAB_RANKS: v32(P.ranks); break;
    case MLORA_TAB_PERM: v32(P.perm); break;
    case MLORA_TAB_OPT_BLOCKS: v32(P.oblk); break;
    case MLORA_TAB_PROJ_COLS: v32(P.pcol); break;
    case MLORA_TAB_SEG_START: v64(P.seg0); break;
    case MLORA_TAB_CHUNK_BOFF: v64(P.cboff); break;
    case MLORA_TAB_KSPLIT: v32(P.ksplit); break;
    case MLORA_TAB_OPT_FIRST: v32(P.oblk_first); break;
    default: return fail(MLORA_ERR_INVALID_ARG, "unknown table id " + std::to_string(table));
  }
  if (!dst) {
    *bytes_inout = bytes;
    return MLORA_OK;
  }
  if (*bytes_inout < bytes) {
    *bytes_inout = bytes;
    return fail(MLORA_ERR_INVALID_ARG, "destination too small for table");
  }
  if (bytes) std::memcpy(dst, src, bytes);
  *bytes_inout = bytes;
  return MLORA_OK;
}

mlora_status mlora_plan_upload(mlora_plan_t p, void* ws, size_t ws_bytes, void* stream) {
  if (!p) return fail(MLORA_ERR_INVALID_ARG, "plan is NULL");
  if (!ws) return fail(MLORA_ERR_INVALID_ARG, "workspace is NULL");
  if (!aligned16(ws)) return fail(MLORA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  if (ws_bytes < p->L.workspace_bytes)
    return fail(MLORA_ERR_WORKSPACE, "workspace has " + std::to_string(ws_bytes) + " bytes, plan needs " +
                                         std::to_string(p->L.workspace_bytes));
  hipError_t e = hipMemcpyAsync(ws, p->blob.data(), p->blob.size(), hipMemcpyHostToDevice,
                                static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync (plan tables)");
  p->uploaded_ws = ws;
  return MLORA_OK;
}

}  // extern "C"

namespace {

// Device buffers of one forward call: the uploaded plan tables (the
// DevTables offsets are relative to their base), the rank-padded
// concatenations the kernels read, the split-K partial tiles and, for a
// microscaled base, its bf16 decoding.
struct FwdBufs {
  uint8_t* tables;
  uint16_t* acat_t;
  uint16_t* bcat_t;
  float* kpart;
  uint16_t* w0deq;
  uint8_t* xq;  // MXFP8 activations: codes [T][d_in], then scales [T][d_in / 32]
};

bool forward_args_ok(const mlora_plan_s* p, const void* X, const void* W0, const void* const* A,
                     const void* const* B, const float* scales, const void* Y, const void* Z,
                     mlora_status* st) {
  // With no rows at all, the row-indexed buffers may be NULL.
  const bool rows = p->P.T > 0;
  if ((rows && (!X || !Y || !Z)) || !W0 || !A || !B || !scales) {
    *st = fail(MLORA_ERR_INVALID_ARG, "forward: X, W0, A, B, scales, Y and Z must be non-NULL");
    return false;
  }
  for (const void* q : {X, W0, (const void*)A, (const void*)B, (const void*)scales, Y, Z})
    if (!aligned16(q)) {
      *st = fail(MLORA_ERR_INVALID_ARG, "forward: device pointers must be 16-byte aligned");
      return false;
    }
  return true;
}

mlora_status forward_impl(mlora_plan_s* p, const void* X, const void* W0, const void* const* A,
                          const void* const* B, const float* scales, void* Y, void* Z, const FwdBufs& fb,
                          hipStream_t cs) {
  const auto& P = p->P;
  mlora_status st = check_capture(p, cs);
  if (st != MLORA_OK) return st;
  mlora::DevTables t = dev_tables(p, fb.tables);
  // The forward reads [d_out][d_in] when it has it: the second half of a
  // two-layout base.
  const bool nk = P.opts.w0_layout != MLORA_W0_KN;
  if (P.opts.w0_layout == MLORA_W0_BOTH)
    W0 = static_cast<const uint8_t*>(W0) + (size_t)P.d_in * (size_t)P.d_out * (P.dtype == MLORA_FP32 ? 4 : 2);

  if (P.dtype == MLORA_FP32) {
    st = timed(p, MLORA_K_SHRINK, cs, [&] {
      mlora::launch_f32_shrink(t, P.n, P.T, P.d_in, (const float*)X, A, scales, (float*)Z, cs);
    });
    if (st != MLORA_OK) return st;
    return timed(p, MLORA_K_GEMM_FWD, cs, [&] {
      mlora::launch_f32_gemm(true, nk, t, P.n, P.T, (const float*)X, P.d_in, (const float*)W0,
                             nk ? P.d_in : P.d_out, (float*)Y, P.d_out, (int32_t)P.d_in,
                             (int32_t)P.d_out, (const float*)Z, B, cs);
    });
  }

  // MXFP8 activations: X quantized first; the base GEMM reads its codes and
  // the base's own codes, with no decoded copy of W0.
  const bool mxact = P.opts.act_format == MLORA_ACT_MXFP8;
  uint8_t* xq_codes = fb.xq;
  uint8_t* xq_scales = fb.xq + (size_t)P.T * (size_t)P.d_in;
  if (mxact) {
    st = timed(p, MLORA_K_QUANT_ACT, cs, [&] {
      mlora::launch_quant_act_mx8((const uint16_t*)X, P.T, P.d_in, xq_codes, xq_scales, cs);
    });
    if (st != MLORA_OK) return st;
  }
  // A microscaled base is otherwise decoded first; the GEMMs read that.
  const uint16_t* W0b = static_cast<const uint16_t*>(W0);
  if (P.opts.w0_format != MLORA_W0_BF16 && !mxact) {
    st = decode_base(p, W0, fb.w0deq, nk, cs);
    if (st != MLORA_OK) return st;
    W0b = fb.w0deq;
  }
  // A_cat^T feeds the shrink; with W0 as [d_out][d_in] the expand steps read
  // B in k-contiguous form, B_cat^T.
  st = timed(p, MLORA_K_PREP, cs, [&] {
    mlora::launch_prep(t, P.nv(), P.d_in, P.d_out, P.rpad_total, A, fb.acat_t, nullptr, B,
                       nk ? fb.bcat_t : nullptr, cs);
  });
  if (st != MLORA_OK) return st;
  // Several groups: the shrinks run on the side stream, group by group, and
  // each group's base GEMM on the caller's stream waits only for its own
  // group's shrink, so the shrink of group g+1 overlaps the GEMM of group g
  // while the GEMMs themselves run one at a time.  One group: all in order
  // on the caller's stream.
  const bool pipe = P.n_groups > 1;
  if (pipe) {
    st = fork_side(p, cs);
    if (st != MLORA_OK) return st;
  }
  hipStream_t ss = pipe ? p->side : cs;
  for (int g = 0; g < P.n_groups; ++g) {
    st = timed(p, MLORA_K_SHRINK, ss, [&] {
      mlora::launch_skinny(0, t, P.nano_start[g], P.nano_start[g + 1] - P.nano_start[g],
                           (const uint16_t*)X, P.d_in, fb.acat_t, nullptr, scales, (uint16_t*)Z, ss);
    });
    if (st != MLORA_OK) return st;
    if (pipe) {
      hipError_t e = hipEventRecord(p->group_ev[g], ss);
      if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
    }
  }
  for (int g = 0; g < P.n_groups; ++g) {
    if (pipe) {
      hipError_t e = hipStreamWaitEvent(cs, p->group_ev[g], 0);
      if (e != hipSuccess) return hip_fail(e, "hipStreamWaitEvent");
    }
    mlora::GemmArgs ga;
    ga.A = (const uint16_t*)X;
    ga.lda = P.d_in;
    ga.B = W0b;
    ga.ldb = nk ? P.d_in : P.d_out;
    ga.C = (uint16_t*)Y;
    ga.ldc = P.d_out;
    ga.K = (int32_t)P.d_in;
    ga.N = (int32_t)P.d_out;
    ga.tile_begin = P.tile_start[g];
    ga.n_mtiles = P.tile_start[g + 1] - P.tile_start[g];
    ga.n_ntiles = (int32_t)((P.d_out + 255) / 256);
    ga.ebuf = (const uint16_t*)Z;
    ga.eb = B;
    ga.ext_n = nullptr;
    ga.ext_k = fb.bcat_t;
    ga.rtot = P.rpad_total;
    ga.ksplit = P.ksplit[2 * g];
    ga.kper = (int32_t)((P.d_in / 32 + ga.ksplit - 1) / ga.ksplit);
    ga.part = fb.kpart + P.kpart_off[g];
    ga.t = t;
    if (mxact) {
      mlora::GemmMxArgs gm;
      gm.g = ga;
      gm.g.ksplit = 1;
      gm.Aq = xq_codes;
      gm.Asc = xq_scales;
      gm.b4 = P.opts.w0_format == MLORA_W0_MXFP4 ? 1 : 0;
      gm.Bq = static_cast<const uint8_t*>(W0);
      gm.Bsc = static_cast<const uint8_t*>(W0) + (size_t)P.d_in * (size_t)P.d_out / (gm.b4 ? 2 : 1);
      st = timed(p, MLORA_K_GEMM_FWD, cs, [&] { mlora::launch_gemm_mx8(gm, cs); });
    } else {
      st = timed(p, MLORA_K_GEMM_FWD, cs, [&] { mlora::launch_gemm(true, nk, ga, cs); });
    }
    if (st != MLORA_OK) return st;
  }
  // the last GEMM waited for the side stream's last event: it is joined
  return MLORA_OK;
}

mlora_status scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t e = mlora::noalloc_scratch(out, &dev);
  if (e == hipErrorInvalidDevice && dev >= 0)
    return fail(MLORA_ERR_UNSUPPORTED, "device " + std::to_string(dev) + " is beyond the static scratch table");
  if (e != hipSuccess) return hip_fail(e, "static scratch address (hipGetDevice / hipGetSymbolAddress)");
  return MLORA_OK;
}

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// The forward's buffers packed after the tables: A_cat^T, B_cat^T (a
// [d_out][d_in] base only), split-K partial tiles, the decoded base (a
// microscaled base only).  Sizes as in the workspace layout.
size_t noalloc_layout(const mlora_plan_s* p, size_t off[5]) {
  const auto& P = p->P;
  size_t at = p->L.table_bytes;
  const bool bf16 = P.dtype == MLORA_BF16;
  const bool nk = P.opts.w0_layout != MLORA_W0_KN;
  const bool mxact = P.opts.act_format == MLORA_ACT_MXFP8;
  const size_t sz[5] = {bf16 ? (size_t)P.rpad_total * (size_t)P.d_in * 2 : 0,
                        bf16 && nk ? (size_t)P.rpad_total * (size_t)P.d_out * 2 : 0,
                        bf16 ? (size_t)P.kpart_off.back() * 4 : 0,
                        bf16 && P.opts.w0_format != MLORA_W0_BF16 && !mxact ? (size_t)P.d_in * (size_t)P.d_out * 2 : 0,
                        mxact ? (size_t)P.T * (size_t)P.d_in * 33 / 32 : 0};
  for (int k = 0; k < 5; ++k) {
    off[k] = at;
    at += align256(sz[k]);
  }
  return at;
}

}  // namespace

extern "C" {

mlora_status mlora_forward(mlora_plan_t p, const void* X, const void* W0, const void* const* A,
                           const void* const* B, const float* scales, void* Y, void* Z, void* ws,
                           size_t ws_bytes, void* stream) {
  if (!p) return fail(MLORA_ERR_INVALID_ARG, "plan is NULL");
  mlora_status st;
  if (!forward_args_ok(p, X, W0, A, B, scales, Y, Z, &st)) return st;
  st = check_ws(p, ws, ws_bytes);
  if (st != MLORA_OK) return st;
  uint8_t* wsb = static_cast<uint8_t*>(ws);
  const auto& L = p->L;
  const FwdBufs fb{wsb, reinterpret_cast<uint16_t*>(wsb + L.acat_t), reinterpret_cast<uint16_t*>(wsb + L.bcat_t),
                   reinterpret_cast<float*>(wsb + L.kpart), reinterpret_cast<uint16_t*>(wsb + L.w0deq), wsb + L.xq};
  return forward_impl(p, X, W0, A, B, scales, Y, Z, fb, static_cast<hipStream_t>(stream));
}

mlora_status mlora_forward_noalloc(mlora_plan_t p, const void* X, const void* W0, const void* const* A,
                                   const void* const* B, const float* scales, void* Y, void* Z,
                                   void* stream) {
  if (!p) return fail(MLORA_ERR_INVALID_ARG, "plan is NULL");
  mlora_status st;
  if (!forward_args_ok(p, X, W0, A, B, scales, Y, Z, &st)) return st;
  size_t off[5];
  const size_t need = noalloc_layout(p, off);
  if (need > mlora::kNoallocScratchBytes)
    return fail(MLORA_ERR_UNSUPPORTED, "forward_noalloc: the layer needs " + std::to_string(need) +
                                           " bytes of scratch; the static scratch holds " +
                                           std::to_string(mlora::kNoallocScratchBytes) + " (use mlora_forward)");
  hipStream_t cs = static_cast<hipStream_t>(stream);
  st = check_capture(p, cs);
  if (st != MLORA_OK) return st;
  void* sp = nullptr;
  st = scratch_for_current_device(&sp);
  if (st != MLORA_OK) return st;
  uint8_t* b = static_cast<uint8_t*>(sp);
  // The scratch keeps whatever the last call on this device left: the plan
  // tables (the zero page among them) go in first, and every other byte the
  // kernels read is written earlier in this call.
  hipError_t e = hipMemcpyAsync(b, p->blob.data(), p->blob.size(), hipMemcpyHostToDevice, cs);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync (plan tables into the static scratch)");
  const FwdBufs fb{b, reinterpret_cast<uint16_t*>(b + off[0]), reinterpret_cast<uint16_t*>(b + off[1]),
                   reinterpret_cast<float*>(b + off[2]), reinterpret_cast<uint16_t*>(b + off[3]), b + off[4]};
  return forward_impl(p, X, W0, A, B, scales, Y, Z, fb, cs);
}

mlora_status mlora_backward(mlora_plan_t p, const void* dY, const void* X, const void* W0,
                            const void* const* A, const void* const* B, const float* scales,
                            const void* Z, void* dX, void* const* dA, void* const* dB, void* ws,
                            size_t ws_bytes, void* stream) {
  if (!p) return fail(MLORA_ERR_INVALID_ARG, "plan is NULL");
  const bool rows = p->P.T > 0;
  if ((rows && (!dY || !X || !Z)) || !W0 || !A || !B || !scales || !dA || !dB)
    return fail(MLORA_ERR_INVALID_ARG,
                "backward: dY, X, W0, A, B, scales, Z, dA and dB must be non-NULL (dX may be NULL)");
  for (const void* q : {dY, X, W0, (const void*)A, (const void*)B, (const void*)scales, Z,
                        (const void*)dA, (const void*)dB})
    if (!aligned16(q)) return fail(MLORA_ERR_INVALID_ARG, "backward: device pointers must be 16-byte aligned");
  if (dX && !aligned16(dX)) return fail(MLORA_ERR_INVALID_ARG, "backward: dX must be 16-byte aligned");
  mlora_status st = check_ws(p, ws, ws_bytes);
  if (st != MLORA_OK) return st;
  const auto& P = p->P;
  const auto& L = p->L;
  hipStream_t cs = static_cast<hipStream_t>(stream);
  st = check_capture(p, cs);
  if (st != MLORA_OK) return st;
  mlora::DevTables t = dev_tables(p, ws);
  uint8_t* wsb = static_cast<uint8_t*>(ws);
  // dX reads [d_in][d_out] when it has it: the first half of a two-layout base.
  const bool nk = P.opts.w0_layout == MLORA_W0_NK;

  if (P.dtype == MLORA_FP32) {
    float* dZ = reinterpret_cast<float*>(wsb + L.dz);
    st = timed(p, MLORA_K_DZ, cs, [&] {
      mlora::launch_f32_dz(t, P.n, P.T, P.d_out, (const float*)dY, B, scales, dZ, cs);
    });
    if (st != MLORA_OK) return st;
    st = timed(p, MLORA_K_TOKEN_REDUCE, cs, [&] {
      mlora::launch_f32_db(t, P.nv(), P.d_out, (const float*)Z, (const float*)dY, dB, p->max_rank, cs);
    });
    if (st != MLORA_OK) return st;
    st = timed(p, MLORA_K_TOKEN_REDUCE, cs, [&] {
      mlora::launch_f32_da(t, P.nv(), P.d_in, (const float*)X, dZ, dA, p->max_rank, cs);
    });
    if (st != MLORA_OK) return st;
    if (!dX) return MLORA_OK;
    return timed(p, MLORA_K_GEMM_DX, cs, [&] {
      mlora::launch_f32_gemm(false, !nk, t, P.n, P.T, (const float*)dY, P.d_out, (const float*)W0,
                             nk ? P.d_in : P.d_out, (float*)dX, P.d_in, (int32_t)P.d_out,
                             (int32_t)P.d_in, dZ, A, cs);
    });
  }

  uint16_t* dZ = reinterpret_cast<uint16_t*>(wsb + L.dz);
  float* partA = reinterpret_cast<float*>(wsb + L.part_a);
  float* partB = reinterpret_cast<float*>(wsb + L.part_b);
  uint16_t* acat_t = reinterpret_cast<uint16_t*>(wsb + L.acat_t);
  uint16_t* acat = reinterpret_cast<uint16_t*>(wsb + L.acat);
  // The dZ.A^T extension steps of the dX GEMM read A in the layout of the
  // main B operand: k-contiguous A_cat with W0 as [d_in][d_out], n-contiguous
  // A_cat^T otherwise.  Rebuilt here so the backward does not depend on what
  // the workspace held before.
  if (dX) {
    st = timed(p, MLORA_K_PREP, cs, [&] {
      mlora::launch_prep_a(t, P.nv(), P.d_in, P.rpad_total, A, nk ? acat_t : nullptr,
                           nk ? nullptr : acat, cs);
    });
    if (st != MLORA_OK) return st;
  }
  // dX reads the base weight; a microscaled base is decoded into the workspace.
  const uint16_t* W0b = static_cast<const uint16_t*>(W0);
  if (dX && P.opts.w0_format != MLORA_W0_BF16) {
    st = decode_base(p, W0, reinterpret_cast<uint16_t*>(wsb + L.w0deq), nk, cs);
    if (st != MLORA_OK) return st;
    W0b = reinterpret_cast<const uint16_t*>(wsb + L.w0deq);
  }
  auto dz = [&](int g, hipStream_t s) -> mlora_status {
    return timed(p, MLORA_K_DZ, s, [&] {
      mlora::launch_skinny(1, t, P.nano_start[g], P.nano_start[g + 1] - P.nano_start[g],
                           (const uint16_t*)dY, P.d_out, nullptr, B, scales, dZ, s);
    });
  };
  // Weight gradients of group g: token reductions, then the fixed-order
  // partial sums.
  auto weight_grads = [&](int g, hipStream_t sw) -> mlora_status {
    for (const Range& r : p->chunk_b[g]) {
      mlora_status s2 = timed(p, MLORA_K_TOKEN_REDUCE, sw, [&] {
        const int64_t c0 = P.pcol[r.proj], w = P.pcol[r.proj + 1] - c0;
        mlora::launch_token_reduce(r.rp, t, r.begin, r.count, (const uint16_t*)dY + c0, P.d_out,
                                   (const uint16_t*)Z, partB, w, (const uint16_t*)X, dZ, partA, P.d_in, dA, dB,
                                   sw);
      });
      if (s2 != MLORA_OK) return s2;
    }
    return timed(p, MLORA_K_REDUCE, sw, [&] {
      mlora::launch_reduce_partials(t, P.groups[g] * P.nproj, P.groups[g + 1] * P.nproj, P.d_in, P.d_out,
                                    partA, partB, dA, dB, p->group_max_rank[g], sw);
    });
  };
  auto dx_gemm = [&](int g) -> mlora_status {
    mlora::GemmArgs ga;
    ga.A = (const uint16_t*)dY;
    ga.lda = P.d_out;
    ga.B = W0b;
    ga.ldb = nk ? P.d_in : P.d_out;
    ga.C = (uint16_t*)dX;
    ga.ldc = P.d_in;
    ga.K = (int32_t)P.d_out;
    ga.N = (int32_t)P.d_in;
    ga.tile_begin = P.tile_start[g];
    ga.n_mtiles = P.tile_start[g + 1] - P.tile_start[g];
    ga.n_ntiles = (int32_t)((P.d_in + 255) / 256);
    ga.ebuf = dZ;
    ga.eb = A;
    ga.ext_n = acat_t;
    ga.ext_k = acat;
    ga.rtot = P.rpad_total;
    ga.ksplit = P.ksplit[2 * g + 1];
    ga.kper = (int32_t)((P.d_out / 32 + ga.ksplit - 1) / ga.ksplit);
    ga.part = reinterpret_cast<float*>(wsb + L.kpart) + P.kpart_off[g];
    ga.t = t;
    return timed(p, MLORA_K_GEMM_DX, cs, [&] { mlora::launch_gemm(false, !nk, ga, cs); });
  };

  if (!dX) {
    for (int g = 0; g < P.n_groups; ++g) {
      if ((st = dz(g, cs)) != MLORA_OK || (st = weight_grads(g, cs)) != MLORA_OK) return st;
    }
    return MLORA_OK;
  }
  if (P.n_groups == 1) {
    // The weight gradients need dZ but not dX.  Side: they run on the side
    // stream, enqueued after the dX GEMM so the GEMM's tiles take the chip
    // first and the reductions fill the CUs its last round of tiles leaves
    // idle.  After: on the caller's stream once the GEMM is done.
    if (!p->wg_side) {
      if ((st = dz(0, cs)) != MLORA_OK || (st = dx_gemm(0)) != MLORA_OK) return st;
      return weight_grads(0, cs);
    }
    if ((st = dz(0, cs)) != MLORA_OK || (st = fork_side(p, cs)) != MLORA_OK || (st = dx_gemm(0)) != MLORA_OK ||
        (st = weight_grads(0, p->side)) != MLORA_OK)
      return st;
    return wait_side(p, p->done_ev, cs);
  }
  // Several groups: every group's dZ on the side stream, then (side) every
  // group's weight gradients there too; the dX GEMM of group g, on the
  // caller's stream, waits only for group g's dZ, so the GEMMs run one at a
  // time while the side stream's HBM-bound work runs beside them.  After:
  // the weight gradients follow the last GEMM on the caller's stream.
  if ((st = fork_side(p, cs)) != MLORA_OK) return st;
  for (int g = 0; g < P.n_groups; ++g) {
    if ((st = dz(g, p->side)) != MLORA_OK) return st;
    hipError_t e = hipEventRecord(p->group_ev[g], p->side);
    if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
  }
  if (p->wg_side)
    for (int g = 0; g < P.n_groups; ++g)
      if ((st = weight_grads(g, p->side)) != MLORA_OK) return st;
  hipError_t e = hipEventRecord(p->done_ev, p->side);
  if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
  for (int g = 0; g < P.n_groups; ++g) {
    e = hipStreamWaitEvent(cs, p->group_ev[g], 0);
    if (e != hipSuccess) return hip_fail(e, "hipStreamWaitEvent");
    if ((st = dx_gemm(g)) != MLORA_OK) return st;
  }
  e = hipStreamWaitEvent(cs, p->done_ev, 0);
  if (e != hipSuccess) return hip_fail(e, "join of the side stream");
  if (!p->wg_side)
    for (int g = 0; g < P.n_groups; ++g)
      if ((st = weight_grads(g, cs)) != MLORA_OK) return st;
  return MLORA_OK;
}

mlora_status mlora_adamw_step(mlora_plan_t p, const mlora_adamw_hparams* hparams, void* const* A,
                              void* const* B, const void* const* dA, const void* const* dB,
                              void* const* mA, void* const* vA, void* const* mB, void* const* vB,
                              void* const* A_copy, void* const* B_copy, int32_t clip_grads,
                              void* ws, size_t ws_bytes, void* stream) {
  if (!p) return fail(MLORA_ERR_INVALID_ARG, "plan is NULL");
  for (const void* q : {(const void*)hparams, (const void*)A, (const void*)B, (const void*)dA,
                        (const void*)dB, (const void*)mA, (const void*)vA, (const void*)mB,
                        (const void*)vB})
    if (!q || !aligned16(q))
      return fail(MLORA_ERR_INVALID_ARG,
                  "adamw: hparams, A, B, dA, dB, mA, vA, mB and vB must be non-NULL and 16-byte aligned");
  if ((A_copy == nullptr) != (B_copy == nullptr))
    return fail(MLORA_ERR_INVALID_ARG, "adamw: A_copy and B_copy must be both NULL or both non-NULL");
  if (A_copy && p->P.dtype != MLORA_BF16)
    return fail(MLORA_ERR_INVALID_ARG, "adamw: an fp32 plan takes no weight copies (A_copy, B_copy must be NULL)");
  if (A_copy && (!aligned16(A_copy) || !aligned16(B_copy)))
    return fail(MLORA_ERR_INVALID_ARG, "adamw: A_copy and B_copy must be 16-byte aligned");
  if (!p->P.oblk_ok)
    return fail(MLORA_ERR_UNSUPPORTED, "adamw: the layer has more than 2^27 optimizer work items");
  if (clip_grads != 0 && clip_grads != 1)
    return fail(MLORA_ERR_INVALID_ARG, "adamw: clip_grads must be 0 or 1");
  mlora_status st = check_ws(p, ws, ws_bytes);
  if (st != MLORA_OK) return st;
  hipStream_t cs = static_cast<hipStream_t>(stream);
  mlora::AdamwArgs a;
  a.t = dev_tables(p, ws);
  a.hp = hparams;
  a.d_in = p->P.d_in;
  a.d_out = p->P.d_out;
  a.A = reinterpret_cast<float* const*>(A);
  a.B = reinterpret_cast<float* const*>(B);
  a.dA = reinterpret_cast<const float* const*>(dA);
  a.dB = reinterpret_cast<const float* const*>(dB);
  a.mA = reinterpret_cast<float* const*>(mA);
  a.vA = reinterpret_cast<float* const*>(vA);
  a.mB = reinterpret_cast<float* const*>(mB);
  a.vB = reinterpret_cast<float* const*>(vB);
  a.A_copy = reinterpret_cast<uint16_t* const*>(A_copy);
  a.B_copy = reinterpret_cast<uint16_t* const*>(B_copy);
  a.gsq = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + p->L.gnorm);
  a.coef = clip_grads ? a.gsq + p->P.n_oblk() : nullptr;
  if (clip_grads) {
    st = timed(p, MLORA_K_GRAD_NORM, cs, [&] { mlora::launch_grad_norm(a, p->P.n_oblk(), p->P.nv(), cs); });
    if (st != MLORA_OK) return st;
  }
  return timed(p, MLORA_K_ADAMW, cs, [&] { mlora::launch_adamw(a, p->P.n_oblk(), cs); });
}

mlora_status mlora_profile_enable(mlora_plan_t p, int32_t mask) {
  if (!p) return fail(MLORA_ERR_INVALID_ARG, "plan is NULL");
  p->prof = (uint32_t)mask & ((1u << MLORA_K_COUNT) - 1u);
  return MLORA_OK;
}

mlora_status mlora_profile_read(mlora_plan_t p, double* total_ms, int64_t* launches) {
  if (!p || !total_ms || !launches) return fail(MLORA_ERR_INVALID_ARG, "NULL argument");
  for (int k = 0; k < MLORA_K_COUNT; ++k) {
    total_ms[k] = 0.0;
    launches[k] = 0;
  }
  mlora_status st = MLORA_OK;
  for (auto& r : p->recs) {
    hipError_t e = hipEventSynchronize(r.b);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.a, r.b);
    if (e != hipSuccess && st == MLORA_OK) st = hip_fail(e, "profile event");
    total_ms[r.kind] += ms;
    launches[r.kind] += 1;
    p->pool.push_back(r.a);
    p->pool.push_back(r.b);
  }
  p->recs.clear();
  return st;
}

mlora_status mlora_device_check(void) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(MLORA_ERR_UNSUPPORTED, std::string("device is ") + prop.gcnArchName + ", library is built for gfx950");
  return MLORA_OK;
}

mlora_status mlora_base_transpose(const void* in, void* out, int64_t rows, int64_t cols,
                                  mlora_dtype dtype, void* stream) {
  if (!in || !out || !aligned16(in) || !aligned16(out))
    return fail(MLORA_ERR_INVALID_ARG, "base_transpose: in and out must be non-NULL and 16-byte aligned");
  if (rows <= 0 || cols <= 0 || rows % 64 != 0 || cols % 64 != 0 || rows > (1 << 20) || cols > (1 << 20))
    return fail(MLORA_ERR_INVALID_ARG, "base_transpose: rows and cols must be positive multiples of 64");
  if (dtype != MLORA_BF16 && dtype != MLORA_FP32)
    return fail(MLORA_ERR_INVALID_ARG, "base_transpose: dtype must be MLORA_BF16 or MLORA_FP32");
  const size_t bytes = (size_t)rows * (size_t)cols * (dtype == MLORA_FP32 ? 4 : 2);
  const uintptr_t a = reinterpret_cast<uintptr_t>(in), b = reinterpret_cast<uintptr_t>(out);
  if (a < b + bytes && b < a + bytes) return fail(MLORA_ERR_INVALID_ARG, "base_transpose: in and out overlap");
  hipStream_t s = static_cast<hipStream_t>(stream);
  mlora::launch_transpose(in, out, rows, cols, dtype == MLORA_FP32 ? 4 : 2, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "base_transpose launch");
  return MLORA_OK;
}

}  // extern "C"
