// Random-input driver of the host side of libmlora: the plan builders
// (segments, per-token ids, projections sharing the input, both), every
// table export, plan info, and the argument checks of forward, backward,
// the optimizer step and the base transpose.  Built with AddressSanitizer
// and UndefinedBehaviorSanitizer by tests/test_sanitize_cpu.py; any report
// aborts the run.  Arguments that pass the checks are never handed to the
// device: no workspace is ever uploaded, so every layer call must stop at
// the workspace check, and the kernel launchers below abort if reached.
#include <cinttypes>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../../include/mlora.h"
#include "../../adapter_lora_segments_amd/csrc/kernels.hpp"

namespace mlora {
[[noreturn]] static void reached(const char* what) {
  std::fprintf(stderr, "kernel launcher %s reached from the host checks\n", what);
  std::abort();
}
void launch_prep_a(const DevTables&, int32_t, int64_t, int64_t, const void* const*, uint16_t*, uint16_t*,
                   hipStream_t) { reached("prep_a"); }
void launch_prep_b(const DevTables&, int32_t, int64_t, int64_t, const void* const*, uint16_t*, hipStream_t) {
  reached("prep_b");
}
void launch_prep(const DevTables&, int32_t, int64_t, int64_t, int64_t, const void* const*, uint16_t*, uint16_t*,
                 const void* const*, uint16_t*, hipStream_t) { reached("prep"); }
void launch_skinny(int, const DevTables&, int32_t, int32_t, const uint16_t*, int64_t, const uint16_t*,
                   const void* const*, const float*, uint16_t*, hipStream_t) { reached("skinny"); }
void launch_token_reduce(int, const DevTables&, int32_t, int32_t, const uint16_t*, int64_t, const uint16_t*,
                         float*, int64_t, const uint16_t*, const uint16_t*, float*, int64_t, void* const*,
                         void* const*, hipStream_t) {
  reached("token_reduce");
}
void launch_reduce_partials(const DevTables&, int32_t, int32_t, int64_t, int64_t, const float*, const float*,
                            void* const*, void* const*, int32_t, hipStream_t) { reached("reduce_partials"); }
void launch_gemm(bool, bool, const GemmArgs&, hipStream_t) { reached("gemm"); }
void launch_transpose(const void*, void*, int64_t, int64_t, int, hipStream_t) { reached("transpose"); }
void launch_dequant_mx(bool, const uint8_t*, const uint8_t*, int64_t, int64_t, uint16_t*, hipStream_t) {
  reached("dequant_mx");
}
void launch_dequant_mx4(bool, const uint8_t*, const uint8_t*, int64_t, int64_t, uint16_t*, hipStream_t) {
  reached("dequant_mx4");
}
void launch_f32_shrink(const DevTables&, int32_t, int64_t, int64_t, const float*, const void* const*,
                       const float*, float*, hipStream_t) { reached("f32_shrink"); }
void launch_f32_dz(const DevTables&, int32_t, int64_t, int64_t, const float*, const void* const*, const float*,
                   float*, hipStream_t) { reached("f32_dz"); }
void launch_f32_gemm(bool, bool, const DevTables&, int32_t, int64_t, const float*, int64_t, const float*,
                     int64_t, float*, int64_t, int32_t, int32_t, const float*, const void* const*, hipStream_t) {
  reached("f32_gemm");
}
void launch_f32_db(const DevTables&, int32_t, int64_t, const float*, const float*, void* const*, int32_t,
                   hipStream_t) { reached("f32_db"); }
void launch_f32_da(const DevTables&, int32_t, int64_t, const float*, const float*, void* const*, int32_t,
                   hipStream_t) { reached("f32_da"); }
void launch_adamw(const AdamwArgs&, int64_t, hipStream_t) { reached("adamw"); }
void launch_gemm_mx8(const GemmMxArgs&, hipStream_t) { reached("gemm_mx8"); }
void launch_quant_act_mx8(const uint16_t*, int64_t, int64_t, uint8_t*, uint8_t*, hipStream_t) {
  reached("quant_act_mx8");
}
void launch_grad_norm(const AdamwArgs&, int64_t, int32_t, hipStream_t) { reached("grad_norm"); }
// the static scratch lives in device code, which this build does not have
hipError_t noalloc_scratch(void**, int* dev) {
  *dev = -1;
  return hipErrorNoDevice;
}
}  // namespace mlora

namespace {

uint64_t g_state = 0x9E3779B97F4A7C15ull;
uint64_t next() {  // xorshift64*
  g_state ^= g_state >> 12;
  g_state ^= g_state << 25;
  g_state ^= g_state >> 27;
  return g_state * 0x2545F4914F6CDD1Dull;
}
int64_t uni(int64_t lo, int64_t hi) { return lo + (int64_t)(next() % (uint64_t)(hi - lo + 1)); }
bool chance(int pct) { return uni(0, 99) < pct; }

long g_ok = 0, g_err = 0;

void expect_error(mlora_status s, const char* what) {
  if (s >= 0) {
    std::fprintf(stderr, "%s: a malformed call returned %d\n", what, (int)s);
    std::abort();
  }
  if (std::strlen(mlora_last_error()) == 0) {
    std::fprintf(stderr, "%s: error without a message\n", what);
    std::abort();
  }
}

int64_t dim() {
  if (chance(8)) return std::vector<int64_t>{0, -64, 63, 100, 1 << 22, INT64_MAX}[uni(0, 5)];
  return 64 * uni(1, 24);
}

mlora_plan_opts opts() {
  mlora_plan_opts o{};
  if (chance(50)) return o;
  o.nano_rows = chance(10) ? (int32_t)uni(-5, 300) : (int32_t)(32 * uni(0, 4));
  o.gemm_rows = chance(10) ? (int32_t)uni(-5, 300) : (chance(80) ? 0 : 256);
  o.n_streams = (int32_t)uni(chance(5) ? -1 : 0, chance(5) ? 9 : 4);
  o.chunk_min = chance(10) ? (int32_t)uni(-4, 5000) : (int32_t)(16 * uni(0, 16));
  o.chunk_max = chance(10) ? (int32_t)uni(-4, 5000) : (int32_t)(256 * uni(0, 8));
  o.chunk_per_rank = (int32_t)uni(chance(5) ? -2 : 0, 16);
  o.w0_layout = (int32_t)uni(chance(5) ? -1 : 0, chance(5) ? 5 : 2);
  o.w0_format = (int32_t)uni(chance(5) ? -1 : 0, chance(5) ? 5 : 2);
  o.act_format = (int32_t)uni(chance(5) ? -1 : 0, chance(5) ? 3 : 1);
  o.wg_overlap = (int32_t)uni(chance(5) ? -1 : 0, chance(5) ? 4 : 2);
  o.grad_accumulate = (int32_t)uni(chance(5) ? -1 : 0, chance(5) ? 3 : 1);
  return o;
}

void exercise(mlora_plan_t p) {
  mlora_plan_info info{};
  if (mlora_plan_get_info(p, &info) != MLORA_OK) std::abort();
  if (info.wg_side != 0 && info.wg_side != 1) std::abort();
  for (int32_t t = -1; t <= MLORA_TAB_COUNT; ++t) {
    size_t bytes = 0;
    mlora_status s = mlora_plan_export(p, t, nullptr, &bytes);
    if (t < 0 || t >= MLORA_TAB_COUNT) {
      expect_error(s, "export of an unknown table");
      continue;
    }
    if (s != MLORA_OK) std::abort();
    std::vector<uint8_t> buf(bytes + 8);
    size_t cap = bytes;
    if (mlora_plan_export(p, t, buf.data(), &cap) != MLORA_OK || cap != bytes) std::abort();
    if (bytes >= 4) {
      size_t small = bytes - 4;
      expect_error(mlora_plan_export(p, t, buf.data(), &small), "export into a small buffer");
      if (small != bytes) std::abort();
    }
  }
  // layer calls: pointers that look valid (aligned, non-NULL) but a
  // workspace that was never uploaded, NULL and misaligned pointers
  void* fake = reinterpret_cast<void*>(uintptr_t(1) << 40);
  void* odd = reinterpret_cast<void*>((uintptr_t(1) << 40) + 8);
  const void* const* pp = reinterpret_cast<const void* const*>(fake);
  void* const* wp = reinterpret_cast<void* const*>(fake);
  const float* sc = reinterpret_cast<const float*>(fake);
  const size_t ws = (size_t)info.workspace_bytes;
  expect_error(mlora_forward(p, fake, fake, pp, pp, sc, fake, fake, fake, ws, nullptr), "forward, not uploaded");
  expect_error(mlora_forward(p, fake, nullptr, pp, pp, sc, fake, fake, fake, ws, nullptr), "forward, NULL W0");
  expect_error(mlora_forward(p, odd, fake, pp, pp, sc, fake, fake, fake, ws, nullptr), "forward, misaligned");
  expect_error(mlora_forward(p, fake, fake, pp, pp, sc, fake, fake, nullptr, ws, nullptr), "forward, NULL ws");
  expect_error(mlora_forward(p, fake, fake, pp, pp, sc, fake, fake, fake, ws ? ws - 1 : 0, nullptr),
               "forward, small ws");
  expect_error(mlora_forward_noalloc(p, fake, nullptr, pp, pp, sc, fake, fake, nullptr), "noalloc, NULL W0");
  expect_error(mlora_forward_noalloc(p, odd, fake, pp, pp, sc, fake, fake, nullptr), "noalloc, misaligned");
  // well-formed arguments: refused for size, or at the scratch lookup (no device in this build)
  expect_error(mlora_forward_noalloc(p, fake, fake, pp, pp, sc, fake, fake, nullptr), "noalloc, no device");
  expect_error(mlora_backward(p, fake, fake, fake, pp, pp, sc, fake, fake, wp, wp, fake, ws, nullptr),
               "backward, not uploaded");
  expect_error(mlora_backward(p, fake, fake, fake, pp, pp, sc, fake, odd, wp, wp, fake, ws, nullptr),
               "backward, misaligned dX");
  expect_error(mlora_backward(p, fake, fake, fake, pp, pp, sc, fake, nullptr, nullptr, wp, fake, ws, nullptr),
               "backward, NULL dA");
  const mlora_adamw_hparams* hp = reinterpret_cast<const mlora_adamw_hparams*>(fake);
  expect_error(mlora_adamw_step(p, hp, wp, wp, pp, pp, wp, wp, wp, wp, nullptr, nullptr, 0, fake, ws, nullptr),
               "adamw, not uploaded");
  expect_error(mlora_adamw_step(p, hp, wp, wp, pp, pp, wp, wp, wp, wp, wp, nullptr, 0, fake, ws, nullptr),
               "adamw, one copy table");
  expect_error(mlora_adamw_step(p, hp, wp, wp, pp, pp, wp, wp, wp, wp, nullptr, nullptr, 2, fake, ws, nullptr),
               "adamw, clip flag");
  expect_error(mlora_plan_upload(p, nullptr, ws, nullptr), "upload, NULL");
  expect_error(mlora_plan_upload(p, odd, ws, nullptr), "upload, misaligned");
  if (ws > 1) expect_error(mlora_plan_upload(p, fake, ws - 1, nullptr), "upload, small");
  if (mlora_profile_enable(p, (int32_t)uni(-1, 1023)) != MLORA_OK) std::abort();
  double ms[MLORA_K_COUNT];
  int64_t cnt[MLORA_K_COUNT];
  if (mlora_profile_read(p, ms, cnt) != MLORA_OK) std::abort();
  for (int k = 0; k < MLORA_K_COUNT; ++k)
    if (cnt[k] != 0) std::abort();
}

void one_case() {
  const int kind = (int)uni(0, 3);  // segments, ids, projections, projections from ids
  int32_t n = (int32_t)(chance(5) ? uni(-2, 0) : uni(1, 40));
  if (chance(2)) n = MLORA_MAX_ADAPTERS + 1;
  const int32_t P = kind >= 2 ? (int32_t)(chance(5) ? uni(-1, 10) : uni(1, 4)) : 1;
  // every array is sized for the n and P passed, so a refusal is the
  // library's own decision, never an out-of-range read by the driver
  const size_t na = (size_t)std::max<int32_t>(n, 0), pa = (size_t)std::max<int32_t>(P, 1);
  std::vector<int32_t> ranks(std::max<size_t>(na * pa, 1));
  for (auto& r : ranks) r = chance(3) ? (int32_t)uni(-3, 400) : (int32_t)uni(1, 256);
  const int64_t d_in = dim(), d_out = dim();
  const mlora_dtype dt = (mlora_dtype)(chance(3) ? uni(-1, 4) : uni(0, 1));
  const mlora_plan_opts o = opts();
  const mlora_plan_opts* op = chance(20) ? nullptr : &o;
  std::vector<int64_t> widths(pa);
  for (auto& w : widths) w = chance(5) ? dim() : 256 * uni(1, 3);
  mlora_plan_t p = nullptr;
  mlora_status s;
  if (kind == 0 || kind == 2) {
    std::vector<int64_t> off(na + 1, 0);
    for (size_t i = 0; i < na; ++i) off[i + 1] = off[i] + (chance(15) ? 0 : uni(1, na > 64 ? 2 : 700));
    if (chance(5) && na > 0) off[(size_t)uni(0, (int64_t)na)] -= uni(1, 50);   // decreasing or negative
    if (chance(3)) off[0] = 7;
    const int64_t* offp = chance(2) ? nullptr : off.data();
    s = kind == 0 ? mlora_plan(n, offp, ranks.data(), d_in, d_out, dt, op, &p)
                  : mlora_plan_multi(n, offp, P, widths.data(), ranks.data(), d_in, dt, op, &p);
  } else {
    const int64_t T = chance(5) ? uni(-3, 0) : uni(0, 3000);
    std::vector<int32_t> ids((size_t)std::max<int64_t>(T, 1));
    for (auto& a : ids) a = (int32_t)(chance(2) ? uni(-2, (int64_t)n + 2) : uni(0, std::max<int64_t>(n - 1, 0)));
    s = kind == 1 ? mlora_plan_from_ids(n, T, ids.data(), ranks.data(), d_in, d_out, dt, op, &p)
                  : mlora_plan_multi_from_ids(n, T, ids.data(), P, widths.data(), ranks.data(), d_in, dt, op, &p);
  }
  if (s == MLORA_OK) {
    ++g_ok;
    exercise(p);
    mlora_plan_destroy(p);
  } else {
    ++g_err;
    if (p != nullptr) {
      std::fprintf(stderr, "a failed plan call wrote *out\n");
      std::abort();
    }
    expect_error(s, "plan");
  }
}

}  // namespace

int main(int argc, char** argv) {
  const long cases = argc > 1 ? std::atol(argv[1]) : 20000;
  g_state ^= argc > 2 ? (uint64_t)std::atoll(argv[2]) * 0x100000001B3ull : 0;
  for (long c = 0; c < cases; ++c) one_case();
  // base transpose: every malformed call is refused before a launch
  void* a = reinterpret_cast<void*>(uintptr_t(1) << 40);
  void* b = reinterpret_cast<void*>(uintptr_t(1) << 41);
  expect_error(mlora_base_transpose(nullptr, b, 64, 64, MLORA_BF16, nullptr), "transpose NULL");
  expect_error(mlora_base_transpose(a, reinterpret_cast<char*>(b) + 4, 64, 64, MLORA_BF16, nullptr), "misaligned");
  expect_error(mlora_base_transpose(a, b, 64, 96, MLORA_BF16, nullptr), "not a multiple of 64");
  expect_error(mlora_base_transpose(a, reinterpret_cast<char*>(a) + 4096, 64, 64, MLORA_BF16, nullptr), "overlap");
  expect_error(mlora_base_transpose(a, b, 64, 64, (mlora_dtype)5, nullptr), "dtype");
  expect_error(mlora_plan_get_info(nullptr, nullptr), "info of NULL");
  mlora_plan_destroy(nullptr);
  std::printf("cases %ld: %ld plans built, %ld refused\n", cases, g_ok, g_err);
  return 0;
}
