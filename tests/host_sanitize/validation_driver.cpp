// Drives every entry point of include/moe.h through the host validation
// layer with the launches stubbed out: valid calls must reach exactly one
// stage launch (or none where the entry point says so), each invalid call
// must return its status before any launch.  Built and run under the
// address and undefined-behaviour sanitizers by tests/test_host_sanitize.py;
// extreme sizes (INT_MAX tokens, capacities near 2^31, huge hidden sizes)
// exercise the overflow guards.
#include <climits>
#include <cstdint>
#include <cstdio>

#include "moe.h"

namespace moe {
extern int g_launches;
}

static int g_fail = 0, g_cases = 0;

static void expect(const char* what, int got, int want, int launches) {
  ++g_cases;
  const bool launched_ok = want == MOE_OK ? true : launches == 0;
  if (got != want || !launched_ok) {
    std::printf("FAIL %s: status %d (want %d), launches %d\n", what, got, want,
                launches);
    ++g_fail;
  }
}

#define CASE(what, want, call)                  \
  do {                                          \
    moe::g_launches = 0;                        \
    const int st_ = (call);                     \
    expect(what, st_, want, moe::g_launches);   \
  } while (0)

// fake, 256-aligned, far-apart device addresses (never dereferenced)
static void* P(int i) { return (void*)(uintptr_t)(0x100000000ull * (i + 1)); }
template <typename T>
static T* Q(int i) { return (T*)P(i); }

int main() {
  // ---------------------------------------------------------- sizes
  CASE("capacity", MOE_OK, moe_rows_capacity(100, 16, 2, 4) == 248 ? 0 : 1);
  CASE("capacity int overflow", MOE_OK,
       moe_rows_capacity(INT_MAX, 256, 16, 128) == 0 ? 0 : 1);
  CASE("workspace T=0", MOE_OK, moe_workspace_bytes(0, 8, 2) == 0 ? 0 : 1);
  CASE("workspace E too large", MOE_OK,
       moe_workspace_bytes(10, MOE_MAX_EXPERTS + 1, 2) == 0 ? 0 : 1);
  CASE("workspace huge T", MOE_OK,
       moe_workspace_bytes(INT_MAX, MOE_MAX_EXPERTS, MOE_MAX_TOPK) > 0 ? 0 : 1);
  CASE("noalloc bytes", MOE_OK,
       moe_noalloc_scratch_bytes(65536, 512, 16) <= MOE_NOALLOC_SCRATCH_BYTES
           ? 0 : 1);
  CASE("gemm workspace", MOE_OK,
       moe_expert_gemm_workspace_bytes(1u << 20, 256) > 0 ? 0 : 1);
  for (int s = -10; s <= 1; ++s)
    CASE("status string", MOE_OK, moe_status_string(s) != nullptr ? 0 : 1);

  // ---------------------------------------------------------- route
  const size_t wsb = moe_workspace_bytes(100, 16, 2);
  auto route = [&](const void* x, int xdt, int T, int H, int E, int k,
                   int pad, void* ws, size_t wsb_) {
    return moe_route(x, xdt, T, H, P(1), E, nullptr, k, pad, Q<int32_t>(2),
                     Q<float>(3), Q<int32_t>(4), Q<int32_t>(5), nullptr, ws,
                     wsb_, nullptr);
  };
  CASE("route ok", MOE_OK, route(P(0), MOE_BF16, 100, 256, 16, 2, 4, P(6), wsb));
  CASE("route T=0", MOE_OK, route(P(0), MOE_BF16, 0, 256, 16, 2, 4, P(6), 0));
  CASE("route INT_MAX tokens", MOE_ERR_SHAPE,
       route(P(0), MOE_BF16, INT_MAX, 256, 16, 16, 4, P(6), wsb));
  CASE("route huge H", MOE_ERR_WORKSPACE,
       route(P(0), MOE_BF16, 100, INT_MAX - 7, 16, 2, 4, P(6), 0));
  CASE("route H%8", MOE_ERR_SHAPE,
       route(P(0), MOE_BF16, 100, 12, 16, 2, 4, P(6), wsb));
  CASE("route k>E", MOE_ERR_SHAPE,
       route(P(0), MOE_BF16, 100, 256, 4, 5, 4, P(6), wsb));
  CASE("route pad INT_MAX", MOE_ERR_SHAPE,
       route(P(0), MOE_BF16, 100, 256, 16, 2, INT_MAX, P(6), wsb));
  CASE("route dtype", MOE_ERR_DTYPE,
       route(P(0), MOE_FP8_E4M3, 100, 256, 16, 2, 4, P(6), wsb));
  CASE("route align", MOE_ERR_ALIGN,
       route((char*)P(0) + 8, MOE_BF16, 100, 256, 16, 2, 4, P(6), wsb));
  CASE("route null ws", MOE_ERR_NULL,
       route(P(0), MOE_BF16, 100, 256, 16, 2, 4, nullptr, wsb));
  CASE("route alias", MOE_ERR_ALIAS,
       route(P(0), MOE_BF16, 100, 256, 16, 2, 4, P(0), wsb));

  // ---------------------------------------------------------- plan
  CASE("plan ok", MOE_OK,
       moe_plan(Q<int32_t>(0), 100, 2, 16, 4, Q<int32_t>(1), Q<int32_t>(2),
                P(3), wsb, nullptr));
  CASE("plan small ws", MOE_ERR_WORKSPACE,
       moe_plan(Q<int32_t>(0), 100, 2, 16, 4, Q<int32_t>(1), Q<int32_t>(2),
                P(3), 16, nullptr));

  // ---------------------------------------------------------- dispatch
  const size_t cap = moe_rows_capacity(100, 16, 2, 4);
  auto disp = [&](int T, int H, int pdt, float* sc, size_t cap_, void* ws) {
    return moe_dispatch(P(0), MOE_BF16, T, H, Q<int32_t>(1), 2, 16, 4,
                        Q<int32_t>(2), Q<int32_t>(3), ws, wsb, pdt, P(5),
                        cap_, sc, Q<int32_t>(6), Q<int32_t>(7), nullptr);
  };
  CASE("dispatch ok", MOE_OK, disp(100, 256, MOE_BF16, nullptr, cap, P(4)));
  CASE("dispatch fp8 ok", MOE_OK,
       disp(100, 256, MOE_FP8_E4M3, Q<float>(8), cap, P(4)));
  CASE("dispatch cap", MOE_ERR_CAPACITY,
       disp(100, 256, MOE_BF16, nullptr, cap - 1, P(4)));
  CASE("dispatch cap 2^62", MOE_ERR_SHAPE,
       disp(100, 256, MOE_BF16, nullptr, (size_t)1 << 62, P(4)));
  CASE("dispatch null ws", MOE_ERR_NULL,
       disp(100, 256, MOE_BF16, nullptr, cap, nullptr));
  auto dna = [&](int T, int E, int k, size_t cap_) {
    return moe_dispatch_noalloc(P(0), MOE_BF16, T, 8, Q<int32_t>(1), k, E, 4,
                                Q<int32_t>(2), Q<int32_t>(3), MOE_BF16, P(5),
                                cap_, nullptr, Q<int32_t>(6), Q<int32_t>(7),
                                nullptr);
  };
  CASE("noalloc ok", MOE_OK, dna(100, 16, 2, cap));
  CASE("noalloc scratch", MOE_ERR_SCRATCH,
       dna(300000, 16, 8, moe_rows_capacity(300000, 16, 8, 4)));
  CASE("noalloc cap", MOE_ERR_CAPACITY, dna(100, 16, 2, cap - 1));

  auto rd = [&](int T, int H, int pdt, float* sc, size_t cap_, void* ws,
                void* rows) {
    return moe_route_dispatch(P(0), MOE_BF16, T, H, P(1), 16, nullptr, 2, 4,
                              Q<int32_t>(2), Q<float>(3), Q<int32_t>(4),
                              Q<int32_t>(5), nullptr, ws,
                              moe_workspace_bytes(T > 0 ? T : 1, 16, 2), pdt,
                              rows, cap_, sc, Q<int32_t>(8), Q<int32_t>(9),
                              nullptr);
  };
  CASE("route_dispatch ok", MOE_OK,
       rd(100, 256, MOE_BF16, nullptr, cap, P(6), P(7)));
  CASE("route_dispatch fp8 ok", MOE_OK,
       rd(100, 256, MOE_FP8_E4M3, Q<float>(10), cap, P(6), P(7)));
  CASE("route_dispatch cap", MOE_ERR_CAPACITY,
       rd(100, 256, MOE_BF16, nullptr, cap - 1, P(6), P(7)));
  CASE("route_dispatch alias rows/ws", MOE_ERR_ALIAS,
       rd(100, 256, MOE_BF16, nullptr, cap, P(6), P(6)));
  CASE("route_dispatch alias rows/x", MOE_ERR_ALIAS,
       rd(100, 256, MOE_BF16, nullptr, cap, P(6), P(0)));
  CASE("route_dispatch INT_MAX", MOE_ERR_SHAPE,
       rd(INT_MAX, 256, MOE_BF16, nullptr, cap, P(6), P(7)));

  auto rd1 = [&](int T, int xdt, size_t cap_) {
    return moe_route_dispatch_one_launch(
        P(0), xdt, T, 256, P(1), 16, nullptr, 2, 4, Q<int32_t>(2),
        Q<float>(3), Q<int32_t>(4), Q<int32_t>(5), nullptr, P(6),
        moe_workspace_bytes(T > 0 ? T : 1, 16, 2), xdt, P(7), cap_, nullptr,
        Q<int32_t>(8), Q<int32_t>(9), nullptr);
  };
  CASE("route_dispatch_one_launch ok", MOE_OK, rd1(100, MOE_BF16, cap));
  CASE("route_dispatch_one_launch fp32", MOE_ERR_DTYPE,
       rd1(100, MOE_F32, cap));
  CASE("route_dispatch_one_launch T", MOE_ERR_SHAPE,
       rd1(257, MOE_BF16, moe_rows_capacity(257, 16, 2, 4)));
  CASE("route_dispatch_one_launch INT_MAX", MOE_ERR_SHAPE,
       rd1(INT_MAX, MOE_BF16, cap));

  // ---------------------------------------------------------- combine
  auto comb = [&](int T, int H, size_t y_rows, void* res_in, void* res_out,
                  void* rnr, void* out) {
    return moe_combine_residual(P(0), MOE_BF16, H, y_rows, Q<int32_t>(1),
                                Q<float>(2), T, 8, P(3), res_in, res_out, rnr,
                                out, MOE_BF16, nullptr);
  };
  CASE("combine ok", MOE_OK, comb(100, 256, 1000, P(4), P(5), P(6), nullptr));
  CASE("combine in place", MOE_OK,
       comb(100, 256, 1000, P(4), P(4), P(6), nullptr));
  CASE("combine routed", MOE_OK,
       comb(100, 256, 1000, nullptr, nullptr, nullptr, P(7)));
  CASE("combine T=0", MOE_OK, comb(0, 256, 0, P(4), P(5), P(6), nullptr));
  // a y larger than the address space wraps the overlap arithmetic (size_t):
  // any status is acceptable, the sanitizers must stay quiet
  (void)comb(100, 256, (size_t)1 << 62, P(4), P(5), P(6), nullptr);
  CASE("combine partial alias", MOE_ERR_ALIAS,
       comb(100, 256, 1000, P(4), (char*)P(4) + 256, nullptr, nullptr));
  CASE("combine k", MOE_ERR_SHAPE,
       moe_combine_residual(P(0), MOE_BF16, 256, 1000, Q<int32_t>(1),
                            Q<float>(2), 100, 17, nullptr, P(4), P(5), P(6),
                            nullptr, MOE_BF16, nullptr));

  // ---------------------------------------------------------- the rest
  CASE("farskip ok", MOE_OK, moe_farskip_aux(P(0), P(1), P(2), 100, 256,
                                             nullptr));
  CASE("farskip alias", MOE_ERR_ALIAS,
       moe_farskip_aux(P(0), P(1), P(1), 100, 256, nullptr));
  CASE("combine backward ok", MOE_OK,
       moe_combine_backward(P(0), P(1), MOE_BF16, 256, 1000, Q<int32_t>(2),
                            Q<float>(3), 100, 8, P(4), Q<float>(5), nullptr));
  CASE("dispatch backward ok", MOE_OK,
       moe_dispatch_backward(P(0), MOE_BF16, 256, 1000, Q<int32_t>(1), 100, 8,
                             P(2), MOE_F32, nullptr));
  const size_t gcap = 4096;
  const size_t gws = moe_expert_gemm_workspace_bytes(gcap, 16);
  CASE("gemm ok", MOE_OK,
       moe_expert_gemm_fp8(P(0), Q<float>(1), 1024, gcap, Q<int32_t>(2),
                           Q<int32_t>(3), 16, P(4), Q<float>(5), 512, P(6),
                           MOE_BF16, P(7), gws, nullptr));
  CASE("gemm K*cap overflow", MOE_ERR_SHAPE,
       moe_expert_gemm_fp8(P(0), Q<float>(1), 8192, (size_t)1 << 20,
                           Q<int32_t>(2), Q<int32_t>(3), 16, P(4),
                           Q<float>(5), 512, P(6), MOE_BF16, P(7), gws,
                           nullptr));
  CASE("fixture ok", MOE_OK,
       moe_expert_fixture(P(0), MOE_BF16, nullptr, 256, Q<int32_t>(1),
                          Q<int32_t>(2), 16, Q<float>(3), 1000, P(4),
                          MOE_BF16, nullptr));

  std::printf("%s: %d cases, %d failed\n", g_fail ? "FAIL" : "ok", g_cases,
              g_fail);
  return g_fail ? 1 : 0;
}
