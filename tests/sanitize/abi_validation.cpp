// Host-side checks of the C ABI (include/pararnn.h) for a sanitizer build: every entry point's argument
// validation and the workspace queries, driven with invalid and boundary values that must be rejected
// with the documented status before anything reaches the GPU.  Built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code (tests/test_sanitize_cpu.py); exits nonzero on the first
// wrong status, and the sanitizers stop it on any invalid access or undefined operation.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "pararnn.h"

static int g_checks = 0;

#define EXPECT(cond)                                                                 \
  do {                                                                               \
    ++g_checks;                                                                      \
    if (!(cond)) {                                                                   \
      std::fprintf(stderr, "abi_validation: check failed at line %d: %s\n", __LINE__, #cond); \
      return 1;                                                                      \
    }                                                                                \
  } while (0)

static const void* fake(uintptr_t a) { return reinterpret_cast<const void*>(a); }

static pararnn_problem problem(int cell, int dtype, int64_t B, int64_t T, int64_t D) {
  pararnn_problem p;
  std::memset(&p, 0, sizeof p);
  p.cell = cell;
  p.pre_dtype = dtype;
  p.B = B; p.T = T; p.D = D;
  for (int i = 0; i < 4; ++i) p.pre[i] = fake(4096);
  p.w = static_cast<const float*>(fake(4096));
  p.bias = static_cast<const float*>(fake(4096));
  p.head_size = cell == PARARNN_CELL_HEAD_GRU ? 16 : 0;
  return p;
}

static pararnn_newton_opts opts(int K, float tol) {
  pararnn_newton_opts o;
  std::memset(&o, 0, sizeof o);
  o.max_iters = K;
  o.tol = tol;
  return o;
}

int main() {
  const int64_t big = int64_t(1) << 40;
  float* out = static_cast<float*>(const_cast<void*>(fake(1 << 20)));
  void* ws = const_cast<void*>(fake(1 << 22));
  pararnn_report rep;

  // ---- problem validation (shared by every Newton / VJP entry point) ----
  for (int cell = -1; cell <= 5; ++cell) {
    pararnn_problem p = problem(cell, PARARNN_F32, 2, 100, 64);
    const bool ok = cell >= 0 && cell <= 4;
    EXPECT((pararnn_newton_workspace_bytes(&p, nullptr) > 0) == ok);
    EXPECT((pararnn_vjp_workspace_bytes(&p) > 0) == ok);
  }
  EXPECT(pararnn_newton_workspace_bytes(nullptr, nullptr) == 0);
  {
    pararnn_problem p = problem(PARARNN_CELL_DIAG_GRU, 2, 2, 100, 64);   // bad dtype
    EXPECT(pararnn_newton_workspace_bytes(&p, nullptr) == 0);
  }
  const int64_t shapes[][3] = {{-1, 10, 8}, {1, -1, 8}, {1, 10, -2}, {big * 2, 1, 2}, {1, 1, big * 2},
                               {big, 1, big}, {big, big, 2}, {1, INT64_MAX / 4, 2}, {INT64_MAX, INT64_MAX, INT64_MAX},
                               {int64_t(1) << 20, int64_t(1) << 20, int64_t(1) << 20}};
  for (const auto& s : shapes) {
    pararnn_problem p = problem(PARARNN_CELL_DIAG_GRU, PARARNN_F32, s[0], s[1], s[2]);
    pararnn_newton_opts o = opts(3, 0.0f);
    EXPECT(pararnn_newton_workspace_bytes(&p, &o) == 0);
    EXPECT(pararnn_vjp_workspace_bytes(&p) == 0);
    EXPECT(pararnn_newton_solve(&p, &o, out, ws, 1 << 30, nullptr, nullptr) == PARARNN_ERR_INVALID_ARG);
    EXPECT(pararnn_newton_solve_noalloc(&p, &o, out, nullptr, nullptr) == PARARNN_ERR_INVALID_ARG);
    EXPECT(pararnn_scan_vjp(&p, out, out, out, nullptr, nullptr, nullptr, nullptr, ws, 1 << 30, nullptr) ==
           PARARNN_ERR_INVALID_ARG);
    EXPECT(pararnn_scan_workspace_bytes(1, s[0], s[1], s[2]) == 0);
    EXPECT(pararnn_linear_scan(1, s[0], s[1], s[2], PARARNN_F32, fake(4096), fake(4096), nullptr, nullptr, 0, out,
                               0, ws, 1 << 30, nullptr) == PARARNN_ERR_INVALID_ARG);
  }
  {
    // large but valid sizes: the queries must not overflow
    const int64_t ok_shapes[][3] = {{1, int64_t(1) << 30, 2}, {int64_t(1) << 20, 1 << 10, 64}, {3, 1, big},
                                    {1, 1, 2}, {7, 13, 6}};
    for (const auto& s : ok_shapes) {
      for (int cell = 0; cell <= 3; ++cell) {
        pararnn_problem p = problem(cell, PARARNN_BF16, s[0], s[1], s[2]);
        EXPECT(pararnn_newton_workspace_bytes(&p, nullptr) > 0);
        EXPECT(pararnn_vjp_workspace_bytes(&p) > 0);
      }
      EXPECT(pararnn_scan_workspace_bytes(2, s[0], s[1], s[2]) > 0);
    }
  }
  {
    pararnn_problem p = problem(PARARNN_CELL_DIAG_LSTM, PARARNN_F32, 2, 100, 63);   // odd D
    pararnn_newton_opts o = opts(3, 0.0f);
    EXPECT(pararnn_newton_solve(&p, &o, out, ws, 1 << 30, nullptr, nullptr) == PARARNN_ERR_UNSUPPORTED);
  }
  {
    pararnn_problem p = problem(PARARNN_CELL_HEAD_GRU, PARARNN_F32, 2, 100, 64);
    pararnn_newton_opts o = opts(3, 0.0f);
    p.head_size = 0;
    EXPECT(pararnn_newton_solve(&p, &o, out, ws, 1 << 30, nullptr, nullptr) == PARARNN_ERR_INVALID_ARG);
    p.head_size = 24;   // does not divide D
    EXPECT(pararnn_newton_solve(&p, &o, out, ws, 1 << 30, nullptr, nullptr) == PARARNN_ERR_INVALID_ARG);
    p.head_size = 8;    // divides D, not built
    EXPECT(pararnn_newton_solve(&p, &o, out, ws, 1 << 30, nullptr, nullptr) == PARARNN_ERR_UNSUPPORTED);
    p.head_size = 32;
    o.max_iters = 0;    // no measured budget for this cell
    EXPECT(pararnn_newton_solve(&p, &o, out, ws, 1 << 30, nullptr, nullptr) == PARARNN_ERR_INVALID_ARG);
  }
  {
    pararnn_problem p = problem(PARARNN_CELL_DIAG_GRU, PARARNN_BF16, 2, 100, 64);
    pararnn_newton_opts o = opts(3, 1e-5f);
    p.pre[2] = nullptr;
    EXPECT(pararnn_newton_solve(&p, &o, out, ws, 1 << 30, nullptr, nullptr) == PARARNN_ERR_INVALID_ARG);
    p.pre[2] = fake(4097);   // misaligned
    EXPECT(pararnn_newton_solve(&p, &o, out, ws, 1 << 30, nullptr, nullptr) == PARARNN_ERR_INVALID_ARG);
    p.pre[2] = fake(4096);
    p.w = nullptr;
    EXPECT(pararnn_newton_solve(&p, &o, out, ws, 1 << 30, nullptr, nullptr) == PARARNN_ERR_INVALID_ARG);
    p.w = static_cast<const float*>(fake(4096));
    p.s0 = static_cast<const float*>(fake(4100));
    EXPECT(pararnn_newton_solve(&p, &o, out, ws, 1 << 30, nullptr, nullptr) == PARARNN_ERR_INVALID_ARG);
    p.s0 = nullptr;
    p.cu_seqlens = static_cast<const int32_t*>(fake(4098));
    p.n_seqs = 3;
    EXPECT(pararnn_newton_solve(&p, &o, out, ws, 1 << 30, nullptr, nullptr) == PARARNN_ERR_INVALID_ARG);
    p.cu_seqlens = static_cast<const int32_t*>(fake(4096));
    p.n_seqs = -1;
    EXPECT(pararnn_newton_solve(&p, &o, out, ws, 1 << 30, nullptr, nullptr) == PARARNN_ERR_INVALID_ARG);
    p.cu_seqlens = nullptr;
  }

  // ---- Newton options, output and workspace ----
  {
    pararnn_problem p = problem(PARARNN_CELL_DIAG_GRU, PARARNN_F32, 2, 100, 64);
    EXPECT(pararnn_newton_solve(&p, nullptr, out, ws, 1 << 30, nullptr, nullptr) == PARARNN_ERR_INVALID_ARG);
    const int bad_k[] = {-1, PARARNN_MAX_ITERS + 1, 1 << 30};
    for (int k : bad_k) {
      pararnn_newton_opts o = opts(k, 0.0f);
      EXPECT(pararnn_newton_solve(&p, &o, out, ws, 1 << 30, nullptr, nullptr) == PARARNN_ERR_INVALID_ARG);
      EXPECT(pararnn_newton_solve_noalloc(&p, &o, out, nullptr, nullptr) == PARARNN_ERR_INVALID_ARG);
    }
    pararnn_newton_opts o = opts(3, 0.0f);
    o.init_mode = 2;
    EXPECT(pararnn_newton_solve(&p, &o, out, ws, 1 << 30, nullptr, nullptr) == PARARNN_ERR_INVALID_ARG);
    o = opts(3, 0.0f);
    o.picard_iters = -1;
    EXPECT(pararnn_newton_solve(&p, &o, out, ws, 1 << 30, nullptr, nullptr) == PARARNN_ERR_INVALID_ARG);
    o.picard_iters = PARARNN_MAX_ITERS + 1;
    EXPECT(pararnn_newton_solve(&p, &o, out, ws, 1 << 30, nullptr, nullptr) == PARARNN_ERR_INVALID_ARG);
    o = opts(3, 0.0f);
    o.fuse_iters = PARARNN_MAX_FUSE + 1;
    EXPECT(pararnn_newton_solve(&p, &o, out, ws, 1 << 30, nullptr, nullptr) == PARARNN_ERR_INVALID_ARG);
    o.fuse_iters = -1;
    EXPECT(pararnn_newton_solve(&p, &o, out, ws, 1 << 30, nullptr, nullptr) == PARARNN_ERR_INVALID_ARG);
    o = opts(3, 0.0f);
    EXPECT(pararnn_newton_solve(&p, &o, nullptr, ws, 1 << 30, nullptr, nullptr) == PARARNN_ERR_INVALID_ARG);
    EXPECT(pararnn_newton_solve(&p, &o, out + 1, ws, 1 << 30, nullptr, nullptr) == PARARNN_ERR_INVALID_ARG);
    o.init_guess = out + 1;
    EXPECT(pararnn_newton_solve(&p, &o, out, ws, 1 << 30, nullptr, nullptr) == PARARNN_ERR_INVALID_ARG);
    o.init_guess = nullptr;
    const size_t need = pararnn_newton_workspace_bytes(&p, &o);
    EXPECT(need > 0 && need <= pararnn_newton_workspace_bytes(&p, nullptr));
    EXPECT(pararnn_newton_solve(&p, &o, out, nullptr, need, nullptr, nullptr) == PARARNN_ERR_WORKSPACE);
    EXPECT(pararnn_newton_solve(&p, &o, out, static_cast<char*>(ws) + 128, need, nullptr, nullptr) ==
           PARARNN_ERR_WORKSPACE);
    EXPECT(pararnn_newton_solve(&p, &o, out, ws, need - 1, nullptr, nullptr) == PARARNN_ERR_WORKSPACE);
    EXPECT(pararnn_newton_prepare(&p, &o, ws, need - 1, nullptr) == PARARNN_ERR_WORKSPACE);
    EXPECT(pararnn_newton_iterate(&p, &o, 0, out, ws, need - 1, nullptr) == PARARNN_ERR_WORKSPACE);
    EXPECT(pararnn_newton_iterate(&p, &o, -1, out, ws, need, nullptr) == PARARNN_ERR_INVALID_ARG);
    EXPECT(pararnn_newton_iterate(&p, &o, 3, out, ws, need, nullptr) == PARARNN_ERR_INVALID_ARG);
    // a problem too large for the allocation-free solve's static array, at every launch length asked for
    pararnn_problem q = problem(PARARNN_CELL_DIAG_LSTM, PARARNN_F32, 4, 8192, 2048);
    o = opts(8, 1e-5f);
    o.fuse_iters = 8;
    EXPECT(pararnn_newton_solve_noalloc(&q, &o, out, nullptr, nullptr) == PARARNN_ERR_WORKSPACE);
  }
  {
    // empty problems: no launch, the report filled
    pararnn_problem p = problem(PARARNN_CELL_DIAG_LSTM, PARARNN_F32, 3, 0, 64);
    pararnn_newton_opts o = opts(3, 1e-5f);
    std::memset(&rep, 0x5a, sizeof rep);
    EXPECT(pararnn_newton_solve(&p, &o, nullptr, nullptr, 0, nullptr, &rep) == PARARNN_OK);
    EXPECT(rep.iters == 0 && rep.converged == 1 && rep.n_residual == 0);
    EXPECT(pararnn_newton_solve_noalloc(&p, &o, nullptr, nullptr, &rep) == PARARNN_OK);
    EXPECT(pararnn_newton_workspace_bytes(&p, &o) > 0);
    EXPECT(pararnn_scan_vjp(&p, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0,
                            nullptr) == PARARNN_OK);
  }

  // ---- linear scan ----
  {
    EXPECT(pararnn_scan_workspace_bytes(0, 1, 10, 8) == 0 && pararnn_scan_workspace_bytes(3, 1, 10, 8) == 0);
    const size_t need = pararnn_scan_workspace_bytes(1, 2, 1000, 64);
    EXPECT(need > 0 && pararnn_scan_workspace_bytes(1, 2, 100000, 64) > need);
    EXPECT(pararnn_linear_scan(3, 2, 1000, 64, PARARNN_F32, fake(4096), fake(4096), nullptr, nullptr, 0, out, 0, ws,
                               need, nullptr) == PARARNN_ERR_INVALID_ARG);
    EXPECT(pararnn_linear_scan(1, 2, 1000, 64, 7, fake(4096), fake(4096), nullptr, nullptr, 0, out, 0, ws, need,
                               nullptr) == PARARNN_ERR_INVALID_ARG);
    EXPECT(pararnn_linear_scan(1, 2, 1000, 64, PARARNN_F32, nullptr, fake(4096), nullptr, nullptr, 0, out, 0, ws,
                               need, nullptr) == PARARNN_ERR_INVALID_ARG);
    EXPECT(pararnn_linear_scan(1, 2, 1000, 64, PARARNN_F32, fake(4096), fake(4097), nullptr, nullptr, 0, out, 0, ws,
                               need, nullptr) == PARARNN_ERR_INVALID_ARG);
    EXPECT(pararnn_linear_scan(1, 2, 1000, 64, PARARNN_F32, fake(4096), fake(4096), nullptr,
                               static_cast<const int32_t*>(fake(4096)), -3, out, 0, ws, need, nullptr) ==
           PARARNN_ERR_INVALID_ARG);
    EXPECT(pararnn_linear_scan(1, 2, 1000, 64, PARARNN_F32, fake(4096), fake(4096), nullptr, nullptr, 0, out, 0, ws,
                               need - 1, nullptr) == PARARNN_ERR_WORKSPACE);
    EXPECT(pararnn_linear_scan(1, 2, 0, 64, PARARNN_F32, nullptr, nullptr, nullptr, nullptr, 0, nullptr, 0, nullptr,
                               0, nullptr) == PARARNN_OK);
  }

  // ---- VJP ----
  {
    pararnn_problem p = problem(PARARNN_CELL_DIAG_GRU, PARARNN_F32, 2, 100, 64);
    const size_t need = pararnn_vjp_workspace_bytes(&p);
    EXPECT(need > 0);
    EXPECT(pararnn_scan_vjp(&p, nullptr, out, out, nullptr, nullptr, nullptr, nullptr, ws, need, nullptr) ==
           PARARNN_ERR_INVALID_ARG);
    EXPECT(pararnn_scan_vjp(&p, out, out, out + 1, nullptr, nullptr, nullptr, nullptr, ws, need, nullptr) ==
           PARARNN_ERR_INVALID_ARG);
    EXPECT(pararnn_scan_vjp(&p, out, out, out, nullptr, nullptr, nullptr, out + 1, ws, need, nullptr) ==
           PARARNN_ERR_INVALID_ARG);
    EXPECT(pararnn_scan_vjp(&p, out, out, out, nullptr, nullptr, nullptr, nullptr, ws, need - 1, nullptr) ==
           PARARNN_ERR_WORKSPACE);
  }

  // ---- budget, status strings, version ----
  EXPECT(pararnn_newton_budget(PARARNN_CELL_DIAG_GRU, PARARNN_INIT_ZERO, 131072, 0) == 3);
  EXPECT(pararnn_newton_budget(PARARNN_CELL_DIAG_GRU, PARARNN_INIT_ZERO, 131073, 0) == 4);
  EXPECT(pararnn_newton_budget(PARARNN_CELL_LINEAR, PARARNN_INIT_WARM, 5, 0) == 1);
  EXPECT(pararnn_newton_budget(PARARNN_CELL_DIAG_LSTM, PARARNN_INIT_ZERO, 100, 7) == 7);
  EXPECT(pararnn_newton_budget(PARARNN_CELL_DIAG_SLSTM, PARARNN_INIT_ZERO, 100, 0) == PARARNN_ERR_INVALID_ARG);
  EXPECT(pararnn_newton_budget(9, PARARNN_INIT_ZERO, 100, 0) == PARARNN_ERR_INVALID_ARG);
  EXPECT(pararnn_newton_budget(PARARNN_CELL_DIAG_GRU, 5, 100, 0) == PARARNN_ERR_INVALID_ARG);
  EXPECT(pararnn_newton_budget(PARARNN_CELL_DIAG_GRU, PARARNN_INIT_ZERO, -1, 0) == PARARNN_ERR_INVALID_ARG);
  EXPECT(pararnn_newton_budget(PARARNN_CELL_DIAG_GRU, PARARNN_INIT_ZERO, INT64_MAX, 0) >= 1);
  EXPECT(pararnn_newton_budget(PARARNN_CELL_DIAG_GRU, PARARNN_INIT_ZERO, 100, PARARNN_MAX_ITERS + 1) ==
         PARARNN_ERR_INVALID_ARG);
  for (int s = -7; s <= 2; ++s) EXPECT(pararnn_status_string(s) != nullptr && std::strlen(pararnn_status_string(s)) > 0);
  EXPECT(pararnn_abi_version() == PARARNN_ABI_VERSION);

  std::printf("abi_validation: %d checks passed\n", g_checks);
  return 0;
}
