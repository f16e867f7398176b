"""Host-side checks of the C ABI that need no GPU: the library loads, exports every function the
header declares, the Python binding's struct layouts match the header, and argument validation
returns the documented status codes before anything is launched."""
import ctypes
import json
import os
import re
import subprocess

import pytest

from nonlinear_rnn_solve_amd import api, build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pararnn.h")
DEBUG_HEADER = os.path.join(ROOT, "include", "pararnn_debug.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(api.library_path()):
        build.build(verbose=False)
    return api.load_library()


def declared_functions(header=HEADER):
    txt = open(header).read()
    return sorted(set(re.findall(r"^\s*(?:size_t|pararnn_status|const char\*|int)\s+(pararnn_\w+)\s*\(", txt, re.M)))


def test_library_exports_every_declared_function(lib):
    names = declared_functions()
    assert len(names) == 13, names
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", api.library_path()], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (pararnn_\w+)", out))
    assert exported == set(names)


def test_stress_build_exports_the_same_and_its_debug_query(lib):
    # the look-back stress build: the same entry points plus the one pararnn_debug.h declares
    if not os.path.exists(api.STRESS_LIB_PATH):
        build.build(verbose=False)
    debug = declared_functions(DEBUG_HEADER)
    assert debug == ["pararnn_debug_lookback_depth"]
    out = subprocess.run(["nm", "-D", "--defined-only", api.STRESS_LIB_PATH], capture_output=True, text=True).stdout
    assert set(re.findall(r"\bT (pararnn_\w+)", out)) == set(declared_functions()) | set(debug)
    with api.using_library(api.STRESS_LIB_PATH) as slib:
        assert slib.pararnn_abi_version() == api.ABI_VERSION
    assert api.library_path() != api.STRESS_LIB_PATH


def test_struct_layouts_match_header(tmp_path):
    src = tmp_path / "layout.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "pararnn.h"\n'
                   'int main(void){printf("%zu %zu %zu %zu %zu %zu %zu %zu %zu %zu %zu %zu %zu\\n", sizeof(pararnn_problem),'
                   ' offsetof(pararnn_problem, pre), offsetof(pararnn_problem, s0),'
                   ' offsetof(pararnn_problem, cu_seqlens), offsetof(pararnn_problem, n_seqs),'
                   ' offsetof(pararnn_problem, head_size),'
                   ' sizeof(pararnn_newton_opts),'
                   ' offsetof(pararnn_newton_opts, final_residual), offsetof(pararnn_newton_opts, init_mode),'
                   ' offsetof(pararnn_newton_opts, picard_iters), offsetof(pararnn_newton_opts, fuse_iters),'
                   ' sizeof(pararnn_report),'
                   ' offsetof(pararnn_report, residual)); return 0;}\n')
    exe = tmp_path / "layout"
    subprocess.check_call(["gcc", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)])
    got = [int(x) for x in subprocess.check_output([str(exe)]).split()]
    want = [ctypes.sizeof(api._Problem), api._Problem.pre.offset, api._Problem.s0.offset,
            api._Problem.cu_seqlens.offset, api._Problem.n_seqs.offset, api._Problem.head_size.offset,
            ctypes.sizeof(api._Opts), api._Opts.final_residual.offset, api._Opts.init_mode.offset,
            api._Opts.picard_iters.offset, api._Opts.fuse_iters.offset,
            ctypes.sizeof(api._Report),
            api._Report.residual.offset]
    assert got == want


def _problem(cell=1, dtype=0, B=2, T=100, D=64, ptr=4096, head_size=0):
    p = api._Problem()
    p.cell, p.pre_dtype, p.B, p.T, p.D = cell, dtype, B, T, D
    p.head_size = head_size
    for i in range(4):
        p.pre[i] = ptr
    p.w = p.bias = ptr
    p.s0 = None
    return p


def test_workspace_queries(lib):
    p = _problem()
    n1 = lib.pararnn_newton_workspace_bytes(ctypes.byref(p), None)
    p.T = 100000
    n2 = lib.pararnn_newton_workspace_bytes(ctypes.byref(p), None)
    assert 0 < n1 < n2
    assert lib.pararnn_scan_workspace_bytes(1, 8, 16384, 1024) > 0
    assert lib.pararnn_scan_workspace_bytes(3, 8, 16384, 1024) == 0
    assert lib.pararnn_vjp_workspace_bytes(ctypes.byref(_problem(cell=2))) > 0
    p.D = 0
    assert lib.pararnn_newton_workspace_bytes(ctypes.byref(p), None) == 4096   # empty problem: header only
    # head-wise block GRU: chunk aggregates (hs^2 + hs floats per chunk), entering states and 6 factors per
    # element; the VJP adds the parameter partials
    h = _problem(cell=4, B=4, T=64, D=512, head_size=64)
    nh = lib.pararnn_newton_workspace_bytes(ctypes.byref(h), None)
    assert nh > 6 * 4 * 4 * 64 * 512                                # at least the per-step factors
    assert lib.pararnn_vjp_workspace_bytes(ctypes.byref(h)) > nh
    h.T = 1024
    assert lib.pararnn_newton_workspace_bytes(ctypes.byref(h), None) > 10 * nh
    h.head_size = 8                                                  # not built
    assert lib.pararnn_newton_workspace_bytes(ctypes.byref(h), None) == 0


def test_workspace_grows_with_fused_iterations(lib):
    # one set of look-back words per iteration of the longest fused launch; NULL options size for the most
    p = _problem(B=2, T=4096, D=1024)
    size = lambda o: lib.pararnn_newton_workspace_bytes(ctypes.byref(p), ctypes.byref(o) if o else None)  # noqa
    one = size(api._Opts(3, 0.0, None, 0, 0, 0, 1))
    three = size(api._Opts(3, 0.0, None, 0, 0, 0, 0))     # fixed budget 3: all three in one launch
    eight = size(api._Opts(10, 0.0, None, 0, 0, 0, 0))    # fixed budget 10: PARARNN_MAX_FUSE at a time
    assert one < three < eight == size(None)
    assert (three - one) * 7 == (eight - one) * 2          # the same region size per fused iteration
    assert size(api._Opts(8, 0.0, None, 0, 0, 0, 4)) == size(api._Opts(4, 0.0, None, 0, 0, 0, 0))
    # tolerance mode: the first launch runs the measured K*(T) (3 for the GRU at this length) above the 1e-4
    # bar K*(T) was measured at, else the count tolerance mode reached on the campaign's inputs (4 at 1e-4,
    # 5 at 1e-5 here)
    four = size(api._Opts(4, 0.0, None, 0, 0, 0, 0))
    five = size(api._Opts(5, 0.0, None, 0, 0, 0, 0))
    assert (four - one) * 2 == (three - one) * 3
    assert size(api._Opts(8, 1e-3, None, 0, 0, 0, 0)) == three
    assert size(api._Opts(8, 1e-4, None, 0, 0, 0, 0)) == four
    assert size(api._Opts(8, 1e-5, None, 0, 0, 0, 0)) == five
    assert size(api._Opts(3, 1e-5, None, 0, 0, 0, 0)) == three        # never beyond the budget
    # Picard sweeps, and cells without a fused kernel, use one launch per iteration
    assert size(api._Opts(3, 0.0, None, 0, 0, 1, 0)) == one
    q = _problem(cell=3, B=2, T=4096, D=1024)
    sl = lambda o: lib.pararnn_newton_workspace_bytes(ctypes.byref(q), ctypes.byref(o) if o else None)  # noqa
    assert sl(api._Opts(8, 0.0, None, 0, 0, 0, 0)) == sl(api._Opts(8, 0.0, None, 0, 0, 0, 1)) == sl(None)


def test_validation_codes_without_launching(lib):
    opts = api._Opts(3, 0.0, None, 0)
    ws = ctypes.c_void_p(1 << 20)
    out = ctypes.c_void_p(4096)
    solve = lambda p, o=opts, w=ws, n=1 << 40: lib.pararnn_newton_solve(  # noqa: E731
        ctypes.byref(p), ctypes.byref(o), out, w, n, None, None)
    assert lib.pararnn_newton_solve(None, ctypes.byref(opts), out, ws, 1 << 40, None, None) == -1
    assert solve(_problem(cell=7)) == -1
    assert solve(_problem(dtype=5)) == -1
    assert solve(_problem(B=-1)) == -1
    assert solve(_problem(D=63)) == -2                      # odd D is not built
    p = _problem()
    p.pre[1] = None
    assert solve(p) == -1
    p = _problem()
    p.pre[0] = 4097                                         # misaligned
    assert solve(p) == -1
    assert solve(_problem(), o=api._Opts(-1, 0.0, None, 0)) == -1
    assert solve(_problem(), o=api._Opts(65, 0.0, None, 0)) == -1
    assert solve(_problem(), o=api._Opts(3, 0.0, None, 0, 2)) == -1   # unknown init mode
    assert solve(_problem(), o=api._Opts(3, 0.0, None, 0, 0, -1)) == -1   # negative Picard count
    assert solve(_problem(), o=api._Opts(3, 0.0, None, 0, 0, 0, -1)) == -1   # fused iterations out of range
    assert solve(_problem(), o=api._Opts(3, 0.0, None, 0, 0, 0, api.MAX_FUSE + 1)) == -1
    assert solve(_problem(cell=3), o=api._Opts(0, 0.0, None, 0)) == -1   # sLSTM has no measured budget
    # head-wise block GRU: the head size must divide D; only 16, 32 and 64 are built; no measured budget
    assert solve(_problem(cell=4, head_size=0)) == -1
    assert solve(_problem(cell=4, D=96, head_size=64)) == -1
    assert solve(_problem(cell=4, D=64, head_size=8)) == -2
    assert solve(_problem(cell=4, head_size=64), o=api._Opts(0, 0.0, None, 0)) == -1
    p = _problem()
    p.cu_seqlens, p.n_seqs = 4098, 3                          # offsets not 4-byte aligned
    assert solve(p) == -1
    p.cu_seqlens, p.n_seqs = 4096, -1
    assert solve(p) == -1
    assert solve(_problem(), w=ctypes.c_void_p(0)) == -3
    assert solve(_problem(), w=ctypes.c_void_p(4096 + 8)) == -3   # not 256-byte aligned
    assert solve(_problem(), n=16) == -3
    assert solve(_problem(T=0)) == 0                        # empty problem: no-op
    it = lambda p, k: lib.pararnn_newton_iterate(ctypes.byref(p), ctypes.byref(opts), k, out, ws, 1 << 40, None)  # noqa
    assert it(_problem(), -1) == -1 and it(_problem(), 3) == -1   # k outside [0, max_iters)
    assert lib.pararnn_newton_prepare(ctypes.byref(_problem()), ctypes.byref(opts), ws, 16, None) == -3
    scan = lambda S, dt, a=4096, n=1 << 40, cu=None, ns=0: lib.pararnn_linear_scan(  # noqa: E731
        S, 8, 100, 64, dt, ctypes.c_void_p(a), ctypes.c_void_p(4096), None, cu, ns, ctypes.c_void_p(4096), 0,
        ctypes.c_void_p(1 << 20), n, None)
    assert scan(3, 0) == -1
    assert scan(1, 9) == -1
    assert scan(1, 0, a=0) == -1
    assert scan(1, 0, n=8) == -3
    assert scan(1, 0, cu=ctypes.c_void_p(4097), ns=2) == -1
    assert scan(1, 0, cu=ctypes.c_void_p(4096), ns=-2) == -1
    vjp = lambda p: lib.pararnn_scan_vjp(ctypes.byref(p), None, ctypes.c_void_p(4096),  # noqa: E731
                                         ctypes.c_void_p(4096), None, None, None, None, ws, 1 << 40, None)
    assert vjp(_problem()) == -1                            # trajectory missing


def test_status_strings(lib):
    for s in (0, -1, -2, -3, -4, -5):
        assert lib.pararnn_status_string(s).decode() != "unknown status"
    assert lib.pararnn_abi_version() == api.ABI_VERSION == 6


def test_binding_refuses_cpu_tensors():
    import torch
    a = torch.zeros(1, 8, 4)
    with pytest.raises(ValueError, match="GPU tensor"):
        api.linear_scan(a, a)


def test_automatic_budget_is_the_measured_kstar(lib):
    # the library's K*(T) table must be the one the oracle campaign measured (tests/golden/kstar.json)
    with open(os.path.join(os.path.dirname(__file__), "golden", "kstar.json")) as f:
        gold = json.load(f)
    grid = gold["t_grid"]
    for e in gold["entries"]:
        c, init = api.CELLS[e["cell"]], 1 if e["init"] == "warm" else 0
        assert e["kstar"] is not None
        assert lib.pararnn_newton_budget(c, init, e["T"], 0) == e["kstar"], e
        # between grid points: the next larger point's budget; beyond the grid: one more
        i = grid.index(e["T"])
        lo = grid[i - 1] + 1 if i else 1
        assert lib.pararnn_newton_budget(c, init, lo, 0) == e["kstar"]
        if e["T"] == grid[-1]:
            assert lib.pararnn_newton_budget(c, init, grid[-1] + 1, 0) == e["kstar"] + 1
    assert lib.pararnn_newton_budget(0, 0, 10 ** 9, 0) == 1          # LINEAR: one exact scan
    assert lib.pararnn_newton_budget(1, 0, 100, 5) == 5              # an explicit budget wins
    assert lib.pararnn_newton_budget(1, 2, 100, 0) == -1
    assert lib.pararnn_newton_budget(3, 0, 100, 0) == -1          # sLSTM: no measured budget
    assert lib.pararnn_newton_budget(3, 0, 100, 7) == 7
    assert lib.pararnn_newton_budget(4, 0, 100, 0) == -1
    assert lib.pararnn_newton_budget(1, 0, -1, 0) == -1
    assert lib.pararnn_newton_budget(1, 0, 100, 65) == -1
    assert api.newton_budget("gru", 4096) == lib.pararnn_newton_budget(1, 0, 4096, 0)


def test_noalloc_solve_validates_before_touching_the_gpu(lib):
    # argument errors and a problem too large for the static array are reported before any HIP call
    p = _problem(cell=2, dtype=0, B=4, T=8192, D=2048)
    o = api._Opts(8, 1e-5, None, 0, 0, 0, 8)                  # 8 fused iterations: 320 MiB of words
    assert lib.pararnn_newton_solve_noalloc(ctypes.byref(p), ctypes.byref(o), ctypes.c_void_p(4096), None,
                                            None) == -3
    assert lib.pararnn_newton_solve_noalloc(ctypes.byref(p), ctypes.byref(o), None, None, None) == -1
    o.max_iters = 65
    assert lib.pararnn_newton_solve_noalloc(ctypes.byref(p), ctypes.byref(o), ctypes.c_void_p(4096), None,
                                            None) == -1
    assert lib.pararnn_newton_solve_noalloc(None, ctypes.byref(o), ctypes.c_void_p(4096), None, None) == -1


def test_speculation_length_is_the_measured_tolerance_mode_count(lib):
    # in tolerance mode the library's launch length (seen through the workspace size, which grows by one set
    # of look-back words per fused iteration) is the iteration count the K*(T) campaign's oracle run reached
    # at the nearest of its tolerances at or above tol (tests/golden/kstar.json), K*(T) above 1e-4
    with open(os.path.join(os.path.dirname(__file__), "golden", "kstar.json")) as f:
        gold = json.load(f)
    cells = {"gru": 1, "lstm": 2}
    for e in gold["entries"]:
        p = _problem(cell=cells[e["cell"]], dtype=1 if e["dtype"] == "bf16" else 0, B=gold["B"], T=e["T"], D=gold["D"])
        init = 1 if e["init"] == "warm" else 0
        for tol, key in ((1e-4, "0.0001"), (3e-5, "0.0001"), (1e-5, "1e-05"), (2e-6, "1e-05"), (1e-6, "1e-06"),
                         (1e-9, "1e-06"), (1e-3, None)):
            want = e["kstar"] if key is None else e["stop_iters"][key]
            assert e["kstar"] <= want <= e["kstar"] + 2
            o = api._Opts(8, tol, None, 0, init, 0, 0)
            m = api._Opts(8, tol, None, 0, init, 0, want)
            assert lib.pararnn_newton_workspace_bytes(ctypes.byref(p), ctypes.byref(o)) == \
                lib.pararnn_newton_workspace_bytes(ctypes.byref(p), ctypes.byref(m)), (e["cell"], e["init"], e["T"], tol)

