"""MI355X-native ParaRNN hot path: Newton solves of diagonal GRU/LSTM recurrences
with parallel scans over time, and the reverse-scan VJP.

The compute lives in ``libpararnn.so`` (hand-written HIP for gfx950, C ABI in
``include/pararnn.h``).  This package is a thin binding over it.  Importing the
package loads nothing; the first call into the binding loads the library and
fails loudly if it is missing.  ``synth`` (seeded inputs) has no dependency on
the library or on torch.
"""
_API = ("CELLS", "NewtonDivergenceError", "PararnnError", "library_path", "linear_scan", "load_library",
        "newton_solve", "scan_vjp", "newton_workspace_bytes", "scan_workspace_bytes", "vjp_workspace_bytes",
        "NewtonReport")


def __getattr__(name):
    if name in _API:
        from . import api
        return getattr(api, name)
    raise AttributeError(name)


__all__ = list(_API)
