"""Dual-weight GLU GEMV for MI355X (gfx950).

``dual_gemv(hidden, gate_w, up_w, out=None)`` computes the decode-time GLU
projection out = bf16(bf16(silu(bf16(h @ Wg^T))) * bf16(h @ Wu^T)) from the
separate gate and up weight matrices, through the C-ABI library built from
``csrc/`` (declared in ``include/glu_gemv.h``).  The library is loaded on the
first call; if it is missing or cannot be loaded the call raises, there is no
fallback path.

``inputs`` holds the seeded synthetic input generators.
"""
from . import inputs  # noqa: F401

__all__ = ["inputs", "dual_gemv", "library"]


def __getattr__(name):
    if name in ("dual_gemv", "library", "status_string", "GluError"):
        from . import api
        return getattr(api, name)
    raise AttributeError(name)
