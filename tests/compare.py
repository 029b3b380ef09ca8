"""Bitwise comparison of float32 results.

Finite values and infinities must match bit for bit (so +0 and -0 differ). NaN outputs match any NaN: the IEEE
operations fix that the result is NaN, not which payload or sign a given implementation propagates.
"""

from __future__ import annotations

import numpy as np


def same_bits(got: np.ndarray, want: np.ndarray) -> np.ndarray:
    got = np.ascontiguousarray(got, dtype=np.float32)
    want = np.ascontiguousarray(want, dtype=np.float32)
    if got.shape != want.shape:
        raise AssertionError(f"shape {got.shape} != {want.shape}")
    eq = got.view(np.uint32) == want.view(np.uint32)
    return eq | (np.isnan(got) & np.isnan(want))


def mismatch_report(got: np.ndarray, want: np.ndarray, ok: np.ndarray, limit: int = 8) -> str:
    bad = np.argwhere(~ok)
    lines = [f"{len(bad)} of {ok.size} elements differ"]
    g = np.ascontiguousarray(got, dtype=np.float32)
    w = np.ascontiguousarray(want, dtype=np.float32)
    for idx in bad[:limit]:
        t = tuple(int(v) for v in idx)
        lines.append(f"  at {t}: got {g[t]!r} (0x{int(g.view(np.uint32)[t]):08x}) "
                     f"want {w[t]!r} (0x{int(w.view(np.uint32)[t]):08x})")
    return "\n".join(lines)


def assert_same_bits(got: np.ndarray, want: np.ndarray, what: str = "") -> None:
    ok = same_bits(got, want)
    if not ok.all():
        raise AssertionError((what + ": " if what else "") + mismatch_report(got, want, ok))
