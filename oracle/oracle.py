"""Python side of the CPU oracle for exact row-wise Top-K.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module; the selector library never does, and
this module imports nothing from the selector package.

`topk` runs the C oracle (topk_oracle.c: a complete descending sort of every
valid row prefix, the plain definition of the operator contract in
"Sample-Guided Exact Top-K Selection for Long-Context Sparse Attention",
Sec. 2.1).  `check_rows` compares a selector's output with that result under
the set-valued exactness criterion of Sec. 6.1, Eq. 30:

  * L <= K: slots [0, L) hold exactly 0..L-1 in ascending order and slots
    [L, K) hold -1 (the contract only asks for every valid index; writing them
    ascending is this library's documented layout);
  * L > K: K distinct indices in [0, L); the multiset of their float32 bit
    patterns equals the oracle's; every index strictly above the K-th value is
    selected.  Ties at the K-th value may resolve to any indices.

Together these imply Eq. 30 (no unselected valid value exceeds a selected
one); `check_rows` also asserts Eq. 30 numerically on each row.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "topk_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile topk_oracle.c with gcc (no fast-math, so subnormals compare exactly)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
                               "-fno-fast-math", "-o", tmp, _SRC])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        lib.oracle_topk.restype = ctypes.c_int
        lib.oracle_topk.argtypes = [
            ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
            ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p]
        lib.oracle_coarse_check.restype = ctypes.c_int64
        lib.oracle_coarse_check.argtypes = [ctypes.c_uint32, ctypes.c_int64, ctypes.c_void_p,
                                            ctypes.c_int32, ctypes.c_void_p]
        _lib = lib
    return _lib


def default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


@dataclass
class OracleResult:
    k: int
    rows: int              # rows computed: min(m_live, M)
    sel_bits: np.ndarray   # [rows, K] uint32, descending value order
    sel_idx: np.ndarray    # [rows, K] int32
    n_strict: np.ndarray   # [rows] int32
    lengths: np.ndarray    # [rows] int64, clamped valid lengths


def topk(x: np.ndarray, ke: np.ndarray, k: int, m_live: int | None = None,
         threads: int | None = None) -> OracleResult:
    """Exact Top-K of every row r < min(m_live, M) of x[:, :ke[r]]."""
    if x.dtype != np.float32 or x.ndim != 2:
        raise TypeError("x must be a 2-D float32 array")
    if x.strides[1] != 4:
        raise ValueError("x rows must be contiguous")
    m, n = x.shape
    stride = x.strides[0] // 4 if m > 0 else n
    ke = np.ascontiguousarray(ke, dtype=np.int32)
    if ke.shape != (m,):
        raise ValueError("ke must have one entry per row")
    rows = m if m_live is None else max(0, min(int(m_live), m))
    sel_bits = np.zeros((max(rows, 0), k), dtype=np.uint32)
    sel_idx = np.full((max(rows, 0), k), -2, dtype=np.int32)
    n_strict = np.zeros(max(rows, 0), dtype=np.int32)
    if rows > 0:
        rc = _load().oracle_topk(x.ctypes.data, m, n, stride, ke.ctypes.data, rows, k,
                                 threads or default_threads(), sel_bits.ctypes.data,
                                 sel_idx.ctypes.data, n_strict.ctypes.data)
        if rc != 0:
            raise RuntimeError("oracle_topk failed with code %d" % rc)
    lengths = np.clip(ke[:rows].astype(np.int64), 0, n)
    return OracleResult(k, rows, sel_bits, sel_idx, n_strict, lengths)


def check_row(out_row: np.ndarray, x_row: np.ndarray, L: int, k: int, sel_bits: np.ndarray,
              sel_idx: np.ndarray, n_strict: int) -> str | None:
    """Returns None when out_row is an exact answer for the row, else a reason."""
    out_row = np.asarray(out_row, dtype=np.int64)
    if out_row.shape != (k,):
        return "wrong output length %s" % (out_row.shape,)
    if L <= k:
        want = np.concatenate([np.arange(L), np.full(k - L, -1)])
        if not np.array_equal(out_row, want):
            bad = int(np.flatnonzero(out_row != want)[0])
            return "sentinel layout differs at slot %d: got %d want %d" % (
                bad, out_row[bad], want[bad])
        return None
    if out_row.min() < 0 or out_row.max() >= L:
        return "index out of range [0, %d): min %d max %d" % (L, out_row.min(), out_row.max())
    if np.unique(out_row).size != k:
        return "duplicate indices (%d distinct of %d)" % (np.unique(out_row).size, k)
    bits = x_row[:L].view(np.uint32)
    got = np.sort(bits[out_row])
    want = np.sort(sel_bits.astype(np.uint32))
    if not np.array_equal(got, want):
        d = int(np.flatnonzero(got != want)[0])
        return "value multiset differs (first at sorted slot %d: got %08x want %08x)" % (
            d, got[d], want[d])
    strict = sel_idx[:n_strict]
    if n_strict and not np.isin(strict, out_row).all():
        miss = strict[~np.isin(strict, out_row)]
        return "%d indices strictly above the K-th value are missing (e.g. %d)" % (
            miss.size, miss[0])
    # Eq. 30 numerically: min selected >= max unselected
    vals = x_row[:L]
    mask = np.ones(L, dtype=bool)
    mask[out_row] = False
    if mask.any():
        if not (vals[out_row].min() >= vals[mask].max()):
            return "Eq. 30 violated: min selected %r < max unselected %r" % (
                vals[out_row].min(), vals[mask].max())
    return None


def check_rows(out: np.ndarray, x: np.ndarray, res: OracleResult,
               rows=None, max_report: int = 5) -> list[str]:
    """Checks rows (default: all computed rows); returns failure descriptions."""
    fails = []
    it = range(res.rows) if rows is None else rows
    for r in it:
        msg = check_row(out[r], x[r], int(res.lengths[r]), res.k, res.sel_bits[r],
                        res.sel_idx[r], int(res.n_strict[r]))
        if msg is not None:
            fails.append("row %d (L=%d): %s" % (r, int(res.lengths[r]), msg))
            if len(fails) >= max_report:
                break
    return fails


def coarse_check(start: int, got: np.ndarray, threads: int | None = None) -> tuple[int, int | None]:
    """Compares got[i] with c(x) of float32 pattern start + i (Sec. 4.2, Eq. 11;
    the host CPU's IEEE round-to-nearest-even binary16 conversion), NaN
    patterns skipped.  Returns (mismatches, first mismatching pattern or None).
    Raises RuntimeError when the host CPU has no F16C conversion."""
    got = np.ascontiguousarray(got, dtype=np.uint16)
    if start < 0 or start + got.size > 1 << 32:
        raise ValueError("pattern range outside 32 bits")
    first = np.zeros(1, dtype=np.uint32)
    r = _load().oracle_coarse_check(start, got.size, got.ctypes.data,
                                    threads or default_threads(), first.ctypes.data)
    if r == -1:
        raise RuntimeError("the host CPU has no F16C conversion")
    if r < 0:
        raise ValueError("oracle_coarse_check: bad arguments")
    return int(r), (int(first[0]) if r else None)
