"""CPU oracle for the exact per-row top-K -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  The product path (``exact_row_top_amd``) never
does, and nothing here imports the product path.

Contents:
- ``build()`` compiles ``oracle_topk.c`` with gcc into ``liboracle_topk.so``.
- ``topk_decode`` / ``topk_prefill`` run the plain C oracle (full sort by IEEE
  value, ties by smaller position; see the C file's header for the passages it
  follows).
- ``brute_force_row`` is an independent pure-Python definition used to pin the
  C oracle on small rows.
- ``check_rows`` is the tie-aware comparison the GPU results must pass.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle_topk.c")
_LIB = os.path.join(_HERE, "liboracle_topk.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle (plain gcc -O2, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-D_POSIX_C_SOURCE=200809L",
                               "-fno-fast-math", "-shared", "-fPIC", "-pthread",
                               _SRC, "-o", tmp])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        lib.oracle_topk_decode.restype = ctypes.c_int64
        lib.oracle_topk_decode.argtypes = [P, ctypes.c_int64, P, ctypes.c_int64,
                                           ctypes.c_int32, P, ctypes.c_int32]
        lib.oracle_topk_prefill.restype = ctypes.c_int64
        lib.oracle_topk_prefill.argtypes = [P, ctypes.c_int64, P, P, ctypes.c_int64,
                                            ctypes.c_int32, P, ctypes.c_int32]
        lib.oracle_topk_window.restype = ctypes.c_int
        lib.oracle_topk_window.argtypes = [P, ctypes.c_int64, ctypes.c_int32, P, P]
        lib.oracle_online_cores.restype = ctypes.c_int32
        _lib = lib
    return _lib


def online_cores() -> int:
    return int(_load().oracle_online_cores())


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data


def topk_decode(logits: np.ndarray, n_valid: np.ndarray, k: int,
                nthreads: int = 0, return_rejected: bool = False):
    """Exact top-k per row of a decode batch (host arrays)."""
    lib = _load()
    x, xp = _c(logits, np.float32)
    assert x.ndim == 2
    nv, nvp = _c(n_valid, np.int32)
    assert nv.shape == (x.shape[0],)
    out = np.empty((x.shape[0], k), dtype=np.int32)
    rej = lib.oracle_topk_decode(xp, x.shape[1], nvp, x.shape[0], k,
                                 out.ctypes.data, nthreads)
    return (out, int(rej)) if return_rejected else out


def topk_prefill(logits: np.ndarray, row_starts: np.ndarray, row_ends: np.ndarray,
                 k: int, nthreads: int = 0, return_rejected: bool = False):
    """Exact top-k per row of a prefill batch, windows [row_starts, row_ends)."""
    lib = _load()
    x, xp = _c(logits, np.float32)
    assert x.ndim == 2
    ks, ksp = _c(row_starts, np.int32)
    ke, kep = _c(row_ends, np.int32)
    assert ks.shape == ke.shape == (x.shape[0],)
    out = np.empty((x.shape[0], k), dtype=np.int32)
    rej = lib.oracle_topk_prefill(xp, x.shape[1], ksp, kep, x.shape[0], k,
                                  out.ctypes.data, nthreads)
    return (out, int(rej)) if return_rejected else out


def topk_window(w: np.ndarray, k: int) -> np.ndarray:
    """The C oracle's core on one window with any k >= 1."""
    lib = _load()
    x, xp = _c(w, np.float32)
    out = np.empty(k, dtype=np.int32)
    scratch = np.empty(max(x.shape[0], 1) * 8, dtype=np.uint8)
    rc = lib.oracle_topk_window(xp, x.shape[0], k, out.ctypes.data, scratch.ctypes.data)
    if rc:
        raise ValueError("window holds a NaN (outside the contract)")
    return out


def varlen_n_valid(kv_lens, num_rows: int, next_n: int, compress_ratio: int,
                   row_stride: int) -> np.ndarray:
    """Valid length of each row of the varlen / MTP decode form.

    "Block-skip fast path ..." (PR 18122), run_varlen commit: kv_lens holds one
    total cache length per request (uncompressed token space); row r belongs
    to request r // next_n and sees
        n = (kv_len - next_n + r % next_n + 1) // compress_ratio
    positions; a request with kv_len < next_n has empty rows (its "next_n"
    query tokens are not all in the cache yet).  The boundary then clamps n
    to the row stride.  Plain Python integers, one row at a time.
    """
    out = np.zeros(num_rows, dtype=np.int64)
    for r in range(num_rows):
        kv = int(kv_lens[r // next_n])
        n = 0 if kv < next_n else (kv - next_n + r % next_n + 1) // compress_ratio
        out[r] = min(max(n, 0), row_stride)
    return out


def topk_varlen(logits: np.ndarray, kv_lens, next_n: int, compress_ratio: int, k: int):
    """Exact top-k per row of a varlen / MTP decode batch: the decode form on
    the windows ``varlen_n_valid`` gives."""
    x = np.asarray(logits)
    nv = varlen_n_valid(kv_lens, x.shape[0], next_n, compress_ratio, x.shape[1])
    return topk_decode(x, nv.astype(np.int32), k)


def topk_workload(w) -> np.ndarray:
    """Oracle output for a ``workloads.Workload``."""
    if w.mode == "decode":
        return topk_decode(w.logits, w.n_valid, w.k)
    return topk_prefill(w.logits, w.row_starts, w.row_ends, w.k)


# ---------------------------------------------------------------------------
# Independent pure-Python definition (small rows only).
# ---------------------------------------------------------------------------
def brute_force_row(values, k: int):
    """Top-k of a list of Python floats by the plain definition.

    Sort positions by (value descending, position ascending) with Python's
    float comparisons (-0.0 == 0.0 there), take k; pad with -1 / identity for
    short rows.
    """
    n = len(values)
    if n <= k:
        return list(range(n)) + [-1] * (k - n)
    order = sorted(range(n), key=lambda i: (-float(values[i]), i))
    return order[:k]


# ---------------------------------------------------------------------------
# Tie-aware checker.
# ---------------------------------------------------------------------------
def _canon_bits(v: np.ndarray) -> np.ndarray:
    """fp32 bit patterns with -0 mapped to +0."""
    v = np.asarray(v, dtype=np.float32).copy()
    v[v == 0] = 0.0
    return v.view(np.uint32)


def check_row(window: np.ndarray, got: np.ndarray, want: np.ndarray, k: int) -> Optional[str]:
    """None if ``got`` is a correct top-k of ``window``, else a reason.

    Short rows (nv <= k) must equal the identity + -1 pad exactly.  Long rows
    must hold k distinct positions in [0, nv) whose canonical fp32 values, as
    a multiset, equal the oracle's bit for bit -- i.e. indices may differ from
    the oracle's only inside the k-th value's tie class.
    """
    nv = window.shape[0]
    got = np.asarray(got, dtype=np.int64)
    want = np.asarray(want, dtype=np.int64)
    if got.shape != (k,):
        return f"shape {got.shape} != ({k},)"
    if nv <= k:
        if not np.array_equal(got, want):
            bad = np.nonzero(got != want)[0]
            return f"short row (nv={nv}) differs at {bad[:8].tolist()}: got {got[bad[:8]].tolist()}"
        return None
    if got.min() < 0 or got.max() >= nv:
        return f"index out of [0,{nv}): min {got.min()} max {got.max()}"
    if np.unique(got).shape[0] != k:
        return "duplicate indices"
    gv = np.sort(_canon_bits(window[got]).view(np.float32))
    wv = np.sort(_canon_bits(window[want]).view(np.float32))
    if not np.array_equal(gv.view(np.uint32), wv.view(np.uint32)):
        diff = np.nonzero(gv.view(np.uint32) != wv.view(np.uint32))[0]
        return f"value multiset differs at {diff.shape[0]} slots (first {diff[:4].tolist()})"
    return None


def check_rows(w, got: np.ndarray, want: Optional[np.ndarray] = None, rows=None) -> list:
    """Check every row (or ``rows``) of a Workload; returns [(row, reason)]."""
    if want is None:
        want = topk_workload(w)
    ks, ke = w.windows()
    bad = []
    it = range(w.num_rows) if rows is None else rows
    for r in it:
        win = w.logits[r, int(ks[r]):int(ke[r])]
        why = check_row(win, got[r], want[r], w.k)
        if why:
            bad.append((int(r), why))
    return bad
