"""Seeded synthetic score matrices for the exact per-row top-K path.

This module only draws inputs: fp32 score rows, their valid extents and the
poison written outside each row's window.  It holds none of the selection
arithmetic, so both the CPU oracle and the GPU path can take their inputs from
it without sharing any part of the method.

Every row is drawn from its own generator, ``numpy.random.default_rng([cfg,
row, 0])`` (PCG64), as float64 and cast to float32, so a row's content does not
depend on how many other rows are generated.

The five workloads stand in for the captured indexer rows the pages measure
(DeepSeek V3.2 / V4 and GLM-5.3-Flash decode and prefill captures, which are
not public):

1. decode, batch-uniform: 4 x 4096, K=512, N(0, 1);
2. decode varlen: 64 rows, stride 131072, n_valid uniform in [8192, 131072],
   a +/-16 position ramp over N(0, 4) noise, four boundary rows, poisoned pad;
3. prefill packed causal tile: 4 requests x 1024 rows, stride 16640, request
   offsets with every ks % 4, causal ramp lengths 1..16384, K=1024;
4. long position-skewed decode: N=114963 in stride 131072, bulk N(40, 15),
   1% of positions in the last 20% drawn from N(180, 20), K=512 (BS 1 or 8);
5. adversarial tie-heavy decode: 8 x 262144, K=2048, one row recipe per row.

N(mu, s) is read as mean mu and standard deviation s.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

POISON_DECODE = (np.inf, np.nan, np.float32(3e38))
POISON_PREFILL = (np.inf, np.nan, -np.inf)


@dataclasses.dataclass
class Workload:
    """One batch of rows in the layout the C-ABI takes.

    ``logits`` is float32 [num_rows, row_stride].  Decode batches carry
    ``n_valid`` (int32 [num_rows]); prefill batches carry ``row_starts`` and
    ``row_ends`` (int32 [num_rows]).  ``k`` is the selection size.
    """

    name: str
    mode: str  # "decode" or "prefill"
    logits: np.ndarray
    k: int
    n_valid: Optional[np.ndarray] = None
    row_starts: Optional[np.ndarray] = None
    row_ends: Optional[np.ndarray] = None

    @property
    def num_rows(self) -> int:
        return int(self.logits.shape[0])

    @property
    def row_stride(self) -> int:
        return int(self.logits.shape[1])

    def windows(self):
        """(ks, ke) per row after the boundary's clamps (ints, host side)."""
        s = self.row_stride
        if self.mode == "decode":
            nv = np.clip(self.n_valid.astype(np.int64), 0, s)
            return np.zeros_like(nv), nv
        ks = np.clip(self.row_starts.astype(np.int64), 0, s)
        ke = np.clip(self.row_ends.astype(np.int64), 0, s)
        ke = np.maximum(ke, ks)
        return ks, ke

    def valid_lengths(self) -> np.ndarray:
        ks, ke = self.windows()
        return ke - ks

    def algorithmic_bytes(self) -> int:
        """Bytes the selection itself must move for this batch.

        4 B per score of every row longer than K (short rows read no score),
        4 B per output index, and 4 B (decode) or 8 B (prefill) of extents per
        row.
        """
        nv = self.valid_lengths()
        reads = int(4 * nv[nv > self.k].sum())
        writes = 4 * self.k * self.num_rows
        ext = (4 if self.mode == "decode" else 8) * self.num_rows
        return reads + writes + ext


def row_rng(cfg: int, row: int) -> np.random.Generator:
    return np.random.default_rng([cfg, row, 0])


def poison_fill(n: int, pattern) -> np.ndarray:
    """Column-cycled poison values (column c gets pattern[c % len])."""
    pat = np.asarray(pattern, dtype=np.float32)
    return pat[np.arange(n) % len(pat)]


def _poison_row_outside(row: np.ndarray, ks: int, ke: int, pattern) -> None:
    cols = np.arange(row.shape[0])
    mask = (cols < ks) | (cols >= ke)
    row[mask] = poison_fill(row.shape[0], pattern)[mask]


# --------------------------------------------------------------------------
# Workload 1: decode, batch-uniform, 4 x 4096, K=512.
# --------------------------------------------------------------------------
def decode_uniform(rows: int = 4, n: int = 4096, k: int = 512, cfg: int = 1) -> Workload:
    x = np.empty((rows, n), dtype=np.float32)
    for r in range(rows):
        x[r] = row_rng(cfg, r).standard_normal(n).astype(np.float32)
    return Workload("decode_uniform_4x4096_k512", "decode", x, k,
                    n_valid=np.full(rows, n, dtype=np.int32))


# --------------------------------------------------------------------------
# Workload 2: decode varlen, 64 rows, stride 131072, K=2048.
# --------------------------------------------------------------------------
DECODE_VARLEN_FORCED = {7: 2047, 23: 2048, 40: 2049, 63: 0}


def decode_varlen(rows: int = 64, stride: int = 131072, k: int = 2048,
                  lo: int = 8192, hi: int = 131072, cfg: int = 2,
                  forced: Optional[dict] = None) -> Workload:
    if forced is None:
        forced = {r: v for r, v in DECODE_VARLEN_FORCED.items() if r < rows}
    x = np.empty((rows, stride), dtype=np.float32)
    nv = np.empty(rows, dtype=np.int32)
    for r in range(rows):
        g = row_rng(cfg, r)
        n_r = int(g.integers(lo, hi, endpoint=True))
        if r in forced:
            n_r = int(forced[r])
        nv[r] = n_r
        z = g.standard_normal(stride)
        a = 16.0 if r % 2 == 0 else -16.0
        ramp = a * np.arange(stride, dtype=np.float64) / max(n_r, 1)
        row = (4.0 * z + ramp).astype(np.float32)
        _poison_row_outside(row, 0, n_r, POISON_DECODE)
        x[r] = row
    return Workload(f"decode_varlen_{rows}x{stride}_k{k}", "decode", x, k, n_valid=nv)


# --------------------------------------------------------------------------
# Hinted decode step: workload 2's shape with the previous step's top-K.
# --------------------------------------------------------------------------
def decode_step(rows: int = 64, stride: int = 131072, k: int = 2048, lo: int = 8192,
                hi: int = 131072, rho: float = 0.96, cfg: int = 6,
                forced: Optional[dict] = None):
    """A decode step and the previous step's top-K positions as hints.

    Built by construction, without any selection: per long row, a random set
    H of k positions is the previous step's top-K -- its previous scores are
    drawn from the N(0, 1) tail above the 1 - k/n quantile (inverse CDF of a
    uniform on that tail), the other positions' from below it -- and the
    current scores are rho * previous + sqrt(1 - rho^2) * fresh N(0, 1),
    times 4 (workload 2's N(0, 4) scale, without its ramp, which would move
    the top-K away from H).  rho = 0.96 puts the overlap of H with the
    current top-K near the 0.77 the pages report for raw hints on real
    decode captures.  Short rows' hints are their own output (identity, then
    -1).  Returns (Workload, hints int32 [rows, k] in random order)."""
    from scipy.special import ndtri

    if forced is None:
        forced = {r: v for r, v in DECODE_VARLEN_FORCED.items() if r < rows}
    x = np.empty((rows, stride), dtype=np.float32)
    nv = np.empty(rows, dtype=np.int32)
    hints = np.full((rows, k), -1, dtype=np.int32)
    c = float(np.sqrt(1.0 - rho * rho))
    for r in range(rows):
        g = row_rng(cfg, r)
        n_r = int(g.integers(lo, hi, endpoint=True))
        if r in forced:
            n_r = int(forced[r])
        nv[r] = n_r
        row = np.zeros(stride, dtype=np.float64)
        if n_r > k:
            q = 1.0 - k / n_r
            h = g.choice(n_r, size=k, replace=False)
            prev = ndtri(g.uniform(1e-12, q, size=n_r))
            prev[h] = ndtri(g.uniform(q, 1.0, size=k))
            row[:n_r] = 4.0 * (rho * prev + c * g.standard_normal(n_r))
            hints[r] = h.astype(np.int32)
        else:
            row[:n_r] = 4.0 * g.standard_normal(n_r)
            hints[r, :n_r] = np.arange(n_r, dtype=np.int32)
        row = row.astype(np.float32)
        _poison_row_outside(row, 0, n_r, POISON_DECODE)
        x[r] = row
    w = Workload(f"decode_step_hinted_{rows}x{stride}_k{k}", "decode", x, k, n_valid=nv)
    return w, hints


# --------------------------------------------------------------------------
# Block-skip batch: at the block-skip gate's size, rows with locality.
# --------------------------------------------------------------------------
def decode_blockskip(rows: int = 256, stride: int = 131072, k: int = 512, lo: int = 65536,
                     hi: int = 131072, cfg: int = 7, smooth: float = 2.0,
                     span: int = 256) -> Workload:
    """A decode batch at the block-skip gate's size: rows * stride * 4 =
    128 MiB and stride >= 72 K (PR 18122 "Description").  Scores are N(0, 1)
    noise plus a smooth component -- N(0, smooth^2) knots every `span`
    positions, linearly interpolated -- so high scores gather in stretches
    of the row, as attention scores do around the tokens a query attends to
    (the pages measure captured decode rows, which are not public; this
    locality stands in for theirs).  smooth = 0 gives i.i.d. rows, the
    case where block maxima skip least.  n_valid uniform in [lo, hi]; the pad
    is poisoned (+inf, NaN, 3e38)."""
    x = np.empty((rows, stride), dtype=np.float32)
    nv = np.empty(rows, dtype=np.int32)
    knots = stride // span + 2
    grid = np.arange(stride, dtype=np.float64) / span
    for r in range(rows):
        g = row_rng(cfg, r)
        n_r = int(g.integers(lo, hi, endpoint=True))
        nv[r] = n_r
        row = g.standard_normal(stride)
        if smooth > 0.0:
            kv = smooth * g.standard_normal(knots)
            row += np.interp(grid, np.arange(knots, dtype=np.float64), kv)
        row = row.astype(np.float32)
        _poison_row_outside(row, 0, n_r, POISON_DECODE)
        x[r] = row
    tag = "bsk" if smooth > 0.0 else "bsk_iid"
    return Workload(f"decode_{tag}_{rows}x{stride}_k{k}", "decode", x, k, n_valid=nv)


# --------------------------------------------------------------------------
# Workload 3: prefill packed causal tile, 4 x 1024 rows, stride 16640, K=1024.
# --------------------------------------------------------------------------
PREFILL_OFFSETS = (0, 65, 130, 195)


def prefill_causal(requests: int = 4, rows_per_req: int = 1024, max_len: int = 16384,
                   stride: int = 16640, k: int = 1024, cfg: int = 3,
                   offsets=PREFILL_OFFSETS) -> Workload:
    rows = requests * rows_per_req
    x = np.empty((rows, stride), dtype=np.float32)
    ks = np.empty(rows, dtype=np.int32)
    ke = np.empty(rows, dtype=np.int32)
    pois = poison_fill(stride, POISON_PREFILL)
    for q in range(requests):
        for j in range(rows_per_req):
            r = q * rows_per_req + j
            if rows_per_req > 1:
                ln = 1 + (j * (max_len - 1)) // (rows_per_req - 1)
            else:
                ln = max_len
            s = int(offsets[q % len(offsets)])
            e = s + ln
            assert e <= stride
            ks[r], ke[r] = s, e
            row = pois.copy()
            row[s:e] = row_rng(cfg, r).standard_normal(ln).astype(np.float32)
            x[r] = row
    return Workload(f"prefill_causal_{rows}x{stride}_k{k}", "prefill", x, k,
                    row_starts=ks, row_ends=ke)


# --------------------------------------------------------------------------
# Workload 4: long position-skewed decode, N=114963, stride 131072, K=512.
# --------------------------------------------------------------------------
def long_skewed(bs: int = 1, n: int = 114963, stride: int = 131072, k: int = 512,
                cfg: int = 4) -> Workload:
    x = np.empty((bs, stride), dtype=np.float32)
    n_hot = int(round(0.01 * n))
    tail_lo = int(0.8 * n)
    for r in range(bs):
        g = row_rng(cfg, r)
        v = 40.0 + 15.0 * g.standard_normal(n)
        hot = g.choice(np.arange(tail_lo, n), size=n_hot, replace=False)
        v[hot] = 180.0 + 20.0 * g.standard_normal(n_hot)
        row = poison_fill(stride, POISON_DECODE).copy()
        row[:n] = v.astype(np.float32)
        x[r] = row
    return Workload(f"long_skewed_bs{bs}_{n}_k{k}", "decode", x, k,
                    n_valid=np.full(bs, n, dtype=np.int32))


# --------------------------------------------------------------------------
# Workload 5: adversarial tie-heavy decode, 8 x 262144, K=2048.
# --------------------------------------------------------------------------
TIE_ROW_KINDS = (
    "quantised64",      # r0: N(0,1) quantised to 64 levels
    "uniform64",        # r1: floor(64u)/64, a ~4K-member top tie class
    "all_equal",        # r2: every score 0.5
    "two_valued",       # r3: 2.0 with probability 1/256, else 1.0
    "neginf_class",     # r4: 700 N(3,1), 700 signed zeros, the rest -inf
    "zero_class",       # r5: 1000 N(5,1), 30000 signed zeros, the rest N(-5,1)
    "dense_bin40k",     # r6: 1500 U(100,200), 40000 distinct floats near 1.0, rest U(-1,0.5)
    "quantised64_sorted",  # r7: r0's values sorted ascending
)


def tie_row(kind: str, n: int, g: np.random.Generator, cfg: int = 5) -> np.ndarray:
    if kind == "quantised64":
        z = g.standard_normal(n)
        lvl = np.clip(np.floor((z + 4.0) * 8.0), 0, 63)
        return (-4.0 + (lvl + 0.5) / 8.0).astype(np.float32)
    if kind == "uniform64":
        return (np.floor(64.0 * g.random(n)) / 64.0).astype(np.float32)
    if kind == "all_equal":
        return np.full(n, 0.5, dtype=np.float32)
    if kind == "two_valued":
        return np.where(g.random(n) < 1.0 / 256.0, 2.0, 1.0).astype(np.float32)
    if kind == "neginf_class":
        v = np.full(n, -np.inf, dtype=np.float64)
        pos = g.permutation(n)
        a, b = min(700, n), min(1400, n)
        v[pos[:a]] = 3.0 + g.standard_normal(a)
        sign = g.random(b - a) < 0.5
        v[pos[a:b]] = np.where(sign, -0.0, 0.0)
        return v.astype(np.float32)
    if kind == "zero_class":
        v = -5.0 + g.standard_normal(n)
        pos = g.permutation(n)
        a, b = min(1000, n), min(31000, n)
        v[pos[:a]] = 5.0 + g.standard_normal(a)
        sign = g.random(b - a) < 0.5
        v[pos[a:b]] = np.where(sign, -0.0, 0.0)
        return v.astype(np.float32)
    if kind == "dense_bin40k":
        v = g.uniform(-1.0, 0.5, n).astype(np.float32)
        pos = g.permutation(n)
        a, b = min(1500, n), min(41500, n)
        v[pos[:a]] = g.uniform(100.0, 200.0, a).astype(np.float32)
        bits = (np.uint32(0x3F800000) + np.arange(b - a, dtype=np.uint32))
        v[pos[a:b]] = bits.view(np.float32)
        return v
    if kind == "quantised64_sorted":
        return np.sort(tie_row("quantised64", n, row_rng(cfg, 0)))
    raise ValueError(kind)


def tie_heavy(n: int = 262144, k: int = 2048, cfg: int = 5, kinds=TIE_ROW_KINDS) -> Workload:
    x = np.empty((len(kinds), n), dtype=np.float32)
    for r, kind in enumerate(kinds):
        x[r] = tie_row(kind, n, row_rng(cfg, r), cfg=cfg)
    return Workload(f"tie_heavy_{len(kinds)}x{n}_k{k}", "decode", x, k,
                    n_valid=np.full(len(kinds), n, dtype=np.int32))


def config(i: int, **kw) -> Workload:
    """The five workloads by number (1-based)."""
    if i == 1:
        return decode_uniform(**kw)
    if i == 2:
        return decode_varlen(**kw)
    if i == 3:
        return prefill_causal(**kw)
    if i == 4:
        return long_skewed(**kw)
    if i == 5:
        return tie_heavy(**kw)
    raise ValueError(f"no workload {i}")


# --------------------------------------------------------------------------
# Small building blocks for edge-case tests.
# --------------------------------------------------------------------------
def random_decode(rows: int, stride: int, n_valid, k: int, seed: int,
                  dist: str = "normal", pattern=POISON_DECODE) -> Workload:
    """Rows of ``dist`` scores with the given per-row valid lengths."""
    nv = np.asarray(n_valid, dtype=np.int32).reshape(rows)
    x = np.empty((rows, stride), dtype=np.float32)
    for r in range(rows):
        g = np.random.default_rng([seed, r, 1])
        x[r] = _draw(dist, stride, g)
        _poison_row_outside(x[r], 0, int(np.clip(nv[r], 0, stride)), pattern)
    return Workload(f"random_decode_{dist}_{rows}x{stride}_k{k}", "decode", x, k, n_valid=nv)


def random_prefill(starts, ends, stride: int, k: int, seed: int,
                   dist: str = "normal", pattern=POISON_PREFILL) -> Workload:
    ks = np.asarray(starts, dtype=np.int32)
    ke = np.asarray(ends, dtype=np.int32)
    rows = ks.shape[0]
    x = np.empty((rows, stride), dtype=np.float32)
    for r in range(rows):
        g = np.random.default_rng([seed, r, 2])
        x[r] = _draw(dist, stride, g)
        s = int(np.clip(ks[r], 0, stride))
        e = int(np.clip(ke[r], s, stride))
        _poison_row_outside(x[r], s, e, pattern)
    return Workload(f"random_prefill_{dist}_{rows}x{stride}_k{k}", "prefill", x, k,
                    row_starts=ks, row_ends=ke)


def _draw(dist: str, n: int, g: np.random.Generator) -> np.ndarray:
    if dist == "normal":
        return g.standard_normal(n).astype(np.float32)
    if dist == "uniform":
        return g.random(n).astype(np.float32)
    if dist == "levels4":
        return (np.floor(4.0 * g.random(n)) - 1.5).astype(np.float32)
    if dist == "all_equal":
        return np.full(n, 1.25, dtype=np.float32)
    if dist == "two_valued":
        return np.where(g.random(n) < 0.02, 3.0, -1.0).astype(np.float32)
    if dist == "signed_zero":
        v = np.where(g.random(n) < 0.5, -0.0, 0.0)
        hi = g.random(n) < 0.001
        v[hi] = 1.0 + g.random(int(hi.sum()))
        return v.astype(np.float32)
    if dist == "neg_inf":
        v = np.full(n, -np.inf)
        hi = g.random(n) < 0.002
        v[hi] = g.standard_normal(int(hi.sum()))
        return v.astype(np.float32)
    if dist == "pos_inf":
        v = g.standard_normal(n)
        v[g.random(n) < 0.01] = np.inf
        return v.astype(np.float32)
    if dist == "ramp_up":
        return (np.arange(n) * 1e-3 + 0.01 * g.standard_normal(n)).astype(np.float32)
    if dist == "ramp_down":
        return (-np.arange(n) * 1e-3 + 0.01 * g.standard_normal(n)).astype(np.float32)
    if dist == "hidden_peak":
        v = g.standard_normal(n)
        c = int(g.integers(0, max(n - 1, 1)))
        w = max(1, n // 200)
        v[c:c + w] += 50.0
        return v.astype(np.float32)
    if dist == "huge":
        with np.errstate(over="ignore"):  # |z| > 3.4 overflows to +-inf: wanted
            return (g.standard_normal(n) * 1e38).astype(np.float32)
    if dist == "tiny":
        return (g.standard_normal(n) * 1e-42).astype(np.float32)
    raise ValueError(dist)


DISTS = ("normal", "uniform", "levels4", "all_equal", "two_valued", "signed_zero",
         "neg_inf", "pos_inf", "ramp_up", "ramp_down", "hidden_peak", "huge", "tiny")
