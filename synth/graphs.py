"""Seeded CSR sparsity patterns.

Degree multisets are drawn either iid (small graphs) or from stratified
quantiles of a stated law, q_i = (i + 0.5) / N, which makes them deterministic
and free of sampling noise; a seeded permutation then assigns them to rows.
Columns are uniform without replacement within a row and sorted ascending.
"""

from __future__ import annotations

import hashlib
from dataclasses import dataclass

import numpy as np


@dataclass
class CSR:
    """A CSR pattern: ``row_ptr`` int32 [n_rows + 1], ``col_idx`` int32 [nnz]."""

    n_rows: int
    n_cols: int
    row_ptr: np.ndarray
    col_idx: np.ndarray

    @property
    def nnz(self) -> int:
        return int(self.row_ptr[-1])

    def degrees(self) -> np.ndarray:
        return np.diff(self.row_ptr.astype(np.int64))

    def row_of_edge(self) -> np.ndarray:
        """Row id of every stored entry (int64 [nnz])."""
        return np.repeat(np.arange(self.n_rows, dtype=np.int64), self.degrees())


def _row_ptr_from_degrees(deg: np.ndarray) -> np.ndarray:
    rp = np.zeros(len(deg) + 1, dtype=np.int64)
    np.cumsum(deg, out=rp[1:])
    if rp[-1] >= 2**31:
        raise ValueError("nnz does not fit int32 indices")
    return rp.astype(np.int32)


# --------------------------------------------------------------------------
# degree laws
# --------------------------------------------------------------------------

def _quantiles(n: int) -> np.ndarray:
    return (np.arange(n, dtype=np.float64) + 0.5) / n


def powerlaw_degrees(n: int, gamma: float, kmax: int) -> np.ndarray:
    """Stratified quantiles of the discrete law P(k) ~ k^-gamma on 1..kmax.

    Degree i is the smallest k whose CDF reaches q_i (sorted ascending).
    """
    k = np.arange(1, kmax + 1, dtype=np.float64)
    p = k ** (-gamma)
    cdf = np.cumsum(p) / p.sum()
    return np.searchsorted(cdf, _quantiles(n), side="left").astype(np.int64) + 1


def powerlaw_gamma_for_nnz(n: int, kmax: int, target_nnz: int) -> float:
    """Bisect gamma so that the quantile degrees of ``powerlaw_degrees`` sum
    as close as possible to ``target_nnz`` (sum is decreasing in gamma)."""
    lo, hi = 0.5, 3.0
    for _ in range(60):
        mid = 0.5 * (lo + hi)
        s = int(powerlaw_degrees(n, mid, kmax).sum())
        if s > target_nnz:
            lo = mid
        else:
            hi = mid
    return hi


def lognormal_degrees(n: int, mu: float, sigma: float) -> np.ndarray:
    """Stratified quantiles of a log-normal law, rounded to nearest, at least 1."""
    from scipy.stats import norm

    x = np.exp(mu + sigma * norm.ppf(_quantiles(n)))
    return np.maximum(1, np.rint(x)).astype(np.int64)


def rank_size_lengths(n_nonempty: int, cap: int, target_nnz: int) -> np.ndarray:
    """Rank-size row lengths L(r) = min(cap, max(1, floor(A / r^2))), r = 1..n.

    ``A`` is bisected so that the lengths sum to at most ``target_nnz``; the
    remainder is spread +1 over the singleton rows of highest rank so that the
    sum is exactly ``target_nnz``.  r^-2 is the rank-size form of a Zipf density
    with exponent 1.5.
    """
    r = np.arange(1, n_nonempty + 1, dtype=np.float64)

    def lengths(a: float) -> np.ndarray:
        return np.minimum(cap, np.maximum(1, np.floor(a / (r * r)))).astype(np.int64)

    lo, hi = 1.0, 1e15
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if lengths(mid).sum() > target_nnz:
            hi = mid
        else:
            lo = mid
    out = lengths(lo)
    rem = int(target_nnz - out.sum())
    if rem < 0:
        raise RuntimeError("bisection overshoot")
    if rem:
        ones = np.nonzero(out == 1)[0]
        if len(ones) < rem:
            raise RuntimeError("not enough singleton rows to absorb the remainder")
        out[ones[:rem]] += 1
    return out


# --------------------------------------------------------------------------
# column sampling
# --------------------------------------------------------------------------

def sample_columns(deg: np.ndarray, n_cols: int, rng: np.random.Generator,
                   heavy: int = 64) -> np.ndarray:
    """Per row, ``deg[i]`` distinct columns uniform over [0, n_cols), sorted.

    Rows longer than ``heavy`` are drawn one by one without replacement.  Short
    rows are drawn together with replacement; the few rows that drew a
    duplicate are redrawn one by one without replacement.  Every row's column
    set is therefore a uniform random subset of its size.
    """
    deg = np.asarray(deg, dtype=np.int64)
    if (deg > n_cols).any():
        raise ValueError("a row is longer than the number of columns")
    n = len(deg)
    rp = np.zeros(n + 1, dtype=np.int64)
    np.cumsum(deg, out=rp[1:])
    col = np.empty(int(rp[-1]), dtype=np.int32)

    light = deg <= heavy
    light_rows = np.nonzero(light & (deg > 0))[0]
    if len(light_rows):
        ld = deg[light_rows]
        total = int(ld.sum())
        draws = rng.integers(0, n_cols, size=total, dtype=np.int64)
        owner = np.repeat(np.arange(len(light_rows), dtype=np.int64), ld)
        keys = owner * n_cols + draws
        keys.sort()
        vals = (keys - owner * n_cols).astype(np.int32)
        dup = np.zeros(total, dtype=bool)
        same = keys[1:] == keys[:-1]
        dup[1:] = same
        bad_owner = np.unique(owner[dup])
        # scatter the sorted light rows into place
        starts = rp[light_rows]
        lrp = np.zeros(len(light_rows) + 1, dtype=np.int64)
        np.cumsum(ld, out=lrp[1:])
        dest = np.repeat(starts - lrp[:-1], ld) + np.arange(total, dtype=np.int64)
        col[dest] = vals
        redo = light_rows[bad_owner]
    else:
        redo = np.zeros(0, dtype=np.int64)

    heavy_rows = np.nonzero(~light)[0]
    for i in np.concatenate([heavy_rows, redo]).astype(np.int64):
        d = int(deg[i])
        c = rng.choice(n_cols, size=d, replace=False, shuffle=False)
        c.sort()
        col[rp[i]:rp[i + 1]] = c
    return col


def csr_from_degrees(deg: np.ndarray, n_cols: int, rng: np.random.Generator) -> CSR:
    deg = np.asarray(deg, dtype=np.int64)
    col = sample_columns(deg, n_cols, rng)
    return CSR(len(deg), n_cols, _row_ptr_from_degrees(deg), col)


def poisson_graph(n: int, mean: float, rng: np.random.Generator,
                  n_cols: int | None = None) -> CSR:
    """iid Poisson(mean) in-degrees, uniform sorted unique columns."""
    n_cols = n if n_cols is None else n_cols
    deg = np.minimum(rng.poisson(mean, size=n), n_cols)
    return csr_from_degrees(deg, n_cols, rng)


def configuration_model_symmetric(deg: np.ndarray, rng: np.random.Generator) -> CSR:
    """Symmetric simple graph from target degrees via the configuration model.

    One stub per unit of degree (one stub is dropped from the largest node if
    the total is odd), a seeded permutation pairs the stubs, self-loops are
    dropped, every pair is stored in both directions and duplicate pairs are
    merged.  Realized degrees are therefore at most the targets.
    """
    deg = np.asarray(deg, dtype=np.int64).copy()
    n = len(deg)
    if deg.sum() % 2:
        deg[np.argmax(deg)] -= 1
    stubs = np.repeat(np.arange(n, dtype=np.int32), deg)
    rng.shuffle(stubs)
    a = stubs[0::2]
    b = stubs[1::2]
    keep = a != b
    a = a[keep].astype(np.int64)
    b = b[keep].astype(np.int64)
    del stubs, keep
    m = len(a)
    keys = np.empty(2 * m, dtype=np.int64)
    np.multiply(a, n, out=keys[:m])
    keys[:m] += b
    np.multiply(b, n, out=keys[m:])
    keys[m:] += a
    del a, b
    keys.sort()
    first = np.empty(len(keys), dtype=bool)
    first[:1] = True
    np.not_equal(keys[1:], keys[:-1], out=first[1:])
    keys = keys[first]
    del first
    rows = keys // n
    counts = np.bincount(rows, minlength=n)
    np.multiply(rows, n, out=rows)
    np.subtract(keys, rows, out=keys)
    cols = keys.astype(np.int32)
    del keys, rows
    return CSR(n, n, _row_ptr_from_degrees(counts), cols)


def window_global_pattern(L: int, window: int, n_global: int) -> CSR:
    """Sliding window plus global tokens, as CSR over L tokens.

    Row i holds the columns [i - window/2, i + window/2) clipped to [0, L),
    the global columns [0, n_global), and the global rows [0, n_global) hold
    every column.  Sorted and unique.
    """
    half = window // 2
    deg = np.empty(L, dtype=np.int64)
    cols = []
    for i in range(L):
        if i < n_global:
            c = np.arange(L, dtype=np.int32)
        else:
            lo, hi = max(0, i - half), min(L, i + half)
            w = np.arange(lo, hi, dtype=np.int32)
            g = np.arange(0, min(n_global, lo), dtype=np.int32)
            c = np.concatenate([g, w])
        deg[i] = len(c)
        cols.append(c)
    return CSR(L, L, _row_ptr_from_degrees(deg), np.concatenate(cols))


def random_small_graph(n_rows: int, n_cols: int, density: float,
                       rng: np.random.Generator, empty_frac: float = 0.0,
                       allow_dup: bool = False) -> CSR:
    """Small Bernoulli pattern for parity and pin tests; optional empty rows and
    (unsorted) duplicate entries."""
    mask = rng.random((n_rows, n_cols)) < density
    if empty_frac > 0:
        mask[rng.random(n_rows) < empty_frac] = False
    rows, cols = np.nonzero(mask)
    if allow_dup and len(rows):
        k = max(1, len(rows) // 5)
        pick = rng.integers(0, len(rows), size=k)
        rows = np.concatenate([rows, rows[pick]])
        cols = np.concatenate([cols, cols[pick]])
        order = np.lexsort((rng.random(len(rows)), rows))
        rows, cols = rows[order], cols[order]
    counts = np.bincount(rows, minlength=n_rows)
    return CSR(n_rows, n_cols, _row_ptr_from_degrees(counts), cols.astype(np.int32))


def pattern_hash(csr: CSR) -> str:
    """Stable 64-bit hex digest of (n_rows, n_cols, row_ptr, col_idx)."""
    h = hashlib.blake2b(digest_size=8)
    h.update(np.array([csr.n_rows, csr.n_cols], dtype=np.int64).tobytes())
    h.update(np.ascontiguousarray(csr.row_ptr, dtype=np.int32).tobytes())
    h.update(np.ascontiguousarray(csr.col_idx, dtype=np.int32).tobytes())
    return h.hexdigest()
