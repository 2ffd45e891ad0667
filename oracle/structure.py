"""Integer bookkeeping of the schedule path, written from its definitions
(test infrastructure only).

* Degree histogram: the input features the AutoSAGE page's scheduler reads
  (Abstract: performance varies with degree skew and feature width).  Row i has
  degree d_i = row_ptr[i+1] - row_ptr[i]; bucket 0 holds the empty rows and
  bucket b >= 1 the rows with 2^(b-1) <= d_i < 2^b.  Per bucket: the number of
  rows and the sum of their degrees; plus the maximum degree.

* Merge-path partition: the nnz-balanced split of the work.  Walk the rows'
  entries and the rows' ends as one merged sequence in which the end of row i
  comes right after the row's last entry; chunk c owns the items
  [c * D, (c + 1) * D) of that sequence.  Its start is the pair (x, y) = (row
  ends, entries) that precede item c * D.

* Transpose: the CSR pattern of A^T, i.e. the entries regrouped by column,
  each column listing its rows in increasing order (a stable sort by column).

* Column-part segment format: the composition of a column partition and a
  row compaction (the SparseTIR page, abstract: formats compose, and no one
  format serves every input).  Columns are cut into P equal parts, part of
  column c = c // ceil(n_cols / P); segment (p, r) is the list of row r's
  entries (original order) whose columns lie in part p; the non-empty
  segments are listed by part, then row; each row lists its segments by part.
  A row with fewer than whole_below entries stays whole: one segment in an
  extra part P, after all the column parts.

* FNV-1a 64: the published Fowler-Noll-Vo hash (offset basis
  0xcbf29ce484222325, prime 0x100000001b3; per byte: xor, then multiply).
"""

from __future__ import annotations

import numpy as np

N_BUCKETS = 33


def degree_histogram(row_ptr):
    """Returns (counts int64[33], nnz int64[33], max_degree)."""
    rp = np.asarray(row_ptr, dtype=np.int64)
    deg = rp[1:] - rp[:-1]
    counts = np.zeros(N_BUCKETS, dtype=np.int64)
    sums = np.zeros(N_BUCKETS, dtype=np.int64)
    # bucket = number of powers of two 1, 2, 4, ... that are <= d (0 for d = 0)
    b = np.zeros(len(deg), dtype=np.int64)
    for k in range(N_BUCKETS - 1):
        b += deg >= (1 << k)
    counts = np.bincount(b, minlength=N_BUCKETS).astype(np.int64)
    sums = np.bincount(b, weights=deg, minlength=N_BUCKETS).astype(np.int64)
    mx = int(deg.max()) if len(deg) else 0
    return counts, sums, mx


def merge_path_partition(row_ptr, items_per_chunk: int):
    """(x, y) int32 arrays of length n_chunks + 1.

    x(d) = number of rows i whose end precedes item d, i.e. whose
    (i + 1) + row_ptr[i + 1] <= d; y(d) = d - x(d).
    """
    rp = np.asarray(row_ptr, dtype=np.int64)
    n, nnz = len(rp) - 1, int(rp[-1])
    total = n + nnz
    n_chunks = max(1, -(-total // items_per_chunk))
    d = np.minimum(np.arange(n_chunks + 1, dtype=np.int64) * items_per_chunk, total)
    key = rp[1:] + np.arange(1, n + 1, dtype=np.int64)  # strictly increasing
    x = np.searchsorted(key, d, side="right")
    y = d - x
    return x.astype(np.int32), y.astype(np.int32)


def merge_path_bruteforce(row_ptr, items_per_chunk: int):
    """Same partition by walking the merged sequence item by item (tiny inputs)."""
    rp = [int(v) for v in row_ptr]
    n, nnz = len(rp) - 1, rp[-1]
    xs, ys = [0], [0]
    x = y = 0
    count = 0
    while x < n or y < nnz:
        if x < n and y >= rp[x + 1]:
            x += 1  # every entry of row x has been consumed: its end comes next
        else:
            y += 1
        count += 1
        if count % items_per_chunk == 0:
            xs.append(x)
            ys.append(y)
    if count % items_per_chunk or count == 0:
        xs.append(x)
        ys.append(y)
    return np.array(xs, dtype=np.int32), np.array(ys, dtype=np.int32)


def fnv1a64(data: bytes) -> int:
    h = 0xCBF29CE484222325
    for byte in data:
        h ^= byte
        h = (h * 0x100000001B3) & 0xFFFFFFFFFFFFFFFF
    return h


def transpose(row_ptr, col_idx, n_cols):
    """The CSR pattern of A^T by its definition: the entries sorted by column
    with a stable sort (so each column lists its rows in order), the row of
    each entry as the new column index, and per-column counts accumulated into
    the new row_ptr.  Returns (t_row_ptr, t_col_idx, perm) with perm[k] the
    original entry index of transposed entry k."""
    rp = np.asarray(row_ptr, dtype=np.int64)
    ci = np.asarray(col_idx, dtype=np.int64)
    rows = np.repeat(np.arange(len(rp) - 1, dtype=np.int64), np.diff(rp))
    perm = np.argsort(ci, kind="stable")
    counts = np.bincount(ci, minlength=n_cols)[:n_cols]
    t_rp = np.zeros(n_cols + 1, dtype=np.int64)
    np.cumsum(counts, out=t_rp[1:])
    return t_rp.astype(np.int32), rows[perm].astype(np.int32), perm.astype(np.int32)


def hybrid_format_loops(row_ptr, col_idx, n_cols, parts, whole_below=0):
    """The column-part segment format by its definition, with plain loops
    (tiny inputs): for each part p, for each row r, the entries of r whose
    column lies in p, in their original order, form segment (p, r) when there
    are any; a row with fewer than whole_below entries is not split but forms
    one segment in part P = parts, after all column parts.  Returns a dict of
    int64 arrays: part_cols, perm, col_idx, seg_ptr, seg_row, seg_part,
    row_seg_ptr, row_seg."""
    rp = [int(v) for v in row_ptr]
    ci = [int(v) for v in col_idx]
    n_rows = len(rp) - 1
    part_cols = -(-n_cols // parts) if n_cols > 0 else 1

    def part_of(r, e):
        return parts if rp[r + 1] - rp[r] < whole_below else ci[e] // part_cols

    perm, seg_ptr, seg_row, seg_part = [], [], [], []
    for p in range(parts + 1):
        for r in range(n_rows):
            mine = [e for e in range(rp[r], rp[r + 1]) if part_of(r, e) == p]
            if mine:
                seg_ptr.append(len(perm))
                seg_row.append(r)
                seg_part.append(p)
                perm += mine
    seg_ptr.append(len(perm))
    row_seg_ptr, row_seg = [0], []
    for r in range(n_rows):
        row_seg += [s for s in range(len(seg_row)) if seg_row[s] == r]  # ascending s = ascending part
        row_seg_ptr.append(len(row_seg))
    a = lambda v: np.asarray(v, dtype=np.int64)  # noqa: E731
    return {"part_cols": part_cols, "perm": a(perm), "col_idx": a([ci[e] for e in perm]), "seg_ptr": a(seg_ptr),
            "seg_row": a(seg_row), "seg_part": a(seg_part), "row_seg_ptr": a(row_seg_ptr), "row_seg": a(row_seg)}


def hybrid_format(row_ptr, col_idx, n_cols, parts, whole_below=0):
    """The same format for larger inputs: the entries ordered by the key
    (part, row) with a stable sort (which keeps each segment's entries in
    their original order), a segment wherever the key changes, and each row's
    segments found by a stable sort of the segments by row."""
    rp = np.asarray(row_ptr, dtype=np.int64)
    ci = np.asarray(col_idx, dtype=np.int64)
    n_rows = len(rp) - 1
    part_cols = -(-n_cols // parts) if n_cols > 0 else 1
    deg = np.diff(rp)
    rows = np.repeat(np.arange(n_rows, dtype=np.int64), deg)
    part = np.where(deg[rows] < whole_below, parts, ci // part_cols)
    key = part * n_rows + rows
    perm = np.argsort(key, kind="stable")
    k = key[perm]
    starts = np.flatnonzero(np.r_[True, k[1:] != k[:-1]]) if len(k) else np.zeros(0, dtype=np.int64)
    seg_row = k[starts] % max(n_rows, 1)
    row_seg = np.argsort(seg_row, kind="stable")
    row_seg_ptr = np.zeros(n_rows + 1, dtype=np.int64)
    np.cumsum(np.bincount(seg_row, minlength=n_rows)[:n_rows], out=row_seg_ptr[1:])
    return {"part_cols": part_cols, "perm": perm.astype(np.int64), "col_idx": ci[perm],
            "seg_ptr": np.r_[starts, len(k)].astype(np.int64), "seg_row": seg_row.astype(np.int64),
            "seg_part": (k[starts] // max(n_rows, 1)).astype(np.int64), "row_seg_ptr": row_seg_ptr,
            "row_seg": row_seg.astype(np.int64)}
