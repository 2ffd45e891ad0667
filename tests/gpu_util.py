"""Helpers of the GPU parity tests: device transfer and the error measure.

Error measure: for each output element, |gpu - ref| / mag where mag is the
oracle's sum of absolute terms (sum |a||x|, sum |u||v|, sum p|v|); an element
with mag = 0 must be exactly 0 on the GPU.  For non-negative data mag equals
the value itself, so this is then the plain relative error.
"""

import numpy as np
import torch

TOL_F32 = 1e-5
TOL_BF16 = 1e-2


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def bf16_dev(bits):
    """uint16 bf16 bit patterns -> device bfloat16 tensor."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def max_err(gpu, ref, mag):
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    m = np.asarray(mag, dtype=np.float64)
    assert g.shape == r.shape == m.shape, (g.shape, r.shape, m.shape)
    if g.size == 0:
        return 0.0
    zero = m == 0
    if zero.any():
        assert np.all(g[zero] == 0), "elements with an all-zero oracle sum must be exactly 0"
    nz = ~zero
    if not nz.any():
        return 0.0
    e = np.abs(g[nz] - r[nz]) / m[nz]
    # a NaN anywhere is an infinite error (np.max would return NaN, which
    # Python's max() and comparisons with a tolerance would then pass over)
    return float("inf") if np.isnan(e).any() else float(np.max(e))


def assert_close(gpu, ref, mag, tol=TOL_F32, what=""):
    e = max_err(gpu, ref, mag)
    assert e <= tol, f"{what}: max error {e:.3e} > {tol:.0e}"
    return e


def compare_all_rows(got, oracle_block, row_ptr, width, tol, what, per_entry=False,
                     work_per_block=3e9, elems_per_block=4e7):
    """Compares a full GPU output with the oracle over every row: the rows
    are cut into blocks of about work_per_block multiply-adds (entries times
    width) and at most elems_per_block output elements, oracle_block(r0, r1)
    returns (ref, mag) of rows [r0, r1) (per-entry arrays for per_entry), and
    each block is checked before the next is computed, so host memory stays
    bounded.  Returns the largest error."""
    rp = np.asarray(row_ptr, dtype=np.int64)
    n = len(rp) - 1
    w = max(1, int(width))
    worst = 0.0
    r0 = 0
    while r0 < n:
        r1 = int(np.searchsorted(rp, rp[r0] + max(1, int(work_per_block / w)), side="right")) - 1
        r1 = min(max(r1, r0 + 1), n, r0 + max(1, int(elems_per_block / w)))
        ref, mag = oracle_block(r0, r1)
        g = got[rp[r0]:rp[r1]] if per_entry else got[r0:r1]
        worst = max(worst, max_err(g, ref, mag))
        r0 = r1
    assert worst <= tol, f"{what}: max error {worst:.3e} > {tol:.0e}"
    return worst
