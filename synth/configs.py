"""The five workloads, as seeded generators.

c1   fused CSR attention, tiny: 2,048 nodes, Poisson(18) in-degrees, scores
     fp32 N(0,1), values 2048 x 32 fp32 U(-1,1), scale 1.
p4   the trace page's own tiny size: 384 nodes, feature width 64, Poisson(18).
c2   SpMM on a dense-ish power-law graph: 232,965 rows, ~114.6M nnz, max
     degree ~20k (a stand-in for the Reddit graph's shape), edge values
     1/deg(row), X fp32 N(0,1) with F in {32, 64, 128, 602}.
c3   SpMM + SDDMM on a large symmetric log-normal graph: 2,449,029 rows,
     ~123.7M nnz, max degree ~17k (a stand-in for OGBN-Products' shape), edge
     values 1/deg(row), X fp32 N(0,1) with F in {100, 128}, SDDMM operands
     U, V fp32 N(0,1) of width 128.
c4   skew stress test: 1,000,000 rows, 32,000,000 nnz, 300,000 empty rows,
     rank-size (Zipf 1.5) lengths capped at 200,000; every fp32 array U(0,1);
     F in {4, 8, 16, 32}.
c5a  8-head attention on the c3 pattern: Q, K, V bf16 [N, 8, 64] from
     fp32 N(0,1), scale 1/sqrt(64).
c5b  8-head attention on a 16,384-token sliding window of 512 plus 64 global
     tokens.

Seeds are 20251117 + c for c = 1..5 (p4 uses c1's seed + 100).
"""

from __future__ import annotations

import numpy as np

from .dense import dense_normal, dense_uniform, to_bf16_bits
from .graphs import (
    CSR,
    configuration_model_symmetric,
    csr_from_degrees,
    lognormal_degrees,
    poisson_graph,
    powerlaw_degrees,
    rank_size_lengths,
    window_global_pattern,
)

CONFIG_SEED_BASE = 20251117
CONFIG_NAMES = ("c1", "p4", "c2", "c3", "c4", "c5a", "c5b")

_NUM = {"c1": 1, "p4": 1, "c2": 2, "c3": 3, "c4": 4, "c5a": 5, "c5b": 5}

# c2 power law: gamma solved (by bisection over the quantile degree sum, see
# synth.graphs.powerlaw_gamma_for_nnz) so that the degrees sum to ~114.6M.
C2_N, C2_KMAX, C2_GAMMA = 232_965, 20_000, 1.2613554
C3_N, C3_MU, C3_SIGMA = 2_449_029, 3.0495, 1.3211
C4_N, C4_EMPTY, C4_CAP, C4_NNZ = 1_000_000, 300_000, 200_000, 32_000_000
C5_HEADS, C5_DIM, C5B_L, C5B_WINDOW, C5B_GLOBAL = 8, 64, 16_384, 512, 64


def config_seed(name: str) -> int:
    return CONFIG_SEED_BASE + _NUM[name] + (100 if name == "p4" else 0)


def _streams(name: str, k: int = 8):
    return np.random.SeedSequence(config_seed(name)).spawn(k)


def _int_seed(ss: np.random.SeedSequence) -> int:
    return int(ss.generate_state(1, dtype=np.uint64)[0] >> np.uint64(1))


def config_pattern(name: str) -> CSR:
    s = _streams(name)
    rng = np.random.Generator(np.random.PCG64(s[0]))
    if name == "c1":
        return poisson_graph(2048, 18.0, rng)
    if name == "p4":
        return poisson_graph(384, 18.0, rng)
    if name == "c2":
        deg = powerlaw_degrees(C2_N, C2_GAMMA, C2_KMAX)
        return csr_from_degrees(rng.permutation(deg), C2_N, rng)
    if name in ("c3", "c5a"):
        # c5a runs on the c3 pattern: draw it from c3's stream
        s3 = _streams("c3")
        rng3 = np.random.Generator(np.random.PCG64(s3[0]))
        deg = lognormal_degrees(C3_N, C3_MU, C3_SIGMA)
        return configuration_model_symmetric(rng3.permutation(deg), rng3)
    if name == "c4":
        deg = np.zeros(C4_N, dtype=np.int64)
        empty = rng.choice(C4_N, size=C4_EMPTY, replace=False)
        live = np.setdiff1d(np.arange(C4_N), empty)
        lengths = rank_size_lengths(len(live), C4_CAP, C4_NNZ)
        deg[live] = rng.permutation(lengths)
        return csr_from_degrees(deg, C4_N, rng)
    if name == "c5b":
        return window_global_pattern(C5B_L, C5B_WINDOW, C5B_GLOBAL)
    raise KeyError(name)


def inverse_degree_values(csr: CSR) -> np.ndarray:
    """Edge value fp32(1) / fp32(deg(row)) for every stored entry."""
    deg = csr.degrees().astype(np.float32)
    inv = np.where(deg > 0, np.float32(1.0) / np.maximum(deg, np.float32(1.0)), 0).astype(np.float32)
    return np.repeat(inv, csr.degrees())


def config_dense(name: str, what: str, csr: CSR, width: int | None = None) -> np.ndarray:
    """Dense operand ``what`` of workload ``name``.

    what: 'vals' (edge values [nnz]), 'scores' (edge scores [nnz]), 'X'
    ([n_cols, width] features), 'U' ([n_rows, width]), 'V' ([n_cols, width]),
    'Q' / 'K' / 'Vh' (bf16 bit patterns [n, 8, 64], uint16).
    """
    s = _streams(name, 16)
    idx = {"vals": 1, "scores": 2, "X": 3, "U": 4, "V": 5, "Q": 6, "K": 7, "Vh": 8}[what]
    seed = _int_seed(s[idx]) + (width or 0) * 7919
    nnz, n, m = csr.nnz, csr.n_rows, csr.n_cols
    if what == "vals":
        if name in ("c2", "c3"):
            return inverse_degree_values(csr)
        return dense_uniform((nnz,), seed) if name == "c4" else dense_normal((nnz,), seed)
    if what == "scores":
        return dense_normal((nnz,), seed)
    if what in ("Q", "K", "Vh"):
        rows = n if what == "Q" else m
        return to_bf16_bits(dense_normal((rows, C5_HEADS, C5_DIM), seed))
    rows = n if what == "U" else m
    if width is None:
        raise ValueError("width required")
    if name in ("c1", "p4") and what == "X":
        return dense_uniform((rows, width), seed, -1.0, 1.0)
    if name == "c4":
        return dense_uniform((rows, width), seed)
    return dense_normal((rows, width), seed)


def make_config(name: str):
    """Pattern plus the operands every test of that workload uses at its
    default width (the dense arrays of the large configs are produced on
    demand with ``config_dense``)."""
    csr = config_pattern(name)
    out = {"csr": csr}
    if name in ("c1", "p4"):
        out["scores"] = config_dense(name, "scores", csr)
        out["V"] = config_dense(name, "X", csr, 32 if name == "c1" else 64)
    return out
