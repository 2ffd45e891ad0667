"""Benchmark of the CSR aggregation hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config c2]

One step is one pass of the hot path over one synthetic workload (inputs
resident in HBM): for the default workload (a 232,965-row power-law graph
with ~114.6M entries, edge values 1/deg, dense X fp32 N(0,1)) that is CSR
SpMM at every feature width of the sweep F = 32, 64, 128, 602, each call
replaying the schedule the selector chose for it (the argument checks,
merge-path partition, main kernel and split-row fix-up run every step; the
degree histogram, signature, cost model and micro-probes run once, before
the warm-up, and are reported separately).

Throughput ("value") is effective bandwidth: algorithmic bytes (one
gathered feature row per stored entry plus the CSR arrays and the output)
over time; GNNZ*F/s is stored entries times width per second.  These count a
gather served by a cache like one from HBM, so they can exceed the HBM peak.
The roofline object is about HBM itself: for the dominant call, the bytes
its kernels move to and from memory as counted by rocprofv3 (committed
counter records of the same sources, profiles/traffic.json) over its live
HIP-event time, against 8 TB/s, beside the compulsory-traffic model of the
method it runs.  Prints one JSON line.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "effective HBM GB/s and GNNZ*F/s per kernel; % of MI355X HBM roofline"


# calls without a schedule: per-entry value moves
NO_SCHEDULE = ("gather", "permute")


def b_alg(op, n_rows, nnz, width, heads=8, head_dim=64, esize=4):
    """Algorithmic bytes of one call (index arrays, values, one gathered row
    per stored entry, dense row operands, output); esize = bytes per element
    of the dense operands (4 fp32, 2 bf16; outputs are fp32)."""
    if op == "spmm":
        return 4 * (n_rows + 1) + nnz * 8 + nnz * width * esize + n_rows * width * 4
    if op == "sddmm":
        return 4 * (n_rows + 1) + nnz * 8 + n_rows * width * esize + nnz * width * esize
    if op == "attention_qk":
        # Q row per row, K and V rows per stored entry, output row per row
        return 4 * (n_rows + 1) + nnz * 4 + n_rows * width * esize + 2 * nnz * width * esize + n_rows * width * 4
    if op == "attention":
        return 4 * (n_rows + 1) + nnz * 8 + nnz * width * 4 + n_rows * width * 4
    if op == "row_softmax":
        return 4 * (n_rows + 1) + nnz * 8
    if op == "row_softmax_backward":
        return 4 * (n_rows + 1) + nnz * 12
    if op == "gather":
        return nnz * 12
    if op == "permute":
        # two passes: an index, a value and a write each
        return nnz * 24
    if op == "spmm_sddmm":
        # the SpMM's bytes, the U row per row and the per-entry output
        return 4 * (n_rows + 1) + nnz * 8 + nnz * width * esize + 2 * n_rows * width * 4 + nnz * 4
    if op == "mha":
        hd = heads * head_dim
        return 4 * (n_rows + 1) + nnz * 4 + n_rows * hd * 2 + 2 * nnz * hd * 2 + n_rows * hd * 4
    raise ValueError(op)


def compulsory_bytes(c, torch):
    """HBM bytes the call cannot avoid under the method it runs (the model the
    counted traffic is held against).  Plain CSR: the algorithmic bytes (one
    gathered row per stored entry: the gathered operands of these workloads
    are far larger than the caches, so a gather finds no earlier copy).  Over
    the column-part segment format (SpMM): the dense operand once (each
    part's slice is read into the cache once), the rows kept whole gathered
    in full (they read from all of the operand), every segment's partial row
    written and read once, the format's column indices and values, the
    segment and row-segment offsets, and the output.  SDDMM over the format:
    V once, each segment's U row, the indices and the permuted output."""
    pl = c.plan
    if pl is None or pl.parts == 1:
        return c.bytes
    rp = c.args[0]
    deg = (rp[1:] - rp[:-1]).long()
    T = pl.whole_below
    F = c.width
    n_cols = c.args[3].shape[0]
    n_seg = pl.n_seg
    seg_idx = 4 * (n_seg + 1) + 4 * n_seg + 4 * (c.n_rows + 1)
    if c.op == "spmm":
        whole_nnz = int(deg[deg < T].sum().item()) if T > 0 else 0
        return (n_cols * F * 4 + whole_nnz * F * 4 + 2 * n_seg * F * 4 + 8 * c.nnz + seg_idx
                + c.n_rows * F * 4)
    return n_cols * F * 4 + n_seg * F * 4 + 12 * c.nnz + seg_idx


class Call:
    """One library call of the step with its operands.  SpMM and SDDMM run
    through a plan (the library's joint choice of layout and schedule);
    the other calls replay their selected schedule."""

    def __init__(self, name, op, fn, args, kwargs, n_rows, nnz, width, oracle_fn, esize=4):
        self.name, self.op, self.fn, self.args, self.kwargs = name, op, fn, args, kwargs
        self.n_rows, self.nnz, self.width, self.esize = n_rows, nnz, width, esize
        self.bytes = b_alg(op, n_rows, nnz, width, esize=esize)
        self.oracle_fn = oracle_fn
        self.schedule = None
        self.times = []
        self.plan = None  # csa.Plan of an SpMM / SDDMM call
        self.csa = None
        # SpMM values that the step itself produces (probabilities): passed
        # to every planned call, not taken from the plan's copy
        self.step_values = False

    def run(self, schedule=None):
        """The call as the step makes it (through its plan, when it has one),
        or with ``schedule`` on the plain CSR pattern."""
        if schedule is None and self.plan is not None:
            out = self.kwargs.get("out")
            if self.op == "spmm":
                vals = self.args[2] if self.step_values else None
                return self.csa.plan_spmm(self.plan, self.args[3], vals=vals, out=out)
            return self.csa.plan_sddmm(self.plan, self.args[2], self.args[3], out=out)
        s = schedule if schedule is not None else self.schedule
        return self.fn(*self.args, schedule=s, **self.kwargs)

    def select(self, csa, mode="auto"):
        sel_args = (self.args[0], None) + tuple(self.args[1:]) if self.op.startswith("row_softmax") else self.args
        kw = {k: self.kwargs[k] for k in ("scale", "val_idx", "z_idx") if k in self.kwargs}
        return csa.select(self.op, *sel_args, mode=mode, **kw)

    def label(self):
        """The call's layout and schedule as one dict."""
        if self.plan is not None:
            return {"format_parts": self.plan.parts, "whole_below": self.plan.whole_below,
                    **self.plan.schedule.as_dict()}
        return {"format_parts": 1, **self.schedule.as_dict()}


def make_plan(c, csa, torch):
    """Plans call c through the library (csr_plan_create, mode auto): the
    first creation runs the histogram, the cost model and the micro-probes
    over the plain pattern and the format's candidate part counts and caches
    the choice; a second creation replays it (histogram, cache lookup and
    the chosen format's construction).  The replayed plan is kept.  Returns
    the one-time costs in ms."""
    operands = c.args[2:4]
    out = c.kwargs.get("out")
    torch.cuda.synchronize()
    t = time.perf_counter()
    first = csa.plan(c.op, c.args[0], c.args[1], *operands, out=out)
    torch.cuda.synchronize()
    first_ms = (time.perf_counter() - t) * 1e3
    probe_ms = first.desc.probe_ms
    del first
    torch.cuda.synchronize()
    t = time.perf_counter()
    c.plan = csa.plan(c.op, c.args[0], c.args[1], *operands, out=out, mode="replay")
    torch.cuda.synchronize()
    c.csa = csa
    return {"plan_create_ms": round(first_ms, 3), "plan_probe_ms": round(probe_ms, 3),
            "plan_replay_ms": round((time.perf_counter() - t) * 1e3, 3), "signature": f"{c.plan.signature:016x}"}


def format_candidate(csa, torch, c, P, cache, whole_below=0):
    """The column-part segment format of call c at P parts and whole-row
    threshold whole_below, built once per pattern (SpMM values moved into the
    format's order), with closures that run and select over it: the
    candidates a plan weighs, rebuilt here so the study can time each."""
    rp, ci = c.args[0], c.args[1]
    dense = c.args[3]
    key = (rp.data_ptr(), ci.data_ptr(), P, whole_below)
    if key not in cache:
        cache[key] = csa.hybrid_format(rp, ci, dense.shape[0], P, whole_below=whole_below)
    h = cache[key]
    out = c.kwargs.get("out")
    if c.op == "spmm":
        vals, X = c.args[2], c.args[3]
        hv = None if vals is None else csa.hybrid_values(h, vals)
        run = lambda s: csa.hybrid_spmm(h, hv, X, out=out, schedule=s)  # noqa: E731
        select = lambda mode: csa.hybrid_select(h, "spmm", hv, X, mode=mode)  # noqa: E731
        a, b = hv, X
    else:
        U, V = c.args[2], c.args[3]
        run = lambda s: csa.hybrid_sddmm(h, U, V, out=out, schedule=s)  # noqa: E731
        select = lambda mode: csa.hybrid_select(h, "sddmm", U, V, mode=mode, out=out)  # noqa: E731
        a, b = U, V
    return {"h": h, "parts": P, "whole_below": whole_below, "run": run, "select": select, "operands": (a, b)}


def build_workload(name, torch, csa):
    from synth import configs

    def d(a):
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    def b16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()

    calls = []
    t0 = time.time()
    if name in ("c2", "c3", "c4", "c3sweep"):
        pat = "c3" if name == "c3sweep" else name
        csr = configs.config_pattern(pat)
        rp, ci = d(csr.row_ptr), d(csr.col_idx)
        vals = configs.config_dense(pat, "vals", csr)
        vd = d(vals)
        # c3sweep: the c3 SpMM at growing widths, i.e. a growing gathered operand
        widths = {"c2": (32, 64, 128, 602), "c3": (100, 128), "c4": (4, 8, 16, 32),
                  "c3sweep": (128, 256, 384, 512)}[name]
        for F in widths:
            X = configs.config_dense(pat, "X", csr, F)
            Xd = d(X)
            Y = torch.empty((csr.n_rows, F), dtype=torch.float32, device="cuda")
            calls.append(Call(f"spmm_F{F}", "spmm", csa.spmm, (rp, ci, vd, Xd), {"out": Y}, csr.n_rows, csr.nnz, F,
                              ("spmm", csr, vals, X)))
        sd_widths = {"c2": (), "c3": (128,), "c4": (4, 8, 16, 32), "c3sweep": ()}[name]
        for K in sd_widths:
            U = configs.config_dense(pat, "U", csr, K)
            V = configs.config_dense(pat, "V", csr, K)
            out = torch.empty(csr.nnz, dtype=torch.float32, device="cuda")
            calls.append(Call(f"sddmm_K{K}", "sddmm", csa.sddmm, (rp, ci, d(U), d(V)), {"out": out}, csr.n_rows,
                              csr.nnz, K, ("sddmm", csr, U, V)))
    elif name == "c3qk":
        # single-head fp32 attention on the c3 graph from Q, K, V of width 64
        # in one pass (scores formed in registers, never written)
        csr = configs.config_pattern("c3")
        rp, ci = d(csr.row_ptr), d(csr.col_idx)
        Q = configs.config_dense("c3", "U", csr, 64)
        K = configs.config_dense("c3", "V", csr, 64)
        V = configs.config_dense("c3", "X", csr, 64)
        Y = torch.empty((csr.n_rows, 64), dtype=torch.float32, device="cuda")
        calls.append(Call("attention_qk_F64", "attention_qk", csa.attention_qk, (rp, ci, d(Q), d(K), d(V)),
                          {"out": Y, "scale": 0.125}, csr.n_rows, csr.nnz, 64, ("attention_qk", csr, Q, K, V)))
    elif name == "c3bf16":
        # bf16 features on the c3 graph: SpMM F = 128 and SDDMM K = 128, fp32 accumulation
        from synth import to_bf16_bits

        csr = configs.config_pattern("c3")
        rp, ci = d(csr.row_ptr), d(csr.col_idx)
        vals = configs.config_dense("c3", "vals", csr)
        Xb = to_bf16_bits(configs.config_dense("c3", "X", csr, 128))
        Y = torch.empty((csr.n_rows, 128), dtype=torch.float32, device="cuda")
        calls.append(Call("spmm_bf16_F128", "spmm", csa.spmm, (rp, ci, d(vals), b16(Xb)), {"out": Y}, csr.n_rows,
                          csr.nnz, 128, ("spmm", csr, vals, Xb), esize=2))
        Ub = to_bf16_bits(configs.config_dense("c3", "U", csr, 128))
        Vb = to_bf16_bits(configs.config_dense("c3", "V", csr, 128))
        out = torch.empty(csr.nnz, dtype=torch.float32, device="cuda")
        calls.append(Call("sddmm_bf16_K128", "sddmm", csa.sddmm, (rp, ci, b16(Ub), b16(Vb)), {"out": out},
                          csr.n_rows, csr.nnz, 128, ("sddmm", csr, Ub, Vb), esize=2))
    elif name in ("c3pipe", "c3fused"):
        # single-head fp32 attention on the c3 graph from Q, K, V of width 64:
        # SDDMM -> row softmax -> SpMM as three calls, or SDDMM -> fused
        # softmax-aggregation as two
        csr = configs.config_pattern("c3")
        rp, ci = d(csr.row_ptr), d(csr.col_idx)
        Q = configs.config_dense("c3", "U", csr, 64)
        K = configs.config_dense("c3", "V", csr, 64)
        V = configs.config_dense("c3", "X", csr, 64)
        S = torch.empty(csr.nnz, dtype=torch.float32, device="cuda")
        P = torch.empty(csr.nnz, dtype=torch.float32, device="cuda")
        Y = torch.empty((csr.n_rows, 64), dtype=torch.float32, device="cuda")
        Vd = d(V)
        calls.append(Call("sddmm_K64", "sddmm", csa.sddmm, (rp, ci, d(Q), d(K)), {"out": S}, csr.n_rows, csr.nnz,
                          64, ("sddmm", csr, Q, K)))
        if name == "c3pipe":
            calls.append(Call("row_softmax", "row_softmax", csa.row_softmax, (rp, S), {"out": P, "scale": 0.125},
                              csr.n_rows, csr.nnz, 1, None))
            calls.append(Call("spmm_F64", "spmm", csa.spmm, (rp, ci, P, Vd), {"out": Y}, csr.n_rows, csr.nnz, 64,
                              None))
            calls[-1].step_values = True
        else:
            calls.append(Call("attention_F64", "attention", csa.attention, (rp, ci, S, Vd),
                              {"out": Y, "scale": 0.125}, csr.n_rows, csr.nnz, 64, None))
    elif name == "c3qkbwd":
        # backward of the one-head fp32 attention from Q, K, V (width 64) on
        # the c3 graph: scores s = SDDMM(Q, K), P = row softmax, P into A^T's
        # order, dV and dP in one pass over A^T, dP back, d s = softmax
        # backward (in place), dQ = A_ds K, d s into A^T's order, dK =
        # A_ds^T Q.  The transposed pattern and its permutation plans are
        # built once, outside the step.
        csr = configs.config_pattern("c3")
        rp, ci = d(csr.row_ptr), d(csr.col_idx)
        Q = d(configs.config_dense("c3", "U", csr, 64))
        K = d(configs.config_dense("c3", "V", csr, 64))
        Vd = d(configs.config_dense("c3", "X", csr, 64))
        dO = d(configs.config_dense("c3", "U", csr, 65)[:, :64])
        torch.cuda.synchronize()
        tt = time.perf_counter()
        At = csa.transpose(rp, ci, csr.n_cols, plans=True)
        torch.cuda.synchronize()
        build_workload.transpose_first_ms = (time.perf_counter() - tt) * 1e3
        # again with the buffers already in torch's pool: the build's own time
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        del At
        ev0.record()
        At = csa.transpose(rp, ci, csr.n_cols, plans=True)
        ev1.record()
        ev1.synchronize()
        build_workload.transpose_ms = ev0.elapsed_time(ev1)
        e = lambda: torch.empty(csr.nnz, dtype=torch.float32, device="cuda")  # noqa: E731
        S, P, Pt, dPt, dP, tmp = e(), e(), e(), e(), e(), e()
        dV = torch.empty((csr.n_cols, 64), dtype=torch.float32, device="cuda")
        dQ = torch.empty((csr.n_rows, 64), dtype=torch.float32, device="cuda")
        dK = torch.empty((csr.n_cols, 64), dtype=torch.float32, device="cuda")

        def permute(plan, src, out, schedule=None):
            return csa.permute_values(plan, src, out=out, tmp=tmp)

        calls.append(Call("sddmm_S", "sddmm", csa.sddmm, (rp, ci, Q, K), {"out": S}, csr.n_rows, csr.nnz, 64, None))
        calls.append(Call("row_softmax", "row_softmax", csa.row_softmax, (rp, S), {"out": P, "scale": 0.125},
                          csr.n_rows, csr.nnz, 1, None))
        calls.append(Call("permute_Pt", "permute", permute, (At.to_t, P, Pt), {}, csr.n_rows, csr.nnz, 1, None))
        calls.append(Call("spmm_sddmm_dV_dP", "spmm_sddmm", csa.spmm_sddmm, (At.row_ptr, At.col_idx, Pt, dO, Vd),
                          {"out": dV, "z": dPt}, csr.n_cols, csr.nnz, 64, None))
        calls.append(Call("permute_dP", "permute", permute, (At.from_t, dPt, dP), {}, csr.n_rows, csr.nnz, 1, None))
        calls.append(Call("softmax_bwd", "row_softmax_backward", csa.row_softmax_backward, (rp, P, dP),
                          {"out": dP, "scale": 0.125}, csr.n_rows, csr.nnz, 1, None))
        calls.append(Call("spmm_dQ", "spmm", csa.spmm, (rp, ci, dP, K), {"out": dQ}, csr.n_rows, csr.nnz, 64, None))
        calls[-1].step_values = True
        calls.append(Call("permute_dSt", "permute", permute, (At.to_t, dP, dPt), {}, csr.n_rows, csr.nnz, 1, None))
        calls.append(Call("spmm_dK", "spmm", csa.spmm, (At.row_ptr, At.col_idx, dPt, Q), {"out": dK}, csr.n_cols,
                          csr.nnz, 64, None))
        calls[-1].step_values = True
    elif name in ("c3bwd", "c3bwd_perm", "c3bwd_gather"):
        # backward of the single-head fp32 attention on the c3 graph (scores
        # given, F = 64): P = row softmax; dV = P^T dOut and dP = dOut V^T;
        # d scores = softmax backward.  c3bwd: P moved into A^T's order by
        # a two-pass permutation, dV and dP in one pass over A^T
        # (csr_spmm_sddmm), dP moved back the same way; c3bwd_perm: SDDMM
        # dP on A, then the
        # SpMM on A^T reading P through the perm; c3bwd_gather: P gathered
        # into A^T's order first.  The transposed pattern is built once,
        # outside the step.
        csr = configs.config_pattern("c3")
        rp, ci = d(csr.row_ptr), d(csr.col_idx)
        S = d(configs.config_dense("c3", "scores", csr) * 3.0)
        Vd = d(configs.config_dense("c3", "X", csr, 64))
        dO = d(configs.config_dense("c3", "V", csr, 64))
        plans = name == "c3bwd"  # the fused backward moves values through two-pass permutation plans
        torch.cuda.synchronize()
        tt = time.perf_counter()
        At = csa.transpose(rp, ci, csr.n_cols, plans=plans)
        torch.cuda.synchronize()
        build_workload.transpose_first_ms = (time.perf_counter() - tt) * 1e3
        # again with the buffers already in torch's pool: the build's own time
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        del At
        ev0.record()
        At = csa.transpose(rp, ci, csr.n_cols, plans=plans)
        ev1.record()
        ev1.synchronize()
        build_workload.transpose_ms = ev0.elapsed_time(ev1)
        P = torch.empty(csr.nnz, dtype=torch.float32, device="cuda")
        dP = torch.empty(csr.nnz, dtype=torch.float32, device="cuda")
        Pt = torch.empty(csr.nnz, dtype=torch.float32, device="cuda")
        dV = torch.empty((csr.n_cols, 64), dtype=torch.float32, device="cuda")
        calls.append(Call("row_softmax", "row_softmax", csa.row_softmax, (rp, S), {"out": P, "scale": 0.125},
                          csr.n_rows, csr.nnz, 1, None))
        if name == "c3bwd":
            # P moved into A^T's order and dP back by two-pass permutations;
            # the softmax backward runs in place on dP
            dPt = torch.empty(csr.nnz, dtype=torch.float32, device="cuda")
            tmp = torch.empty(csr.nnz, dtype=torch.float32, device="cuda")

            def permute(plan, src, out, schedule=None):
                return csa.permute_values(plan, src, out=out, tmp=tmp)

            calls.append(Call("permute_Pt", "permute", permute, (At.to_t, P, Pt), {}, csr.n_rows, csr.nnz, 1, None))
            calls.append(Call("spmm_sddmm_dV_dP", "spmm_sddmm", csa.spmm_sddmm, (At.row_ptr, At.col_idx, Pt, dO, Vd),
                              {"out": dV, "z": dPt}, csr.n_cols, csr.nnz, 64, None))
            calls.append(Call("permute_dP", "permute", permute, (At.from_t, dPt, dP), {}, csr.n_rows, csr.nnz, 1,
                              None))
            calls.append(Call("softmax_bwd", "row_softmax_backward", csa.row_softmax_backward, (rp, P, dP),
                              {"out": dP, "scale": 0.125}, csr.n_rows, csr.nnz, 1, None))
            return calls, time.time() - t0
        calls.append(Call("sddmm_dP", "sddmm", csa.sddmm, (rp, ci, dO, Vd), {"out": dP}, csr.n_rows, csr.nnz, 64,
                          None))
        calls.append(Call("softmax_bwd", "row_softmax_backward", csa.row_softmax_backward, (rp, P, dP),
                          {"out": dP, "scale": 0.125}, csr.n_rows, csr.nnz, 1, None))
        if name == "c3bwd_gather":
            calls.append(Call("gather_Pt", "gather", lambda perm, src, out, schedule=None: csa.gather_values(
                perm, src, out=out), (At.perm, P, Pt), {}, csr.n_rows, csr.nnz, 1, None))
            calls.append(Call("spmm_dV", "spmm", csa.spmm, (At.row_ptr, At.col_idx, Pt, dO), {"out": dV},
                              csr.n_cols, csr.nnz, 64, None))
        else:
            # P read through the transposed pattern's perm inside the SpMM
            calls.append(Call("spmm_dV", "spmm", csa.spmm, (At.row_ptr, At.col_idx, P, dO),
                              {"out": dV, "val_idx": At.perm}, csr.n_cols, csr.nnz, 64, None))
            calls[-1].bytes += 4 * csr.nnz  # the value index
    elif name in ("c1", "p4"):
        c = configs.make_config(name)
        csr = c["csr"]
        rp, ci = d(csr.row_ptr), d(csr.col_idx)
        F = c["V"].shape[1]
        calls.append(Call(f"attention_F{F}", "attention", csa.attention, (rp, ci, d(c["scores"]), d(c["V"])), {},
                          csr.n_rows, csr.nnz, F, ("attention", csr, c["scores"], c["V"])))
    elif name in ("c5a", "c5b"):
        csr = configs.config_pattern(name)
        rp, ci = d(csr.row_ptr), d(csr.col_idx)
        Q = configs.config_dense(name, "Q", csr)
        K = configs.config_dense(name, "K", csr)
        V = configs.config_dense(name, "Vh", csr)
        out = torch.empty((csr.n_rows, 8, 64), dtype=torch.float32, device="cuda")
        calls.append(Call("mha_8x64", "mha", csa.mha_attention, (rp, ci, b16(Q), b16(K), b16(V)),
                          {"scale": 0.125, "out": out}, csr.n_rows, csr.nnz, 512, ("mha", csr, Q, K, V)))
    else:
        raise SystemExit(f"unknown config {name}")
    return calls, time.time() - t0


def check_shapes(calls):
    """Host-side check, before any launch, that every operand has the size its
    call implies (per-entry arrays: nnz values; pattern arrays: rows + 1 and
    nnz), so that no kernel is handed a buffer shorter than it reads."""
    for c in calls:
        a = c.args
        if c.op == "gather":
            assert all(t.numel() == c.nnz for t in a), (c.name, "gather operands")
            continue
        if c.op == "permute":
            plan, src, out = a
            assert all(t.numel() == c.nnz for t in (plan.q1, plan.pos, src, out)), (c.name, "permute operands")
            continue
        assert a[0].numel() == c.n_rows + 1, (c.name, "row_ptr")
        if c.op in ("row_softmax", "row_softmax_backward"):
            for t in a[1:]:
                assert t.numel() == c.nnz, (c.name, "per-entry operand")
            out = c.kwargs.get("out")
            assert out is None or out.numel() == c.nnz, (c.name, "out")
        else:
            assert a[1].numel() == c.nnz, (c.name, "col_idx")
            if c.op in ("spmm", "attention", "spmm_sddmm") and a[2] is not None:
                assert a[2].numel() == c.nnz, (c.name, "per-entry values")
            for k in ("val_idx", "z_idx", "z"):
                if k in c.kwargs:
                    assert c.kwargs[k].numel() == c.nnz, (c.name, k)
            if c.op == "spmm_sddmm":
                assert a[4].shape[0] == c.n_rows and a[4].shape[1] == a[3].shape[1], (c.name, "U")


def stream_bandwidth(torch, gib=4):
    """Streaming reference on this GPU: best of 5 device copies (read + write)
    and of 5 full reductions (read only) of a `gib` GiB fp32 buffer."""
    n = gib * (1 << 28)
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    stream = torch.cuda.current_stream()
    res = {}
    for name, fn, nbytes in (("copy", lambda: y.copy_(x), 2 * 4 * n), ("read", lambda: x.sum(), 4 * n)):
        best = None
        for _ in range(6):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            b.synchronize()
            t = a.elapsed_time(b)
            best = t if best is None else min(best, t)
        res[f"{name}_GB_s"] = round(nbytes / (best * 1e-3) / 1e9, 1)
    del x, y
    torch.cuda.empty_cache()
    return res


def committed_traffic(config, call):
    """HBM traffic per launch of the dominant kernel from the committed counter
    summary (profiles/traffic.json), or None when the kernel's sources or the
    selected schedule differ from those the counters were taken with."""
    import hashlib

    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        recs = json.load(f).get(config) or []
    if isinstance(recs, dict):
        recs = [recs]
    sd = call.label()
    parts, whole = sd.pop("format_parts"), sd.pop("whole_below", 0)
    for rec in recs:
        if rec.get("call") != call.name or any(sd.get(k) != v for k, v in rec["schedule"].items()):
            continue
        if rec.get("format_parts", 1) != parts or rec.get("whole_below", 0) != whole:  # another pattern or format
            continue
        h = hashlib.sha256()
        for src in rec["sources"]:
            with open(os.path.join(ROOT, src), "rb") as f:
                h.update(f.read())
        if h.hexdigest() == rec["sources_sha256"]:
            return rec["traffic_bytes"]
    return None


def selector_study(calls, torch, csa, rounds=5, per_round=3):
    """Times every candidate of each call under one protocol and compares the
    library's pick with the best: every candidate schedule of the plain CSR
    problem; for SpMM / SDDMM also the format at each part count a plan
    weighs (the cost model's part count and threshold, half and twice that
    count, the same count with no whole rows; or 4 and 16 parts when the
    model keeps the plain pattern), each with its own selected schedule, and
    every candidate schedule of the format the plan chose; for SpMM the
    degree classes at short thresholds 8 and 32 with the selector's schedule
    for their long rows.  The library's
    pick is the call as the step makes it (through its plan for SpMM /
    SDDMM, the selected schedule otherwise).  The distinct candidates run in
    interleaved rounds (so clock and thermal drift bias none of them),
    `per_round` HIP-event timed runs each, and the median over all rounds is
    kept."""
    stream = torch.cuda.current_stream()
    formats = {}

    def timed(run):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        run()
        b.record(stream)
        b.synchronize()
        return a.elapsed_time(b)

    out = {}
    for c in calls:
        if c.op in NO_SCHEDULE:
            continue
        scale = c.kwargs.get("scale", 1.0)
        args = (c.args[0], None) + tuple(c.args[1:]) if c.op.startswith("row_softmax") else c.args
        p, _ = csa.make_problem(c.op, *args, out=c.kwargs.get("out"), scale=scale, val_idx=c.kwargs.get("val_idx"),
                                z_idx=c.kwargs.get("z_idx"))
        counts, sums, mx = csa.degree_histogram(c.args[0])
        hist = counts + sums + [mx]
        cands = [({"format_parts": 1, **s.as_dict()}, lambda s=s: c.fn(*c.args, schedule=s, **c.kwargs))
                 for s in csa.candidates(p, hist)]
        if c.op in ("spmm", "sddmm") and "val_idx" not in c.kwargs:
            P0, T0 = csa.hybrid_plan(p, hist)
            fmts = ([(P0, T0), (P0 // 2, T0), (P0 * 2, T0)] + ([(P0, 0)] if T0 > 0 else [])) if P0 > 1 \
                else [(4, 0), (16, 0)]
            chosen = (c.plan.parts, c.plan.whole_below) if c.plan is not None and c.plan.parts > 1 else None
            for P, T in fmts:
                if not 2 <= P <= 256:
                    continue
                f = format_candidate(csa, torch, c, P, formats, T)
                if (P, T) == chosen:
                    hp = csa.hybrid_problem(f["h"], c.op, *f["operands"])
                    sc, ss, smx = csa.degree_histogram(f["h"].seg_ptr)
                    cands += [({"format_parts": P, "whole_below": T, **s.as_dict()},
                               lambda f=f, s=s: f["run"](s)) for s in csa.candidates(hp, sc + ss + [smx])]
                else:
                    s_alt, _ = f["select"]("auto")
                    cands.append(({"format_parts": P, "whole_below": T, **s_alt.as_dict()},
                                  lambda f=f, s=s_alt: f["run"](s)))
        if c.op == "spmm" and "val_idx" not in c.kwargs:
            # the degree classes at both short thresholds, the long rows on the selector's schedule
            for E in (8, 32):
                try:
                    pc = csa.plan("spmm", c.args[0], c.args[1], c.args[2], c.args[3], layout=(0, E),
                                  out=c.kwargs.get("out"))
                except csa.CsrError:
                    continue
                cands.append(({"format_parts": 0, "whole_below": E, **pc.schedule.as_dict()},
                              lambda pc=pc: csa.plan_spmm(pc, c.args[3], out=c.kwargs.get("out"))))
        n_cand = len(cands)
        selected = c.label()
        # the pick, run as the step runs it (its own entry when a fixed
        # candidate has the same layout and schedule: the two are one kernel)
        cands = [(lab, run) for lab, run in cands if lab != selected] + [(selected, lambda: c.run())]
        labels = [lab for lab, _ in cands]
        times = [[] for _ in cands]
        for _, run in cands:
            timed(run)
        for _ in range(rounds):
            for i, (_, run) in enumerate(cands):
                for _ in range(per_round):
                    times[i].append(timed(run))
        med = [float(np.median(t)) for t in times]
        sel = med[-1]
        best = int(np.argmin(med))
        out[c.name] = {"selected_ms": round(sel, 4), "best_fixed_ms": round(med[best], 4),
                       "selected": selected, "best_fixed": labels[best], "n_candidates": n_cand,
                       "selected_over_best": round(sel / med[best], 4),
                       "picked_by": "csr_plan_create (auto)" if c.plan is not None else "csr_select (auto)",
                       "candidate_ms": [round(t, 4) for t in med],
                       "candidate_format_parts": [lab["format_parts"] for lab in labels]}
    return out


def cold_times(calls, torch, reps=5, flush_gib=1):
    """Per-call time with cold caches: before each HIP-event timed call a
    kernel writes a 1 GiB buffer (four times the 256 MB Infinity Cache and far
    beyond L2), so the call finds none of its operands cached.  Median of
    `reps`."""
    stream = torch.cuda.current_stream()
    scratch = torch.empty(flush_gib << 30, dtype=torch.uint8, device="cuda")
    out = {}
    for c in calls:
        ts = []
        for r in range(reps):
            scratch.fill_(r & 0xFF)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            c.run()
            b.record(stream)
            b.synchronize()
            ts.append(a.elapsed_time(b))
        out[c.name] = float(np.median(ts))
    del scratch
    torch.cuda.empty_cache()
    return out


class Rocsparse:
    """rocSPARSE's generic CSR SpMM and SDDMM through ctypes: a measurement
    beside this library, never a dispatch target.  Each call takes device
    tensors and returns (median ms of ``reps`` HIP-event timed compute calls,
    status); the analysis / preprocess stage runs outside the timed region."""

    ALGS = {"default": 0, "csr_row_split": 4, "csr_nnz_split": 5, "csr_merge_path": 9}

    def __init__(self, torch, reps=5):
        import ctypes

        self.ct, self.torch, self.reps = ctypes, torch, reps
        self.rs = ctypes.CDLL("librocsparse.so.1")  # OSError when not installed
        P, I64, INT = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        rs = self.rs
        self.h = P()
        assert rs.rocsparse_create_handle(ctypes.byref(self.h)) == 0
        self.stream = torch.cuda.current_stream()
        rs.rocsparse_set_stream(self.h, P(self.stream.cuda_stream))
        rs.rocsparse_create_csr_descr.argtypes = [ctypes.POINTER(P), I64, I64, I64, P, P, P, INT, INT, INT, INT]
        rs.rocsparse_create_dnmat_descr.argtypes = [ctypes.POINTER(P), I64, I64, I64, P, INT, INT]
        rs.rocsparse_spmm.argtypes = [P, INT, INT, P, P, P, P, P, INT, INT, INT, ctypes.POINTER(ctypes.c_size_t), P]
        rs.rocsparse_sddmm_buffer_size.argtypes = [P, INT, INT, P, P, P, P, P, INT, INT,
                                                   ctypes.POINTER(ctypes.c_size_t)]
        for f in ("rocsparse_sddmm_preprocess", "rocsparse_sddmm"):
            getattr(rs, f).argtypes = [P, INT, INT, P, P, P, P, P, INT, INT, P]
        self.one, self.zero = ctypes.c_float(1.0), ctypes.c_float(0.0)

    def close(self):
        self.rs.rocsparse_destroy_handle(self.h)

    def _timed(self, fn):
        ts = []
        if fn() != 0:
            return None, -1
        for _ in range(self.reps):
            a, b = self.torch.cuda.Event(enable_timing=True), self.torch.cuda.Event(enable_timing=True)
            a.record(self.stream)
            rc = fn()
            b.record(self.stream)
            b.synchronize()
            if rc != 0:
                return None, rc
            ts.append(a.elapsed_time(b))
        return float(np.median(ts)), 0

    def spmm(self, rp, ci, vals, X, Y, alg):
        """Y = A X (fp32, row-major X and Y) with rocSPARSE algorithm ``alg``."""
        ct, rs, P = self.ct, self.rs, self.ct.c_void_p
        n_rows, nnz = rp.numel() - 1, ci.numel()
        v = vals if vals is not None else self.torch.ones(nnz, device=X.device)
        A, B, C = P(), P(), P()
        rs.rocsparse_create_csr_descr(ct.byref(A), n_rows, X.shape[0], nnz, P(rp.data_ptr()), P(ci.data_ptr()),
                                      P(v.data_ptr()), 2, 2, 0, 151)
        rs.rocsparse_create_dnmat_descr(ct.byref(B), X.shape[0], X.shape[1], X.stride(0), P(X.data_ptr()), 151, 0)
        rs.rocsparse_create_dnmat_descr(ct.byref(C), n_rows, X.shape[1], Y.stride(0), P(Y.data_ptr()), 151, 0)
        try:
            sz = ct.c_size_t(0)
            args = lambda stage, buf: (self.h, 111, 111, ct.byref(self.one), A, B, ct.byref(self.zero), C,  # noqa: E731
                                       151, alg, stage, ct.byref(sz), buf)
            rc = rs.rocsparse_spmm(*args(1, None))
            if rc != 0:
                return None, rc
            buf = self.torch.empty(max(1, sz.value), dtype=self.torch.uint8, device=X.device)
            rc = rs.rocsparse_spmm(*args(2, P(buf.data_ptr())))
            if rc != 0:
                return None, rc
            return self._timed(lambda: rs.rocsparse_spmm(*args(3, P(buf.data_ptr()))))
        finally:
            rs.rocsparse_destroy_dnmat_descr(B)
            rs.rocsparse_destroy_dnmat_descr(C)
            rs.rocsparse_destroy_spmat_descr(A)

    def sddmm(self, rp, ci, U, V, out):
        """out[e] = <U[row_e], V[col_e]> (fp32, row-major U and V) with rocSPARSE's default algorithm."""
        ct, rs, P = self.ct, self.rs, self.ct.c_void_p
        n_rows, nnz = rp.numel() - 1, ci.numel()
        A, B, C = P(), P(), P()
        rs.rocsparse_create_dnmat_descr(ct.byref(A), n_rows, U.shape[1], U.stride(0), P(U.data_ptr()), 151, 0)
        rs.rocsparse_create_dnmat_descr(ct.byref(B), V.shape[0], V.shape[1], V.stride(0), P(V.data_ptr()), 151, 0)
        rs.rocsparse_create_csr_descr(ct.byref(C), n_rows, V.shape[0], nnz, P(rp.data_ptr()), P(ci.data_ptr()),
                                      P(out.data_ptr()), 2, 2, 0, 151)
        try:
            sz = ct.c_size_t(0)
            head = (self.h, 111, 112, ct.byref(self.one), A, B, ct.byref(self.zero), C, 151, 0)
            rc = rs.rocsparse_sddmm_buffer_size(*head, ct.byref(sz))
            if rc != 0:
                return None, rc
            buf = self.torch.empty(max(1, sz.value), dtype=self.torch.uint8, device=U.device)
            rc = rs.rocsparse_sddmm_preprocess(*head, P(buf.data_ptr()))
            if rc != 0:
                return None, rc
            return self._timed(lambda: rs.rocsparse_sddmm(*head, P(buf.data_ptr())))
        finally:
            rs.rocsparse_destroy_dnmat_descr(A)
            rs.rocsparse_destroy_dnmat_descr(B)
            rs.rocsparse_destroy_spmat_descr(C)


def vendor_compare(calls, torch, reps=5):
    """The step's fp32 SpMM and SDDMM calls timed with rocSPARSE (every CSR
    SpMM algorithm it offers for row-major dense operands; its default
    SDDMM), each output compared with this library's output of the same call
    (max |difference| / max |this library's output|).  Returns per call the
    vendor times, the ratio vendor best / this library, and the differences."""
    try:
        rs = Rocsparse(torch, reps)
    except OSError as e:  # pragma: no cover - library not installed
        return {"error": str(e)}
    out = {}
    for c in calls:
        if c.op not in ("spmm", "sddmm") or c.esize != 4 or "val_idx" in c.kwargs:
            continue
        mine_out = c.kwargs["out"]
        c.run()
        ref = mine_out.clone()
        scale = float(ref.abs().max()) or 1.0
        vout = torch.empty_like(ref)
        res, diff = {}, {}
        if c.op == "spmm":
            for name, alg in Rocsparse.ALGS.items():
                vout.fill_(float("nan"))
                ms, rc = rs.spmm(c.args[0], c.args[1], c.args[2], c.args[3], vout, alg)
                res[name] = round(ms, 4) if ms is not None else f"status {rc}"
                if ms is not None:
                    diff[name] = float((vout - ref).abs().max()) / scale
        else:
            vout.zero_()  # rocSPARSE's SDDMM forms beta * C even for beta = 0
            ms, rc = rs.sddmm(c.args[0], c.args[1], c.args[2], c.args[3], vout)
            res["default"] = round(ms, 4) if ms is not None else f"status {rc}"
            if ms is not None:
                diff["default"] = float((vout - ref).abs().max()) / scale
        ok = [n for n, t in res.items() if isinstance(t, float) and diff.get(n, 1.0) <= 1e-5]
        best = min((res[n] for n in ok), default=None)
        mine = float(np.mean(c.times)) if c.times else None
        out[c.name] = {"rocsparse_ms": res, "rocsparse_best_ms": best, "this_ms": round(mine, 4) if mine else None,
                       "vendor_over_this": round(best / mine, 3) if best and mine else None,
                       "max_rel_diff_vs_this": {n: float(f"{d:.3g}") if np.isfinite(d) else None
                                                for n, d in diff.items()}}
    rs.close()
    return out


def cpu_model():
    """The host CPU's model name, with its family / model / stepping numbers
    (virtual machines often report a generic name)."""
    fields = {}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if not line.strip():
                    break  # the first processor's block
                k, _, v = line.partition(":")
                fields.setdefault(k.strip(), v.strip())
    except OSError:  # pragma: no cover
        pass
    name = fields.get("model name")
    if not name:
        import platform

        return platform.processor() or "unknown"
    ids = [f"{k} {fields[k]}" for k in ("cpu family", "model", "stepping") if k in fields]
    return f"{name} ({', '.join(ids)})" if ids else name


def cpu_baseline(calls, target_s=8.0, runs=3):
    """Times the oracle (as it is) on a bounded sample of the step: the same
    contiguous block of leading rows for every call, sized so that one pass
    over the sample takes about target_s seconds on this host's cores; the
    median of ``runs`` passes.  Also the oracle single-threaded on the two
    tiny attention workloads (2,048 and 384 nodes), whole."""
    import oracle
    from synth import configs

    threads = oracle.default_threads()
    calls = [c for c in calls if c.oracle_fn is not None]

    def run(call, r1, th):
        kind, csr, *ops = call.oracle_fn
        if call.esize == 2:  # bf16 bit patterns, read exactly by the oracle
            ops = [o if o.dtype != np.uint16 else oracle.bf16_to_f32(o) for o in ops]
        t = time.perf_counter()
        if kind == "attention_qk":
            oracle.attention_qk(csr.row_ptr, csr.col_idx, ops[0], ops[1], ops[2], 0.125, 0, r1, th)
        elif kind == "spmm":
            oracle.spmm(csr.row_ptr, csr.col_idx, ops[0], ops[1], 0, r1, th)
        elif kind == "sddmm":
            oracle.sddmm(csr.row_ptr, csr.col_idx, ops[0], ops[1], 0, r1, th)
        elif kind == "attention":
            oracle.attention(csr.row_ptr, csr.col_idx, ops[0], ops[1], 1.0, 0, r1, th)
        else:
            oracle.mha(csr.row_ptr, csr.col_idx, ops[0], ops[1], ops[2], 0.125, 0, r1, th)
        return time.perf_counter() - t

    single = {}
    for name in ("c1", "p4"):
        c = configs.make_config(name)
        csr = c["csr"]
        t = time.perf_counter()
        oracle.attention(csr.row_ptr, csr.col_idx, c["scores"], c["V"], 1.0, 0, csr.n_rows, 1)
        dt = time.perf_counter() - t
        single[f"{name}_attention"] = {"s": round(dt, 5), "GB_s": round(
            b_alg("attention", csr.n_rows, csr.nnz, c["V"].shape[1]) / dt / 1e9, 4), "cores": 1}
    out = {"unit": "GB/s", "cores": threads, "kind": "oracle", "cpu_model": cpu_model(),
           "single_thread": single}
    if not calls:
        return out
    csr = calls[0].oracle_fn[1]
    rp = csr.row_ptr.astype(np.int64)

    def sample(r1):
        t, b = 0.0, 0.0
        for c in calls:
            t += run(c, r1, threads)
            b += b_alg(c.op, r1, int(rp[r1]), c.width, esize=c.esize)
        return t, b

    # calibrate on ~1% of the entries, then size the row block for target_s
    r1 = min(csr.n_rows, max(1, int(np.searchsorted(rp, max(1, csr.nnz // 100)))))
    t_cal, _ = sample(r1)
    frac = (rp[r1] / max(1, csr.nnz)) * target_s / max(t_cal, 1e-3)
    r1 = min(csr.n_rows, max(r1, int(np.searchsorted(rp, int(min(1.0, frac) * csr.nnz)))))
    ts, total_b = [], 0.0
    for _ in range(runs):
        t, total_b = sample(r1)
        ts.append(t)
    total_t = float(np.median(ts))
    out.update({"value": round(total_b / total_t / 1e9, 4), "runs_s": [round(t, 3) for t in ts],
                "sample": f"rows [0, {r1}) ({int(rp[r1])} entries, {100.0 * rp[r1] / max(1, csr.nnz):.2f}% of nnz) "
                          f"of every call of the step, float64 oracle, median of {runs} passes "
                          f"({total_t:.1f} s each)"})
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="c2",
                    help="c2 (default), c1, p4, c3, c4, c5a, c5b, c3pipe, c3fused, c3qk, c3bf16, c3bwd, "
                         "c3bwd_perm, c3bwd_gather, c3qkbwd, c3sweep")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=8.0, help="seconds per pass of the CPU oracle sample")
    ap.add_argument("--no-study", action="store_true", help="skip the selector-vs-fixed-mapping study")
    ap.add_argument("--no-cold", action="store_true", help="skip the cold-cache timing of every call")
    ap.add_argument("--no-format", action="store_true",
                    help="run SpMM / SDDMM with the selector on the plain CSR pattern instead of through a plan "
                         "(no column-part segment format)")
    ap.add_argument("--vendor", action="store_true",
                    help="also time the SpMM / SDDMM calls with rocSPARSE (a measured comparison, not a dispatch)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="for counter runs: first run one device copy of 1 GiB (a known-size reference for HBM "
                         "counters), and launch a short spin kernel before each call of the timed steps (outside "
                         "its timed region) so that the dispatches can be told apart by call")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this library's hot path runs on a single MI355X "
              "(multi-GPU sharding is a design note, not built); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import csr_sparse_attention_amd as csa

    torch.cuda.init()
    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        src.fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    stream_ref = stream_bandwidth(torch)
    calls, gen_s = build_workload(args.config, torch, csa)
    check_shapes(calls)
    print(f"[bench] workload {args.config}: {len(calls)} calls, generated in {gen_s:.1f}s", file=sys.stderr, flush=True)
    # SpMM / SDDMM: one plan per call (layout and schedule chosen together
    # by the library); the other calls: the selector (histogram, signature,
    # cost model, probes) once per call
    sel = {}
    for c in calls:
        if c.op in NO_SCHEDULE:
            continue
        if c.op in ("spmm", "sddmm") and not args.no_format and "val_idx" not in c.kwargs:
            info = make_plan(c, csa, torch)
            pl = c.plan
            sel[c.name] = {"plan": {"parts": pl.parts, "whole_below": pl.whole_below, "segments": pl.n_seg,
                                    **info}, "schedule": pl.schedule.as_dict()}
            print(f"[bench] {c.name}: {pl} created in {info['plan_create_ms']:.1f} ms, replayed in "
                  f"{info['plan_replay_ms']:.1f} ms", file=sys.stderr, flush=True)
            continue
        torch.cuda.synchronize()
        t = time.perf_counter()
        s, sig = c.select(csa)
        torch.cuda.synchronize()
        first = time.perf_counter() - t
        t = time.perf_counter()
        s2, sig2 = c.select(csa, mode="replay")
        torch.cuda.synchronize()
        replay = time.perf_counter() - t
        assert bytes(s) == bytes(s2) and sig == sig2
        c.schedule = s
        sel[c.name] = {"schedule": s.as_dict(), "signature": f"{sig:016x}", "select_ms": round(first * 1e3, 3),
                       "replay_select_ms": round(replay * 1e3, 3)}
        print(f"[bench] {c.name}: {s} select {first * 1e3:.1f} ms", file=sys.stderr, flush=True)

    dom = max(calls, key=lambda c: c.bytes)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        for c in calls:
            c.run()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    per_call = {c.name: [] for c in calls}
    cev = {c.name: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                    for _ in range(args.steps)] for c in calls}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        for c in calls:
            a, b = cev[c.name][k]
            if args.calibrate_copy:
                torch.cuda._sleep(1)  # a spin kernel before each call: counter runs split the dispatches by call
            a.record(stream)
            c.run()
            b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for c in calls:
        per_call[c.name] = [a.elapsed_time(b) for a, b in cev[c.name]]
        c.times = per_call[c.name]
    step_bytes = sum(c.bytes for c in calls)
    ms_step = wall * 1e3 / args.steps
    value = step_bytes / (wall / args.steps) / 1e9
    gnnzf = sum(c.nnz * c.width for c in calls) / (wall / args.steps) / 1e9

    cold = {} if args.no_cold else cold_times(calls, torch)
    kernels = {}
    for c in calls:
        ms = float(np.mean(per_call[c.name]))
        kernels[c.name] = {
            "ms": round(ms, 4), "GB_s": round(c.bytes / (ms * 1e-3) / 1e9, 1),
            "GNNZF_s": round(c.nnz * c.width / (ms * 1e-3) / 1e9, 1),
            "frac_hbm": round(c.bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "bytes_alg": c.bytes, **sel.get(c.name, {})}
        if c.name in cold:
            mc = cold[c.name]
            kernels[c.name].update({"ms_cold": round(mc, 4), "GB_s_cold": round(c.bytes / (mc * 1e-3) / 1e9, 1),
                                    "frac_hbm_cold": round(c.bytes / (mc * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)})
    dom_ms = float(np.mean(per_call[dom.name]))
    gather_rate = dom.bytes / (dom_ms * 1e-3) / 1e9
    model = compulsory_bytes(dom, torch)
    traffic = committed_traffic(args.config, dom)
    # HBM rate of the dominant call: counted bytes (FETCH_SIZE + WRITE_SIZE of
    # its kernels, scaled by the counters' reading of a copy of known size)
    # over the live HIP-event time; the compulsory-traffic model stands in
    # when no counter record matches the current sources and schedule
    hbm_bytes = traffic if traffic else model
    achieved = hbm_bytes / (dom_ms * 1e-3) / 1e9
    for c in calls:
        kernels[c.name]["bytes_compulsory"] = compulsory_bytes(c, torch)
        # counted HBM bytes of the call (committed counter record for these sources, layout and schedule)
        t = committed_traffic(args.config, c) if c.op not in NO_SCHEDULE else None
        kernels[c.name]["traffic_bytes"] = t
        kernels[c.name]["frac_hbm_counted"] = (round(t / (kernels[c.name]["ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
                                               if t else None)
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if calls[0].op == "mha" or calls[0].esize == 2 else "f32",
        "data": "synthetic",
        "config": {"workload": {"c2": "CSR SpMM, power-law graph 232,965 rows ~114.6M nnz, F in {32,64,128,602}",
                                "c1": "fused CSR attention, 2,048 nodes Poisson(18), F=32",
                                "p4": "fused CSR attention, 384 nodes Poisson(18), F=64",
                                "c3": "CSR SpMM F in {100,128} + SDDMM K=128, log-normal graph 2,449,029 rows ~123.7M nnz",
                                "c4": "skew stress SpMM + SDDMM, 1M rows 32M nnz Zipf(1.5), F in {4,8,16,32}",
                                "c5a": "8-head bf16 CSR attention on the 2,449,029-row log-normal graph",
                                "c5b": "8-head bf16 CSR attention, 16,384 tokens, window 512 + 64 global",
                                "c3pipe": "unfused single-head fp32 attention on the log-normal graph: "
                                          "SDDMM K=64 -> row softmax -> SpMM F=64",
                                "c3fused": "single-head fp32 attention on the log-normal graph: "
                                           "SDDMM K=64 -> fused softmax-SpMM F=64",
                                "c3qk": "single-head fp32 attention on the log-normal graph from Q, K, V of "
                                        "width 64 in one pass (SDDMM -> softmax -> SpMM, scores in registers)",
                                "c3bf16": "CSR SpMM F=128 + SDDMM K=128 over bf16 features, fp32 accumulation, "
                                          "log-normal graph 2,449,029 rows ~123.7M nnz",
                                "c3sweep": "CSR SpMM on the log-normal graph at F in {128,256,384,512}: "
                                           "gathered operand of 1.25 to 5.0 GB",
                                "c3qkbwd": "backward of single-head fp32 attention from Q, K, V (width 64) on "
                                           "the log-normal graph: SDDMM scores, row softmax, P into A^T's order, "
                                           "dV and dP in one pass over A^T, dP back, softmax backward, dQ (SpMM), "
                                           "d scores into A^T's order, dK (SpMM on A^T)",
                                "c3bwd": "backward of single-head fp32 attention on the log-normal graph, F=64: "
                                         "row softmax, P into A^T's order (two-pass permutation), dV = P^T dOut "
                                         "and dP = dOut V^T in one pass over A^T, dP back into A's order, "
                                         "softmax backward",
                                "c3bwd_perm": "backward of single-head fp32 attention on the log-normal graph, "
                                              "F=64: row softmax, SDDMM dP, softmax backward, SpMM dV on A^T "
                                              "reading P through the transposed pattern's perm",
                                "c3bwd_gather": "backward of single-head fp32 attention on the log-normal graph, "
                                                "F=64: row softmax, SDDMM dP, softmax backward, gather P^T, "
                                                "SpMM dV on A^T"
                                }[args.config],
                   "name": args.config, "n_rows": calls[0].n_rows, "nnz": calls[0].nnz,
                   "widths": [c.width for c in calls], "parallelism": "1 GPU"},
        "gnnzf_per_s": round(gnnzf, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "achieved_from": ("counted HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, profiles/traffic.json)"
                                       if traffic else "compulsory-traffic model (no counter record for these sources)"),
                     "kernel": dom.name, "launch_ms": round(dom_ms, 4),
                     "bytes_compulsory": model, "compulsory_GB_s": round(model / (dom_ms * 1e-3) / 1e9, 1),
                     "compulsory_frac": round(model / (dom_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "traffic_over_compulsory": round(traffic / model, 3) if traffic else None,
                     "bytes_gathered_alg": dom.bytes, "gather_rate_GB_s": round(gather_rate, 1)},
        "kernels": kernels,
        "stream_measured": stream_ref,
        **({"transpose_once_ms": round(build_workload.transpose_ms, 3),
            "transpose_first_call_ms": round(build_workload.transpose_first_ms, 3)}
           if getattr(build_workload, "transpose_ms", None) is not None else {}),
    }
    result["roofline"]["frac_of_measured_copy"] = round(achieved / stream_ref["copy_GB_s"], 4)
    if not args.no_study:
        print("[bench] selector study: every candidate schedule of every call", file=sys.stderr, flush=True)
        result["selector"] = selector_study(calls, torch, csa)
        result["selector_worst_ratio"] = max(v["selected_over_best"] for v in result["selector"].values())
    if args.vendor:
        print("[bench] vendor comparison (rocSPARSE)", file=sys.stderr, flush=True)
        result["vendor"] = vendor_compare(calls, torch)
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(calls, args.cpu_seconds)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
