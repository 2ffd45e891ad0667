"""Host-side checks of the benchmark's workload assembly (no GPU): every
operand must have the size its call implies before anything is launched."""

import importlib.util
import os

import pytest

torch = pytest.importorskip("torch")

_spec = importlib.util.spec_from_file_location("bench", os.path.join(os.path.dirname(__file__), "..", "bench.py"))
bench = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(bench)


def _call(op, args, n_rows, nnz, **kw):
    return bench.Call("x", op, None, args, kw, n_rows, nnz, 1, None)


def test_shapes_accepted():
    rp, ci, v = torch.zeros(11, dtype=torch.int32), torch.zeros(40, dtype=torch.int32), torch.zeros(40)
    bench.check_shapes([_call("row_softmax", (rp, v), 10, 40, out=torch.zeros(40)),
                        _call("spmm", (rp, ci, v, torch.zeros(5, 3)), 10, 40),
                        _call("gather", (ci, v, v), 10, 40)])


def test_per_entry_array_of_the_wrong_length_is_caught():
    # scores drawn per row instead of per entry
    rp = torch.zeros(11, dtype=torch.int32)
    with pytest.raises(AssertionError):
        bench.check_shapes([_call("row_softmax", (rp, torch.zeros(10)), 10, 40)])
    with pytest.raises(AssertionError):
        bench.check_shapes([_call("row_softmax_backward", (rp, torch.zeros(40), torch.zeros(39)), 10, 40)])
    with pytest.raises(AssertionError):
        bench.check_shapes([_call("spmm", (rp, torch.zeros(40, dtype=torch.int32), torch.zeros(39),
                                           torch.zeros(5, 3)), 10, 40)])


def test_committed_traffic_records_are_self_consistent():
    # each record's per-launch bytes follow from its counter medians and the
    # copy-calibrated factors, and names sources that exist and a summary file
    import json

    root = os.path.join(os.path.dirname(__file__), "..")
    with open(os.path.join(root, "profiles", "traffic.json")) as f:
        recs = json.load(f)
    assert recs.get("c2"), "the default workload has a record"
    for config, lst in recs.items():
        for r in (lst if isinstance(lst, list) else [lst]):
            fk = r["fetch_kib"] if isinstance(r["fetch_kib"], list) else [r["fetch_kib"]]
            wk = r["write_kib"] if isinstance(r["write_kib"], list) else [r["write_kib"]]
            want = sum(f * r["fetch_factor"] * 1024 + w * r["write_factor"] * 1024 for f, w in zip(fk, wk))
            assert abs(r["traffic_bytes"] - want) <= 1, (config, r["call"])
            assert 1.9 < r["fetch_factor"] < 2.1 and 0.95 < r["write_factor"] < 1.05
            assert set(r["schedule"]) <= {"mapping", "vec", "group_lanes", "passes", "chunk_items", "long_row", "flags"}
            for src in r["sources"]:
                assert os.path.exists(os.path.join(root, src)), src
            assert os.path.exists(os.path.join(root, r["profile"]))


def test_cpu_model_names_the_host():
    """The CPU baseline's model string: /proc/cpuinfo's model name of the
    first processor, with its family / model / stepping numbers."""
    name = bench.cpu_model()
    assert isinstance(name, str) and name
    if os.path.exists("/proc/cpuinfo"):
        with open("/proc/cpuinfo") as f:
            first = [l.split(":", 1)[1].strip() for l in f if l.startswith("model name")][:1]
        if first:
            assert name.startswith(first[0]) and "cpu family" in name
