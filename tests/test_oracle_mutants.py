"""The pins catch plausible mistakes: each mutant below plants one mistake in
a copy of oracle.c (a dropped term or factor, a flipped sign, a wrong or
transposed index, a missing normalisation, a missing max subtraction), the
copy is built, and at least one pin of tests/test_oracle_pins.py must fail on
it.  Mutants never index outside the arrays the pins pass in."""

import os
import subprocess

import pytest

import oracle
import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

# (name, [(old, new, occurrence index or None for all)])
MUTANTS = [
    ("spmm drops the edge value", [("y[f] += a * (double)x[f];", "y[f] += (double)x[f];", None)]),
    ("spmm flips the sign", [("y[f] += a * (double)x[f];", "y[f] -= a * (double)x[f];", None)]),
    ("spmm reads the value of the wrong entry", [("(double)vals[e] : 1.0", "(double)vals[row_ptr[i]] : 1.0", None)]),
    ("spmm gathers the first column only", [("const float *x = X + (int64_t)col_idx[e] * ldx;",
                                             "const float *x = X + (int64_t)col_idx[row_ptr[i]] * ldx;", None)]),
    ("spmm drops the last entry of a row", [(
        "for (int64_t e = row_ptr[i]; e < row_ptr[i + 1]; ++e) {\n            double a",
        "for (int64_t e = row_ptr[i]; e < row_ptr[i + 1] - 1; ++e) {\n            double a", None)]),
    ("spmm magnitude keeps the sign", [("g[f] += fabs(a) * fabs((double)x[f]);", "g[f] += a * fabs((double)x[f]);",
                                        None)]),
    ("sddmm transposes the dense operands", [("const float *v = V + (int64_t)col_idx[e] * ldv;",
                                              "const float *v = V + (int64_t)col_idx[row_ptr[i]] * ldv;", None)]),
    ("sddmm drops the first feature", [("for (int64_t k = 0; k < K; ++k) {", "for (int64_t k = 1; k < K; ++k) {",
                                        None)]),
    ("sddmm writes the magnitude as the value", [("out[e - base] = s;", "out[e - base] = m;", None)]),
    ("attention without the max subtraction", [
        ("l += exp(scale * (double)scores[e] - m);", "l += exp(scale * (double)scores[e]);", None),
        ("double p = exp(scale * (double)scores[e] - m) / l;", "double p = exp(scale * (double)scores[e]) / l;",
         None)]),
    ("attention subtracts the minimum", [("if (t > m) m = t;", "if (t < m) m = t;", None)]),
    ("attention without normalisation", [("double p = exp(scale * (double)scores[e] - m) / l;",
                                          "double p = exp(scale * (double)scores[e] - m);", None)]),
    ("attention drops the scale in the weights", [("double p = exp(scale * (double)scores[e] - m) / l;",
                                                   "double p = exp((double)scores[e] - m) / l;", None)]),
    ("attention aggregates the first neighbour only", [("const float *v = Vv + (int64_t)col_idx[e] * ldv;",
                                                        "const float *v = Vv + (int64_t)col_idx[b] * ldv;", None)]),
    ("attention sums exp over all but the first entry", [("for (int64_t e = b; e < end; ++e) l += exp",
                                                          "for (int64_t e = b + 1; e < end; ++e) l += exp", None)]),
    ("multi-head scores use head 0's keys", [(
        "const uint16_t *k = K + (int64_t)col_idx[e] * HD + h * D;\n                const uint16_t *v",
        "const uint16_t *k = K + (int64_t)col_idx[e] * HD;\n                const uint16_t *v", None)]),
    ("multi-head weights drop the scale", [("double p = exp(scale * t - m) / l;", "double p = exp(t - m) / l;",
                                            None)]),
    ("multi-head values of head 0", [("const uint16_t *v = V + (int64_t)col_idx[e] * HD + h * D;",
                                      "const uint16_t *v = V + (int64_t)col_idx[e] * HD;", None)]),
    ("fp32 q-k scores use head 0's keys", [(
        "const float *kq = K + (int64_t)col_idx[e] * HD + h * D;\n                const float *vq",
        "const float *kq = K + (int64_t)col_idx[e] * HD;\n                const float *vq", None)]),
    ("fp32 q-k weights from the first neighbour's key", [(
        "const float *kq = K + (int64_t)col_idx[e] * HD + h * D;\n                const float *vq",
        "const float *kq = K + (int64_t)col_idx[b] * HD + h * D;\n                const float *vq", None)]),
    ("fp32 q-k weights drop the scale", [("double p = exp(scale * t - m) / l;\n                if (probs) probs[(e - base) * H + h] = p;\n                for (int64_t d = 0; d < D; ++d) {\n                    y[h * D + d] += p * (double)vq[d];",
                                          "double p = exp(t - m) / l;\n                if (probs) probs[(e - base) * H + h] = p;\n                for (int64_t d = 0; d < D; ++d) {\n                    y[h * D + d] += p * (double)vq[d];", None)]),
    ("fp32 q-k values of head 0", [("const float *vq = V + (int64_t)col_idx[e] * HD + h * D;",
                                    "const float *vq = V + (int64_t)col_idx[e] * HD;", None)]),
    ("fp32 q-k drops the last feature of the dot product", [(
        "for (int64_t d = 0; d < D; ++d) t += (double)q[d] * (double)kq[d];",
        "for (int64_t d = 0; d < D - 1; ++d) t += (double)q[d] * (double)kq[d];", None)]),
    ("bfloat16 widened with the wrong shift", [("uint32_t u = (uint32_t)b << 16;", "uint32_t u = (uint32_t)b << 15;",
                                                None)]),
    ("softmax backward drops the row sum", [("out[e - base] = scale * p * ((double)grad[e] - S);",
                                             "out[e - base] = scale * p * (double)grad[e];", None)]),
    ("softmax backward drops the scale", [("out[e - base] = scale * p * ((double)grad[e] - S);",
                                           "out[e - base] = p * ((double)grad[e] - S);", None)]),
    ("softmax backward sums g instead of p g", [("S += (double)probs[e] * (double)grad[e];",
                                                 "S += (double)grad[e];", None)]),
    ("attention backward dots with the wrong value row", [(
        "const float *v = Vv + (int64_t)col_idx[e] * F;\n            double dp",
        "const float *v = Vv + (int64_t)col_idx[b] * F;\n            double dp", None)]),
    ("attention backward flips the sign", [("ds[e - base] = scale * p * (ds[e - base] - S);",
                                            "ds[e - base] = scale * p * (S - ds[e - base]);", None)]),
    ("transpose product gathers by column", [("const float *y = dY + i * F;",
                                              "const float *y = dY + (i % n_cols) * F;", None)]),
    ("transpose product scatters to the row", [("double *x = dX + (int64_t)col_idx[e] * F;",
                                                "double *x = dX + (i % n_cols) * F;", None)]),
]


def all_pins():
    """Every oracle pin, as (name, callable)."""
    out = []
    for name in dir(pins):
        if not name.startswith("test_"):
            continue
        fn = getattr(pins, name)
        params = getattr(fn, "pytestmark", [])
        seeds = None
        for m in params:
            if m.name == "parametrize" and m.args[0] == "seed":
                seeds = list(m.args[1])
        argnames = fn.__code__.co_varnames[:fn.__code__.co_argcount]
        if "oracle_lib" not in argnames:
            continue
        if seeds is None:
            out.append((name, lambda fn=fn: fn(oracle)))
        else:
            for s in seeds[:4]:
                out.append((f"{name}[{s}]", lambda fn=fn, s=s: fn(oracle, s)))
    return out


def build_mutant(tmp_path, edits):
    src = open(SRC).read()
    for old, new, _ in edits:
        assert src.count(old) >= 1, f"mutation site not found: {old!r}"
        src = src.replace(old, new)
    c = tmp_path / "mutant.c"
    c.write_text(src)
    so = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math", "-ffp-contract=off",
                           "-o", str(so), str(c), "-lm"])
    return str(so)


def test_unmutated_oracle_passes_every_pin():
    failures = []
    for name, fn in all_pins():
        try:
            fn()
        except Exception as e:  # pragma: no cover - reported below
            failures.append((name, repr(e)[:200]))
    assert not failures


@pytest.mark.parametrize("name,edits", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, name, edits):
    so = build_mutant(tmp_path, edits)
    caught = []
    with oracle.use_library(so):
        for pin, fn in all_pins():
            try:
                fn()
            except Exception:
                caught.append(pin)
    assert caught, f"no pin catches the mutant '{name}'"



# Mistakes planted in a copy of the Python structure oracle (both of its
# constructions of the column-part segment format where the mistake is a
# misreading of the definition rather than a slip in one of them).
PY_SRC = os.path.join(os.path.dirname(oracle.__file__), "structure.py")
PY_MUTANTS = [
    ("format reverses equal keys (unstable order)", [
        ('perm = np.argsort(key, kind="stable")', 'perm = np.argsort(-key, kind="stable")[::-1]')]),
    ("format parts columns by proportional scaling", [
        ("part = np.where(deg[rows] < whole_below, parts, ci // part_cols)",
         "part = np.where(deg[rows] < whole_below, parts, ci * parts // max(n_cols, 1))"),
        ("return parts if rp[r + 1] - rp[r] < whole_below else ci[e] // part_cols",
         "return parts if rp[r + 1] - rp[r] < whole_below else ci[e] * parts // n_cols")]),
    ("format keeps rows of exactly whole_below entries whole", [
        ("part = np.where(deg[rows] < whole_below, parts, ci // part_cols)",
         "part = np.where(deg[rows] <= whole_below, parts, ci // part_cols)"),
        ("return parts if rp[r + 1] - rp[r] < whole_below else ci[e] // part_cols",
         "return parts if rp[r + 1] - rp[r] <= whole_below else ci[e] // part_cols")]),
    ("format puts whole rows before the column parts", [
        ("part = np.where(deg[rows] < whole_below, parts, ci // part_cols)",
         "part = np.where(deg[rows] < whole_below, 0, ci // part_cols + 1)"),
        ("return parts if rp[r + 1] - rp[r] < whole_below else ci[e] // part_cols",
         "return 0 if rp[r + 1] - rp[r] < whole_below else ci[e] // part_cols + 1")]),
    ("format orders segments by row first", [
        ("key = part * n_rows + rows", "key = rows * (parts + 1) + part"),
        ("    for p in range(parts + 1):\n        for r in range(n_rows):",
         "    for r in range(n_rows):\n        for p in range(parts + 1):")]),
    ("format lists a row's segments last part first", [
        ('row_seg = np.argsort(seg_row, kind="stable")',
         'row_seg = np.lexsort((-np.arange(len(seg_row)), seg_row))'),
        ("if seg_row[s] == r]  # ascending", "if seg_row[s] == r][::-1]  # ascending")]),
    ("format drops the last segment's end", [
        ('"seg_ptr": np.r_[starts, len(k)]', '"seg_ptr": np.r_[starts, len(k) - 1]'),
        ("    seg_ptr.append(len(perm))\n    row_seg_ptr", "    seg_ptr.append(len(perm) - 1)\n    row_seg_ptr")]),
]


def structure_pins():
    out = [("hand example", pins.test_hybrid_format_hand_example)]
    out += [(f"bruteforce[{s}]", lambda s=s: pins.test_hybrid_format_bruteforce(s)) for s in range(8)]
    out += [(f"invariants[{s}]", lambda s=s: pins.test_hybrid_format_invariants(s)) for s in range(4)]
    out += [(f"identity[{s}]", lambda s=s: pins.test_hybrid_product_identity(oracle, s)) for s in range(4)]
    return out


def test_unmutated_structure_passes_every_pin():
    for name, fn in structure_pins():
        fn()


@pytest.mark.parametrize("name,edits", PY_MUTANTS, ids=[m[0] for m in PY_MUTANTS])
def test_pins_catch_structure_mutant(monkeypatch, name, edits):
    import types

    src = open(PY_SRC).read()
    for old, new in edits:
        assert src.count(old) == 1, f"mutation site not found: {old!r}"
        src = src.replace(old, new)
    mod = types.ModuleType("structure_mutant")
    exec(compile(src, "structure_mutant.py", "exec"), mod.__dict__)
    for fn in ("hybrid_format", "hybrid_format_loops"):
        monkeypatch.setattr(oracle, fn, getattr(mod, fn))
    caught = []
    for pin, fn in structure_pins():
        try:
            fn()
        except Exception:
            caught.append(pin)
    assert caught, f"no pin catches the mutant '{name}'"
