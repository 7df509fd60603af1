"""Plant plausible mistakes in copies of the CPU oracle and check that the pins
catch every one of them (CPU only; mutants are built with gcc in a temp dir)."""
import inspect
import os
import subprocess
import tempfile

import pytest

import tests.test_oracle_pins as pins
from oracle import loki_oracle

SRC = os.path.join(os.path.dirname(loki_oracle.__file__), "loki_oracle.c")

# (name, original text, mutated text)
MUTANTS = [
    ("transposed_P", "* P[(size_t)i * D + j]", "* P[(size_t)j * D + i]"),
    ("no_softmax_scale", "z[i] = scale * acc;", "z[i] = acc;"),
    ("smallest_instead_of_largest", "if (x->s > y->s) return -1;", "if (x->s < y->s) return -1;"),
    ("ties_to_higher_index", "return (x->t > y->t) - (x->t < y->t);",
     "return (x->t < y->t) - (x->t > y->t);"),
    ("last_d_dims", "acc += qr[j] * load_elem(krot, dtype, head_off + (size_t)t * D + j);",
     "acc += qr[D - 1 - j] * load_elem(krot, dtype, head_off + (size_t)t * D + D - 1 - j);"),
    ("dropped_normalisation", "out[j] /= L;", "out[j] /= 1.0;"),
    ("scores_use_only_d_minus_1", "for (int j = 0; j < d; j++)\n                acc += qr[j]",
     "for (int j = 1; j < d; j++)\n                acc += qr[j]"),
    ("wrong_gqa_map", "int kv = h / g;\n        double *qr", "int kv = h % Hkv;\n        double *qr"),
    ("final_logits_low_dim_only", "for (int j = 0; j < D; j++)\n            acc += qr[j] * load_elem(krot",
     "for (int j = 0; j < D / 2; j++)\n            acc += qr[j] * load_elem(krot"),
    ("half_round_down", "if (frac > 0.5 || (frac == 0.5 && fmod(f, 2.0) != 0.0))",
     "if (frac > 0.5)"),
    ("pca_no_scale", "w[t] = scale * dot;", "w[t] = dot;"),
    ("pca_all_coordinates", "for (int c = 0; c < d; c++)\n                dot +=",
     "for (int c = 0; c < D; c++)\n                dot +="),
    ("pca_mean_instead_of_softmax", "o[c] = acc / denom;", "o[c] = acc / S;"),
    ("cov_not_centred", "xc[i] = load_elem(keys, dtype, kbase + (size_t)t * D + i) - mean[i];",
     "xc[i] = load_elem(keys, dtype, kbase + (size_t)t * D + i);"),
    ("cov_n_minus_1", "C[e] /= (double)n;", "C[e] /= (double)(n - 1);"),
    ("bf16_bias_off", "return sign | (uint16_t)encode_small_float(fabs(v), 7, -126, 127, ovf, 0x7f80);",
     "return sign | (uint16_t)encode_small_float(fabs(v), 7, -126, 126, ovf, 0x7f80);"),
]


def _pin_functions():
    out = []
    for name, fn in inspect.getmembers(pins, inspect.isfunction):
        if not name.startswith("test_"):
            continue
        params = list(inspect.signature(fn).parameters)
        marks = getattr(fn, "pytestmark", [])
        calls = []
        for m in marks:
            if m.name == "parametrize":
                argnames = [a.strip() for a in m.args[0].split(",")] if isinstance(m.args[0], str) else list(m.args[0])
                for vals in m.args[1]:
                    vals = vals if isinstance(vals, (tuple, list)) else (vals,)
                    calls.append(dict(zip(argnames, vals)))
        if not calls:
            calls = [{}]
        out.append((name, fn, params, calls))
    return out


def _run_pins():
    """Run every pin against the currently loaded oracle; return names that failed."""
    failed = []
    for name, fn, params, calls in _pin_functions():
        for kw in calls:
            args = dict(kw)
            if "oracle" in params:
                args["oracle"] = loki_oracle
            try:
                fn(**args)
            except Exception:  # noqa: BLE001 - any failure counts as caught
                failed.append(name)
                break
    return failed


@pytest.mark.parametrize("mutant", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(mutant):
    name, orig, new = mutant
    src = open(SRC).read()
    assert src.count(orig) == 1, f"mutation site for {name} not unique/absent"
    with tempfile.TemporaryDirectory() as td:
        c = os.path.join(td, "m.c")
        so = os.path.join(td, "libm.so")
        open(c, "w").write(src.replace(orig, new))
        subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-o", so, c,
                        "-lm"], check=True)
        saved_lib, saved_path = loki_oracle._lib, loki_oracle.LIB_PATH
        try:
            loki_oracle._lib, loki_oracle.LIB_PATH = None, so
            failed = _run_pins()
        finally:
            loki_oracle._lib, loki_oracle.LIB_PATH = saved_lib, saved_path
    assert failed, f"mutant {name} survived every pin"


def test_unmutated_oracle_passes_every_pin():
    assert _run_pins() == []
