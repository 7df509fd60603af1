"""bench.py on the CPU: the one-GPU contract and the parity check of its
cpu_baseline leg (fed with the oracle's own results, then with a corrupted
output and a corrupted index set)."""
import importlib.util
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402
from oracle import loki_oracle as oracle  # noqa: E402


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_cpu_baseline_parity_check():
    bench = _bench()
    wl = W.custom(name="tiny", wid=400, B=1, Hq=4, Hkv=2, D=128, S=600, d=32, k=64,
                  dtype="f16", tau=40.0, n_calib=2048)
    x = W.generate(wl)
    r = oracle.decode(x["q"], x["krot"], x["v"], x["P"], wl.d, wl.k, wl.dtype)
    good = {"out": r["out"].copy(), "idx": r["idx"].copy()}
    res = bench.cpu_baseline(wl, x, 0.3, good)
    assert res["parity"]["ok"] and res["parity"]["units"] == 4
    assert res["parity"]["max_rel_out"] == 0.0
    # a wrong output
    bad = {"out": good["out"].copy(), "idx": good["idx"]}
    bad["out"][0, 1] *= 1.01
    assert not bench.cpu_baseline(wl, x, 0.3, bad)["parity"]["ok"]
    # a token far below the threshold in place of a selected one
    bad = {"out": good["out"], "idx": good["idx"].copy()}
    s = r["scores"][0, 2]
    low = int(np.argmin(s))
    row = bad["idx"][0, 2]
    if low not in row:
        row[np.argmin(s[row])] = low
        row.sort()
        res = bench.cpu_baseline(wl, x, 0.3, bad)["parity"]
        assert res["index_sets_within_tie_band"] == 3 and not res["ok"]


def test_parity_check_reports_elementwise_error():
    bench = _bench()
    wl = W.custom(name="tiny", wid=401, B=1, Hq=2, Hkv=2, D=128, S=500, d=32, k=50,
                  dtype="bf16", tau=40.0, n_calib=2048)
    x = W.generate(wl)
    r = oracle.decode(x["q"], x["krot"], x["v"], x["P"], wl.d, wl.k, wl.dtype)
    out = r["out"].copy()
    # one small element off by 1% of its own size: tiny normwise, large elementwise
    j = int(np.argmin(np.abs(out[0, 1])))
    out[0, 1, j] += 0.01 * max(abs(out[0, 1, j]), 1e-3 * np.abs(out[0, 1]).max())
    res = bench.parity_check(wl, x, out, r["idx"], [0, 1])
    assert res["ok"] and res["units"] == 2
    assert res["max_rel_out"] < 1e-3
    assert abs(res["max_rel_out_elementwise_floor"] - 0.01) < 1e-6


def test_gather_rows_counts_the_union_per_kv_group():
    bench = _bench()
    wl = W.custom(name="tiny", wid=402, B=2, Hq=4, Hkv=2, D=128, S=100, d=32, k=5,
                  dtype="f16", tau=40.0, n_calib=64)
    idx = np.zeros((2, 4, 5), np.int32)
    idx[0, 0] = [0, 1, 2, 3, 4]
    idx[0, 1] = [0, 1, 2, 3, 4]      # same set: group (0, 0) gathers 5 rows
    idx[0, 2] = [0, 1, 2, 3, 4]
    idx[0, 3] = [5, 6, 7, 8, 9]      # disjoint: group (0, 1) gathers 10
    idx[1, 0] = [0, 2, 4, 6, 8]
    idx[1, 1] = [1, 2, 3, 4, 5]      # shares 2 and 4: group (1, 0) gathers 8
    idx[1, 2] = [10, 11, 12, 13, 14]
    idx[1, 3] = [10, 11, 12, 13, 15]  # group (1, 1) gathers 6
    union, nominal = bench.gather_rows(wl, idx)
    assert union == 5 + 10 + 8 + 6
    assert nominal == 2 * 4 * 5
