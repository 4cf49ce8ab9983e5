"""Host logic of bench.py (CPU only): the one-GPU guard, the roofline
arithmetic and the algorithmic byte and flop counts the roofline uses."""
import importlib.util
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)
    assert r.stdout.strip() == "" or not r.stdout.strip().startswith("{")


def test_roof_entry_picks_the_binding_roof():
    b = _bench()
    # 8 MB at 8 TB/s is 1 us; 2.5 GFLOP at 2.5 PFLOP/s is 1 us
    e = b.roof_entry(8_000_000, 1_000_000, 2.0, "bf16")
    assert e["bound"] == "hbm" and abs(e["roof_us"] - 1.0) < 1e-9 and abs(e["frac"] - 0.5) < 1e-9
    e = b.roof_entry(1_000, 5_000_000_000, 4.0, "bf16")
    assert e["bound"] == "mfma" and abs(e["roof_us"] - 2.0) < 1e-9 and abs(e["frac"] - 0.5) < 1e-9
    # the fp32 path is priced against the vector fp32 peak (157.3 TFLOP/s)
    e = b.roof_entry(1_000, 157_300_000, 1.0, "f32")
    assert e["bound"] == "mfma" and abs(e["roof_us"] - 1.0) < 1e-9


def test_algorithmic_work_of_the_default_workload():
    b = _bench()
    from workloads import WORKLOADS
    wl = WORKLOADS[b.DEFAULT_WORKLOAD]
    assert (wl.B, wl.N, wl.hidden, wl.V, wl.Hq, wl.Hkv, wl.D) == (1, 64, 4096, 151936, 32, 8, 128)
    depth = np.arange(64, dtype=np.int32)[None, :] % 20
    a = {"seq_lens": np.array([1024], np.int32), "depth": depth}
    path = np.zeros((1, 21), np.int32)
    path[0, :5] = [0, 3, 9, 10, 40]       # 4 of 5 rows move (row i != i)
    path_len = np.array([5], np.int32)
    w = b.algorithmic_work(wl, a, path, path_len)
    # LM head: the bf16 vocabulary matrix and hidden states once, one int32 per row
    assert w["lmhead"] == (151936 * 4096 * 2 + 64 * 4096 * 2 + 4 * 64, 2 * 64 * 4096 * 151936)
    assert w["lmhead"][0] == 1_245_184_256
    # attention: prefix K and V once; per node its Q, output and own K/V, and its parent
    prefix = 2 * 1024 * 8 * 128 * 2
    per_node = 2 * 32 * 128 * 2 + 2 * 8 * 128 * 2 + 4
    assert w["attn"][0] == prefix + 64 * per_node
    # flops: 4 Hq D per visible key; node i sees the prefix, its ancestors and itself
    assert w["attn"][1] == 4 * 32 * 128 * int((1024 + depth + 1).sum())
    # compaction: K and V rows read and written for each moved row, lengths in and out
    assert w["compact"][0] == 4 * 4 * 8 * 128 * 2 + 8
