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
    """The default line is the largest workload: Qwen3-30B-A3B-shaped
    attention and LM head, 4 sequences of 1024 nodes on 4096-token prefixes."""
    b = _bench()
    from workloads import WORKLOADS
    wl = WORKLOADS[b.DEFAULT_WORKLOAD]
    assert (wl.B, wl.N, wl.hidden, wl.V, wl.Hq, wl.Hkv, wl.D) == (4, 1024, 2048, 151936, 32, 4, 128)
    depth = np.tile(np.arange(1024, dtype=np.int32) % 25, (4, 1))
    a = {"seq_lens": np.full(4, 4096, np.int32), "depth": depth}
    path = np.full((4, 32), -1, np.int32)
    path_len = np.array([5, 1, 3, 2], np.int32)
    path[0, :5] = [0, 3, 9, 10, 40]       # 4 of 5 rows move (row i != i)
    path[1, :1] = [0]                     # none
    path[2, :3] = [0, 1, 7]               # 1 moves
    path[3, :2] = [0, 2]                  # 1 moves
    w = b.algorithmic_work(wl, a, path, path_len)
    # LM head: the bf16 vocabulary matrix and hidden states once, one int32 per row
    M = 4 * 1024
    assert w["lmhead"] == (151936 * 2048 * 2 + M * 2048 * 2 + 4 * M, 2 * M * 2048 * 151936)
    assert w["lmhead"] == (639_123_456, 2_549_063_090_176)
    # attention: prefix K and V once per sequence; per node its Q, output and
    # own K/V, and its parent
    prefix = 4 * 2 * 4096 * 4 * 128 * 2
    per_node = 2 * 32 * 128 * 2 + 2 * 4 * 128 * 2 + 4
    assert w["attn"][0] == prefix + M * per_node == 109_068_288
    # flops: 4 Hq D per visible key; node i sees the prefix, its ancestors and itself
    assert w["attn"][1] == 4 * 32 * 128 * int((4096 + depth + 1).sum())
    # compaction: K and V rows read and written for each moved row, lengths in and out
    assert w["compact"][0] == 4 * 6 * 4 * 128 * 2 + 8 * 4


def test_lmhead_kernel_label_follows_the_library_choice():
    """The labels the profiles show for each workload's LM head."""
    b = _bench()
    both = "gemm8_argmax_kernel<384, {0}> + gemm8_argmax_kernel<256, {0}> + argmax_reduce_kernel"
    assert b.lmhead_kernel_name(4096, 151936, "bf16") == \
        "gemm8_argmax_kernel<384, false> + argmax_reduce_kernel"
    assert b.lmhead_kernel_name(512, 151936, "bf16") == both.format("false")
    assert b.lmhead_kernel_name(256, 151936, "bf16") == both.format("true")
    assert b.lmhead_kernel_name(256, 4163, "bf16") == "gemm8_argmax_kernel<256, true> + argmax_reduce_kernel"
    assert b.lmhead_kernel_name(64, 151936, "bf16") == "lmhead_stream_kernel (packed W)"
    assert b.lmhead_kernel_name(7, 1000, "f32") == "lmhead_f32_kernel"


def test_lmhead_tile_plan():
    """The split of the vocabulary into 384-row then 256-row W tiles: every
    row covered once, the 384-row run whole when a tail follows, and the
    rounds of 256 workgroups it saves at the workloads' sizes."""
    b = _bench()
    # one H slice: 256 tiles of 384 (one round) + 210 of 256 (one round)
    # instead of 396 tiles of 384 (two rounds)
    assert b.gemm8_plan(256, 151936) == (256, 210)
    assert b.gemm8_plan(4096, 151936) == (396, 0)     # 24.75 rounds: one width
    assert b.gemm8_plan(300, 66000) == (128, 66)
    assert b.gemm8_plan(256, 4163) == (0, 17)
    for M in (256, 300, 512, 1000, 2048, 4096):
        for V in (1000, 4163, 66000, 151936, 152064):
            n384, n256 = b.gemm8_plan(M, V)
            if n256:
                assert 384 * n384 < V <= 384 * n384 + 256 * n256 < V + 256
            else:
                assert V <= 384 * n384 < V + 384
