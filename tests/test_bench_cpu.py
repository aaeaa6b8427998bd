"""Host-side checks of the benchmark's accounting (no GPU): the algorithmic
bytes and FLOPs it divides by, written out by hand for the workloads' shapes,
the fraction guard, and the one-GPU contract of its command line."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

import bench  # noqa: E402
from workloads import CONFIGS  # noqa: E402


def test_decode_128k_bytes_by_hand():
    wl = CONFIGS["c2"]
    assert (wl.B, wl.N, wl.HI, wl.dI, wl.H, wl.d, wl.k, wl.W, wl.m) == (32, 32768, 64, 128, 64, 512, 1024, 128, 4)
    keys = 32768 * 128 * 2                      # every visible index key, bf16
    iq = 64 * 128 * 2 + 64 * 4                  # index query (bf16) and head weights (f32)
    q, out = 64 * 512 * 2, 64 * 512 * 4         # query heads (bf16), fp32 output
    sel = 2 * 1024 * 4                          # the selection written and read back
    rows = (1024 + 128) * 512 * 2               # selected entries and window rows
    new_group = 4 * 4 + 512 * 2                 # its logits read, its entry written
    ab = bench.algorithmic_bytes(wl)
    assert ab["indexer"] == 32 * (keys + iq) == 268_967_936
    assert ab["step"] == 32 * (keys + iq + q + out + sel + rows + new_group)
    # one attention call alone: q, fp32 output and lse, the selection read, the rows
    assert bench.attention_bytes(wl) == 32 * (q + out + 64 * 4 + 1024 * 4 + rows)


def test_hca_1m_bytes_by_hand():
    wl = CONFIGS["c3"]
    assert (wl.B, wl.N, wl.m, wl.mode) == (16, 8192, 128, "hca")
    rows = (8192 + 128) * 512 * 2
    ab = bench.algorithmic_bytes(wl)
    assert ab["indexer"] == 0
    assert ab["step"] == 16 * (64 * 512 * 2 + 64 * 512 * 4 + rows + 128 * 4 + 512 * 2)
    assert bench.attention_bytes(wl) == 16 * (64 * 512 * 2 + 64 * 512 * 4 + 64 * 4 + rows)


def test_prefill_chunk_counts_each_key_once():
    """4096 queries share one key cache: its bytes count once, not once per query."""
    wl = CONFIGS["c4"]
    assert (wl.Tq, wl.N, wl.q_pos0 + wl.Tq) == (4096, 16384, 65536)
    ab = bench.algorithmic_bytes(wl)
    assert ab["indexer"] == 16384 * 128 * 2 + 4096 * (64 * 128 * 2 + 64 * 4)
    # the whole step stays within a few index-key caches plus the per-query traffic
    per_query = 64 * 512 * 2 + 64 * 512 * 4 + 2 * 1024 * 4
    assert ab["step"] <= ab["indexer"] + 4096 * per_query + (16384 + 4096 + 127) * 1024 + 1024 * (16 + 1024)


def test_prefill_chunk_flops_closed_form():
    """Indexer 2 n_vis H_I d_I and attention 4 (min(k, n_vis) + window) H d FLOPs per query. For
    the chunk's positions t0 .. t1 - 1 (multiples of 4, every n_vis >= k) the sum of
    n_vis(t) = (t + 1) // 4 has a closed form: s = t + 1 runs over 4 v + 1 .. 4 v + 4 for
    v = t0/4 .. t1/4 - 1, giving v, v, v, v + 1, i.e. 4 v + 1 per v."""
    wl = CONFIGS["c4"]
    t0, t1 = wl.q_pos0, wl.q_pos0 + wl.Tq
    assert t0 % 4 == 0 and t1 % 4 == 0 and t0 // 4 >= wl.k and t1 // 4 <= wl.N and wl.W <= t0
    v0, v1 = t0 // 4, t1 // 4
    sum_nv = 4 * (v1 * (v1 - 1) // 2 - v0 * (v0 - 1) // 2) + (v1 - v0)
    fl = bench.algorithmic_flops(wl)
    assert fl["indexer"] == 2 * sum_nv * 64 * 128
    assert fl["attention"] == 4 * wl.Tq * (wl.k + wl.W) * 64 * 512
    assert abs(fl["indexer"] - 1.065e12) / 1.065e12 < 2e-3
    assert abs(fl["attention"] - 0.618e12) / 0.618e12 < 2e-3


def test_fractions_above_one_are_refused():
    assert bench.checked_frac(0.73, "x") == 0.73
    with pytest.raises(Exception):
        bench.checked_frac(1.2, "x")


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stderr + r.stdout) or "--gpus 1" in (r.stderr + r.stdout)
    assert not any(line.startswith("{") for line in r.stdout.splitlines())
