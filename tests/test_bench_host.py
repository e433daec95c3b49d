"""Host logic of bench.py (CPU only): the one-GPU exit, the counters that
stay attached to unchanged kernel sources, and the rows of --next-table."""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

import bench
import split_dense_gemm_amd as sdg
from split_dense_gemm_amd import inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_default_timed_steps():
    old = sys.argv
    try:
        sys.argv = ["bench.py"]
        args = bench.parse()
    finally:
        sys.argv = old
    assert args.steps == 4000 and args.gpus == 1 and args.check == "full"


def test_source_digest_ignores_comments_and_spacing(tmp_path):
    a, b, c = tmp_path / "a.hip", tmp_path / "b.hip", tmp_path / "c.hip"
    a.write_text("int f(int x) {\n  return x + 1;  // one more\n}\n")
    b.write_text("/* the\n   same */ int f(int x)\n{ return x + 1; }\n")
    c.write_text("int f(int x) { return x + 2; }\n")
    assert bench.source_digest(str(a)) == bench.source_digest(str(b))
    assert bench.source_digest(str(a)) != bench.source_digest(str(c))


@pytest.mark.parametrize("workload", ["bf16_m256_n1024_k2048_s2", "bf16_m2048_n4096_k4096_s8"])
def test_counters_attach_only_to_the_profiled_sources(workload, monkeypatch):
    rec = bench.measured_counters(workload)
    # The committed counters were taken from the committed kernel sources.
    assert set(rec) == {"gemm_bt", "slab_reduce", "source"}
    for key in ("gemm_bt", "slab_reduce"):
        assert rec[key]["traffic_bytes"] > 0 and rec[key]["rocprof_avg_us"] > 0
    # Any change to a kernel source (comments aside) detaches them.
    real = bench.source_digest
    monkeypatch.setattr(bench, "source_digest",
                        lambda path: "0" * 64 if path.endswith("gemm_bt.hip") else real(path))
    rec = bench.measured_counters(workload)
    assert "gemm_bt" not in rec and "slab_reduce" in rec


def test_counter_rates():
    entry = {"traffic_bytes": 8_000_000, "mfma_util_pct": 3.0, "rocprof_avg_us": 5.0}
    out = bench.counter_rates(entry, 2e-6, "src")
    assert out["hbm_gbs"] == 4000.0 and out["hbm_frac"] == 0.5 and out["mfma_util_pct"] == 3.0
    assert bench.counter_rates({}, 1e-6, "src") is None


def test_next_table_rows():
    rows = bench.next_rows()
    ids = [r[0] for r in rows]
    assert len(ids) == len(set(ids))
    kinds = {}
    for rid, kind, w, out in rows:
        kinds.setdefault(kind, []).append((w.name, out))
        assert rid.split(":")[0] == kind and rid.split(":")[1] == w.name
        code = inputs.DTYPE_CODES[w.dtype]
        # Every row names a problem the library accepts, in its layout.
        if kind in ("kn", "ntail_kn"):
            assert sdg.describe_bn(w.M, w.N, w.K, w.kps, w.splits, code)
        elif kind == "auto":
            kps, s, _ = sdg.choose_splits(w.M, w.N, w.K, code)
            assert (s - 1) * kps < w.K <= s * kps
        else:
            assert sdg.describe(w.M, w.N, w.K, w.kps, w.splits, code)
    configs = [w.name for w in inputs.CONFIGS]
    assert sorted(kinds["typed"]) == sorted((n, o) for n in configs for o in ("f16", "bf16"))
    assert [n for n, _ in kinds["kn"]] == configs and [n for n, _ in kinds["auto"]] == configs
    tails = [w.name for w in inputs.NTAIL_SHAPES]
    assert [n for n, _ in kinds["ntail"]] == tails and [n for n, _ in kinds["ntail_kn"]] == tails
    # The tail shapes really have a narrowed last column tile.
    for w in inputs.NTAIL_SHAPES:
        assert w.N % 64 != 0 and w.N % 8 == 0
