"""Host-side logic of bench.py (no GPU): the one-GPU guard, the useful-FLOP
accounting against the oracle's pair counts, and the source-hash gate on the
committed HBM-traffic figure."""
import os
import shutil
import subprocess
import sys

import numpy as np

import bench
import oracle
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_shard_pairs_match_the_oracle_for_every_workload():
    """bench.py's own placement arithmetic agrees with the oracle's partition
    and pair counts on every workload and every shard."""
    for w in workloads.WORKLOADS:
        perm = oracle.partition_perm(w.seq_len, w.n_shards, w.split)
        for r in range(w.n_shards):
            pos = perm[r * w.n_loc:(r + 1) * w.n_loc]
            want = int((pos + 1).sum()) if w.causal else w.n_loc * w.seq_len
            assert bench.shard_pairs(w, r) == want, (w.name, r)


def test_useful_flop_of_the_headline_shard():
    """4 d H_q B pairs: 4.398e12 FLOP for one shard of the 131 072-token workload
    (the pages' per-device attention work for that layer shape)."""
    w = workloads.WORKLOAD_BY_NAME["s128k_c16_zigzag_16x1"]
    pairs = bench.shard_pairs(w, 0)
    n = w.seq_len // (2 * w.n_shards)
    assert pairs == n * n * (2 * w.n_shards - 1) + n * (n + 1)
    assert bench.useful_flop(w, pairs) == 4.0 * 128 * 16 * pairs
    assert abs(bench.useful_flop(w, pairs) - 4.398e12) / 4.398e12 < 1e-3
    assert len({bench.shard_pairs(w, r) for r in range(w.n_shards)}) == 1  # zig-zag: equal work


def test_traffic_figure_is_gated_on_the_kernel_source(tmp_path, monkeypatch):
    """A counter figure is reported only while the kernel source it was
    measured on is unchanged (the gate, on a stand-in profile)."""
    import hashlib
    fake = tmp_path / "root"
    (fake / "profiles").mkdir(parents=True)
    (fake / "ring_parallelism_amd" / "csrc").mkdir(parents=True)
    src = fake / "ring_parallelism_amd" / "csrc" / "fwd_bf16.hip"
    shutil.copy(os.path.join(ROOT, "ring_parallelism_amd", "csrc", "fwd_bf16.hip"), src)
    sha = hashlib.sha256(src.read_bytes()).hexdigest()
    (fake / "profiles" / "fwd_bf16_s128k_c16_zigzag_hbm_traffic.md").write_text(
        f"# stand-in\n\nsource_sha256: {sha}\ntraffic_bytes_per_launch: 123456789\n")
    monkeypatch.setattr(bench, "ROOT", str(fake))
    assert bench.measured_traffic() == 123456789.0
    src.write_text(src.read_text() + "\n// edited\n")
    assert bench.measured_traffic() is None


def test_counters_report_prices_requests_by_size(tmp_path, capsys):
    """--counters-report: bytes = 32/64/128 x the read requests of each size and
    64 / 32 x the 64-byte / other write requests, per dispatch, beside the
    algorithmic bytes of the --traffic kernels."""
    import csv
    import json
    w = workloads.WORKLOAD_BY_NAME[bench.TRAFFIC_WORKLOAD]
    known = {sub: (r, wr) for _, sub, r, wr in bench.traffic_known(w)}
    counts = {"TCC_EA0_RDREQ_sum": 110.0, "TCC_EA0_RDREQ_32B_sum": 10.0, "TCC_EA0_RDREQ_64B_sum": 20.0,
              "TCC_EA0_RDREQ_128B_sum": 80.0, "TCC_EA0_WRREQ_sum": 50.0, "TCC_EA0_WRREQ_64B_sum": 40.0,
              "TCC_EA0_RDREQ_DRAM_sum": 110.0, "TCC_EA0_WRREQ_DRAM_sum": 50.0}
    f = tmp_path / "run" / "x_counter_collection.csv"
    f.parent.mkdir()
    with open(f, "w", newline="") as fh:
        wr = csv.writer(fh)
        wr.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for disp in range(2):  # two dispatches of the shard pass; the second doubles every count
            for k, v in counts.items():
                wr.writerow([disp, "void ra::fwd_bf16_kernel<128>(FwdParams)", k, v * (1 + disp)])
    bench.counters_report([str(tmp_path)])
    rows = [json.loads(line) for line in capsys.readouterr().out.splitlines()]
    assert len(rows) == 1 and rows[0]["dispatches"] == 2
    r = rows[0]
    assert r["read_bytes"] == 1.5 * (10 * 32 + 20 * 64 + 80 * 128)
    assert r["write_bytes"] == 1.5 * (40 * 64 + 10 * 32)
    assert r["read_requests_without_size"] == 0
    assert (r["algorithmic_read_bytes"], r["algorithmic_write_bytes"]) == known["fwd_bf16_kernel"]
    # Algorithmic bytes of the shard pass: Q of the shard plus K and V of every block, out (bf16) + lse.
    assert known["fwd_bf16_kernel"] == (33554432 + 2 * 33554432, 33554432 + 524288)


def test_matrix_core_stream_is_outside_the_attention_library():
    """The measurement aid behind bench.py --power lives in its own library:
    the attention library exports no such symbol."""
    import ctypes
    from ring_parallelism_amd import build as hip_build
    import ring_parallelism_amd as ra
    if not os.path.exists(hip_build.STREAM_LIB):
        hip_build.build_stream()
    assert hasattr(ctypes.CDLL(hip_build.STREAM_LIB), "mfma_stream")
    assert not hasattr(ra.lib(), "mfma_stream")
