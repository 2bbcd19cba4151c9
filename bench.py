"""Benchmark: one MI355X's share of exact causal ring attention.

A step is one pass of the hot path over one batch of synthetic input: the
zig-zag placement of Q, K and V into shards (zigzag_partition), then every
shard's queries against its c key/value blocks in ring order
(ring_attn_shard_fwd), the shards run one after another on one GPU.
Inputs are resident in HBM before the timed region starts.

Prints one JSON line: causal-useful TFLOP/s (4 * d * visible pairs per query
head, summed over shards, divided by step time), the roofline entry of the
attention kernel (MFMA bf16 dense peak), and the fp64 oracle timed on a
bounded sample on the host's cores as a CPU baseline.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import workloads  # noqa: E402

METRIC = "causal attention TFLOP/s per shard on 1 MI355X + % of bf16 MFMA peak"
# MI355X bf16 dense matrix peak: 256 CUs x 2.4 GHz x 4096 FLOP/clk/CU.
PEAK_BF16_TFLOPS = 256 * 2.4e9 * 4096 / 1e12
PEAK_F32_TFLOPS = 157.3


def useful_flop(w, pairs_per_head):
    return 4.0 * w.head_dim * w.h_q * w.batch * pairs_per_head


def cpu_baseline(w, target_s):
    """The fp64 oracle on a bounded row sample of shard 0, one query head at a time."""
    import oracle
    q_pos_all = oracle.partition_perm(w.seq_len, w.n_shards, w.split)[:w.n_loc]
    # Rows in a seeded random order so that the sample's spread of early and
    # late tokens is the shard's; heads 0, 1, ... in turn.
    order = np.random.default_rng(0).permutation(w.n_loc)
    k = workloads.draw(w.seed, workloads.TENSOR_K, w.batch, w.h_kv, w.seq_len, w.head_dim, w.sigma, w.dtype)
    v = workloads.draw(w.seed, workloads.TENSOR_V, w.batch, w.h_kv, w.seq_len, w.head_dim, w.sigma, w.dtype)
    group = w.h_q // w.h_kv
    done, flop, elapsed, n, head, lo = 0, 0.0, 0.0, 16, 0, 0
    while elapsed < target_s and head < w.h_q:
        pos = q_pos_all[order[lo:lo + n]]
        qs = workloads.draw(w.seed, workloads.TENSOR_Q, w.batch, w.h_q, w.seq_len, w.head_dim, w.sigma,
                            w.dtype, positions=pos)[:, head:head + 1]
        hk = head // group
        t0 = time.perf_counter()
        oracle.attention(qs, np.ascontiguousarray(k[:, hk:hk + 1]), np.ascontiguousarray(v[:, hk:hk + 1]),
                         w.scale, w.causal, q_pos=pos)
        elapsed += time.perf_counter() - t0
        flop += 4.0 * w.head_dim * w.batch * float((pos + 1).sum() if w.causal else len(pos) * w.seq_len)
        done += len(pos)
        lo += len(pos)
        if lo >= w.n_loc:
            lo, head = 0, head + 1
        if elapsed < target_s / 4:
            n *= 2
    return {"value": flop / elapsed / 1e12, "unit": "TFLOP/s", "cores": oracle.threads(), "kind": "oracle",
            "sample": f"{done} (query row, head) items of shard 0 with all their visible keys "
                      f"({flop / 1e9:.1f} GFLOP useful in {elapsed:.1f} s, fp64, timed around the oracle call)"}


def cpu_baseline_full(w):
    """The fp64 oracle over the whole problem of a small workload: full causal
    attention of every query head over the natural-order sequence (every
    shard's rows at once)."""
    import oracle
    q, k, v = workloads.draw_qkv(w)
    t0 = time.perf_counter()
    oracle.attention(q, k, v, w.scale, w.causal)
    elapsed = time.perf_counter() - t0
    pairs = w.seq_len * (w.seq_len + 1) // 2 if w.causal else w.seq_len * w.seq_len
    flop = useful_flop(w, pairs)
    return {"seconds": elapsed, "value": flop / elapsed / 1e12, "unit": "TFLOP/s", "cores": oracle.threads(),
            "kind": "oracle", "sample": f"whole problem: {w.batch * w.h_q * w.seq_len} (query row, head) items, "
                                        f"{flop / 1e9:.2f} GFLOP useful, fp64"}


def measured_traffic():
    """HBM bytes per attention launch from the committed counter summary, or
    None when the kernel source has changed since the counters were taken."""
    import hashlib
    prof = os.path.join(ROOT, "profiles", "fwd_bf16_s128k_c16_zigzag_hbm_traffic.md")
    src = os.path.join(ROOT, "ring_parallelism_amd", "csrc", "fwd_bf16.hip")
    try:
        fields = dict(line.split(": ", 1) for line in open(prof).read().splitlines() if ": " in line)
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    except OSError:
        return None
    if fields.get("source_sha256", "").strip() != sha:
        return None
    return float(fields["traffic_bytes_per_launch"])


def measured_clock():
    """Shader clock (GHz) the chip held during the attention kernel, from the
    committed counter summary (GRBM_GUI_ACTIVE per XCD / kernel duration), or
    None when the kernel source has changed since the counters were taken."""
    import hashlib
    prof = os.path.join(ROOT, "profiles", "fwd_bf16_s128k_c16_zigzag_mfma_counters.md")
    src = os.path.join(ROOT, "ring_parallelism_amd", "csrc", "fwd_bf16.hip")
    try:
        fields = dict(line.split(": ", 1) for line in open(prof).read().splitlines() if ": " in line)
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    except OSError:
        return None
    if fields.get("source_sha256", "").strip() != sha or "held_clock_ghz" not in fields:
        return None
    return float(fields["held_clock_ghz"])


def host_info():
    """The host the run is on: CPU model and the core count the oracle uses."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"cpu_model": model, "cpu_count": os.cpu_count()}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="s128k_c16_zigzag_16x1", choices=sorted(workloads.WORKLOAD_BY_NAME))
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="oracle CPU-baseline budget (0: skip)")
    ap.add_argument("--suite", action="store_true",
                    help="instead of the headline line, print one JSON line per secondary measurement: "
                         "per-shard balance (32k tokens), all shards in one launch (8k, 32k, 131k tokens), "
                         "warm/cold and overlap on/off "
                         "(131k tokens), partial+merge and bidirectional passes (262k tokens), split-KV "
                         "decode, and every workload's GPU time beside the fp64 oracle's")
    ap.add_argument("--reps", type=int, default=10, help="timed repetitions per launch in --suite (after 3 warm-ups)")
    ap.add_argument("--traffic", action="store_true",
                    help="run the kernels whose memory traffic is measured (under rocprofv3 --pmc): a plain "
                         "conversion copy, the shard gather of Q, a two-part merge and the benchmarked shard pass, "
                         f"{TRAFFIC_DISPATCHES} dispatches each")
    ap.add_argument("--power", action="store_true",
                    help="board power (hwmon) and rate while one kernel runs back to back for a few seconds: "
                         "the benchmarked shard pass on the benchmark's inputs and on zero inputs, and a "
                         "matrix-core stream (libmfma_stream.so) on N(0,1) and on zero operands")
    ap.add_argument("--counters-report", nargs="+", metavar="DIR",
                    help="summarise rocprofv3 counter CSVs under these directories for the --traffic kernels: "
                         "bytes per dispatch from request counts by request size, beside the algorithmic bytes")
    args = ap.parse_args()
    if args.counters_report:
        counters_report(args.counters_report)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share of the ring: run with --gpus 1 (got {args.gpus}); "
              "the multi-GPU ring is not implemented here", file=sys.stderr)
        sys.exit(2)

    import torch
    import ring_parallelism_amd as ra

    if args.suite:
        suite(args)
        return
    if args.traffic:
        traffic_run()
        return
    if args.power:
        power_run()
        return
    w = workloads.WORKLOAD_BY_NAME[args.workload]
    # The CPU baseline runs first, bounded, so that the GPU leg that follows is
    # one uninterrupted stretch of device work.
    host = host_info()
    cpu = cpu_baseline(w, args.cpu_seconds) if args.cpu_seconds > 0 else None
    dev = torch.device("cuda:0")
    in_dt = ra.BF16 if w.dtype == "bf16" else ra.F32
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    def up(a):
        a = np.ascontiguousarray(a)
        return (torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if w.dtype == "bf16"
                else torch.from_numpy(a)).to(dev)

    q, k, v = workloads.draw_qkv(w)
    qn, kn, vn = up(q), up(k), up(v)
    del q, k, v
    c, n_loc = w.n_shards, w.n_loc
    qs = torch.empty((c, w.batch, w.h_q, n_loc, w.head_dim), dtype=tdt, device=dev)
    ks = torch.empty((c, w.batch, w.h_kv, n_loc, w.head_dim), dtype=tdt, device=dev)
    vs = torch.empty_like(ks)
    out = torch.empty((w.batch, w.h_q, n_loc, w.head_dim), dtype=tdt, device=dev)
    lse = torch.empty((w.batch, w.h_q, n_loc), dtype=torch.float32, device=dev)
    stats = torch.zeros(4, dtype=torch.int64, device=dev)
    desc = ra.make_desc(w.seq_len, c, w.split, w.batch, w.h_q, w.h_kv, w.head_dim, in_dt, in_dt, w.causal, w.scale)
    esz = qn.element_size()
    owners = [[(r - t) % c for t in range(c)] for r in range(c)]
    kb = [[ks[j] for j in owners[r]] for r in range(c)]
    vb = [[vs[j] for j in owners[r]] for r in range(c)]
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(c)]

    batch_ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))

    def step(timed_kernels=False, timed_batch=False):
        ra.zigzag_partition(w.seq_len, c, w.split, None, qn, qs, w.batch * w.h_q, w.head_dim * esz)
        ra.zigzag_partition(w.seq_len, c, w.split, None, kn, ks, w.batch * w.h_kv, w.head_dim * esz)
        ra.zigzag_partition(w.seq_len, c, w.split, None, vn, vs, w.batch * w.h_kv, w.head_dim * esz)
        if timed_batch:
            batch_ev[0].record()
        for r in range(c):
            if timed_kernels:
                ev[r][0].record()
            ra.ring_attn_shard_fwd(desc, r, qs[r], kb[r], vb[r], out, lse, stats=stats)
            if timed_kernels:
                ev[r][1].record()
        if timed_batch:
            batch_ev[1].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stats.zero_()

    # Timed region: exactly K steps back to back.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    st = stats.cpu().tolist()

    # Kernel durations with HIP events on the launch stream (separate passes):
    # one event pair around each step's c back-to-back launches gives the
    # average (no event between launches), one pair around each launch the
    # median and minimum.
    kernel_ms, batch_ms = [], []
    for _ in range(max(1, min(args.steps, 3))):
        step(timed_batch=True)
        torch.cuda.synchronize()
        batch_ms.append(batch_ev[0].elapsed_time(batch_ev[1]) / c)
    for _ in range(max(1, min(args.steps, 3))):
        step(timed_kernels=True)
        torch.cuda.synchronize()
        kernel_ms.extend(ev[r][0].elapsed_time(ev[r][1]) for r in range(c))

    pairs = [shard_pairs(w, r) for r in range(c)]               # per query head
    flop_step = sum(useful_flop(w, pr) for pr in pairs)
    pairs_counted = st[0] / args.steps
    if abs(pairs_counted - sum(pairs) * w.h_q * w.batch) > 0.5:
        raise SystemExit(f"kernel pair count {pairs_counted} != {sum(pairs) * w.h_q * w.batch}")
    ms_step = elapsed * 1e3 / args.steps
    value = flop_step / (elapsed / args.steps) / 1e12
    avg_kernel_s = float(np.mean(batch_ms)) / 1e3
    flop_launch = flop_step / c
    achieved = flop_launch / avg_kernel_s / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    res = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "seq_len": w.seq_len, "n_shards": c,
                   "split": {0: "contiguous", 1: "zigzag", 2: "striped"}[w.split], "batch": w.batch,
                   "h_q": w.h_q, "h_kv": w.h_kv, "head_dim": w.head_dim, "causal": w.causal,
                   "shards_per_step": c, "inputs": f"N(0,{w.sigma}^2) seeded, bf16-rounded" if w.dtype == "bf16" else "N(0,1) seeded"},
        "pct_of_peak": round(100.0 * value / peak, 2),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": round(peak, 1),
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": measured_traffic() if w.name == "s128k_c16_zigzag_16x1" else None,
                     "kernel": "fwd_bf16_kernel" if w.dtype == "bf16" else "fwd_f32_kernel",
                     "flop_per_launch": flop_launch, "avg_launch_ms": round(avg_kernel_s * 1e3, 4),
                     "median_launch_ms": round(float(np.median(kernel_ms)), 4),
                     "min_launch_ms": round(float(np.min(kernel_ms)), 4),
                     "launches_timed": len(batch_ms) * c,
                     "per_launch_event_avg_ms": round(float(np.mean(kernel_ms)), 4),
                     "held_shader_clock_ghz": measured_clock() if w.name == "s128k_c16_zigzag_16x1" else None},
        "stats_per_step": {"pairs": int(pairs_counted), "tiles_full": st[1] // args.steps,
                           "tiles_partial": st[2] // args.steps, "tiles_skipped": st[3] // args.steps},
    }
    if cpu is not None:
        res["cpu_baseline"] = cpu
    res["host"] = host
    print(json.dumps(res), flush=True)


# Memory-traffic measurement.  The L2 (TCC) counts the requests it sends to
# the memory side by size (32, 64 or 128 bytes for reads; 32 or 64 for
# writes), so bytes = sum of count x size, with no calibration factor.  The
# kernels of known byte counts run beside the attention launch to check that.
TRAFFIC_WORKLOAD = "s128k_c16_zigzag_16x1"
TRAFFIC_DISPATCHES = 3
TRAFFIC_PASSES = {
    "reads": ["TCC_EA0_RDREQ_sum", "TCC_EA0_RDREQ_32B_sum", "TCC_EA0_RDREQ_64B_sum", "TCC_EA0_RDREQ_128B_sum"],
    "writes": ["TCC_EA0_WRREQ_sum", "TCC_EA0_WRREQ_64B_sum", "TCC_EA0_RDREQ_DRAM_sum", "TCC_EA0_WRREQ_DRAM_sum"],
}


def traffic_known(w):
    """(label, kernel-name substring, algorithmic read bytes, write bytes) per
    dispatch of the kernels traffic_run launches."""
    esz = 2
    q_all = w.batch * w.h_q * w.seq_len * w.head_dim * esz
    kv_all = w.batch * w.h_kv * w.seq_len * w.head_dim * esz
    rows = w.batch * w.h_q * w.n_loc
    part = rows * w.head_dim * 4 + rows * 4          # one fp32 partial: out + lse
    return [
        ("conversion copy of Q, bf16 -> fp32 (torch)", "copy", q_all, 2 * q_all),
        ("shard gather of Q (zigzag_partition)", "move_rows_kernel", q_all, q_all),
        ("merge of two fp32 partials (ring_attn_merge_strided)", "merge_kernel", 2 * part, part),
        ("shard pass, rank 0 (ring_attn_shard_fwd, bf16 out)", "fwd_bf16_kernel",
         rows * w.head_dim * esz + 2 * kv_all, rows * w.head_dim * esz + rows * 4),
    ]


def traffic_run():
    """The --traffic kernels, TRAFFIC_DISPATCHES launches each, on the
    131 072-token workload's shapes (inputs drawn on the device)."""
    import torch
    import ring_parallelism_amd as ra
    w = workloads.WORKLOAD_BY_NAME[TRAFFIC_WORKLOAD]
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(w.seed)
    c, n = w.n_shards, w.n_loc
    rnd = lambda *shape: (torch.randn(shape, generator=g, device=dev) * w.sigma).to(torch.bfloat16)  # noqa: E731
    qn = rnd(w.batch, w.h_q, w.seq_len, w.head_dim)
    q32 = torch.empty(qn.shape, dtype=torch.float32, device=dev)
    qs = torch.empty((c, w.batch, w.h_q, n, w.head_dim), dtype=torch.bfloat16, device=dev)
    parts = torch.randn((2, w.batch, w.h_q, n, w.head_dim), generator=g, device=dev)
    part_lse = torch.randn((2, w.batch, w.h_q, n), generator=g, device=dev)
    m_out = torch.empty(parts.shape[1:], dtype=torch.float32, device=dev)
    m_lse = torch.empty(part_lse.shape[1:], dtype=torch.float32, device=dev)
    ks = rnd(c, w.batch, w.h_kv, n, w.head_dim)
    vs = rnd(c, w.batch, w.h_kv, n, w.head_dim)
    out = torch.empty((w.batch, w.h_q, n, w.head_dim), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.batch, w.h_q, n), dtype=torch.float32, device=dev)
    stats = torch.zeros(4, dtype=torch.int64, device=dev)
    desc = ra.make_desc(w.seq_len, c, w.split, w.batch, w.h_q, w.h_kv, w.head_dim, ra.BF16, ra.BF16, w.causal, w.scale)
    own = [(0 - t) % c for t in range(c)]
    torch.cuda.synchronize()
    for _ in range(TRAFFIC_DISPATCHES):
        q32.copy_(qn)
        ra.zigzag_partition(w.seq_len, c, w.split, None, qn, qs, w.batch * w.h_q, w.head_dim * 2)
        ra.ring_attn_merge_strided(w.batch, w.h_q, n, w.head_dim, parts, ra.F32, part_lse, m_out, ra.F32, m_lse)
        ra.ring_attn_shard_fwd(desc, 0, qs[0], [ks[j] for j in own], [vs[j] for j in own], out, lse, stats=stats)
        torch.cuda.synchronize()
    print(json.dumps({"traffic_run": w.name, "dispatches_each": TRAFFIC_DISPATCHES}), flush=True)


def counters_report(dirs):
    """Per-dispatch means of the TRAFFIC_PASSES counters for the --traffic
    kernels, bytes from request counts x request sizes."""
    import csv
    import glob
    vals = {}
    for d in dirs:
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                vals.setdefault((r["Kernel_Name"], r["Counter_Name"]), []).append(float(r["Counter_Value"]))
    w = workloads.WORKLOAD_BY_NAME[TRAFFIC_WORKLOAD]
    rows = []
    for label, sub, alg_r, alg_w in traffic_known(w):
        m, n_disp = {}, 0
        for (name, counter), v in vals.items():
            if sub in name and "distribution" not in name:
                m[counter] = float(np.mean(v))
                n_disp = max(n_disp, len(v))
        if not m:
            continue
        g = lambda k: m.get(k, float("nan"))  # noqa: E731
        rd = 32 * g("TCC_EA0_RDREQ_32B_sum") + 64 * g("TCC_EA0_RDREQ_64B_sum") + 128 * g("TCC_EA0_RDREQ_128B_sum")
        unsized = g("TCC_EA0_RDREQ_sum") - g("TCC_EA0_RDREQ_32B_sum") - g("TCC_EA0_RDREQ_64B_sum") \
            - g("TCC_EA0_RDREQ_128B_sum")
        wr = 64 * g("TCC_EA0_WRREQ_64B_sum") + 32 * (g("TCC_EA0_WRREQ_sum") - g("TCC_EA0_WRREQ_64B_sum"))
        rows.append({"kernel": label, "dispatches": n_disp, "read_bytes": rd, "write_bytes": wr,
                     "read_requests_without_size": unsized,
                     "read_requests_to_dram_frac": g("TCC_EA0_RDREQ_DRAM_sum") / g("TCC_EA0_RDREQ_sum"),
                     "write_requests_to_dram_frac": g("TCC_EA0_WRREQ_DRAM_sum") / g("TCC_EA0_WRREQ_sum"),
                     "algorithmic_read_bytes": alg_r, "algorithmic_write_bytes": alg_w,
                     "read_over_algorithmic": rd / alg_r, "write_over_algorithmic": wr / alg_w,
                     "requests": {k: m[k] for k in sorted(m)}})
    for r in rows:
        print(json.dumps(r), flush=True)


POWER_SECONDS = 3.0


def hwmon_power_files():
    """(power reading, power cap, junction temperature) sysfs files of the
    GPU's hwmon, or None."""
    import glob
    for d in sorted(glob.glob("/sys/class/drm/card*/device/hwmon/hwmon*")):
        for name in ("power1_input", "power1_average"):
            f = os.path.join(d, name)
            if os.path.exists(f):
                temp = None
                for t in sorted(glob.glob(os.path.join(d, "temp*_label"))):
                    try:
                        if open(t).read().strip() == "junction":
                            temp = t.replace("_label", "_input")
                    except OSError:
                        pass
                return f, os.path.join(d, "power1_cap"), temp
    return None


def power_run():
    """Board power while one kernel runs back to back for POWER_SECONDS (the
    reading is sampled every 50 ms by a host thread; the median of the last
    three quarters is reported), beside the rate the kernel reached."""
    import ctypes
    import threading
    import torch
    import ring_parallelism_amd as ra
    files = hwmon_power_files()

    def read_w(f):
        try:
            return int(open(f).read().strip()) / 1e6
        except (OSError, ValueError):
            return None

    cap = read_w(files[1]) if files else None
    w = workloads.WORKLOAD_BY_NAME["s128k_c16_zigzag_16x1"]
    dev = torch.device("cuda:0")
    c = w.n_shards
    qs, ks, vs = device_inputs(w, torch, dev, blocks_for=[0])
    out = torch.empty((w.batch, w.h_q, w.n_loc, w.head_dim), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.batch, w.h_q, w.n_loc), dtype=torch.float32, device=dev)
    desc = ra.make_desc(w.seq_len, c, w.split, w.batch, w.h_q, w.h_kv, w.head_dim, ra.BF16, ra.BF16, w.causal, w.scale)
    own = [(0 - t) % c for t in range(c)]
    zq, zk, zv = torch.zeros_like(qs[0]), torch.zeros_like(ks), torch.zeros_like(vs)

    def shard(q, k, v):
        return lambda: ra.ring_attn_shard_fwd(desc, 0, q, [k[j] for j in own], [v[j] for j in own], out, lse)

    from ring_parallelism_amd import build as hip_build
    slib = ctypes.CDLL(hip_build.STREAM_LIB)
    slib.mfma_stream.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_uint32, ctypes.c_void_p,
                                 ctypes.c_void_p]
    slib.mfma_stream.restype = ctypes.c_int
    n_wg, iters = 1024, 15000
    sink = torch.empty((n_wg * 512,), dtype=torch.float32, device=dev)

    def stream(zero):
        def run():
            rc = slib.mfma_stream(n_wg, iters, int(zero), 11, sink.data_ptr(),
                                  ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
            if rc != 0:
                raise RuntimeError(f"mfma_stream failed: hip error {rc}")
        return run

    shard_flop = useful_flop(w, shard_pairs(w, 0))
    stream_flop = float(n_wg) * 8 * iters * 16 * 32 * 32 * 16 * 2
    cases = [("fwd_bf16_kernel, shard 0 of the 131 072-token workload", f"N(0,{w.sigma}^2)", shard(qs[0], ks, vs),
              shard_flop),
             ("fwd_bf16_kernel, shard 0 of the 131 072-token workload", "zeros", shard(zq, zk, zv), shard_flop),
             ("mfma_stream (matrix-core products only, operands in registers)", "N(0,1)", stream(False), stream_flop),
             ("mfma_stream (matrix-core products only, operands in registers)", "zeros", stream(True), stream_flop)]
    for kernel, inputs, fn, flop in cases:
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        samples, stop = [], threading.Event()

        temps = []

        def sample():
            while not stop.is_set():
                if files:
                    samples.append(read_w(files[0]))
                    if files[2]:
                        temps.append(read_w(files[2]))
                time.sleep(0.05)

        th = threading.Thread(target=sample)
        th.start()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record()
        calls = 0
        while time.perf_counter() - t0 < POWER_SECONDS:
            for _ in range(8):
                fn()
            calls += 8
            torch.cuda.synchronize()
        e1.record()
        torch.cuda.synchronize()
        stop.set()
        th.join()
        ms = e0.elapsed_time(e1) / calls
        tail = [x for x in samples[len(samples) // 4:] if x is not None]
        tf = flop / (ms / 1e3) / 1e12
        emit({"measurement": "power", "kernel": kernel, "inputs": inputs, "calls": calls,
              "ms_per_call": round(ms, 4), "tflops": round(tf, 1), "pct_of_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2),
              "board_power_w_median": float(np.median(tail)) if tail else None, "board_power_cap_w": cap,
              "power_samples": len(tail), "power_file": files[0] if files else None,
              "junction_temp_c_max": max((x * 1e3 for x in temps if x is not None), default=None)})


def emit(d):
    print(json.dumps(d), flush=True)


def device_inputs(w, torch, dev, blocks_for=None):
    """Seeded synthetic Q shards and K/V blocks drawn on the device: N(0, sigma^2)
    rounded to bf16, in shard layout [c, B, H, S/c, d] (timing inputs; the values
    only matter through their distribution).  blocks_for: only Q of these shards."""
    g = torch.Generator(device=dev).manual_seed(w.seed)
    c, n = w.n_shards, w.n_loc
    ranks = range(c) if blocks_for is None else blocks_for
    qs = {r: (torch.randn((w.batch, w.h_q, n, w.head_dim), generator=g, device=dev) * w.sigma).to(torch.bfloat16)
          for r in ranks}
    ks = (torch.randn((c, w.batch, w.h_kv, n, w.head_dim), generator=g, device=dev) * w.sigma).to(torch.bfloat16)
    vs = (torch.randn((c, w.batch, w.h_kv, n, w.head_dim), generator=g, device=dev) * w.sigma).to(torch.bfloat16)
    return qs, ks, vs


def timed(torch, fn, reps, scrub=None, warmup=3):
    """Per-launch milliseconds of fn() from HIP events on the current stream,
    after `warmup` untimed launches; with `scrub` (a large device tensor) the
    caches are flushed by a full write of it before every launch."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ms = []
    for _ in range(reps):
        if scrub is not None:
            scrub.fill_(1.0)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
    return ms


def stat(ms):
    return {"median_ms": round(float(np.median(ms)), 4), "min_ms": round(float(np.min(ms)), 4), "reps": len(ms)}


def suite(args):
    """Secondary measurements, one JSON line each (inputs resident in HBM)."""
    import torch
    import ring_parallelism_amd as ra
    dev = torch.device("cuda:0")
    reps = max(1, args.reps)

    def fwd(w, desc, r, q, ks, vs, out, lse, owners=None):
        c = w.n_shards
        own = [(r - t) % c for t in range(c)] if owners is None else owners
        return lambda: ra.ring_attn_shard_fwd(desc, r, q, [ks[j] for j in own], [vs[j] for j in own], out, lse,
                                              block_owner=own)

    # Per-shard work and time under the three placements (32 768 tokens, c = 16).
    for name in ("s32k_c16_contig_16x1", "s32k_c16_zigzag_16x1", None):
        if name is None:
            w = workloads.WORKLOAD_BY_NAME["s32k_c16_zigzag_16x1"]
            w = workloads.Workload(**{**w.__dict__, "name": "s32k_c16_striped_16x1", "split": workloads.SPLIT_STRIPED})
        else:
            w = workloads.WORKLOAD_BY_NAME[name]
        qs, ks, vs = device_inputs(w, torch, dev)
        out = torch.empty((w.batch, w.h_q, w.n_loc, w.head_dim), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((w.batch, w.h_q, w.n_loc), dtype=torch.float32, device=dev)
        desc = ra.make_desc(w.seq_len, w.n_shards, w.split, w.batch, w.h_q, w.h_kv, w.head_dim, ra.BF16, ra.BF16,
                            w.causal, w.scale)
        med, flops = [], []
        for r in range(w.n_shards):
            m = stat(timed(torch, fwd(w, desc, r, qs[r], ks, vs, out, lse), reps))["median_ms"]
            med.append(m)
            flops.append(useful_flop(w, shard_pairs(w, r)))
        work = [f / np.mean(flops) for f in flops]
        emit({"measurement": "per_shard_balance", "workload": w.name,
              "split": {0: "contiguous", 1: "zigzag", 2: "striped"}[w.split],
              "shard_median_ms": med, "busiest_over_mean_time": round(max(med) / float(np.mean(med)), 4),
              "busiest_over_mean_work": round(max(work), 4),
              "max_over_min_time": round(max(med) / min(med), 4),
              "total_ms": round(sum(med), 3),
              "tflops_all_shards": round(sum(flops) / (sum(med) / 1e3) / 1e12, 1)})
        del qs, ks, vs

    # 131 072 tokens, shard 0: warm vs cold caches, loads overlapped vs not.
    w = workloads.WORKLOAD_BY_NAME["s128k_c16_zigzag_16x1"]
    qs, ks, vs = device_inputs(w, torch, dev, blocks_for=[0])
    out = torch.empty((w.batch, w.h_q, w.n_loc, w.head_dim), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.batch, w.h_q, w.n_loc), dtype=torch.float32, device=dev)
    f0 = useful_flop(w, shard_pairs(w, 0))
    scrub = torch.empty(512 * 2**20 // 4, dtype=torch.float32, device=dev)
    for mode, flags, sc in (("warm", 0, None), ("cold", 0, scrub), ("warm_no_overlap", ra.FLAG_SYNC_LOADS, None)):
        desc = ra.make_desc(w.seq_len, w.n_shards, w.split, w.batch, w.h_q, w.h_kv, w.head_dim, ra.BF16, ra.BF16,
                            True, w.scale, flags)
        st = stat(timed(torch, fwd(w, desc, 0, qs[0], ks, vs, out, lse), reps, sc))
        emit({"measurement": "shard_pass", "workload": w.name, "mode": mode, **st,
              "tflops": round(f0 / (st["median_ms"] / 1e3) / 1e12, 1)})
    del qs, ks, vs, scrub

    all_shards_suite(torch, ra, dev, reps)
    split_suite(torch, ra, dev, reps)
    natural_step_suite(torch, ra, dev, reps)
    decode_suite(torch, ra, dev, reps)
    if args.cpu_seconds > 0:
        oracle_suite(torch, ra, dev, reps, min(args.cpu_seconds, 4.0))

    # 262 144 tokens, c = 32, 64/8 heads, shard 0: fused pass, per-block partials
    # folded by 31 two-way merges, and the bidirectional (non-causal) pass.
    w = workloads.WORKLOAD_BY_NAME["s256k_c32_zigzag_64x8"]
    qs, ks, vs = device_inputs(w, torch, dev, blocks_for=[0])
    c, n = w.n_shards, w.n_loc
    out = torch.empty((w.batch, w.h_q, n, w.head_dim), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.batch, w.h_q, n), dtype=torch.float32, device=dev)
    for causal in (True, False):
        desc = ra.make_desc(w.seq_len, c, w.split, w.batch, w.h_q, w.h_kv, w.head_dim, ra.BF16, ra.BF16, causal,
                            w.scale)
        st = stat(timed(torch, fwd(w, desc, 0, qs[0], ks, vs, out, lse), reps))
        fl = useful_flop(w, shard_pairs(w, 0)) if causal else 4.0 * w.head_dim * w.h_q * w.batch * n * w.seq_len
        emit({"measurement": "shard_pass", "workload": w.name, "mode": "fused_causal" if causal else "fused_bidirectional",
              **st, "tflops": round(fl / (st["median_ms"] / 1e3) / 1e12, 1)})
    acc = torch.empty((w.batch, w.h_q, n, w.head_dim), dtype=torch.float32, device=dev)
    acc_l = torch.empty((w.batch, w.h_q, n), dtype=torch.float32, device=dev)
    part = torch.empty_like(acc)
    part_l = torch.empty_like(acc_l)
    pdesc = ra.make_desc(w.seq_len, c, w.split, w.batch, w.h_q, w.h_kv, w.head_dim, ra.BF16, ra.F32, True, w.scale)
    merge_ms = []

    def partial_merge(record):
        for t in range(c):
            j = (0 - t) % c
            dst, dst_l = (acc, acc_l) if t == 0 else (part, part_l)
            ra.ring_attn_shard_fwd(pdesc, 0, qs[0], [ks[j]], [vs[j]], dst, dst_l, block_owner=[j])
            if t > 0:
                if record:
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record()
                ra.ring_attn_merge(w.batch, w.h_q, n, w.head_dim, [acc, part], ra.F32, [acc_l, part_l], acc, ra.F32,
                                   acc_l)
                if record:
                    e1.record()
                    merge_ms.append((e0, e1))

    st = stat(timed(torch, lambda: partial_merge(False), reps))
    partial_merge(True)
    torch.cuda.synchronize()
    mm = [a.elapsed_time(b) for a, b in merge_ms]
    merge_bytes = 3 * (acc.numel() * 4 + acc_l.numel() * 4)
    emit({"measurement": "partials_plus_merges", "workload": w.name, "partial_calls": c, "merges": c - 1, **st,
          "tflops": round(useful_flop(w, shard_pairs(w, 0)) / (st["median_ms"] / 1e3) / 1e12, 1),
          "merge_median_ms": round(float(np.median(mm)), 4), "merge_bytes": merge_bytes,
          "merge_roofline": {"bound": "hbm", "achieved": round(merge_bytes / (np.median(mm) / 1e3) / 1e9, 1),
                             "peak": 8000.0, "unit": "GB/s",
                             "frac": round(merge_bytes / (np.median(mm) / 1e3) / 1e9 / 8000.0, 4)}})


def all_shards_suite(torch, ra, dev, reps):
    """Every shard's ring pass in one launch (ring_attn_all_shards_fwd): the
    8 192-token workload (all 8 shards), the 32 768-token one under each
    placement (all 16 shards) and the 131 072-token one.  A shard of the small
    workloads alone has too few query tiles to fill the device; together they
    do.  Per-shard figures are the launch time divided by c (zig-zag shards
    carry equal work)."""
    names = ["s8k_c8_zigzag_gqa32x8", "s32k_c16_contig_16x1", "s32k_c16_zigzag_16x1", None, "s128k_c16_zigzag_16x1"]
    for name in names:
        if name is None:
            w = workloads.WORKLOAD_BY_NAME["s32k_c16_zigzag_16x1"]
            w = workloads.Workload(**{**w.__dict__, "name": "s32k_c16_striped_16x1", "split": workloads.SPLIT_STRIPED})
        else:
            w = workloads.WORKLOAD_BY_NAME[name]
        c, n = w.n_shards, w.n_loc
        g = torch.Generator(device=dev).manual_seed(w.seed)
        rnd = lambda *shape: (torch.randn(shape, generator=g, device=dev) * w.sigma).to(torch.bfloat16)  # noqa: E731
        qs = rnd(c, w.batch, w.h_q, n, w.head_dim)
        ks, vs = rnd(c, w.batch, w.h_kv, n, w.head_dim), rnd(c, w.batch, w.h_kv, n, w.head_dim)
        out = torch.empty_like(qs)
        lse = torch.empty((c, w.batch, w.h_q, n), dtype=torch.float32, device=dev)
        desc = ra.make_desc(w.seq_len, c, w.split, w.batch, w.h_q, w.h_kv, w.head_dim, ra.BF16, ra.BF16, w.causal,
                            w.scale)
        st = stat(timed(torch, lambda: ra.ring_attn_all_shards_fwd(desc, qs, list(ks), list(vs), out, lse), reps))
        flop = sum(useful_flop(w, shard_pairs(w, r)) for r in range(c))
        tf = flop / (st["median_ms"] / 1e3) / 1e12
        emit({"measurement": "all_shards_one_launch", "workload": w.name,
              "split": {0: "contiguous", 1: "zigzag", 2: "striped"}[w.split], "shards": c, **st,
              "per_shard_ms": round(st["median_ms"] / c, 4), "useful_flop": flop, "tflops": round(tf, 1),
              "pct_of_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2)})
        del qs, ks, vs, out, lse


def split_suite(torch, ra, dev, reps):
    """Small shards (8 192 tokens / c = 8 with 32/8 heads; 32 768 / c = 16 with
    16/1 heads) leave most compute units idle in one pass (64 workgroups);
    ring_attn_shard_fwd_split runs groups of blocks concurrently and merges."""
    for name in ("s8k_c8_zigzag_gqa32x8", "s32k_c16_zigzag_16x1"):
        w = workloads.WORKLOAD_BY_NAME[name]
        qs, ks, vs = device_inputs(w, torch, dev, blocks_for=[0])
        c, n = w.n_shards, w.n_loc
        out = torch.empty((w.batch, w.h_q, n, w.head_dim), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((w.batch, w.h_q, n), dtype=torch.float32, device=dev)
        desc = ra.make_desc(w.seq_len, c, w.split, w.batch, w.h_q, w.h_kv, w.head_dim, ra.BF16, ra.BF16, True,
                            w.scale)
        own = [(0 - t) % c for t in range(c)]
        kb, vb = [ks[j] for j in own], [vs[j] for j in own]
        fl = useful_flop(w, shard_pairs(w, 0))
        res = {}
        for ns in (1, 2, 4, 8):
            if ns > c:
                continue
            if ns == 1:
                fn = lambda: ra.ring_attn_shard_fwd(desc, 0, qs[0], kb, vb, out, lse, block_owner=own)  # noqa: E731
            else:
                work = torch.empty((ns, w.batch, w.h_q, n, w.head_dim), dtype=torch.float32, device=dev)
                work_l = torch.empty((ns, w.batch, w.h_q, n), dtype=torch.float32, device=dev)
                fn = lambda: ra.ring_attn_shard_fwd_split(desc, 0, qs[0], kb, vb, ns, work, work_l, out,  # noqa: E731
                                                          lse, block_owner=own)
            st = stat(timed(torch, fn, reps))
            res[str(ns)] = {**st, "tflops": round(fl / (st["median_ms"] / 1e3) / 1e12, 1)}
        emit({"measurement": "small_shard_split", "workload": w.name, "rank": 0, "by_n_splits": res})
        del qs, ks, vs


def natural_step_suite(torch, ra, dev, reps):
    """A whole 131 072-token step in two forms: (a) Q, K, V gathered into shard
    tensors, then the 16 shard passes; (b) only K, V gathered, each pass reading
    Q and writing out / lse at global positions (RA_FLAG_NATURAL_QO), so the
    result lands in natural order with no shard copy of Q or out."""
    w = workloads.WORKLOAD_BY_NAME["s128k_c16_zigzag_16x1"]
    c, n = w.n_shards, w.n_loc
    g = torch.Generator(device=dev).manual_seed(w.seed)
    mk = lambda h: (torch.randn((w.batch, h, w.seq_len, w.head_dim), generator=g, device=dev)  # noqa: E731
                    * w.sigma).to(torch.bfloat16)
    qn, kn, vn = mk(w.h_q), mk(w.h_kv), mk(w.h_kv)
    esz = 2
    qs = torch.empty((c, w.batch, w.h_q, n, w.head_dim), dtype=torch.bfloat16, device=dev)
    ks = torch.empty((c, w.batch, w.h_kv, n, w.head_dim), dtype=torch.bfloat16, device=dev)
    vs = torch.empty_like(ks)
    out_s = torch.empty((w.batch, w.h_q, n, w.head_dim), dtype=torch.bfloat16, device=dev)
    lse_s = torch.empty((w.batch, w.h_q, n), dtype=torch.float32, device=dev)
    out_n = torch.empty((w.batch, w.h_q, w.seq_len, w.head_dim), dtype=torch.bfloat16, device=dev)
    lse_n = torch.empty((w.batch, w.h_q, w.seq_len), dtype=torch.float32, device=dev)
    d_s = ra.make_desc(w.seq_len, c, w.split, w.batch, w.h_q, w.h_kv, w.head_dim, ra.BF16, ra.BF16, True, w.scale)
    d_n = ra.make_desc(w.seq_len, c, w.split, w.batch, w.h_q, w.h_kv, w.head_dim, ra.BF16, ra.BF16, True, w.scale,
                       ra.FLAG_NATURAL_QO)
    own = [[(r - t) % c for t in range(c)] for r in range(c)]

    def kv():
        ra.zigzag_partition(w.seq_len, c, w.split, None, kn, ks, w.batch * w.h_kv, w.head_dim * esz)
        ra.zigzag_partition(w.seq_len, c, w.split, None, vn, vs, w.batch * w.h_kv, w.head_dim * esz)

    def step_shard():
        ra.zigzag_partition(w.seq_len, c, w.split, None, qn, qs, w.batch * w.h_q, w.head_dim * esz)
        kv()
        for r in range(c):
            ra.ring_attn_shard_fwd(d_s, r, qs[r], [ks[j] for j in own[r]], [vs[j] for j in own[r]], out_s, lse_s)

    def step_natural():
        kv()
        for r in range(c):
            ra.ring_attn_shard_fwd(d_n, r, qn, [ks[j] for j in own[r]], [vs[j] for j in own[r]], out_n, lse_n)

    flop = sum(useful_flop(w, shard_pairs(w, r)) for r in range(c))
    for mode, fn in (("gathered_qkv", step_shard), ("natural_q_out", step_natural)):
        st = stat(timed(torch, fn, max(1, reps // 2)))
        emit({"measurement": "whole_step", "workload": w.name, "mode": mode, **st,
              "tflops": round(flop / (st["median_ms"] / 1e3) / 1e12, 1)})


def decode_suite(torch, ra, dev, reps):
    """Split-KV decode of the 262 144-token cache (c = 32 blocks, 64/8 heads):
    one query token per head, each block's keys in n_splits ranges, partials
    folded by one strided merge.  HBM-bound: K and V are read once."""
    w = workloads.WORKLOAD_BY_NAME["s256k_c32_zigzag_64x8"]
    _, ks, vs = device_inputs(w, torch, dev, blocks_for=[])
    g = torch.Generator(device=dev).manual_seed(w.seed + 1)
    q = (torch.randn((w.batch, w.h_q, w.head_dim), generator=g, device=dev) * w.sigma).to(torch.bfloat16)
    desc = ra.make_desc(w.seq_len, w.n_shards, w.split, w.batch, w.h_q, w.h_kv, w.head_dim, ra.BF16, ra.F32, True,
                        w.scale)
    kv_bytes = 2 * ks.numel() * ks.element_size()
    for n_splits in (4, 8, 16):
        n_parts = w.n_shards * n_splits
        outs = torch.empty((n_parts, w.batch, w.h_q, w.head_dim), dtype=torch.float32, device=dev)
        lses = torch.empty((n_parts, w.batch, w.h_q), dtype=torch.float32, device=dev)
        out = torch.empty((w.batch, w.h_q, w.head_dim), dtype=torch.float32, device=dev)
        lse = torch.empty((w.batch, w.h_q), dtype=torch.float32, device=dev)
        blocks_k, blocks_v = list(ks), list(vs)
        dec = lambda: ra.ring_attn_decode(desc, q, blocks_k, blocks_v, n_splits, outs, lses)  # noqa: E731
        mrg = lambda: ra.ring_attn_merge_strided(w.batch, w.h_q, 1, w.head_dim, outs, ra.F32, lses, out,  # noqa: E731
                                                 ra.F32, lse)
        sd = stat(timed(torch, dec, reps))
        sm = stat(timed(torch, mrg, reps))
        st = stat(timed(torch, lambda: (dec(), mrg()), reps))
        byts = kv_bytes + q.numel() * 2 + outs.numel() * 4 + lses.numel() * 4
        gbs = byts / (sd["median_ms"] / 1e3) / 1e9
        emit({"measurement": "split_kv_decode", "workload": "decode of " + w.name, "n_splits": n_splits,
              "partials": n_parts, "decode": sd, "merge": sm, "decode_plus_merge": st,
              "decode_roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": 8000.0, "unit": "GB/s",
                                  "frac": round(gbs / 8000.0, 4), "bytes": byts}})


def oracle_suite(torch, ra, dev, reps, sample_s):
    """GPU time beside the fp64 oracle's time for every workload (a CPU
    baseline only).  Workloads of at most 8 192 tokens: the whole problem, i.e.
    every shard's ring pass on the GPU against full attention over the sequence
    in the oracle.  Larger ones: shard 0's pass on the GPU; the oracle timed on
    a bounded row sample (cpu_baseline) and scaled to the shard's useful FLOP
    (marked extrapolated)."""
    for w in workloads.WORKLOADS:
        c, n = w.n_shards, w.n_loc
        whole = w.seq_len <= 8192
        ranks = list(range(c)) if whole else [0]
        dt, in_dt = (torch.bfloat16, ra.BF16) if w.dtype == "bf16" else (torch.float32, ra.F32)
        g = torch.Generator(device=dev).manual_seed(w.seed)
        rnd = lambda *shape: (torch.randn(shape, generator=g, device=dev) * w.sigma).to(dt)  # noqa: E731
        qs = {r: rnd(w.batch, w.h_q, n, w.head_dim) for r in ranks}
        ks, vs = rnd(c, w.batch, w.h_kv, n, w.head_dim), rnd(c, w.batch, w.h_kv, n, w.head_dim)
        out = torch.empty((w.batch, w.h_q, n, w.head_dim), dtype=dt, device=dev)
        lse = torch.empty((w.batch, w.h_q, n), dtype=torch.float32, device=dev)
        desc = ra.make_desc(w.seq_len, c, w.split, w.batch, w.h_q, w.h_kv, w.head_dim, in_dt, in_dt, w.causal,
                            w.scale)
        own = {r: [(r - t) % c for t in range(c)] for r in ranks}

        def run():
            for r in ranks:
                ra.ring_attn_shard_fwd(desc, r, qs[r], [ks[j] for j in own[r]], [vs[j] for j in own[r]], out, lse)

        st = stat(timed(torch, run, reps))
        flop = sum(useful_flop(w, shard_pairs(w, r)) for r in ranks)
        del qs, ks, vs, out, lse
        if whole:
            cb = cpu_baseline_full(w)
            oracle_s = cb.pop("seconds")
        else:
            cb = cpu_baseline(w, sample_s)
            oracle_s = flop / (cb["value"] * 1e12)
        gpu_s = st["median_ms"] / 1e3
        emit({"measurement": "gpu_vs_oracle", "workload": w.name,
              "scope": f"all {c} shards" if whole else "shard 0", "useful_flop": flop,
              "gpu": {**st, "tflops": round(flop / gpu_s / 1e12, 3)},
              "oracle": {"seconds": round(oracle_s, 3), "extrapolated": not whole, **cb},
              "gpu_speedup_over_oracle": round(oracle_s / gpu_s, 1)})


def shard_pairs(w, r):
    """Visible (query, key) pairs of shard r for one query head: each token at
    global position p sees p + 1 keys under the causal mask, S without it."""
    n_loc = w.n_loc
    t = np.arange(n_loc, dtype=np.int64)
    if w.split == workloads.SPLIT_ZIGZAG:
        n = n_loc // 2
        pos = np.where(t < n, r * n + t, (2 * w.n_shards - 1 - r) * n + (t - n))
    elif w.split == workloads.SPLIT_STRIPED:
        pos = t * w.n_shards + r
    else:
        pos = r * n_loc + t
    return int((pos + 1).sum()) if w.causal else n_loc * w.seq_len


if __name__ == "__main__":
    main()
