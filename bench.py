"""Benchmark of the SparsePR attention call on one MI355X.

A step is one whole attention call (partition, route, block-sparse attention + probe
rows, probe fit, correction) over all heads of the Wan2.1-1.3B-shaped 720p workload
(12 heads, N = 75,600 = 21 x 45 x 80 tokens, d = 128, bf16) at routed density 0.26
(k = 67 of 256 key groups), inputs resident in HBM. Prints one JSON line on stdout;
progress goes to stderr.

The timed calls run in a context without stage timing (no events between stages). A second
context with stage timing then repeats the same calls: its HIP events, recorded by the
library on the stream each stage runs on, give the per-stage times and the sparse-attention
kernel's executed-pair TFLOPS against the bf16 MFMA peak (the roofline figure). Also
reported: this library's dense attention at the same shape, the oracle on the host cores for
a bounded sample (one head; optionally every head in parallel processes), and bit-exact /
tolerance parity of that head.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "ms per sparse attention call + executed-pair TFLOPS (% bf16 MFMA peak) @75.6k tok"
BF16_PEAK_TFLOPS = 2516.6
HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "vbsa_c3_traffic.json")
# sources that define the sparse attention stage: its kernel, its work units and their
# launches (the traffic counters are tied to them)
KERNEL_SRCS = [os.path.join(ROOT, "free_block_sparse_eigen_amd", "csrc", f)
               for f in ("kernels_attn.hip", "attn_tile.h", "common.h", "kernels.h",
                         "kernels_route.hip", "api.cpp")]


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


TRAFFIC_WORKLOAD = "C3 rho=0.26"        # the workload the committed traffic counters ran on


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def copy_calibration(mib: int) -> int:
    """A plain device-to-device copy of known size, the reference reading for the HBM
    traffic counters (run under the same counter pass as the kernel)."""
    import torch
    x = torch.ones(mib * 2**20 // 4, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    y = x.clone()
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": x.numel() * 4, "copy_bytes_written": y.numel() * 4}))
    return 0


def measured_traffic(flops_per_launch: float, ms: float, workload: str):
    """HBM bytes of the sparse attention stage (its two kernel launches) from the committed
    counter summary, valid only for the workload it was measured on and while the sources
    of the stage are unchanged."""
    if workload != TRAFFIC_WORKLOAD:
        return None
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_stage")


def _oracle_head(args):
    """One head of the oracle call in a worker process with single-threaded BLAS; returns
    the wall seconds."""
    cfg_name, density, head = args
    from threadpoolctl import threadpool_limits
    import oracle as orc
    from synthetic import get_config, make_inputs
    cfg = get_config(cfg_name)
    if density is not None:
        cfg = cfg.with_settings(density=density)
    q, k, v = make_inputs(cfg, heads=[head])
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        orc.oracle_call(q, k, v, cfg.settings)
        return time.perf_counter() - t0


def oracle_all_heads(cfg_name, density, heads, workers):
    """The whole oracle call: every head in its own single-threaded worker process, `workers`
    at a time. Returns (wall seconds, sum of per-head seconds)."""
    import multiprocessing as mp
    ctx = mp.get_context("spawn")
    t0 = time.perf_counter()
    with ctx.Pool(workers) as pool:
        per_head = pool.map(_oracle_head, [(cfg_name, density, h) for h in range(heads)])
    return time.perf_counter() - t0, float(sum(per_head))


def oracle_baseline(cfg, q, k, v, gpu_head0, threads_limit=None):
    """Time the fp64 oracle on head 0 (a bounded sample of the call) on the host cores,
    and check parity of the GPU's head 0 against it."""
    import contextlib
    import oracle as orc
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        limit = threadpool_limits(limits=threads_limit) if threads_limit else contextlib.nullcontext()
    except Exception:
        threadpool_info = None
        limit = contextlib.nullcontext()
    cores = len(os.sched_getaffinity(0))
    with limit:
        try:
            threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        except Exception:
            threads = int(os.environ.get("OMP_NUM_THREADS", "1"))
        t0 = time.perf_counter()
        ref = orc.oracle_call(q[:1], k[:1], v[:1], cfg.settings)[0]
        secs = time.perf_counter() - t0
    g = gpu_head0
    parity = {
        "head": 0,
        "key_labels_exact": bool(np.array_equal(g["key_labels"], ref.key_labels)),
        "q_labels_exact": bool(np.array_equal(g["q_labels"], ref.q_labels)),
        "perms_exact": bool(np.array_equal(g["key_perm"], ref.key_perm)
                            and np.array_equal(g["q_perm"], ref.q_perm)),
        "blocks_exact": bool(np.array_equal(g["blocks"], ref.blocks)),
        "probes_exact": bool(np.array_equal(g["probe_orig"], ref.probe_orig)),
        "o_rel_fro": float(np.linalg.norm(g["o"] - ref.o) / np.linalg.norm(ref.o)),
        "o_max_abs": float(np.abs(g["o"] - ref.o).max()),
        "o_sparse_rel_fro": float(np.linalg.norm(g["o_sparse"] - ref.o_sparse)
                                  / np.linalg.norm(ref.o_sparse)),
    }
    parity["pass"] = bool(parity["key_labels_exact"] and parity["q_labels_exact"]
                          and parity["perms_exact"] and parity["blocks_exact"]
                          and parity["probes_exact"] and parity["o_rel_fro"] <= 5e-3
                          and parity["o_max_abs"] <= 2e-2)
    cpu = {"value": secs * cfg.heads * 1e3, "unit": "ms", "cores": threads, "host_cores": cores,
           "kind": "oracle",
           "sample": (f"head 0 of {cfg.heads} of one call (whole fp64 oracle: partition, routing, "
                      f"sparse attention of all {cfg.n} rows, probes, fit, correction) timed once "
                      f"= {secs:.1f} s, scaled x{cfg.heads} heads")}
    return cpu, parity


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="C3")
    ap.add_argument("--density", type=float, default=None)
    ap.add_argument("--no-oracle", action="store_true", help="skip the CPU baseline and parity leg")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--host-solve", action="store_true",
                    help="eigensolve of the key metric on the host (SPARSEPR_F_HOST_SOLVE)")
    ap.add_argument("--fp8-qk", action="store_true",
                    help="experiment: the sparse kernel's logits from FP8 E4M3 Q and K "
                         "(SPARSEPR_F_FP8_QK); not the method's precision, never the headline")
    ap.add_argument("--serial-partition", action="store_true",
                    help="every head's partition on one stream (SPARSEPR_F_SERIAL_PARTITION)")
    ap.add_argument("--uniform-units", action="store_true",
                    help="sparse kernel in 128-row units only (SPARSEPR_F_UNIFORM_UNITS)")
    ap.add_argument("--raw-key-screen", action="store_true",
                    help="the key k-means screens raw keys, not their coordinates x W "
                         "(SPARSEPR_F_RAW_KEY_SCREEN; same labels)")
    ap.add_argument("--oracle-threads", type=int, default=None,
                    help="limit the oracle leg's BLAS threads (1: single-threaded baseline)")
    ap.add_argument("--oracle-all-heads", type=int, default=0, metavar="WORKERS",
                    help="also time the whole oracle call, every head in its own "
                         "single-threaded process, WORKERS at a time")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only copy MIB MiB on the device (traffic counter calibration) and exit")
    args = ap.parse_args()
    if args.copy_calibration:
        return copy_calibration(args.copy_calibration)
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path "
              f"(--gpus {args.gpus} requested). Heads shard across GPUs with no exchange; "
              f"run one process per GPU on its own heads instead.", file=sys.stderr)
        return 2

    import torch

    import free_block_sparse_eigen_amd as spr
    from synthetic import get_config, make_inputs

    cfg = get_config(args.config)
    if args.density is not None:
        cfg = cfg.with_settings(density=args.density)
    st = cfg.settings
    log(f"generating {args.config} inputs: {cfg.heads} heads x {cfg.n} tokens x d={cfg.d}")
    q, k, v = make_inputs(cfg)
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    qd, kd, vd = (torch.from_numpy(x).to(tdt).to(dev).contiguous() for x in (q, k, v))
    od = torch.empty_like(qd)
    dt = spr.BF16 if cfg.dtype == "bf16" else spr.F32
    base_flags = ((spr.F_HOST_SOLVE if args.host_solve else 0) |
                  (spr.F_SERIAL_PARTITION if args.serial_partition else 0) |
                  (spr.F_FP8_QK if args.fp8_qk else 0) |
                  (spr.F_RAW_KEY_SCREEN if args.raw_key_screen else 0) |
                  (spr.F_UNIFORM_UNITS if args.uniform_units else 0))
    ctx = spr.SparsePR.from_settings(cfg.heads, cfg.n, cfg.d, dt, st, flags=base_flags)
    stream = torch.cuda.current_stream()

    log(f"warmup {args.warmup} calls")
    for _ in range(args.warmup):
        ctx.sparsepr_attention(qd, kd, vd, od)
    torch.cuda.synchronize()
    log(f"timing {args.steps} calls")
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        ctx.sparsepr_attention(qd, kd, vd, od)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    ev_ms = ev0.elapsed_time(ev1) / args.steps
    ms_call = max(wall_ms, ev_ms)
    run_stats = ctx.sparsepr_get_stats()
    # the partition stage alone, back to back in the same context without stage events
    # (the stage-event context below records events between the stages)
    ev0.record(stream)
    for _ in range(args.steps):
        ctx.sparsepr_partition(qd, kd)
    ev1.record(stream)
    torch.cuda.synchronize()
    partition_only_ms = ev0.elapsed_time(ev1) / args.steps
    ctx.sparsepr_attention(qd, kd, vd, od)          # leave the context after a whole call
    torch.cuda.synchronize()
    # One context at a time: each holds streams of its own, and the runtime maps streams onto
    # a few hardware queues in the order they are made, so the streams of a second context
    # alive beside the first would share queues with it (and with the caller's stream).
    ctx.close()

    # stage times and the kernel's own events, in a context of their own
    log(f"stage timing: {args.steps} calls in a second context")
    sctx = spr.SparsePR.from_settings(cfg.heads, cfg.n, cfg.d, dt, st,
                                      flags=base_flags | spr.F_STAGE_TIMING)
    sctx.sparsepr_attention(qd, kd, vd, od)
    torch.cuda.synchronize()
    sctx.sparsepr_get_stats()                      # start stage averages at the timed calls
    for _ in range(args.steps):
        sctx.sparsepr_attention(qd, kd, vd, od)
    torch.cuda.synchronize()
    stats = sctx.sparsepr_get_stats()
    sctx.close()
    # the dense baseline and the parity leg in a third context
    ctx = spr.SparsePR.from_settings(cfg.heads, cfg.n, cfg.d, dt, st, flags=base_flags)
    assert stats["routed_pairs"] == run_stats["routed_pairs"], "the two contexts routed differently"
    stage = dict(zip(["partition", "route", "sparse_attention_kernel", "probe_rows", "probe_fit",
                      "correct"], [round(x, 4) for x in stats["stage_ms"]]))
    kernel_ms = stats["stage_ms"][2]
    attn_flops = 4.0 * cfg.d * stats["routed_pairs"]
    kernel_tflops = attn_flops / (kernel_ms * 1e-3) / 1e12
    call_flops = 4.0 * cfg.d * (stats["routed_pairs"] + stats["probe_pairs"])
    log(f"call {ms_call:.3f} ms; kernel {kernel_ms:.3f} ms = {kernel_tflops:.1f} TFLOP/s; stages {stage}")

    dense = None
    if not args.no_dense:
        log("dense baseline")
        for _ in range(2):
            ctx.sparsepr_dense_attn(qd, kd, vd, od)
        torch.cuda.synchronize()
        nd = max(3, args.steps // 4)
        ev0.record(stream)
        for _ in range(nd):
            ctx.sparsepr_dense_attn(qd, kd, vd, od)
        ev1.record(stream)
        torch.cuda.synchronize()
        dense_ms = ev0.elapsed_time(ev1) / nd
        dense_flops = 4.0 * cfg.d * cfg.n * cfg.n * cfg.heads
        dense = {"ms": round(dense_ms, 4),
                 "tflops": round(dense_flops / (dense_ms * 1e-3) / 1e12, 2),
                 "pct_bf16_peak": round(100 * dense_flops / (dense_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 2),
                 "speedup_sparse_call": round(dense_ms / ms_call, 3),
                 "sparse_call_over_dense": round(ms_call / dense_ms, 4)}
        log(f"dense {dense}")

    cpu = parity = None
    if not args.no_oracle:
        log("parity and CPU baseline on head 0 (oracle)")
        ctx.sparsepr_attention(qd, kd, vd, od)
        torch.cuda.synchronize()
        part = ctx.sparsepr_get_partition()
        rout = ctx.sparsepr_get_routing()
        g0 = {"key_labels": part["key_labels"][0], "q_labels": part["q_labels"][0],
              "key_perm": part["key_perm"][0], "q_perm": part["q_perm"][0],
              "blocks": rout["blocks"][0], "probe_orig": rout["probe_orig"][0],
              "o_sparse": ctx.sparsepr_get_sparse_out()[0].astype(np.float64),
              "o": od[0].float().cpu().numpy().astype(np.float64)}
        cpu, parity = oracle_baseline(cfg, q, k, v, g0, args.oracle_threads)
        log(f"parity {parity}; cpu {cpu['value']:.0f} ms/call ({cpu['cores']} cores)")
        if args.oracle_all_heads:
            log(f"whole oracle call: {cfg.heads} heads, {args.oracle_all_heads} single-threaded workers")
            wall, total = oracle_all_heads(args.config, args.density, cfg.heads, args.oracle_all_heads)
            cpu["whole_call"] = {"wall_ms": round(wall * 1e3, 1), "sum_of_heads_ms": round(total * 1e3, 1),
                                 "workers": args.oracle_all_heads, "threads_per_worker": 1}
            log(f"whole oracle call {cpu['whole_call']}")

    traffic = None if args.fp8_qk else measured_traffic(
        attn_flops, kernel_ms, f"{args.config} rho={st.density}")
    # with fp8 logits half the flops run at the fp8 rate: the time at peak is
    # (F/2) / 5033.2 + (F/2) / 2516.6, a blended peak of 3355.5 TFLOP/s
    peak = 2.0 / (1.0 / (2.0 * BF16_PEAK_TFLOPS) + 1.0 / BF16_PEAK_TFLOPS) if args.fp8_qk else BF16_PEAK_TFLOPS
    out = {
        "metric": METRIC,
        "value": round(ms_call, 4),
        "unit": "ms",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_call, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3(QK^T)+fp16(PV)" if args.fp8_qk else "bf16",
        "data": "synthetic",
        "config": {"workload": f"{args.config} {cfg.name}: {cfg.heads} heads, N={cfg.n} "
                               f"({cfg.frames}x{cfg.patch_rows}x{cfg.patch_cols}), d={cfg.d}, "
                               f"{cfg.dtype}, rho={st.density}",
                   "heads": cfg.heads, "n": cfg.n, "d": cfg.d, "density": st.density,
                   "routed_k": stats["routed_k"], "kv_groups": st.kv_groups,
                   "q_groups": st.q_groups, "probes": st.probes, "corr_rank": st.corr_rank},
        "executed_pair_tflops_kernel": round(kernel_tflops, 2),
        "pct_bf16_peak_kernel": round(100 * kernel_tflops / BF16_PEAK_TFLOPS, 2),
        "executed_pair_tflops_call": round(call_flops / (ms_call * 1e-3) / 1e12, 2),
        "exec_density": round(stats["exec_density"], 4),
        "routed_pair_density": round(stats["routed_pairs"] / (cfg.heads * cfg.n ** 2), 4),
        "stage_ms": stage,
        "stage_timing": "second context with stage events; the timed calls above ran without",
        "partition_only_ms": round(partition_only_ms, 4),
        "experiment": ("fp8 logits (SPARSEPR_F_FP8_QK): Q and K rounded to FP8 E4M3 for the sparse "
                       "kernel's Q K^T; not the method's precision") if args.fp8_qk else None,
        "metric_eigensolve": "host" if args.host_solve else "device",
        "partition_streams": 1 if args.serial_partition or cfg.heads < 2 else 2,
        "recheck_points": stats["recheck_points"],
        "key_screen": "raw keys" if args.raw_key_screen else "key coordinates where they apply",
        "work_units": ("128-row" if args.uniform_units or args.fp8_qk
                       else "256-row units (8-wave blocks) for whole chunks and rests over 128 rows, "
                            "128-row units for shorter rests, two launches side by side"),
        "dense": dense,
        "roofline": {"kernel": ("k_vbsa (variable-block-sparse attention): the sparse stage, 256-row "
                                "and 128-row units in two launches side by side" if not (args.uniform_units or args.fp8_qk)
                                else "k_vbsa (variable-block-sparse attention), 128-row units"),
                     "bound": "mfma",
                     "achieved": round(kernel_tflops, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(kernel_tflops / peak, 4),
                     "traffic": traffic,
                     "algorithmic_flops_per_launch": attn_flops,
                     "launch_ms": round(kernel_ms, 4)},
        "cpu_baseline": cpu,
        "parity": parity,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
