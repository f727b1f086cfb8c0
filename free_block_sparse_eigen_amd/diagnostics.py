"""Partition diagnostics (measurement, not the attention path): how much of the attention
the routed blocks keep, and how much support a query group needs compared with its rows.

"Partition the Support, Reconstruct the Residual" (gist.science summary), section 2A: rows
that share one routing decision need the union of their keys, which can be much larger than
any single row's support; the response-coupled partition is meant to lower the hard-drop
error (the error of keeping only the routed blocks) and so what the probe fit must repair.
Two comparison partitioners: independent raw Q and K k-means (SPARSEPR_F_RAW_KMEANS) and
the alternating Q/K co-clustering of "Attention Sparsity is Input-Stable ..." (SPARSEPR_F_SVOO).

Per partitioner, for the given config:
  * hard-drop error  |O_s - O_dense|_F / |O_dense|_F over all rows and heads (GPU);
  * corrected error  |O - O_dense|_F / |O_dense|_F (GPU; probe rows are exact by design);
  * the corrected error again with the fit redone on the host (the library's fp64 probe
    fit, on the GPU's own probe rows) for other ridge lambdas, applied to O_s in fp32;
  * on a sample of query groups of head 0 (host fp64, from the library's own partition
    and routing): the routed mass (softmax mass of each row inside its group's routed key
    union, averaged over rows), the mean row support (smallest key set holding a fraction
    tau of the row's mass), the group's aggregate support (union of its rows' supports) and
    the ratio of the two, and the routed union's size.

python -m free_block_sparse_eigen_amd.diagnostics --config C3 [--groups 8] [--tau 0.9]
    [--partitioners response_coupled,raw_kmeans,svoo] [--probes-sweep 0,64,128,256,512]
prints one JSON object per partitioner, then (with --probes-sweep) one per probe budget for
the method's partition: the corrected error as the number of probe rows P varies (the
hard-drop error does not depend on P).

    [--stride-sweep 1,2,4,8 --steps 8 --theta 0.1]
reuse experiment (not the method): over `steps` successive calls of one layer
(make_step_inputs: the fine detail of every token turned by theta radians per step), the
partition and routing are recomputed every S-th call and reused in between
(sparsepr_attention_reuse). One JSON object per stride: the hard-drop and corrected errors
against dense at every step, and the amortised call time (t_full + (S - 1) t_reuse) / S
from separately timed full and reused calls.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys

import numpy as np


LAMBDA_SWEEP = (1e-3, 1e-1, 1.0, 10.0, 100.0)


def _gpu_errors(spr, torch, cfg, q, k, v, flags):
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    qd, kd, vd = (torch.from_numpy(x).to(tdt).to(dev).contiguous() for x in (q, k, v))
    od = torch.empty_like(qd)
    odense = torch.empty_like(qd)
    ctx = spr.SparsePR.from_settings(cfg.heads, cfg.n, cfg.d,
                                     spr.BF16 if cfg.dtype == "bf16" else spr.F32,
                                     cfg.settings, flags=flags)
    ctx.sparsepr_attention(qd, kd, vd, od)
    ctx.sparsepr_dense_attn(qd, kd, vd, odense)
    torch.cuda.synchronize()
    part = ctx.sparsepr_get_partition()
    rout = ctx.sparsepr_get_routing()
    o_s_perm = torch.from_numpy(ctx.sparsepr_get_sparse_out()).to(dev)       # group-major
    qperm = torch.from_numpy(part["q_perm"].astype(np.int64)).to(dev)
    o_s = torch.empty_like(o_s_perm)
    for h in range(cfg.heads):
        o_s[h].index_copy_(0, qperm[h], o_s_perm[h])
    ref = odense.float()
    den = torch.linalg.vector_norm(ref).item()
    hard = torch.linalg.vector_norm(o_s - ref).item() / den
    corr = torch.linalg.vector_norm(od.float() - ref).item() / den
    stats = ctx.sparsepr_get_stats()
    # corrected error with the fit redone for other lambdas (rank as configured)
    x, y = ctx.sparsepr_get_probes()
    porig = rout["probe_orig"]
    sweep = {}
    for lam in LAMBDA_SWEEP:
        o = torch.empty_like(o_s)
        for h in range(cfg.heads):
            bm, bv = spr.sparsepr_host_probe_fit(x[h].astype(np.float64), y[h].astype(np.float64),
                                                 lam, cfg.settings.corr_rank)
            bmt = torch.from_numpy(bm.astype(np.float32)).to(dev)
            bvt = torch.from_numpy(bv.astype(np.float32)).to(dev)
            o[h] = o_s[h] + bvt + o_s[h] @ bmt
            pr = torch.from_numpy(porig[h].astype(np.int64)).to(dev)
            o[h].index_copy_(0, pr, ref[h].index_select(0, pr))   # probe rows: exact dense
        sweep[f"{lam:g}"] = torch.linalg.vector_norm(o - ref).item() / den
    del ctx
    return hard, corr, part, rout, stats, sweep


def _stride_sweep(spr, torch, cfg, strides, steps, theta):
    from synthetic import make_step_inputs
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    dt = spr.BF16 if cfg.dtype == "bf16" else spr.F32
    inputs = []
    for s in range(steps):
        print(f"[diag] step {s} inputs", file=sys.stderr, flush=True)
        inputs.append(tuple(torch.from_numpy(x).to(tdt).to(dev).contiguous()
                            for x in make_step_inputs(cfg, s, theta)))
    ctx = spr.SparsePR.from_settings(cfg.heads, cfg.n, cfg.d, dt, cfg.settings)
    od = torch.empty_like(inputs[0][0])
    dense = torch.empty_like(od)
    # timings: full and reused calls on step 0, medians of event-timed calls
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn, reps=7):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            ev0.record()
            fn()
            ev1.record()
            torch.cuda.synchronize()
            ts.append(ev0.elapsed_time(ev1))
        return float(np.median(ts))

    q, k, v = inputs[0]
    t_full = timed(lambda: ctx.sparsepr_attention(q, k, v, od))
    t_reuse = timed(lambda: ctx.sparsepr_attention_reuse(q, k, v, od))
    out = []
    for S in strides:
        hard, corr = [], []
        for s in range(steps):
            q, k, v = inputs[s]
            if s % S == 0:
                ctx.sparsepr_attention(q, k, v, od)
            else:
                ctx.sparsepr_attention_reuse(q, k, v, od)
            ctx.sparsepr_dense_attn(q, k, v, dense)
            torch.cuda.synchronize()
            part = ctx.sparsepr_get_partition()
            o_s_perm = torch.from_numpy(ctx.sparsepr_get_sparse_out()).to(dev)
            qperm = torch.from_numpy(part["q_perm"].astype(np.int64)).to(dev)
            o_s = torch.empty_like(o_s_perm)
            for h in range(cfg.heads):
                o_s[h].index_copy_(0, qperm[h], o_s_perm[h])
            ref = dense.float()
            den = torch.linalg.vector_norm(ref).item()
            hard.append(torch.linalg.vector_norm(o_s - ref).item() / den)
            corr.append(torch.linalg.vector_norm(od.float() - ref).item() / den)
        out.append({"stride": S, "steps": steps, "theta": theta, "t_full_ms": t_full,
                    "t_reuse_ms": t_reuse, "amortised_ms": (t_full + (S - 1) * t_reuse) / S,
                    "hard_drop_rel_fro": hard, "corrected_rel_fro": corr,
                    "mean_hard_drop": float(np.mean(hard)), "mean_corrected": float(np.mean(corr))})
    del ctx
    return out


def _support_stats(q, k, part, rout, groups, tau, d):
    """Host fp64 on head 0: routed mass and supports for `groups` evenly spaced non-empty
    query groups."""
    q0, k0 = q[0].astype(np.float64), k[0].astype(np.float64)
    qperm, qoff = part["q_perm"][0], part["q_off"][0]
    kperm, koff = part["key_perm"][0], part["key_off"][0]
    blocks = rout["blocks"][0]
    sizes = np.diff(qoff)
    nonempty = np.flatnonzero(sizes > 0)
    pick = nonempty[np.linspace(0, len(nonempty) - 1, min(groups, len(nonempty))).round().astype(int)]
    scale = 1.0 / math.sqrt(d)
    res = []
    for g in pick:
        rows = qperm[qoff[g]:qoff[g + 1]]
        routed = np.concatenate([kperm[koff[j]:koff[j + 1]] for j in blocks[g] if j >= 0]
                                or [np.zeros(0, np.int64)])
        in_routed = np.zeros(k0.shape[0], bool)
        in_routed[routed] = True
        union = np.zeros(k0.shape[0], bool)
        row_support, routed_mass = [], []
        for r0 in range(0, len(rows), 256):
            logits = q0[rows[r0:r0 + 256]] @ k0.T * scale
            logits -= logits.max(axis=1, keepdims=True)
            p = np.exp(logits)
            p /= p.sum(axis=1, keepdims=True)
            routed_mass.extend(p[:, in_routed].sum(axis=1).tolist())
            order = np.argsort(-p, axis=1, kind="stable")
            cum = np.cumsum(np.take_along_axis(p, order, axis=1), axis=1)
            cnt = (cum < tau).sum(axis=1) + 1
            for i, c in enumerate(cnt):
                row_support.append(int(c))
                union[order[i, :c]] = True
        mean_row = float(np.mean(row_support))
        res.append({"group": int(g), "rows": int(len(rows)), "routed_keys": int(in_routed.sum()),
                    "routed_mass": float(np.mean(routed_mass)), "mean_row_support": mean_row,
                    "aggregate_support": int(union.sum()),
                    "expansion": float(union.sum() / mean_row)})
    return res


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--config", default="C3")
    ap.add_argument("--groups", type=int, default=8)
    ap.add_argument("--tau", type=float, default=0.9)
    ap.add_argument("--partitioners", default="response_coupled,raw_kmeans,svoo")
    ap.add_argument("--probes-sweep", default="", help="comma-separated probe budgets")
    ap.add_argument("--stride-sweep", default="", help="comma-separated reuse strides")
    ap.add_argument("--steps", type=int, default=8)
    ap.add_argument("--theta", type=float, default=0.1)
    args = ap.parse_args()
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    sys.path.insert(0, root)
    import torch
    import free_block_sparse_eigen_amd as spr
    from synthetic import get_config, make_inputs
    cfg = get_config(args.config)
    print(f"[diag] generating {args.config}: {cfg.heads} heads x {cfg.n}", file=sys.stderr, flush=True)
    strides = [int(x) for x in args.stride_sweep.split(",") if x]
    if strides:
        for rec in _stride_sweep(spr, torch, cfg, strides, args.steps, args.theta):
            rec.update({"partitioner": "response_coupled", "config": args.config})
            print(json.dumps(rec), flush=True)
        return 0
    q, k, v = make_inputs(cfg)
    flag_of = {"response_coupled": 0, "raw_kmeans": spr.F_RAW_KMEANS, "svoo": spr.F_SVOO}
    names = [x for x in args.partitioners.split(",") if x]
    for name, flags in ((nm, flag_of[nm]) for nm in names):
        print(f"[diag] {name}: GPU call and dense", file=sys.stderr, flush=True)
        hard, corr, part, rout, stats, sweep = _gpu_errors(spr, torch, cfg, q, k, v, flags)
        print(f"[diag] {name}: supports on {args.groups} groups of head 0", file=sys.stderr, flush=True)
        sup = _support_stats(q, k, part, rout, args.groups, args.tau, cfg.d)
        out = {"partitioner": name, "config": args.config, "density": cfg.settings.density,
               "routed_pair_density": stats["routed_pairs"] / (cfg.heads * cfg.n ** 2),
               "hard_drop_rel_fro": hard, "corrected_rel_fro": corr,
               "corrected_rel_fro_by_lambda": sweep, "tau": args.tau,
               "sample_routed_mass": float(np.mean([s["routed_mass"] for s in sup])),
               "sample_mean_row_support": float(np.mean([s["mean_row_support"] for s in sup])),
               "sample_aggregate_support": float(np.mean([s["aggregate_support"] for s in sup])),
               "sample_expansion": float(np.mean([s["expansion"] for s in sup])),
               "sample_routed_keys": float(np.mean([s["routed_keys"] for s in sup])),
               "groups": sup}
        print(json.dumps(out), flush=True)
    for p in (int(x) for x in args.probes_sweep.split(",") if x):
        pc = cfg.with_settings(probes=p, corr_rank=min(cfg.settings.corr_rank, max(p, 1)))
        print(f"[diag] probe budget {p}: GPU call and dense", file=sys.stderr, flush=True)
        hard, corr, _, _, stats, sweep = _gpu_errors(spr, torch, pc, q, k, v, 0)
        print(json.dumps({"partitioner": "response_coupled", "config": args.config, "probes": p,
                          "corr_rank": pc.settings.corr_rank,
                          "probe_row_fraction": p / cfg.n, "hard_drop_rel_fro": hard,
                          "corrected_rel_fro": corr, "corrected_rel_fro_by_lambda": sweep}),
              flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
