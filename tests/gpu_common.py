"""Helpers shared by the GPU tests: run the HIP path through the C ABI and gather every
intermediate, and the tolerance checks used against the fp64 oracle."""
from __future__ import annotations

import math
import sys

import numpy as np

import oracle as orc

# Output tolerances (relative Frobenius, max-abs) for floating-point results.
REL_FRO = 5e-3
MAX_ABS = 2e-2


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray, dtype: str):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, np.float32))
    t = t.to(torch.bfloat16) if dtype == "bf16" else t
    return t.cuda().contiguous()


def from_dev(t) -> np.ndarray:
    import torch
    return t.float().cpu().numpy().astype(np.float64)


def rel_fro(a, b) -> float:
    return float(np.linalg.norm(np.asarray(a) - np.asarray(b)) / max(np.linalg.norm(np.asarray(b)), 1e-300))


def max_abs(a, b) -> float:
    return float(np.max(np.abs(np.asarray(a) - np.asarray(b)))) if np.size(a) else 0.0


# Rounding of the output format itself: round-to-nearest into bf16 moves a value by at
# most 2^-8 of its magnitude (half an ulp), which exceeds 2e-2 once |O| >= 8. The max-abs
# bound is therefore applied to the error beyond that unavoidable rounding.
BF16_HALF_ULP_REL = 2.0 ** -8


def max_abs_beyond_rounding(got, ref, out_rel: float) -> float:
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    return float(np.max(np.abs(got - ref) - out_rel * np.abs(ref))) if got.size else 0.0


def check_close(got, ref, what: str, rel: float = REL_FRO, mabs: float = MAX_ABS,
                out_rel: float = BF16_HALF_ULP_REL) -> None:
    """Relative Frobenius <= rel and |got - ref| <= mabs + out_rel |ref| elementwise
    (out_rel = the output format's rounding: 2^-8 for bf16, 2^-24 for fp32)."""
    r, m = rel_fro(got, ref), max_abs_beyond_rounding(got, ref, out_rel)
    assert r <= rel and m <= mabs, (f"{what}: rel_fro={r:.3e} (<= {rel}), max_abs beyond output "
                                    f"rounding={m:.3e} (<= {mabs}), plain max_abs={max_abs(got, ref):.3e}")


def run_gpu_call(ctx, q, k, v, dtype: str, stages: bool = True):
    """Run the five stages on the GPU and read every intermediate back."""
    import torch
    qd, kd, vd = to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype)
    od = torch.empty_like(qd)
    ctx.sparsepr_partition(qd, kd)
    ctx.sparsepr_route(qd, kd, vd)
    ctx.sparsepr_sparse_attn()
    ctx.sparsepr_probe_fit()
    ctx.sparsepr_correct(od)
    torch.cuda.synchronize()
    out = dict(ctx.sparsepr_get_partition())
    out.update(ctx.sparsepr_get_routing())
    out["o_sparse"] = ctx.sparsepr_get_sparse_out().astype(np.float64)
    out["x"], out["y"] = ctx.sparsepr_get_probes()
    out["b_mat"], out["b_vec"] = ctx.sparsepr_get_fit()
    out["key_centroids"], out["q_centroids"] = ctx.sparsepr_get_centroids()
    out["o"] = from_dev(od)
    out["stats"] = ctx.sparsepr_get_stats()
    return out


def settings_kw(settings) -> dict:
    return dict(n_sample=settings.n_sample, key_rank=settings.key_rank,
                kv_groups=settings.kv_groups, q_groups=settings.q_groups,
                kmeans_iters=settings.kmeans_iters, density=settings.density,
                probes=settings.probes, ridge_lambda=settings.ridge_lambda,
                corr_rank=settings.corr_rank)


def oracle_given_partition(q, k, v, key_labels, q_labels, st_kw):
    """The oracle's route/attend/fit/correct steps on a given partition (labels)."""
    part = orc.Partition(key_labels.astype(np.int32), q_labels.astype(np.int32), None, None, None)
    return orc.oracle_head(q, k, v, part=part, **st_kw)
