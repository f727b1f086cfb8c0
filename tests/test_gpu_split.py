"""The partition's two-stream head split against the serial partition.

By default the partition stage runs the first and the second half of the heads on two
streams (SPARSEPR_F_SERIAL_PARTITION runs them all on the caller's stream). Every step is
per head, so both must give identical bits everywhere: labels, permutations, offsets,
centroids, block lists, probes, the sparse and the final outputs. An odd head count makes
the groups unequal, and one head of the second group is also checked against the oracle so
that its buffer offsets are pinned to something outside the library. A
second call on the same context must repeat the first, and the one-call entry
(sparsepr_attention, which permutes bf16 V on the side stream during the partition) must
repeat the stage-by-stage call.
"""
import numpy as np
import pytest

import oracle as orc
from synthetic import get_config, make_inputs
from tests.gpu_common import run_gpu_call, say

pytestmark = pytest.mark.gpu

HEADS = [0, 3, 7]          # head groups of 1 and 2 heads
KEYS = ("key_labels", "q_labels", "key_perm", "q_perm", "key_off", "q_off", "blocks",
        "probe_orig", "o_sparse", "x", "y", "b_mat", "b_vec", "key_centroids", "q_centroids", "o")


@pytest.fixture(scope="module")
def spr():
    import torch
    assert torch.cuda.is_available()
    import free_block_sparse_eigen_amd as mod
    return mod


def _one_call(ctx, q, k, v, dtype):
    """sparsepr_attention, which hands bf16 V to the partition stage, read back like
    run_gpu_call's stage-by-stage call."""
    import torch
    from tests.gpu_common import from_dev, to_dev
    qd, kd, vd = to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype)
    od = torch.empty_like(qd)
    ctx.sparsepr_attention(qd, kd, vd, od)
    torch.cuda.synchronize()
    out = dict(ctx.sparsepr_get_partition())
    out.update(ctx.sparsepr_get_routing())
    out["o_sparse"] = ctx.sparsepr_get_sparse_out().astype(np.float64)
    out["x"], out["y"] = ctx.sparsepr_get_probes()
    out["b_mat"], out["b_vec"] = ctx.sparsepr_get_fit()
    out["key_centroids"], out["q_centroids"] = ctx.sparsepr_get_centroids()
    out["o"] = from_dev(od)
    return out


def _same(a, b, what):
    for key in KEYS:
        assert np.array_equal(np.asarray(a[key]), np.asarray(b[key])), f"{what}: {key} differs"


@pytest.mark.timeout(600)
@pytest.mark.parametrize("groups", [None, (96, 160)], ids=["C2", "C2-Gk96-Gq160"])
def test_split_partition_matches_serial_and_oracle(spr, groups):
    cfg = get_config("C2")
    if groups is not None:                      # unequal G: the groups' scratch rows differ
        cfg = cfg.with_settings(kv_groups=groups[0], q_groups=groups[1])
    say(f"C2 split partition: generating heads {HEADS}, N={cfg.n}")
    q, k, v = make_inputs(cfg, heads=HEADS)
    dt = spr.BF16 if cfg.dtype == "bf16" else spr.F32
    split = spr.SparsePR.from_settings(len(HEADS), cfg.n, cfg.d, dt, cfg.settings)
    serial = spr.SparsePR.from_settings(len(HEADS), cfg.n, cfg.d, dt, cfg.settings,
                                        flags=spr.F_SERIAL_PARTITION)
    say("C2 split partition: split call 1")
    g1 = run_gpu_call(split, q, k, v, cfg.dtype)
    say("C2 split partition: split call 2")
    g2 = run_gpu_call(split, q, k, v, cfg.dtype)
    say("C2 split partition: serial call")
    gs = run_gpu_call(serial, q, k, v, cfg.dtype)
    say("C2 split partition: one-call entry (V permuted beside the partition)")
    gc = _one_call(split, q, k, v, cfg.dtype)
    split.close()
    serial.close()
    _same(g1, gs, "split vs serial")
    _same(g1, g2, "second split call")
    _same(g1, gc, "one-call entry vs stage by stage")
    i = len(HEADS) - 1                          # a head of the second group
    say(f"C2 split partition: oracle head {HEADS[i]}")
    ref = orc.oracle_call(q[i:i + 1], k[i:i + 1], v[i:i + 1], cfg.settings)[0]
    assert np.array_equal(g1["key_labels"][i], ref.key_labels), "second group: key labels"
    assert np.array_equal(g1["q_labels"][i], ref.q_labels), "second group: query labels"
    assert np.array_equal(g1["blocks"][i], ref.blocks), "second group: blocks"
