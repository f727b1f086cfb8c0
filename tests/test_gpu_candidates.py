"""GPU parity of the candidate-list recheck (large G with the full metric).

When a head's centroids do not fit in LDS (G = 384 at d = 128), the assignment streams
them, and the points its certified screen leaves open are screened again for the few
centroids whose screened score lies inside the error window of the best; the fp64 recheck
then looks at those only. The exact argmin is always among them, so the labels must stay
bit-exact against the oracle. C2's inputs with 384 groups make both sides take that path
(the keys with the factor W, the queries with the full metric), the raw k-means
partitioner takes it with the full metric on both sides, and 384 key groups against 192
query groups mix it with the resident-centroid assignment.
"""
import numpy as np
import pytest

import oracle as orc
from synthetic import get_config, make_inputs
from tests.gpu_common import check_close, run_gpu_call, say

pytestmark = pytest.mark.gpu

HEADS = [0, 5]


@pytest.fixture(scope="module")
def spr():
    import torch
    assert torch.cuda.is_available()
    import free_block_sparse_eigen_amd as mod
    return mod


@pytest.mark.timeout(900)
@pytest.mark.parametrize("raw,groups", [(False, (384, 384)), (True, (384, 384)), (False, (384, 192))],
                         ids=["method", "raw-kmeans", "method-Gq192"])
def test_candidate_recheck_keeps_labels_exact(spr, raw, groups):
    cfg = get_config("C2")
    cfg = cfg.with_settings(kv_groups=groups[0], q_groups=groups[1])
    say(f"C2 with G = {groups} ({'raw k-means' if raw else 'the method'}): generating heads {HEADS}")
    q, k, v = make_inputs(cfg, heads=HEADS)
    dt = spr.BF16 if cfg.dtype == "bf16" else spr.F32
    ctx = spr.SparsePR.from_settings(len(HEADS), cfg.n, cfg.d, dt, cfg.settings,
                                     flags=spr.F_RAW_KMEANS if raw else 0)
    g = run_gpu_call(ctx, q, k, v, cfg.dtype)
    st = ctx.sparsepr_get_stats()
    ctx.close()
    say(f"recheck points per call: {st['recheck_points']}")
    assert st["recheck_points"] > 0                      # the path ran
    for i, hh in enumerate(HEADS):
        say(f"oracle head {hh}")
        ref = orc.oracle_call(q[i:i + 1], k[i:i + 1], v[i:i + 1], cfg.settings, raw_kmeans=raw)[0]
        assert np.array_equal(g["key_labels"][i], ref.key_labels), f"h{hh} key labels"
        assert np.array_equal(g["q_labels"][i], ref.q_labels), f"h{hh} query labels"
        assert np.array_equal(g["blocks"][i], ref.blocks), f"h{hh} blocks"
        check_close(g["o_sparse"][i], ref.o_sparse, f"h{hh} O_s", rel=3e-3, out_rel=2.0 ** -24)
