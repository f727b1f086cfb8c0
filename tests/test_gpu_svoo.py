"""GPU parity of the co-clustering comparison partitioner (SPARSEPR_F_SVOO: alternating
key and query assignments, each in the affinity space of the other side's current
centroids) against the oracle's svoo_partition path: labels, permutations, offsets, block
lists and probe rows bit-exact; the sparse and final outputs within the same tolerances as
the method's own partition."""
import numpy as np
import pytest

import oracle as orc
from synthetic import get_config, make_inputs
from tests.gpu_common import check_close, max_abs, rel_fro, run_gpu_call, say

pytestmark = pytest.mark.gpu

# (config, heads run on the GPU and checked against the oracle)
CASES = [("C1", [0]), ("C2", [0, 7])]


@pytest.fixture(scope="module")
def spr():
    import torch
    assert torch.cuda.is_available()
    import free_block_sparse_eigen_amd as mod
    return mod


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,heads", CASES)
def test_svoo_partition_parity(spr, name, heads):
    cfg = get_config(name)
    say(f"{name} co-clustering: generating {len(heads)} heads, N={cfg.n}")
    q, k, v = make_inputs(cfg, heads=heads)
    dt = spr.BF16 if cfg.dtype == "bf16" else spr.F32
    ctx = spr.SparsePR.from_settings(len(heads), cfg.n, cfg.d, dt, cfg.settings, flags=spr.F_SVOO)
    g = run_gpu_call(ctx, q, k, v, cfg.dtype)
    assert np.all(np.isfinite(g["o"]))
    for i, hh in enumerate(heads):
        say(f"{name} co-clustering: oracle head {hh}")
        ref = orc.oracle_call(q[i:i + 1], k[i:i + 1], v[i:i + 1], cfg.settings, svoo=True)[0]
        assert np.array_equal(g["key_labels"][i], ref.key_labels), f"{name} h{hh} key labels"
        assert np.array_equal(g["q_labels"][i], ref.q_labels), f"{name} h{hh} query labels"
        assert np.array_equal(g["key_perm"][i], ref.key_perm)
        assert np.array_equal(g["q_perm"][i], ref.q_perm)
        assert np.array_equal(g["key_off"][i], ref.key_off)
        assert np.array_equal(g["q_off"][i], ref.q_off)
        assert np.array_equal(g["blocks"][i], ref.blocks), f"{name} h{hh} blocks"
        assert np.array_equal(g["probe_orig"][i], ref.probe_orig), f"{name} h{hh} probes"
        check_close(g["o_sparse"][i], ref.o_sparse, f"{name} h{hh} O_s", rel=3e-3, out_rel=2.0 ** -24)
        say(f"{name} h{hh}: O rel_fro={rel_fro(g['o'][i], ref.o):.3e} "
            f"max_abs={max_abs(g['o'][i], ref.o):.3e}")
        check_close(g["o"][i], ref.o, f"{name} h{hh} O")
    st = ctx.sparsepr_get_stats()
    say(f"{name} co-clustering: recheck points {st['recheck_points']}")
    with pytest.raises(spr.SparsePRError):
        ctx.sparsepr_get_metric()                       # no M_K with this partitioner
    ctx.close()

