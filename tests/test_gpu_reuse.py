"""The partition/route reuse experiment (sparsepr_reuse_route, sparsepr_attention_reuse)
through the C ABI: a full call on the inputs of one step, then a reused call on the inputs
of a later step (make_step_inputs), against the oracle's oracle_head(reuse=...) for the same
pair of steps. The reused call keeps the first call's labels, permutations, block lists and
probe rows bit for bit; its sparse output, probe rows and final output meet the method's
own bar."""
import numpy as np
import pytest

import oracle as orc
from synthetic import get_config, make_step_inputs
from tests.gpu_common import (check_close, from_dev, max_abs, rel_fro, say, settings_kw,
                              to_dev)

pytestmark = pytest.mark.gpu

CASES = [("C1", [0]), ("C2", [0, 5])]


@pytest.fixture(scope="module")
def spr():
    import torch
    assert torch.cuda.is_available()
    import free_block_sparse_eigen_amd as mod
    return mod


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,heads", CASES)
def test_reused_call_matches_the_oracle(spr, name, heads):
    import torch
    cfg = get_config(name)
    dt, dts = (spr.BF16, "bf16") if cfg.dtype == "bf16" else (spr.F32, "f32")
    say(f"{name} reuse: steps 0 and 2 of {len(heads)} heads")
    q0, k0, v0 = make_step_inputs(cfg, 0, heads=heads)
    q2, k2, v2 = make_step_inputs(cfg, 2, heads=heads)
    ctx = spr.SparsePR.from_settings(len(heads), cfg.n, cfg.d, dt, cfg.settings)
    ctx.sparsepr_attention(to_dev(q0, dts), to_dev(k0, dts), to_dev(v0, dts))
    torch.cuda.synchronize()
    first = dict(ctx.sparsepr_get_partition())
    first.update(ctx.sparsepr_get_routing())
    o = ctx.sparsepr_attention_reuse(to_dev(q2, dts), to_dev(k2, dts), to_dev(v2, dts))
    torch.cuda.synchronize()
    g = dict(ctx.sparsepr_get_partition())
    g.update(ctx.sparsepr_get_routing())
    o_s = ctx.sparsepr_get_sparse_out().astype(np.float64)
    x, y = ctx.sparsepr_get_probes()
    o = from_dev(o)
    for key in ("key_perm", "q_perm", "key_off", "q_off", "blocks", "probe_orig"):
        assert np.array_equal(g[key], first[key]), key
    st = settings_kw(cfg.settings)
    for i, hh in enumerate(heads):
        r0 = orc.oracle_head(q0[i], k0[i], v0[i], **st)
        r2 = orc.oracle_head(q2[i], k2[i], v2[i], reuse=r0, **st)
        assert np.array_equal(first["key_perm"][i], r0.key_perm), f"h{hh} first-call key perm"
        assert np.array_equal(first["blocks"][i], r0.blocks), f"h{hh} first-call blocks"
        check_close(o_s[i], r2.o_sparse, f"{name} h{hh} reused O_s", rel=3e-3, out_rel=2.0 ** -24)
        assert rel_fro(x[i], r2.x) < 1e-4, f"h{hh} reused X"
        say(f"{name} h{hh} reused: O rel_fro={rel_fro(o[i], r2.o):.3e} max_abs={max_abs(o[i], r2.o):.3e}")
        check_close(o[i], r2.o, f"{name} h{hh} reused O")
    ctx.close()


def test_reuse_needs_an_earlier_route(spr):
    cfg = get_config("C1")
    q, k, v = make_step_inputs(cfg, 0)
    ctx = spr.SparsePR.from_settings(1, cfg.n, cfg.d, spr.F32, cfg.settings)
    with pytest.raises(spr.SparsePRError) as e:
        ctx.sparsepr_reuse_route(to_dev(q, "f32"), to_dev(k, "f32"), to_dev(v, "f32"))
    assert e.value.status == 5
    ctx.close()
