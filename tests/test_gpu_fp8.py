"""GPU parity of the fp8-logit experiment (SPARSEPR_F_FP8_QK) against the oracle's fp8_qk path.

The sparse kernel's logits come from Q and K rounded to FP8 E4M3 after per-head
power-of-two scales, on the 32x32x64 fp8 matrix instruction. The oracle rounds the same
values the same way (e4m3_round, pinned on the CPU against a decoded code table), so the
GPU's sparse output must meet the same bar against the oracle's fp8 sparse output as the
bf16 kernel meets against the plain one: the products of E4M3 values are exact in fp32 and
only the accumulation order differs. The partition, routing and probes do not change. The
cost of the rounding itself (fp8 against the plain oracle) is printed, not bounded: it is
what the experiment measures.
"""
import numpy as np
import pytest

import oracle as orc
from synthetic import get_config, make_inputs
from tests.gpu_common import check_close, max_abs, rel_fro, run_gpu_call, say

pytestmark = pytest.mark.gpu

CASES = [("C1", [0]), ("C2", [0, 7])]


@pytest.fixture(scope="module")
def spr():
    import torch
    assert torch.cuda.is_available()
    import free_block_sparse_eigen_amd as mod
    return mod


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,heads", CASES)
def test_fp8_logits_match_the_oracle(spr, name, heads):
    cfg = get_config(name)
    say(f"{name} fp8 logits: generating {len(heads)} heads, N={cfg.n}")
    q, k, v = make_inputs(cfg, heads=heads)
    dt = spr.BF16 if cfg.dtype == "bf16" else spr.F32
    ctx = spr.SparsePR.from_settings(len(heads), cfg.n, cfg.d, dt, cfg.settings, flags=spr.F_FP8_QK)
    g = run_gpu_call(ctx, q, k, v, cfg.dtype)
    ctx.close()
    assert np.all(np.isfinite(g["o"]))
    for i, hh in enumerate(heads):
        say(f"{name} fp8 logits: oracle head {hh}")
        ref = orc.oracle_call(q[i:i + 1], k[i:i + 1], v[i:i + 1], cfg.settings, fp8_qk=True)[0]
        plain = orc.oracle_call(q[i:i + 1], k[i:i + 1], v[i:i + 1], cfg.settings)[0]
        assert np.array_equal(g["key_labels"][i], ref.key_labels), f"{name} h{hh} key labels"
        assert np.array_equal(g["q_labels"][i], ref.q_labels), f"{name} h{hh} query labels"
        assert np.array_equal(g["blocks"][i], ref.blocks), f"{name} h{hh} blocks"
        assert np.array_equal(g["probe_orig"][i], ref.probe_orig), f"{name} h{hh} probes"
        check_close(g["o_sparse"][i], ref.o_sparse, f"{name} h{hh} fp8 O_s", rel=3e-3, out_rel=2.0 ** -24)
        check_close(g["o"][i], ref.o, f"{name} h{hh} fp8 O")
        say(f"{name} h{hh}: the rounding's own cost, fp8 against the plain oracle: O_s "
            f"rel_fro={rel_fro(g['o_sparse'][i], plain.o_sparse):.3e} "
            f"max_abs={max_abs(g['o_sparse'][i], plain.o_sparse):.3e}; O "
            f"rel_fro={rel_fro(g['o'][i], plain.o):.3e} max_abs={max_abs(g['o'][i], plain.o):.3e}")


@pytest.mark.timeout(600)
def test_fp8_logits_in_a_reused_call(spr):
    """The reuse path takes the new inputs' own scales: a reused call with fp8 logits against
    the oracle's reused call with fp8 logits (C2, steps 0 and 2)."""
    import torch
    from synthetic import make_step_inputs
    from tests.gpu_common import from_dev, settings_kw, to_dev
    cfg = get_config("C2")
    heads = [3]
    q0, k0, v0 = make_step_inputs(cfg, 0, heads=heads)
    q2, k2, v2 = make_step_inputs(cfg, 2, heads=heads)
    q2, k2 = q2 * 4.0, k2 * 0.25                     # new magnitudes (exact in bf16): new scales
    ctx = spr.SparsePR.from_settings(1, cfg.n, cfg.d, spr.BF16, cfg.settings, flags=spr.F_FP8_QK)
    ctx.sparsepr_attention(to_dev(q0, "bf16"), to_dev(k0, "bf16"), to_dev(v0, "bf16"))
    o = ctx.sparsepr_attention_reuse(to_dev(q2, "bf16"), to_dev(k2, "bf16"), to_dev(v2, "bf16"))
    torch.cuda.synchronize()
    o_s = ctx.sparsepr_get_sparse_out().astype(np.float64)
    o = from_dev(o)
    ctx.close()
    st = settings_kw(cfg.settings)
    r0 = orc.oracle_head(q0[0], k0[0], v0[0], fp8_qk=True, **st)
    r2 = orc.oracle_head(q2[0], k2[0], v2[0], reuse=r0, fp8_qk=True, **st)
    check_close(o_s[0], r2.o_sparse, "C2 reused fp8 O_s", rel=3e-3, out_rel=2.0 ** -24)
    check_close(o[0], r2.o, "C2 reused fp8 O")
