"""Stage-isolated GPU checks through the C ABI.

* Injected partitions (sparsepr_set_partition): the route, attention, probe-fit and
  correction stages run on labels given from outside, and are compared with the oracle's
  same stages on the same labels, so a partition difference cannot hide or cause them.
* The finite-check flag counts non-finite inputs and outputs on the device.
* The spectral gaps reported by the library match the oracle's eigenvalues of M_K and
  singular values of the probe residuals.
"""
import math

import numpy as np
import pytest

import oracle as orc
from synthetic import bf16_round, get_config, make_inputs
from tests.gpu_common import (check_close, from_dev, max_abs, oracle_given_partition, rel_fro,
                              say, settings_kw, to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def spr():
    import torch
    assert torch.cuda.is_available()
    import free_block_sparse_eigen_amd as mod
    return mod


def _run_injected(spr, cfg, q, k, v, key_labels, q_labels, dtype):
    import torch
    dt = spr.BF16 if dtype == "bf16" else spr.F32
    ctx = spr.SparsePR.from_settings(q.shape[0], cfg.n, cfg.d, dt, cfg.settings)
    qd, kd, vd = to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype)
    od = torch.empty_like(qd)
    ctx.sparsepr_set_partition(qd, kd, key_labels, q_labels)
    ctx.sparsepr_route(qd, kd, vd)
    ctx.sparsepr_sparse_attn()
    ctx.sparsepr_probe_fit()
    ctx.sparsepr_correct(od)
    torch.cuda.synchronize()
    g = dict(ctx.sparsepr_get_partition())
    g.update(ctx.sparsepr_get_routing())
    g["o_sparse"] = ctx.sparsepr_get_sparse_out().astype(np.float64)
    g["x"], g["y"] = ctx.sparsepr_get_probes()
    g["key_centroids"], g["q_centroids"] = ctx.sparsepr_get_centroids()
    g["o"] = from_dev(od)
    ctx.close()
    return g


def _compare_downstream(name, g, ref, i, out_rel):
    assert np.array_equal(g["key_perm"][i], ref.key_perm), f"{name} key perm"
    assert np.array_equal(g["q_perm"][i], ref.q_perm), f"{name} query perm"
    assert np.array_equal(g["key_off"][i], ref.key_off) and np.array_equal(g["q_off"][i], ref.q_off)
    assert np.array_equal(g["blocks"][i], ref.blocks), f"{name} blocks"
    assert np.array_equal(g["probe_orig"][i], ref.probe_orig), f"{name} probes"
    check_close(g["o_sparse"][i], ref.o_sparse, f"{name} O_s", rel=3e-3, out_rel=2.0 ** -24)
    assert rel_fro(g["x"][i], ref.x) < 1e-4, f"{name} X"
    assert max_abs(g["y"][i], ref.y) < 1e-4 * max(1.0, np.abs(ref.x).max()), f"{name} Y"
    say(f"{name}: O rel_fro={rel_fro(g['o'][i], ref.o):.3e} max_abs={max_abs(g['o'][i], ref.o):.3e}")
    check_close(g["o"][i], ref.o, f"{name} O", out_rel=out_rel)


def test_injected_random_partition_c1(spr):
    """Labels drawn at random (not a k-means result; one empty key group and one empty
    query group): every stage after the partition must still match the oracle."""
    cfg = get_config("C1")
    q, k, v = make_inputs(cfg)
    rng = np.random.default_rng(17)
    kl = rng.integers(0, 16, size=(1, cfg.n)).astype(np.int32)
    ql = rng.integers(0, 16, size=(1, cfg.n)).astype(np.int32)
    kl[kl == 5] = 6                                     # key group 5 empty
    ql[ql == 9] = 2                                     # query group 9 empty
    say("C1 injected random partition")
    g = _run_injected(spr, cfg, q, k, v, kl, ql, "f32")
    assert np.array_equal(g["key_labels"][0], kl[0]) and np.array_equal(g["q_labels"][0], ql[0])
    ref = oracle_given_partition(q[0], k[0], v[0], kl[0], ql[0], settings_kw(cfg.settings))
    assert np.allclose(g["key_centroids"][0], orc.group_means(k[0], kl[0], 16), rtol=0, atol=1e-12)
    assert np.allclose(g["q_centroids"][0], orc.group_means(q[0], ql[0], 16), rtol=0, atol=1e-12)
    assert np.all(g["blocks"][0] != 5), "an empty key group was routed"
    _compare_downstream("C1 injected", g, ref, 0, 2.0 ** -24)


@pytest.mark.timeout(600)
def test_injected_oracle_partition_c2(spr):
    """The oracle's own labels for two 480p heads, injected: route, attention, fit and
    correction compared with the oracle stage by stage."""
    cfg = get_config("C2")
    heads = [0, 6]
    q, k, v = make_inputs(cfg, heads=heads)
    st = settings_kw(cfg.settings)
    parts = [orc.partition(q[i], k[i], st["n_sample"], st["key_rank"], st["kv_groups"],
                           st["q_groups"], st["kmeans_iters"]) for i in range(2)]
    kl = np.stack([p.key_labels for p in parts]).astype(np.int32)
    ql = np.stack([p.q_labels for p in parts]).astype(np.int32)
    say("C2 injected oracle partition")
    g = _run_injected(spr, cfg, q, k, v, kl, ql, "bf16")
    for i, hh in enumerate(heads):
        ref = oracle_given_partition(q[i], k[i], v[i], kl[i], ql[i], st)
        _compare_downstream(f"C2 h{hh} injected", g, ref, i, 2.0 ** -8)


def test_check_finite_counts_inputs_and_outputs(spr):
    """SPARSEPR_F_CHECK_FINITE: non-finite values planted in V are counted as inputs, and the
    output rows whose routed keys include them come out non-finite and are counted; with
    the flag off nothing is counted. (No probes, so the fit stays finite.)"""
    import torch
    n, d = 1024, 64
    rng = np.random.default_rng(23)
    q = bf16_round(rng.standard_normal((1, n, d)) * math.sqrt(3.0))
    k = bf16_round(rng.standard_normal((1, n, d)) * math.sqrt(3.0))
    v = bf16_round(rng.standard_normal((1, n, d)))
    v[0, 10, 3] = np.inf
    v[0, 500, 0] = np.nan
    v[0, 900, 7] = -np.inf
    kw = dict(kv_groups=8, q_groups=8, density=0.5, probes=0, corr_rank=0, n_sample=64, key_rank=16)
    for flags, expect in ((spr.F_CHECK_FINITE, True), (0, False)):
        ctx = spr.SparsePR(spr.make_params(1, n, d, spr.BF16, flags=flags, **kw))
        qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
        o = ctx.sparsepr_attention(qd, kd, vd)
        torch.cuda.synchronize()
        st = ctx.sparsepr_get_stats()
        o_np = from_dev(o)
        bad_out = int(np.sum(~np.isfinite(o_np)))
        say(f"finite check flags={flags}: inputs={st['nonfinite_inputs']} outputs={st['nonfinite_outputs']} "
            f"(numpy sees {bad_out} non-finite outputs)")
        if expect:
            assert st["nonfinite_inputs"] == 3
            assert bad_out > 0 and st["nonfinite_outputs"] == bad_out
        else:
            assert st["nonfinite_inputs"] == 0 and st["nonfinite_outputs"] == 0
        ctx.close()
    # finite inputs: nothing counted
    v2 = bf16_round(rng.standard_normal((1, n, d)))
    ctx = spr.SparsePR(spr.make_params(1, n, d, spr.BF16, flags=spr.F_CHECK_FINITE, **kw))
    ctx.sparsepr_attention(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v2, "bf16"))
    torch.cuda.synchronize()
    st = ctx.sparsepr_get_stats()
    assert st["nonfinite_inputs"] == 0 and st["nonfinite_outputs"] == 0


def test_spectral_gaps_match_the_oracle(spr):
    """lambda_r/lambda_{r+1} of M_K and sigma_r/sigma_{r+1} of the probe residuals, per head,
    against numpy's eigenvalues of the oracle's M_K and singular values of the GPU's Y."""
    import torch
    cfg = get_config("C1")
    q, k, v = make_inputs(cfg)
    st = cfg.settings
    ctx = spr.SparsePR.from_settings(1, cfg.n, cfg.d, spr.F32, st)
    ctx.sparsepr_attention(to_dev(q, "f32"), to_dev(k, "f32"), to_dev(v, "f32"))
    torch.cuda.synchronize()
    mg, rg = ctx.sparsepr_get_gaps()
    stats = ctx.sparsepr_get_stats()
    _, y = ctx.sparsepr_get_probes()
    lam = np.linalg.eigvalsh(orc.key_metric(q[0], st.n_sample))[::-1]
    r = st.key_rank
    assert abs(mg[0] / (lam[r - 1] / lam[r]) - 1) < 1e-9
    s = np.linalg.svd(y[0].astype(np.float64), compute_uv=False)
    rr = st.corr_rank
    assert abs(rg[0] / (s[rr - 1] / s[rr]) - 1) < 1e-6
    assert stats["metric_gap_min"] == mg.min() and stats["resid_gap_min"] == rg.min()
    say(f"C1 gaps: metric {mg[0]:.4f} residual {rg[0]:.4f}")
