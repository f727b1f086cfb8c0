"""The device eigensolve of the key metric M_K (section 2A of the method summary): the
metric, and the map W = U_r diag(sqrt(lambda_r)) through W W^T (the only part that is
defined), against the oracle's numpy eigh of the same M_K; key labels bit-exact. Designed
metrics come from choosing the sampled query rows: rank-deficient, a repeated leading
eigenvalue, a spectrum twelve orders wide, and all-zero."""
import math

import numpy as np
import pytest

import oracle as orc
from synthetic import bf16_round, get_config, make_inputs
from tests.gpu_common import run_gpu_call, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def spr():
    import torch
    assert torch.cuda.is_available()
    import free_block_sparse_eigen_amd as mod
    return mod


def _check_metric(name, ctx, q, n_sample, r, heads):
    mk, w = ctx.sparsepr_get_metric()
    for i in range(heads):
        ref_mk = orc.key_metric(q[i], n_sample)
        scale = max(np.abs(ref_mk).max(), 1e-300)
        assert np.abs(mk[i] - ref_mk).max() <= 1e-13 * scale, f"{name} h{i} M_K"
        w_o, _ = orc.key_projection(mk[i], r)
        err = np.abs(w[i] @ w[i].T - w_o @ w_o.T).max()
        say(f"{name} h{i}: |W W^T - W_o W_o^T| = {err:.3e} (|M_K| {scale:.3e})")
        assert err <= 1e-11 * scale, f"{name} h{i} W W^T"


def test_metric_eigensolve_c1_c3(spr):
    for name, heads in (("C1", [0]), ("C3", [0, 7])):
        cfg = get_config(name)
        q, k, v = make_inputs(cfg, heads=heads)
        dt, dts = (spr.BF16, "bf16") if cfg.dtype == "bf16" else (spr.F32, "f32")
        ctx = spr.SparsePR.from_settings(len(heads), cfg.n, cfg.d, dt, cfg.settings)
        say(f"{name}: device eigensolve")
        g = run_gpu_call(ctx, q, k, v, dts)
        st = cfg.settings
        _check_metric(name, ctx, q, st.n_sample, st.key_rank, len(heads))
        for i in range(len(heads)):
            part = orc.partition(q[i], k[i], st.n_sample, st.key_rank, st.kv_groups, st.q_groups,
                                 st.kmeans_iters)
            assert np.array_equal(g["key_labels"][i], part.key_labels), f"{name} h{i} key labels"
            assert np.array_equal(g["q_labels"][i], part.q_labels), f"{name} h{i} query labels"
        ctx.close()


def _designed_q(kind, n, d, ms, seed):
    """Queries whose Weyl-sampled rows give a chosen metric; the other rows are random."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((n, d))
    idx = orc.weyl_indices(n, ms)
    basis, _ = np.linalg.qr(rng.standard_normal((d, d)))
    if kind == "rank8":                     # 8 directions only: eigenvalue 0 inside the top 16
        rows = rng.standard_normal((ms, 8)) @ basis[:, :8].T
    elif kind == "repeated":                # leading eigenvalue of multiplicity 6, then distinct
        rows = np.zeros((ms, d))
        for t in range(6):
            rows[t] = 4.0 * basis[:, t]
        for t in range(6, ms):
            rows[t] = (3.0 * 0.8 ** (t - 6)) * basis[:, t % d]
    elif kind == "wide":                    # eigenvalues from 1 down to about 1e-12
        rows = np.zeros((ms, d))
        for t in range(ms):
            rows[t] = (10.0 ** (-6.0 * t / (ms - 1))) * basis[:, t]
    elif kind == "zero":
        rows = np.zeros((ms, d))
    q[idx] = rows
    return bf16_round(q * math.sqrt(3.0))


@pytest.mark.parametrize("kind", ["rank8", "repeated", "wide", "zero"])
def test_designed_metrics(spr, kind):
    n, d, ms, r = 1024, 64, 40, 16
    q = _designed_q(kind, n, d, ms, seed=31)[None]
    rng = np.random.default_rng(32)
    k = bf16_round(rng.standard_normal((1, n, d)) * math.sqrt(3.0))
    v = bf16_round(rng.standard_normal((1, n, d)))
    kw = dict(n_sample=ms, key_rank=r, kv_groups=12, q_groups=10, density=0.5, probes=16,
              corr_rank=4, kmeans_iters=4)
    ctx = spr.SparsePR(spr.make_params(1, n, d, spr.F32, **kw))
    say(f"designed metric: {kind}")
    g = run_gpu_call(ctx, q, k, v, "f32")
    _check_metric(kind, ctx, q, ms, r, 1)
    if kind == "zero":
        _, w = ctx.sparsepr_get_metric()
        assert np.all(w == 0)
    part = orc.partition(q[0], k[0], ms, r, 12, 10, 4)
    assert np.array_equal(g["key_labels"][0], part.key_labels), f"{kind} key labels"
    assert np.array_equal(g["q_labels"][0], part.q_labels), f"{kind} query labels"
    assert np.all(np.isfinite(g["o"]))


def test_host_solve_flag_gives_the_same_partition(spr):
    """SPARSEPR_F_HOST_SOLVE (eigensolve on the host) and the device eigensolve give the same
    labels and, to rounding, the same W W^T."""
    cfg = get_config("C1")
    q, k, v = make_inputs(cfg)
    out = {}
    for flags in (0, spr.F_HOST_SOLVE):
        ctx = spr.SparsePR.from_settings(1, cfg.n, cfg.d, spr.F32, cfg.settings, flags=flags)
        g = run_gpu_call(ctx, q, k, v, "f32")
        out[flags] = (g, ctx.sparsepr_get_metric()[1][0])
        ctx.close()
    (g0, w0), (g1, w1) = out[0], out[spr.F_HOST_SOLVE]
    assert np.array_equal(g0["key_labels"], g1["key_labels"])
    assert np.array_equal(g0["q_labels"], g1["q_labels"])
    assert np.abs(w0 @ w0.T - w1 @ w1.T).max() < 1e-11 * np.abs(w1 @ w1.T).max()
